// Per-block local Hessian, activation-aware cross matrix and importance accumulation.
//
//   H_g[n] = (1/T_g) sum_t x_t[n] x_t[n]^T            ("add local hessian calibration", Overview)
//   P_g[n] = (1/T_g) sum_t xq_t[n] (xq_t[n]-x_t[n])^T  ("Add activation-aware local Hessian scale
//                                                      calibration", What does this PR do?)
//   Imp_g[i] = sum_t X[t,i]^2                         ("Add WMSE weight scale search calibration",
//                                                      What / How)
//
// Design (HBM-bound streaming contraction over tokens):
//  * A workgroup owns a tile of kAccTileRows rows x 64 channels (four 16-channel blocks, one per
//    wave).  X is read once, with 16-byte coalesced loads (each 64-channel row slice is one
//    128-byte line), staged through LDS, and each wave gathers its block's operand with the token
//    index along K.
//  * bf16 inputs use v_mfma_f32_16x16x32_bf16: 32 tokens per instruction, products exact, fp32
//    accumulation.  The operand A[i][k] = x_{t_k}[i] is also B[k][i], so one register set feeds
//    both.  fp32 inputs use v_mfma_f32_16x16x4_f32 with the same mapping.
//  * The cross matrix uses D = X_q - X formed in fp32 (exact for bf16 data) and split into a bf16
//    high part (truncation) and the exact bf16 remainder, so P = X_q^T D_hi + X_q^T D_lo needs two
//    more MFMAs and no catastrophic cancellation.
//  * Rows of one tile can belong to several groups (MoE experts).  The tile is walked segment by
//    segment; a group wholly inside the tile is finalized in place (beta, 1/T_g), a group that
//    crosses a tile edge leaves its partial sums in scratch slot 0 (it started earlier) or 1 (it
//    continues later), and k_acc_finalize adds the pieces of each such group in tile order.
//    Nothing uses atomics, so results are bit-identical run to run.
#include "lh_internal.hpp"

namespace lh {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunk = 32;      // rows staged per step
constexpr int kCh = 64;         // channels per workgroup
constexpr int kPitchH = kCh + 8;    // bf16 LDS row pitch (halves); 144 bytes keeps 16-byte alignment
constexpr int kPitchF = kCh + 4;    // fp32 LDS row pitch (floats)

// Row offset j of the group table; a dense layer passes no table (one group of all rows).
__device__ inline int64_t offv(const int64_t* off, int64_t j, int64_t rows) {
  return off ? off[j] : (j == 0 ? 0 : rows);
}

__device__ inline int64_t find_group(const int64_t* off, int64_t G, int64_t t, int64_t rows) {
  // largest g with off[g] <= t; then off[g+1] > t because off[G] = rows > t
  int64_t lo = 0, hi = G - 1;
  while (lo < hi) {
    int64_t mid = (lo + hi + 1) >> 1;
    if (offv(off, mid, rows) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline float bf16_lo(unsigned v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(unsigned v) { return __uint_as_float(v & 0xFFFF0000u); }

// Writes one wave's 16x16 result (lane layout of the 16x16 MFMA: lane l holds rows 4*(l/16)+r,
// column l%16) either finalized into out (beta, /T) or raw into a scratch slot.
__device__ inline void store_block(const v4f acc, float* dst, bool final_, float beta, float T,
                                   int lane) {
  const int i = lane & 15, gg = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int idx = (4 * gg + r) * 16 + i;
    float v = acc[r];
    if (final_) {
      v = v / T;
      if (beta != 0.0f) v = beta * dst[idx] + v;
    }
    dst[idx] = v;
  }
}

__device__ inline void store_imp(const v4f acc, float* imp_blk, float beta, int lane) {
  const int i = lane & 15, gg = lane >> 4;
  const int r = i - 4 * gg;
  if (r >= 0 && r < 4) {
    float v = acc[r];
    if (beta != 0.0f) v = beta * imp_blk[i] + v;
    imp_blk[i] = v;
  }
}

template <bool BF16, bool ACT>
__global__ __launch_bounds__(kThreads) void k_acc_tile(
    const void* __restrict__ Xv, const void* __restrict__ Xqv, int64_t rows, int64_t cin,
    const int64_t* __restrict__ off, int64_t G, float beta, float* __restrict__ H,
    float* __restrict__ P, float* __restrict__ imp, float* __restrict__ ws, int64_t nb) {
  constexpr int kTiles = ACT ? 2 : 1;
  constexpr int kTileElems = BF16 ? kChunk * kPitchH / 2 : kChunk * kPitchF;  // in 4-byte words
  __shared__ __attribute__((aligned(16))) unsigned lds[kTiles][kTileElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, gg = lane >> 4;
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kAccTileRows;
  const int64_t t1 = min(rows, t0 + kAccTileRows);
  const int64_t ch0 = (int64_t)blockIdx.y * kCh;
  const int64_t n = blockIdx.y * 4 + wave;        // this wave's block
  const bool wave_on = n < nb;

  // loader mapping: bf16 -> 8 threads per 64-channel row, 32 rows; fp32 -> 16 threads per row,
  // 16 rows per pass, two passes.
  constexpr int kPass = BF16 ? 1 : 2;
  const int lrow = BF16 ? (tid >> 3) : (tid >> 4);
  const int lcol = BF16 ? (tid & 7) * 8 : (tid & 15) * 4;          // in elements
  const bool col_on = ch0 + lcol < cin;
  const int esz = BF16 ? 2 : 4;
  const char* Xb = (const char*)Xv;
  const char* Xqb = (const char*)Xqv;

  v4u pre[kTiles][kPass];
  auto load = [&](int64_t r0, int64_t rend) {
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int64_t r = r0 + lrow + p * 16;
      const bool on = col_on && r < rend;
      const int64_t byte = (r * cin + ch0 + lcol) * esz;
#pragma unroll
      for (int m = 0; m < kTiles; ++m) {
        const char* base = (m == 0) ? (ACT ? Xqb : Xb) : Xb;    // act-aware: tile 0 = X_q, 1 = X
        pre[m][p] = on ? __builtin_nontemporal_load((const v4u*)(base + byte)) : v4u{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int row = lrow + p * 16;
      const int word = BF16 ? (row * kPitchH + lcol) / 2 : row * kPitchF + lcol;
#pragma unroll
      for (int m = 0; m < kTiles; ++m) *(v4u*)&lds[m][word] = pre[m][p];
    }
  };

  int64_t g = find_group(off, G, t0, rows);
  int64_t a = t0;
  while (a < t1 && g < G) {
    const int64_t gbeg = offv(off, g, rows), gend = offv(off, g + 1, rows);
    const int64_t b = max(a, min(gend, t1));   // never below a, even for offsets outside the contract
    v4f accH = {0.f, 0.f, 0.f, 0.f};
    v4f accP = {0.f, 0.f, 0.f, 0.f};

    load(a, b);
    for (int64_t r0 = a; r0 < b; r0 += kChunk) {
      __syncthreads();                 // every wave is done with the previous chunk
      stash();
      __syncthreads();
      if (r0 + kChunk < b) load(r0 + kChunk, b);   // in flight while this chunk is contracted
      if (wave_on) {
        if (BF16) {
          const unsigned short* t0h = (const unsigned short*)&lds[0][0];
          v4u aq;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const unsigned lo = t0h[(8 * gg + 2 * j) * kPitchH + 16 * wave + i];
            const unsigned hi = t0h[(8 * gg + 2 * j + 1) * kPitchH + 16 * wave + i];
            aq[j] = lo | (hi << 16);
          }
          const v8bf A = __builtin_bit_cast(v8bf, aq);
          accH = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, A, accH, 0, 0, 0);
          if (ACT) {
            const unsigned short* t1h = (const unsigned short*)&lds[kTiles - 1][0];
            v4u dh, dl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const unsigned x0 = t1h[(8 * gg + 2 * j) * kPitchH + 16 * wave + i];
              const unsigned x1 = t1h[(8 * gg + 2 * j + 1) * kPitchH + 16 * wave + i];
              const float d0 = bf16_lo(aq[j]) - bf16_lo(x0);     // exact: both are bf16
              const float d1 = bf16_hi(aq[j]) - bf16_lo(x1);
              const unsigned h0 = __float_as_uint(d0) & 0xFFFF0000u;
              const unsigned h1 = __float_as_uint(d1) & 0xFFFF0000u;
              const float l0 = d0 - __uint_as_float(h0);         // exact remainder
              const float l1 = d1 - __uint_as_float(h1);
              dh[j] = (h0 >> 16) | h1;
              dl[j] = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xFFFF0000u);
            }
            accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(v8bf, dh), accP, 0, 0, 0);
            accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(v8bf, dl), accP, 0, 0, 0);
          }
        } else {
          const float* t0f = (const float*)&lds[0][0];
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float q = t0f[(4 * s + gg) * kPitchF + 16 * wave + i];
            accH = __builtin_amdgcn_mfma_f32_16x16x4f32(q, q, accH, 0, 0, 0);
            if (ACT) {
              const float x = ((const float*)&lds[kTiles - 1][0])[(4 * s + gg) * kPitchF + 16 * wave + i];
              accP = __builtin_amdgcn_mfma_f32_16x16x4f32(q, q - x, accP, 0, 0, 0);
            }
          }
        }
      }
    }

    if (wave_on) {
      const bool head = gbeg < t0, tail = gend > t1;
      const float T = (float)(gend - gbeg);
      const int64_t blk = g * nb + n;
      if (!head && !tail) {
        if (H) store_block(accH, H + blk * 256, true, beta, T, lane);
        if (ACT) store_block(accP, P + blk * 256, true, beta, T, lane);
        if (imp) store_imp(accH, imp + g * nb * 16 + n * 16, beta, lane);
      } else {
        const int slot = head ? 0 : 1;
        float* w = ws + ((tile * 2 + slot) * kTiles * nb + n) * 256;
        store_block(accH, w, false, 0.f, 1.f, lane);
        if (ACT) store_block(accP, w + nb * 256, false, 0.f, 1.f, lane);
      }
    }
    a = b;
    ++g;
    while (g < G && offv(off, g + 1, rows) <= a) ++g;     // skip empty groups
  }
}

// One workgroup per (group, 4 blocks): combines the partial sums of groups that cross tile
// edges, in tile order, and writes empty groups (T_g = 0: only the beta term remains).
template <bool ACT>
__global__ __launch_bounds__(kThreads) void k_acc_finalize(
    const int64_t* __restrict__ off, int64_t rows, int64_t nb, float beta, float* __restrict__ H,
    float* __restrict__ P, float* __restrict__ imp, const float* __restrict__ ws) {
  constexpr int kMats = ACT ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t g = blockIdx.x;
  const int64_t n = blockIdx.y * 4 + wave;
  if (n >= nb) return;
  const int64_t gbeg = offv(off, g, rows), gend = offv(off, g + 1, rows);
  if (gbeg < 0 || gend > rows || gbeg > gend) return;     // offsets outside the contract
  const int64_t T = gend - gbeg;
  const int64_t blk = g * nb + n;
  float* outs[2] = {H ? H + blk * 256 : nullptr, ACT ? P + blk * 256 : nullptr};
  float* imp_blk = imp ? imp + g * nb * 16 + n * 16 : nullptr;
  if (T == 0) {
    for (int m = 0; m < kMats; ++m) {
      if (!outs[m]) continue;
      for (int q = 0; q < 4; ++q) {
        const int idx = lane * 4 + q;
        outs[m][idx] = beta != 0.0f ? beta * outs[m][idx] : 0.0f;
      }
    }
    if (imp_blk && lane < 16) imp_blk[lane] = beta != 0.0f ? beta * imp_blk[lane] : 0.0f;
    return;
  }
  const int64_t ta = gbeg / kAccTileRows, tb = (gend - 1) / kAccTileRows;
  if (ta == tb) return;                   // finalized by its tile
  for (int m = 0; m < kMats; ++m) {
    float s[4];
    for (int q = 0; q < 4; ++q) s[q] = ws[((ta * 2 + 1) * kMats * nb + m * nb + n) * 256 + lane * 4 + q];
    for (int64_t t = ta + 1; t <= tb; ++t)
      for (int q = 0; q < 4; ++q) s[q] += ws[((t * 2 + 0) * kMats * nb + m * nb + n) * 256 + lane * 4 + q];
    for (int q = 0; q < 4; ++q) {
      const int idx = lane * 4 + q;
      if (m == 0 && imp_blk && (idx >> 4) == (idx & 15)) {
        const int c = idx & 15;
        imp_blk[c] = beta != 0.0f ? beta * imp_blk[c] + s[q] : s[q];
      }
      if (outs[m]) {
        const float v = s[q] / (float)T;
        outs[m][idx] = beta != 0.0f ? beta * outs[m][idx] + v : v;
      }
    }
  }
}

}  // namespace

size_t accumulate_scratch_floats(int64_t rows, int64_t nb, bool act_aware) {
  const int64_t tiles = (rows + kAccTileRows - 1) / kAccTileRows;
  return (size_t)tiles * 2 * (act_aware ? 2 : 1) * nb * 256;
}

hipError_t launch_accumulate(const void* X, const void* Xq, bool bf16, int64_t rows, int64_t cin,
                             const int64_t* offsets, int64_t n_groups, float beta, float* H,
                             float* P, float* imp, float* scratch, hipStream_t stream) {
  const int64_t nb = cin / 16;
  const bool act = Xq != nullptr;
  const int64_t tiles = (rows + kAccTileRows - 1) / kAccTileRows;
  const unsigned gy = (unsigned)((nb + 3) / 4);
  if (tiles > 0) {
    dim3 grid((unsigned)tiles, gy);
    if (bf16 && act)
      hipLaunchKernelGGL((k_acc_tile<true, true>), grid, dim3(kThreads), 0, stream, X, Xq, rows, cin, offsets, n_groups, beta, H, P, imp, scratch, nb);
    else if (bf16)
      hipLaunchKernelGGL((k_acc_tile<true, false>), grid, dim3(kThreads), 0, stream, X, Xq, rows, cin, offsets, n_groups, beta, H, P, imp, scratch, nb);
    else if (act)
      hipLaunchKernelGGL((k_acc_tile<false, true>), grid, dim3(kThreads), 0, stream, X, Xq, rows, cin, offsets, n_groups, beta, H, P, imp, scratch, nb);
    else
      hipLaunchKernelGGL((k_acc_tile<false, false>), grid, dim3(kThreads), 0, stream, X, Xq, rows, cin, offsets, n_groups, beta, H, P, imp, scratch, nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 fgrid((unsigned)n_groups, gy);
  if (act)
    hipLaunchKernelGGL((k_acc_finalize<true>), fgrid, dim3(kThreads), 0, stream, offsets, rows, nb, beta, H, P, imp, scratch);
  else
    hipLaunchKernelGGL((k_acc_finalize<false>), fgrid, dim3(kThreads), 0, stream, offsets, rows, nb, beta, H, P, imp, scratch);
  return hipGetLastError();
}

}  // namespace lh
