// Per-block local Hessian, activation-aware cross matrix and importance accumulation.
//
//   H_g[n] = (1/T_g) sum_t x_t[n] x_t[n]^T            ("add local hessian calibration", Overview)
//   P_g[n] = (1/T_g) sum_t xq_t[n] (xq_t[n]-x_t[n])^T  ("Add activation-aware local Hessian scale
//                                                      calibration", What does this PR do?)
//   Imp_g[i] = sum_t X[t,i]^2                         ("Add WMSE weight scale search calibration",
//                                                      What / How)
//
// Design (HBM-bound streaming contraction over tokens):
//  * Work is split into 64-channel slices (four 16-channel blocks) and row ranges.  A wave streams
//    32-row chunks of its range with coalesced 16-byte loads (a 64-channel row slice is one
//    128-byte line), keeps the next chunk's loads in flight, stages the chunk in its own LDS
//    buffer and gathers, for each of the four blocks, the MFMA operand with the token index along
//    K.
//  * bf16 inputs use v_mfma_f32_16x16x32_bf16: 32 tokens per instruction, products exact, fp32
//    accumulation.  The operand A[i][k] = x_{t_k}[i] is also B[k][i], so one register set feeds
//    both.  fp32 inputs use v_mfma_f32_16x16x4_f32 with the same mapping.
//  * The cross matrix uses D = X_q - X formed in fp32 (one rounding, none when X_q and X are
//    within 2^15 of each other) and split exactly into bf16 pieces: P = X_q^T D_hi + X_q^T D_lo
//    (+ X_q^T D_rest when D has more than 16 significant bits), never a difference of two
//    products, so no catastrophic cancellation.
//  * Dense layer (one group): a workgroup of 16 waves owns a tile of R rows whose chunks the
//    waves take in turn; the waves add their sums in LDS at the end.  With several tiles, each
//    tile stores its sums and the last tile of a slice to finish adds them all in tile order.
//  * Grouped rows (MoE experts): every group is cut into pieces of at most R rows (a group
//    without rows is one empty piece), each workgroup finding its own pieces from a scan of the
//    group offsets; each wave owns one piece, so a group of at most R rows is finished by one wave
//    with no synchronization.  Pieces of larger groups leave
//    partial sums and the last of them to finish adds them in piece order.
//  * Partial sums and arrival counters that cross workgroups are touched only through relaxed
//    agent-scope atomics (aligned 4 or 8 bytes), so no access is a data race; gfx950 performs each
//    at the device's coherence point, past the per-XCD L2 caches (stores and loads carry the sc1
//    scope bit; the counter add is a returning atomic).  The order the last arriver relies on --
//    every piece's partial stores before its own loads -- is made by the instruction stream: a
//    wave waits for its stores to complete (s_waitcnt vmcnt(0); in the dense kernels every wave
//    waits, then a workgroup barrier, then one thread adds) before it adds to the counter, and the
//    last arriver issues its loads only once the add has returned the count.  That is the
//    compiler's own agent-scope release/acquire sequence minus the L2 writeback and invalidate,
//    which serve non-atomic data, and no non-atomic data is shared here.  A CPU test checks the
//    generated code for the wait.  Declaring the add release or acq_rel puts the writeback on
//    every arrival and doubles the 512-expert layer's accumulation time, so it is not done.  The
//    last arrival clears the counter for the next call.  Summation orders never depend on timing:
//    results are bit-identical run to run.
//  * When only the importance is wanted, partial sums keep just the 16 diagonal entries.
#include "lh_internal.hpp"
#include "acc_stream.hpp"

#include <type_traits>

namespace lh {
namespace {

using namespace stream;

__device__ inline void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_agent2(float* p, float a, float b) {   // 8-byte aligned pair
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void ld_agent2(const float* p, float& a, float& b) {
  const uint64_t v = __hip_atomic_load((uint64_t*)const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  a = __uint_as_float((unsigned)v);
  b = __uint_as_float((unsigned)(v >> 32));
}
__device__ inline unsigned arrive(unsigned* c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void clear(unsigned* c) {
  __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// X_q written out: the same fake-quant act_fake_quant applies inside the accumulation, as its own
// streaming pass (the layer's input quantizer alone).  Thread u of the grid-stride walk owns the
// 16-byte unit u of the row-major array, so the two (bf16) or four (fp32) lanes holding one
// 16-channel block are a lane pair or quad of one wave; each lane finds its row's group by a
// binary search of the offsets.  Four units per thread are loaded before any is converted.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_act_fake_quant(const v4u* __restrict__ X, v4u* __restrict__ Xq,
                                                            int64_t units, int64_t units_per_row,
                                                            const int64_t* __restrict__ off, int64_t G,
                                                            const float* __restrict__ x_amax) {
  constexpr int kU = 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t base = (int64_t)blockIdx.x * kThreads + threadIdx.x; base < units; base += kU * stride) {
    v4u x[kU];
#pragma unroll
    for (int k = 0; k < kU; ++k) {       // every lane loads (clamped), so the DPP partners exist
      const int64_t u = min(base + k * stride, units - 1);
      x[k] = __builtin_nontemporal_load(&X[u]);
    }
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int64_t u = base + k * stride;
      const int64_t row = min(u, units - 1) / units_per_row;
      int64_t g = 0;
      if (off) {                         // last group whose first row is <= row
        int64_t lo = 0, hi = G - 1;
        while (lo < hi) {
          const int64_t mid = (lo + hi + 1) >> 1;
          if (off[mid] <= row) lo = mid; else hi = mid - 1;
        }
        g = lo;
      }
      const float amax = x_amax[g];
      const float gx = amax / 2688.0f;   // fp32(amax / (6*448)), correctly rounded
      const double inv6g = 1.0 / (6.0 * (double)gx);
      const v4u q = act_fake_quant<BF16>(x[k], gx, inv6g, gx >= 0x1p-100f && gx <= 0x1p100f);
      if (u < units) __builtin_nontemporal_store(q, &Xq[u]);
    }
  }
}

// Output writer for one finished block (lane layout of the MFMA result: lane holds rows 4*gg + r,
// column i): H or P (sum / T, beta), and the importance from H's diagonal.
template <bool DIAG>
__device__ inline void emit_block(int m, const v4f s, int64_t T, int64_t blk, float beta, float* H,
                                  float* P, float* imp_blk, int i, int gg) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * gg + r;
    if (m == 0 && imp_blk && row == i) imp_blk[i] = beta != 0.0f ? beta * imp_blk[i] + s[r] : s[r];
    if (!DIAG) {
      float* o = (m == 0 ? H : P) + blk * 256 + row * 16 + i;
      const float v = T > 0 ? s[r] / (float)T : 0.0f;
      *o = beta != 0.0f ? beta * *o + v : v;
    }
  }
}

__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Same output as emit_block, written as one contiguous 1 KiB row-major block: the wave turns its
// MFMA-layout sums into rows through `tmp` (256 floats of its own LDS), then every lane stores 16
// bytes (row lane/4, columns 4*(lane%4)..+3).
template <bool DIAG>
__device__ inline void emit_block_rows(int m, const v4f s, int64_t T, int64_t blk, float beta,
                                       float* H, float* P, float* imp_blk, int lane, int i, int gg,
                                       float* tmp) {
  if (DIAG) {
    emit_block<true>(m, s, T, blk, beta, H, P, imp_blk, i, gg);
    return;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) tmp[(4 * gg + r) * 16 + i] = s[r];
  wave_sync_lds();
  const v4f v = *(const v4f*)&tmp[4 * lane];
  wave_sync_lds();                            // tmp may be rewritten by the next block
  const int row = lane >> 2, c0 = (lane & 3) * 4;
  if (m == 0 && imp_blk && (row >> 2) == (lane & 3)) {
    const float d = v[row - c0];
    imp_blk[row] = beta != 0.0f ? beta * imp_blk[row] + d : d;
  }
  v4f o = T > 0 ? v / (float)T : v4f{0.f, 0.f, 0.f, 0.f};
  v4f* dst = (v4f*)((m == 0 ? H : P) + blk * 256 + 4 * lane);
  if (beta != 0.0f) o += beta * *dst;
  *dst = o;
}

// Partial sums of one block: lane-major (lane l's four accumulator values at 4l..4l+3), or the 16
// diagonal entries (entry c = H[c][c]) when only the importance is produced.
template <bool DIAG>
__device__ inline void store_partial(float* w, const v4f s, int lane, int i, int gg) {
  if (DIAG) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * gg + r == i) st_agent(w + i, s[r]);
  } else {
    st_agent2(w + 4 * lane, s[0], s[1]);
    st_agent2(w + 4 * lane + 2, s[2], s[3]);
  }
}
template <bool DIAG>
__device__ inline v4f load_partial(const float* w, int lane, int i, int gg) {
  v4f s = {0.f, 0.f, 0.f, 0.f};
  if (DIAG) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * gg + r == i) s[r] = ld_agent(w + i);
  } else {
    float a, b, c, d;
    ld_agent2(w + 4 * lane, a, b);
    ld_agent2(w + 4 * lane + 2, c, d);
    s = v4f{a, b, c, d};
  }
  return s;
}

// Sum of n partial blocks w0, w0 + stride, ... in order, KF loads in flight (few enough that
// this tail does not set the kernel's register count).
template <bool DIAG, int KF = 4>
__device__ inline v4f sum_partials(const float* w0, int64_t stride, int64_t n, int lane, int i, int gg) {
  v4f s = {0.f, 0.f, 0.f, 0.f};
  int64_t t = 0;
  for (; t + KF <= n; t += KF) {
    v4f p[KF];
#pragma unroll
    for (int u = 0; u < KF; ++u) p[u] = load_partial<DIAG>(w0 + (t + u) * stride, lane, i, gg);
#pragma unroll
    for (int u = 0; u < KF; ++u) s += p[u];
  }
  for (; t < n; ++t) s += load_partial<DIAG>(w0 + t * stride, lane, i, gg);
  return s;
}

// ---------------------------------------------------------------------------------------------
// Dense layer: grid (tiles, slices), NW waves per tile, chunks interleaved between the waves
// (many waves per tile: few tiles, so few partial sums, yet enough loads in flight).
// Partial layout: [slice][tile][m][block][kPart].
// ---------------------------------------------------------------------------------------------
// Waves per dense workgroup (measured on MI355X): 8 for bf16 H alone, so two workgroups share a
// compute unit; 16 for bf16 H and P (both forms: X_q read or made in the kernel, which therefore
// tile alike and sum in the same order); 4 for fp32.
constexpr int dense_waves(bool bf16, bool act) { return bf16 ? (act ? 16 : 8) : 4; }

template <bool BF16, bool ACT, bool DIAG, int NW, bool FQ>
__global__ __launch_bounds__(NW * 64) void k_acc_dense(
    const void* __restrict__ Xv, const void* __restrict__ Xqv, const float* __restrict__ x_amax,
    int64_t rows, int64_t cin, int64_t R, float beta, float* __restrict__ H, float* __restrict__ P,
    float* __restrict__ imp, float* __restrict__ ws, unsigned* __restrict__ counters, int64_t nb) {
  using St = Streamer<BF16, ACT, FQ>;
  constexpr int kM = St::kM;
  constexpr int kPart = DIAG ? 16 : 256;
  constexpr int kStage = NW * kM * Geo<BF16>::kWords;
  constexpr int kComb = NW * 4 * 64 * 4;      // [wave][block][lane] v4f, in words
  __shared__ __attribute__((aligned(16))) unsigned smem[kStage > kComb ? kStage : kComb];
  __shared__ int last_tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, gg = lane >> 4;
  const int64_t tiles = gridDim.x, tile = blockIdx.x, slice = blockIdx.y;
  const int64_t n0 = slice * 4;
  const int nblk = (int)min((int64_t)4, nb - n0);
  const int64_t t0 = tile * R, t1 = min(rows, t0 + R);

  St st{(const char*)Xv, (const char*)Xqv, cin, slice * kCh, nblk, lane, i, gg,
        smem + wave * kM * Geo<BF16>::kWords, {}, {}};
  if (FQ) st.set_fake_quant(x_amax[0]);
  st.run(t0, t1, wave, NW);

  const bool mine = wave < nblk;              // waves 0..3 own the slice's four blocks
  const int64_t blk = n0 + wave;              // group 0
  float* imp_blk = imp ? imp + blk * 16 : nullptr;
  v4f* comb = (v4f*)smem;
  v4f tot[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    __syncthreads();                          // stage (or previous comb) no longer read
#pragma unroll
    for (int b = 0; b < 4; ++b) comb[(wave * 4 + b) * 64 + lane] = m == 0 ? st.accH[b] : st.accP[b];
    __syncthreads();
    tot[m] = v4f{0.f, 0.f, 0.f, 0.f};
    if (wave < 4) {
#pragma unroll
      for (int v = 0; v < NW; ++v) tot[m] += comb[(v * 4 + wave) * 64 + lane];   // wave order
    }
  }
  if (tiles == 1) {
    if (mine)
#pragma unroll
      for (int m = 0; m < kM; ++m) emit_block<DIAG>(m, tot[m], rows, blk, beta, H, P, imp_blk, i, gg);
    return;
  }
  // several tiles: each stores its sums; the slice's last tile to finish adds all of them in
  // tile order and writes the outputs
  float* part = ws + slice * tiles * kM * 4 * kPart;          // [tile][m][block][kPart]
  if (mine) {
#pragma unroll
    for (int m = 0; m < kM; ++m)
      store_partial<DIAG>(part + ((tile * kM + m) * 4 + wave) * kPart, tot[m], lane, i, gg);
  }
  __builtin_amdgcn_s_waitcnt(0);              // this wave's partial stores have completed
  __syncthreads();                            // ... and every other wave's
  if (tid == 0) last_tile = arrive(&counters[slice]) == (unsigned)(tiles - 1);
  __syncthreads();
  if (!last_tile) return;
  if (mine) {
#pragma unroll
    for (int m = 0; m < kM; ++m)
      emit_block<DIAG>(m, sum_partials<DIAG>(part + (m * 4 + wave) * kPart, kM * 4 * kPart, tiles, lane, i, gg),
                       rows, blk, beta, H, P, imp_blk, i, gg);
  }
  if (tid == 0) clear(&counters[slice]);
}

// ---------------------------------------------------------------------------------------------
// Dense layer, importance alone (no H): every lane squares and adds the channels it loads, in
// fp32 registers (the square of a bf16 value is exact in fp32), with no staging and no matrix
// instructions; the lanes that share channels, then the waves, then the tiles are added in a
// fixed order.  A workgroup owns kCW channels of a tile of R rows: for bf16 that is 512 bytes
// of every row, read by 32 lanes (two rows per load instruction), which HBM serves faster than
// the 128-byte row pieces of the H kernels' 64-channel slices.  Grid (tiles, channel slices);
// partial layout [slice][tile][kCW channels].
// ---------------------------------------------------------------------------------------------
template <bool BF16>
struct ImpGeo {
  static constexpr int kVals = BF16 ? 8 : 4;         // channels per lane (one 16-byte load per row)
  static constexpr int kCW = BF16 ? 256 : 64;        // channels per workgroup
  static constexpr int kLPR = kCW / kVals;           // lanes per row
  static constexpr int kRPL = 64 / kLPR;             // rows per load instruction
  static constexpr int kCR = BF16 ? 8 : 32;          // rows per chunk (bf16: 4 loads; 8 beat 4, 16, 32)
  static constexpr int kLoads = kCR / kRPL;          // loads per lane per chunk
};
// waves per workgroup (measured on MI355X: 4 beat 8 and 16 on the dense bf16 shapes)
constexpr int imp_waves(bool) { return 4; }

template <bool BF16, int NW>
__global__ __launch_bounds__(NW * 64) void k_imp_dense(const void* __restrict__ Xv, int64_t rows,
                                                        int64_t cin, int64_t R, float beta,
                                                        float* __restrict__ imp, float* __restrict__ ws,
                                                        unsigned* __restrict__ counters) {
  using Ig = ImpGeo<BF16>;
  constexpr int kVals = Ig::kVals, kCW = Ig::kCW, kL = Ig::kLoads;
  static_assert(kCW <= NW * 64, "one thread per channel of the slice for the final sums");
  __shared__ float comb[NW][kCW];
  __shared__ int last_tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tiles = gridDim.x, tile = blockIdx.x, slice = blockIdx.y;
  const int64_t ch0 = slice * kCW;
  const int64_t t0 = tile * R, t1 = min(rows, t0 + R);
  const int lrow = lane / Ig::kLPR;
  const int lcol = (lane % Ig::kLPR) * kVals;
  const bool col_on = ch0 + lcol < cin;
  const char* X = (const char*)Xv;
  const int nchunks = t1 > t0 ? (int)((t1 - t0 + Ig::kCR - 1) / Ig::kCR) : 0;
  float acc[kVals];
#pragma unroll
  for (int e = 0; e < kVals; ++e) acc[e] = 0.0f;
  // Every lane issues the same loads on every path (rows past the range re-read its last row and
  // are not added; channels past cin read channel 0 and land in channels that are not written).
  auto issue = [&](v4u (&p)[kL], int j) {
#pragma unroll
    for (int q = 0; q < kL; ++q) {
      const int64_t r = min(t0 + (int64_t)j * Ig::kCR + lrow + q * Ig::kRPL, t1 - 1);
      const int64_t byte = (r * cin + (col_on ? ch0 + lcol : 0)) * (BF16 ? 2 : 4);
      p[q] = __builtin_nontemporal_load((const v4u*)(X + byte));
    }
  };
  auto add = [&](const v4u (&p)[kL], int j) {
    const int64_t c0 = t0 + (int64_t)j * Ig::kCR;
    const bool full = c0 + Ig::kCR <= t1;
#pragma unroll
    for (int q = 0; q < kL; ++q) {
      const float f = (full || c0 + lrow + q * Ig::kRPL < t1) ? 1.0f : 0.0f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (BF16) {
          const float lo = __uint_as_float(p[q][u] << 16), hi = __uint_as_float(p[q][u] & 0xFFFF0000u);
          if (full) {
            acc[2 * u] = fmaf(lo, lo, acc[2 * u]);
            acc[2 * u + 1] = fmaf(hi, hi, acc[2 * u + 1]);
          } else {
            acc[2 * u] = fmaf(lo * f, lo, acc[2 * u]);
            acc[2 * u + 1] = fmaf(hi * f, hi, acc[2 * u + 1]);
          }
        } else {
          const float x = __uint_as_float(p[q][u]);
          acc[u] = full ? fmaf(x, x, acc[u]) : fmaf(x * f, x, acc[u]);
        }
      }
    }
  };
  // two register sets: a chunk's loads complete, the next chunk's are issued, then the chunk is
  // added while they are in flight (the empty asm takes the loaded registers, so the wait for
  // them comes before the next issue and never covers it)
  auto ready = [](const v4u (&p)[kL]) {
#pragma unroll
    for (int q = 0; q < kL; ++q) asm volatile("" : : "v"(p[q]));
  };
  v4u pa[kL], pb[kL];
  int j = wave;
  if (j < nchunks) issue(pa, j);
  while (j < nchunks) {
    ready(pa);
    if (j + NW < nchunks) issue(pb, j + NW);
    add(pa, j);
    j += NW;
    if (j >= nchunks) break;
    ready(pb);
    if (j + NW < nchunks) issue(pa, j + NW);
    add(pb, j);
    j += NW;
  }
  // lanes with the same channels: bf16 lanes l and l+32; fp32 lanes l, l+16, l+32, l+48
#pragma unroll
  for (int o = Ig::kLPR; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < kVals; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  if (lrow == 0)
#pragma unroll
    for (int e = 0; e < kVals; ++e) comb[wave][lcol + e] = acc[e];
  __syncthreads();
  const bool owner = tid < kCW;                 // thread tid owns channel ch0 + tid
  float tot = 0.0f;
  if (owner)
#pragma unroll
    for (int v = 0; v < NW; ++v) tot += comb[v][tid];           // wave order
  const int64_t ch = ch0 + tid;
  if (tiles == 1) {
    if (owner && ch < cin) imp[ch] = beta != 0.0f ? beta * imp[ch] + tot : tot;
    return;
  }
  // several tiles: each stores its sums; the slice's last tile to finish adds all of them in
  // tile order and writes the outputs
  float* part = ws + slice * tiles * kCW;
  if (owner) st_agent(part + tile * kCW + tid, tot);
  __builtin_amdgcn_s_waitcnt(0);              // every wave's partial stores have completed
  __syncthreads();
  if (tid == 0) last_tile = arrive(&counters[slice]) == (unsigned)(tiles - 1);
  __syncthreads();
  if (!last_tile || !owner) return;
  float s = 0.0f;
  int64_t t = 0;
  for (; t + 8 <= tiles; t += 8) {
    float p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = ld_agent(part + (t + u) * kCW + tid);
#pragma unroll
    for (int u = 0; u < 8; ++u) s += p[u];
  }
  for (; t < tiles; ++t) s += ld_agent(part + t * kCW + tid);
  if (ch < cin) imp[ch] = beta != 0.0f ? beta * imp[ch] + s : s;
  if (tid == 0) clear(&counters[slice]);
}

// ---------------------------------------------------------------------------------------------
// Grouped rows.  Every group is cut into pieces of at most R rows (a group without rows is one
// empty piece).  Pieces are numbered in group order, the pieces of one group consecutive; the
// schedule runs the R-row pieces first (longest work first), then the others, each part in piece
// order.  A 1-D grid of capacity x ceil(slices / 4) workgroups: the four waves of a workgroup take
// the same piece in four neighbouring slices (the same rows, so the same work, and 512
// contiguous bytes of every row), the slices of one piece run together.  Each workgroup derives
// its piece itself from a scan of the group offsets in LDS (no planning kernel, no table in
// memory).  Only groups of several pieces leave partial sums; their pieces
// own the slots, numbered in group order among themselves (fewer than 2 rows / R of them).
// Partial layout: [slot][slice][m][block][kPart]; counters: [group][slice].
// ---------------------------------------------------------------------------------------------
template <bool BF16, bool ACT, bool DIAG, bool FQ>
__global__ __launch_bounds__(kThreads) void k_acc_pieces(
    const void* __restrict__ Xv, const void* __restrict__ Xqv, const float* __restrict__ x_amax,
    int64_t cin, const int64_t* __restrict__ off, int64_t G, int64_t rows, int64_t R, int64_t cap,
    int64_t mcap, float beta, float* __restrict__ H, float* __restrict__ P, float* __restrict__ imp,
    float* __restrict__ ws, unsigned* __restrict__ counters, int64_t nb) {
  using St = Streamer<BF16, ACT, FQ>;
  constexpr int kM = St::kM;
  constexpr int kPart = DIAG ? 16 : 256;
  __shared__ __attribute__((aligned(16))) unsigned smem[4 * kM * Geo<BF16>::kWords];
  __shared__ int64_t scan[kThreads];
  __shared__ int64_t scan_m[kThreads];        // pieces of groups of more than one piece
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, gg = lane >> 4;
  // workgroup x: the piece in schedule slot x / sgroups, its wave w the slice 4 (x % sgroups) + w
  const int64_t slices = (nb + 3) / 4, sgroups = (slices + 3) / 4;
  const int64_t slice = (int64_t)(blockIdx.x % sgroups) * 4 + wave;

  // rows of group g, clamped to [0, rows] so that offsets outside the contract never address
  // memory outside X; its pieces: f of exactly R rows and n in all
  auto span = [&](int64_t g, int64_t& a, int64_t& e) {
    a = min(max(off[g], (int64_t)0), rows);
    e = min(max(off[g + 1], a), rows);
  };
  auto counts = [&](int64_t a, int64_t e, int64_t& f, int64_t& n) {
    f = (e - a) / R;
    n = e > a ? (e - a + R - 1) / R : 1;
  };
  // thread t counts the full and the other pieces of groups [t per, (t + 1) per); both counts are
  // scanned at once (each < 2^31), and beside them the pieces of groups of several pieces, the only
  // ones that leave partial sums (their slots are numbered among themselves)
  const int64_t per = (G + kThreads - 1) / kThreads;
  {
    const int64_t g0 = min(G, tid * per), g1 = min(G, g0 + per);
    int64_t nfull = 0, nrest = 0, nmulti = 0;
    for (int64_t g = g0; g < g1; ++g) {
      int64_t a, e, f, n;
      span(g, a, e);
      counts(a, e, f, n);
      nfull += f;
      nrest += n - f;
      nmulti += n > 1 ? n : 0;
    }
    scan[tid] = nfull | (nrest << 32);
    scan_m[tid] = nmulti;
  }
  __syncthreads();
  for (int d = 1; d < kThreads; d <<= 1) {    // inclusive scans
    const int64_t v = tid >= d ? scan[tid - d] : 0;
    const int64_t vm = tid >= d ? scan_m[tid - d] : 0;
    __syncthreads();
    scan[tid] += v;
    scan_m[tid] += vm;
    __syncthreads();
  }
  // wave-uniform values (LDS reads of one address) are moved to scalar registers
  auto uni = [](int64_t v) -> int64_t {
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  const int64_t last = uni(scan[kThreads - 1]);
  const int64_t tot_full = last & 0xFFFFFFFF;
  const int64_t total = tot_full + (last >> 32);
  const int64_t sidx = (int64_t)blockIdx.x / sgroups;
  // more pieces than the capacity only if the offsets break the contract: then nothing is done
  if (total > cap || uni(scan_m[kThreads - 1]) > mcap || sidx >= total || slice >= slices) return;   // whole wave leaves
  // schedule slot -> piece: the thread whose groups hold it (first inclusive count above the
  // rank), then a walk over that thread's groups (wave-uniform)
  const bool full = sidx < tot_full;
  const int sh = full ? 0 : 32;
  const int64_t rank = full ? sidx : sidx - tot_full;
  int lo = 0, hi = kThreads - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (((uni(scan[mid]) >> sh) & 0xFFFFFFFF) > rank) hi = mid; else lo = mid + 1;
  }
  const int t = lo;
  const int64_t before = t > 0 ? uni(scan[t - 1]) : 0;
  int64_t left = rank - ((before >> sh) & 0xFFFFFFFF);
  // partial-sum slots before this group: those of the groups of earlier threads, then of this
  // thread's earlier groups
  int64_t p = t > 0 ? uni(scan_m[t - 1]) : 0;
  const int64_t gend_t = min(G, (t + 1) * per);
  int64_t g = min(G, t * per), a = 0, e = 0, k = -1, npieces = 1;
  for (; g < gend_t; ++g) {
    int64_t f, n;
    span(g, a, e);
    counts(a, e, f, n);
    const int64_t c = full ? f : n - f;
    if (left < c) {
      k = full ? left : f;
      npieces = n;
      break;
    }
    left -= c;
    p += n > 1 ? n : 0;
  }
  if (k < 0) return;                          // not reached: the scan counted this slot here
  // the piece's numbers are wave-uniform: keep them in scalar registers
  g = uni(g);
  k = uni(k);
  p = uni(p + k);                             // its partial-sum slot (groups of several pieces)
  npieces = uni(npieces);
  const int64_t r0 = uni(a + k * R), r1 = uni(min(e, a + k * R + R)), T = uni(e - a);
  const int64_t n0 = slice * 4;
  const int nblk = (int)min((int64_t)4, nb - n0);

  St st{(const char*)Xv, (const char*)Xqv, cin, slice * kCh, nblk, lane, i, gg,
        smem + wave * kM * Geo<BF16>::kWords, {}, {}};
  if (FQ) st.set_fake_quant(x_amax[g]);
  st.run(r0, r1, 0, 1);

  float* imp_g = imp ? imp + g * nb * 16 : nullptr;
  // (block loops have a constant trip count so the accumulators stay in registers)
  if (npieces == 1) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b >= nblk) break;
#pragma unroll
      for (int m = 0; m < kM; ++m)
        emit_block_rows<DIAG>(m, m == 0 ? st.accH[b] : st.accP[b], T, g * nb + n0 + b, beta, H, P,
                              imp_g ? imp_g + (n0 + b) * 16 : nullptr, lane, i, gg, (float*)st.stage);
    }
    return;
  }
  auto part = [&](int64_t q, int m, int b) { return ws + (((q * slices + slice) * kM + m) * 4 + b) * kPart; };
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b >= nblk) break;
#pragma unroll
    for (int m = 0; m < kM; ++m) store_partial<DIAG>(part(p, m, b), m == 0 ? st.accH[b] : st.accP[b], lane, i, gg);
  }
  __builtin_amdgcn_s_waitcnt(0);              // the partial stores have completed
  unsigned prev = 0;
  if (lane == 0) prev = arrive(&counters[g * slices + slice]);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != (unsigned)(npieces - 1)) return;
  // the group's last piece to arrive adds all pieces in order
  const int64_t pfirst = p - k;
  for (int b = 0; b < nblk; ++b)
    for (int m = 0; m < kM; ++m)
      emit_block_rows<DIAG>(m, sum_partials<DIAG>(part(pfirst, m, b), slices * kM * 4 * kPart, npieces, lane, i, gg),
                            T, g * nb + n0 + b, beta, H, P, imp_g ? imp_g + (n0 + b) * 16 : nullptr,
                            lane, i, gg, (float*)st.stage);
  if (lane == 0) clear(&counters[g * slices + slice]);
}

// Rows per tile of a dense layer with H: NW waves x 32 rows x c chunks per wave, with the largest
// c of 1, 2, 4, 8 that still gives 256 workgroups.  Measured on MI355X for the dense shapes.
int64_t dense_tile_rows(int64_t rows, int64_t nb, bool bf16, bool act) {
  const int64_t slices = (nb + 3) / 4;
  const int64_t base = dense_waves(bf16, act) * kChunk;
  int64_t R = base;
  while (R < 8 * base && ((rows + 2 * R - 1) / (2 * R)) * slices >= 256) R *= 2;
  return R;
}

// Importance-only dense layer: channel slices of ImpGeo::kCW channels and tiles of R rows, R
// doubling from one chunk per wave while at least 384 workgroups remain (measured on MI355X for
// the dense shapes: fewer, longer tiles leave HBM idle at the ends, more add partial sums).
int64_t imp_slices(int64_t cin, bool bf16) {
  const int64_t cw = bf16 ? ImpGeo<true>::kCW : ImpGeo<false>::kCW;
  return (cin + cw - 1) / cw;
}
int64_t imp_tile_rows(int64_t rows, int64_t cin, bool bf16) {
  const int64_t slices = imp_slices(cin, bf16);
  const int64_t base = imp_waves(bf16) * (int64_t)(bf16 ? ImpGeo<true>::kCR : ImpGeo<false>::kCR);
  int64_t R = base;
  while (R < 64 * base && ((rows + 2 * R - 1) / (2 * R)) * slices >= 384) R *= 2;
  return R;
}

bool is_dense(const int64_t* offsets, int64_t n_groups) { return !offsets || n_groups == 1; }

// Pieces of groups of more than one piece (the ones with partial-sum slots): such a group has
// T_g > R rows and ceil(T_g / R) < 2 T_g / R pieces, so together fewer than 2 rows / R.
int64_t multi_piece_cap(int64_t rows, int64_t R) { return 2 * rows / R; }

template <bool BF16, bool ACT, bool DIAG, bool FQ = false>
hipError_t launch_kind(bool dense, int64_t rows, int64_t cin, const int64_t* off, int64_t G,
                       const void* X, const void* Xq, const float* x_amax, float beta, float* H,
                       float* P, float* imp, void* work, unsigned* counters, hipStream_t stream) {
  const int64_t nb = cin / 16, slices = (nb + 3) / 4;
  if (dense) {
    if constexpr (DIAG && !ACT) {
      constexpr int NW = imp_waves(BF16);
      const int64_t R = imp_tile_rows(rows, cin, BF16);
      const int64_t tiles = max((int64_t)1, (rows + R - 1) / R);
      hipLaunchKernelGGL((k_imp_dense<BF16, NW>), dim3((unsigned)tiles, (unsigned)imp_slices(cin, BF16)),
                         dim3(NW * 64), 0, stream, X, rows, cin, R, beta, imp, (float*)work, counters);
      return hipGetLastError();
    } else {
      constexpr int NW = dense_waves(BF16, ACT);
      const int64_t R = dense_tile_rows(rows, nb, BF16, ACT);
      const int64_t tiles = max((int64_t)1, (rows + R - 1) / R);
      hipLaunchKernelGGL((k_acc_dense<BF16, ACT, DIAG, NW, FQ>), dim3((unsigned)tiles, (unsigned)slices),
                         dim3(NW * 64), 0, stream, X, Xq, x_amax, rows, cin, R, beta, H, P, imp,
                         (float*)work, counters, nb);
      return hipGetLastError();
    }
  }
  const int64_t R = piece_rows(rows, nb);
  const int64_t cap = rows / R + G;           // >= sum over groups of max(1, ceil(T_g / R))
  const int64_t mcap = multi_piece_cap(rows, R);
  float* ws = (float*)work;
  hipLaunchKernelGGL((k_acc_pieces<BF16, ACT, DIAG, FQ>), dim3((unsigned)(cap * ((slices + 3) / 4))),
                     dim3(kThreads), 0, stream, X, Xq, x_amax, cin, off, G, rows, R, cap, mcap, beta, H, P, imp,
                     ws, counters, nb);
  return hipGetLastError();
}

}  // namespace

__global__ void k_zero_fill(unsigned* p, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_fill(unsigned* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_fill, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     p, (int64_t)n);
  return hipGetLastError();
}

hipError_t launch_act_fake_quant(const void* X, bool bf16, int64_t rows, int64_t cin, const int64_t* offsets,
                                 int64_t n_groups, const float* x_amax, void* Xq, hipStream_t stream) {
  const int64_t units = rows * cin * (bf16 ? 2 : 4) / 16;
  if (units == 0) return hipSuccess;
  const int64_t upr = cin * (bf16 ? 2 : 4) / 16;
  const int64_t want = (units + kThreads * 4 - 1) / (kThreads * 4);
  const unsigned grid = (unsigned)min(want, (int64_t)8192);
  const int64_t* off = (offsets && n_groups > 1) ? offsets : nullptr;
  if (bf16)
    hipLaunchKernelGGL(k_act_fake_quant<true>, dim3(grid), dim3(kThreads), 0, stream, (const v4u*)X, (v4u*)Xq,
                       units, upr, off, n_groups, x_amax);
  else
    hipLaunchKernelGGL(k_act_fake_quant<false>, dim3(grid), dim3(kThreads), 0, stream, (const v4u*)X, (v4u*)Xq,
                       units, upr, off, n_groups, x_amax);
  return hipGetLastError();
}

AccScratch accumulate_scratch(int64_t rows, int64_t nb, const int64_t* offsets, int64_t n_groups,
                              bool bf16, bool act_aware, bool imp_only) {
  const int64_t slices = (nb + 3) / 4;
  const size_t part = (size_t)(act_aware ? 2 : 1) * 4 * (imp_only ? 16 : 256) * sizeof(float);
  AccScratch s;
  if (is_dense(offsets, n_groups) && imp_only && !act_aware) {
    const int64_t cin = nb * 16, R = imp_tile_rows(rows, cin, bf16);
    const int64_t tiles = (rows + R - 1) / R, cw = bf16 ? ImpGeo<true>::kCW : ImpGeo<false>::kCW;
    s.work_bytes = (size_t)imp_slices(cin, bf16) * tiles * cw * sizeof(float);
    s.counters = (size_t)slices;
  } else if (is_dense(offsets, n_groups)) {
    const int64_t R = dense_tile_rows(rows, nb, bf16, act_aware);
    const int64_t tiles = (rows + R - 1) / R;
    s.work_bytes = (size_t)slices * tiles * part;
    s.counters = (size_t)slices;
  } else {
    const int64_t R = piece_rows(rows, nb);
    s.work_bytes = (size_t)multi_piece_cap(rows, R) * slices * part;
    s.counters = (size_t)n_groups * slices;
  }
  return s;
}

hipError_t launch_accumulate(const void* X, const void* Xq, const float* x_amax, bool bf16,
                             int64_t rows, int64_t cin, const int64_t* offsets, int64_t n_groups,
                             float beta, float* H, float* P, float* imp, void* work,
                             size_t work_bytes, unsigned* counters, size_t n_counters,
                             hipStream_t stream) {
  const bool fq = x_amax != nullptr;
  const bool act = Xq != nullptr || fq;
  const bool diag = !act && H == nullptr;
  const bool dense = is_dense(offsets, n_groups);
  const AccScratch need = accumulate_scratch(rows, cin / 16, offsets, n_groups, bf16, act, diag);
  if (work_bytes < need.work_bytes || n_counters < need.counters) return hipErrorInvalidValue;
#define LH_ACC_KIND(B, A, D, F) \
  launch_kind<B, A, D, F>(dense, rows, cin, offsets, n_groups, X, Xq, x_amax, beta, H, P, imp, work, counters, stream)
  if (fq) return bf16 ? LH_ACC_KIND(true, true, false, true) : LH_ACC_KIND(false, true, false, true);
  if (act) return bf16 ? LH_ACC_KIND(true, true, false, false) : LH_ACC_KIND(false, true, false, false);
  if (diag) return bf16 ? LH_ACC_KIND(true, false, true, false) : LH_ACC_KIND(false, false, true, false);
  return bf16 ? LH_ACC_KIND(true, false, false, false) : LH_ACC_KIND(false, false, false, false);
#undef LH_ACC_KIND
}

}  // namespace lh
