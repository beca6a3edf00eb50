// Streaming pieces of the per-block Hessian accumulation shared by the accumulation kernels and
// the fused MoE accumulate-and-sweep kernel: the 32-row chunk streamer that contracts a 64-channel
// slice of X (and X_q) into four 16x16 blocks on the matrix cores, the activation fake-quant it
// can apply on the way, and the piece size of grouped rows.  Both users include it, so a block's
// Hessian is summed in the same order wherever it is made.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lh {
namespace stream {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short v2us __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kChunk = 32;          // rows per chunk (one 16x16x32 MFMA per block)
constexpr int kCh = 64;             // channels per slice (four blocks)
constexpr int kPitchH = kCh + 8;    // bf16 LDS row pitch (halves); 144 bytes keeps 16-byte alignment
constexpr int kPitchF = kCh + 4;    // fp32 LDS row pitch (floats)

template <bool BF16>
struct Geo {
  static constexpr int kLoads = BF16 ? 4 : 8;             // 16-byte loads per lane per chunk
  static constexpr int kRowsPerLoad = BF16 ? 8 : 4;       // rows one wave-wide load covers
  static constexpr int kWords = BF16 ? kChunk * kPitchH / 2 : kChunk * kPitchF;  // per matrix
};

__device__ inline float bf16_lo(unsigned v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(unsigned v) { return __uint_as_float(v & 0xFFFF0000u); }

// ---------------------------------------------------------------------------------------------
// NVFP4 fake-quant of the activations, applied while a chunk streams in (the layer's input
// quantizer).  Per group: gX = fp32(amax_X / (6*448)).  Per row and 16-channel block: v = the E4M3
// value (0 or one of the 126 positive finite values) nearest to max|x| / (6 gX), ties to the even
// code, so it saturates at 448 and flushes small blocks to 0; s = fp32(v gX); each element becomes
// E2M1(x / s) * s (nearest grid value of |x|/s, ties to the even index, saturating at 6, sign of
// x) computed in fp32 and stored in the input dtype (rounded to nearest-even bf16 for bf16 data).
// ---------------------------------------------------------------------------------------------
template <int CTRL>
__device__ inline unsigned dpp_u(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// E4M3 value nearest to y >= 0, ties to the even code, saturating at 448.  y = amax * (1/(6 gX))
// carries at most 2^-52 relative error; the exact quotient of a bf16 or fp32 amax by 6 gX either
// equals an E4M3 midpoint or lies more than 2^-31 of itself away from every midpoint, so a y
// within 2^-40 of a midpoint is that midpoint and every other y is on the exact quotient's side.
__device__ inline float e4m3_nearest(double y) {
  if (!(y < 448.0)) return 448.0f;
  if (y == 0.0) return 0.0f;
  const int e = max(ilogb(y), -6);                // spacing 2^(e-3); 2^-9 below 2^-6
  const double t = ldexp(y, 3 - e);               // exact, in [0, 16)
  const double k = floor(t), f = t - k;
  const double q = fabs(f - 0.5) <= 0x1p-40 * t ? k + (double)((int)k & 1) : rint(t);
  return (float)fmin(ldexp(q, e - 3), 448.0);
}

// The same value from fp32 arithmetic: y = amax * fp32(1/(6 gX)) is within 2^-23 of itself of the
// exact quotient (two roundings of 2^-24), i.e. within 2 units of y's last place in the E4M3 normal
// range and 2^-20 of a grid step below 2^-6, so rounding y to the E4M3 grid decides as the exact
// quotient would unless y lies within 8 units (normal range) or 2^-18 steps (below 2^-6) of a
// midpoint; those blocks take the float64 path.  Normal range: round the fp32 significand to 3
// bits, ties to even (the even code); below 2^-6 the grid is the multiples of 2^-9.  For gX in
// [2^-100, 2^100], so that 1/(6 gX) is a normal fp32 value.
__device__ inline float e4m3_nearest_f32(float amax, double inv6g) {
  const float y = amax * (float)inv6g;
  const unsigned b = __float_as_uint(y);
  const unsigned low = b & 0xFFFFFu;                                // bits below the 3 kept
  const float vn = __uint_as_float((b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u);
  const float t = y * 512.0f;                                       // grid steps below 2^-6
  const float vs = rintf(t) * 0x1p-9f;
  const bool normal = y >= 0x1p-6f;
  const bool near = normal ? low - 0x7FFF8u <= 16u : fabsf(t - floorf(t) - 0.5f) <= 0x1p-18f;
  if (!(y < 448.0f)) return 448.0f;
  if (near) return e4m3_nearest((double)amax * inv6g);
  return normal ? vn : vs;
}

__device__ inline float e2m1_value(int c) {
  return c <= 4 ? 0.5f * (float)c : (c == 5 ? 3.0f : (c == 6 ? 4.0f : 6.0f));
}
// Exact E2M1 index of |x|/s between grid indices lo and lo + 1: the sign of m s - |x| (m their
// midpoint, at most 3 significant bits) is exact in one fma; a tie goes to the even index.
__device__ inline int e2m1_resolve(float ax, float s, int lo) {
  const float m = lo < 4 ? 0.25f + 0.5f * (float)lo : (lo == 4 ? 2.5f : (lo == 5 ? 3.5f : 5.0f));
  const float d = fmaf(m, s, -ax);
  return d < 0.0f ? lo + 1 : (d > 0.0f ? lo : lo + (lo & 1));
}
// E2M1 index of r = |x|/s given as an exactly rounded float64 quotient (ties to the even index).
__device__ inline int e2m1_index_f64(double r) {
  return (int)(r > 0.25) + (int)(r >= 0.75) + (int)(r > 1.25) + (int)(r >= 1.75) +
         (int)(r > 2.5) + (int)(r >= 3.5) + (int)(r > 5.0);
}

// Fake-quantizes the 16 bytes a lane holds of one row: 8 bf16 (half a block; the other half is in
// lane ^ 1) or 4 fp32 (a quarter; the block is the lane's quad).  gx = gX, inv6g = 1/(6 gX) in
// float64, fast = gX in [2^-100, 2^100] (all scales and quotients normal).
// *d_exact is set to false when the block's scale may have saturated far below its amax
// (max|x| / (6 gX) > 672 or NaN): otherwise every x_q - x is exact in the input format (see
// finish_stage).
template <bool BF16>
__device__ inline v4u act_fake_quant(const v4u x, float gx, double inv6g, bool fast, bool* d_exact = nullptr) {
  constexpr int n = BF16 ? 8 : 4;
  float xf[n];
  unsigned am = 0;
  if constexpr (BF16) {
    // magnitudes as 15-bit integers order like the values: packed 16-bit maxima, then the halves
    v2us m2 = {0, 0};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      xf[2 * p] = __uint_as_float(x[p] << 16);
      xf[2 * p + 1] = __uint_as_float(x[p] & 0xFFFF0000u);
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(v2us, x[p] & 0x7FFF7FFFu));
    }
    am = (unsigned)max(m2[0], m2[1]) << 16;
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      xf[p] = __uint_as_float(x[p]);
      am = max(am, x[p] & 0x7FFFFFFFu);
    }
  }
  am = max(am, dpp_u<0xB1>(am));                  // quad_perm [1,0,3,2]: the lane pair
  if (!BF16) am = max(am, dpp_u<0x4E>(am));       // quad_perm [2,3,0,1]: the whole quad
  const float v = fast ? e4m3_nearest_f32(__uint_as_float(am), inv6g)
                       : (gx > 0.0f ? e4m3_nearest((double)__uint_as_float(am) * inv6g) : 0.0f);
  const float s = v * gx;                         // fp32(v gX): one rounding of an exact product
  if (d_exact) *d_exact = s == 0.0f || (double)__uint_as_float(am) * inv6g <= 672.0;
  float q[n];
  if (fast) {
    // Nearest grid values of x * (1/s) pushed up and down by 2^-19 bracket the exact quotient
    // (the quotient through the 1-ulp hardware reciprocal is within 2^-21 of it) and agree unless
    // it is within about 2^-18 of a midpoint; those elements take the exact decision.  s = 0
    // (a block that rounds to 0) uses 1/s = 0, so every element becomes 0.
    const float is = s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
    const float iu = is * 1.0000019073486328125f, id = is * 0.9999980926513671875f;
    unsigned up = 0u, dn = 0u;
    auto pack = [&](auto sel) {                   // the convert's byte select is an immediate
      constexpr int p = decltype(sel)::value;
      up = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(up, xf[2 * p] * iu, xf[2 * p + 1] * iu, 1.0f, p);
      dn = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dn, xf[2 * p] * id, xf[2 * p + 1] * id, 1.0f, p);
    };
    pack(std::integral_constant<int, 0>{});
    pack(std::integral_constant<int, 1>{});
    if constexpr (n == 8) {
      pack(std::integral_constant<int, 2>{});
      pack(std::integral_constant<int, 3>{});
    }
    if (up != dn) {
#pragma unroll
      for (int k = 0; k < n; ++k) {
        const int cu = (up >> (4 * k)) & 7, cd = (dn >> (4 * k)) & 7;
        if (cu != cd)
          up = (up & ~(7u << (4 * k))) | ((unsigned)e2m1_resolve(fabsf(xf[k]), s, cd) << (4 * k));
      }
    }
    auto unpack = [&](auto sel) {
      constexpr int p = decltype(sel)::value;
      const v2f g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(up, 1.0f, p);   // signed grid values
      q[2 * p] = g[0] * s;
      q[2 * p + 1] = g[1] * s;
    };
    unpack(std::integral_constant<int, 0>{});
    unpack(std::integral_constant<int, 1>{});
    if constexpr (n == 8) {
      unpack(std::integral_constant<int, 2>{});
      unpack(std::integral_constant<int, 3>{});
    }
  } else {
#pragma unroll
    for (int k = 0; k < n; ++k) {
      const int c = s == 0.0f ? 0 : e2m1_index_f64((double)fabsf(xf[k]) / (double)s);
      q[k] = copysignf(e2m1_value(c) * s, xf[k]);
    }
  }
  v4u out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (BF16) {
      const v2bf b = __builtin_convertvector((v2f){q[2 * p], q[2 * p + 1]}, v2bf);   // nearest-even
      out[p] = __builtin_bit_cast(unsigned, b);
    } else {
      out[p] = __float_as_uint(q[p]);
    }
  }
  return out;
}

// One wave's streaming contraction of 64-channel row slices into four blocks of accumulators,
// using the wave's own LDS stage.  A chunk is 32 rows starting at row c0 of a range that ends at
// r1: issue() puts its loads in flight (rows past the range re-read its last row, channels past
// cin read channel 0; every lane issues the same loads on every path), stage_chunk() writes it to
// the stage with those rows and channels zeroed,
// finish_stage() makes the stage visible to the whole wave (with FQ it first makes X_q from the
// staged X, kept in registers: X_q is not read, it is made while the next chunk's loads are in
// flight),
// and contract() adds it to the accumulators.  The next chunk's loads are issued between
// stage_chunk() and contract(), so one chunk is in flight while a chunk is contracted.
template <bool BF16, bool ACT, bool FQ = false>
struct Streamer {
  using Gm = Geo<BF16>;
  static constexpr int kM = ACT ? 2 : 1;
  const char* X;
  const char* Xq;
  int64_t cin, ch0;
  int nblk, lane, i, gg;
  unsigned* stage;              // [kM][kWords] of this wave
  v4f accH[4], accP[4];
  float gx = 0.0f;              // FQ: the group's gX, 1/(6 gX) in float64, gX in the fast range
  double inv6g = 0.0;
  bool fq_fast = false;
  v4u pre[kM][Gm::kLoads];      // the chunk in flight
  v4u xs[Gm::kLoads];           // FQ: the staged chunk's X, kept for the fake-quant
  bool d_exact = false;         // FQ: the stage holds D = X_q - X (exact) in place of X

  __device__ void set_fake_quant(float x_amax) {
    gx = x_amax / 2688.0f;                       // fp32(amax / (6*448)), correctly rounded
    inv6g = 1.0 / (6.0 * (double)gx);
    fq_fast = gx >= 0x1p-100f && gx <= 0x1p100f;
  }

  __device__ void zero() {
#pragma unroll
    for (int b = 0; b < 4; ++b) accH[b] = accP[b] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  __device__ int lrow() const { return BF16 ? (lane >> 3) : (lane >> 4); }
  __device__ int lcol() const { return BF16 ? (lane & 7) * 8 : (lane & 15) * 4; }
  __device__ bool col_on() const { return ch0 + lcol() < cin; }
  __device__ static int word(int row, int col) { return BF16 ? (row * kPitchH + col) / 2 : row * kPitchF + col; }

  __device__ void issue(int64_t c0, int64_t r1) {
    const int esz = BF16 ? 2 : 4;
    const int64_t col = col_on() ? ch0 + lcol() : 0;
#pragma unroll
    for (int q = 0; q < Gm::kLoads; ++q) {
      const int64_t r = min(c0 + lrow() + q * Gm::kRowsPerLoad, r1 - 1);
      const int64_t byte = (r * cin + col) * esz;
#pragma unroll
      for (int m = FQ ? 1 : 0; m < kM; ++m) {
        const char* base = (m == 0) ? (ACT ? Xq : X) : X;    // act-aware: matrix 0 = X_q, 1 = X
        pre[m][q] = __builtin_nontemporal_load((const v4u*)(base + byte));
      }
    }
  }

  // With FQ, X is kept in registers and finish_stage writes the stage.
  __device__ void stage_chunk(int64_t c0, int64_t r1) {
#pragma unroll
    for (int q = 0; q < Gm::kLoads; ++q) {
      const int row = lrow() + q * Gm::kRowsPerLoad;
      const bool on = col_on() && c0 + row < r1;
      if constexpr (FQ) {
        xs[q] = on ? pre[1][q] : v4u{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int m = 0; m < kM; ++m)
          *(v4u*)&stage[m * Gm::kWords + word(row, lcol())] = on ? pre[m][q] : v4u{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ void finish_stage() {
    if constexpr (FQ) {
      // Each lane quantizes the 16 bytes of X it holds (an X of zeros stays zero) and stages X_q
      // and D = X_q - X.  Every x_q is 0 or has the sign of x and lies within a factor of 2 of it:
      // the E2M1 cell of |x|/s keeps grid / |x|/s in [2/3, 2], the value 0.5 s rounded to the input
      // format cannot pass 2|x| (a value of that format above it), and a scale v gX that did not
      // saturate far below the block's amax (max|x| / (6 gX) <= 672, so max|x| <= 9 s even for the
      // smallest subnormal v) keeps saturated elements within 2/3 of 6 s.  By Sterbenz's lemma D is
      // then exact in the input format, one bf16 piece, and the cross matrix takes one MFMA on it.
      // When some block of the chunk may have saturated further, X is staged instead and the
      // contraction splits D as for a stored X_q.
      bool ok = true;
#pragma unroll
      for (int q = 0; q < Gm::kLoads; ++q) {
        const int w = word(lrow() + q * Gm::kRowsPerLoad, lcol());
        bool okq;
        const v4u xq = act_fake_quant<BF16>(xs[q], gx, inv6g, fq_fast, &okq);   // every lane: uses its pair/quad
        ok = ok && okq;
        *(v4u*)&stage[w] = xq;
        v4u d;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if constexpr (BF16) {
            const float d0 = bf16_lo(xq[p]) - bf16_lo(xs[q][p]);    // exact, a bf16 value
            const float d1 = bf16_hi(xq[p]) - bf16_hi(xs[q][p]);
            d[p] = (__float_as_uint(d0) >> 16) | (__float_as_uint(d1) & 0xFFFF0000u);
          } else {
            d[p] = __float_as_uint(__uint_as_float(xq[p]) - __uint_as_float(xs[q][p]));
          }
        }
        *(v4u*)&stage[Gm::kWords + w] = d;
      }
      d_exact = !__builtin_amdgcn_ballot_w64(!ok);
      if (!d_exact) {
#pragma unroll
        for (int q = 0; q < Gm::kLoads; ++q)
          *(v4u*)&stage[Gm::kWords + word(lrow() + q * Gm::kRowsPerLoad, lcol())] = xs[q];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Rows [r0, r1) from zero, chunks taken with a stride of `step` chunks starting at chunk `first`
  // (counted from r0), so several waves can share a range.
  __device__ void run(int64_t r0, int64_t r1, int first, int step) {
    zero();
    if (r1 <= r0) return;
    const int nchunks = (int)((r1 - r0 + kChunk - 1) / kChunk);
    auto at = [&](int j) { return r0 + (int64_t)j * kChunk; };
    int j = first;
    if (j < nchunks) issue(at(j), r1);
    for (; j < nchunks; j += step) {
      stage_chunk(at(j), r1);
      if (j + step < nchunks) issue(at(j + step), r1);
      finish_stage();
      contract();
    }
  }

  // Adds the staged chunk (rows past the range are zero) to the four blocks' accumulators.
  __device__ void contract() {
    if (BF16) {
      const unsigned short* th = (const unsigned short*)stage;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b >= nblk) break;
        v4u aq;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const unsigned a0 = th[(8 * gg + 2 * u) * kPitchH + 16 * b + i];
          const unsigned a1 = th[(8 * gg + 2 * u + 1) * kPitchH + 16 * b + i];
          aq[u] = a0 | (a1 << 16);
        }
        const v8bf A = __builtin_bit_cast(v8bf, aq);
        accH[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, A, accH[b], 0, 0, 0);
        if (FQ && d_exact) {
          // D = X_q - X staged as one exact bf16 piece (finish_stage): the same value the split
          // below gives (its remainders are zero), one MFMA
          const unsigned short* td = (const unsigned short*)(stage + Gm::kWords);
          v4u dq;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const unsigned d0 = td[(8 * gg + 2 * u) * kPitchH + 16 * b + i];
            const unsigned d1 = td[(8 * gg + 2 * u + 1) * kPitchH + 16 * b + i];
            dq[u] = d0 | (d1 << 16);
          }
          accP[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(v8bf, dq), accP[b], 0, 0, 0);
        } else if (ACT) {
          // d = fp32(xq - x) (relative error <= 2^-24, exact whenever the two are within 2^15 of
          // each other) is split exactly into bf16 pieces: hi = its top 8 significant bits, lo =
          // the next 8 bits of the remainder, rest = the at most 8 bits left.  rest is zero when d
          // has at most 16 significant bits (always for a fake-quant of x); its MFMA runs only on
          // the chunks where some lane has one.
          const unsigned short* tx = (const unsigned short*)(stage + (kM - 1) * Gm::kWords);
          v4u dh, dl;
          float rest[8];
          unsigned any_rest = 0u;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const unsigned x0 = tx[(8 * gg + 2 * u) * kPitchH + 16 * b + i];
            const unsigned x1 = tx[(8 * gg + 2 * u + 1) * kPitchH + 16 * b + i];
            const float d0 = bf16_lo(aq[u]) - bf16_lo(x0);
            const float d1 = bf16_hi(aq[u]) - bf16_lo(x1);
            const unsigned h0 = __float_as_uint(d0) & 0xFFFF0000u;
            const unsigned h1 = __float_as_uint(d1) & 0xFFFF0000u;
            const float l0 = d0 - __uint_as_float(h0);         // exact remainders
            const float l1 = d1 - __uint_as_float(h1);
            dh[u] = (h0 >> 16) | h1;
            dl[u] = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xFFFF0000u);
            rest[2 * u] = l0;
            rest[2 * u + 1] = l1;
            any_rest |= (__float_as_uint(l0) | __float_as_uint(l1)) & 0xFFFFu;
          }
          accP[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(v8bf, dh), accP[b], 0, 0, 0);
          accP[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(v8bf, dl), accP[b], 0, 0, 0);
          if (__builtin_amdgcn_ballot_w64(any_rest != 0u)) {
            v4u dr;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float r0 = rest[2 * u] - __uint_as_float(__float_as_uint(rest[2 * u]) & 0xFFFF0000u);
              const float r1 = rest[2 * u + 1] - __uint_as_float(__float_as_uint(rest[2 * u + 1]) & 0xFFFF0000u);
              dr[u] = (__float_as_uint(r0) >> 16) | (__float_as_uint(r1) & 0xFFFF0000u);   // exact bf16
            }
            accP[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(v8bf, dr), accP[b], 0, 0, 0);
          }
        }
      }
    } else {
      const float* tf = (const float*)stage;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b >= nblk) break;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float q = tf[(4 * s + gg) * kPitchF + 16 * b + i];
          accH[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(q, q, accH[b], 0, 0, 0);
          if (ACT) {
            const float x = ((const float*)(stage + (kM - 1) * Gm::kWords))[(4 * s + gg) * kPitchF + 16 * b + i];
            // FQ with an exact D staged: x is already q - x
            accP[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(q, (FQ && d_exact) ? x : q - x, accP[b], 0, 0, 0);
          }
        }
      }
    }
  }
};

// Rows per piece of grouped rows: about 4096 pieces over all slices (16 waves per compute unit),
// a multiple of the chunk, between 64 and 1024 rows.  Measured on MI355X at the 512-expert
// gate_up shape: 1.4-1.8% faster than 8192 pieces, 2048 and 6144 slower.
inline int64_t piece_rows(int64_t rows, int64_t nb) {
  const int64_t slices = (nb + 3) / 4;
  int64_t R = rows * slices / 4096;
  R = (R + kChunk - 1) / kChunk * kChunk;
  return R < 64 ? 64 : (R > 1024 ? 1024 : R);
}


}  // namespace stream
}  // namespace lh
