// Exhaustive E4M3 block-scale sweep with the local-Hessian objective and its diagonal (WMSE) form.
//
// For every 16-element weight block w (row c, block n of group g) and every candidate byte
// k = 0x01..0x7E: s_k = fp32(v_k * fp32(amax_g / (6*448))), q = E2M1(w / s_k) * s_k, e = q - w,
//   L_k = e^T H_n e + 2 e^T (P_n w)          (full form; "add local hessian calibration", review:
//                                             cnb,nbd,cnd->cn; "Add activation-aware local Hessian
//                                             scale calibration", review: dw = quant(w) - w and the
//                                             2 dw^T(P W0) coupling term, best_loss = inf)
//   L_k = sum_i Imp_i e_i^2                  (diagonal form; "Add WMSE weight scale search
//                                             calibration", How: cnb,nb->cn, DIAGONAL kernel)
// and the block keeps the argmin (lowest code on ties).
//
// MI355X design
//  * Full form: one wave per block column n (H_n is loaded once and kept in registers) walking 32
//    rows c; per block, 8 tiles of 16 candidates cover the 126 codes, the top two tiles first and
//    the others only where a lower bound from the column's smallest eigenvalue does not rule them
//    out (see sweep_full_column).  Lane l owns candidate l%16 of a tile and elements 4*(l/16)..+3.  The lane quantizes its 4 elements in fp32
//    (r = w * (1/s), the gfx950 FP4 convert, which rounds to nearest-even on the E2M1 grid and
//    saturates at 6, and the convert back), and forms e = fma(q, s, -w).
//  * The contraction H_n e is reorganized so the matrix cores see exact small integers:
//    (H e)_i = s (H q)_i - (H w)_i, where q holds E2M1 grid values times a power of 4 (at most
//    2 significant bits, exact in bf16).  H_n is split once per column into two bf16 pieces
//    (H1 + H2 equals H to 2^-18 relative, a residual the error bound below covers), so two
//    chained v_mfma_f32_16x16x16_bf16 (H2 q onto the accumulator input, then H1 q) give H q for
//    16 candidates with exact products and fp32 accumulation.  (One 16x16x32 instruction with K
//    slots [H1 | H2] needs q twice in its B operand, two register copies per tile.)  H w (and P w, |P||w| in the coupled form) comes from v_mfma_f32_16x16x4_f32
//    once per 16-row tile; -(H w - 2 P w)/s is the accumulator input of the H q MFMA, so its
//    result times s is H e + 2 P w.  The loss L = e^T (H e + 2 P w) is a 4-term dot per lane
//    reduced over the 4 lane groups with permlane swaps and scaled by s once; the argmin over lanes uses DPP row rotations and
//    permlane swaps.  Quantization of the next tile is issued before the current tile's MFMA
//    result is consumed.
//  * Diagonal form: VALU only (there is no contraction to map onto MFMA); a lane scores two
//    candidates of one E4M3 mantissa class over all 16 elements, whose weights are wave-uniform,
//    in the frame scaled by sqrt(Imp) (see k_sweep_diag).
//  * Exactness.  The float32 pass is a filter: each candidate carries a rigorous bound c*A_k on
//    its rounding error, with A_k >= S_e^2 + S_e S_w + 2|e|^T(|P||w|), S_e = sum_i |e_i| d_i,
//    S_w = sum_i |w_i| d_i and d_i^2 = max_j max(|H_ij|, |H_ji|) (A_k = S_e (4 S_e + S_w)
//    without P; with P the 4 S_e^2 is taken as 4 times the sum of the squared parts of S_e over
//    the four lane groups, which is >= S_e^2; the diagonal form has a bound of its own, see
//    k_sweep_diag).  Every exact
//    L_k lies in [L_k - cA_k, L_k + cA_k]; the candidates whose interval starts below the
//    lowest upper end are the only ones that can be the minimum.  If there is one, it is
//    the exact argmin; with 2 to 4 contenders the wave re-scores them in
//    float64 with exact quantization; otherwise the block's code is left at 0 and a second
//    kernel re-scores all 126 candidates in float64.  The fp32 quotient w*(1/s) can fall on the
//    wrong side of an E2M1 rounding midpoint m only when |w|/s_k is within a few ulps of m, i.e.
//    when |w|/(m g) is within a few ulps of an E4M3 value; in the full form every (element,
//    midpoint) pair of a block is tested once, and for a flagged pair the one affected candidate
//    gets the exact decision (the sign of fma(m, s_k, -|w|)) in place of its fp32 quotient.  The
//    diagonal form needs no such override (see k_sweep_diag).  A winner's nibbles are always
//    exact rounding decisions and its reported loss is evaluated again from them.  The result
//    is the argmin of the float64 objective.
//  * Options (SweepOpts): the global scale's normalization, g = fp32(amax / (6 norm)) with norm
//    448 or 256 (the "4/6" variant, "Add composable scale calibration to GPTQ"), and the
//    amax-multiplier search ("add local hessian calibration", Changes: configurable step size and
//    multipliers): a block of amax a then takes only the candidates whose code is the E4M3 value
//    nearest to a m / (6 g) for one of its multipliers m; the others score +inf before the
//    filter and the float64 passes.  Each row marks the proposed codes in a per-wave LDS table
//    tagged with the row, so a lane reads its own codes' flags.
#include "lh_internal.hpp"
#include "acc_stream.hpp"

#include <type_traits>

namespace lh {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;            // waves per workgroup; wave w takes block column 4*bx + w
constexpr int kRowsPerWave = 32;     // rows (blocks of one column) per wave
constexpr int kExactRows = 16;       // rows per wave of the float64 passes
// Filter error bound factor.  Full form: per element i the computed s y_i misses (H e + 2b)_i by
// at most d_i (S_w + S_e) 2^-18 (two-piece split of H), gamma_33 d_i (2 S_w + S_e) (fp32
// accumulation of 32 exact products onto the accumulator input, whose size is at most
// d_i S_w + 2(|P||w|)_i, in two chained instructions of 16 products each: gamma_16 for each plus
// the hand-over, at most gamma_33 of the terms' absolute sum), 2^-20 d_i S_w (H w on fp32 MFMA)
// and 2^-23 d_i S_w (the accumulator input's two roundings); weighted by |e_i| and summed, with
// the dot product's own roundings, that is at most about 2^-16.8 (S_e^2 + S_e S_w +
// 2|e|^T(|P||w|)) <= 2^-16.8 A (A_k as in the header), so 2^-16 leaves a margin of about 1.7x.
constexpr float kErrC = 0x1p-16f;
constexpr int kNearUlps = 16;        // midpoint proximity test, in ulps of |w|/(m g)

__device__ const float kMid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};

// Value of E4M3 byte k (1..126): 4 exponent bits (bias 7), 3 mantissa bits, subnormal below 2^-6.
__device__ inline double e4m3_value(int k) {
  const int e = k >> 3, m = k & 7;
  if (e == 0) return (double)m * 0x1p-9;
  return (double)(8 + m) * __longlong_as_double((long long)(e - 10 + 1023) << 52);
}

// g = fp32(amax / gdiv), gdiv = 6 * norm exact in fp32: one float64 divide rounded to fp32 is the
// correctly rounded quotient.
__device__ inline float global_scale(float amax, float gdiv) { return (float)((double)amax / (double)gdiv); }
__device__ inline float cand_scale(int k, float g) { return (float)(e4m3_value(k) * (double)g); }
__device__ inline float inv_scale(float s) { return s > 0.0f ? (float)(1.0 / (double)s) : 0.0f; }
// The float32 filter is used only where scales and quotients stay normal and finite.
__device__ inline bool filter_ok(float g) { return g >= 0x1p-100f && g <= 0x1p+100f; }

// Exact E2M1 grid index of the quotient r = |w|/s given as float64 (ties to the even index).
// |w| and m*s have at most 27 significant bits, so a float64 quotient is on the same side of
// every midpoint m as the exact one, and equal to it only when the exact quotient is.
__device__ inline int e2m1_index_exact(double r) {
  return (int)(r > 0.25) + (int)(r >= 0.75) + (int)(r > 1.25) + (int)(r >= 1.75) + (int)(r > 2.5) +
         (int)(r >= 3.5) + (int)(r > 5.0);
}
__device__ inline double e2m1_value(int c) {
  return c <= 4 ? 0.5 * c : (c == 5 ? 3.0 : (c == 6 ? 4.0 : 6.0));
}

// Exact fake-quant of one element: returns e = q - w in float64 and the nibble.
__device__ inline double exact_err(float wf, float s, int* nib) {
  const double w = (double)wf;
  int c = 0;
  if (s > 0.0f) c = e2m1_index_exact(fabs(w) / (double)s);
  const double mag = e2m1_value(c) * (double)s;
  *nib = c | (wf < 0.0f ? 8 : 0);
  return (wf < 0.0f ? -mag : mag) - w;
}

// Code (1..126) of the positive E4M3 value nearest to am / g6, ties to the even code, saturating
// at 448 and at 2^-9: the candidate a multiplier m proposes for a block of amax a (am = a m, exact
// in float64, at most 48 bits; g6 = 6 g exact, ig6 ~ 1/g6).  The float64 quotient only places y
// in its binade and between two neighbouring values j, j + 1 (it is within 2^-51 of the exact
// one, so an estimate off by one is off next to a value, far from their midpoint); the choice
// between j and j + 1 is the sign of am - (2j + 1) 2^(e-4) g6, both terms exact in float64
// (the midpoint has at most 6 significant bits, g6 at most 26).
__device__ inline int mult_code(double am, double g6, double ig6) {
  if (!(am > 0.0)) return 1;                 // zero block: every candidate is 0; lowest code
  const double y = am * ig6;
  if (!(y < 448.0)) return 126;              // saturation (also g6 == 0)
  const int e = max(ilogb(y), -6);           // value spacing 2^(e-3); subnormal below 2^-6
  const double t = ldexp(y, 3 - e);          // in [0, 16]
  int j = (int)floor(t);
  const double mid = ldexp((double)(2 * j + 1), e - 4) * g6;
  if (am > mid || (am == mid && (j & 1))) ++j;
  return min(max(((e + 7) << 3) + j - 8, 1), 126);   // code of j 2^(e-3), valid for j in [0, 16]
}

// Multiplier search: marks in mk (this wave's 128-entry table) the codes the lane's multipliers
// m0, m1 (0: none) propose for a block of amax ab, tagged with `tag` (unique per block), and
// returns whether codes k0 and k1 (0: none) are proposed.  Wave-wide: every lane must call it.
__device__ inline void mark_allowed(float ab, double g6, double ig6, float m0, float m1, int tag, int* mk,
                                   int k0, int k1, bool& a0, bool& a1) {
  if (m0 != 0.0f) mk[mult_code((double)ab * (double)m0, g6, ig6)] = tag;
  if (m1 != 0.0f) mk[mult_code((double)ab * (double)m1, g6, ig6)] = tag;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  a0 = k0 > 0 && mk[k0] == tag;
  a1 = k1 > 0 && mk[k1] == tag;
}

// The lane's two multipliers (lane and lane + 64 of the grid; 0 where the grid has none).
__device__ inline void lane_multipliers(const SweepOpts& o, int lane, float& m0, float& m1) {
  m0 = lane < o.nm ? o.mult[lane] : 0.0f;
  m1 = lane + 64 < o.nm ? o.mult[lane + 64] : 0.0f;
}

// True when |w|/s_k may lie within a few ulps of an E2M1 midpoint m for some candidate k:
// |w|/(m g) is then within a few ulps of an E4M3 value (3 significant bits).
__device__ inline bool near_midpoint(float aw, float inv_mg) {
  const float z = aw * inv_mg;
  if (!(z >= 0x1p-10f && z <= 480.0f)) return false;
  const unsigned t = (__float_as_uint(z) << 12) + ((unsigned)kNearUlps << 12);
  return t < ((unsigned)(2 * kNearUlps) << 12);
}

// For a flagged (element, midpoint m) pair with z = |w|/(m g): the candidate k whose scale puts
// |w|/s_k next to m (0 if there is none), i.e. the E4M3 value nearest z.
__device__ inline int near_candidate(float z) {
  if (z < 0x1p-6f) {
    const int m = (int)rintf(z * 512.0f);             // subnormal E4M3: m * 2^-9 (m = 8 is 2^-6)
    return (m >= 1 && m <= 8) ? m : 0;
  }
  const unsigned b = (__float_as_uint(z) + 0x80000u) & 0xFFF00000u;   // round to 3 mantissa bits
  const int e = (int)(b >> 23) - 127, mant = (int)((b >> 20) & 7u);
  const int k = ((e + 7) << 3) | mant;
  return (k >= 8 && k <= 126) ? k : 0;
}

// Quotient to hand the FP4 convert for |w| near m*s: it lands on the side of the midpoint where
// the exact quotient |w|/s lies (sign of the exactly rounded fma), or exactly on m for a true tie,
// which the convert then rounds to the even grid index like the exact rule.
__device__ inline float exact_side(float w, float m, float s) {
  const float aw = fabsf(w);
  const float d = fmaf(m, s, -aw);
  const float r = d < 0.0f ? m * 1.0009765625f : (d > 0.0f ? m * 0.9990234375f : m);
  return w < 0.0f ? -r : r;
}

// Per-lane description of this lane's flagged (element, midpoint m) pair, inv_mg = fp32(1/(m g))
// as near_midpoint used it: the affected candidate (0 if none) and the quotient to use for it.
__device__ inline void pair_override(bool near, float m, float inv_mg, float w_el, float gsc, int* kv,
                                     float* rv) {
  *kv = 0;
  *rv = 0.0f;
  if (!near) return;
  const float z = fabsf(w_el) * inv_mg;           // as near_midpoint formed it
  const int k = near_candidate(z);
  if (k == 0) return;
  *kv = k;
  *rv = exact_side(w_el, m, cand_scale(k, gsc));
}

// Apply the overrides of one ballot mask (pairs pbase + bit) to the quotients r[0..3] of a lane
// that holds candidate (16*tau + i + 1) and elements 4*gg..4*gg+3; with tau < 0 the lane's
// candidate is kmatch instead.
__device__ inline void apply_overrides(unsigned long long m, int pbase, int kv, float rv, int tau,
                                       int kmatch, int i, int gg, float r[4]) {
  while (m) {
    const int b = __builtin_ctzll(m);
    m &= m - 1;
    const int k = __builtin_amdgcn_readlane(kv, b);
    if (k == 0) continue;
    if (tau >= 0 ? (((k - 1) >> 4) != tau) : (k != kmatch)) continue;
    const int el = (b + pbase) / 7;
    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rv), b));
    const bool me = (gg == (el >> 2)) && (tau < 0 || i == ((k - 1) & 15));
    const int t = el & 3;
    r[0] = (me && t == 0) ? v : r[0];
    r[1] = (me && t == 1) ? v : r[1];
    r[2] = (me && t == 2) ? v : r[2];
    r[3] = (me && t == 3) ? v : r[3];
  }
}

// The same overrides applied to the packed FP4 codes of tile tau (elements 4*gg..4*gg+3 of the
// lane's candidate 16*tau + i + 1, nibble t at bits 4t): a flagged pair's nibble becomes the
// convert of its exact-side quotient w / s_k (scale 1, the same rounding as that quotient times
// 4^(tau-1) under the tile's power-of-4 scale).  The quotients themselves are left alone, so the
// common path and the override path read the same registers.
__device__ inline unsigned patch_overrides(unsigned long long m, int pbase, int kv, float rv, int tau,
                                           int i, int gg, unsigned pk) {
  while (m) {
    const int b = __builtin_ctzll(m);
    m &= m - 1;
    const int k = __builtin_amdgcn_readlane(kv, b);
    if (k == 0 || ((k - 1) >> 4) != tau) continue;
    const int el = (b + pbase) / 7;
    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rv), b));
    const unsigned nib = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, v, 1.0f, 0) & 0xFu;
    const unsigned sh = 4u * (unsigned)(el & 3);
    const bool me = gg == (el >> 2) && i == ((k - 1) & 15);
    pk = me ? ((pk & ~(0xFu << sh)) | (nib << sh)) : pk;
  }
  return pk;
}

// Overrides for element el of candidate kmatch (used when emitting the winner's codes).
__device__ inline float override_for(unsigned long long m, int pbase, int kv, float rv, int kmatch,
                                     int el, float r) {
  while (m) {
    const int b = __builtin_ctzll(m);
    m &= m - 1;
    const int k = __builtin_amdgcn_readlane(kv, b);
    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rv), b));
    if (k != 0 && k == kmatch && (b + pbase) / 7 == el) r = v;
  }
  return r;
}

__device__ inline float load_w(const void* W, bool bf16, int64_t idx) {
  if (bf16) return __uint_as_float((unsigned)((const unsigned short*)W)[idx] << 16);
  return ((const float*)W)[idx];
}

// Wave minima, returned wave-uniform: rotations inside each 16-lane row leave the row minimum in
// every lane, then the row broadcasts carry rows 0 and 2 into rows 1 and 3 and lane 31 into
// rows 2 and 3 (the masked-off rows take the identity), so lane 63 ends with the minimum.
template <int CTRL>
__device__ inline int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// Of a value >= 0 (or +inf): the bit patterns of such floats are ordered like unsigned
// integers, so the reduction needs no float canonicalization.
__device__ inline float wave_min_nonneg(float x) {
  unsigned v = __float_as_uint(x);
  v = min(v, (unsigned)dppi<0x128>((int)v));
  v = min(v, (unsigned)dppi<0x124>((int)v));
  v = min(v, (unsigned)dppi<0x122>((int)v));
  v = min(v, (unsigned)dppi<0x121>((int)v));
  v = min(v, (unsigned)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xA, 0xF, false));
  v = min(v, (unsigned)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xC, 0xF, false));
  return __uint_as_float((unsigned)__builtin_amdgcn_readlane((int)v, 63));
}
// Of a float that is not NaN, taken on integer keys whose signed order is the float order
// (negative values have their magnitude bits flipped).
__device__ inline int order_key(int b) { return b ^ ((b >> 31) & 0x7FFFFFFF); }   // an involution
__device__ inline float wave_min_ordered(float x) {
  int v = order_key(__float_as_int(x));
  v = min(v, dppi<0x128>(v));
  v = min(v, dppi<0x124>(v));
  v = min(v, dppi<0x122>(v));
  v = min(v, dppi<0x121>(v));
  v = min(v, __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0x142, 0xA, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0x143, 0xC, 0xF, false));
  return __int_as_float(order_key(__builtin_amdgcn_readlane(v, 63)));
}
// Lowest (loss, code) over the wave in float64 (exact re-scoring).
__device__ inline void wave_argmin_d(double& L, int& k) {
  for (int o = 1; o < 64; o <<= 1) {
    const double oL = __shfl_xor(L, o, 64);
    const int oK = __shfl_xor(k, o, 64);
    if (oL < L || (oL == L && oK < k)) { L = oL; k = oK; }
  }
}

// Sums each of p[0..3] over the 4 rows (16-lane groups) of the wave and leaves the total of p[r]
// in row r.
__device__ inline float quad_sum(const float p[4]) {
  auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
  const float s02 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
  const float s13 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// Issue priority by progress.  The SIMD's arbiter favours the oldest wave, so waves that share
// a SIMD and carry the same work finish far apart and the last one runs alone, which one wave
// cannot keep busy.  A wave that has done less of its rows gets a higher priority, so the waves
// on a SIMD advance together: 3 for the first half, 2 to three quarters, 1 to fifteen
// sixteenths, 0 for the rest.  Within one level the oldest wave still goes first; the geometric
// steps leave only the last sixteenth to that order, and a wave that runs ahead drops a level
// and waits for the others.
__device__ inline void wave_priority_by_progress(int done, int total) {
  if (16 * done % total >= 16) return;            // only where a sixteenth begins
  const int q = 16 * done / total;
  if (q == 0) __builtin_amdgcn_s_setprio(3);
  else if (q == 8) __builtin_amdgcn_s_setprio(2);
  else if (q == 12) __builtin_amdgcn_s_setprio(1);
  else if (q == 15) __builtin_amdgcn_s_setprio(0);
}

// ------------------------------------------------------------------------------------------
// Full-Hessian sweep: float32 filter
// ------------------------------------------------------------------------------------------
struct FullLds {
  float H[256];
  float P[256];
  float w[16][16];     // current 16-row tile: w[row][elem]
  float g[16][16];     // (H w - 2 P w)[row][elem]
  float pw[16][16];    // bound weights d S_w + 2 |P||w| [row][elem] (coupled form)
  float sw[16];        // S_w = sum_j d_j |w_j| per row
  float b[16][16];     // (P w)[row][elem]           } the loss of the tile's
  float ws[16];        // winner's scale per row      } filter-decided winners
  float wi[16];        // winner's 1/scale per row    }
  int kw[16];          // winner's code per row       }
  unsigned short wn[16][4];   // winner's signed nibbles per row and lane group (override rows)
  double ex[4][16];    // float64 refinement: e of up to 4 contenders
  float ab[16];        // block amax per row of the tile (multiplier search)
  float lb96[16];      // LB_96 and LB_64 per row of the tile (-inf: no bound)
  float lb64[16];
  int mk[128];         // codes proposed by the multipliers, tagged with the row
};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// bf16 round-to-nearest-even of a finite float, as bits in the low half.
__device__ inline unsigned bf16_rne(float x) {
  const unsigned b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
__device__ inline float bf16_val(unsigned h) { return __uint_as_float(h << 16); }

// Sum over the 4 rows of the wave, result in every lane.
__device__ inline float group_sum(float v) {
  auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}
// Maximum of a value >= 0 over the wave, wave-uniform (bit patterns of such floats order like
// unsigned integers).
__device__ inline float wave_max_nonneg(float x) {
  unsigned v = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max(a[0], a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(b[0], b[1]);
  v = max(v, (unsigned)dppi<0x128>((int)v));
  v = max(v, (unsigned)dppi<0x124>((int)v));
  v = max(v, (unsigned)dppi<0x122>((int)v));
  v = max(v, (unsigned)dppi<0x121>((int)v));
  return __uint_as_float((unsigned)__builtin_amdgcn_readfirstlane((int)v));
}

// Lane group gg's Cholesky test of A = S - m I (S in registers, lane i holding row i; the column
// being eliminated passes through the 16 floats of LDS at cbuf + 16 gg): true when every pivot is
// positive.
__device__ __attribute__((always_inline)) inline bool chol_positive(const float (&srow)[16], float m, int i,
                                                                     int gg, float* cbuf) {
  float a[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) a[k] = k == i ? srow[k] - m : srow[k];
  bool ok = true;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    cbuf[16 * gg + i] = a[j];                        // column j of the reduced matrix
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float piv = cbuf[16 * gg + j];
    ok = ok && piv > 0.0f;
    const float isr = __builtin_amdgcn_rsqf(fmaxf(piv, 0x1p-100f));
    const float li = a[j] * isr;
#pragma unroll
    for (int k = j + 1; k < 16; ++k) a[k] = fmaf(-li, cbuf[16 * gg + k] * isr, a[k]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  return ok;
}

// A lower bound mu of the smallest eigenvalue of S = (H + H^T)/2 for a column's Hessian H (16x16
// row-major in LDS), the same value in every lane: every e then has e^T H e = e^T S e >= mu |e|^2.  S is scaled by a power of two to max |S_ij| in [1/2, 1).  If a float32 Cholesky
// factorization of S - m I completes with positive pivots, R^T R = S - m I + E with
// |E_ij| <= gamma_17 (|R^T||R|)_ij (the standard backward error of Cholesky, here with unit
// roundoff 2^-22 for the reciprocal square root and product), and (|R^T||R|)_ij <=
// sqrt((R^T R)_ii (R^T R)_jj) <= 1.01, so the 2-norm of E is below 16 * 17 * 2^-22 * 1.01 <
// 2^-13.8; with the roundings of S's entries (2^-20 in norm) the smallest eigenvalue of S is at
// least m - 2^-13.7.  The four lane groups test four values of m at a time, below d, the smallest
// diagonal entry (which bounds the smallest eigenvalue from above): d 2^-2, 2^-6, 2^-10, 2^-14,
// then the three doublings of the largest that passed.  When none passes (or d <= 0: a singular
// or nearly singular S), they test the negative shifts m = -2^-14, -2^-12, -2^-10, -2^-8, for which
// the same argument holds (the diagonal of S - m I stays below 1.004).  mu is the largest m that
// passed less 2^-12, scaled back: S - mu I is positive semidefinite, and mu can be <= 0.  No
// passing m, or non-finite H, gives -inf (no bound).  A column of zero trace is scored as H = I:
// mu = 1.  Inlined where the caller's LDS arrays are visible, so its LDS accesses are LDS
// instructions rather than generic ones.
__device__ __attribute__((always_inline)) inline float column_mu(const float* Hs, bool dead, int lane,
                                                                     float* cbuf) {
  if (dead) return 1.0f;
  const int i = lane & 15, gg = lane >> 4;
  float a[16];
  float mx = 0.0f;
  bool fin = true;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    a[k] = 0.5f * Hs[i * 16 + k] + 0.5f * Hs[k * 16 + i];
    fin = fin && fabsf(a[k]) <= 0x1.fffffep127f;     // false for inf and NaN
    mx = fmaxf(mx, fabsf(a[k]));
  }
  if (__ballot(!fin)) return -__builtin_inff();
  mx = wave_max_nonneg(mx);
  if (!(mx > 0.0f)) return -__builtin_inff();
  const int ex = __builtin_amdgcn_frexp_expf(mx);   // mx = f 2^ex, f in [1/2, 1)
#pragma unroll
  for (int k = 0; k < 16; ++k) a[k] = __builtin_amdgcn_ldexpf(a[k], -ex);
  float di = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) di = k == i ? a[k] : di;
  const float d = wave_min_ordered(di);
  int e1 = 0;                                        // exponent of the largest m that passed
  unsigned long long okm = 0ull;
  if (d > 0.0f) {
    // round 1: m = d 2^-(4 gg + 2)
    okm = __ballot(chol_positive(a, __builtin_amdgcn_ldexpf(d, -(4 * gg + 2)), i, gg, cbuf));
#pragma unroll
    for (int q = 3; q >= 0; --q)
      if ((okm >> (16 * q)) & 1ull) e1 = -(4 * q + 2);
  }
  if (e1 == 0) {
    // negative shifts m = -2^(2 gg - 14); the least negative that passes
    okm = __ballot(chol_positive(a, -__builtin_amdgcn_ldexpf(1.0f, 2 * gg - 14), i, gg, cbuf));
    if (okm == 0ull) return -__builtin_inff();
    const int q = (int)__builtin_ctzll(okm) >> 4;
    return __builtin_amdgcn_ldexpf(-__builtin_amdgcn_ldexpf(1.0f, 2 * q - 14) - 0x1p-12f, ex);
  }
  // round 2: m = d 2^(e1 + 1 + gg) for gg < 3 (group 3 repeats the passed value)
  const int e2 = gg < 3 ? e1 + 1 + gg : e1;
  okm = __ballot(e2 <= -1 && chol_positive(a, __builtin_amdgcn_ldexpf(d, e2), i, gg, cbuf));
  int eb = e1;
#pragma unroll
  for (int q = 0; q < 3; ++q)
    if ((okm >> (16 * q)) & 1ull) eb = e1 + 1 + q;
  return __builtin_amdgcn_ldexpf(__builtin_amdgcn_ldexpf(d, eb) - 0x1p-12f, ex);
}

// Float64 re-scoring of one block by a whole wave: lane l scores codes l + 1 and l + 65 (those
// with al0 / al1 set) with exact quantization, and the winner's code, nibbles and loss are written
// to code_p, fp4_p (the block's 8 bytes, or NULL) and loss_p (or NULL).  Hs, Ps (16x16 row-major)
// and ws (16 weights) are in LDS; bs is 16 doubles of LDS scratch for P w.  dead: the block's H
// has zero trace and is scored as H = I without the cross term.
template <bool COUPLED>
__device__ inline void exact_block(const float* Hs, const float* Ps,
                                   const float* ws, double* bs, bool dead,
                                   float gsc, bool al0, bool al1, int lane, uint8_t* code_p, uint8_t* fp4_p,
                                   float* loss_p) {
  const bool coupled = COUPLED && !dead;
  if (lane < 16) {
    double acc = 0.0;
    if (coupled)
      for (int j = 0; j < 16; ++j) acc += (double)Ps[lane * 16 + j] * (double)ws[j];
    bs[lane] = acc;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  double best = __builtin_inf();
  int bestK = 1 << 20;
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    const int k = lane + 1 + 64 * h;
    if (k > 126 || !(h == 0 ? al0 : al1)) continue;
    const float sk = cand_scale(k, gsc);
    double e[16], er[16];
    int nib;
#pragma unroll
    for (int j = 0; j < 16; ++j) er[j] = e[j] = exact_err(ws[j], sk, &nib);
    // L = sum_r e_r ((H e)_r + 2 b_r), one row of H per step; er turns so that er[0] = e_r
    // (a rolled loop keeps the register count low: this path is rare)
    double Ls = 0.0;
#pragma unroll 1
    for (int r2 = 0; r2 < 16; ++r2) {
      double y = 0.0;
      if (dead) {
        y = er[0];
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) y += (double)Hs[r2 * 16 + j] * e[j];
      }
      Ls += er[0] * (y + 2.0 * bs[r2]);
#pragma unroll
      for (int j = 0; j < 15; ++j) er[j] = er[j + 1];
    }
    if (Ls < best) { best = Ls; bestK = k; }
  }
  wave_argmin_d(best, bestK);
  const float sw = cand_scale(bestK, gsc);
  if (lane < 8 && fp4_p) {
    int lo, hi;
    exact_err(ws[2 * lane], sw, &lo);
    exact_err(ws[2 * lane + 1], sw, &hi);
    fp4_p[lane] = (uint8_t)(lo | (hi << 4));
  }
  if (lane == 0) {
    *code_p = (uint8_t)bestK;
    if (loss_p) *loss_p = (float)best;
  }
  __builtin_amdgcn_wave_barrier();
}

// The full-Hessian float32 filter over rows [c_begin, c_end) of block column n of group g by one
// wave, with H_n (and P_n) already in L.H (and L.P).  Blocks the filter cannot decide get code 0
// and are left to k_sweep_full_exact, or with RECORD are marked in the wave's LDS bit array `undec_bits`
// (bit c - c_begin) for the caller to re-score in float64 (the fused accumulate-and-sweep kernel,
// which keeps H in LDS only).  EQUALIZE: wave priority by progress (short launches, see
// wave_priority_by_progress).
template <bool BF16, bool COUPLED, bool EQUALIZE, bool RECORD, bool MSEARCH>
__device__ inline void sweep_full_column(FullLds& L, const void* __restrict__ W, int64_t cout, int64_t cin,
                                         int64_t g, int64_t n, int64_t c_begin, int64_t c_end, float gsc,
                                         uint8_t* __restrict__ code, uint8_t* __restrict__ fp4,
                                         float* __restrict__ loss, int rows_per_wave, const SweepOpts& opt,
                                         const float* mu_col, unsigned* undec_bits = nullptr) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, gg = lane >> 4;
  const int64_t nb = cin / 16;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  double tr = 0.0;
  for (int j = 0; j < 16; ++j) tr += (double)L.H[j * 17];
  const bool dead = (tr == 0.0);                   // no activation energy: plain weight MSE
  const bool coupled = COUPLED && !dead;
  // Lane (row i, group gg) holds, for elements col = 4*gg + t:
  //   a[t]   = H[i][col] in fp32 (H w per 16-row tile), pv/pa = P and |P| (P w, |P||w|)
  //   h1, h2 = H[i][col] split into two bf16 pieces, |H - H1 - H2| <= 2^-18 |H|: A operand of
  //            the bf16 MFMA that forms H q for the candidates
  //   dm[t]  = d_col = sqrt(max_j max(|H_col,j|, |H_j,col|)), so |H_ij| <= d_i d_j for any H
  //            (2 d_col in the coupled form)
  float a[4], dm[4], pa[4], pv[4];
  unsigned h1[4], h2[4];
  float hpmax = 0.0f;                               // max |H_ij|, |P_ij| of the column
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int col = 4 * gg + t;
    a[t] = dead ? (i == col ? 1.0f : 0.0f) : L.H[i * 16 + col];
    h1[t] = bf16_rne(a[t]);
    const float r1 = a[t] - bf16_val(h1[t]);      // exact
    h2[t] = bf16_rne(r1);
    float mx = 1.0f;
    if (!dead) {
      mx = 0.0f;
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fmaxf(fabsf(L.H[col * 16 + j]), fabsf(L.H[j * 16 + col])));
    }
    dm[t] = sqrtf(mx) * (COUPLED ? 2.0000004f : 1.0000002f);   // (2x when coupled) with sqrt margin
    pv[t] = coupled ? L.P[i * 16 + col] : 0.0f;
    pa[t] = fabsf(pv[t]);
    hpmax = fmaxf(hpmax, fmaxf(mx, pa[t]));
  }
  // two chained 16x16x16 bf16 MFMAs per tile: H2 q onto the accumulator input, then H1 q
  const v2u A1u = {h1[0] | (h1[1] << 16), h1[2] | (h1[3] << 16)};
  const v2u A2u = {h2[0] | (h2[1] << 16), h2[2] | (h2[3] << 16)};
  const v4s A1 = __builtin_bit_cast(v4s, A1u), A2 = __builtin_bit_cast(v4s, A2u);

  // ---- candidate scales.  Tile tau holds codes 16*tau + i + 1.  Tile 0 (codes 1..16) uses
  // s0/is0 directly.  For tau >= 1 the lane's codes share one E4M3 mantissa and step the exponent
  // by 2 per tile, so s_k = s1 * 4^(tau-1) and 1/s_k = is1 * 4^-(tau-1) exactly (normal range):
  // the lane forms w * is1 once per block and the FP4 converts apply the power of 4 through their
  // exponent-only scale operand (on the way in and out), which is exact.  Codes 127 and 128
  // (tile 7, i >= 14) do not exist and are masked.
  // The filter's fp32 values stay finite and normal-range for every candidate when |H|, |P| <=
  // 2^100 and g^2 max(|H|, |P|) <= 2^76 (quotients |w|/s <= 2^20.4, |e| <= 2^12.4 g, 16 terms);
  // other columns go to the float64 pass whole.
  const float hpm = wave_max_nonneg(hpmax);
  // multiplier search (its own instantiation, so the plain sweep keeps its registers): the lane's
  // multipliers and the float64 6g, 1/(6g)
  constexpr bool msearch = MSEARCH;
  float mu0 = 0.0f, mu1 = 0.0f;
  double g6 = 0.0, ig6 = 0.0;
  if (msearch) {
    lane_multipliers(opt, lane, mu0, mu1);
    L.mk[lane] = -1;
    L.mk[lane + 64] = -1;
    g6 = 6.0 * (double)gsc;
    ig6 = 1.0 / g6;
  }
  const bool fast = filter_ok(gsc) && hpm <= 0x1p100f && (double)gsc * (double)gsc * (double)hpm <= 0x1p76;
  const float s0 = cand_scale(i + 1, gsc), is0 = inv_scale(s0);
  const float s1 = cand_scale(i + 17, gsc), is1 = inv_scale(s1);
  // midpoint proximity: this lane tests pairs p = lane and lane + 64 of (element, midpoint)
  const int p0 = lane, p1 = lane + 64;
  const float mid0 = kMid[p0 % 7], mid1 = kMid[(p1 < 112 ? p1 : 0) % 7];
  const float img0 = fast ? (float)(1.0 / ((double)mid0 * (double)gsc)) : 0.0f;
  const float img1 = (fast && p1 < 112) ? (float)(1.0 / ((double)mid1 * (double)gsc)) : 0.0f;
  const float sl0 = gg == 0 ? s0 : s1;             // scale of tile gg (first half of the tiles)
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  // Codes 97..126 (tiles 6, 7) are scored first, codes 65..96 (tiles 4, 5) only when the bound
  // below does not rule them out for K = 96, and codes 1..64 only when it does not for K = 64 once
  // codes 65..96 are scored: for k <= K every element keeps an error |e_i| >= |w_i| - 6 s_k >=
  // |w_i| - 6 s_K whatever its FP4 value (at most 6), so with mu <= the smallest eigenvalue of the
  // column's (symmetrized) Hessian, L_k >= mu sum_i (|w_i| - 6 s_K)_+^2 =: LB_K (and
  // L_k >= c (mu c - 2|b|) with c^2 = that sum, b = P w, when mu c >= |b|, in the coupled form).
  // LB_K > U (the lowest upper end among the codes scored, at least their exact minimum) means no
  // code <= K is or ties the argmin.  The multiplier search scores all codes.
  constexpr bool kWindow = !MSEARCH;
  // (the plain sweep always receives mu_col from k_column_mu; the fused kernel forms it here)
  float mu = -__builtin_inff();                   // no bound
  if (kWindow && fast) {
    if constexpr (RECORD) mu = column_mu(L.H, dead, lane, &L.g[0][0]);
    else mu = *mu_col;
  }
  const float s64 = cand_scale(64, gsc), s96 = cand_scale(96, gsc);
  // In the uncoupled form (the COUPLED kernels keep the bound above) a second bound needs only mu > -inf (S - mu I positive semidefinite):
  // for k <= K the block's FP4 values q (e = q - w) have |q_i| <= tau = 6 s_K, so in the seminorm
  // of S - mu I the triangle inequality and |q^T A q| <= tau^2 sum |A_ij| give
  //   L_k >= (sqrt(w^T H w - mu |w|^2) - tau sqrt(sum |H_ij| + 16 |mu|))_+^2 + mu_term,
  // mu_term = mu sum_i (|w_i| - tau)_+^2 (mu >= 0) or mu (|w| + 4 tau)^2 (mu < 0), which decides
  // most rows of near-singular Hessians (experts with few routed tokens).  habs >= sum |H_ij|.
  const bool tri_ok = kWindow && !COUPLED && mu > -__builtin_inff();
  float habs = 0.0f;
  if (tri_ok) {
    float hp = fabsf(a[0]) + fabsf(a[1]) + fabsf(a[2]) + fabsf(a[3]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) hp += __shfl_xor(hp, o, 64);
    habs = group_sum(hp) * (1.0f + 0x1p-17f);     // 64 terms: rounded up
  }

  for (int64_t c0 = c_begin; c0 < c_end; c0 += 16) {
    // ---- 16-row tile: w, H w, P w and |P||w| (fp32 MFMA, K index = element 4*gg + t)
    const int64_t crow = c0 + i;
    const bool row_on = crow < c_end;
    float wt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)   // + 0 turns -0 into +0, so the FP4 converts' sign bit is (w < 0)
      wt[t] = row_on ? load_w(W, BF16, (g * cout + crow) * cin + n * 16 + 4 * gg + t) + 0.0f : 0.0f;
    v4f hw = zero4, bt = zero4, pwt = zero4;
#pragma unroll
    for (int t = 0; t < 4; ++t) hw = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], wt[t], hw, 0, 0, 0);
    if (coupled) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bt = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[t], wt[t], bt, 0, 0, 0);
        pwt = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[t], fabsf(wt[t]), pwt, 0, 0, 0);
      }
    }
    // S_w of row i (rounded up; the coupled form's dm carries 2 d)
    float swt = fabsf(wt[0]) * dm[0];
    swt = fmaf(fabsf(wt[1]), dm[1], swt);
    swt = fmaf(fabsf(wt[2]), dm[2], swt);
    swt = fmaf(fabsf(wt[3]), dm[3], swt);
    const float swr = group_sum(swt) * (COUPLED ? 0.50000025f : 1.0000005f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < 4; ++t) {                  // lane holds elements 4gg+t of row i
      L.w[i][4 * gg + t] = wt[t];
      L.g[i][4 * gg + t] = coupled ? fmaf(-2.0f, bt[t], hw[t]) : hw[t];
      if (COUPLED) {
        // weight of |e_t| in the linear part of the bound: d_t S_w + 2 (|P||w|)_t
        L.pw[i][4 * gg + t] = fmaf(dm[t], 0.5f * swr, coupled ? 2.0f * pwt[t] : 0.0f);
        L.b[i][4 * gg + t] = bt[t];
      }
    }
    if (gg == 0) L.sw[i] = swr;
    if (kWindow) {
      // LB_96 and LB_64 of row i (see the column set-up) from the lane's 4 elements of row i;
      // -inf where there is no bound
      float lb96 = -__builtin_inff(), lb64 = -__builtin_inff();
      if (mu > -__builtin_inff()) {
        float c96p = 0.0f, c64p = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float d96 = fmaxf(fmaf(-6.0f, s96, fabsf(wt[t])), 0.0f);   // one rounding of |w| - 6 s_K
          const float d64 = fmaxf(fmaf(-6.0f, s64, fabsf(wt[t])), 0.0f);
          c96p = fmaf(d96, d96, c96p);
          c64p = fmaf(d64, d64, c64p);
        }
        const float c96 = group_sum(c96p) * (1.0f - 0x1p-18f);   // rounded down (7 roundings < 2^-21)
        const float c64 = group_sum(c64p) * (1.0f - 0x1p-18f);
        if (mu > 0.0f) {
          lb96 = mu * c96 * (1.0f - 0x1p-22f);
          lb64 = mu * c64 * (1.0f - 0x1p-22f);
        }
        if (coupled && mu > 0.0f) {
          // |b_i| <= |fp32 (P w)_i| + 2^-20 (|P||w|)_i, and om_i >= 2 (|P||w|)_i
          float bp = 0.0f;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float om = fmaf(dm[t], 0.5f * swr, 2.0f * pwt[t]);
            const float bb = fmaf(0x1p-19f, om, fabsf(bt[t]));
            bp = fmaf(bb, bb, bp);
          }
          const float bn = sqrtf(group_sum(bp)) * (1.0f + 0x1p-17f);     // >= |b|
          auto lbc = [&](float c2) -> float {
            const float cd = sqrtf(c2) * (1.0f - 0x1p-20f);               // <= c
            const float tm = fmaf(mu, cd, -2.0f * bn);
            return (mu * cd >= bn * (1.0f + 0x1p-20f) && tm > 0.0f) ? cd * tm * (1.0f - 0x1p-20f)
                                                                     : -__builtin_inff();
          };
          lb96 = lbc(c96);
          lb64 = lbc(c64);
        }
        if (tri_ok) {
          // w^T H w from the fp32 H w of the tile: |w^T H w - sum w_i (H w)_i| <= 2^-18 S_w^2
          // (2^-20 S_w^2 from H w, the 16-term sum's roundings below 2^-21 S_w^2)
          float whp = 0.0f, wwp = 0.0f;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            whp = fmaf(wt[t], hw[t], whp);
            wwp = fmaf(wt[t], wt[t], wwp);
          }
          const float whw = group_sum(whp) - 0x1p-18f * swr * swr;        // <= w^T H w (rounding aside)
          const float ww = group_sum(wwp);                                 // |w|^2 within 2^-21
          // whw - mu |w|^2, rounded down: mu |w|^2 taken 2^-20 larger (mu > 0) or smaller (mu < 0)
          const float pw = (whw - mu * ww * (mu > 0.0f ? 1.0f + 0x1p-20f : 1.0f - 0x1p-20f)) *
                           (1.0f - 0x1p-20f) - 0x1p-22f * fabsf(whw);
          const float hq = sqrtf(habs + 16.0f * fabsf(mu)) * (1.0f + 0x1p-20f);
          auto lbt = [&](float sK, float c2) -> float {
            const float tau = 6.0f * sK * (1.0f + 0x1p-22f);                // >= 6 s_K
            const float tq = tau * hq * (1.0f + 0x1p-22f);
            const float rt = sqrtf(fmaxf(pw, 0.0f)) * (1.0f - 0x1p-20f);
            const float tv = (rt - tq) - 0x1p-22f * rt;                     // rounded down
            const float t2 = tv > 0.0f ? tv * tv * (1.0f - 0x1p-21f) : 0.0f;
            float mt;                                                       // mu_term, rounded down
            if (mu >= 0.0f) {
              mt = mu * c2 * (1.0f - 0x1p-22f);
            } else {
              const float en = (sqrtf(ww) * (1.0f + 0x1p-20f) + 4.0f * tau) * (1.0f + 0x1p-22f);
              mt = mu * en * en * (1.0f + 0x1p-20f);
            }
            return (t2 + mt) - 0x1p-22f * (t2 + fabsf(mt));
          };
          lb96 = fmaxf(lb96, lbt(s96, c96));
          lb64 = fmaxf(lb64, lbt(s64, c64));
        }
      }
      if (gg == 0) {
        L.lb96[i] = lb96;
        L.lb64[i] = lb64;
      }
    }
    if (msearch) {
      // block amax of row i: the lane's 4 elements, then the 4 lane groups
      unsigned am = max(max(__float_as_uint(fabsf(wt[0])), __float_as_uint(fabsf(wt[1]))),
                        max(__float_as_uint(fabsf(wt[2])), __float_as_uint(fabsf(wt[3]))));
      auto x = __builtin_amdgcn_permlane32_swap(am, am, false, false);
      am = max(x[0], x[1]);
      auto y = __builtin_amdgcn_permlane16_swap(am, am, false, false);
      am = max(y[0], y[1]);
      if (gg == 0) L.ab[i] = __uint_as_float(am);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    const int rows_here = (int)min((int64_t)16, c_end - c0);
    unsigned batched = 0u;   // rows whose unique winner is emitted by the per-tile pass below
    unsigned emitted = 0u;   // rows with midpoint overrides, emitted at once (loss per tile)
    unsigned undec = 0u;     // rows the filter leaves undecided (RECORD)
    for (int rr = 0; rr < rows_here; ++rr) {
      const int64_t c = c0 + rr;
      const int64_t oblk = (g * cout + c) * nb + n;
      if constexpr (EQUALIZE) wave_priority_by_progress((int)(c - c_begin), rows_per_wave);
      float w[4], gq[4], om[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w[t] = L.w[rr][4 * gg + t];
        gq[t] = L.g[rr][4 * gg + t];
        om[t] = COUPLED ? L.pw[rr][4 * gg + t] : 0.0f;
      }
      const float S_w = L.sw[rr];

      // quotients within a few ulps of an E2M1 midpoint are decided exactly (fma sign test)
      const float wp0 = L.w[rr][p0 / 7], wp1 = L.w[rr][(p1 < 112 ? p1 : 0) / 7];
      const bool near0 = near_midpoint(fabsf(wp0), img0);
      const bool near1 = p1 < 112 && near_midpoint(fabsf(wp1), img1);
      const unsigned long long m0 = __ballot(near0), m1 = __ballot(near1);
      if (!fast) {
        if (RECORD) undec |= 1u << rr;
        else if (lane == 0) code[oblk] = 0;         // resolved by the float64 pass
        continue;
      }
      const bool has_ovr = (m0 | m1) != 0ull;
      int kv0 = 0, kv1 = 0;
      float rv0 = 0.0f, rv1 = 0.0f;
      unsigned tile_hit = 0u;                        // bit tau: some override falls in tile tau
      if (has_ovr) {
        pair_override(near0, mid0, img0, wp0, gsc, &kv0, &rv0);
        pair_override(near1, mid1, img1, wp1, gsc, &kv1, &rv1);
        for (unsigned long long m = m0; m; m &= m - 1) {
          const int k = __builtin_amdgcn_readlane(kv0, (int)__builtin_ctzll(m));
          if (k != 0) tile_hit |= 1u << ((k - 1) >> 4);
        }
        for (unsigned long long m = m1; m; m &= m - 1) {
          const int k = __builtin_amdgcn_readlane(kv1, (int)__builtin_ctzll(m));
          if (k != 0) tile_hit |= 1u << ((k - 1) >> 4);
        }
      }
      // w / s for this lane's tile-0 and tile-1 codes, and the accumulator inputs -(H w - 2 P w)_i / s
      // of tile 0 and of tiles 1..7 (which share s1); the tile-0 values are formed only when codes
      // 1..64 are scored
      float ra[4], rb[4];
      v4f cacc0, cacc1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        rb[t] = w[t] * is1;
        cacc1[t] = -gq[t] * is1;
      }
      auto tile0_inputs = [&]() {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          ra[t] = w[t] * is0;
          cacc0[t] = -gq[t] * is0;
        }
      };

      // Scoring of tile tau (16 codes): quotients (with exact overrides) -> FP4 round trip
      // q' = q * 4^(tau-1) (exact in bf16), e = fma(q', s, -w), y = H q' - (H w - 2b)/s on bf16
      // MFMA (H in two pieces, products exact, fp32 accumulation onto the accumulator input), so
      // (H e + 2b)_i = s y_i and L = s sum_i e_i y_i, with s applied once after the sum over the
      // lane groups.  Instantiated twice so the common case has no override code.
      // NT = 4 scores tiles T0..T0+3 and leaves tile T0 + r in lane group r; NT = 2 scores tiles
      // T0, T0+1 and leaves tile T0 + (r & 1) in lane group r (the quad sum of {T0, T0+1, T0,
      // T0+1}), so with T0 = 4 q + 2 h the lane groups 2h, 2h+1 hold them in the quad's layout.
      unsigned pkc = 0u;
      auto score_quad = [&](auto ovr_tag, auto t0_tag, auto nt_tag, float& Lo, float& Ao) {
        constexpr bool OVR = decltype(ovr_tag)::value;
        constexpr int T0 = decltype(t0_tag)::value;
        constexpr int NT = decltype(nt_tag)::value;
        static_assert((NT == 4 && T0 % 4 == 0) || (NT == 2 && T0 % 2 == 0), "tile group");
        auto tile_err = [&](int tau, float e[4], unsigned& p01, unsigned& p23) {
          const float sc = tau == 0 ? 1.0f : (float)(1u << (2 * (tau - 1)));   // 4^(tau-1)
          const float* r = tau == 0 ? ra : rb;
          // bytes 0 and 1 of the pack register are written and read; its other bytes never
          // are, so the register carried from the previous tile serves as the old value
          pkc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pkc, r[0], r[1], sc, 0);
          pkc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pkc, r[2], r[3], sc, 1);
          if (OVR && ((tile_hit >> tau) & 1u)) {      // exact decisions replace their nibbles
            pkc = patch_overrides(m0, 0, kv0, rv0, tau, i, gg, pkc);
            pkc = patch_overrides(m1, 64, kv1, rv1, tau, i, gg, pkc);
          }
          const unsigned pk = pkc;
          const v2f q01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, sc, 0);
          const v2f q23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, sc, 1);
          const float sb = tau == 0 ? s0 : s1;
          e[0] = fmaf(q01[0], sb, -w[0]);
          e[1] = fmaf(q01[1], sb, -w[1]);
          e[2] = fmaf(q23[0], sb, -w[2]);
          e[3] = fmaf(q23[1], sb, -w[3]);
          // q' has at most 2 significant bits: its bf16 is the top half of the float
          p01 = __builtin_amdgcn_perm(__float_as_uint(q01[1]), __float_as_uint(q01[0]), 0x07060302u);
          p23 = __builtin_amdgcn_perm(__float_as_uint(q23[1]), __float_as_uint(q23[0]), 0x07060302u);
        };
        float e[4], en[4];
        unsigned p01, p23, pn01 = 0, pn23 = 0;
        tile_err(T0, e, p01, p23);
        {
          float pl[4], pa4[4];
#pragma unroll
          for (int u = 0; u < NT; ++u) {
            const int tau = T0 + u;
            const v2u Bu = {p01, p23};
            const v4s B = __builtin_bit_cast(v4s, Bu);
            const v4f y = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                A1, B, __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A2, B, tau == 0 ? cacc0 : cacc1, 0, 0, 0), 0, 0, 0);
            if (u < NT - 1) tile_err(tau + 1, en, pn01, pn23);      // overlaps the MFMAs
            // bound: uncoupled, this lane's part of S_e = sum_i d_i |e_i| (A follows after the
            // group sum); coupled, (2 S_e,g)^2 + sum_i |e_i| om_i over the lane's 4 elements,
            // whose sum over the 4 groups is >= S_e^2 + S_e S_w + 2|e|^T(|P||w|) (Cauchy-Schwarz)
            float sp = fabsf(e[0]) * dm[0];
            sp = fmaf(fabsf(e[1]), dm[1], sp);
            sp = fmaf(fabsf(e[2]), dm[2], sp);
            sp = fmaf(fabsf(e[3]), dm[3], sp);
            float ap = sp;
            if (COUPLED) {
              float tp = fabsf(e[0]) * om[0];
              tp = fmaf(fabsf(e[1]), om[1], tp);
              tp = fmaf(fabsf(e[2]), om[2], tp);
              tp = fmaf(fabsf(e[3]), om[3], tp);
              ap = fmaf(sp, sp, tp);
            }
            float lp = e[0] * y[0];
            lp = fmaf(e[1], y[1], lp);
            lp = fmaf(e[2], y[2], lp);
            lp = fmaf(e[3], y[3], lp);
            pl[u] = lp;
            pa4[u] = ap;
            if (u < NT - 1) {
#pragma unroll
              for (int t = 0; t < 4; ++t) e[t] = en[t];
              p01 = pn01;
              p23 = pn23;
            }
          }
          if (NT == 2) {
            pl[2] = pl[0];
            pl[3] = pl[1];
            pa4[2] = pa4[0];
            pa4[3] = pa4[1];
          }
          Lo = quad_sum(pl) * (T0 == 0 ? sl0 : s1);     // tiles >= 1 share the scale s1
          Ao = quad_sum(pa4);
          if (!COUPLED) Ao *= fmaf(4.0f, Ao, S_w);       // A = S_e (4 S_e + S_w)
        }
      };
      auto score = [&](auto t0_tag, auto nt_tag, float& Lo, float& Ao) {
        if (has_ovr) score_quad(std::true_type{}, t0_tag, nt_tag, Lo, Ao);
        else score_quad(std::false_type{}, t0_tag, nt_tag, Lo, Ao);
      };
      using I0 = std::integral_constant<int, 0>;
      using I2 = std::integral_constant<int, 2>;
      using I4 = std::integral_constant<int, 4>;
      using I6 = std::integral_constant<int, 6>;
      // lane l holds codes l + 1 (tiles 0..3) and l + 65 (tiles 4..7); 127 and 128 do not exist
      float Lq[2], Aq[2];
      float U1 = 0.0f;
      bool win = false;
      if (kWindow) {
        score(I6{}, I2{}, Lq[1], Aq[1]);             // codes 97..126 in lanes 32..61
        if (lane < 32 || lane >= 62) Lq[1] = __builtin_inff();
        U1 = wave_min_ordered(fmaf(kErrC, Aq[1], Lq[1]));
        win = L.lb96[rr] > U1;                         // LB_96, LB_64 of the row are in L
        if (!win) {
          float L45, A45;                              // codes 65..96 in lanes 0..31 (and again in 32..63)
          score(I4{}, I2{}, L45, A45);
          U1 = fminf(U1, wave_min_ordered(fmaf(kErrC, A45, L45)));
          if (lane < 32) {
            Lq[1] = L45;
            Aq[1] = A45;
          }
          win = L.lb64[rr] > U1;
        }
      } else {
        score(I4{}, I4{}, Lq[1], Aq[1]);
        if (lane >= 62) Lq[1] = __builtin_inff();
      }
      if (win) {
        Lq[0] = __builtin_inff();
        Aq[0] = 0.0f;
      } else {
        tile0_inputs();
        score(I0{}, I4{}, Lq[0], Aq[0]);
      }
      if (msearch) {                                 // candidates no multiplier proposes drop out
        bool al0, al1;
        mark_allowed(L.ab[rr], g6, ig6, mu0, mu1, (int)(c - c_begin), L.mk, lane + 1, lane + 65, al0, al1);
        if (!al0) Lq[0] = __builtin_inff();
        if (!al1) Lq[1] = __builtin_inff();
      }
      // Each candidate's exact loss lies in [L_k - cA_k, L_k + cA_k].  U, the lowest upper end,
      // is >= the exact minimum, so the exact argmin is one of the candidates whose lower end is
      // <= U; when there is only one, it is the argmin.
      const float u0 = fmaf(kErrC, Aq[0], Lq[0]), u1 = fmaf(kErrC, Aq[1], Lq[1]);
      const float U = win ? U1 : wave_min_ordered(u1 < u0 ? u1 : u0);
      const unsigned long long M0 = __ballot(fmaf(-kErrC, Aq[0], Lq[0]) <= U);
      const unsigned long long M1 = __ballot(fmaf(-kErrC, Aq[1], Lq[1]) <= U);
      // |L_k| <= A_k, so |U| >= 2^-100 keeps every bound that matters far above the absolute
      // rounding of the subnormal range; smaller (or NaN) U goes to the float64 pass.
      const int cnt = fabsf(U) >= 0x1p-100f ? __popcll(M0) + __popcll(M1) : 0;
      if (cnt == 1) {
        // unique winner: emit its codes.  Its scale and reciprocal come from the lane that owns
        // it (tiles >= 1 apply their power of 4 exactly).
        const int k_best = M0 ? (int)__builtin_ctzll(M0) + 1 : (int)__builtin_ctzll(M1) + 65;
        const int kb0 = k_best - 1;
        const int src = kb0 & 15;
        float iw, sw;
        if (kb0 < 16) {
          iw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(is0), src));
          sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s0), src));
        } else {
          const int sh = 2 * ((kb0 >> 4) - 1);
          iw = __builtin_amdgcn_ldexpf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(is1), src)), -sh);
          sw = __builtin_amdgcn_ldexpf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(s1), src)), sh);
        }
        if (!has_ovr) {
          // codes, nibbles and loss come from the per-tile pass, 16 rows at once
          if (lane == 0) {
            L.ws[rr] = sw;
            L.wi[rr] = iw;
            L.kw[rr] = k_best;
          }
          batched |= 1u << rr;
        } else {
          float rw[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) rw[t] = w[t] * iw;
          apply_overrides(m0, 0, kv0, rv0, -1, k_best, i, gg, rw);
          apply_overrides(m1, 64, kv1, rv1, -1, k_best, i, gg, rw);
          // the converts' sign bit is the sign of w, which is (w < 0) since w is never -0
          unsigned nb4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, rw[0], rw[1], 1.0f, 0);
          nb4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(nb4, rw[2], rw[3], 1.0f, 1);
          if (i == 0 && fp4) *(unsigned short*)(fp4 + (g * cout + c) * (cin / 2) + n * 8 + 2 * gg) = (unsigned short)nb4;
          if (lane == 0) code[oblk] = (uint8_t)k_best;
          if (loss) {
            if (i == 0) L.wn[rr][gg] = (unsigned short)nb4;
            if (lane == 0) L.ws[rr] = sw;
            emitted |= 1u << rr;
          }
        }
      } else if (cnt >= 2 && cnt <= 4) {
        // 2..4 contenders: re-score them exactly in float64, 16 lanes (one per element) each
        unsigned long long ma = M0, mb = M1;
        auto next = [&]() -> int {
          if (ma) { const int b = __builtin_ctzll(ma); ma &= ma - 1; return b + 1; }
          if (mb) { const int b = __builtin_ctzll(mb); mb &= mb - 1; return b + 65; }
          return 0;
        };
        const int kc0 = next(), kc1 = next(), kc2 = next(), kc3 = next();
        const int my_k = gg == 0 ? kc0 : (gg == 1 ? kc1 : (gg == 2 ? kc2 : kc3));
        const float sk = cand_scale(my_k > 0 ? my_k : 1, gsc);
        int nib;
        const double ei = exact_err(L.w[rr][i], sk, &nib);
        L.ex[gg][i] = ei;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        double y = 0.0, bi = 0.0;
        if (dead) {
          y = ei;
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) y = fma((double)L.H[i * 16 + j], L.ex[gg][j], y);
        }
        if (coupled) {
#pragma unroll
          for (int j = 0; j < 16; ++j) bi = fma((double)L.P[i * 16 + j], (double)L.w[rr][j], bi);
        }
        double z = ei * (y + 2.0 * bi);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);   // sum over the row's lanes
        double bestD = __builtin_inf();
        int bestKD = 1 << 20;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kr = r == 0 ? kc0 : (r == 1 ? kc1 : (r == 2 ? kc2 : kc3));
          const double Lr = __shfl(z, 16 * r, 64);
          if (kr > 0 && (Lr < bestD || (Lr == bestD && kr < bestKD))) { bestD = Lr; bestKD = kr; }
        }
        const float sw = cand_scale(bestKD, gsc);
        if (lane < 8 && fp4) {
          int n0, n1;
          exact_err(L.w[rr][2 * lane], sw, &n0);
          exact_err(L.w[rr][2 * lane + 1], sw, &n1);
          fp4[(g * cout + c) * (cin / 2) + n * 8 + lane] = (uint8_t)(n0 | (n1 << 4));
        }
        if (lane == 0) {
          code[oblk] = (uint8_t)bestKD;
          if (loss) loss[oblk] = (float)bestD;
        }
        __builtin_amdgcn_wave_barrier();
      } else {
        if (RECORD) undec |= 1u << rr;
        else if (lane == 0) code[oblk] = 0;         // many contenders: float64 pass
      }
    }
    if (batched | emitted) {
      // The filter-decided winners of this tile, lane (row i, elements 4gg..4gg+3): nibbles of
      // the batched rows (w * (1/s*) through the FP4 converts; no midpoint is near), code and
      // nibble stores, then the loss from the codes -- the filter's value carries the
      // cancellation of s(Hq) - Hw -- as e* = q s* - w, (H e*) on fp32 MFMA in the layout of
      // H w and e*^T (H e* + 2 P w).
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const bool on_b = (batched >> i) & 1u;
      const bool on = on_b || ((emitted >> i) & 1u);
      unsigned nbits = 0u;
      if (on_b) {
        const float iw = L.wi[i];
        nbits = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, L.w[i][4 * gg] * iw, L.w[i][4 * gg + 1] * iw, 1.0f, 0);
        nbits = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(nbits, L.w[i][4 * gg + 2] * iw, L.w[i][4 * gg + 3] * iw, 1.0f, 1);
        nbits &= 0xFFFFu;
        if (fp4) *(unsigned short*)(fp4 + (g * cout + c0 + i) * (cin / 2) + n * 8 + 2 * gg) = (unsigned short)nbits;
        if (gg == 0) code[(g * cout + c0 + i) * nb + n] = (uint8_t)L.kw[i];
      } else if (on) {
        nbits = (unsigned)L.wn[i][gg];
      }
      if (loss) {
        const float sw = on ? L.ws[i] : 0.0f;
        const v2f q01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nbits, 1.0f, 0);
        const v2f q23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nbits, 1.0f, 1);
        const float qv[4] = {q01[0], q01[1], q23[0], q23[1]};
        float ev[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) ev[t] = on ? fmaf(qv[t], sw, -L.w[i][4 * gg + t]) : 0.0f;
        v4f he = zero4;
#pragma unroll
        for (int t = 0; t < 4; ++t) he = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], ev[t], he, 0, 0, 0);
        float part = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          part = fmaf(ev[t], coupled ? fmaf(2.0f, L.b[i][4 * gg + t], he[t]) : he[t], part);
        const float Lrow = group_sum(part);
        if (gg == 0 && on) loss[((g * cout + c0 + i) * nb) + n] = Lrow;
      }
    }
    if (RECORD && lane == 0 && undec) {             // the tile's 16 rows share one word
      const int64_t rel = c0 - c_begin;
      undec_bits[rel >> 5] |= undec << (rel & 31);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// 4 waves per SIMD: the register budget is capped at 128 (the coupled form would otherwise take
// more and drop to 3 waves, which costs about 10%).  rows_per_wave: 32, 64 when one round holds
// them all, 256 for launches of more than 64 rounds.
template <bool BF16, bool COUPLED, bool EQUALIZE, bool MSEARCH>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_sweep_full(
    const void* __restrict__ W, int64_t cout, int64_t cin, const float* __restrict__ amax,
    const float* __restrict__ Hg, const float* __restrict__ Pg, uint8_t* __restrict__ code,
    uint8_t* __restrict__ fp4, float* __restrict__ loss, int rows_per_wave, const SweepOpts opt,
    const float* __restrict__ mu) {
  __shared__ FullLds lds_all[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  FullLds& L = lds_all[wave];
  const int64_t nb = cin / 16;
  const int64_t n = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t g = blockIdx.z;
  const int64_t c_begin = (int64_t)blockIdx.y * rows_per_wave;
  if (n >= nb || c_begin >= cout) return;          // whole wave leaves; no workgroup barriers below
  const int64_t c_end = min(cout, c_begin + rows_per_wave);
  // column set-up: H_n (and P_n) through LDS into registers
  const float* Hn = Hg + (g * nb + n) * 256;
  for (int q = 0; q < 4; ++q) L.H[lane * 4 + q] = Hn[lane * 4 + q];
  if (COUPLED) {
    const float* Pn = Pg + (g * nb + n) * 256;
    for (int q = 0; q < 4; ++q) L.P[lane * 4 + q] = Pn[lane * 4 + q];
  }
  sweep_full_column<BF16, COUPLED, EQUALIZE, false, MSEARCH>(L, W, cout, cin, g, n, c_begin, c_end,
                                                    global_scale(amax[g], opt.gdiv), code, fp4, loss,
                                                    rows_per_wave, opt, mu + g * nb + n);
}

// Each block column's eigenvalue bound (column_mu) once, for all the waves that sweep its rows: a
// wave per column, H_n through LDS.
__global__ __launch_bounds__(kWaves * 64) void k_column_mu(const float* __restrict__ Hg, int64_t ncols,
                                                           float* __restrict__ mu) {
  __shared__ float hs[kWaves][256];
  __shared__ float cb[kWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * kWaves + wave;
  if (col >= ncols) return;                        // whole wave leaves; no workgroup barriers below
  const float* Hn = Hg + col * 256;
  for (int q = 0; q < 4; ++q) hs[wave][lane * 4 + q] = Hn[lane * 4 + q];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  double tr = 0.0;                                 // zero trace: scored as H = I (as the sweep)
  for (int j = 0; j < 16; ++j) tr += (double)hs[wave][j * 17];
  const float m = column_mu(hs[wave], tr == 0.0, lane, cb[wave]);
  if (lane == 0) mu[col] = m;
}

// ------------------------------------------------------------------------------------------
// Fused accumulate-and-sweep for grouped rows (MoE experts): one workgroup per (group, 64-channel
// slice) builds that expert's four block Hessians in LDS and sweeps the four block columns over
// all cout rows, one wave per column; blocks the filter leaves undecided are re-scored in float64
// by the same wave.  H never goes to memory.  The Hessian is summed exactly as k_acc_pieces sums
// it: the same pieces of at most R rows, each contracted by one wave over its 32-row chunks in
// order, the pieces added in piece order and divided by T; so H, and with it every code, nibble
// and loss, is bit-identical to lh_accumulate followed by lh_scale_sweep.
// ------------------------------------------------------------------------------------------

template <bool BF16>
union FusedLds {
  struct {
    unsigned stage[kWaves * stream::Geo<BF16>::kWords];   // each wave's chunk stage
    v4f part[kWaves][4][64];                              // one round of pieces: [piece][block][lane]
  } acc;
  struct {
    FullLds L[kWaves];                                    // the sweep, after the Hessian is made
    unsigned undec[kWaves][kFusedMaxCout / 32];           // rows the filter leaves undecided
  } sw;
};

template <bool BF16, bool MSEARCH>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_moe_fused(
    const void* __restrict__ X, const void* __restrict__ W, int64_t rows, int64_t cin, int64_t cout,
    const int64_t* __restrict__ off, int64_t R, const float* __restrict__ amax, uint8_t* __restrict__ code,
    uint8_t* __restrict__ fp4, float* __restrict__ loss, const SweepOpts opt) {
  __shared__ FusedLds<BF16> sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, gg = lane >> 4;
  const int64_t nb = cin / 16;
  const int64_t slice = blockIdx.x, g = blockIdx.y;
  const int64_t n0 = slice * 4;
  const int nblk = (int)min((int64_t)4, nb - n0);
  // rows of group g, clamped to [0, rows] as k_acc_pieces clamps them; pieces of at most R rows
  int64_t a = 0, e = rows;
  if (off) {
    a = min(max(off[g], (int64_t)0), rows);
    e = min(max(off[g + 1], a), rows);
  }
  const int64_t T = e - a;
  const int64_t npieces = T > 0 ? (T + R - 1) / R : 1;

  stream::Streamer<BF16, false, false> st{(const char*)X, nullptr, cin, slice * stream::kCh, nblk, lane, i, gg,
                                          sm.acc.stage + wave * stream::Geo<BF16>::kWords, {}, {}};
  v4f tot = {0.f, 0.f, 0.f, 0.f};                 // wave b: the running sum of block b
  for (int64_t k0 = 0; k0 < npieces; k0 += kWaves) {
    const int64_t k = k0 + wave;
    if (k < npieces) {
      st.run(a + k * R, min(e, a + k * R + R), 0, 1);
#pragma unroll
      for (int b = 0; b < 4; ++b) sm.acc.part[wave][b][lane] = st.accH[b];
    }
    __syncthreads();
    const int nk = (int)min((int64_t)kWaves, npieces - k0);
    if (wave < nblk) {
      if (npieces == 1) {
        tot = sm.acc.part[0][wave][lane];         // one piece: its sums as they are
      } else {
        for (int w = 0; w < nk; ++w) tot += sm.acc.part[w][wave][lane];   // piece order
      }
    }
    __syncthreads();                              // the round's stages and partials are free again
  }
  if (wave >= nblk) return;                       // whole wave leaves; no workgroup barriers below
  FullLds& L = sm.sw.L[wave];
  unsigned* ub = sm.sw.undec[wave];
  const int64_t n = n0 + wave;
  // H[4gg + r][i] = sum / T (zero for a group without rows)
#pragma unroll
  for (int r = 0; r < 4; ++r) L.H[(4 * gg + r) * 16 + i] = T > 0 ? tot[r] / (float)T : 0.0f;
  const float gsc = global_scale(amax[g], opt.gdiv);
  // the float32 filter over all rows records the undecided ones; the wave then re-scores those in
  // float64 (so the filter's registers are not live during the float64 pass, nor the reverse)
  for (int q = lane; q < kFusedMaxCout / 32; q += 64) ub[q] = 0u;
  sweep_full_column<BF16, false, false, true, MSEARCH>(L, W, cout, cin, g, n, 0, cout, gsc, code, fp4, loss,
                                                       (int)cout, opt, nullptr, ub);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double tr = 0.0;
  for (int j = 0; j < 16; ++j) tr += (double)L.H[j * 17];
  const bool dead = (tr == 0.0);
  float mu0 = 0.0f, mu1 = 0.0f;
  double g6 = 0.0, ig6 = 0.0;
  if (MSEARCH) {
    lane_multipliers(opt, lane, mu0, mu1);
    g6 = 6.0 * (double)gsc;
    ig6 = 1.0 / g6;
  }
  int tag = -2;                                   // below the filter's row tags and the initial -1
  for (int wi = 0; wi < (int)((cout + 31) / 32); ++wi) {
    for (unsigned u = ub[wi]; u; u &= u - 1) {
      const int64_t c = 32 * wi + __builtin_ctz(u);
      const int64_t oblk = (g * cout + c) * nb + n;
      if (lane < 16) L.w[0][lane] = load_w(W, BF16, (g * cout + c) * cin + n * 16 + lane);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      bool al0 = true, al1 = true;
      if (MSEARCH) {
        float ab = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) ab = fmaxf(ab, fabsf(L.w[0][j]));
        mark_allowed(ab, g6, ig6, mu0, mu1, tag--, L.mk, lane + 1, lane + 65, al0, al1);
      }
      exact_block<false>(L.H, L.P, L.w[0], &L.ex[0][0], dead, gsc, al0, al1, lane, code + oblk,
                         fp4 ? fp4 + (g * cout + c) * (cin / 2) + n * 8 : nullptr, loss ? loss + oblk : nullptr);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Full-Hessian sweep: float64 re-scoring of the blocks the filter left at code 0
// ------------------------------------------------------------------------------------------
struct ExactLds {
  float H[256];
  float P[256];
  float w[16];
  double b[16];
  int mk[128];         // codes proposed by the multipliers, tagged with the block
};

// Bit r: block (row c0 + r, column myn) was left undecided (code 0) by the filter.  The rows are
// read all at once (addresses clamped into the array, so every lane issues every load); rows past
// cout and columns past nb read as decided.
__device__ inline unsigned undecided_rows(const uint8_t* code, int64_t g, int64_t cout, int64_t nb,
                                          int64_t c0, int64_t myn) {
  uint8_t v[kExactRows];
  const int64_t n = min(myn, nb - 1);
#pragma unroll
  for (int r = 0; r < kExactRows; ++r) v[r] = code[(g * cout + min(c0 + r, cout - 1)) * nb + n];
  unsigned m = 0u;
#pragma unroll
  for (int r = 0; r < kExactRows; ++r) m |= (unsigned)(v[r] == 0 && c0 + r < cout && myn < nb) << r;
  return m;
}

template <bool BF16, bool COUPLED>
__global__ __launch_bounds__(kWaves * 64) void k_sweep_full_exact(
    const void* __restrict__ W, int64_t cout, int64_t cin, const float* __restrict__ amax,
    const float* __restrict__ Hg, const float* __restrict__ Pg, uint8_t* __restrict__ code,
    uint8_t* __restrict__ fp4, float* __restrict__ loss, const SweepOpts opt) {
  __shared__ ExactLds lds_all[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  ExactLds& L = lds_all[wave];
  const int64_t nb = cin / 16;
  // wave: rows c0 .. c0+kExactRows-1, block columns n0 .. n0+63 (a row's code bytes are
  // contiguous, so each row's scan is one coalesced 64-byte read)
  const int64_t c0 = ((int64_t)blockIdx.x * kWaves + wave) * kExactRows;
  const int64_t n0 = (int64_t)blockIdx.y * 64;
  const int64_t g = blockIdx.z;
  const float gsc = global_scale(amax[g], opt.gdiv);
  const bool msearch = opt.nm > 0;
  float mu0 = 0.0f, mu1 = 0.0f;
  if (msearch) lane_multipliers(opt, lane, mu0, mu1);
  L.mk[lane] = -1;
  L.mk[lane + 64] = -1;
  const double g6 = 6.0 * (double)gsc, ig6 = 1.0 / g6;
  int tag = 0;
  const int64_t myn = n0 + lane;
  const unsigned undecided = undecided_rows(code, g, cout, nb, c0, myn);
  for (int r = 0; r < kExactRows; ++r) {
    const int64_t c = c0 + r;
    if (c >= cout) break;
    unsigned long long todo = __ballot((undecided >> r) & 1u);
    while (todo) {
      const int64_t n = n0 + __builtin_ctzll(todo);
      todo &= todo - 1;
      const float* Hn = Hg + (g * nb + n) * 256;
      for (int q = 0; q < 4; ++q) L.H[lane * 4 + q] = Hn[lane * 4 + q];
      if (COUPLED) {
        const float* Pn = Pg + (g * nb + n) * 256;
        for (int q = 0; q < 4; ++q) L.P[lane * 4 + q] = Pn[lane * 4 + q];
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      double tr = 0.0;
      for (int j = 0; j < 16; ++j) tr += (double)L.H[j * 17];
      const bool dead = (tr == 0.0);
      const int64_t base = (g * cout + c) * cin + n * 16;
      if (lane < 16) L.w[lane] = load_w(W, BF16, base + lane);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      bool al0 = true, al1 = true;
      if (msearch) {
        float ab = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) ab = fmaxf(ab, fabsf(L.w[j]));
        mark_allowed(ab, g6, ig6, mu0, mu1, tag++, L.mk, lane + 1, lane + 65, al0, al1);
      }
      const int64_t oblk = (g * cout + c) * nb + n;
      exact_block<COUPLED>(L.H, L.P, L.w, L.b, dead, gsc, al0, al1, lane, code + oblk,
                           fp4 ? fp4 + (g * cout + c) * (cin / 2) + n * 8 : nullptr, loss ? loss + oblk : nullptr);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Diagonal (importance-weighted) sweep: float32 filter
// ------------------------------------------------------------------------------------------
template <bool BF16>
__device__ inline void load_w16(const void* W, int64_t base, float w[16]) {
  if (BF16) {
    const unsigned* p = (const unsigned*)((const unsigned short*)W + base);   // 32-byte aligned
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const unsigned v = p[j];
      w[2 * j] = __uint_as_float(v << 16);
      w[2 * j + 1] = __uint_as_float(v & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = ((const float*)W)[base + j];
  }
}

// Exact E2M1 grid index of |w|/s for s > 0 (normal range): each rounding midpoint m is compared
// through the sign of fma(m, s, -|w|), which is the sign of the exact m*s - |w|; ties go to the
// even index (down at 0.25, 1.25, 2.5, 5; up at 0.75, 1.75, 3.5).
__device__ inline int e2m1_index_fma(float aw, float s) {
  return (int)(fmaf(0.25f, s, -aw) < 0.0f) + (int)(fmaf(0.75f, s, -aw) <= 0.0f) +
         (int)(fmaf(1.25f, s, -aw) < 0.0f) + (int)(fmaf(1.75f, s, -aw) <= 0.0f) +
         (int)(fmaf(2.5f, s, -aw) < 0.0f) + (int)(fmaf(3.5f, s, -aw) <= 0.0f) +
         (int)(fmaf(5.0f, s, -aw) < 0.0f);
}
__device__ inline float e2m1_valf(int c) {
  return c <= 4 ? 0.5f * (float)c : (c == 5 ? 3.0f : (c == 6 ? 4.0f : 6.0f));
}

// Diagonal form.  The loss L_k = sum_j Imp_j e_j^2 is scored in a weighted frame: with
// a_j = sqrt(Imp_j) (float64 root rounded to fp32), t_kj = s_k a_j and u_j = w_j a_j, a lane forms
// e'_j = fma(q_j, t_kj, -u_j) ~ a_j e_j and L'_k = sum_j e'_j^2 (two VALU operations per element
// and candidate after the quantization).  Error bound, with delta = 2^-24 and W = sum_j Imp_j w_j^2:
//  * quantization: a quotient r' = w (1/s) on the wrong side of an E2M1 midpoint by its rounding
//    error (|r' - r| <= 2^-23 r) picks the other neighbour, which changes that element's e^2 by at
//    most 4 (m/h) 2^-23 <= 56 delta of itself (m a midpoint, h the half spacing around it), so
//    the loss L of the codes the converts pick lies in [L*, (1 + 56 delta) L*], L* the exact one;
//  * arithmetic: q t - u = a (e + eta) with |eta| <= delta (|q| s + |w|) <= delta (2|w| + |e|)
//    (|q s| <= |w| + |e| and |e| <= |w|: 0 is on the grid), so with the roundings of a, of the fma
//    and of the 16-term sum, |L' - L| <= 22 delta L + 4 delta sqrt(L W) + 9 delta^2 W; moving
//    from L to L' on the right costs under 2% plus 400 delta^2 W.
// Hence L* lies within B(L') = C1 L' + C2 sqrt(L' W) + C3 W of L' (C1 = 2^-17 >= 80 delta,
// C2 = 2^-21 >= 4.1 delta, C3 = 2^-38), provided nothing overflows or leaves the normal range:
// the filter runs only for 2^-100 <= g <= 2^100, 448 g max_j a_j <= 2^120 and, per row,
// 2^-100 <= W <= 2^100 (then |e'| <= 3 |u| and L' stays finite; underflowed products are covered
// by C3 W); other rows go to the float64 kernel.  The square root is linearized once per wave:
// for any lam > 0, C2 sqrt(L' W) <= C2/2 (lam L' + W/lam), so B(L') <= alpha L' + beta with
// alpha = C1 + C2 lam/2 and beta = (C2/(2 lam) + C3) W; lam = sqrt(W/m) from the first row's
// lowest L' makes the line tangent where it matters.  U = (1 + alpha) min L' + beta bounds the
// exact minimum from above, and only candidates with (1 - alpha) L' - beta <= U can be the
// argmin (the tests are written so a NaN or infinite L' counts as a contender).  Only the
// winner's nibbles and loss are then recomputed with exact rounding decisions.
//
// Candidate pairs: a lane scores two codes that share one E4M3 mantissa, so s_b = 2^p s_a exactly
// and one quotient w (1/s_a) serves both: the FP4 convert divides it by 2^p through its
// exponent-only scale operand, exactly.  Lanes 7..61 hold codes (l+1, l+65) (p = 8); the
// subnormal codes 1..7 and codes 63..71 are paired by hand.  Four mantissa classes hold an odd
// number of codes, so one code (69) is left without a partner: it is scored in a separate pass
// over the wave's rows and its loss stands in lane 5's second slot.  Lanes 6 and 63 hold one code.
constexpr float kDiagC1 = 0x1p-17f;
constexpr float kDiagC2h = 0x1p-22f;      // C2 / 2
constexpr float kDiagC3 = 0x1p-38f;
constexpr int kDiagLoneCode = 69;
constexpr int kDiagLoneLane = 5;

struct DiagPair {
  int k0, k1;        // codes of the two slots (k1 = 0: no second code)
  float sc1;         // s_k1 / s_k0, a power of two
};
__device__ inline DiagPair diag_pair(int lane) {
  switch (lane) {
    case 0: return {1, 2, 2.0f};
    case 1: return {3, 6, 2.0f};
    case 2: return {5, 66, 256.0f};
    case 3: return {7, 70, 256.0f};
    case 4: return {4, 64, 256.0f};
    case 5: return {65, kDiagLoneCode, 1.0f};   // second slot: the separate pass
    case 6: return {67, 0, 1.0f};
    case 62: return {63, 71, 2.0f};
    case 63: return {68, 0, 1.0f};
    default: return {lane + 1, lane + 65, 256.0f};
  }
}

// A wave-uniform float kept in a scalar register.
__device__ inline float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}


// 6 waves per SIMD (80 registers; a few values outside the row loop go to scratch) measured
// about 1% faster than 5 waves without the cap.
template <bool BF16, bool MSEARCH>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(6))) void k_sweep_diag(
    const void* __restrict__ W, int64_t cout, int64_t cin, const float* __restrict__ amax,
    const float* __restrict__ imp, uint8_t* __restrict__ code, uint8_t* __restrict__ fp4,
    float* __restrict__ loss, const SweepOpts opt) {
  __shared__ __attribute__((aligned(16))) float wt_all[kWaves][kRowsPerWave][16];   // w (+0 for -0)
  __shared__ float ab_all[kWaves][kRowsPerWave];      // block amax of the row (multiplier search)
  __shared__ int mk_all[kWaves][128];                 // codes proposed by the multipliers
  __shared__ __attribute__((aligned(16))) float ut_all[kWaves][kRowsPerWave][16];   // w a
  __shared__ __attribute__((aligned(16))) float sa_all[kWaves][16];                 // a = sqrt(Imp)
  __shared__ float im_all[kWaves][16];
  __shared__ float wr_all[kWaves][kRowsPerWave];      // W of the row (-1: not filtered)
  __shared__ float lone_all[kWaves][kRowsPerWave];    // L' of the unpaired code
  __shared__ int win_k[kWaves][kRowsPerWave];         // winner's code per row (0: no winner)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nb = cin / 16;
  const int64_t n = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t g = blockIdx.z;
  const int64_t c_begin = (int64_t)blockIdx.y * kRowsPerWave;
  if (n >= nb || c_begin >= cout) return;
  const int64_t c_end = min(cout, c_begin + kRowsPerWave);
  const int nrows = (int)(c_end - c_begin);

  // importance of the block column (all ones when it sums to zero or none is given: plain MSE),
  // a_j = sqrt(Imp_j)
  const float* ip = imp ? imp + g * cin + n * 16 : nullptr;
  double isum = 0.0;
  if (ip) {
#pragma unroll
    for (int j = 0; j < 16; ++j) isum += (double)ip[j];
  }
  if (lane < 16) {
    const float v = isum == 0.0 ? 1.0f : ip[lane];
    im_all[wave][lane] = v;
    sa_all[wave][lane] = (float)sqrt((double)v);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float gsc = uniform(global_scale(amax[g], opt.gdiv));
  constexpr bool msearch = MSEARCH;               // multiplier search: its own instantiation
  float mu0 = 0.0f, mu1 = 0.0f;
  double g6 = 0.0, ig6 = 0.0;
  if (msearch) {
    lane_multipliers(opt, lane, mu0, mu1);
    mk_all[wave][lane] = -1;
    mk_all[wave][lane + 64] = -1;
    g6 = 6.0 * (double)gsc;
    ig6 = 1.0 / g6;
  }
  float a[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4f t = *(const v4f*)&sa_all[wave][4 * q];
    a[4 * q] = t[0]; a[4 * q + 1] = t[1]; a[4 * q + 2] = t[2]; a[4 * q + 3] = t[3];
  }
  float amx = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) amx = fmaxf(amx, a[j]);
  const bool fast = filter_ok(gsc) && 448.0 * (double)gsc * (double)amx <= 0x1p120;

  const DiagPair pr = diag_pair(lane);
  const bool lone = lane == kDiagLoneLane, single = pr.k1 == 0;
  const float s0 = cand_scale(pr.k0, gsc), is0 = inv_scale(s0), sc1 = pr.sc1;
  const float sl = uniform(cand_scale(kDiagLoneCode, gsc)), isl = uniform(inv_scale(sl));
  // t_k1,j = sc1 t_k0,j exactly; the second slot's grid values come back from the convert
  // already multiplied by sc1, so one set of products serves both slots
  float t0[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) t0[j] = s0 * a[j];

  bool have_line = false;                         // alpha, beta set from the first filtered row
  float A1 = 0.0f, K2 = 0.0f;
  unsigned pkc[4] = {0u, 0u, 0u, 0u};             // FP4 pack registers carried between rows
  float (*wt)[16] = wt_all[wave];
  float (*ut)[16] = ut_all[wave];

  {
    const int sub = lane & 7, el0 = 2 * sub, el1 = el0 + 1;

    // The wave's 32 blocks (rows c_begin.., column n) come in with one coalesced load per lane
    // (lane l: row l/2, elements 8*(l%2)..+7) and wait in LDS as w and w a, with the row's W; the
    // same lane scores the unpaired code over its 8 elements.
    {
      const int rr = lane >> 1, h = lane & 1;
      const int64_t c = c_begin + rr;
      const int64_t e0 = (g * cout + min(c, c_end - 1)) * cin + n * 16 + 8 * h;
      float v[8];
      if (BF16) {
        const v4u u = *(const v4u*)((const unsigned short*)W + e0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = __uint_as_float(u[q] << 16) + 0.0f;           // + 0 turns -0 into +0
          v[2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u) + 0.0f;
        }
      } else {
        const v4f u0 = *(const v4f*)((const float*)W + e0), u1 = *(const v4f*)((const float*)W + e0 + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) { v[q] = u0[q] + 0.0f; v[4 + q] = u1[q] + 0.0f; }
      }
      const v4f a0 = *(const v4f*)&sa_all[wave][8 * h], a1 = *(const v4f*)&sa_all[wave][8 * h + 4];
      const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      float uv[8];
      float wp = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uv[q] = v[q] * av[q];
        wp = fmaf(uv[q], uv[q], wp);
      }
      *(v4f*)&wt[rr][8 * h] = v4f{v[0], v[1], v[2], v[3]};
      *(v4f*)&wt[rr][8 * h + 4] = v4f{v[4], v[5], v[6], v[7]};
      *(v4f*)&ut[rr][8 * h] = v4f{uv[0], uv[1], uv[2], uv[3]};
      *(v4f*)&ut[rr][8 * h + 4] = v4f{uv[4], uv[5], uv[6], uv[7]};
      float lp = 0.0f;
      unsigned pk = 0u;
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, v[q] * isl, v[q + 1] * isl, 1.0f, 0);
        const v2f qq = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 0);
        const float ea = fmaf(qq[0], sl * av[q], -uv[q]), eb = fmaf(qq[1], sl * av[q + 1], -uv[q + 1]);
        lp = fmaf(ea, ea, lp);
        lp = fmaf(eb, eb, lp);
      }
      const float wrow = wp + __shfl_xor(wp, 1, 64);
      lp += __shfl_xor(lp, 1, 64);
      float am = 0.0f;
      if (msearch) {
#pragma unroll
        for (int q = 0; q < 8; ++q) am = fmaxf(am, fabsf(v[q]));
        am = fmaxf(am, __shfl_xor(am, 1, 64));
      }
      if (h == 0) {
        wr_all[wave][rr] = (wrow >= 0x1p-100f && wrow <= 0x1p+100f) ? wrow : -1.0f;
        lone_all[wave][rr] = lp;
        ab_all[wave][rr] = am;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    for (int rr = 0; rr < nrows; ++rr) {
      const int64_t oblk = (g * cout + c_begin + rr) * nb + n;
      const float wrow = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wr_all[wave][rr])));
      if (!fast || !(wrow >= 0.0f)) {
        if (lane == 0) {
          code[oblk] = 0;                         // resolved by the float64 pass
          win_k[wave][rr] = 0;
        }
        continue;
      }
      float w[16], u[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f t = *(const v4f*)&wt[rr][4 * q];
        const v4f z = *(const v4f*)&ut[rr][4 * q];
        w[4 * q] = t[0]; w[4 * q + 1] = t[1]; w[4 * q + 2] = t[2]; w[4 * q + 3] = t[3];
        u[4 * q] = z[0]; u[4 * q + 1] = z[1]; u[4 * q + 2] = z[2]; u[4 * q + 3] = z[3];
      }
      float L0 = 0.0f, L1 = 0.0f;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        // elements 4 j4..+3: bytes 0/1 hold the first pair for the two slots, bytes 2/3 the
        // second; all four bytes are rewritten before they are read
        const int j = 4 * j4;
        const float x0 = w[j] * is0, x1 = w[j + 1] * is0, x2 = w[j + 2] * is0, x3 = w[j + 3] * is0;
        unsigned pk = pkc[j4];
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x0, x1, 1.0f, 0);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x0, x1, sc1, 1);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x2, x3, 1.0f, 2);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x2, x3, sc1, 3);
        pkc[j4] = pk;
        const v2f qa = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 0);
        const v2f qb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, sc1, 1);
        const v2f qc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 2);
        const v2f qd = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, sc1, 3);
        const float ea0 = fmaf(qa[0], t0[j], -u[j]), ea1 = fmaf(qa[1], t0[j + 1], -u[j + 1]);
        const float eb0 = fmaf(qb[0], t0[j], -u[j]), eb1 = fmaf(qb[1], t0[j + 1], -u[j + 1]);
        const float ec0 = fmaf(qc[0], t0[j + 2], -u[j + 2]), ec1 = fmaf(qc[1], t0[j + 3], -u[j + 3]);
        const float ed0 = fmaf(qd[0], t0[j + 2], -u[j + 2]), ed1 = fmaf(qd[1], t0[j + 3], -u[j + 3]);
        L0 = fmaf(ea0, ea0, L0);
        L0 = fmaf(ea1, ea1, L0);
        L1 = fmaf(eb0, eb0, L1);
        L1 = fmaf(eb1, eb1, L1);
        L0 = fmaf(ec0, ec0, L0);
        L0 = fmaf(ec1, ec1, L0);
        L1 = fmaf(ed0, ed0, L1);
        L1 = fmaf(ed1, ed1, L1);
      }
      const float lone_L = lone_all[wave][rr];
      L1 = single ? __builtin_inff() : (lone ? lone_L : L1);
      if (msearch) {                                 // candidates no multiplier proposes drop out
        bool al0, al1;
        mark_allowed(ab_all[wave][rr], g6, ig6, mu0, mu1, rr, mk_all[wave], pr.k0,
                     single ? 0 : (lone ? kDiagLoneCode : pr.k1), al0, al1);
        if (!al0) L0 = __builtin_inff();
        if (!al1) L1 = __builtin_inff();
      }
      // losses are >= 0 or +inf, ordered like their bit patterns
      const float m = wave_min_nonneg(__uint_as_float(min(__float_as_uint(L0), __float_as_uint(L1))));
      if (!have_line) {
        // lam = sqrt(W/m), kept within [1, 4096]; any lam > 0 gives a valid line.  The factors
        // (1 + 2^-18) cover the roundings of alpha and beta, (1 + 2^-16) those of W, of the
        // division by 1 - alpha folded into A1 and K2, and of the test.
        const float mm = m > wrow * 0x1p-40f ? m : wrow * 0x1p-40f;
        const float lam = fminf(fmaxf(__builtin_amdgcn_rsqf(mm / wrow), 1.0f), 4096.0f);
        const float alpha = fmaf(kDiagC2h, lam, kDiagC1) * (1.0f + 0x1p-18f);
        const float bet = fmaf(kDiagC2h * (1.0f + 0x1p-18f), 1.0f / lam, kDiagC3);
        const float ioma = 1.0f / (1.0f - alpha);
        A1 = uniform((1.0f + alpha) * ioma * (1.0f + 0x1p-16f));
        K2 = uniform(2.0f * bet * ioma * (1.0f + 0x1p-16f));
        have_line = true;
      }
      // the exact argmin is among the slots with (1 - alpha) L' - beta <= U = (1 + alpha) m + beta,
      // i.e. L' <= ((1 + alpha) m + 2 beta) / (1 - alpha)
      const float rhs = fmaf(A1, m, K2 * wrow);
      const unsigned long long M0 = __ballot(!(L0 > rhs)), M1 = __ballot(!(L1 > rhs));
      const int cnt = __popcll(M0) + __popcll(M1);
      int kwin = 0;
      if (cnt == 1) {
        const bool in0 = M0 != 0ull;
        const int b = (int)__builtin_ctzll(in0 ? M0 : M1);
        const DiagPair pb = diag_pair(b);
        kwin = in0 ? pb.k0 : pb.k1;
      } else if (cnt > 1 && cnt <= 4) {
        // 2..4 contenders: exact float64 losses, one contender per 16 lanes (lane: element l%16)
        unsigned long long ma = M0, mb = M1;
        auto next = [&]() -> int {
          if (ma) { const int bb = __builtin_ctzll(ma); ma &= ma - 1; return diag_pair(bb).k0; }
          if (mb) { const int bb = __builtin_ctzll(mb); mb &= mb - 1; return diag_pair(bb).k1; }
          return 0;
        };
        const int kc0 = next(), kc1 = next(), kc2 = next(), kc3 = next();
        const int q = lane >> 4, j = lane & 15;
        const int my_k = q == 0 ? kc0 : (q == 1 ? kc1 : (q == 2 ? kc2 : kc3));
        int nib;
        const double e = exact_err(wt[rr][j], cand_scale(my_k > 0 ? my_k : 1, gsc), &nib);
        double z = (double)im_all[wave][j] * e * e;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
        double bestD = __builtin_inf();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kr = r == 0 ? kc0 : (r == 1 ? kc1 : (r == 2 ? kc2 : kc3));
          const double Lr = __shfl(z, 16 * r, 64);
          if (kr > 0 && (Lr < bestD || (Lr == bestD && kr < kwin))) { bestD = Lr; kwin = kr; }
        }
      }
      if (lane == 0) {
        const bool decided = cnt >= 1 && cnt <= 4;
        if (!decided) code[oblk] = 0;             // many contenders (or none): float64 pass
        win_k[wave][rr] = decided ? kwin : 0;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Exact nibbles and loss of every row's winner, eight rows at a time: lane l takes row
    // 8*pass + l/8 and its elements 2*(l%8), 2*(l%8)+1.  The hardware reciprocal is within one
    // ulp, so |w| (1/s)(1 -+ 2^-19) fall strictly below and above the exact quotient |w|/s; the
    // FP4 convert is monotone in its input, so when the two give the same code that is the exact
    // rounding (an exact midpoint gives two different codes).  Otherwise the element is within
    // about 2^-18 of a midpoint and the sign of fma(m, s, -|w|) decides each midpoint.
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int rr = 8 * pass + (lane >> 3);
      const int64_t c = c_begin + rr;
      const bool row_on = rr < nrows;
      const int kw = row_on ? win_k[wave][rr] : 0;
      const float sw = cand_scale(kw > 0 ? kw : 1, gsc);        // as the filter formed it
      const float wa = wt[rr][el0], wb = wt[rr][el1];
      const float ima = im_all[wave][el0], imb = im_all[wave][el1];
      const float is = __builtin_amdgcn_rcpf(sw);
      const float isp = is * (1.0f + 0x1p-19f), ism = is * (1.0f - 0x1p-19f);
      unsigned byte = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, wa * isp, wb * isp, 1.0f, 0);
      const unsigned blo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, wa * ism, wb * ism, 1.0f, 0);
      if (byte != blo) {
        const int ca = e2m1_index_fma(fabsf(wa), sw), cb = e2m1_index_fma(fabsf(wb), sw);
        byte = (unsigned)(ca | (wa < 0.0f ? 8 : 0)) | ((unsigned)(cb | (wb < 0.0f ? 8 : 0)) << 4);
      }
      const v2f qv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);   // signed grid values
      const float ea = fmaf(qv[0], sw, -wa), eb = fmaf(qv[1], sw, -wb);
      float part = fmaf(imb * eb, eb, ima * ea * ea);
      part += __shfl_xor(part, 1, 64);
      part += __shfl_xor(part, 2, 64);
      part += __shfl_xor(part, 4, 64);
      if (kw != 0) {
        if (fp4) fp4[(g * cout + c) * (cin / 2) + n * 8 + sub] = (uint8_t)byte;
        if (sub == 0) {
          code[(g * cout + c) * nb + n] = (uint8_t)kw;
          if (loss) loss[(g * cout + c) * nb + n] = part;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ------------------------------------------------------------------------------------------
// Diagonal sweep over a window of 32 codes (float32 filter; no amax-multiplier search)
// ------------------------------------------------------------------------------------------
// Which codes can win.  Let kmax be a code with 6 s_kmax >= amax (the smallest such code or one
// above it) and let the window be the 32 codes from start = clamp(kmax - 12, 1, 95) to
// end = start + 31.  Below its amax a block's scale clips: every element keeps an error of at
// least |w_i| - 6 s_k whatever its FP4 code, so for every k < start
//   L_k >= LB_lo = sum_i Imp_i (|w_i| - 6 s_{start-1})_+^2.
// Above the window every scale is at least s_hi = s_{end+1}; an element with |w_i| < s_hi / 2
// then has a quotient below 1/2 and rounds to 0 or 1/2, so for every k > end
//   L_k >= LB_hi = sum_{|w_i| < s_hi/2} Imp_i min(|w_i|, s_hi/2 - |w_i|)^2.
// With U an upper bound of the window's exact minimum, LB_lo > U and LB_hi >= U (the lowest code
// wins a tie, and codes above the window are higher) make the window's argmin the block's.  The
// pages' score and candidate set are unchanged: the window only skips codes these bounds rule
// out.  On the WMSE down_proj layer the argmin lies 11 codes below to 6 above kmax and both
// bounds decide the block almost always; the others, like blocks whose window starts below
// code 8 or that keep more than four contenders, are left at code 0 for the float64 kernel.
//
// Scoring.  Lane j of an 8-lane row group takes the codes start + j + 8t, t = 0..3, with scales
// s, 2s, 4s, 8s (exact powers of two for codes >= 8 in fp32's normal range), so one quotient
// w (1/s) per element serves all four through the FP4 convert's exponent-only scale operand, and
// a wave scores eight rows at a time.  Each candidate's L' and its error bound are those of
// k_sweep_diag (the weighted frame, constants kDiagC1..C3), with the line through lam set per
// row; here 1/s comes from the hardware reciprocal (within one ulp), so a quotient is within
// 1.5 2^-23 of |w|/s and a wrong-side rounding changes an element's e^2 by at most 84 delta of
// itself instead of 56: with the 22 delta of the arithmetic that is 106 delta <= C1 = 128 delta.
// Two to four contenders are scored again in float64 by the whole wave.

// Smallest code k in 1..126 with v_k >= y (126 above 448, 1 at or below 2^-9).
__device__ inline int e4m3_ceil_code(double y) {
  if (!(y > 0x1p-9)) return 1;
  if (y > 448.0) return 126;
  const int e = ilogb(y);
  if (e < -6) return (int)ceil(y * 512.0);                 // subnormal values m 2^-9
  const int f = (int)ceil((ldexp(y, -e) - 1.0) * 8.0);     // 0..8 (8: the next binade's first)
  return min((e + 7) * 8 + f, 126);
}

// Minimum over each group of 8 lanes of values >= 0 or +inf (bit patterns ordered like the
// floats): the two quad permutations, then the half-row mirror.
__device__ inline unsigned oct_min_u(unsigned v) {
  v = min(v, (unsigned)dppi<0xB1>((int)v));
  v = min(v, (unsigned)dppi<0x4E>((int)v));
  v = min(v, (unsigned)dppi<0x141>((int)v));
  return v;
}

// 6 waves per SIMD (at most 80 registers).
template <bool BF16>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(6))) void k_sweep_diag_win(
    const void* __restrict__ W, int64_t cout, int64_t cin, const float* __restrict__ amax,
    const float* __restrict__ imp, uint8_t* __restrict__ code, uint8_t* __restrict__ fp4,
    float* __restrict__ loss, const SweepOpts opt) {
  __shared__ __attribute__((aligned(16))) float wt_all[kWaves][kRowsPerWave][16];   // w (+0 for -0)
  __shared__ __attribute__((aligned(16))) float ut_all[kWaves][kRowsPerWave][16];   // w a
  __shared__ __attribute__((aligned(16))) float sa_all[kWaves][16];                 // a = sqrt(Imp)
  __shared__ float im_all[kWaves][16];
  __shared__ float wr_all[kWaves][kRowsPerWave];      // W of the row (-1: not filtered)
  __shared__ float lb_all[kWaves][kRowsPerWave];      // LB_lo: bound on the codes below the window
  __shared__ float lh_all[kWaves][kRowsPerWave];      // LB_hi: bound on the codes above it
  __shared__ int st_all[kWaves][kRowsPerWave];        // first code of the window (0: no window)
  __shared__ int win_k[kWaves][kRowsPerWave];         // winner's code per row (0: no winner)
  __shared__ unsigned long long ctd_all[kWaves][kRowsPerWave];   // 2..4 contenders: bit b = code start + b
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nb = cin / 16;
  const int64_t n = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t g = blockIdx.z;
  const int64_t c_begin = (int64_t)blockIdx.y * kRowsPerWave;
  if (n >= nb || c_begin >= cout) return;
  const int64_t c_end = min(cout, c_begin + kRowsPerWave);
  const int nrows = (int)(c_end - c_begin);

  // importance of the block column (all ones when it sums to zero or none is given: plain MSE),
  // a_j = sqrt(Imp_j)
  const float* ip = imp ? imp + g * cin + n * 16 : nullptr;
  double isum = 0.0;
  if (ip) {
#pragma unroll
    for (int j = 0; j < 16; ++j) isum += (double)ip[j];
  }
  if (lane < 16) {
    const float v = isum == 0.0 ? 1.0f : ip[lane];
    im_all[wave][lane] = v;
    sa_all[wave][lane] = (float)sqrt((double)v);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float gsc = uniform(global_scale(amax[g], opt.gdiv));
  float amx = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4f t = *(const v4f*)&sa_all[wave][4 * q];
    amx = fmaxf(amx, fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
  }
  const bool fast = filter_ok(gsc) && 448.0 * 64.0 * (double)gsc * (double)amx <= 0x1p120;
  float (*wt)[16] = wt_all[wave];
  float (*ut)[16] = ut_all[wave];

  // The wave's 32 blocks come in with one coalesced load per lane (lane l: row l/2, elements
  // 8*(l%2)..+7) and wait in LDS as w and w a, with the row's W, its window and its bound.
  {
    const int rr = lane >> 1, h = lane & 1;
    const int64_t c = c_begin + rr;
    const int64_t e0 = (g * cout + min(c, c_end - 1)) * cin + n * 16 + 8 * h;
    float v[8];
    if (BF16) {
      const v4u u = *(const v4u*)((const unsigned short*)W + e0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(u[q] << 16) + 0.0f;           // + 0 turns -0 into +0
        v[2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u) + 0.0f;
      }
    } else {
      const v4f u0 = *(const v4f*)((const float*)W + e0), u1 = *(const v4f*)((const float*)W + e0 + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) { v[q] = u0[q] + 0.0f; v[4 + q] = u1[q] + 0.0f; }
    }
    const v4f a0 = *(const v4f*)&sa_all[wave][8 * h], a1 = *(const v4f*)&sa_all[wave][8 * h + 4];
    const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    float uv[8];
    float wp = 0.0f, am = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uv[q] = v[q] * av[q];
      wp = fmaf(uv[q], uv[q], wp);
      am = fmaxf(am, fabsf(v[q]));
    }
    *(v4f*)&wt[rr][8 * h] = v4f{v[0], v[1], v[2], v[3]};
    *(v4f*)&wt[rr][8 * h + 4] = v4f{v[4], v[5], v[6], v[7]};
    *(v4f*)&ut[rr][8 * h] = v4f{uv[0], uv[1], uv[2], uv[3]};
    *(v4f*)&ut[rr][8 * h + 4] = v4f{uv[4], uv[5], uv[6], uv[7]};
    const float wrow = wp + __shfl_xor(wp, 1, 64);
    am = fmaxf(am, __shfl_xor(am, 1, 64));
    // window: kmax one above the smallest code with 6 s >= amax (so that 6 s_kmax >= amax holds
    // after the fp32 rounding of s_kmax), start 12 codes below it
    const int kmax = min(126, e4m3_ceil_code((double)am / (6.0 * (double)gsc)) + 1);
    const int start = min(max(kmax - 12, 1), 95);
    // LB_lo and LB_hi in fp32, lowered by 2^-18 to bound the exact sums from below (each term
    // has at most three roundings, the 16-term sum at most 16 more); |w| - 6 s and s_hi/2 - |w|
    // take one rounding each (fma), so their signs are exact
    const v4f m0 = *(const v4f*)&im_all[wave][8 * h], m1 = *(const v4f*)&im_all[wave][8 * h + 4];
    const float mv[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
    const float sl = cand_scale(max(start - 1, 1), gsc), sh = cand_scale(min(start + 32, 126), gsc);
    float lbp = 0.0f, lhp = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float aw = fabsf(v[q]);
      const float d = fmaf(-6.0f, sl, aw);
      if (d > 0.0f) lbp = fmaf(mv[q] * d, d, lbp);
      const float dh = fminf(aw, fmaf(0.5f, sh, -aw));
      if (dh > 0.0f) lhp = fmaf(mv[q] * dh, dh, lhp);
    }
    lbp += __shfl_xor(lbp, 1, 64);
    lhp += __shfl_xor(lhp, 1, 64);
    if (h == 0) {
      const bool row_ok = fast && wrow >= 0x1p-100f && wrow <= 0x1p+100f && start >= 8;
      wr_all[wave][rr] = row_ok ? wrow : -1.0f;
      st_all[wave][rr] = row_ok ? start : 0;
      lb_all[wave][rr] = start > 1 ? lbp * (1.0f - 0x1p-18f) : __builtin_inff();
      lh_all[wave][rr] = start + 31 < 126 ? lhp * (1.0f - 0x1p-18f) : __builtin_inff();
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int grp = lane >> 3, j = lane & 7;
  for (int pass = 0; pass < (nrows + 7) / 8; ++pass) {
    const int rr = 8 * pass + grp;
    const bool row_on = rr < nrows;
    const int rs = row_on ? rr : 0;
    const int start = row_on ? st_all[wave][rs] : 0;
    const float wrow = wr_all[wave][rs];
    const bool scored = start > 0;                           // the row group's window
    // the lane's codes start + j + 8 t; rows without a window score codes 95 + j + 8 t (valid
    // codes, results unused)
    const int k0 = (scored ? start : 95) + j;
    const float s0 = cand_scale(k0, gsc), is0 = __builtin_amdgcn_rcpf(s0);   // within one ulp of 1/s
    float L0 = 0.0f, L1 = 0.0f, L2 = 0.0f, L3 = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      // elements 2p, 2p+1 (w, w a and a read from LDS as needed): byte t of the pack register
      // holds them for slot t (scale 2^t)
      const v2f wv = *(const v2f*)&wt[rs][2 * p];
      const v2f uv = *(const v2f*)&ut[rs][2 * p];
      const v2f av = *(const v2f*)&sa_all[wave][2 * p];
      const float x0 = wv[0] * is0, x1 = wv[1] * is0;
      unsigned pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x0, x1, 1.0f, 0);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x0, x1, 2.0f, 1);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x0, x1, 4.0f, 2);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x0, x1, 8.0f, 3);
      const v2f qa = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 0);
      const v2f qb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 2.0f, 1);
      const v2f qc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 4.0f, 2);
      const v2f qd = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 8.0f, 3);
      const float ta = s0 * av[0], tb = s0 * av[1], ua = -uv[0], ub = -uv[1];
      const float ea0 = fmaf(qa[0], ta, ua), ea1 = fmaf(qa[1], tb, ub);
      const float eb0 = fmaf(qb[0], ta, ua), eb1 = fmaf(qb[1], tb, ub);
      const float ec0 = fmaf(qc[0], ta, ua), ec1 = fmaf(qc[1], tb, ub);
      const float ed0 = fmaf(qd[0], ta, ua), ed1 = fmaf(qd[1], tb, ub);
      L0 = fmaf(ea0, ea0, L0);
      L0 = fmaf(ea1, ea1, L0);
      L1 = fmaf(eb0, eb0, L1);
      L1 = fmaf(eb1, eb1, L1);
      L2 = fmaf(ec0, ec0, L2);
      L2 = fmaf(ec1, ec1, L2);
      L3 = fmaf(ed0, ed0, L3);
      L3 = fmaf(ed1, ed1, L3);
    }
    // losses are >= 0 or +inf, ordered like their bit patterns
    const float m = __uint_as_float(oct_min_u(min(min(__float_as_uint(L0), __float_as_uint(L1)),
                                                  min(__float_as_uint(L2), __float_as_uint(L3)))));
    // the row's line: lam ~ sqrt(W/m) within [1, 4096] (any lam > 0 gives a valid bound); the
    // factors (1 + 2^-18) cover the roundings of alpha and beta, including the reciprocal of lam
    // (within one ulp), (1 + 2^-16) those of W, of the reciprocal of 1 - alpha folded into A1
    // and K2, and of the tests
    const float wr = fmaxf(wrow, 0x1p-100f);
    const float mm = m > wr * 0x1p-40f ? m : wr * 0x1p-40f;
    const float lam = fminf(fmaxf(__builtin_amdgcn_rsqf(mm * __builtin_amdgcn_rcpf(wr)), 1.0f), 4096.0f);
    const float alpha = fmaf(kDiagC2h, lam, kDiagC1) * (1.0f + 0x1p-18f);
    const float bet = fmaf(kDiagC2h * (1.0f + 0x1p-18f), __builtin_amdgcn_rcpf(lam), kDiagC3);
    const float ioma = __builtin_amdgcn_rcpf(1.0f - alpha);
    const float A1 = (1.0f + alpha) * ioma * (1.0f + 0x1p-16f);
    const float K2 = 2.0f * bet * ioma * (1.0f + 0x1p-16f);
    // contenders: L' <= ((1 + alpha) m + 2 beta) / (1 - alpha); the exact window minimum is at
    // most U = (1 + alpha) m + beta; codes below the window are out when LB_lo > U, codes above
    // it when LB_hi >= U
    const float rhs = fmaf(A1, m, K2 * wrow);
    const float U = fmaf((1.0f + alpha) * (1.0f + 0x1p-16f), m, bet * (1.0f + 0x1p-16f) * wrow);
    const bool lb_ok = lb_all[wave][rs] > U && lh_all[wave][rs] >= U;
    const unsigned long long M0 = __ballot(scored && !(L0 > rhs)), M1 = __ballot(scored && !(L1 > rhs));
    const unsigned long long M2 = __ballot(scored && !(L2 > rhs)), M3 = __ballot(scored && !(L3 > rhs));
    // the row group's contenders: bit b of mk is code start + b (b = 8 t + j)
    const int sh = 8 * grp;
    const unsigned long long mk = ((M0 >> sh) & 0xFFull) | (((M1 >> sh) & 0xFFull) << 8) |
                                  (((M2 >> sh) & 0xFFull) << 16) | (((M3 >> sh) & 0xFFull) << 24);
    const int cnt = __popcll(mk);
    const bool ok = scored && lb_ok;
    const bool rescore = ok && cnt >= 2 && cnt <= 4;
    if (j == 0 && row_on) {
      if (!(ok && cnt >= 1 && cnt <= 4)) code[(g * cout + c_begin + rr) * nb + n] = 0;   // float64 pass
      win_k[wave][rr] = ok && cnt == 1 ? start + (int)__builtin_ctzll(mk) : 0;
      ctd_all[wave][rr] = rescore ? mk : 0ull;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // Rows with 2..4 contenders: exact float64 losses, one contender per 16 lanes (lane: element)
  {
    const unsigned long long todo0 = __ballot(lane < nrows && ctd_all[wave][lane < nrows ? lane : 0] != 0ull);
    for (unsigned long long todo = todo0; todo; todo &= todo - 1) {
      const int rq = (int)__builtin_ctzll(todo);
      const int st = st_all[wave][rq];
      unsigned long long mr = ctd_all[wave][rq];
      int kc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kc[r] = mr ? st + (int)__builtin_ctzll(mr) : 0;       // ascending codes, 0 past the last
        mr &= mr - 1;
      }
      const int rg = lane >> 4, el = lane & 15;              // contender rg, element el
      const int myk = rg == 0 ? kc[0] : (rg == 1 ? kc[1] : (rg == 2 ? kc[2] : kc[3]));
      int nib;
      const double e = exact_err(wt[rq][el], cand_scale(myk > 0 ? myk : 1, gsc), &nib);
      double z = (double)im_all[wave][el] * e * e;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
      double bestD = __builtin_inf();
      int kwin = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double Lr = __shfl(z, 16 * r, 64);
        if (kc[r] > 0 && (Lr < bestD || (Lr == bestD && kc[r] < kwin))) { bestD = Lr; kwin = kc[r]; }
      }
      if (lane == 0) win_k[wave][rq] = kwin;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // Exact nibbles and loss of every row's winner, eight rows at a time (as in k_sweep_diag).
  const int sub = lane & 7, el0 = 2 * sub, el1 = el0 + 1;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int rr = 8 * pass + (lane >> 3);
    const int64_t c = c_begin + rr;
    const bool row_on = rr < nrows;
    const int kw = row_on ? win_k[wave][rr] : 0;
    const float sw = cand_scale(kw > 0 ? kw : 1, gsc);
    const float wa = wt[rr][el0], wb = wt[rr][el1];
    const float ima = im_all[wave][el0], imb = im_all[wave][el1];
    const float is = __builtin_amdgcn_rcpf(sw);
    const float isp = is * (1.0f + 0x1p-19f), ism = is * (1.0f - 0x1p-19f);
    unsigned byte = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, wa * isp, wb * isp, 1.0f, 0);
    const unsigned blo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, wa * ism, wb * ism, 1.0f, 0);
    if (byte != blo) {
      const int ca = e2m1_index_fma(fabsf(wa), sw), cb = e2m1_index_fma(fabsf(wb), sw);
      byte = (unsigned)(ca | (wa < 0.0f ? 8 : 0)) | ((unsigned)(cb | (wb < 0.0f ? 8 : 0)) << 4);
    }
    const v2f qv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);   // signed grid values
    const float ea = fmaf(qv[0], sw, -wa), eb = fmaf(qv[1], sw, -wb);
    float part = fmaf(imb * eb, eb, ima * ea * ea);
    part += __shfl_xor(part, 1, 64);
    part += __shfl_xor(part, 2, 64);
    part += __shfl_xor(part, 4, 64);
    if (kw != 0) {
      if (fp4) fp4[(g * cout + c) * (cin / 2) + n * 8 + sub] = (uint8_t)byte;
      if (sub == 0) {
        code[(g * cout + c) * nb + n] = (uint8_t)kw;
        if (loss) loss[(g * cout + c) * nb + n] = part;
      }
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kWaves * 64) void k_sweep_diag_exact(
    const void* __restrict__ W, int64_t cout, int64_t cin, const float* __restrict__ amax,
    const float* __restrict__ imp, uint8_t* __restrict__ code, uint8_t* __restrict__ fp4,
    float* __restrict__ loss, const SweepOpts opt) {
  __shared__ int mk_all[kWaves][128];                 // codes proposed by the multipliers
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nb = cin / 16;
  // wave: rows c0 .. c0+kExactRows-1, block columns n0 .. n0+63 (see k_sweep_full_exact)
  const int64_t c0 = ((int64_t)blockIdx.x * kWaves + wave) * kExactRows;
  const int64_t n0 = (int64_t)blockIdx.y * 64;
  const int64_t g = blockIdx.z;
  const float gsc = global_scale(amax[g], opt.gdiv);
  const bool msearch = opt.nm > 0;
  float mu0 = 0.0f, mu1 = 0.0f;
  if (msearch) lane_multipliers(opt, lane, mu0, mu1);
  mk_all[wave][lane] = -1;
  mk_all[wave][lane + 64] = -1;
  const double g6 = 6.0 * (double)gsc, ig6 = 1.0 / g6;
  int tag = 0;
  const int64_t myn = n0 + lane;
  const unsigned undecided = undecided_rows(code, g, cout, nb, c0, myn);
  for (int r = 0; r < kExactRows; ++r) {
    const int64_t c = c0 + r;
    if (c >= cout) break;
    unsigned long long todo = __ballot((undecided >> r) & 1u);
    while (todo) {
      const int64_t n = n0 + __builtin_ctzll(todo);
      todo &= todo - 1;
      float im[16];
      double isum = 0.0;
  #pragma unroll
      for (int j = 0; j < 16; ++j) {
        im[j] = imp ? imp[g * cin + n * 16 + j] : 1.0f;
        isum += (double)im[j];
      }
      if (isum == 0.0) {
  #pragma unroll
        for (int j = 0; j < 16; ++j) im[j] = 1.0f;
      }
      const int64_t base = (g * cout + c) * cin + n * 16;
      float w[16];
      load_w16<BF16>(W, base, w);
      bool al[2] = {true, true};
      if (msearch) {
        float ab = 0.0f;
  #pragma unroll
        for (int j = 0; j < 16; ++j) ab = fmaxf(ab, fabsf(w[j]));
        mark_allowed(ab, g6, ig6, mu0, mu1, tag++, mk_all[wave], lane + 1, lane + 65, al[0], al[1]);
      }
      double best = __builtin_inf();
      int bestK = 1 << 20;
      for (int h = 0; h < 2; ++h) {
        const int k = lane + 1 + 64 * h;
        if (k > 126 || !al[h]) continue;
        const float sk = cand_scale(k, gsc);
        double Ls = 0.0;
        int nib;
  #pragma unroll
        for (int j = 0; j < 16; ++j) {
          const double e = exact_err(w[j], sk, &nib);
          Ls += (double)im[j] * e * e;
        }
        if (Ls < best) { best = Ls; bestK = k; }
      }
      wave_argmin_d(best, bestK);
      if (lane < 8 && fp4) {
        const float sw = cand_scale(bestK, gsc);
        int lo, hi;
        exact_err(load_w(W, BF16, base + 2 * lane), sw, &lo);
        exact_err(load_w(W, BF16, base + 2 * lane + 1), sw, &hi);
        fp4[(g * cout + c) * (cin / 2) + n * 8 + lane] = (uint8_t)(lo | (hi << 4));
      }
      if (lane == 0) {
        code[(g * cout + c) * nb + n] = (uint8_t)bestK;
        if (loss) loss[(g * cout + c) * nb + n] = (float)best;
      }
    }
  }
}

}  // namespace

hipError_t launch_sweep(const void* W, bool bf16, int64_t n_groups, int64_t cout, int64_t cin,
                        const float* amax, const float* H, const float* P, uint8_t* code,
                        uint8_t* fp4, float* loss, const SweepOpts& opt, float* mu, hipStream_t stream) {
  const int64_t nb = cin / 16;
  if (cout == 0) return hipSuccess;
  if (opt.nm == 0) {                               // the multiplier search scores every code
    const int64_t ncols = n_groups * nb;
    hipLaunchKernelGGL(k_column_mu, dim3((unsigned)((ncols + kWaves - 1) / kWaves)), dim3(kWaves * 64), 0, stream,
                       H, ncols, mu);
  }
  // a launch of at most four rounds of resident waves (4096 at a time) ends in a tail that the
  // progress-based priority shortens; longer launches keep the arbiter's own order, which mixes
  // phases better.  A launch of at most two rounds takes 64 rows per wave and runs as one; one of
  // more than 64 rounds takes 256 rows per wave, so each wave's column set-up serves more rows
  // (512-expert gate_up: 32 -> 128 rows 51.6 -> 46.2 ms when the set-up held the eigenvalue bound,
  // 128 -> 256 rows 38.17 -> 37.70 ms; 320 and 640 rows measured the same as 256).
  const int64_t waves32 = (nb + kWaves - 1) / kWaves * kWaves * ((cout + kRowsPerWave - 1) / kRowsPerWave) * n_groups;
  const bool equalize = waves32 <= 16384;
  const int rpw = waves32 > 262144 ? 8 * kRowsPerWave
                                   : ((waves32 <= 8192 && cout > kRowsPerWave) ? 2 * kRowsPerWave : kRowsPerWave);
  dim3 grid((unsigned)((nb + kWaves - 1) / kWaves), (unsigned)((cout + rpw - 1) / rpw), (unsigned)n_groups);
  dim3 block(kWaves * 64);
  // float64 pass: a wave per (kExactRows rows, 64 block columns)
  const dim3 xgrid((unsigned)((cout + kWaves * kExactRows - 1) / (kWaves * kExactRows)),
                   (unsigned)((nb + 63) / 64), (unsigned)n_groups);
#define LH_SWEEP_PAIR(B, C)                                                                        \
  if (opt.nm > 0)                                                                                  \
    hipLaunchKernelGGL((k_sweep_full<B, C, false, true>), grid, block, 0, stream, W, cout, cin, amax, \
                       H, P, code, fp4, loss, rpw, opt, mu);                                       \
  else if (equalize)                                                                               \
    hipLaunchKernelGGL((k_sweep_full<B, C, true, false>), grid, block, 0, stream, W, cout, cin, amax, \
                       H, P, code, fp4, loss, rpw, opt, mu);                                       \
  else                                                                                             \
    hipLaunchKernelGGL((k_sweep_full<B, C, false, false>), grid, block, 0, stream, W, cout, cin, amax, \
                       H, P, code, fp4, loss, rpw, opt, mu);                                       \
  hipLaunchKernelGGL((k_sweep_full_exact<B, C>), xgrid, block, 0, stream, W, cout, cin, amax, H, P, \
                     code, fp4, loss, opt)
  if (bf16 && P) {
    LH_SWEEP_PAIR(true, true);
  } else if (bf16) {
    LH_SWEEP_PAIR(true, false);
  } else if (P) {
    LH_SWEEP_PAIR(false, true);
  } else {
    LH_SWEEP_PAIR(false, false);
  }
#undef LH_SWEEP_PAIR
  return hipGetLastError();
}

hipError_t launch_accumulate_sweep(const void* X, const void* W, bool bf16, int64_t rows, int64_t cin,
                                   const int64_t* offsets, int64_t n_groups, int64_t cout, const float* amax,
                                   uint8_t* code, uint8_t* fp4, float* loss, const SweepOpts& opt,
                                   hipStream_t stream) {
  const int64_t nb = cin / 16;
  if (cout == 0) return hipSuccess;
  const int64_t R = stream::piece_rows(rows, nb);
  const dim3 grid((unsigned)((nb + 3) / 4), (unsigned)n_groups);
#define LH_FUSED(B, M)                                                                             \
  hipLaunchKernelGGL((k_moe_fused<B, M>), grid, dim3(kWaves * 64), 0, stream, X, W, rows, cin, cout,  \
                     offsets, R, amax, code, fp4, loss, opt)
  if (bf16) {
    if (opt.nm > 0) LH_FUSED(true, true); else LH_FUSED(true, false);
  } else {
    if (opt.nm > 0) LH_FUSED(false, true); else LH_FUSED(false, false);
  }
#undef LH_FUSED
  return hipGetLastError();
}

hipError_t launch_sweep_diag(const void* W, bool bf16, int64_t n_groups, int64_t cout,
                             int64_t cin, const float* amax, const float* imp, uint8_t* code,
                             uint8_t* fp4, float* loss, const SweepOpts& opt, hipStream_t stream) {
  const int64_t nb = cin / 16;
  if (cout == 0) return hipSuccess;
  dim3 grid((unsigned)((nb + kWaves - 1) / kWaves), (unsigned)((cout + kRowsPerWave - 1) / kRowsPerWave),
            (unsigned)n_groups);
  dim3 block(kWaves * 64);
  const dim3 xgrid((unsigned)((cout + kWaves * kExactRows - 1) / (kWaves * kExactRows)),
                   (unsigned)((nb + 63) / 64), (unsigned)n_groups);
#define LH_DIAG(B, M)                                                                              \
  if (M)                                                                                           \
    hipLaunchKernelGGL((k_sweep_diag<B, true>), grid, block, 0, stream, W, cout, cin, amax, imp, code, fp4, loss, opt); \
  else                                                                                             \
    hipLaunchKernelGGL((k_sweep_diag_win<B>), grid, block, 0, stream, W, cout, cin, amax, imp, code, fp4, loss, opt)
  if (bf16) {
    if (opt.nm > 0) LH_DIAG(true, true); else LH_DIAG(true, false);
    hipLaunchKernelGGL((k_sweep_diag_exact<true>), xgrid, block, 0, stream, W, cout, cin, amax, imp, code, fp4, loss, opt);
  } else {
    if (opt.nm > 0) LH_DIAG(false, true); else LH_DIAG(false, false);
    hipLaunchKernelGGL((k_sweep_diag_exact<false>), xgrid, block, 0, stream, W, cout, cin, amax, imp, code, fp4, loss, opt);
  }
#undef LH_DIAG
  return hipGetLastError();
}

}  // namespace lh
