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
//  * Full form: one wave per block, 16 candidates per MFMA tile (8 tiles = 128 lanes-candidates,
//    126 used).  Lane l owns candidate l%16 of the tile and elements 4*(l/16)..+3.  The lane
//    quantizes its 4 elements (r = w * (1/s) in fp32, then the gfx950 FP4 convert, which rounds
//    to nearest-even on the E2M1 grid and saturates at 6, and the FP4->fp32 convert back), forms
//    e = fma(q, s, -w), and four chained v_mfma_f32_16x16x4_f32 compute H e + 2b for the 16
//    candidates (H_n is the A operand, resident in registers for the whole column; the K index is
//    permuted so that each lane's output rows are exactly its own 4 elements).  The quadratic
//    form and an error bound are reduced across the 4 lane groups with two permlane swaps.
//    b = P_n w and |P_n||w| come from the same MFMA once per 16-row tile.
//  * Diagonal form: VALU only (no contraction to map onto MFMA); lane l scores candidates l+1 and
//    l+65 over all 16 elements, so no cross-lane reduction is needed until the argmin.
//  * Exactness.  The float32 pass is a filter: each candidate carries a rigorous bound c*A_k on
//    its rounding error (A_k = (sum|e_i| dmax_i)^2 + 2|e|^T(|P||w|), dmax_i^2 = max_j |H_ij|, or
//    L_k itself in the diagonal form).  If exactly one candidate can be the minimum, it is the
//    exact argmin.  Otherwise -- or when some |w_i|/s_k lies within a few ulps of an E2M1 rounding
//    midpoint, where the fp32 quotient could round the other way (detected once per block by
//    testing whether |w_i|/(m_j g) is near an E4M3 value) -- the block is re-scored in float64
//    with exact quotient rounding.  The result is the argmin of the float64 objective.
#include "lh_internal.hpp"

namespace lh {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;            // waves per workgroup; wave w takes block column 4*bx + w
constexpr int kRowsPerWave = 64;     // rows (blocks of one column) per wave
constexpr float kErrC = 0x1p-17f;    // filter error bound factor (about 3x the derived bound)
constexpr int kNearUlps = 16;        // midpoint proximity test, in ulps of |w|/(m g)

__device__ const float kMid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};

// Value of E4M3 byte k (1..126): 4 exponent bits (bias 7), 3 mantissa bits, subnormal below 2^-6.
__device__ inline double e4m3_value(int k) {
  const int e = k >> 3, m = k & 7;
  if (e == 0) return (double)m * 0x1p-9;
  return (double)(8 + m) * __longlong_as_double((long long)(e - 10 + 1023) << 52);
}

__device__ inline float global_scale(float amax) { return (float)((double)amax / 2688.0); }
__device__ inline float cand_scale(int k, float g) { return (float)(e4m3_value(k) * (double)g); }

// Exact E2M1 grid index of the quotient r = |w|/s given as float64 (ties to the even index).
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

// True when |w|/s_k may lie within a few ulps of an E2M1 midpoint for some candidate k.
__device__ inline bool near_midpoint(float aw, float inv_mg) {
  const float z = aw * inv_mg;
  if (!(z >= 0x1p-10f && z <= 480.0f)) return false;
  const unsigned t = (__float_as_uint(z) << 12) + ((unsigned)kNearUlps << 12);
  return t < ((unsigned)(2 * kNearUlps) << 12);
}

__device__ inline float load_w(const void* W, bool bf16, int64_t idx) {
  if (bf16) return __uint_as_float((unsigned)((const unsigned short*)W)[idx] << 16);
  return ((const float*)W)[idx];
}

// ------------------------------------------------------------------------------------------
// Full-Hessian sweep
// ------------------------------------------------------------------------------------------
struct WaveLds {
  float H[256];
  float P[256];
  float w[16][16];     // current 16-row tile: w[row][elem]
  float b2[16][16];    // 2 * (P w)[row][elem]
  float pw2[16][16];   // 2 * (|P| |w|)[row][elem]
  double wide[16];     // exact-path exchange
  int nib[16];
};

template <bool BF16, bool COUPLED>
__global__ __launch_bounds__(kWaves * 64) void k_sweep_full(
    const void* __restrict__ W, int64_t cout, int64_t cin, const float* __restrict__ amax,
    const float* __restrict__ Hg, const float* __restrict__ Pg, uint8_t* __restrict__ code,
    uint8_t* __restrict__ fp4, float* __restrict__ loss) {
  __shared__ WaveLds lds_all[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  WaveLds& L = lds_all[wave];
  const int i = lane & 15, gg = lane >> 4;
  const int64_t nb = cin / 16;
  const int64_t n = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t g = blockIdx.z;
  const int64_t c_begin = (int64_t)blockIdx.y * kRowsPerWave;
  if (n >= nb || c_begin >= cout) return;          // whole wave leaves; no workgroup barriers below
  const int64_t c_end = min(cout, c_begin + kRowsPerWave);

  // ---- column set-up: H_n (and P_n) into LDS and registers
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
  const bool dead = (tr == 0.0);                   // no activation energy: plain weight MSE
  const bool coupled = COUPLED && !dead;
  float a[4], dm[4], pa[4], pv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int col = 4 * gg + t;
    a[t] = dead ? (i == col ? 1.0f : 0.0f) : L.H[i * 16 + col];
    float mx = 0.0f;
    if (dead) mx = 1.0f;
    else
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fmaxf(fabsf(L.H[col * 16 + j]), fabsf(L.H[j * 16 + col])));
    dm[t] = sqrtf(mx) * 1.0000002f;               // sqrt rounding margin
    pv[t] = coupled ? L.P[i * 16 + col] : 0.0f;
    pa[t] = fabsf(pv[t]);
  }

  // ---- candidate scales for this lane's 8 tiles
  const float gsc = global_scale(amax[g]);
  const bool force_exact = !(gsc >= 0x1p-116f) || !(gsc <= 0x1p+100f);
  float s[8], is[8];
  bool valid[8];
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) {
    int k = 16 * tau + i + 1;
    valid[tau] = k <= 126;
    if (!valid[tau]) k = 126;
    s[tau] = cand_scale(k, gsc);
    is[tau] = s[tau] > 0.0f ? (float)(1.0 / (double)s[tau]) : 0.0f;
  }
  // midpoint proximity constants: this lane tests pairs p = lane and lane + 64 of (elem, midpoint)
  const int p0 = lane, p1 = lane + 64;
  const float img0 = (float)(1.0 / ((double)kMid[p0 % 7] * (double)gsc));
  const float img1 = p1 < 112 ? (float)(1.0 / ((double)kMid[p1 % 7] * (double)gsc)) : 0.0f;

  for (int64_t c0 = c_begin; c0 < c_end; c0 += 16) {
    // ---- 16-row tile: w, b = P w and |P||w| (MFMA, K index = element 4*gg + t)
    const int64_t crow = c0 + i;
    const bool row_on = crow < c_end;
    float wt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      wt[t] = row_on ? load_w(W, BF16, (g * cout + crow) * cin + n * 16 + 4 * gg + t) : 0.0f;
    v4f bt = {0.f, 0.f, 0.f, 0.f}, pwt = {0.f, 0.f, 0.f, 0.f};
    if (coupled) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bt = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[t], wt[t], bt, 0, 0, 0);
        pwt = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[t], fabsf(wt[t]), pwt, 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      L.w[i][4 * gg + t] = wt[t];
      L.b2[i][4 * gg + t] = 2.0f * bt[t];          // lane holds rows 4gg+t of column (row) i
      L.pw2[i][4 * gg + t] = 2.0f * pwt[t];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    const int rows_here = (int)min((int64_t)16, c_end - c0);
    for (int rr = 0; rr < rows_here; ++rr) {
      const int64_t c = c0 + rr;
      float w[4], twob[4], pw2[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w[t] = L.w[rr][4 * gg + t];
        twob[t] = L.b2[rr][4 * gg + t];
        pw2[t] = L.pw2[rr][4 * gg + t];
      }
      // midpoint proximity (exact-path trigger)
      bool near = near_midpoint(fabsf(L.w[rr][p0 / 7]), img0);
      if (p1 < 112) near = near || near_midpoint(fabsf(L.w[rr][p1 / 7]), img1);
      const bool flag = __ballot(near) != 0ull || force_exact;

      float bestL = __builtin_inff(), minUB = __builtin_inff(), LB[8];
      int bestK = 127;
      if (!flag) {
        const v4f cinit = {twob[0], twob[1], twob[2], twob[3]};
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) {
          const float r0 = w[0] * is[tau], r1 = w[1] * is[tau], r2 = w[2] * is[tau], r3 = w[3] * is[tau];
          unsigned pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, r0, r1, 1.0f, 0);
          pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, r2, r3, 1.0f, 1);
          const v2f q01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 0);
          const v2f q23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 1);
          const float e0 = fmaf(q01[0], s[tau], -w[0]);
          const float e1 = fmaf(q01[1], s[tau], -w[1]);
          const float e2 = fmaf(q23[0], s[tau], -w[2]);
          const float e3 = fmaf(q23[1], s[tau], -w[3]);
          v4f D = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], e0, cinit, 0, 0, 0);
          D = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], e1, D, 0, 0, 0);
          D = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], e2, D, 0, 0, 0);
          D = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], e3, D, 0, 0, 0);
          float lp = e0 * D[0];
          lp = fmaf(e1, D[1], lp);
          lp = fmaf(e2, D[2], lp);
          lp = fmaf(e3, D[3], lp);
          float sp = fabsf(e0) * dm[0];
          sp = fmaf(fabsf(e1), dm[1], sp);
          sp = fmaf(fabsf(e2), dm[2], sp);
          sp = fmaf(fabsf(e3), dm[3], sp);
          float ap = 4.0f * sp * sp;
          if (coupled) {
            float bp = fabsf(e0) * pw2[0];
            bp = fmaf(fabsf(e1), pw2[1], bp);
            bp = fmaf(fabsf(e2), pw2[2], bp);
            bp = fmaf(fabsf(e3), pw2[3], bp);
            ap += bp;
          }
          // reduce lp and ap over the 4 lane groups: lanes 0-31 end with L, 32-63 with A
          auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(lp), __float_as_uint(ap), false, false);
          float z = __uint_as_float(x[0]) + __uint_as_float(x[1]);
          auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
          z = __uint_as_float(y[0]) + __uint_as_float(y[1]);
          auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(z), __float_as_uint(z), false, false);
          const float Lk = __uint_as_float(u[0]);
          const float Ak = __uint_as_float(u[1]);
          if (valid[tau]) {
            LB[tau] = fmaf(-kErrC, Ak, Lk);
            minUB = fminf(minUB, fmaf(kErrC, Ak, Lk));
            if (Lk < bestL) { bestL = Lk; bestK = 16 * tau + i + 1; }
          } else {
            LB[tau] = __builtin_inff();
          }
        }
        // argmin and min upper bound over the 16 candidate lanes of a row
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float oL = __shfl_xor(bestL, o, 64);
          const int oK = __shfl_xor(bestK, o, 64);
          if (oL < bestL || (oL == bestL && oK < bestK)) { bestL = oL; bestK = oK; }
          minUB = fminf(minUB, __shfl_xor(minUB, o, 64));
        }
        int cnt = 0;
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) cnt += __popcll(__ballot(LB[tau] <= minUB) & 0xFFFFull);
        if (cnt != 1) bestK = -1;
      } else {
        bestK = -1;
      }

      const int64_t oblk = (g * cout + c) * nb + n;
      if (bestK > 0) {
        // unique float32 winner: emit its codes
        const float sw = cand_scale(bestK, gsc);
        const float iw = (float)(1.0 / (double)sw);
        unsigned pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, w[0] * iw, w[1] * iw, 1.0f, 0);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, w[2] * iw, w[3] * iw, 1.0f, 1);
        unsigned nb4 = pk & 0x7777u;                                   // magnitudes
        nb4 |= (w[0] < 0.0f ? 0x8u : 0u) | (w[1] < 0.0f ? 0x80u : 0u) |
               (w[2] < 0.0f ? 0x800u : 0u) | (w[3] < 0.0f ? 0x8000u : 0u);
        if (i == 0 && fp4) *(unsigned short*)(fp4 + (g * cout + c) * (cin / 2) + n * 8 + 2 * gg) = (unsigned short)nb4;
        if (lane == 0) {
          code[oblk] = (uint8_t)bestK;
          if (loss) loss[oblk] = bestL;
        }
      } else {
        // exact float64 re-scoring of all 126 candidates
        double wd[16], bd[16];
        for (int j = 0; j < 16; ++j) wd[j] = (double)L.w[rr][j];
        for (int r2 = 0; r2 < 16; ++r2) {
          double acc = 0.0;
          if (coupled)
            for (int j = 0; j < 16; ++j) acc += (double)L.P[r2 * 16 + j] * wd[j];
          bd[r2] = acc;
        }
        double bestD = __builtin_inf();
        int bestKD = 127;
        for (int h = 0; h < 2; ++h) {
          const int k = lane + 1 + 64 * h;
          if (k > 126) continue;
          const float sk = cand_scale(k, gsc);
          double e[16];
          int dummy;
          for (int j = 0; j < 16; ++j) e[j] = exact_err(L.w[rr][j], sk, &dummy);
          double Lsum = 0.0;
          for (int r2 = 0; r2 < 16; ++r2) {
            double y = 0.0;
            if (dead) y = e[r2];
            else
              for (int j = 0; j < 16; ++j) y += (double)L.H[r2 * 16 + j] * e[j];
            Lsum += e[r2] * (y + 2.0 * bd[r2]);
          }
          if (Lsum < bestD) { bestD = Lsum; bestKD = k; }
        }
        for (int o = 1; o < 64; o <<= 1) {
          const double oL = __shfl_xor(bestD, o, 64);
          const int oK = __shfl_xor(bestKD, o, 64);
          if (oL < bestD || (oL == bestD && oK < bestKD)) { bestD = oL; bestKD = oK; }
        }
        const float sw = cand_scale(bestKD, gsc);
        if (lane < 8) {
          int n0, n1;
          exact_err(L.w[rr][2 * lane], sw, &n0);
          exact_err(L.w[rr][2 * lane + 1], sw, &n1);
          if (fp4) fp4[(g * cout + c) * (cin / 2) + n * 8 + lane] = (uint8_t)(n0 | (n1 << 4));
        }
        if (lane == 0) {
          code[oblk] = (uint8_t)bestKD;
          if (loss) loss[oblk] = (float)bestD;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------------------------------------
// Diagonal (importance-weighted) sweep
// ------------------------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kWaves * 64) void k_sweep_diag(
    const void* __restrict__ W, int64_t cout, int64_t cin, const float* __restrict__ amax,
    const float* __restrict__ imp, uint8_t* __restrict__ code, uint8_t* __restrict__ fp4,
    float* __restrict__ loss) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nb = cin / 16;
  const int64_t n = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t g = blockIdx.z;
  const int64_t c_begin = (int64_t)blockIdx.y * kRowsPerWave;
  if (n >= nb || c_begin >= cout) return;
  const int64_t c_end = min(cout, c_begin + kRowsPerWave);

  float im[16];
  double isum = 0.0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    im[j] = imp[g * cin + n * 16 + j];
    isum += (double)im[j];
  }
  if (isum == 0.0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) im[j] = 1.0f;
  }
  const float gsc = global_scale(amax[g]);
  const bool force_exact = !(gsc >= 0x1p-116f) || !(gsc <= 0x1p+100f);
  const int k0 = lane + 1, k1 = lane + 65;
  const bool v1 = k1 <= 126;
  const float s0 = cand_scale(k0, gsc), s1 = cand_scale(v1 ? k1 : 126, gsc);
  const float is0 = s0 > 0.0f ? (float)(1.0 / (double)s0) : 0.0f;
  const float is1 = s1 > 0.0f ? (float)(1.0 / (double)s1) : 0.0f;
  const int p0 = lane, p1 = lane + 64;
  const float img0 = (float)(1.0 / ((double)kMid[p0 % 7] * (double)gsc));
  const float img1 = p1 < 112 ? (float)(1.0 / ((double)kMid[p1 % 7] * (double)gsc)) : 0.0f;

  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t base = (g * cout + c) * cin + n * 16;
    float w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = load_w(W, BF16, base + j);
    bool near = near_midpoint(fabsf(load_w(W, BF16, base + p0 / 7)), img0);
    if (p1 < 112) near = near || near_midpoint(fabsf(load_w(W, BF16, base + p1 / 7)), img1);
    const bool flag = __ballot(near) != 0ull || force_exact;

    float L0 = 0.0f, L1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      unsigned pk0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, w[j] * is0, w[j + 1] * is0, 1.0f, 0);
      pk0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk0, w[j] * is1, w[j + 1] * is1, 1.0f, 1);
      const v2f qa = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk0, 1.0f, 0);
      const v2f qb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk0, 1.0f, 1);
      const float ea0 = fmaf(qa[0], s0, -w[j]), ea1 = fmaf(qa[1], s0, -w[j + 1]);
      const float eb0 = fmaf(qb[0], s1, -w[j]), eb1 = fmaf(qb[1], s1, -w[j + 1]);
      L0 = fmaf(im[j] * ea0, ea0, L0);
      L0 = fmaf(im[j + 1] * ea1, ea1, L0);
      L1 = fmaf(im[j] * eb0, eb0, L1);
      L1 = fmaf(im[j + 1] * eb1, eb1, L1);
    }
    if (!v1) L1 = __builtin_inff();
    float bestL = L0;
    int bestK = k0;
    if (L1 < bestL) { bestL = L1; bestK = k1; }
    float minUB = fminf(L0 * (1.0f + kErrC), v1 ? L1 * (1.0f + kErrC) : __builtin_inff());
    for (int o = 1; o < 64; o <<= 1) {
      const float oL = __shfl_xor(bestL, o, 64);
      const int oK = __shfl_xor(bestK, o, 64);
      if (oL < bestL || (oL == bestL && oK < bestK)) { bestL = oL; bestK = oK; }
      minUB = fminf(minUB, __shfl_xor(minUB, o, 64));
    }
    const int cnt = __popcll(__ballot(L0 * (1.0f - kErrC) <= minUB)) +
                    __popcll(__ballot(v1 && L1 * (1.0f - kErrC) <= minUB));
    const int64_t oblk = (g * cout + c) * nb + n;
    float outL = bestL;
    if (flag || cnt != 1) {
      double bestD = __builtin_inf();
      int bestKD = 127;
      for (int h = 0; h < 2; ++h) {
        const int k = lane + 1 + 64 * h;
        if (k > 126) continue;
        const float sk = cand_scale(k, gsc);
        double Ls = 0.0;
        int dummy;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const double e = exact_err(w[j], sk, &dummy);
          Ls += (double)im[j] * e * e;
        }
        if (Ls < bestD) { bestD = Ls; bestKD = k; }
      }
      for (int o = 1; o < 64; o <<= 1) {
        const double oL = __shfl_xor(bestD, o, 64);
        const int oK = __shfl_xor(bestKD, o, 64);
        if (oL < bestD || (oL == bestD && oK < bestKD)) { bestD = oL; bestKD = oK; }
      }
      bestK = bestKD;
      outL = (float)bestD;
      if (lane < 8 && fp4) {
        const float sw = cand_scale(bestK, gsc);
        int n0, n1;
        exact_err(load_w(W, BF16, base + 2 * lane), sw, &n0);
        exact_err(load_w(W, BF16, base + 2 * lane + 1), sw, &n1);
        fp4[(g * cout + c) * (cin / 2) + n * 8 + lane] = (uint8_t)(n0 | (n1 << 4));
      }
    } else if (lane < 8 && fp4) {
      const float sw = cand_scale(bestK, gsc);
      const float iw = (float)(1.0 / (double)sw);
      const float wa = load_w(W, BF16, base + 2 * lane), wb = load_w(W, BF16, base + 2 * lane + 1);
      const unsigned pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, wa * iw, wb * iw, 1.0f, 0);
      unsigned byte = pk & 0x77u;
      byte |= (wa < 0.0f ? 0x8u : 0u) | (wb < 0.0f ? 0x80u : 0u);
      fp4[(g * cout + c) * (cin / 2) + n * 8 + lane] = (uint8_t)byte;
    }
    if (lane == 0) {
      code[oblk] = (uint8_t)bestK;
      if (loss) loss[oblk] = outL;
    }
  }
}

}  // namespace

hipError_t launch_sweep(const void* W, bool bf16, int64_t n_groups, int64_t cout, int64_t cin,
                        const float* amax, const float* H, const float* P, uint8_t* code,
                        uint8_t* fp4, float* loss, hipStream_t stream) {
  const int64_t nb = cin / 16;
  if (cout == 0) return hipSuccess;
  dim3 grid((unsigned)((nb + kWaves - 1) / kWaves), (unsigned)((cout + kRowsPerWave - 1) / kRowsPerWave),
            (unsigned)n_groups);
  dim3 block(kWaves * 64);
  if (bf16 && P)
    hipLaunchKernelGGL((k_sweep_full<true, true>), grid, block, 0, stream, W, cout, cin, amax, H, P, code, fp4, loss);
  else if (bf16)
    hipLaunchKernelGGL((k_sweep_full<true, false>), grid, block, 0, stream, W, cout, cin, amax, H, P, code, fp4, loss);
  else if (P)
    hipLaunchKernelGGL((k_sweep_full<false, true>), grid, block, 0, stream, W, cout, cin, amax, H, P, code, fp4, loss);
  else
    hipLaunchKernelGGL((k_sweep_full<false, false>), grid, block, 0, stream, W, cout, cin, amax, H, P, code, fp4, loss);
  return hipGetLastError();
}

hipError_t launch_sweep_diag(const void* W, bool bf16, int64_t n_groups, int64_t cout,
                             int64_t cin, const float* amax, const float* imp, uint8_t* code,
                             uint8_t* fp4, float* loss, hipStream_t stream) {
  const int64_t nb = cin / 16;
  if (cout == 0) return hipSuccess;
  dim3 grid((unsigned)((nb + kWaves - 1) / kWaves), (unsigned)((cout + kRowsPerWave - 1) / kRowsPerWave),
            (unsigned)n_groups);
  dim3 block(kWaves * 64);
  if (bf16)
    hipLaunchKernelGGL((k_sweep_diag<true>), grid, block, 0, stream, W, cout, cin, amax, imp, code, fp4, loss);
  else
    hipLaunchKernelGGL((k_sweep_diag<false>), grid, block, 0, stream, W, cout, cin, amax, imp, code, fp4, loss);
  return hipGetLastError();
}

}  // namespace lh
