// Fake-quantized weights and per-block amax from the sweep's result: the quantizer state that
// calibration leaves behind ("Add WMSE weight scale search calibration": the refactor check
// compares the quantizers' amax and scales and the final fake-quantized weights bit for bit).
//
//   g   = fp32(global_amax[g] / (6*norm)),  s = fp32(v_code * g)  (the sweep's own scale; norm
//         448, or 256 for the "4/6" variant of "Add composable scale calibration to GPTQ")
//   Wq  = sign * E2M1 value of the nibble * s, rounded to fp32, then to nearest-even bf16 for a
//         bf16 output
//   block_amax = fp32(6 s)
//
// HBM-bound: one thread per 16-element block reads its code byte and 8 nibble bytes and writes
// 32 (bf16) or 64 (fp32) bytes with 16-byte stores; consecutive threads own consecutive blocks.
#include "lh_internal.hpp"

namespace lh {
namespace {

constexpr int kThreads = 256;
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// E4M3 value of byte k (exponent field 0: m * 2^-9; otherwise (1 + m/8) * 2^(e-7)), exact.
__device__ inline double e4m3_byte_value(unsigned k) {
  const unsigned e = (k >> 3) & 15u, m = k & 7u;
  return e == 0 ? (double)m * 0x1p-9 : ldexp(1.0 + (double)m * 0.125, (int)e - 7);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_dequantize(const uint8_t* __restrict__ code,
                                                         const uint8_t* __restrict__ fp4,
                                                         const float* __restrict__ amax,
                                                         int64_t per_group, int64_t n_blocks,
                                                         void* __restrict__ Wq,
                                                         float* __restrict__ block_amax, float gdiv) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= n_blocks) return;
  const int64_t g = b / per_group;
  const float gs = (float)((double)amax[g] / (double)gdiv);
  const float s = (float)(e4m3_byte_value(code[b]) * (double)gs);
  if (block_amax) block_amax[b] = 6.0f * s;
  if (!Wq) return;
  const uint2 nib = *(const uint2*)(fp4 + b * 8);      // 16 nibbles, element 2j low in byte j
  float q[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const unsigned w = h == 0 ? nib.x : nib.y;
    auto dec = [&](auto sel) {                          // the convert's byte select is an immediate
      constexpr int p = decltype(sel)::value;
      const v2f v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, p);   // signed grid values
      q[8 * h + 2 * p] = v[0] * s;
      q[8 * h + 2 * p + 1] = v[1] * s;
    };
    dec(std::integral_constant<int, 0>{});
    dec(std::integral_constant<int, 1>{});
    dec(std::integral_constant<int, 2>{});
    dec(std::integral_constant<int, 3>{});
  }
  if (BF16) {
    v4u o[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const v2bf v = __builtin_convertvector((v2f){q[2 * j], q[2 * j + 1]}, v2bf);   // nearest-even
      o[j / 4][j % 4] = __builtin_bit_cast(unsigned, v);
    }
    v4u* out = (v4u*)((unsigned short*)Wq + b * 16);
    out[0] = o[0];
    out[1] = o[1];
  } else {
    v4u* out = (v4u*)((float*)Wq + b * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[j] = v4u{__float_as_uint(q[4 * j]), __float_as_uint(q[4 * j + 1]), __float_as_uint(q[4 * j + 2]),
                   __float_as_uint(q[4 * j + 3])};
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* code, const uint8_t* fp4, const float* amax, int64_t n_groups,
                             int64_t cout, int64_t cin, bool bf16, void* Wq, float* block_amax, float gdiv,
                             hipStream_t stream) {
  const int64_t per_group = cout * (cin / 16), n = n_groups * per_group;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
  if (bf16)
    hipLaunchKernelGGL(k_dequantize<true>, grid, dim3(kThreads), 0, stream, code, fp4, amax, per_group, n, Wq, block_amax, gdiv);
  else
    hipLaunchKernelGGL(k_dequantize<false>, grid, dim3(kThreads), 0, stream, code, fp4, amax, per_group, n, Wq, block_amax, gdiv);
  return hipGetLastError();
}

}  // namespace lh
