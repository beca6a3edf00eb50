// Per-group max |W| (the max calibration that fixes each weight matrix's global amax before the
// scale search; "add local hessian calibration", Sequence diagram: initial max_calibrate).
//
// HBM-bound streaming reduction.  |x| is compared on raw bit patterns with the sign bit cleared
// (for finite values the unsigned order of those bits is the order of the magnitudes), so the
// bf16 path never converts to float and the result is exact and order-independent.  Workgroups
// combine with an unsigned atomicMax on the output word, which an init kernel sets to 0 first.
#include "lh_internal.hpp"

#include <algorithm>

namespace lh {
namespace {

constexpr int kThreads = 256;       // scalar path
constexpr int kVecThreads = 1024;   // vector path: 16 waves per workgroup
typedef unsigned v4u __attribute__((ext_vector_type(4)));

__global__ void k_absmax_init(unsigned* out, int64_t n) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) out[i] = 0u;
}

__device__ inline unsigned wave_max(unsigned v) {
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, o, 64));
  return v;
}

// Vector path: each thread reads 16 bytes per step (8 bf16 or 4 fp32).  Requires the group's
// base to be 16-byte aligned and elems to be a multiple of the vector width.
template <bool BF16>
__global__ __launch_bounds__(kVecThreads) void k_absmax_vec(const v4u* __restrict__ W,
                                                         int64_t vec_per_group, unsigned* out) {
  const int g = blockIdx.y;
  const v4u* base = W + (int64_t)g * vec_per_group;
  auto absmax16 = [](const v4u v) -> unsigned {       // largest |x| of the 16 bytes, as bits
    if (BF16) {
      const unsigned a = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
      const unsigned b = max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu));
      return max(a, b) << 16;
    }
    return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
  };
  unsigned m = 0;
  const int64_t stride = (int64_t)gridDim.x * kVecThreads;
  int64_t i = blockIdx.x * (int64_t)kVecThreads + threadIdx.x;
  for (; i + 7 * stride < vec_per_group; i += 8 * stride) {   // eight loads in flight
    v4u v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(base + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = max(m, absmax16(v[k]));
  }
  for (; i < vec_per_group; i += stride) m = max(m, absmax16(__builtin_nontemporal_load(base + i)));
  __shared__ unsigned red[kVecThreads / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = red[0];
    for (int w = 1; w < kVecThreads / 64; ++w) r = max(r, red[w]);
    if (r) atomicMax(out + g, r);
  }
}

// Scalar path for unaligned or ragged groups.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_absmax_scalar(const void* __restrict__ W,
                                                            int64_t elems, unsigned* out) {
  const int g = blockIdx.y;
  unsigned m = 0;
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < elems;
       i += (int64_t)gridDim.x * kThreads) {
    if (BF16) {
      unsigned short b = ((const unsigned short*)W)[(int64_t)g * elems + i];
      m = max(m, ((unsigned)b & 0x7FFFu) << 16);
    } else {
      m = max(m, ((const unsigned*)W)[(int64_t)g * elems + i] & 0x7FFFFFFFu);
    }
  }
  __shared__ unsigned red[kThreads / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = max(r, red[w]);
    if (r) atomicMax(out + g, r);
  }
}

}  // namespace

hipError_t launch_absmax(const void* W, bool bf16, int64_t n_groups, int64_t elems, float* amax,
                         hipStream_t stream) {
  unsigned* out = reinterpret_cast<unsigned*>(amax);
  hipLaunchKernelGGL(k_absmax_init, dim3((unsigned)((n_groups + 255) / 256)), dim3(256), 0, stream,
                     out, n_groups);
  if (elems == 0) return hipGetLastError();
  const int vec = bf16 ? 8 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(W) % 16 == 0) && (elems % vec == 0);
  const int64_t units = aligned ? elems / vec : elems;
  // about 32 units per thread (so a workgroup's reduction and atomic serve 512 KiB of bf16: 512
  // experts' gate_up 0.597 -> 0.575 ms against 8 units), but at least ~1024 workgroups in all when
  // the groups are few (and at least one unit per thread); at most 256 workgroups (and as many
  // atomics) per group
  const int64_t tpb = aligned ? kVecThreads : kThreads;
  int64_t bx = std::max((units + tpb * 32 - 1) / (tpb * 32), (1024 + n_groups - 1) / n_groups);
  bx = std::min(bx, (units + tpb - 1) / tpb);
  if (bx < 1) bx = 1;
  if (bx > 256) bx = 256;
  dim3 grid((unsigned)bx, (unsigned)n_groups);
  if (aligned) {
    if (bf16)
      hipLaunchKernelGGL(k_absmax_vec<true>, grid, dim3(kVecThreads), 0, stream, (const v4u*)W, units, out);
    else
      hipLaunchKernelGGL(k_absmax_vec<false>, grid, dim3(kVecThreads), 0, stream, (const v4u*)W, units, out);
  } else {
    if (bf16)
      hipLaunchKernelGGL(k_absmax_scalar<true>, grid, dim3(kThreads), 0, stream, W, elems, out);
    else
      hipLaunchKernelGGL(k_absmax_scalar<false>, grid, dim3(kThreads), 0, stream, W, elems, out);
  }
  return hipGetLastError();
}

}  // namespace lh
