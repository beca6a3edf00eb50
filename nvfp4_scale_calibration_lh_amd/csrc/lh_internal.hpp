// Internal declarations shared by the C-ABI shim and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lh {

// Scratch of one launch_accumulate call: a work area (partial sums of row ranges that are added
// across workgroups) and arrival counters.  The counters must be
// zero when a call starts and are zero again when it ends.  launch_accumulate checks the sizes it
// is given against this and launches nothing if they are short.
struct AccScratch {
  size_t work_bytes;
  size_t counters;
};
AccScratch accumulate_scratch(int64_t rows, int64_t nb, const int64_t* offsets, int64_t n_groups,
                              bool bf16, bool act_aware, bool imp_only);

// Sets n words at p to zero (a kernel, so that graph capture records no memset node).
hipError_t launch_zero_fill(unsigned* p, size_t n, hipStream_t stream);

hipError_t launch_absmax(const void* W, bool bf16, int64_t n_groups, int64_t elems, float* amax,
                         hipStream_t stream);

// Activation-aware: X and Xq given, or X and x_amax (X_q made from X in the kernel, Xq ==
// nullptr); H and P required.  Otherwise Xq == x_amax == nullptr and H and/or imp given.
hipError_t launch_accumulate(const void* X, const void* Xq, const float* x_amax, bool bf16,
                             int64_t rows, int64_t cin, const int64_t* offsets, int64_t n_groups,
                             float beta, float* H, float* P, float* imp, void* work,
                             size_t work_bytes, unsigned* counters, size_t n_counters,
                             hipStream_t stream);

// X_q = the activations' NVFP4 fake-quant (the one the FQ accumulation applies), written to Xq.
hipError_t launch_act_fake_quant(const void* X, bool bf16, int64_t rows, int64_t cin, const int64_t* offsets,
                                 int64_t n_groups, const float* x_amax, void* Xq, hipStream_t stream);

// Options of one sweep launch, passed to the kernels by value: the divisor of the global scale,
// g = fp32(amax / gdiv) with gdiv = 6 * norm (norm an E4M3 value, so gdiv is exact in fp32), and
// the amax-multiplier grid (nm = 0: every one of the 126 candidates; otherwise a block takes only
// the codes its nm multipliers propose).
constexpr int kMaxMultipliers = 128;
struct SweepOpts {
  float gdiv;
  int nm;
  float mult[kMaxMultipliers];
};

// mu: device scratch of n_groups * cin/16 floats (each block column's Hessian eigenvalue bound,
// written and read by the launch).
hipError_t launch_sweep(const void* W, bool bf16, int64_t n_groups, int64_t cout, int64_t cin,
                        const float* amax, const float* H, const float* P, uint8_t* code,
                        uint8_t* fp4, float* loss, const SweepOpts& opts, float* mu, hipStream_t stream);

hipError_t launch_sweep_diag(const void* W, bool bf16, int64_t n_groups, int64_t cout,
                             int64_t cin, const float* amax, const float* imp, uint8_t* code,
                             uint8_t* fp4, float* loss, const SweepOpts& opts, hipStream_t stream);

// Hessians of grouped rows (n_groups >= 1, offsets device int64[n_groups+1] or NULL for one
// group) made in LDS and swept at once; outputs as launch_sweep with P = NULL.  cout <= kFusedMaxCout.
constexpr int kFusedMaxCout = 8192;
hipError_t launch_accumulate_sweep(const void* X, const void* W, bool bf16, int64_t rows, int64_t cin,
                                   const int64_t* offsets, int64_t n_groups, int64_t cout, const float* amax,
                                   uint8_t* code, uint8_t* fp4, float* loss, const SweepOpts& opts,
                                   hipStream_t stream);

// Wq (bf16 or fp32, may be NULL) and block_amax (may be NULL) from scale codes and FP4 nibbles;
// g = fp32(amax / gdiv) as in the sweep.
hipError_t launch_dequantize(const uint8_t* code, const uint8_t* fp4, const float* amax, int64_t n_groups,
                             int64_t cout, int64_t cin, bool bf16, void* Wq, float* block_amax, float gdiv,
                             hipStream_t stream);

}  // namespace lh
