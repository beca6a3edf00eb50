// Internal declarations shared by the C-ABI shim and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lh {

// Rows of X processed by one accumulation workgroup (a "tile"); a group (MoE expert) that spans
// several tiles leaves partial sums in scratch memory that a second kernel combines in tile order.
constexpr int kAccTileRows = 256;

// Scratch floats needed by launch_accumulate for `rows` rows and `nb` 16-channel blocks
// (two partial-sum slots per tile, one or two 16x16 matrices per slot).
size_t accumulate_scratch_floats(int64_t rows, int64_t nb, bool act_aware);

hipError_t launch_absmax(const void* W, bool bf16, int64_t n_groups, int64_t elems, float* amax,
                         hipStream_t stream);

// act_aware: X and Xq given; H and P required.  Otherwise Xq == nullptr and H and/or imp given.
hipError_t launch_accumulate(const void* X, const void* Xq, bool bf16, int64_t rows, int64_t cin,
                             const int64_t* offsets, int64_t n_groups, float beta, float* H,
                             float* P, float* imp, float* scratch, hipStream_t stream);

hipError_t launch_sweep(const void* W, bool bf16, int64_t n_groups, int64_t cout, int64_t cin,
                        const float* amax, const float* H, const float* P, uint8_t* code,
                        uint8_t* fp4, float* loss, hipStream_t stream);

hipError_t launch_sweep_diag(const void* W, bool bf16, int64_t n_groups, int64_t cout,
                             int64_t cin, const float* amax, const float* imp, uint8_t* code,
                             uint8_t* fp4, float* loss, hipStream_t stream);

}  // namespace lh
