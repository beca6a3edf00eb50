/*
 * lh.h -- C ABI of the MI355X (gfx950) local-Hessian NVFP4 weight-scale calibration library.
 *
 * The library computes, on one GPU, the two parts of local-Hessian-weighted NVFP4 weight-scale
 * calibration:
 *   1. per 16-wide input-channel block n, the local Hessian H_n = X[:,n]^T X[:,n] / B, the
 *      activation-aware cross matrix P_n = X_q^T (X_q - X) / B and the importance vector
 *      Imp_i = ||X[:,i]||^2;
 *   2. for every 16-element weight block, the exhaustive search over the 126 positive finite
 *      E4M3 block scales, scoring the E2M1 fake-quantization error e = quant(w) - w by
 *      e^T H_n e + 2 e^T (P_n w) (or sum_i Imp_i e_i^2) and keeping the argmin.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers, row-major and densely packed, owned by the caller.
 *     X, Xq and W must be 16-byte aligned (PyTorch allocations are); fp4 2-byte aligned.
 *     Inputs are never modified.  Outputs are fully overwritten (H, P and imp are read first
 *     only when beta != 0).
 *   - X is [rows, cin] (tokens x input channels, as a linear layer sees its input); W is
 *     [n_groups, cout, cin]; blocks run along cin in 16s (block n = channels 16n..16n+15).
 *   - Groups are MoE experts: rows [off[g], off[g+1]) of X belong to group g.  group_offsets is a
 *     device int64 array of n_groups+1 entries; pass NULL with n_groups == 1 for a dense layer
 *     (all rows).  Offsets must be non-decreasing with off[0] = 0 and off[n_groups] = rows; this is
 *     a caller contract (checking it would need a device read) and is not verified.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL = the null stream of
 *     the pointers' device).  The library never synchronizes the host, launches on the device that
 *     owns the pointers and restores the caller's current device.
 *   - Scratch memory, when an entry point needs it (accumulation partial sums and arrival
 *     counters), is a library-owned buffer per device, grown on demand in stream order from a
 *     device memory pool and kept between calls, so steady-state calls allocate nothing; calls
 *     on different streams are ordered through an event, so two calls never use it at once.
 *   - Return: LH_OK, or an error code with a message available from lh_last_error().  Argument
 *     checks run before any launch.  Faults inside kernels surface at the caller's next
 *     synchronization, as usual in HIP.  NaN or Inf in any input gives undefined results.
 *
 * Numerics
 *   - Accumulation reads bf16 or fp32 values exactly, multiplies them exactly (bf16) or in fp32
 *     (fp32 inputs), and sums in fp32 in a fixed order: results are bit-reproducible run to run.
 *   - The sweep returns the scale code and FP4 codes of the exact argmin of the float64 objective
 *     over all 126 candidates: a float32 pass scores each candidate that a proven lower bound does
 *     not rule out, with a rigorous error bound, and any block whose winner is not certain is
 *     re-scored in float64 with exact quantization.
 *
 * Citations are to the pages this library follows: "Add activation-aware local Hessian scale
 * calibration" (PR #1976), "add local hessian calibration" (PR #788), "Add WMSE weight scale
 * search calibration" (PR #2283) and "Add composable scale calibration to GPTQ" (PR #2004).
 */
#ifndef LH_H_
#define LH_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LH_VERSION 6

typedef enum {
  LH_OK = 0,
  LH_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, host or foreign-device pointer */
  LH_ERR_UNSUPPORTED = 2,      /* unknown dtype or no gfx950 device */
  LH_ERR_HIP = 3               /* a HIP runtime call or launch failed */
} lh_status;

/* The two sentinels widen the enum's value range to every 32-bit int: a value other than F32 or
 * BF16 coming from a caller is then a well-defined lh_dtype in C and C++, and every entry point
 * rejects it with LH_ERR_UNSUPPORTED.  They are not dtypes. */
typedef enum {
  LH_DTYPE_F32 = 0,
  LH_DTYPE_BF16 = 1,
  LH_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  LH_DTYPE_RANGE_MAX_ = 2147483647
} lh_dtype;

/*
 * Per-block local Hessian and importance (PR #788, Overview / Changes: per-block Hessians
 * collected by forward hooks; PR #2283, How: the diagonal path accumulates x.square().sum(-1)).
 *
 *   H[g][n]   = beta * H[g][n]   + (1/T_g) * sum_{t in g} x_t[n] x_t[n]^T     (if H != NULL)
 *   imp[g][i] = beta * imp[g][i] + sum_{t in g} X[t,i]^2                      (if imp != NULL)
 *
 * X        [rows, cin], dtype x_dtype.
 * H        [n_groups, cin/16, 16, 16] fp32 or NULL.      imp  [n_groups, cin] fp32 or NULL.
 * At least one of H, imp must be non-NULL.  T_g = off[g+1]-off[g]; T_g == 0 makes the sum term 0.
 * beta lets a caller stream token batches (beta = 1 with sums, or a running mean).
 * Errors: INVALID_ARGUMENT for rows < 0, cin <= 0 or cin % 16, n_groups < 1, NULL X with rows > 0,
 * both outputs NULL, offsets NULL with n_groups > 1, non-device or mixed-device pointers.
 */
lh_status lh_accumulate(const void* X, lh_dtype x_dtype, int64_t rows, int64_t cin,
                        const int64_t* group_offsets, int64_t n_groups, float beta,
                        float* H, float* imp, void* stream);

/*
 * lh_accumulate for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments, computation, results
 * (bit for bit) and errors as lh_accumulate, but the partial sums and arrival counters live in a
 * fixed array of 64 MiB per device that is part of the library's code object (each device the
 * library runs on holds it until the process ends), instead of the library's memory pool: the
 * call allocates nothing and records no event.  Every call on a device shares that device's
 * array, so calls that overlap on one device (other streams, graph replays in flight at once)
 * race and give wrong results; order them.  The arrival counters are cleared by a kernel at the
 * start of each call.  A problem that needs more scratch than the array holds (dense layers need
 * little; grouped rows need up to 2 * rows / R pieces x cin/64 slices x 4 KiB, R about
 * rows * cin / 262144 rows, between 64 and 1024) fails with INVALID_ARGUMENT before any launch.
 */
lh_status lh_accumulate_noalloc(const void* X, lh_dtype x_dtype, int64_t rows, int64_t cin,
                                const int64_t* group_offsets, int64_t n_groups, float beta,
                                float* H, float* imp, void* stream);

/*
 * Activation-aware Hessian and cross matrix (PR #1976, What does this PR do?):
 *   H[g][n] = beta*H[g][n] + X_q^T X_q / T_g,   P[g][n] = beta*P[g][n] + X_q^T (X_q - X) / T_g
 * per 16-channel block, over the rows of group g.  X and Xq are [rows, cin] of the same dtype.
 * P is formed from the difference D = X_q - X rounded once to fp32 (exact when X_q and X are
 * within a factor 2^15 of each other, as a fake-quant of X is; otherwise within 2^-24 of D) and
 * split exactly into bf16 pieces, never as the difference of two products.  H and P are both
 * required.  Errors as lh_accumulate.
 */
lh_status lh_accumulate_act_aware(const void* X, const void* Xq, lh_dtype dtype, int64_t rows,
                                  int64_t cin, const int64_t* group_offsets, int64_t n_groups,
                                  float beta, float* H, float* P, void* stream);

/*
 * The same H and P with X_q made from X inside the kernel, so the activations are read once
 * (PR #1976, What does this PR do?: X_q is the activation as the layer's NVFP4 input quantizer
 * emits it; the quantizer below is the NVFP4 recipe of PR #2004, What does this PR do?
 * (448-normalized), applied to activations per token):
 *   gX = fp32(x_amax[g] / (6*448)) per group;
 *   per row and 16-channel block: v = the E4M3 value (0 or one of the 126 positive finite values)
 *     nearest to max|x| / (6 gX), ties to the even code (so it saturates at 448 and a block whose
 *     max rounds to 0 becomes 0), s = fp32(v gX);
 *   x_q = sign(x) * E2M1(|x| / s) * s for each element (nearest of {0,0.5,1,1.5,2,3,4,6}, ties
 *     to the even grid index, saturating at 6; every rounding decision is the exact one), the
 *     product taken in fp32 and rounded to nearest-even bf16 when dtype is bf16.
 * x_amax [n_groups] fp32 device: the input quantizer's amax per group (>= 0 and finite; 0 gives
 * X_q = 0).  Other arguments, outputs and errors as lh_accumulate_act_aware, plus
 * INVALID_ARGUMENT for a NULL x_amax.
 */
lh_status lh_accumulate_act_aware_fq(const void* X, lh_dtype dtype, int64_t rows, int64_t cin,
                                     const int64_t* group_offsets, int64_t n_groups,
                                     const float* x_amax, float beta, float* H, float* P,
                                     void* stream);

/*
 * The activation fake-quant alone: writes X_q, the NVFP4 fake-quant of X that
 * lh_accumulate_act_aware_fq applies inside its kernel (same definition, same bits), for callers
 * that need the quantized activations themselves or feed lh_accumulate_act_aware (PR #1976, What
 * does this PR do?: X_q is what the layer's input quantizer emits).
 * X, Xq [rows, cin] of dtype (Xq is written, fully; it must not overlap X).  x_amax [n_groups]
 * fp32 device as in lh_accumulate_act_aware_fq; groups as everywhere (row r uses the amax of the
 * group that holds it).  Errors: INVALID_ARGUMENT for the shape checks of lh_accumulate, NULL
 * x_amax, NULL X or Xq with rows > 0, Xq == X, misaligned, non-device or mixed-device pointers.
 */
lh_status lh_activation_fake_quant(const void* X, lh_dtype dtype, int64_t rows, int64_t cin,
                                   const int64_t* group_offsets, int64_t n_groups, const float* x_amax,
                                   void* Xq, void* stream);

/*
 * Options of the weight-scale search, taken by the *_ex entry points (the others use the
 * defaults: 448-normalized scaling and all 126 candidates).
 *   scale_norm     the E4M3 value the global amax maps to: g = fp32(global_amax / (6 * scale_norm)).
 *                  448 is NVFP4's scaling, 256 that of its "4/6" variant ("Add composable scale
 *                  calibration to GPTQ", What does this PR do?: 448-normalized scaling, 4/6 uses
 *                  256).  It must be one of the 126 positive finite E4M3 values.
 *   n_multipliers  0: the FP8 scale sweep over all 126 candidates.  1..128: the amax-multiplier
 *                  search ("add local hessian calibration", Changes: configurable step size and
 *                  multipliers for the amax search): a block of amax a = max_i |w_i| takes only the
 *                  candidates whose code is the positive finite E4M3 value nearest to the exact
 *                  a * m / (6 g) for one of the multipliers m (ties to the even code, saturating
 *                  at 448 and at 2^-9), and keeps the lowest-loss one of those (lowest code on
 *                  ties, which is the first in an ascending grid).
 *   multipliers    HOST array of n_multipliers positive finite values, any order (a grid
 *                  start + j * step is the usual choice), read during the call.
 */
typedef struct {
  float scale_norm;
  int32_t n_multipliers;
  const float* multipliers;
} lh_sweep_options;

/*
 * Exhaustive FP8 block-scale sweep with the local-Hessian objective (PR #788, review: block loss
 * cnb,nbd,cnd->cn; PR #1976, review: dw = quant(w) - w, coupling term 2 dw^T (P W0) with
 * P.W0 = nbd,cnd->cnb, best_loss = inf so negative losses are handled; PR #2283, How: the 126
 * candidate scales; PR #2004: NVFP4 scaling is 448-normalized).
 *
 * For every block (g, c, n) with weights w = W[g][c][16n..16n+15]:
 *   g_g  = fp32(global_amax[g] / (6*448))
 *   s_k  = fp32(v_k * g_g), v_k the E4M3 value of byte k, k = 0x01..0x7E (126 candidates)
 *   q_k  = E2M1 fake-quant of w with scale s_k: each |w_i|/s_k (exact quotient) is rounded to the
 *          nearest of {0,0.5,1,1.5,2,3,4,6}, ties to the even grid index, saturating at 6
 *   e_k  = q_k - w,  L_k = e_k^T H_n e_k + 2 e_k^T (P_n w)      (P == NULL: no cross term)
 *   k*   = argmin_k L_k, lowest code on ties.
 * A block whose H_n has zero trace (no activation energy) is scored with H = I and no cross term.
 *
 * W           [n_groups, cout, cin] dtype w_dtype.
 * global_amax [n_groups] fp32 device, >= 0 and finite (normally max |W_g|, see lh_absmax).
 * H, P        [n_groups, cin/16, 16, 16] fp32 (P may be NULL).
 * scale_code  [n_groups, cout, cin/16] uint8: the E4M3 byte k* (0x01..0x7E).
 * fp4         [n_groups, cout, cin/2] uint8 or NULL: nibble = (w < 0) << 3 | grid index,
 *             element 2j in the low nibble of byte j.
 * best_loss   [n_groups, cout, cin/16] fp32 or NULL: L_{k*} (may be negative with P).
 * Errors: INVALID_ARGUMENT for n_groups outside [1, 65535], cout outside [0, 2097120], cin <= 0
 * or cin % 16, NULL required pointers, non-device or mixed-device pointers.
 */
lh_status lh_scale_sweep(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                         int64_t cin, const float* global_amax, const float* H, const float* P,
                         uint8_t* scale_code, uint8_t* fp4, float* best_loss, void* stream);

/*
 * lh_scale_sweep with options (see lh_sweep_options; NULL = the defaults, identical to
 * lh_scale_sweep).  Errors as lh_scale_sweep, plus INVALID_ARGUMENT for a scale_norm that is not
 * a positive finite E4M3 value, n_multipliers outside [0, 128], a NULL multipliers array with
 * n_multipliers > 0, or a multiplier that is not positive and finite.
 */
lh_status lh_scale_sweep_ex(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                            int64_t cin, const float* global_amax, const float* H, const float* P,
                            const lh_sweep_options* options, uint8_t* scale_code, uint8_t* fp4,
                            float* best_loss, void* stream);

/*
 * Accumulation and sweep of grouped rows (MoE experts) in one launch, the Hessians kept on chip:
 * per expert, the per-block Hessian of its routed rows and the weight-scale search of its weight
 * matrix against it, without writing H to memory ("[2/3] Speed up layerwise GPTQ on MoE models",
 * embedded #2840 text: one Hessian per expert and projection, over exactly the tokens routed to
 * it; its size per MoE layer is what makes such calibration memory-bound).
 *   H[g][n] = (1/T_g) sum_{t in g} x_t[n] x_t[n]^T   (as lh_accumulate, beta = 0)
 *   then the search of lh_scale_sweep_ex on W[g] with H[g], P = NULL and `options`.
 * For n_groups >= 2 each H is summed in the order lh_accumulate's grouped path uses, so codes,
 * nibbles and losses are bit-identical to lh_accumulate followed by lh_scale_sweep_ex; with one
 * group lh_accumulate takes its dense path, whose order differs (results agree within its
 * rounding).  A group without rows gets H = 0, i.e. the plain weight-MSE search.
 * X [rows, cin] and W [n_groups, cout, cin] of dtype; group_offsets as everywhere (NULL with one
 * group); global_amax [n_groups]; outputs as lh_scale_sweep.
 * Errors: those of lh_accumulate and lh_scale_sweep_ex, plus INVALID_ARGUMENT for cout > 8192.
 */
lh_status lh_accumulate_sweep(const void* X, const void* W, lh_dtype dtype, int64_t rows, int64_t cin,
                              const int64_t* group_offsets, int64_t n_groups, int64_t cout,
                              const float* global_amax, const lh_sweep_options* options,
                              uint8_t* scale_code, uint8_t* fp4, float* best_loss, void* stream);

/*
 * Same sweep scored by the importance-weighted error L_k = sum_i imp[g][16n+i] * e_{k,i}^2
 * (PR #2283, What / How: H replaced by diag(Imp), einsum cnb,nb->cn, no diag_embed and no
 * matmul on the hot path).  A block whose importance sums to zero uses Imp = 1.
 * imp [n_groups, cin] fp32.  Other arguments and errors as lh_scale_sweep.
 */
lh_status lh_scale_sweep_diag(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                              int64_t cin, const float* global_amax, const float* imp,
                              uint8_t* scale_code, uint8_t* fp4, float* best_loss, void* stream);

/*
 * Same sweep scored by the plain squared error L_k = sum_i e_{k,i}^2 (H = I, no activations): the
 * weight-only "mse" calibration that "Add WMSE weight scale search calibration" runs as its control
 * arm (verification: mse control; Ablation table: mse rows).  Equal to lh_scale_sweep_diag with
 * every importance 1 and to lh_scale_sweep with H_n = I, P = NULL.  Arguments and errors as
 * lh_scale_sweep_diag without imp.
 */
lh_status lh_scale_sweep_mse(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                             int64_t cin, const float* global_amax, uint8_t* scale_code, uint8_t* fp4,
                             float* best_loss, void* stream);

/*
 * lh_scale_sweep_diag with options (see lh_sweep_options); imp may be NULL for the plain-MSE
 * objective of lh_scale_sweep_mse.  Errors as lh_scale_sweep_ex.
 */
lh_status lh_scale_sweep_diag_ex(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                                 int64_t cin, const float* global_amax, const float* imp,
                                 const lh_sweep_options* options, uint8_t* scale_code, uint8_t* fp4,
                                 float* best_loss, void* stream);

/*
 * Fake-quantized weights and per-block amax from a sweep's result: the calibrated quantizer state
 * ("Add WMSE weight scale search calibration": the shared-path check fingerprints the quantizers'
 * amax and scales and the final fake-quantized weights):
 *   s_k  = fp32(v_k * fp32(global_amax[g] / (6*448)))  for the block's code k (the sweep's scale)
 *   Wq[g][c][16n+j] = sign * E2M1 value of nibble j * s_k, rounded to fp32 and, for a bf16
 *                     out_dtype, to nearest-even bf16 (a negative value that quantized to 0
 *                     gives -0)
 *   block_amax[g][c][n] = fp32(6 * s_k)
 * scale_code [n_groups, cout, cin/16] u8 and fp4 [n_groups, cout, cin/2] u8 as lh_scale_sweep
 * writes them (codes 0x01..0x7E); global_amax [n_groups] fp32; Wq [n_groups, cout, cin] in
 * out_dtype or NULL (16-byte aligned); block_amax [n_groups, cout, cin/16] fp32 or NULL.
 * Errors: INVALID_ARGUMENT for shapes as lh_scale_sweep, NULL scale_code or global_amax, both
 * outputs NULL, NULL fp4 with Wq, misaligned pointers, non-device or mixed-device pointers.
 */
lh_status lh_dequantize(const uint8_t* scale_code, const uint8_t* fp4, lh_dtype out_dtype,
                        int64_t n_groups, int64_t cout, int64_t cin, const float* global_amax,
                        void* Wq, float* block_amax, void* stream);

/*
 * lh_dequantize for codes a sweep chose under scale_norm (see lh_sweep_options):
 * s_k = fp32(v_k * fp32(global_amax[g] / (6 * scale_norm))).  Errors as lh_dequantize, plus
 * INVALID_ARGUMENT for a scale_norm that is not a positive finite E4M3 value.
 */
lh_status lh_dequantize_ex(const uint8_t* scale_code, const uint8_t* fp4, lh_dtype out_dtype,
                           int64_t n_groups, int64_t cout, int64_t cin, const float* global_amax,
                           float scale_norm, void* Wq, float* block_amax, void* stream);

/*
 * Per-group absolute maximum amax_out[g] = max |W_g| over elems_per_group elements: the max
 * calibration that fixes the weight's global amax before the search (PR #788, Sequence diagram:
 * initial max_calibrate).  W is [n_groups, elems_per_group]; an empty group gives 0.
 * Errors: INVALID_ARGUMENT for n_groups < 1, elems_per_group < 0, NULL pointers, non-device or
 * mixed-device pointers.
 */
lh_status lh_absmax(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t elems_per_group,
                    float* amax_out, void* stream);

/* Message of the last error on the calling thread ("" if none); valid until its next call. */
const char* lh_last_error(void);

/* LH_VERSION of the built library. */
int lh_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LH_H_ */
