// C ABI of the calibration library (declarations and contracts in include/lh.h).
//
// This file validates arguments before anything is launched, selects the device that owns the
// pointers (restoring the caller's current device), keeps per-device accumulation scratch memory
// (from a library-owned stream-ordered pool) that calls hand on in stream order, and launches the
// kernels on the caller's stream.  Its only other state is a thread-local error message.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/lh.h"
#include "lh_internal.hpp"

namespace {

thread_local std::string g_last_error;

lh_status fail(lh_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

lh_status ok() {
  g_last_error.clear();
  return LH_OK;
}

lh_status hip_fail(hipError_t e, const char* what) {
  (void)hipGetLastError();  // clear the sticky launch error so the caller's next call is clean
  return fail(LH_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int d) { return d == LH_DTYPE_F32 || d == LH_DTYPE_BF16; }

// Device that owns `p`, or -1 (with the error message set) if p is not device memory.
int device_of(const void* p, const char* name) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    fail(LH_ERR_INVALID_ARGUMENT, "%s is not a device pointer (%s)", name, hipGetErrorString(e));
    return -1;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) {
    fail(LH_ERR_INVALID_ARGUMENT, "%s is not device memory", name);
    return -1;
  }
  return attr.device;
}

struct PtrCheck {
  const void* p;
  const char* name;
};

// All non-null pointers must be device memory of one device, 16-byte aligned where required.
lh_status check_pointers(std::initializer_list<PtrCheck> ptrs, int* dev_out) {
  int dev = -1;
  for (const PtrCheck& c : ptrs) {
    if (!c.p) continue;
    int d = device_of(c.p, c.name);
    if (d < 0) return LH_ERR_INVALID_ARGUMENT;
    if (dev >= 0 && d != dev) return fail(LH_ERR_INVALID_ARGUMENT, "%s is on device %d, other pointers on device %d", c.name, d, dev);
    dev = d;
  }
  if (dev < 0) return fail(LH_ERR_INVALID_ARGUMENT, "no device pointer given");
  *dev_out = dev;
  return LH_OK;
}

lh_status check_aligned(const void* p, const char* name) {
  if (p && (reinterpret_cast<uintptr_t>(p) % 16) != 0)
    return fail(LH_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  return LH_OK;
}

// Switches to `dev` for the lifetime of the guard and checks that it is a gfx950 device.
class DeviceGuard {
 public:
  lh_status enter(int dev) {
    hipError_t e = hipGetDevice(&prev_);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (prev_ != dev) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
      switched_ = true;
    }
    static std::mutex mu;
    static std::vector<int> arch_ok(64, -1);
    std::lock_guard<std::mutex> lk(mu);
    if (dev < 0 || dev >= (int)arch_ok.size()) return fail(LH_ERR_UNSUPPORTED, "device %d out of range", dev);
    if (arch_ok[dev] < 0) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
      arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    }
    if (!arch_ok[dev]) return fail(LH_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X)", dev);
    return LH_OK;
  }
  ~DeviceGuard() {
    if (switched_) (void)hipSetDevice(prev_);
  }

 private:
  int prev_ = 0;
  bool switched_ = false;
};

// One stream-ordered pool per device; its release threshold keeps freed scratch for reuse.
hipError_t scratch_pool(int dev, hipMemPool_t* pool) {
  static std::mutex mu;
  static std::vector<hipMemPool_t> pools(64, nullptr);
  std::lock_guard<std::mutex> lk(mu);
  if (dev < 0 || dev >= (int)pools.size()) return hipErrorInvalidDevice;
  if (!pools[dev]) {
    hipMemPoolProps props;
    std::memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p;
    hipError_t e = hipMemPoolCreate(&p, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = ~0ull;
    e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) return e;
    pools[dev] = p;
  }
  *pool = pools[dev];
  return hipSuccess;
}

lh_status check_shapes_x(int64_t rows, int64_t cin, const int64_t* offsets, int64_t n_groups) {
  if (rows < 0) return fail(LH_ERR_INVALID_ARGUMENT, "rows must be >= 0 (got %lld)", (long long)rows);
  if (cin <= 0 || cin % 16) return fail(LH_ERR_INVALID_ARGUMENT, "cin must be a positive multiple of 16 (got %lld)", (long long)cin);
  if (cin / 16 > 4LL * 65535) return fail(LH_ERR_INVALID_ARGUMENT, "cin too large");
  if (n_groups < 1 || n_groups > 2147483647LL) return fail(LH_ERR_INVALID_ARGUMENT, "n_groups must be >= 1 (got %lld)", (long long)n_groups);
  if (!offsets && n_groups != 1) return fail(LH_ERR_INVALID_ARGUMENT, "group_offsets is required when n_groups > 1");
  return LH_OK;
}

// Accumulation scratch of one device, kept between calls: a work area and arrival counters
// (zero between calls: set to zero when allocated, and every call leaves them zero).  The memory is
// handed from call to call in stream order: `ready` is recorded on the stream of the last call
// that used it and the next call's stream waits for it, so two calls never use it at once.  Only
// streams of the same device wait for `ready`, so its release needs device scope: the event is
// created without the system-scope fence (which writes back and invalidates the caches on every
// record, about 1.8 us per call measured on MI355X).
struct DeviceScratch {
  std::mutex mu;
  void* work = nullptr;
  size_t work_bytes = 0;
  unsigned* counters = nullptr;
  size_t n_counters = 0;
  hipEvent_t ready = nullptr;
};

DeviceScratch& device_scratch(int dev) {
  static DeviceScratch table[64];
  return table[dev];
}
// The full-Hessian sweep's own scratch (one float per block column: the Hessian's eigenvalue
// bound), handed on in stream order like the accumulation's.
DeviceScratch& sweep_scratch(int dev) {
  static DeviceScratch table[64];
  return table[dev];
}

// Grows a buffer in stream order (the old one is freed on `s` after the waits already queued).
hipError_t grow(void** buf, size_t* have, size_t need, size_t elem, hipMemPool_t pool, hipStream_t s,
                bool zero) {
  if (need <= *have) return hipSuccess;
  if (*buf) {
    hipError_t e = hipFreeAsync(*buf, s);
    if (e != hipSuccess) return e;
    *buf = nullptr;
    *have = 0;
  }
  hipError_t e = hipMallocFromPoolAsync(buf, need * elem, pool, s);
  if (e != hipSuccess) return e;
  *have = need;
  return zero ? lh::launch_zero_fill(static_cast<unsigned*>(*buf), need * elem / sizeof(unsigned), s) : hipSuccess;
}

lh_status run_accumulate(const void* X, const void* Xq, const float* x_amax, lh_dtype dt, int64_t rows,
                         int64_t cin, const int64_t* offsets, int64_t n_groups, float beta, float* H,
                         float* P, float* imp, void* stream) {
  int dev = -1;
  lh_status st = check_pointers({{X, "X"}, {Xq, "Xq"}, {x_amax, "x_amax"}, {offsets, "group_offsets"}, {H, "H"}, {P, "P"}, {imp, "imp"}}, &dev);
  if (st != LH_OK) return st;
  if ((st = check_aligned(X, "X")) != LH_OK) return st;
  if ((st = check_aligned(Xq, "Xq")) != LH_OK) return st;
  DeviceGuard guard;
  if ((st = guard.enter(dev)) != LH_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t nb = cin / 16;
  const bool act = Xq != nullptr || x_amax != nullptr;
  const lh::AccScratch need = lh::accumulate_scratch(rows, nb, offsets, n_groups, dt == LH_DTYPE_BF16, act,
                                                    !act && H == nullptr);
  hipMemPool_t pool;
  hipError_t e = scratch_pool(dev, &pool);
  if (e != hipSuccess) return hip_fail(e, "scratch pool");

  DeviceScratch& sc = device_scratch(dev);
  std::lock_guard<std::mutex> lk(sc.mu);
  if (!sc.ready) {
    e = hipEventCreateWithFlags(&sc.ready, hipEventDisableTiming | hipEventDisableSystemFence);
    if (e != hipSuccess) { sc.ready = nullptr; return hip_fail(e, "hipEventCreateWithFlags"); }
  } else {
    e = hipStreamWaitEvent(s, sc.ready, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  e = grow(&sc.work, &sc.work_bytes, std::max<size_t>(need.work_bytes, 16), 1, pool, s, false);
  if (e == hipSuccess)
    e = grow(reinterpret_cast<void**>(&sc.counters), &sc.n_counters, std::max<size_t>(need.counters, 1), sizeof(unsigned), pool, s, true);
  if (e != hipSuccess) {
    (void)hipEventRecord(sc.ready, s);
    return hip_fail(e, "accumulation scratch");
  }
  e = lh::launch_accumulate(X, Xq, x_amax, dt == LH_DTYPE_BF16, rows, cin, offsets, n_groups, beta, H, P, imp,
                            sc.work, sc.work_bytes, sc.counters, sc.n_counters, s);
  hipError_t e2 = hipEventRecord(sc.ready, s);
  if (e != hipSuccess) return hip_fail(e, "accumulate launch");
  if (e2 != hipSuccess) return hip_fail(e2, "hipEventRecord");
  return ok();
}

// Scratch of the allocation-free accumulation: one fixed array per device, part of the library's
// code object (so each device that loads the library holds it until the process ends).  Host code
// never uses the name `scratch` as an address: each device's own copy is looked up once, with
// that device current, and kept in noalloc_ptr.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of this device's `scratch` (the caller has made `dev` current).
lh_status noalloc_scratch(int dev, unsigned char** out) {
  static std::mutex mu;
  static unsigned char* ptrs[64] = {};
  std::lock_guard<std::mutex> lk(mu);
  if (dev < 0 || dev >= 64) return fail(LH_ERR_UNSUPPORTED, "device %d out of range", dev);
  if (!ptrs[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    ptrs[dev] = static_cast<unsigned char*>(p);
  }
  *out = ptrs[dev];
  return LH_OK;
}

lh_status check_sweep_shapes(int64_t n_groups, int64_t cout, int64_t cin) {
  if (n_groups < 1 || n_groups > 65535) return fail(LH_ERR_INVALID_ARGUMENT, "n_groups must be in [1, 65535] (got %lld)", (long long)n_groups);
  // the sweep grid takes 32 rows per workgroup along its 16-bit y dimension
  if (cout < 0 || cout > 65535LL * 32) return fail(LH_ERR_INVALID_ARGUMENT, "cout must be in [0, 2097120] (got %lld)", (long long)cout);
  if (cin <= 0 || cin % 16) return fail(LH_ERR_INVALID_ARGUMENT, "cin must be a positive multiple of 16 (got %lld)", (long long)cin);
  return LH_OK;
}

// The launch options of a sweep from the caller's: the divisor 6 * norm (norm must be one of the
// 126 positive finite E4M3 values, so 6 * norm is exact in fp32) and the multipliers, copied.
lh_status sweep_opts(const lh_sweep_options* in, lh::SweepOpts* out) {
  std::memset(out, 0, sizeof(*out));
  out->gdiv = 6.0f * 448.0f;
  if (!in) return LH_OK;
  const float norm = in->scale_norm;
  bool e4m3 = false;
  for (int k = 1; k <= 126 && !e4m3; ++k) {
    const int e = k >> 3, m = k & 7;
    const float v = e == 0 ? std::ldexp((float)m, -9) : std::ldexp(1.0f + (float)m / 8.0f, e - 7);
    e4m3 = (v == norm);
  }
  if (!e4m3) return fail(LH_ERR_INVALID_ARGUMENT, "scale_norm must be a positive finite E4M3 value such as 448 or 256 (got %g)", (double)norm);
  out->gdiv = 6.0f * norm;
  if (in->n_multipliers < 0 || in->n_multipliers > lh::kMaxMultipliers)
    return fail(LH_ERR_INVALID_ARGUMENT, "n_multipliers must be in [0, %d] (got %d)", lh::kMaxMultipliers, (int)in->n_multipliers);
  if (in->n_multipliers > 0 && !in->multipliers) return fail(LH_ERR_INVALID_ARGUMENT, "multipliers is NULL");
  for (int j = 0; j < in->n_multipliers; ++j) {
    const float m = in->multipliers[j];
    if (!(m > 0.0f) || !std::isfinite(m)) return fail(LH_ERR_INVALID_ARGUMENT, "multiplier %d is not a positive finite number", j);
    out->mult[j] = m;
  }
  out->nm = in->n_multipliers;
  return LH_OK;
}

}  // namespace

extern "C" {

lh_status lh_accumulate(const void* X, lh_dtype x_dtype, int64_t rows, int64_t cin,
                        const int64_t* group_offsets, int64_t n_groups, float beta, float* H,
                        float* imp, void* stream) {
  if (!dtype_ok(x_dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)x_dtype);
  lh_status st = check_shapes_x(rows, cin, group_offsets, n_groups);
  if (st != LH_OK) return st;
  if (!H && !imp) return fail(LH_ERR_INVALID_ARGUMENT, "at least one of H, imp must be given");
  if (!X && rows > 0) return fail(LH_ERR_INVALID_ARGUMENT, "X is NULL");
  return run_accumulate(X, nullptr, nullptr, x_dtype, rows, cin, group_offsets, n_groups, beta, H, nullptr, imp, stream);
}

lh_status lh_accumulate_noalloc(const void* X, lh_dtype x_dtype, int64_t rows, int64_t cin,
                                const int64_t* group_offsets, int64_t n_groups, float beta, float* H,
                                float* imp, void* stream) {
  if (!dtype_ok(x_dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)x_dtype);
  lh_status st = check_shapes_x(rows, cin, group_offsets, n_groups);
  if (st != LH_OK) return st;
  if (!H && !imp) return fail(LH_ERR_INVALID_ARGUMENT, "at least one of H, imp must be given");
  if (!X && rows > 0) return fail(LH_ERR_INVALID_ARGUMENT, "X is NULL");
  const lh::AccScratch need = lh::accumulate_scratch(rows, cin / 16, group_offsets, n_groups, x_dtype == LH_DTYPE_BF16,
                                                    false, H == nullptr);
  const size_t work = (std::max<size_t>(need.work_bytes, 16) + 255) / 256 * 256;
  const size_t counters = std::max<size_t>(need.counters, 1);
  if (work + counters * sizeof(unsigned) > kNoAllocScratchBytes)
    return fail(LH_ERR_INVALID_ARGUMENT,
                "this accumulation needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                "(use lh_accumulate, or fewer rows or channels per call)",
                work + counters * sizeof(unsigned), kNoAllocScratchBytes);
  int dev = -1;
  st = check_pointers({{X, "X"}, {group_offsets, "group_offsets"}, {H, "H"}, {imp, "imp"}}, &dev);
  if (st != LH_OK) return st;
  if ((st = check_aligned(X, "X")) != LH_OK) return st;
  DeviceGuard guard;
  if ((st = guard.enter(dev)) != LH_OK) return st;
  unsigned char* base = nullptr;
  if ((st = noalloc_scratch(dev, &base)) != LH_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned* ctr = reinterpret_cast<unsigned*>(base + work);
  // the counters must start at zero: every call leaves them zero, but a previous call on this
  // device may not have completed normally, so they are cleared (by a kernel, not a memset node)
  hipError_t e = lh::launch_zero_fill(ctr, counters, s);
  if (e == hipSuccess)
    e = lh::launch_accumulate(X, nullptr, nullptr, x_dtype == LH_DTYPE_BF16, rows, cin, group_offsets, n_groups, beta,
                              H, nullptr, imp, base, work, ctr, counters, s);
  if (e != hipSuccess) return hip_fail(e, "allocation-free accumulate launch");
  return ok();
}

lh_status lh_accumulate_act_aware(const void* X, const void* Xq, lh_dtype dtype, int64_t rows,
                                  int64_t cin, const int64_t* group_offsets, int64_t n_groups,
                                  float beta, float* H, float* P, void* stream) {
  if (!dtype_ok(dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  lh_status st = check_shapes_x(rows, cin, group_offsets, n_groups);
  if (st != LH_OK) return st;
  if (!H || !P) return fail(LH_ERR_INVALID_ARGUMENT, "H and P are both required");
  if ((!X || !Xq) && rows > 0) return fail(LH_ERR_INVALID_ARGUMENT, "X and Xq are required");
  if (rows == 0) {
    // nothing to read: only the beta term remains; run the generic path with an alias for Xq
    return run_accumulate(X ? X : H, Xq ? Xq : H, nullptr, dtype, 0, cin, group_offsets, n_groups, beta, H, P, nullptr, stream);
  }
  return run_accumulate(X, Xq, nullptr, dtype, rows, cin, group_offsets, n_groups, beta, H, P, nullptr, stream);
}

lh_status lh_accumulate_act_aware_fq(const void* X, lh_dtype dtype, int64_t rows, int64_t cin,
                                     const int64_t* group_offsets, int64_t n_groups,
                                     const float* x_amax, float beta, float* H, float* P,
                                     void* stream) {
  if (!dtype_ok(dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  lh_status st = check_shapes_x(rows, cin, group_offsets, n_groups);
  if (st != LH_OK) return st;
  if (!H || !P) return fail(LH_ERR_INVALID_ARGUMENT, "H and P are both required");
  if (!x_amax) return fail(LH_ERR_INVALID_ARGUMENT, "x_amax is required");
  if (!X && rows > 0) return fail(LH_ERR_INVALID_ARGUMENT, "X is NULL");
  // with no rows nothing is read: only the beta term remains (X may then be NULL)
  return run_accumulate(X ? X : H, nullptr, x_amax, dtype, rows, cin, group_offsets, n_groups, beta, H, P, nullptr, stream);
}

lh_status lh_activation_fake_quant(const void* X, lh_dtype dtype, int64_t rows, int64_t cin,
                                   const int64_t* group_offsets, int64_t n_groups, const float* x_amax,
                                   void* Xq, void* stream) {
  if (!dtype_ok(dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  lh_status st = check_shapes_x(rows, cin, group_offsets, n_groups);
  if (st != LH_OK) return st;
  if (!x_amax) return fail(LH_ERR_INVALID_ARGUMENT, "x_amax is required");
  if ((!X || !Xq) && rows > 0) return fail(LH_ERR_INVALID_ARGUMENT, "X and Xq are required");
  if (rows == 0) return ok();
  if (X == Xq) return fail(LH_ERR_INVALID_ARGUMENT, "Xq must not alias X");
  int dev = -1;
  st = check_pointers({{X, "X"}, {Xq, "Xq"}, {x_amax, "x_amax"}, {group_offsets, "group_offsets"}}, &dev);
  if (st != LH_OK) return st;
  if ((st = check_aligned(X, "X")) != LH_OK) return st;
  if ((st = check_aligned(Xq, "Xq")) != LH_OK) return st;
  DeviceGuard guard;
  if ((st = guard.enter(dev)) != LH_OK) return st;
  hipError_t e = lh::launch_act_fake_quant(X, dtype == LH_DTYPE_BF16, rows, cin, group_offsets, n_groups, x_amax, Xq,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "activation fake-quant launch");
  return ok();
}

lh_status lh_scale_sweep_ex(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                            int64_t cin, const float* global_amax, const float* H, const float* P,
                            const lh_sweep_options* options, uint8_t* scale_code, uint8_t* fp4,
                            float* best_loss, void* stream) {
  if (!dtype_ok(w_dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)w_dtype);
  lh_status st = check_sweep_shapes(n_groups, cout, cin);
  if (st != LH_OK) return st;
  if (!global_amax || !H || !scale_code) return fail(LH_ERR_INVALID_ARGUMENT, "global_amax, H and scale_code are required");
  if (!W && cout > 0) return fail(LH_ERR_INVALID_ARGUMENT, "W is NULL");
  lh::SweepOpts opts;
  if ((st = sweep_opts(options, &opts)) != LH_OK) return st;
  int dev = -1;
  st = check_pointers({{W, "W"}, {global_amax, "global_amax"}, {H, "H"}, {P, "P"}, {scale_code, "scale_code"}, {fp4, "fp4"}, {best_loss, "best_loss"}}, &dev);
  if (st != LH_OK) return st;
  if ((st = check_aligned(W, "W")) != LH_OK) return st;
  if (fp4 && (reinterpret_cast<uintptr_t>(fp4) % 2) != 0) return fail(LH_ERR_INVALID_ARGUMENT, "fp4 must be 2-byte aligned");
  DeviceGuard guard;
  if ((st = guard.enter(dev)) != LH_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (cout == 0) return ok();
  // scratch: one float per block column (the sweep's per-column eigenvalue bound)
  hipMemPool_t pool;
  hipError_t e = scratch_pool(dev, &pool);
  if (e != hipSuccess) return hip_fail(e, "scratch pool");
  DeviceScratch& sc = sweep_scratch(dev);
  std::lock_guard<std::mutex> lk(sc.mu);
  if (!sc.ready) {
    e = hipEventCreateWithFlags(&sc.ready, hipEventDisableTiming | hipEventDisableSystemFence);
    if (e != hipSuccess) { sc.ready = nullptr; return hip_fail(e, "hipEventCreateWithFlags"); }
  } else {
    e = hipStreamWaitEvent(s, sc.ready, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  e = grow(&sc.work, &sc.work_bytes, std::max<size_t>((size_t)n_groups * (size_t)(cin / 16) * sizeof(float), 16), 1, pool,
           s, false);
  if (e != hipSuccess) {
    (void)hipEventRecord(sc.ready, s);
    return hip_fail(e, "sweep scratch");
  }
  e = lh::launch_sweep(W, w_dtype == LH_DTYPE_BF16, n_groups, cout, cin, global_amax, H, P, scale_code, fp4,
                       best_loss, opts, static_cast<float*>(sc.work), s);
  hipError_t e2 = hipEventRecord(sc.ready, s);
  if (e != hipSuccess) return hip_fail(e, "sweep launch");
  if (e2 != hipSuccess) return hip_fail(e2, "hipEventRecord");
  return ok();
}

lh_status lh_scale_sweep(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                         int64_t cin, const float* global_amax, const float* H, const float* P,
                         uint8_t* scale_code, uint8_t* fp4, float* best_loss, void* stream) {
  return lh_scale_sweep_ex(W, w_dtype, n_groups, cout, cin, global_amax, H, P, nullptr, scale_code, fp4,
                           best_loss, stream);
}

lh_status lh_accumulate_sweep(const void* X, const void* W, lh_dtype dtype, int64_t rows, int64_t cin,
                              const int64_t* group_offsets, int64_t n_groups, int64_t cout,
                              const float* global_amax, const lh_sweep_options* options,
                              uint8_t* scale_code, uint8_t* fp4, float* best_loss, void* stream) {
  if (!dtype_ok(dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  lh_status st = check_shapes_x(rows, cin, group_offsets, n_groups);
  if (st != LH_OK) return st;
  if ((st = check_sweep_shapes(n_groups, cout, cin)) != LH_OK) return st;
  if (cout > lh::kFusedMaxCout) return fail(LH_ERR_INVALID_ARGUMENT, "cout must be at most %d for the fused path (got %lld)", lh::kFusedMaxCout, (long long)cout);
  if (!global_amax || !scale_code) return fail(LH_ERR_INVALID_ARGUMENT, "global_amax and scale_code are required");
  if (!X && rows > 0) return fail(LH_ERR_INVALID_ARGUMENT, "X is NULL");
  if (!W && cout > 0) return fail(LH_ERR_INVALID_ARGUMENT, "W is NULL");
  lh::SweepOpts opts;
  if ((st = sweep_opts(options, &opts)) != LH_OK) return st;
  int dev = -1;
  st = check_pointers({{X, "X"}, {W, "W"}, {group_offsets, "group_offsets"}, {global_amax, "global_amax"}, {scale_code, "scale_code"}, {fp4, "fp4"}, {best_loss, "best_loss"}}, &dev);
  if (st != LH_OK) return st;
  if ((st = check_aligned(X, "X")) != LH_OK) return st;
  if ((st = check_aligned(W, "W")) != LH_OK) return st;
  if (fp4 && (reinterpret_cast<uintptr_t>(fp4) % 2) != 0) return fail(LH_ERR_INVALID_ARGUMENT, "fp4 must be 2-byte aligned");
  DeviceGuard guard;
  if ((st = guard.enter(dev)) != LH_OK) return st;
  hipError_t e = lh::launch_accumulate_sweep(X, W, dtype == LH_DTYPE_BF16, rows, cin, n_groups > 1 ? group_offsets : nullptr,
                                             n_groups, cout, global_amax, scale_code, fp4, best_loss, opts,
                                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fused accumulate-and-sweep launch");
  return ok();
}

lh_status lh_scale_sweep_diag_ex(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                                 int64_t cin, const float* global_amax, const float* imp,
                                 const lh_sweep_options* options, uint8_t* scale_code, uint8_t* fp4,
                                 float* best_loss, void* stream) {
  if (!dtype_ok(w_dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)w_dtype);
  lh_status st = check_sweep_shapes(n_groups, cout, cin);
  if (st != LH_OK) return st;
  if (!global_amax || !scale_code) return fail(LH_ERR_INVALID_ARGUMENT, "global_amax and scale_code are required");
  if (!W && cout > 0) return fail(LH_ERR_INVALID_ARGUMENT, "W is NULL");
  lh::SweepOpts opts;
  if ((st = sweep_opts(options, &opts)) != LH_OK) return st;
  int dev = -1;
  st = check_pointers({{W, "W"}, {global_amax, "global_amax"}, {imp, "imp"}, {scale_code, "scale_code"}, {fp4, "fp4"}, {best_loss, "best_loss"}}, &dev);
  if (st != LH_OK) return st;
  if ((st = check_aligned(W, "W")) != LH_OK) return st;
  DeviceGuard guard;
  if ((st = guard.enter(dev)) != LH_OK) return st;
  hipError_t e = lh::launch_sweep_diag(W, w_dtype == LH_DTYPE_BF16, n_groups, cout, cin, global_amax, imp,
                                       scale_code, fp4, best_loss, opts, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, imp ? "diagonal sweep launch" : "plain-MSE sweep launch");
  return ok();
}

lh_status lh_scale_sweep_diag(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                              int64_t cin, const float* global_amax, const float* imp,
                              uint8_t* scale_code, uint8_t* fp4, float* best_loss, void* stream) {
  if (!imp) return fail(LH_ERR_INVALID_ARGUMENT, "global_amax, imp and scale_code are required");
  return lh_scale_sweep_diag_ex(W, w_dtype, n_groups, cout, cin, global_amax, imp, nullptr, scale_code, fp4,
                                best_loss, stream);
}

lh_status lh_scale_sweep_mse(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t cout,
                             int64_t cin, const float* global_amax, uint8_t* scale_code, uint8_t* fp4,
                             float* best_loss, void* stream) {
  return lh_scale_sweep_diag_ex(W, w_dtype, n_groups, cout, cin, global_amax, nullptr, nullptr, scale_code, fp4,
                                best_loss, stream);
}

lh_status lh_dequantize_ex(const uint8_t* scale_code, const uint8_t* fp4, lh_dtype out_dtype,
                           int64_t n_groups, int64_t cout, int64_t cin, const float* global_amax,
                           float scale_norm, void* Wq, float* block_amax, void* stream) {
  if (!dtype_ok(out_dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)out_dtype);
  lh_status st = check_sweep_shapes(n_groups, cout, cin);
  if (st != LH_OK) return st;
  if (!scale_code || !global_amax) return fail(LH_ERR_INVALID_ARGUMENT, "scale_code and global_amax are required");
  if (!Wq && !block_amax) return fail(LH_ERR_INVALID_ARGUMENT, "at least one of Wq, block_amax must be given");
  if (Wq && !fp4) return fail(LH_ERR_INVALID_ARGUMENT, "fp4 is required for Wq");
  lh_sweep_options o{scale_norm, 0, nullptr};
  lh::SweepOpts opts;
  if ((st = sweep_opts(&o, &opts)) != LH_OK) return st;
  int dev = -1;
  st = check_pointers({{scale_code, "scale_code"}, {fp4, "fp4"}, {global_amax, "global_amax"}, {Wq, "Wq"}, {block_amax, "block_amax"}}, &dev);
  if (st != LH_OK) return st;
  if ((st = check_aligned(Wq, "Wq")) != LH_OK) return st;
  if (fp4 && (reinterpret_cast<uintptr_t>(fp4) % 8) != 0) return fail(LH_ERR_INVALID_ARGUMENT, "fp4 must be 8-byte aligned");
  DeviceGuard guard;
  if ((st = guard.enter(dev)) != LH_OK) return st;
  hipError_t e = lh::launch_dequantize(scale_code, fp4, global_amax, n_groups, cout, cin, out_dtype == LH_DTYPE_BF16,
                                       Wq, block_amax, opts.gdiv, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return ok();
}

lh_status lh_dequantize(const uint8_t* scale_code, const uint8_t* fp4, lh_dtype out_dtype,
                        int64_t n_groups, int64_t cout, int64_t cin, const float* global_amax,
                        void* Wq, float* block_amax, void* stream) {
  return lh_dequantize_ex(scale_code, fp4, out_dtype, n_groups, cout, cin, global_amax, 448.0f, Wq, block_amax,
                          stream);
}

lh_status lh_absmax(const void* W, lh_dtype w_dtype, int64_t n_groups, int64_t elems_per_group,
                    float* amax_out, void* stream) {
  if (!dtype_ok(w_dtype)) return fail(LH_ERR_UNSUPPORTED, "unknown dtype %d", (int)w_dtype);
  if (n_groups < 1 || n_groups > 65535) return fail(LH_ERR_INVALID_ARGUMENT, "n_groups must be in [1, 65535] (got %lld)", (long long)n_groups);
  if (elems_per_group < 0) return fail(LH_ERR_INVALID_ARGUMENT, "elems_per_group must be >= 0");
  if (!amax_out) return fail(LH_ERR_INVALID_ARGUMENT, "amax_out is required");
  if (!W && elems_per_group > 0) return fail(LH_ERR_INVALID_ARGUMENT, "W is NULL");
  int dev = -1;
  lh_status st = check_pointers({{W, "W"}, {amax_out, "amax_out"}}, &dev);
  if (st != LH_OK) return st;
  DeviceGuard guard;
  if ((st = guard.enter(dev)) != LH_OK) return st;
  hipError_t e = lh::launch_absmax(W, w_dtype == LH_DTYPE_BF16, n_groups, elems_per_group, amax_out,
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "absmax launch");
  return ok();
}

const char* lh_last_error(void) { return g_last_error.c_str(); }

int lh_version(void) { return LH_VERSION; }

}  // extern "C"
