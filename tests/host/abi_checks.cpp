// Host-side checks of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host code (tests/test_host_sanitize.py): every argument check that needs no GPU, on bad sizes,
// null pointers, unknown dtypes, bad options and host memory passed as device memory.  Each call
// must return the documented code with a message and touch no memory it was not given; the
// sanitizers abort the process on any out-of-bounds access, leak of a freed buffer or undefined
// behaviour in the library's host code.
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/lh.h"

static int failures = 0;

static void expect(lh_status got, lh_status want, const char* what, const char* needle = nullptr) {
  const char* msg = lh_last_error();
  const bool ok = got == want && (!needle || std::strstr(msg, needle) != nullptr) && (want == LH_OK || msg[0] != 0);
  if (!ok) {
    std::fprintf(stderr, "FAIL %s: got %d (%s), want %d%s%s\n", what, (int)got, msg, (int)want,
                 needle ? " with " : "", needle ? needle : "");
    ++failures;
  }
}

int main() {
  std::vector<unsigned char> host(1 << 16, 0);            // host memory: never a valid device pointer
  void* h = host.data();
  float* hf = reinterpret_cast<float*>(host.data());
  uint8_t* hb = host.data();
  const int64_t* ho = reinterpret_cast<const int64_t*>(host.data());
  const lh_dtype BF = LH_DTYPE_BF16;
  const lh_dtype BAD = static_cast<lh_dtype>(7);

  // accumulation
  expect(lh_accumulate(h, BAD, 8, 32, nullptr, 1, 0.f, hf, nullptr, nullptr), LH_ERR_UNSUPPORTED, "dtype", "dtype");
  expect(lh_absmax(h, static_cast<lh_dtype>(-3), 1, 16, hf, nullptr), LH_ERR_UNSUPPORTED, "negative dtype", "dtype");
  expect(lh_accumulate(h, BF, 8, 40, nullptr, 1, 0.f, hf, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "cin % 16", "cin");
  expect(lh_accumulate(h, BF, -1, 32, nullptr, 1, 0.f, hf, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "rows < 0", "rows");
  expect(lh_accumulate(h, BF, 8, 32, nullptr, 0, 0.f, hf, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "n_groups 0", "n_groups");
  expect(lh_accumulate(h, BF, 8, 32, nullptr, 3, 0.f, hf, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "offsets", "group_offsets");
  expect(lh_accumulate(h, BF, 8, 32, nullptr, 1, 0.f, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "no outputs", "at least one");
  expect(lh_accumulate(nullptr, BF, 8, 32, nullptr, 1, 0.f, hf, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "null X", "X");
  expect(lh_accumulate(h, BF, 8, 32, nullptr, 1, 0.f, hf, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "host X", "device");
  expect(lh_accumulate_noalloc(h, BF, 8, 32, nullptr, 1, 0.f, hf, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "noalloc host X", "device");
  expect(lh_accumulate_noalloc(h, BF, int64_t(1) << 27, 4096, ho, 2, 0.f, hf, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT,
         "noalloc oversized", "scratch");
  expect(lh_accumulate_act_aware(h, h, BF, 8, 32, nullptr, 1, 0.f, hf, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "act P", "required");
  expect(lh_accumulate_act_aware_fq(h, BF, 8, 32, nullptr, 1, nullptr, 0.f, hf, hf, nullptr), LH_ERR_INVALID_ARGUMENT, "fq amax", "x_amax");
  expect(lh_activation_fake_quant(h, BF, 8, 32, nullptr, 1, hf, h, nullptr), LH_ERR_INVALID_ARGUMENT, "xq alias", "alias");
  expect(lh_activation_fake_quant(h, BF, 8, 32, nullptr, 1, hf, hb + 4096, nullptr), LH_ERR_INVALID_ARGUMENT, "xq host", "device");

  // sweeps and options
  expect(lh_scale_sweep(h, BF, 0, 16, 32, hf, hf, nullptr, hb, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "sweep groups", "n_groups");
  expect(lh_scale_sweep(h, BF, 1, -5, 32, hf, hf, nullptr, hb, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "sweep cout", "cout");
  expect(lh_scale_sweep(h, BF, 1, 16, 32, nullptr, hf, nullptr, hb, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "sweep amax", "required");
  expect(lh_scale_sweep(h, BF, 1, 16, 32, hf, hf, nullptr, hb, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "sweep host", "device");
  const float mults[3] = {0.5f, 1.0f, 1.5f};
  lh_sweep_options o{256.f, 3, mults};
  expect(lh_scale_sweep_ex(h, BF, 1, 16, 32, hf, hf, nullptr, &o, hb, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "sweep_ex host", "device");
  o.scale_norm = 300.f;
  expect(lh_scale_sweep_ex(h, BF, 1, 16, 32, hf, hf, nullptr, &o, hb, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "norm", "scale_norm");
  o.scale_norm = 448.f;
  o.n_multipliers = 129;
  expect(lh_scale_sweep_diag_ex(h, BF, 1, 16, 32, hf, hf, &o, hb, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "n_mult", "n_multipliers");
  const float badm[2] = {1.0f, -1.0f};
  lh_sweep_options ob{448.f, 2, badm};
  expect(lh_scale_sweep_diag_ex(h, BF, 1, 16, 32, hf, nullptr, &ob, hb, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "mult sign", "multiplier");
  expect(lh_scale_sweep_mse(h, BAD, 1, 16, 32, hf, hb, nullptr, nullptr, nullptr), LH_ERR_UNSUPPORTED, "mse dtype", "dtype");
  expect(lh_accumulate_sweep(h, h, BF, 8, 32, ho, 2, 9000, hf, nullptr, hb, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT,
         "fused cout", "8192");
  expect(lh_dequantize(hb, hb, BF, 1, 16, 32, hf, nullptr, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "dequant outputs", "at least one");
  expect(lh_dequantize_ex(hb, hb, BF, 1, 16, 32, hf, 100.f, h, nullptr, nullptr), LH_ERR_INVALID_ARGUMENT, "dequant norm", "scale_norm");
  expect(lh_absmax(h, BF, 0, 16, hf, nullptr), LH_ERR_INVALID_ARGUMENT, "absmax groups", "n_groups");
  expect(lh_absmax(h, BF, 1, 16, hf, nullptr), LH_ERR_INVALID_ARGUMENT, "absmax host", "device");
  if (lh_version() < 1) { std::fprintf(stderr, "FAIL version\n"); ++failures; }
  std::printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
