// Host-side driver of the libhm C ABI for the sanitizer build: every entry point
// with arguments that its validation rejects (nothing reaches a launch, so no
// device is needed), the size queries, the status strings and the host-side
// index function.  Built together with the library's sources, host code under
// AddressSanitizer and UndefinedBehaviorSanitizer; any report fails the run.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hm.h"

static int g_fail = 0;
#define EXPECT(cond)                                                         \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
                   __LINE__, #cond);                                         \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

// Distinct non-NULL, 16-byte aligned fake device addresses: validation never
// dereferences them and every call below is rejected before any launch.
static void* fake(int i) { return reinterpret_cast<void*>(static_cast<uintptr_t>(i) << 20); }

int main() {
  EXPECT(hm_abi_version() == HM_ABI_VERSION);
  for (int s = 0; s < 6; ++s) EXPECT(std::strlen(hm_status_string((hm_status)s)) > 0);
  EXPECT(std::strlen(hm_last_error()) == 0);

  // size queries, including degenerate shapes
  EXPECT(hm_swa_meta_attn_workspace(1, 2176, 5, 64, HM_BF16) > 0);
  EXPECT(hm_swa_meta_attn_workspace(0, 2176, 5, 64, HM_BF16) == 0);
  EXPECT(hm_attn_kv_bytes(2, 16512, 5, 64, HM_BF16) > 0);
  EXPECT(hm_selective_scan_workspace(1, 2176, 1600, 16) > 0);
  EXPECT(hm_selective_scan_workspace(1, 2176, 1600, 8) == 0);
  EXPECT(hm_selective_scan_workspace(-1, 2176, 1600, 16) == 0);
  hm_step_args sa;
  std::memset(&sa, 0, sizeof sa);
  sa.B = 64; sa.Hq = 25; sa.Hkv = 5; sa.Dh = 64; sa.Di = 1600; sa.N = 16; sa.K = 4;
  sa.n_meta = 128; sa.window = 1024; sa.cache_slots = 1024; sa.n_prev = 2048;
  sa.rope_base = 1e4f; sa.eps = 1e-6f; sa.dtype = HM_BF16;
  EXPECT(hm_mixer_step_workspace(&sa) > 0);
  EXPECT(hm_mixer_step_workspace(nullptr) == 0);
  sa.B = 1; sa.window = 0; sa.cache_slots = 16512; sa.n_prev = 16384;
  EXPECT(hm_mixer_step_workspace(&sa) <= hm_mixer_step_noalloc_max_bytes());
  hm_prefill_args pa;
  std::memset(&pa, 0, sizeof pa);
  pa.B = 1; pa.T = 2176; pa.Hq = 25; pa.Hkv = 5; pa.Dh = 64; pa.Di = 1600; pa.N = 16; pa.K = 4;
  pa.n_meta = 128; pa.window = 1024; pa.dtype = HM_BF16;
  EXPECT(hm_mixer_prefill_workspace(&pa) > 0);
  EXPECT(hm_mixer_prefill_workspace(nullptr) == 0);

  // the ring slot, as the decode kernels compute it
  EXPECT(hm_debug_cache_slot(2048, 128, 1024) == 128);
  EXPECT(hm_debug_cache_slot(1023, 128, 1024) == 1151);
  EXPECT(hm_debug_cache_slot(5, 3, 0) == 8);
  EXPECT(hm_debug_cache_slot(-1, 1, 1) == -1);
  int bm = 0, bmw = 0, bn = 0;
  hm_debug_attn_tiles(&bm, &bmw, &bn);
  EXPECT(bm > 0 && bmw > 0 && bn > 0);

  // every compute entry point rejects invalid arguments before launching
  void *q = fake(1), *k = fake(2), *v = fake(3), *o = fake(4), *ws = fake(5);
  const float* f = static_cast<const float*>(fake(6));
  EXPECT(hm_swa_meta_attn(q, k, v, o, 0, 64, 2, 1, 16, 0, 16, 1e4f, 0, 0.f, HM_F32, ws, 1 << 30,
                          nullptr) == HM_ERR_INVALID);
  EXPECT(hm_swa_meta_attn(q, k, v, o, 1, 64, 3, 2, 16, 0, 16, 1e4f, 0, 0.f, HM_F32, ws, 1 << 30,
                          nullptr) == HM_ERR_INVALID);   // Hq % Hkv != 0
  EXPECT(hm_swa_meta_attn(q, k, v, o, 1, 64, 2, 1, 48, 0, 16, 1e4f, 0, 0.f, HM_F32, ws, 1 << 30,
                          nullptr) == HM_ERR_UNSUPPORTED);
  EXPECT(hm_swa_meta_attn(q, k, v, o, 1, 64, 2, 1, 16, 0, 16, 1e4f, 0, 0.f, HM_F32, ws, 16,
                          nullptr) == HM_ERR_WORKSPACE);
  EXPECT(std::strlen(hm_last_error()) > 0);
  EXPECT(hm_attn_kv_prepare(k, v, ws, 16, 1, 64, 1, 16, 1e4f, 0, HM_F32, nullptr) ==
         HM_ERR_WORKSPACE);
  EXPECT(hm_attn_with_kv(q, ws, 1 << 30, o, 1, 64, 3, 2, 16, 0, 16, 1e4f, 0, 0.f, HM_F32,
                         nullptr) == HM_ERR_INVALID);
  EXPECT(hm_causal_conv1d(q, f, nullptr, nullptr, o, nullptr, 1, 64, 32, 3, 1, HM_F32,
                          nullptr) == HM_ERR_UNSUPPORTED);
  EXPECT(hm_causal_conv1d(q, f, nullptr, nullptr, q, nullptr, 1, 64, 32, 4, 1, HM_F32,
                          nullptr) == HM_ERR_INVALID);   // y aliases x
  EXPECT(hm_selective_scan(q, k, f, v, v, nullptr, nullptr, nullptr, o, nullptr, 1, 64, 32, 8,
                           HM_F32, ws, 1 << 30, nullptr) == HM_ERR_UNSUPPORTED);
  EXPECT(hm_conv_selective_scan(q, f, f, nullptr, nullptr, k, f, v, v, nullptr, nullptr, nullptr,
                                o, nullptr, 1, 0, 32, 4, 16, HM_F32, ws, 1 << 30,
                                nullptr) == HM_ERR_INVALID);
  EXPECT(hm_branch_norm_mean(q, k, f, f, 1e-6f, o, 0, 8, HM_F32, nullptr) == HM_ERR_INVALID);
  void* outs[2] = {o, fake(7)};
  int cols[2] = {64, 24};   // not a multiple of 16
  EXPECT(hm_linear_bf16(q, k, 128, 88, 64, 2, outs, cols, nullptr) == HM_ERR_INVALID);
  hm_linear_epilogue ep[2];
  std::memset(ep, 0, sizeof ep);
  ep[0].act = 7;
  cols[1] = 32;
  EXPECT(hm_linear_bf16_ex(q, k, 128, 96, 64, 2, outs, cols, ep, nullptr) == HM_ERR_INVALID);
  EXPECT(hm_rms_norm(q, f, 1e-6f, q, 4, 64, HM_F32, nullptr) == HM_ERR_INVALID);
  EXPECT(hm_mixer_prefill(nullptr, nullptr) == HM_ERR_INVALID);
  pa.q = q;   // most pointers NULL: rejected
  EXPECT(hm_mixer_prefill(&pa, nullptr) == HM_ERR_INVALID);
  hm_block_args ba;
  std::memset(&ba, 0, sizeof ba);
  EXPECT(hm_block_prefill(&ba, nullptr) != HM_OK);
  EXPECT(hm_block_prefill(nullptr, nullptr) == HM_ERR_INVALID);
  EXPECT(hm_mixer_step(nullptr, nullptr) == HM_ERR_INVALID);
  sa.B = 0;
  EXPECT(hm_mixer_step(&sa, nullptr) == HM_ERR_INVALID);
  EXPECT(hm_mixer_step_noalloc(nullptr, nullptr) == HM_ERR_INVALID);
  EXPECT(hm_mixer_step_noalloc(&sa, nullptr) == HM_ERR_INVALID);
  // a step whose scratch exceeds the allocation-free limit, every argument
  // otherwise valid: rejected with HM_ERR_UNSUPPORTED (the test runs with no
  // device visible, so nothing could launch even if the check were missing)
  sa.B = 4096; sa.window = 1024; sa.cache_slots = 1024; sa.n_prev = 2048;
  {
    const void** cps[] = {&sa.q, &sa.x, &sa.delta, &sa.Bm, &sa.Cm, &sa.z};
    int i = 10;
    for (const void** p : cps) *p = fake(i++);
    sa.k_cache = fake(i++); sa.v_cache = fake(i++); sa.out = fake(i++);
    const float** fps[] = {&sa.A, &sa.D, &sa.conv_w, &sa.conv_b, &sa.beta_a, &sa.beta_s};
    for (const float** p : fps) *p = static_cast<const float*>(fake(i++));
    sa.conv_state = static_cast<float*>(fake(i++));
    sa.ssm_state = static_cast<float*>(fake(i++));
  }
  EXPECT(hm_mixer_step_workspace(&sa) > hm_mixer_step_noalloc_max_bytes());
  EXPECT(hm_mixer_step_noalloc(&sa, nullptr) == HM_ERR_UNSUPPORTED);
  EXPECT(std::strstr(hm_last_error(), "8388608") != nullptr);
  sa.n_prev = -1;
  EXPECT(hm_mixer_step_noalloc(&sa, nullptr) == HM_ERR_INVALID);
  EXPECT(hm_debug_attn_mask(0, 0, 0, static_cast<unsigned char*>(o), nullptr) ==
         HM_ERR_INVALID);
  EXPECT(hm_debug_tile_plan(100, 4, 16, 64, 64, static_cast<int*>(o), 2, nullptr) ==
         HM_ERR_INVALID);   // cap too small
  EXPECT(hm_debug_step_positions(0, 5, nullptr, 4, 16, static_cast<long long*>(o), nullptr) ==
         HM_ERR_INVALID);
  if (g_fail == 0) std::printf("host ABI driver: all checks passed\n");
  return g_fail == 0 ? 0 : 1;
}
