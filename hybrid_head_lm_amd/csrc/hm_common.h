// Shared device and host helpers of libhm (gfx950 / CDNA4).
//
// Visibility over X~ = [meta tokens; tokens] follows the Hymba blog (juejin.cn,
// "NVIDIA提出Hymba网络"): meta tokens stay visible to every later token even in
// sliding-window layers ("Hymba简介"); sliding-window and global layers are
// described in "Hymba 的整体架构".  Index convention: rows/columns index X~,
// causal j <= i, the window keeps the W most recent rows (i - j < W) and W <= 0
// means global.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/hm.h"

#define HM_DEV __device__ __forceinline__
#define HM_HD __host__ __device__ __forceinline__

typedef uint16_t bf16_t;   // raw bfloat16 bits in memory

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));

// ----------------------------------------------------------------- numbers
HM_DEV float bf2f(bf16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// Round to nearest even (gfx950 converts in hardware).
HM_DEV bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

HM_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

template <typename T> struct ActIO;
template <> struct ActIO<float> {
  static HM_DEV float ld(const float* p) { return *p; }
  static HM_DEV void st(float* p, float v) { *p = v; }
};
template <> struct ActIO<bf16_t> {
  static HM_DEV float ld(const bf16_t* p) { return bf2f(*p); }
  static HM_DEV void st(bf16_t* p, float v) { *p = f2bf(v); }
};

constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector memory
// operations are outstanding and leaves the other counters unconstrained.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

HM_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// SiLU(x) = x * sigmoid(x) with hardware exp2 and reciprocal (about 1 ulp each).
HM_DEV float siluf_(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// RoPE angle for position `pos` and frequency index d of head dim Dh, reduced
// to [-pi, pi] in double precision, then sin/cos in float.
HM_DEV void rope_sincos(long long pos, int d, int Dh, double log2_base, float* s, float* c) {
  const double two_pi = 6.283185307179586476925286766559;
  double theta = exp2(-2.0 * (double)d / (double)Dh * log2_base);
  double a = (double)pos * theta;
  a -= two_pi * rint(a / two_pi);
  sincosf((float)a, s, c);
}

// ----------------------------------------------------------------- visibility
HM_HD bool hm_visible(int i, int j, int M, int W) {
  if (j > i) return false;
  if (j < M || W <= 0) return true;
  return i - j < W;
}

// Classify the block rows [i0,i1) x keys [j0,j1):
// 0 = no visible pair, 1 = some visible, 2 = all visible.
HM_HD int hm_tile_class(int i0, int i1, int j0, int j1, int M, int W) {
  if (i1 <= i0 || j1 <= j0) return 0;
  if (j0 > i1 - 1) return 0;
  if (!(j0 < M || W <= 0)) {
    int jm = (j1 < i1 ? j1 : i1) - 1;    // largest key not above the diagonal
    int ii = i0 > jm ? i0 : jm;           // earliest row that can see it
    if (ii - jm >= W) return 0;
  }
  bool full = (j1 - 1 <= i0);
  if (full && W > 0 && j1 > M) {
    int jn = j0 > M ? j0 : M;             // first non-meta key
    full = (i1 - 1 - jn) < W;
  }
  return full ? 2 : 1;
}

// Candidate key tiles (units of bn) for query rows [i0,i1): the meta tiles
// [0, e0) and the causal window tiles [b1, e1) (b1 >= e0 after the union).
struct KvRanges { int e0, b1, e1; };
HM_HD KvRanges hm_kv_ranges(int i0, int i1, int M, int W, int bn) {
  KvRanges r;
  int mk = M < i1 ? M : i1;
  r.e0 = (mk + bn - 1) / bn;
  int js;
  if (W <= 0) js = 0;
  else { js = i0 - W + 1; if (js < M) js = M; }
  if (js >= i1) { r.b1 = r.e1 = r.e0; return r; }
  r.b1 = js / bn;
  r.e1 = (i1 + bn - 1) / bn;
  if (r.b1 < r.e0) r.b1 = r.e0;
  if (r.e1 < r.b1) r.e1 = r.b1;
  return r;
}

// ----------------------------------------------------------------- decode positions
// The decode token of sequence b follows n_prev earlier tokens: it sits at
// position n_meta + n_prev, its cache slot is n_meta + (n_prev mod window)
// (window <= 0: n_meta + n_prev) and the cache rows 0 .. L-1 with
// L = n_meta + min(n_prev + 1, window) are visible (all n_meta + n_prev + 1 for
// window <= 0).  Either every sequence is at n_prev_max, or nps holds one
// n_prev per sequence, clamped to [0, n_prev_max].  Used by the decode kernels
// and, on the host, by the slot export.
struct SeqPos {
  const int* nps;
  int n_meta, window;
  long long n_prev_max;
};

HM_HD void seq_pos(const SeqPos& sp, int b, int* L, int* slot, long long* pos) {
  long long np = sp.n_prev_max;
  if (sp.nps) {
    np = (long long)sp.nps[b];
    np = np < 0 ? 0 : (np > sp.n_prev_max ? sp.n_prev_max : np);
  }
  const long long nv = sp.window > 0 ? (np + 1 < sp.window ? np + 1 : (long long)sp.window)
                                     : np + 1;
  *L = (int)(sp.n_meta + nv);
  *slot = (int)(sp.n_meta + (sp.window > 0 ? np % sp.window : np));
  *pos = sp.n_meta + np;
}

// ----------------------------------------------------------------- host side
namespace hm {

void set_error(const std::string& msg);
hm_status fail(hm_status s, const std::string& msg);
hm_status check_launch(const char* what);
hm_status fork_join(hipStream_t main, hipStream_t side, bool fork);

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline size_t act_bytes(hm_dtype dt) { return dt == HM_BF16 ? 2 : 4; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Internal forms of the public entry points: validate every argument, then
// launch unless `dry` (a dry run lets a composite call validate all of its
// parts before the first launch).
hm_status swa_meta_attn_impl(const void* q, const void* k, const void* v, void* o, int B,
                             int T, int Hq, int Hkv, int Dh, int n_meta, int window,
                             float rope_base, long long pos0, float scale, hm_dtype dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t st,
                             bool dry);
hm_status attn_kv_prepare_impl(const void* k, const void* v, void* kv, size_t kv_bytes, int B,
                               int T, int Hkv, int Dh, float rope_base, long long pos0,
                               hm_dtype dtype, hipStream_t st, bool dry);
hm_status attn_with_kv_impl(const void* q, const void* kv, size_t kv_bytes, void* o, int B,
                            int T, int Hq, int Hkv, int Dh, int n_meta, int window,
                            float rope_base, long long pos0, float scale, hm_dtype dtype,
                            hipStream_t st, bool dry);
hm_status conv_scan_impl(const void* x, const float* conv_w, const float* conv_b,
                         const float* conv_state_in, float* conv_state_out,
                         const void* delta, const float* A, const void* Bm, const void* Cm,
                         const float* D, const void* z, const float* h0, void* y,
                         float* h_out, int B, int T, int Di, int K, int N, hm_dtype dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t st,
                         bool fuse_conv, bool dry);
// Fused launch sequence of a bf16 prefill layer (fused.hip); the caller has
// validated every argument.
bool prefill_fusable(const hm_prefill_args* a);
hm_status prefill_fused_bf16(const hm_prefill_args* a, void* kv, void* scan_ws, hipStream_t st);
// The bf16 conv + selective scan in two launches (fused.hip): the aggregate
// pass, then the final pass whose workgroups compose their own incoming
// states; rows and bases 16-byte aligned (Di % 8 == 0), arguments validated.
// conv_scan_two_launch_pays: whether the scan is long enough for that form.
bool conv_scan_two_launch_pays(int B, int T, int Di);
hm_status conv_scan_two_launch_bf16(const void* x, const float* cw, const float* cb,
                                    const float* cst_in, float* cst_out, const void* delta,
                                    const float* A, const void* Bm, const void* Cm,
                                    const float* D, const void* z, const float* h0, void* y,
                                    float* h_out, int B, int T, int Di, void* workspace,
                                    hipStream_t st);
hm_status norm_mean_impl(const void* ya, const void* ys, const float* beta_a,
                         const float* beta_s, float eps, void* out, long long rows,
                         int width, hm_dtype dtype, hipStream_t st, bool dry);
hm_status rms_norm_impl(const void* x, const float* w, float eps, void* out, long long rows,
                        int width, hm_dtype dtype, hipStream_t st, bool dry);
hm_status linear_launch(const void* x, const void* w, int M, int N, int K, int n_seg,
                        void* const* outs, const int* seg_cols, const hm_linear_epilogue* ep,
                        hipStream_t st, bool dry = false);
hm_status mixer_prefill_impl(const hm_prefill_args* a, hipStream_t st, bool dry_only);

}  // namespace hm

#define HM_REQUIRE(cond, status, msg)              \
  do {                                             \
    if (!(cond)) return ::hm::fail((status), (msg)); \
  } while (0)

#define HM_PTR(p) HM_REQUIRE((p) != nullptr && ::hm::aligned16(p), HM_ERR_INVALID, \
                             std::string(#p " must be a non-NULL 16-byte aligned pointer"))
#define HM_OPT_PTR(p) HM_REQUIRE((p) == nullptr || ::hm::aligned16(p), HM_ERR_INVALID, \
                                 std::string(#p " must be 16-byte aligned"))
