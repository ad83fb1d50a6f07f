// Branch normalisation and average of the hybrid-head mixer (Hymba blog,
// juejin.cn "NVIDIA提出Hymba网络": "深入理解混合头模块" — both branches are
// normalised to one scale and averaged; "数学表示" §5 — learnable rescale
// vectors beta_1, beta_2):
//   out = 0.5 * (beta_a * ya / rms(ya) + beta_s * ys / rms(ys)),
//   rms(y) = sqrt(mean(y^2) + eps) over the whole branch width of a token.
// One wave per row: both sums of squares in float32 (16-byte loads), a wave
// reduction, then the output row.  HBM traffic: read ya and ys once, write out.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "hm_common.h"

namespace {

HM_DEV float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <typename Tact>
struct Vec8;
template <>
struct Vec8<bf16_t> {  // 8 bf16 = 16 bytes
  static HM_DEV void ld(const bf16_t* p, float* f) {
    uint4 r = *(const uint4*)p;
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static HM_DEV void st(bf16_t* p, const float* f) {
    uint4 r;
    r.x = pack_bf16x2(f[0], f[1]);
    r.y = pack_bf16x2(f[2], f[3]);
    r.z = pack_bf16x2(f[4], f[5]);
    r.w = pack_bf16x2(f[6], f[7]);
    *(uint4*)p = r;
  }
};
template <>
struct Vec8<float> {  // 8 floats = two 16-byte accesses
  static HM_DEV void ld(const float* p, float* f) {
    float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  static HM_DEV void st(float* p, const float* f) {
    *(float4*)p = make_float4(f[0], f[1], f[2], f[3]);
    *(float4*)(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
};

// Rows of up to 64 * 8 * kMaxC elements are held in registers (norm_mean_rows,
// norm_mean_rows_bf16, rms_norm_rows).
constexpr int kMaxC = 4;

// width % 8 == 0 (16-byte aligned rows), wider than 64 * 8 * kMaxC: one wave
// per row; the row is read twice (the second read is served by L2).

template <typename Tact>
__global__ __launch_bounds__(256) void norm_mean_vec(const Tact* __restrict__ ya,
                                                     const Tact* __restrict__ ys,
                                                     const float* __restrict__ ba,
                                                     const float* __restrict__ bs, float eps,
                                                     Tact* __restrict__ out, long long rows,
                                                     int width) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const Tact* pa = ya + row * width;
  const Tact* ps = ys + row * width;
  Tact* po = out + row * width;
  const int n8 = width >> 3;
  float sa = 0.f, ss = 0.f;
  for (int c = lane; c < n8; c += 64) {
    float a[8], s[8];
    Vec8<Tact>::ld(pa + 8 * c, a);
    Vec8<Tact>::ld(ps + 8 * c, s);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sa += a[i] * a[i];
      ss += s[i] * s[i];
    }
  }
  sa = wave_sum(sa);
  ss = wave_sum(ss);
  const float ra = 0.5f / sqrtf(sa / (float)width + eps);
  const float rs = 0.5f / sqrtf(ss / (float)width + eps);
  for (int c = lane; c < n8; c += 64) {
    float a[8], s[8], r[8];
    Vec8<Tact>::ld(pa + 8 * c, a);
    Vec8<Tact>::ld(ps + 8 * c, s);
    const float4 ba0 = *(const float4*)(ba + 8 * c), ba1 = *(const float4*)(ba + 8 * c + 4);
    const float4 bs0 = *(const float4*)(bs + 8 * c), bs1 = *(const float4*)(bs + 8 * c + 4);
    const float wa[8] = {ba0.x, ba0.y, ba0.z, ba0.w, ba1.x, ba1.y, ba1.z, ba1.w};
    const float wsv[8] = {bs0.x, bs0.y, bs0.z, bs0.w, bs1.x, bs1.y, bs1.z, bs1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = wa[i] * a[i] * ra + wsv[i] * s[i] * rs;
    Vec8<Tact>::st(po + 8 * c, r);
  }
}

// width % 8 == 0 and width <= 64 * 8 * kMaxC: four rows per workgroup (one per
// wave; measured a little faster than eight at 33 024 rows), each row held in
// registers; the two beta vectors are staged in LDS once per workgroup instead
// of being read by every wave.
constexpr int kRowsPerBlock = 4;

template <typename Tact>
__global__ __launch_bounds__(64 * kRowsPerBlock) void norm_mean_rows(
    const Tact* __restrict__ ya, const Tact* __restrict__ ys, const float* __restrict__ ba,
    const float* __restrict__ bs, float eps, Tact* __restrict__ out, long long rows, int width) {
  __shared__ float4 sb[2][64 * kMaxC * 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + wave;
  const bool live = row < rows;
  const int n8 = width >> 3;
  const Tact* pa = ya + row * width;
  const Tact* ps = ys + row * width;
  float a[kMaxC][8], s[kMaxC][8];
  if (live) {
#pragma unroll
    for (int k = 0; k < kMaxC; ++k) {
      const int c = lane + 64 * k;
      if (c < n8) {
        Vec8<Tact>::ld(pa + 8 * c, a[k]);
        Vec8<Tact>::ld(ps + 8 * c, s[k]);
      }
    }
  }
  for (int i = threadIdx.x; i < 2 * n8; i += 64 * kRowsPerBlock) {
    sb[0][i] = ((const float4*)ba)[i];
    sb[1][i] = ((const float4*)bs)[i];
  }
  __syncthreads();
  if (!live) return;
  float sa = 0.f, ss = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxC; ++k)
    if (lane + 64 * k < n8)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sa += a[k][i] * a[k][i];
        ss += s[k][i] * s[k][i];
      }
  sa = wave_sum(sa);
  ss = wave_sum(ss);
  const float ra = 0.5f / sqrtf(sa / (float)width + eps);
  const float rs = 0.5f / sqrtf(ss / (float)width + eps);
  Tact* po = out + row * width;
#pragma unroll
  for (int k = 0; k < kMaxC; ++k) {
    const int c = lane + 64 * k;
    if (c < n8) {
      const float4 a0 = sb[0][2 * c], a1 = sb[0][2 * c + 1];
      const float4 s0 = sb[1][2 * c], s1 = sb[1][2 * c + 1];
      const float w1[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float w2[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = w1[i] * a[k][i] * ra + w2[i] * s[k][i] * rs;
      Vec8<Tact>::st(po + 8 * c, r);
    }
  }
}

// bf16 rows (width % 8 == 0, width <= 64 * 8 * kMaxC): one row per wave,
// held packed in registers (16 bytes per chunk, 32 VGPRs for both branches)
// and unpacked twice (sums of squares, output), so that six waves fit a SIMD
// (the float copy of the row in norm_mean_rows allows five).  The two beta
// vectors are staged in LDS once per workgroup and read from there per chunk.
// Measured at 33 024 rows of 1600: 53 us (6.0 TB/s) against 70 us.  The row
// loop strides over the grid, which the launch sizes to one row per wave.

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6, 6))) void norm_mean_rows_bf16(
    const bf16_t* __restrict__ ya, const bf16_t* __restrict__ ys, const float* __restrict__ ba,
    const float* __restrict__ bs, float eps, bf16_t* __restrict__ out, long long rows,
    int width) {
  __shared__ float4 sb[2][64 * kMaxC * 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n8 = width >> 3;
  for (int i = threadIdx.x; i < 2 * n8; i += 256) {
    sb[0][i] = ((const float4*)ba)[i];
    sb[1][i] = ((const float4*)bs)[i];
  }
  __syncthreads();
  const float inv_w = 1.f / (float)width;
  for (long long row = (long long)blockIdx.x * 4 + wave; row < rows;
       row += (long long)gridDim.x * 4) {
    // beta is read from LDS per row: kept out of registers (64 of them per
    // lane would halve the waves per SIMD)
    __asm__ volatile("" ::: "memory");
    const bf16_t* pa = ya + row * width;
    const bf16_t* ps = ys + row * width;
    uint4 a[kMaxC], sv[kMaxC];
#pragma unroll
    for (int k = 0; k < kMaxC; ++k) {
      const int c = min(lane + 64 * k, n8 - 1);   // clamped: every load unconditional
      a[k] = *(const uint4*)(pa + 8 * c);
      sv[k] = *(const uint4*)(ps + 8 * c);
    }
    float sa = 0.f, ss = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxC; ++k)
      if (lane + 64 * k < n8) {
        const uint32_t wa[4] = {a[k].x, a[k].y, a[k].z, a[k].w};
        const uint32_t ws[4] = {sv[k].x, sv[k].y, sv[k].z, sv[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a0 = __uint_as_float(wa[i] << 16), a1 = __uint_as_float(wa[i] & 0xffff0000u);
          const float s0 = __uint_as_float(ws[i] << 16), s1 = __uint_as_float(ws[i] & 0xffff0000u);
          sa = fmaf(a0, a0, fmaf(a1, a1, sa));
          ss = fmaf(s0, s0, fmaf(s1, s1, ss));
        }
      }
    // the row is unpacked again for the output (not kept as 64 floats)
#pragma unroll
    for (int k = 0; k < kMaxC; ++k)
      __asm__ volatile("" : "+v"(a[k].x), "+v"(a[k].y), "+v"(a[k].z), "+v"(a[k].w),
                       "+v"(sv[k].x), "+v"(sv[k].y), "+v"(sv[k].z), "+v"(sv[k].w));
    sa = wave_sum(sa);
    ss = wave_sum(ss);
    const float ra = 0.5f / sqrtf(sa * inv_w + eps);
    const float rs = 0.5f / sqrtf(ss * inv_w + eps);
    bf16_t* po = out + row * width;
#pragma unroll
    for (int k = 0; k < kMaxC; ++k) {
      const int c = lane + 64 * k;
      if (c < n8) {
        const float4 b0 = sb[0][2 * c], b1 = sb[0][2 * c + 1];
        const float4 c0 = sb[1][2 * c], c1 = sb[1][2 * c + 1];
        const float w1[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const float w2[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const uint32_t wa[4] = {a[k].x, a[k].y, a[k].z, a[k].w};
        const uint32_t ws[4] = {sv[k].x, sv[k].y, sv[k].z, sv[k].w};
        float r[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r[2 * i] = w1[2 * i] * __uint_as_float(wa[i] << 16) * ra +
                     w2[2 * i] * __uint_as_float(ws[i] << 16) * rs;
          r[2 * i + 1] = w1[2 * i + 1] * __uint_as_float(wa[i] & 0xffff0000u) * ra +
                         w2[2 * i + 1] * __uint_as_float(ws[i] & 0xffff0000u) * rs;
        }
        Vec8<bf16_t>::st(po + 8 * c, r);
      }
      __builtin_amdgcn_sched_barrier(0);   // one chunk's beta in registers at a time
    }
  }
}

// any width
template <typename Tact>
__global__ __launch_bounds__(256) void norm_mean_scalar(const Tact* __restrict__ ya,
                                                        const Tact* __restrict__ ys,
                                                        const float* __restrict__ ba,
                                                        const float* __restrict__ bs, float eps,
                                                        Tact* __restrict__ out, long long rows,
                                                        int width) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const Tact* pa = ya + row * width;
  const Tact* ps = ys + row * width;
  float sa = 0.f, ss = 0.f;
  for (int c = lane; c < width; c += 64) {
    const float a = ActIO<Tact>::ld(pa + c), s = ActIO<Tact>::ld(ps + c);
    sa += a * a;
    ss += s * s;
  }
  sa = wave_sum(sa);
  ss = wave_sum(ss);
  const float ra = 0.5f / sqrtf(sa / (float)width + eps);
  const float rs = 0.5f / sqrtf(ss / (float)width + eps);
  Tact* po = out + row * width;
  for (int c = lane; c < width; c += 64)
    ActIO<Tact>::st(po + c, ba[c] * ActIO<Tact>::ld(pa + c) * ra + bs[c] * ActIO<Tact>::ld(ps + c) * rs);
}

template <typename Tact>
void launch_norm(const void* ya, const void* ys, const float* ba, const float* bs, float eps,
                 void* out, long long rows, int width, hipStream_t st) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (std::is_same<Tact, bf16_t>::value && width % 8 == 0 && width <= 64 * 8 * kMaxC) {
    const long long g = std::min<long long>((rows + 3) / 4, 1ll << 30);
    hipLaunchKernelGGL(norm_mean_rows_bf16, dim3((unsigned)g), dim3(256), 0, st,
                       (const bf16_t*)ya, (const bf16_t*)ys, ba, bs, eps, (bf16_t*)out, rows,
                       width);
  } else if (width % 8 == 0 && width <= 64 * 8 * kMaxC)
    hipLaunchKernelGGL(norm_mean_rows<Tact>, dim3((unsigned)((rows + kRowsPerBlock - 1) /
                                                            kRowsPerBlock)),
                       dim3(64 * kRowsPerBlock), 0, st, (const Tact*)ya, (const Tact*)ys, ba, bs,
                       eps, (Tact*)out, rows, width);
  else if (width % 8 == 0)
    hipLaunchKernelGGL(norm_mean_vec<Tact>, grid, dim3(256), 0, st, (const Tact*)ya,
                       (const Tact*)ys, ba, bs, eps, (Tact*)out, rows, width);
  else
    hipLaunchKernelGGL(norm_mean_scalar<Tact>, grid, dim3(256), 0, st, (const Tact*)ya,
                       (const Tact*)ys, ba, bs, eps, (Tact*)out, rows, width);
}

// RMS norm with a learned weight (the block's two normalisation layers):
// out = x / sqrt(mean(x^2) + eps) * w per row.  width % 8 == 0 and width <=
// 64 * 8 * kMaxC: four rows per workgroup, one per wave, held in registers;
// the weight is staged in LDS once per workgroup.
template <typename Tact>
__global__ __launch_bounds__(64 * kRowsPerBlock) void rms_norm_rows(
    const Tact* __restrict__ x, const float* __restrict__ w, float eps, Tact* __restrict__ out,
    long long rows, int width) {
  __shared__ float4 sw[64 * kMaxC * 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + wave;
  const bool live = row < rows;
  const int n8 = width >> 3;
  const Tact* px = x + row * width;
  float a[kMaxC][8];
  if (live) {
#pragma unroll
    for (int k = 0; k < kMaxC; ++k) {
      const int c = lane + 64 * k;
      if (c < n8) Vec8<Tact>::ld(px + 8 * c, a[k]);
    }
  }
  for (int i = threadIdx.x; i < 2 * n8; i += 64 * kRowsPerBlock) sw[i] = ((const float4*)w)[i];
  __syncthreads();
  if (!live) return;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxC; ++k)
    if (lane + 64 * k < n8)
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += a[k][i] * a[k][i];
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)width + eps);
  Tact* po = out + row * width;
#pragma unroll
  for (int k = 0; k < kMaxC; ++k) {
    const int c = lane + 64 * k;
    if (c < n8) {
      const float4 w0 = sw[2 * c], w1 = sw[2 * c + 1];
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = a[k][i] * r * wv[i];
      Vec8<Tact>::st(po + 8 * c, y);
    }
  }
}

// any width: one wave per row, the row read twice (the second read from L2).
template <typename Tact>
__global__ __launch_bounds__(256) void rms_norm_scalar(const Tact* __restrict__ x,
                                                       const float* __restrict__ w, float eps,
                                                       Tact* __restrict__ out, long long rows,
                                                       int width) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const Tact* px = x + row * width;
  float ss = 0.f;
  for (int c = lane; c < width; c += 64) {
    const float v = ActIO<Tact>::ld(px + c);
    ss += v * v;
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)width + eps);
  Tact* po = out + row * width;
  for (int c = lane; c < width; c += 64) ActIO<Tact>::st(po + c, ActIO<Tact>::ld(px + c) * r * w[c]);
}

}  // namespace

namespace hm {

hm_status rms_norm_impl(const void* x, const float* w, float eps, void* out, long long rows,
                        int width, hm_dtype dtype, hipStream_t st, bool dry) {
  HM_PTR(x);
  HM_PTR(w);
  HM_PTR(out);
  HM_REQUIRE(rows > 0 && width > 0, HM_ERR_INVALID, "rows and width must be positive");
  HM_REQUIRE(eps >= 0.f && std::isfinite(eps), HM_ERR_INVALID, "eps must be finite and >= 0");
  HM_REQUIRE(dtype == HM_BF16 || dtype == HM_F32, HM_ERR_UNSUPPORTED, "dtype must be f32 or bf16");
  HM_REQUIRE(out != x, HM_ERR_INVALID, "out must not alias x");
  HM_REQUIRE((rows + 3) / 4 < (1LL << 31), HM_ERR_UNSUPPORTED, "too many rows");
  if (dry) return HM_OK;
  const bool regs = width % 8 == 0 && width <= 64 * 8 * kMaxC;
  const dim3 g8((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), g4((unsigned)((rows + 3) / 4));
  if (dtype == HM_BF16) {
    if (regs)
      hipLaunchKernelGGL(rms_norm_rows<bf16_t>, g8, dim3(64 * kRowsPerBlock), 0, st,
                         (const bf16_t*)x, w, eps, (bf16_t*)out, rows, width);
    else
      hipLaunchKernelGGL(rms_norm_scalar<bf16_t>, g4, dim3(256), 0, st, (const bf16_t*)x, w,
                         eps, (bf16_t*)out, rows, width);
  } else {
    if (regs)
      hipLaunchKernelGGL(rms_norm_rows<float>, g8, dim3(64 * kRowsPerBlock), 0, st,
                         (const float*)x, w, eps, (float*)out, rows, width);
    else
      hipLaunchKernelGGL(rms_norm_scalar<float>, g4, dim3(256), 0, st, (const float*)x, w, eps,
                         (float*)out, rows, width);
  }
  return check_launch("rms_norm");
}

hm_status norm_mean_impl(const void* ya, const void* ys, const float* beta_a,
                         const float* beta_s, float eps, void* out, long long rows, int width,
                         hm_dtype dtype, hipStream_t st, bool dry) {
  HM_PTR(ya);
  HM_PTR(ys);
  HM_PTR(beta_a);
  HM_PTR(beta_s);
  HM_PTR(out);
  HM_REQUIRE(rows > 0 && width > 0, HM_ERR_INVALID, "rows and width must be positive");
  HM_REQUIRE(eps >= 0.f && std::isfinite(eps), HM_ERR_INVALID, "eps must be finite and >= 0");
  HM_REQUIRE(dtype == HM_BF16 || dtype == HM_F32, HM_ERR_UNSUPPORTED, "dtype must be f32 or bf16");
  HM_REQUIRE(out != ya && out != ys, HM_ERR_INVALID, "out must not alias ya or ys");
  HM_REQUIRE((rows + 3) / 4 < (1LL << 31), HM_ERR_UNSUPPORTED, "too many rows");
  if (dry) return HM_OK;
  if (dtype == HM_BF16)
    launch_norm<bf16_t>(ya, ys, beta_a, beta_s, eps, out, rows, width, st);
  else
    launch_norm<float>(ya, ys, beta_a, beta_s, eps, out, rows, width, st);
  return check_launch("norm_mean");
}

}  // namespace hm

extern "C" hm_status hm_branch_norm_mean(const void* ya, const void* ys, const float* beta_a,
                                         const float* beta_s, float eps, void* out,
                                         long long rows, int width, hm_dtype dtype,
                                         void* stream) {
  return hm::norm_mean_impl(ya, ys, beta_a, beta_s, eps, out, rows, width, dtype,
                            (hipStream_t)stream, false);
}

extern "C" hm_status hm_rms_norm(const void* x, const float* w, float eps, void* out,
                                 long long rows, int width, hm_dtype dtype, void* stream) {
  return hm::rms_norm_impl(x, w, eps, out, rows, width, dtype, (hipStream_t)stream, false);
}
