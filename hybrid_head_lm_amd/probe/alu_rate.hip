// Instruction-rate probe of the gfx950 vector ALU, for the benchmark's ALU
// ceilings (not part of libhm).  Every lane runs 8 independent dependency
// chains of register-only instructions written in inline asm, so the
// instruction counts are exactly the ones below; no memory is touched inside
// the loop and each lane stores one float at the end (so nothing is dead).
//   mode 0: v_exp_f32 only (8 per iteration per lane)
//   mode 1: v_fma_f32 only (8 per iteration per lane)
//   mode 2: the selective scan's single-pass instruction mix per
//           token-channel, 20 transcendental + 77 other VALU instructions,
//           on each of the 8 chains (one chain iteration = one token-channel)
// Timing is the caller's (HIP events around the launch on its stream).
#include <hip/hip_runtime.h>

namespace {

__device__ __forceinline__ float vexp(float x) {
  float r;
  asm volatile("v_exp_f32_e64 %0, -%1" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ float vfma(float x, float a, float b) {
  float r;
  asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(a), "v"(b));
  return r;
}

template <int MODE>
__global__ __launch_bounds__(256) void alu_probe(float* __restrict__ out, int iters, float a,
                                                 float b, long long* __restrict__ clk) {
  // shader-clock cycles (s_memtime) and 100 MHz ticks (s_memrealtime) around
  // the loop, recorded by lane 0 of each wave: their ratio is the clock the
  // wave ran at
  const long long c0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.25f + 0.01f * (float)(threadIdx.x & 7) + 0.001f * i;
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = vexp(x[i]);
    } else if constexpr (MODE == 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = vfma(x[i], a, b);
    } else {
      // per chain: 20 exp and 77 fma, interleaved as the scan issues them
      // (one exp, then about four dependent multiply-adds)
#pragma unroll
      for (int k = 0; k < 20; ++k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = vexp(x[i]);
#pragma unroll
        for (int j = 0; j < (k < 17 ? 4 : 3); ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = vfma(x[i], a, b);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  const long long c1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  if (clk != nullptr && (threadIdx.x & 63) == 0) {
    const int w = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    clk[2 * w] = c1 - c0;
    clk[2 * w + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Instructions per lane per iteration of each mode: (transcendental, other VALU).
void hm_probe_alu_counts(int mode, int* trans, int* valu) {
  *trans = mode == 0 ? 8 : (mode == 1 ? 0 : 160);
  *valu = mode == 0 ? 0 : (mode == 1 ? 8 : 8 * 77);
}

// Launch `blocks` workgroups of `threads` lanes (a multiple of 64, at most
// 256), each running `iters` iterations of `mode`; out: device float
// [blocks * threads]; clk: device int64 [2 * blocks * threads / 64] or NULL
// (per wave: shader cycles, 100 MHz ticks).  Returns 0 on success.
int hm_probe_alu(int mode, float* out, int blocks, int threads, int iters, long long* clk,
                 void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0 || mode < 0 || mode > 2 || threads < 64 ||
      threads > 256 || threads % 64 != 0)
    return 1;
  hipStream_t st = (hipStream_t)stream;
  const dim3 g(blocks), t(threads);
  if (mode == 0)
    hipLaunchKernelGGL(alu_probe<0>, g, t, 0, st, out, iters, 0.999f, 0.001f, clk);
  else if (mode == 1)
    hipLaunchKernelGGL(alu_probe<1>, g, t, 0, st, out, iters, 0.999f, 0.001f, clk);
  else
    hipLaunchKernelGGL(alu_probe<2>, g, t, 0, st, out, iters, 0.999f, 0.001f, clk);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
