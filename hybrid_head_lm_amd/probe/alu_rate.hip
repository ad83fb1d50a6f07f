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
                                                 float b) {
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
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Instructions per lane per iteration of each mode: (transcendental, other VALU).
void hm_probe_alu_counts(int mode, int* trans, int* valu) {
  *trans = mode == 0 ? 8 : (mode == 1 ? 0 : 160);
  *valu = mode == 0 ? 0 : (mode == 1 ? 8 : 8 * 77);
}

// Launch `blocks` workgroups of 256 lanes, each running `iters` iterations of
// `mode`; out: device float [blocks * 256].  Returns 0 on success.
int hm_probe_alu(int mode, float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0 || mode < 0 || mode > 2) return 1;
  hipStream_t st = (hipStream_t)stream;
  if (mode == 0)
    hipLaunchKernelGGL(alu_probe<0>, dim3(blocks), dim3(256), 0, st, out, iters, 0.999f, 0.001f);
  else if (mode == 1)
    hipLaunchKernelGGL(alu_probe<1>, dim3(blocks), dim3(256), 0, st, out, iters, 0.999f, 0.001f);
  else
    hipLaunchKernelGGL(alu_probe<2>, dim3(blocks), dim3(256), 0, st, out, iters, 0.999f, 0.001f);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
