// Pieces shared by the projection kernels (bf16 MFMA GEMM, y = x W^T with the
// weight in nn.Linear layout [N, K]): the per-segment output description and
// epilogue, and the launch of the 4-wave 256 x 256 tile kernel.
#pragma once

#include "hm_common.h"

namespace hm_lin {

constexpr int kMaxSeg = 8;
typedef __attribute__((address_space(3))) void lin_lds_t;

struct LinOut {
  bf16_t* p[kMaxSeg];          // segment outputs, [M, col0[s+1] - col0[s]]
  const float* bias[kMaxSeg];  // per segment: [width] f32 or null
  const bf16_t* res[kMaxSeg];  // per segment: [M, width] or null (may be p[s] itself)
  int act[kMaxSeg];            // per segment: HM_ACT_*
  int col0[kMaxSeg + 1];       // segment s holds the output columns [col0[s], col0[s+1])
  int n;                       // segments
};

// The segment holding output column `col`, chosen with compile-time indices
// only (a lane-varying index into the argument struct would copy it to
// scratch memory).
struct SegPick {
  bf16_t* dst;
  const bf16_t* res;
  const float* bias;
  int act, c0, ld;
};
HM_DEV SegPick pick_segment(const LinOut& out, int col) {
  SegPick p{out.p[0], out.res[0], out.bias[0], out.act[0], 0, out.col0[1]};
#pragma unroll
  for (int q = 1; q < kMaxSeg; ++q)
    if (q < out.n && col >= out.col0[q])
      p = SegPick{out.p[q], out.res[q], out.bias[q], out.act[q], out.col0[q],
                  out.col0[q + 1] - out.col0[q]};
  return p;
}

// v + bias, then the activation, then + residual, in float32.
HM_DEV float lin_act(float v, int act) {
  if (act == HM_ACT_SILU) return v / (1.f + __expf(-v));
  if (act == HM_ACT_SOFTPLUS) return v > 20.f ? v : log1pf(__expf(v));
  return v;
}

// The epilogue of one 16-byte output chunk: columns col .. col + 7 of `row`
// (one segment, as segment widths are multiples of 16), v = the float32
// products read back from the staging tile: + bias, activation, + residual,
// rounded to bf16 and stored with one 16-byte store.
HM_DEV void store_chunk8(const LinOut& out, int row, int col, const float4& v0,
                         const float4& v1) {
  float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  const SegPick sp = pick_segment(out, col);
  const int cn = col - sp.c0;
  if (sp.bias) {
    const float4 b0 = *(const float4*)(sp.bias + cn), b1 = *(const float4*)(sp.bias + cn + 4);
    v[0] += b0.x; v[1] += b0.y; v[2] += b0.z; v[3] += b0.w;
    v[4] += b1.x; v[5] += b1.y; v[6] += b1.z; v[7] += b1.w;
  }
  if (sp.act != HM_ACT_NONE)
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = lin_act(v[k], sp.act);
  const size_t e = (size_t)row * sp.ld + cn;
  if (sp.res) {
    const uint4 rr = *(const uint4*)(sp.res + e);
    const uint32_t rw[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] += __uint_as_float(rw[k] << 16);
      v[2 * k + 1] += __uint_as_float(rw[k] & 0xffff0000u);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(v[0], v[1]);
  o.y = pack_bf16x2(v[2], v[3]);
  o.z = pack_bf16x2(v[4], v[5]);
  o.w = pack_bf16x2(v[6], v[7]);
  *(uint4*)(sp.dst + e) = o;
}

// 256 x 256 tiles, 4 waves (linear_w4.hip).  Arguments validated by the caller.
void launch_w4(const bf16_t* x, const bf16_t* w, int M, int N, int K, const LinOut& out,
               hipStream_t st);

}  // namespace hm_lin
