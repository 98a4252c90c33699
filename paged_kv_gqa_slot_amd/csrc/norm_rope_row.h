// Per-head QK-RMSNorm and rotate-half rotary embedding of one 128-dim head
// row, held by the 16 lanes of a DPP row (lane c: dims 8c .. 8c + 7) --
// shared by the fused norm/rotary/append kernel and by the decode kernel's
// form that applies it to q and to the appended k itself ("Make the Engine
// Talk" section 1.3: RMSNorm and rotary position embeddings are forward-pass
// mechanisms; ForgeEngine README, "What it implements": an RMSNorm kernel).
//
//   y = x * w / sqrt(mean(x^2) + eps)
//   y'[d] = y[d] c_d - y[d + 64] s_d,  y'[d + 64] = y[d + 64] c_d + y[d] s_d   (d < 64)
// in fp32, rounded once to bf16.  The rotary table row holds the 64 cosines
// and then the 64 sines of one position.
#pragma once

#include <math.h>

#include "fe_device.h"
#include "fe_kernels.h"

namespace fe {

// Sum over the 16 lanes of a DPP row; every lane gets it.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}

// This lane's cosines (c0, c1) and sines (s0, s1) of its 8 dims.
struct RopeLane {
  float4 c0, c1, s0, s1;
};

// Table row pos (clamped by the caller) of the fp32 table [max_pos][128].
__device__ __forceinline__ RopeLane rope_lane(const float* cos_sin, int pos, int c) {
  const int d0 = 8 * (c & 7);  // angle index of this lane's first dim
  const float4* cs = reinterpret_cast<const float4*>(cos_sin + static_cast<size_t>(pos) * kHeadDim + d0);
  return RopeLane{cs[0], cs[1], cs[16], cs[17]};  // the sines sit 64 floats further
}

// Normalised and rotated row, this lane's 8 dims as packed bf16.  Every lane
// of the 16-lane row must call it (the DPP sum and rotation read the others).
__device__ __forceinline__ uint4 norm_rope_row(uint4 xw, uint4 ww, const RopeLane& cs, float eps, int c) {
  float x[8];
  x[0] = bf16_lo(xw.x); x[1] = bf16_hi(xw.x);
  x[2] = bf16_lo(xw.y); x[3] = bf16_hi(xw.y);
  x[4] = bf16_lo(xw.z); x[5] = bf16_hi(xw.z);
  x[6] = bf16_lo(xw.w); x[7] = bf16_hi(xw.w);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = fmaf(x[j], x[j], ss);
  ss = row_sum16(ss);
  const float inv_rms = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);

  float y[8];
  y[0] = x[0] * inv_rms * bf16_lo(ww.x); y[1] = x[1] * inv_rms * bf16_hi(ww.x);
  y[2] = x[2] * inv_rms * bf16_lo(ww.y); y[3] = x[3] * inv_rms * bf16_hi(ww.y);
  y[4] = x[4] * inv_rms * bf16_lo(ww.z); y[5] = x[5] * inv_rms * bf16_hi(ww.z);
  y[6] = x[6] * inv_rms * bf16_lo(ww.w); y[7] = x[7] * inv_rms * bf16_hi(ww.w);

  // the partner dims (d + 64 for lanes 0-7, d - 64 for lanes 8-15)
  float z[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = dpp<kDppRowRor8>(y[j]);

  const float cv[8] = {cs.c0.x, cs.c0.y, cs.c0.z, cs.c0.w, cs.c1.x, cs.c1.y, cs.c1.z, cs.c1.w};
  const float sv[8] = {cs.s0.x, cs.s0.y, cs.s0.z, cs.s0.w, cs.s1.x, cs.s1.y, cs.s1.z, cs.s1.w};
  // first half: y c - z s; second half: y c + z s
  const float sgn = c < 8 ? -1.0f : 1.0f;
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = fmaf(sgn * z[j], sv[j], y[j] * cv[j]);
  return make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                    pack_bf16x2(o[6], o[7]));
}

}  // namespace fe
