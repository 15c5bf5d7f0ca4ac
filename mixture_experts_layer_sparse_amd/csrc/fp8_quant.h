// FP8 (e4m3) quantisation of bf16 rows, one scale per row, as the dispatch
// step does before the send ("MoE: what it costs to train and serve" / "Worked
// example: how many bytes does one token send?": FP8 payload before dispatch).
// The row's scale is max|x| / 448 (448 the largest e4m3 value), the codes are
// x * (448 / max|x|) rounded to nearest even; rows below 2^-100 (zero included)
// take scale 1.  Shared by the dispatch quantiser and the few-token router
// kernel, so that both write the same bits.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// max |x| over the 8 bf16 values of one 16-byte chunk
__device__ __forceinline__ float absmax8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
    m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
  }
  return m;
}

// 8 bf16 values times inv -> 8 e4m3 codes (nearest even), in element order
__device__ __forceinline__ uint2 quant8(uint4 v, float inv) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16) * inv;
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) * inv;
  }
  // two floats -> two e4m3 codes into the low / high half-word
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
}

// The row's multiplier (448 / amax) and scale (amax / 448), both correctly rounded.
__device__ __forceinline__ void fp8_row_scale(float amax, float* inv, float* scale) {
  const bool tiny = amax < 0x1p-100f;
  *inv = tiny ? 1.f : __fdiv_rn(448.0f, amax);
  *scale = tiny ? 1.f : __fdiv_rn(amax, 448.0f);
}

}  // namespace moe
