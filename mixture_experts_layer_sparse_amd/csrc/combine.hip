// Combine: the single-GPU form of the return all-to-all ("Part 5" / "1.2 Expert
// Parallelism with All-to-All Communication", step 3) fused with the mixture
// y = sum over the selected experts of weight * expert output ("moe
// communication costs" / "Router design").  "MoE: what it costs to train and
// serve" keeps combine in BF16; a dropped slot ("Capacity factor and token
// dropping") passes the token through or contributes nothing.
//
// Written as a gather (one wave per output token reads its k expert rows)
// rather than a scatter-add, so no atomics are needed and the float32 sum runs
// in slot order 0..k-1, then the shared expert, with one rounding at the end.
#include <algorithm>

#include "moe_internal.h"

#ifndef MOE_COMBINE_UNROLL
#define MOE_COMBINE_UNROLL 2
#endif

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void acc_bf16x8(float* acc, uint4 v, float w) {
  const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, __uint_as_float(q[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, __uint_as_float(q[i] & 0xFFFF0000u), acc[2 * i + 1]);
  }
}
__device__ __forceinline__ void add_bf16x8(float* acc, uint4 v) {
  const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += __uint_as_float(q[i] << 16);
    acc[2 * i + 1] += __uint_as_float(q[i] & 0xFFFF0000u);
  }
}

__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const uint16_t* __restrict__ out, const uint16_t* __restrict__ out_shared,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pos, const float* __restrict__ w,
    uint16_t* __restrict__ y, int64_t T, int k, int d, int drop_mode, int wpt) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t t = gw / wpt;                    // wpt waves share a token's row
  const int part = static_cast<int>(gw - t * wpt);
  if (t >= T) return;
  int pj[kMaxTopK];
  float wj[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    pj[j] = j < k ? pos[t * k + j] : -1;
    wj[j] = j < k ? w[t * k + j] : 0.f;
  }
  const int nch = d / 8;
#pragma unroll MOE_COMBINE_UNROLL
  for (int c = part * 64 + lane; c < nch; c += 64 * wpt) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        if (pj[j] >= 0) {
          const u32x4 q = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(out + static_cast<int64_t>(pj[j]) * d) + c);
          const uint4 v = make_uint4(q[0], q[1], q[2], q[3]);
          acc_bf16x8(acc, v, wj[j]);
        } else if (drop_mode == MOE_DROP_PASSTHROUGH) {
          uint4 v = reinterpret_cast<const uint4*>(x + t * d)[c];
          acc_bf16x8(acc, v, wj[j]);
        } else if (drop_mode == MOE_DROP_FALLBACK) {
          uint4 v = reinterpret_cast<const uint4*>(out_shared + t * d)[c];
          acc_bf16x8(acc, v, wj[j]);
        }
      }
    }
    if (out_shared) add_bf16x8(acc, reinterpret_cast<const uint4*>(out_shared + t * d)[c]);
    uint4 r;
    r.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    r.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    r.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    r.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    reinterpret_cast<uint4*>(y + t * d)[c] = r;
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(
    const float* __restrict__ out, const float* __restrict__ out_shared,
    const float* __restrict__ x, const int32_t* __restrict__ pos, const float* __restrict__ w,
    float* __restrict__ y, int64_t T, int k, int d, int drop_mode, int wpt) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t t = gw / wpt;
  const int part = static_cast<int>(gw - t * wpt);
  if (t >= T) return;
  for (int c = part * 64 + lane; c < d; c += 64 * wpt) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      int p = pos[t * k + j];
      float wj = w[t * k + j];
      if (p >= 0) acc = fmaf(wj, out[static_cast<int64_t>(p) * d + c], acc);
      else if (drop_mode == MOE_DROP_PASSTHROUGH) acc = fmaf(wj, x[t * d + c], acc);
      else if (drop_mode == MOE_DROP_FALLBACK) acc = fmaf(wj, out_shared[t * d + c], acc);
    }
    if (out_shared) acc += out_shared[t * d + c];
    y[t * d + c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const void* out, const void* out_shared,
                          const void* x, const int32_t* pos, const float* w, void* y,
                          hipStream_t st) {
  // Several waves per token, each a strided share of the row's 64-lane
  // chunks: enough that a wave's chunk loop is one unrolled pass (all its loads
  // in flight together; a wave walking a long row waits out the memory latency
  // once per pass), and with few tokens enough for ~2048 waves in all.
  // Measured against one wave per token: DBRX shape 195 -> 168 us, DeepSeek-V3
  // 122 -> 102 us, Mixtral 27.2 -> 26.1 us; one chunk per wave was no better.
  const int64_t chunks = s.dtype == MOE_BF16 ? s.d / 8 / 64 : s.d / 64;
  int64_t wpt = std::max<int64_t>(ceil_div(2048, s.T), ceil_div(chunks, MOE_COMBINE_UNROLL));
  if (wpt > chunks) wpt = chunks;
  if (wpt < 1) wpt = 1;
  dim3 grid(static_cast<unsigned>(ceil_div(s.T * wpt, 4)));
  const int pt = s.drop;
  if (s.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_bf16_kernel, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(out_shared),
                       static_cast<const uint16_t*>(x), pos, w, static_cast<uint16_t*>(y), s.T,
                       s.k, s.d, pt, static_cast<int>(wpt));
  else
    hipLaunchKernelGGL(combine_f32_kernel, grid, dim3(256), 0, st,
                       static_cast<const float*>(out), static_cast<const float*>(out_shared),
                       static_cast<const float*>(x), pos, w, static_cast<float*>(y), s.T, s.k,
                       s.d, pt, static_cast<int>(wpt));
  return hipGetLastError();
}

}  // namespace moe
