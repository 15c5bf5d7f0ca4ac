// Combine: the single-GPU form of the return all-to-all ("Part 5" / "1.2 Expert
// Parallelism with All-to-All Communication", step 3) fused with the mixture
// y = sum over the selected experts of weight * expert output ("moe
// communication costs" / "Router design").  "MoE: what it costs to train and
// serve" keeps combine in BF16; a dropped slot ("Capacity factor and token
// dropping") passes the token through or contributes nothing.
//
// Written as a gather (the waves of an output token read its k expert rows)
// rather than a scatter-add, so no atomics are needed and the float32 sum runs
// in slot order 0..k-1, then the shared expert, with one rounding at the end.
#include <algorithm>

#include "moe_internal.h"

#ifndef MOE_COMBINE_UNROLL
#define MOE_COMBINE_UNROLL 1
#endif

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void acc_bf16x8(float* acc, uint4 v, float w) { combine_fma8(acc, v, w); }
__device__ __forceinline__ void add_bf16x8(float* acc, uint4 v) { combine_add8(acc, v); }
__device__ __forceinline__ u32x4 pack_bf16x8(const float* acc) {
  const uint4 p = combine_pack8(acc);
  u32x4 r;
  r[0] = p.x, r[1] = p.y, r[2] = p.z, r[3] = p.w;
  return r;
}

// K slots per token; SHARED: add the shared expert's row.  Each slot's source
// row is wave-uniform: the expert output, or for a dropped slot x (pass-through;
// also read, and not added, where a drop contributes zero) or the shared
// expert's output (fallback).  All of a wave's loads go out unconditionally,
// their chunk index clamped into the row, before the first is used: loads under
// a condition made the compiler wait for each before issuing the next.
template <int K, bool SHARED>
__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const uint16_t* __restrict__ out, const uint16_t* __restrict__ out_shared,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pos, const float* __restrict__ w,
    uint16_t* __restrict__ y, int64_t T, int d, int drop_mode, int wpt) {
  constexpr int U = MOE_COMBINE_UNROLL;
  const int lane = threadIdx.x & 63;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t t = gw / wpt;                    // wpt waves share a token's row
  const int part = static_cast<int>(gw - t * wpt);
  if (t >= T) return;
  const int nch = d / 8;
  const int c0 = part * 64 + lane, cs = 64 * wpt;
  const bool fallback = drop_mode == MOE_DROP_FALLBACK && out_shared != nullptr;
  const u32x4* src[K];
  float wj[K];
  bool use[K];
  int pv[K], wv[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {              // (all loaded before the first is used)
    pv[j] = pos[t * K + j];
    wv[j] = __float_as_int(w[t * K + j]);
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int p = __builtin_amdgcn_readfirstlane(pv[j]);
    wj[j] = __int_as_float(__builtin_amdgcn_readfirstlane(wv[j]));
    const uint16_t* row = p >= 0 ? out + static_cast<int64_t>(p) * d : fallback ? out_shared + t * d : x + t * d;
    src[j] = reinterpret_cast<const u32x4*>(row);
    use[j] = p >= 0 || drop_mode == MOE_DROP_PASSTHROUGH || fallback;
  }
  const u32x4* shr = reinterpret_cast<const u32x4*>(SHARED ? out_shared + t * d : x);
  u32x4* yr = reinterpret_cast<u32x4*>(y + t * d);
  u32x4 v[U][K], sh[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int cc = min(c0 + i * cs, nch - 1);
#pragma unroll
    for (int j = 0; j < K; ++j) v[i][j] = __builtin_nontemporal_load(src[j] + cc);
    if (SHARED) sh[i] = __builtin_nontemporal_load(shr + cc);
  }
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int c = c0 + i * cs;
    if (c < nch) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < K; ++j)
        if (use[j]) acc_bf16x8(acc, make_uint4(v[i][j][0], v[i][j][1], v[i][j][2], v[i][j][3]), wj[j]);
      if (SHARED) add_bf16x8(acc, make_uint4(sh[i][0], sh[i][1], sh[i][2], sh[i][3]));
      yr[c] = pack_bf16x8(acc);
    }
  }
  // rows longer than the host's split assumes: the rest chunk by chunk
  for (int c = c0 + U * cs; c < nch; c += cs) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (use[j]) {
        const u32x4 q = src[j][c];
        acc_bf16x8(acc, make_uint4(q[0], q[1], q[2], q[3]), wj[j]);
      }
    if (SHARED) {
      const u32x4 q = shr[c];
      add_bf16x8(acc, make_uint4(q[0], q[1], q[2], q[3]));
    }
    yr[c] = pack_bf16x8(acc);
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

// Before the combining down GEMM: cnt[t][c] = -(kept slots of t + shared), for
// every column group c; a token that no output row reaches (every slot dropped,
// no shared expert) gets its y here, as the combine kernel computes it: sum of
// w * x[t] over the slots (pass-through) or zero.  One thread per (token, group).
__global__ __launch_bounds__(256) void scatter_init_kernel(const int32_t* __restrict__ pos,
                                                           const float* __restrict__ w,
                                                           const uint16_t* __restrict__ x,
                                                           int32_t* __restrict__ cnt,
                                                           uint16_t* __restrict__ y, int64_t T, int k,
                                                           int d, int G, int shared, int drop_mode) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t t = q / G;
  if (t >= T) return;
  const int grp = static_cast<int>(q - t * G);
  int nk = shared;
  for (int j = 0; j < k; ++j) nk += pos[t * k + j] >= 0 ? 1 : 0;
  cnt[q] = -nk;
  if (nk > 0) return;
  const bool pass = drop_mode == MOE_DROP_PASSTHROUGH;
  for (int col = grp * kScatterCols; col < min(d, (grp + 1) * kScatterCols); col += 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (pass) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + t * d + col);
      for (int j = 0; j < k; ++j) combine_fma8(acc, v, w[t * k + j]);
    }
    *reinterpret_cast<uint4*>(y + t * d + col) = combine_pack8(acc);
  }
}

}  // namespace

hipError_t launch_scatter_init(const moe_shape& s, const int32_t* pos, const float* w, const void* x,
                               int32_t* cnt, void* y, hipStream_t st) {
  const int G = static_cast<int>(ceil_div(s.d, kScatterCols));
  const int64_t n = s.T * G;
  hipLaunchKernelGGL(scatter_init_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, st,
                     pos, w, static_cast<const uint16_t*>(x), cnt, static_cast<uint16_t*>(y), s.T, s.k,
                     s.d, G, s.has_shared ? 1 : 0, s.drop);
  return hipGetLastError();
}

hipError_t launch_combine(const moe_shape& s, const void* out, const void* out_shared,
                          const void* x, const int32_t* pos, const float* w, void* y,
                          hipStream_t st) {
  // Several waves per token, each a strided share of the row's 64-lane
  // chunks: as many as give each lane MOE_COMBINE_UNROLL chunks (its loads, all
  // k slots of all its chunks, in flight together), and with few tokens enough
  // for ~2048 waves in all.  One chunk per lane measured best (Mixtral shape
  // 21.0 us against 21.4 with two and 21.2 with four; DBRX shape 160 / 161 /
  // 161 us; DeepSeek-V3 103 / 104 / 110 us).
  const int64_t chunks = s.dtype == MOE_BF16 ? s.d / 8 / 64 : s.d / 64;
  int64_t wpt = std::max<int64_t>(ceil_div(2048, s.T), ceil_div(chunks, MOE_COMBINE_UNROLL));
  if (wpt > chunks) wpt = chunks;
  if (wpt < 1) wpt = 1;
  dim3 grid(static_cast<unsigned>(ceil_div(s.T * wpt, 4)));
  const int pt = s.drop;
  if (s.dtype == MOE_BF16) {
    const uint16_t* o = static_cast<const uint16_t*>(out);
    const uint16_t* os = static_cast<const uint16_t*>(out_shared);
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    uint16_t* ys = static_cast<uint16_t*>(y);
    const int wp = static_cast<int>(wpt);
    const bool sh = out_shared != nullptr;
    switch (s.k) {
#define MOE_COMBINE_K(K)                                                                          \
  case K:                                                                                         \
    if (sh)                                                                                       \
      hipLaunchKernelGGL((combine_bf16_kernel<K, true>), grid, dim3(256), 0, st, o, os, xs, pos, w, \
                         ys, s.T, s.d, pt, wp);                                                   \
    else                                                                                          \
      hipLaunchKernelGGL((combine_bf16_kernel<K, false>), grid, dim3(256), 0, st, o, os, xs, pos, \
                         w, ys, s.T, s.d, pt, wp);                                                \
    break;
      MOE_COMBINE_K(1) MOE_COMBINE_K(2) MOE_COMBINE_K(3) MOE_COMBINE_K(4)
      MOE_COMBINE_K(5) MOE_COMBINE_K(6) MOE_COMBINE_K(7) MOE_COMBINE_K(8)
#undef MOE_COMBINE_K
      default:
        return hipErrorInvalidValue;
    }
  } else
    hipLaunchKernelGGL(combine_f32_kernel, grid, dim3(256), 0, st,
                       static_cast<const float*>(out), static_cast<const float*>(out_shared),
                       static_cast<const float*>(x), pos, w, static_cast<float*>(y), s.T, s.k,
                       s.d, pt, static_cast<int>(wpt));
  return hipGetLastError();
}

}  // namespace moe
