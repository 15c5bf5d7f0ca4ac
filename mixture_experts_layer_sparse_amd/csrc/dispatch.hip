// Dispatch: the single-GPU form of the dispatch all-to-all.  "Part 5" / "1.2
// Expert Parallelism with All-to-All Communication" builds one send buffer per
// destination from the routing decisions; "MoE: what it costs to train and
// serve" / "Expert parallelism and two all-to-alls" describes the same step.
// With every expert local, the send buffer becomes one expert-contiguous
// buffer: a histogram, a prefix scan, a stable rank, and a row copy.
// "Capacity factor and token dropping" ("moe communication costs") bounds each
// expert's rows; "Worked example: how many bytes does one token send?" gives
// the payload k*d*s per token and FP8 (s = 1) before dispatch.
//
// Kernels
//   disp_hist  per block of 256 tokens, an LDS histogram of the block's
//              assignments (integer atomics: the counts do not depend on order).
//   disp_plan  per block: the block's base per expert (sum over earlier
//              blocks), the kept counts and their exclusive scan (offsets), and
//              the stable in-block rank of every assignment from wave ballots
//              (match on the expert-id bits) plus a wave-ordered LDS prefix.
//              No atomics decide a position, so the permutation is unique.
//   disp_copy  a few waves per token: read the row once, write it to each kept
//              slot's position (bf16/f32 copy, or fp8 e4m3 with a per-token scale).
// Within a whole layer the router has already counted each expert's
// assignments per router tile (8 or 16 tokens), and its finalisation turns them into
// per-tile bases; the copy then places its token itself (the tile's base plus
// the earlier tokens of the same tile that chose the expert), so the layer
// needs neither disp_hist nor disp_plan.  The order is the same token order, so
// the permutation is the same.
#include <algorithm>

#include "fp8_quant.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TB = kDispatchBlock;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void disp_hist_kernel(const int32_t* __restrict__ idx, int64_t T,
                                                        int k, int N, int32_t* __restrict__ hist) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < kMaxExperts; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * TB + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      int e = idx[t * k + j];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(N)) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256) hist[static_cast<int64_t>(blockIdx.x) * N + e] = h[e];
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__global__ __launch_bounds__(256) void disp_plan_kernel(const int32_t* __restrict__ idx, int64_t T,
                                                        int k, int N, int cap,
                                                        const int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ pos,
                                                        int32_t* __restrict__ src,
                                                        uint8_t* __restrict__ drop) {
  __shared__ int base[kMaxExperts];       // assignments to e in earlier blocks
  __shared__ int scan[2][kMaxExperts + 1];
  __shared__ int wh[4][kMaxExperts];      // per-wave counts inside this block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x, nb = gridDim.x;

  // 1. totals and this block's base, kept counts
  for (int e = tid; e < kMaxExperts; e += 256) {
    int tot = 0, bb = 0;
    if (e < N) {
      for (int b = 0; b < nb; ++b) {
        int h = hist[static_cast<int64_t>(b) * N + e];
        if (b < blk) bb += h;
        tot += h;
      }
    }
    base[e] = bb;
    int kept = cap > 0 ? (tot < cap ? tot : cap) : tot;
    scan[0][e] = e < N ? kept : 0;
    wh[0][e] = wh[1][e] = wh[2][e] = wh[3][e] = 0;
  }
  __syncthreads();
  // 2. inclusive scan over experts (Hillis-Steele, ping-pong buffers)
  int cur = 0;
  for (int off = 1; off < kMaxExperts; off <<= 1) {
    for (int e = tid; e < kMaxExperts; e += 256)
      scan[cur ^ 1][e] = scan[cur][e] + (e >= off ? scan[cur][e - off] : 0);
    cur ^= 1;
    __syncthreads();
  }
  // exclusive offset of e = inclusive[e - 1]
  if (blk == 0) {
    for (int e = tid; e <= N; e += 256) offsets[e] = e == 0 ? 0 : scan[cur][e - 1];
  }

  // 3. in-block stable ranks
  const int64_t t = static_cast<int64_t>(blk) * TB + tid;
  const bool valid = t < T;
  int ej[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    int e = -1;
    if (j < k && valid) {
      e = idx[t * k + j];
      if (static_cast<unsigned>(e) >= static_cast<unsigned>(N)) e = -1;
    }
    ej[j] = e;
    if (e >= 0) atomicAdd(&wh[wave][e], 1);
  }
  int nbits = 1;
  while ((1 << nbits) < N) ++nbits;
  int rank[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) rank[j] = 0;
  const uint64_t lt = lanemask_lt(lane);
#pragma unroll
  for (int jp = 0; jp < kMaxTopK; ++jp) {
    if (jp < k) {
      const uint64_t vb = __ballot(ej[jp] >= 0);
      uint64_t bal[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) bal[b] = b < nbits ? __ballot((ej[jp] >> b) & 1) : 0ull;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k) {
          uint64_t m = vb & lt;
#pragma unroll
          for (int b = 0; b < 8; ++b)
            if (b < nbits) m &= ((ej[j] >> b) & 1) ? bal[b] : ~bal[b];
          rank[j] += __popcll(m);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k && valid) {
      const int e = ej[j];
      int p = -1;
      if (e >= 0) {
        int r = base[e] + rank[j];
        for (int w = 0; w < wave; ++w) r += wh[w][e];
        if (cap <= 0 || r < cap) {
          p = (e == 0 ? 0 : scan[cur][e - 1]) + r;
          src[p] = static_cast<int32_t>(t);
        }
      }
      pos[t * k + j] = p;
      drop[t * k + j] = p < 0 ? 1 : 0;
    }
  }
}

// Slot positions of token t when the copy does the planning (see above):
// for slot j with expert e, r = base[tile][e] + (earlier tokens of t's tile
// that chose e); kept when there is no capacity or r < cap, at offsets[e] + r.
// Lane 0 writes pos, drop and src.  pj[] is the same in every lane.
struct PlanArgs {
  const int32_t* idx;
  const int32_t* base;     // [tiles][N]
  const int32_t* offsets;  // [N + 1]
  int32_t* pos;
  int32_t* src;
  uint8_t* drop;
  int N, cap;
  int tile;                // tokens per router tile
};

__device__ __forceinline__ void plan_token(const PlanArgs& pa, int64_t T, int k, int64_t t, int lane,
                                           int pj[kMaxTopK]) {
  const int TM = pa.tile;
  const int64_t tile = t / TM, t0 = tile * TM;
  const int before = static_cast<int>(t - t0) * k;        // idx entries of earlier tokens in the tile
  // The loads go out in two batches: the tile's earlier entries and this
  // token's choices, then the choices' tile bases and offsets (two latencies,
  // not three per choice).  Lane l holds entries l and l + 64 of the tile
  // (TM * k <= 128).
  const int v0 = (lane < before) ? pa.idx[t0 * k + lane] : -1;
  const int v1 = (lane + 64 < before) ? pa.idx[t0 * k + lane + 64] : -1;
  int e[kMaxTopK], b[kMaxTopK], o[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) e[j] = j < k ? pa.idx[t * k + j] : -1;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    const bool ok = static_cast<unsigned>(e[j]) < static_cast<unsigned>(pa.N);
    b[j] = ok ? pa.base[tile * pa.N + e[j]] : 0;
    o[j] = ok ? pa.offsets[e[j]] : 0;
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    int p = -1;
    if (static_cast<unsigned>(e[j]) < static_cast<unsigned>(pa.N)) {
      const int r = b[j] + __popcll(__ballot(v0 == e[j])) + __popcll(__ballot(v1 == e[j]));
      if (pa.cap <= 0 || r < pa.cap) p = o[j] + r;
    }
    // the same in every lane: as a scalar, a slot's row base is an SGPR pair
    pj[j] = __builtin_amdgcn_readfirstlane(p);
  }
}

// pos, drop and src of one token, from lane 0 of one of its waves.  They are
// written after the rows: the row stores then follow each other with no wait
// for a store issued before them.
__device__ __forceinline__ void plan_write(const PlanArgs& pa, int k, int64_t t, const int pj[kMaxTopK]) {
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) {
      pa.pos[t * k + j] = pj[j];
      pa.drop[t * k + j] = pj[j] < 0 ? 1 : 0;
      if (pj[j] >= 0) pa.src[pj[j]] = static_cast<int32_t>(t);
    }
}

// Positions handed in by the caller, one token's k entries (the same address in
// every lane, hence uniform).
__device__ __forceinline__ void given_positions(const int32_t* pos, int k, int64_t t, int pj[kMaxTopK]) {
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) pj[j] = j < k ? __builtin_amdgcn_readfirstlane(pos[t * k + j]) : -1;
}

// The plan alone (the fused layer: the up GEMM reads x through src, so no
// rows are copied): one wave per token writes its pos, drop and src.
__global__ __launch_bounds__(256) void disp_plan_tiles_kernel(int64_t T, int k, PlanArgs pa) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int pj[kMaxTopK];
  plan_token(pa, T, k, t, lane, pj);
  if (lane == 0) plan_write(pa, k, t, pj);
}

// wpt waves per token; 16-byte chunks.  Row bytes must be a multiple of 16.
// PLANNED: positions from plan_token, else read from pos.  A lane's first
// kCopyAhead chunks are loaded before the positions, so that the row's latency
// overlaps theirs (the host picks wpt so that these are all of them).  The
// loads are unconditional, their index clamped into the row: under a
// condition, even a uniform one, the compiler waited for each before the next.
// Rows are then stored slot by slot, to a scalar row base plus a fixed
// per-chunk offset, so that no store waits for an earlier one to leave.
constexpr int kCopyAhead = 4;
template <bool PLANNED>
__global__ __launch_bounds__(256) void disp_copy_kernel(const uint8_t* __restrict__ x, int64_t T,
                                                        int k, int row_bytes,
                                                        const int32_t* __restrict__ pos,
                                                        uint8_t* __restrict__ xp, PlanArgs pa, int wpt) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t t = gw / wpt;                    // wpt waves share a token's row
  const int part = static_cast<int>(gw - t * wpt);
  if (t >= T) return;
  const int nch = row_bytes / 16;
  const int c0 = part * 64 + lane, cs = 64 * wpt;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + t * row_bytes);
  u32x4 q[kCopyAhead];
#pragma unroll
  for (int i = 0; i < kCopyAhead; ++i)       // (index clamped into the row; such lanes store nothing)
    q[i] = __builtin_nontemporal_load(xr + min(c0 + i * cs, nch - 1));
  int pj[kMaxTopK];
  if (PLANNED)
    plan_token(pa, T, k, t, lane, pj);
  else
    given_positions(pos, k, t, pj);
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (pj[j] < 0) continue;
    u32x4* dst = reinterpret_cast<u32x4*>(xp + static_cast<int64_t>(pj[j]) * row_bytes);
#pragma unroll
    for (int i = 0; i < kCopyAhead; ++i)
      if (c0 + i * cs < nch) dst[c0 + i * cs] = q[i];
  }
  for (int c = c0 + kCopyAhead * cs; c < nch; c += cs) {
    const u32x4 r = __builtin_nontemporal_load(xr + c);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (pj[j] >= 0) reinterpret_cast<u32x4*>(xp + static_cast<int64_t>(pj[j]) * row_bytes)[c] = r;
  }
  if (PLANNED && part == 0 && lane == 0) plan_write(pa, k, t, pj);
}

// fp8 dispatch: WPT waves per token in one workgroup (the row's max |x| meets
// in LDS), so that a token's row is read and written by 64 * WPT lanes.  Rows
// up to 64*WPT*MAXC chunks of 8 bf16 stay in registers; longer rows are read
// twice.
//
// TOKEN_ORDER (the fused layer, whose up GEMM gathers its rows through src):
// the codes are written once, to row t of xp ([T][d]), and only the kept
// slots' scales go to their positions.
template <int MAXC, bool PLANNED, int WPT, bool TOKEN_ORDER = false>
__global__ __launch_bounds__(256) void disp_fp8_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                       int k, int d,
                                                       const int32_t* __restrict__ pos,
                                                       uint8_t* __restrict__ xp,
                                                       float* __restrict__ row_scale, PlanArgs pa) {
  static_assert(4 % WPT == 0, "a token's waves share one workgroup");
  __shared__ float wmax[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = wave % WPT;                     // this wave's part of the token's row
  const int tl = sub * 64 + lane;                 // lane within the token
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (4 / WPT) + wave / WPT;
  if (t >= T) return;                             // (whole tokens: the waves of one token agree)
  const int nch = d / 8;
  const uint4* xr = reinterpret_cast<const uint4*>(x + t * d);
  const bool in_regs = nch <= 64 * WPT * MAXC;
  uint4 buf[MAXC];
  float amax = 0.f;
  if (in_regs) {
    // the row's loads go out before the positions' (their latencies overlap)
#pragma unroll
    for (int q = 0; q < MAXC; ++q) {
      int c = tl + 64 * WPT * q;
      buf[q] = c < nch ? xr[c] : make_uint4(0, 0, 0, 0);
    }
  }
  int pj[kMaxTopK];
  if (PLANNED)
    plan_token(pa, T, k, t, lane, pj);
  else
    given_positions(pos, k, t, pj);
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < MAXC; ++q) amax = fmaxf(amax, absmax8(buf[q]));
  } else {
    for (int c = tl; c < nch; c += 64 * WPT) amax = fmaxf(amax, absmax8(xr[c]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (WPT > 1) {
    // (a max is exact in any order)
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WPT; ++w) amax = fmaxf(amax, wmax[wave - sub + w]);
  }
  // rows below 2^-100 (zero included) count as zero rows: 448/amax would overflow
  float inv, scale;
  fp8_row_scale(amax, &inv, &scale);
  if (TOKEN_ORDER) {
    uint2* dst = reinterpret_cast<uint2*>(xp + t * d);
    if (in_regs) {
#pragma unroll
      for (int q = 0; q < MAXC; ++q)
        if (tl + 64 * WPT * q < nch) dst[tl + 64 * WPT * q] = quant8(buf[q], inv);
    } else {
      for (int c = tl; c < nch; c += 64 * WPT) dst[c] = quant8(xr[c], inv);
    }
  } else if (in_regs) {
    // codes first, then slot by slot (scalar row base, fixed per-chunk offsets)
    uint2 code[MAXC];
#pragma unroll
    for (int q = 0; q < MAXC; ++q) code[q] = quant8(buf[q], inv);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (pj[j] < 0) continue;
      uint2* dst = reinterpret_cast<uint2*>(xp + static_cast<int64_t>(pj[j]) * d);
#pragma unroll
      for (int q = 0; q < MAXC; ++q)
        if (tl + 64 * WPT * q < nch) dst[tl + 64 * WPT * q] = code[q];
    }
  } else {
    for (int c = tl; c < nch; c += 64 * WPT) {
      uint2 code = quant8(xr[c], inv);
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (pj[j] >= 0) reinterpret_cast<uint2*>(xp + static_cast<int64_t>(pj[j]) * d)[c] = code;
    }
  }
  if (tl == 0) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (pj[j] >= 0) row_scale[pj[j]] = scale;
    if (PLANNED) plan_write(pa, k, t, pj);
  }
}

}  // namespace

hipError_t launch_dispatch_hist(const moe_shape& s, const int32_t* idx, int32_t* hist,
                                hipStream_t st) {
  dim3 grid(static_cast<unsigned>(ceil_div(s.T, TB)));
  hipLaunchKernelGGL(disp_hist_kernel, grid, dim3(256), 0, st, idx, s.T, s.k, s.N, hist);
  return hipGetLastError();
}

hipError_t launch_dispatch_plan(const moe_shape& s, const int32_t* idx, const int32_t* hist,
                                int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                                hipStream_t st) {
  dim3 grid(static_cast<unsigned>(ceil_div(s.T, TB)));
  hipLaunchKernelGGL(disp_plan_kernel, grid, dim3(256), 0, st, idx, s.T, s.k, s.N, s.capacity,
                     hist, offsets, pos, src, drop);
  return hipGetLastError();
}

namespace {
hipError_t launch_copy(const moe_shape& s, const void* x, const int32_t* pos, void* x_perm,
                       float* row_scale, const PlanArgs* pa, hipStream_t st) {
  const PlanArgs none{};
  if (s.buf_dtype == MOE_FP8_E4M3) {
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    uint8_t* xp = static_cast<uint8_t*>(x_perm);
    // four waves per token, one workgroup (a 7168-wide row: DeepSeek-V3 decode
    // 13.5 -> 8 us, prefill route + dispatch 114 -> 112 us, against one wave);
    // rows past 64 * 4 * 4 chunks of 8 are read twice
    const dim3 g1(static_cast<unsigned>(s.T));
    if (pa)
      hipLaunchKernelGGL((disp_fp8_kernel<4, true, 4>), g1, dim3(256), 0, st, xs, s.T, s.k, s.d, pos, xp,
                         row_scale, *pa);
    else
      hipLaunchKernelGGL((disp_fp8_kernel<4, false, 4>), g1, dim3(256), 0, st, xs, s.T, s.k, s.d, pos, xp,
                         row_scale, none);
  } else {
    const int es = s.dtype == MOE_BF16 ? 2 : 4;
    // waves per token: enough that a wave's chunk loop is one unrolled pass
    // (its loads in flight together), and with few tokens ~2048 waves in all
    // (DBRX shape: route + dispatch 304 -> 292 us)
    const int64_t iters = ceil_div(s.d * es / 16, 64);          // 16-byte chunks per lane, one wave a row
    int64_t wpt = std::max<int64_t>(ceil_div(2048, s.T), ceil_div(iters, kCopyAhead));
    if (wpt > iters) wpt = iters;
    const dim3 gw(static_cast<unsigned>(ceil_div(s.T * wpt, 4)));
    if (pa)
      hipLaunchKernelGGL(disp_copy_kernel<true>, gw, dim3(256), 0, st,
                         static_cast<const uint8_t*>(x), s.T, s.k, s.d * es, pos,
                         static_cast<uint8_t*>(x_perm), *pa, static_cast<int>(wpt));
    else
      hipLaunchKernelGGL(disp_copy_kernel<false>, gw, dim3(256), 0, st,
                         static_cast<const uint8_t*>(x), s.T, s.k, s.d * es, pos,
                         static_cast<uint8_t*>(x_perm), none, static_cast<int>(wpt));
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_dispatch_copy(const moe_shape& s, const void* x, const int32_t* pos,
                                void* x_perm, float* row_scale, hipStream_t st) {
  return launch_copy(s, x, pos, x_perm, row_scale, nullptr, st);
}

hipError_t launch_dispatch_copy_planned(const moe_shape& s, const void* x, const int32_t* idx,
                                        const int32_t* base, const int32_t* offsets,
                                        int32_t* pos, int32_t* src, uint8_t* drop, void* x_perm,
                                        float* row_scale, hipStream_t st) {
  const PlanArgs pa{idx, base, offsets, pos, src, drop, s.N, s.capacity, route_tile(s)};
  return launch_copy(s, x, pos, x_perm, row_scale, &pa, st);
}

hipError_t launch_dispatch_plan_fused(const moe_shape& s, const void* x, const int32_t* idx,
                                      const int32_t* base, const int32_t* offsets, int32_t* pos,
                                      int32_t* src, uint8_t* drop, void* x_tok, float* row_scale,
                                      hipStream_t st) {
  const PlanArgs pa{idx, base, offsets, pos, src, drop, s.N, s.capacity, route_tile(s)};
  if (s.buf_dtype == MOE_FP8_E4M3) {
    hipLaunchKernelGGL((disp_fp8_kernel<4, true, 4, true>), dim3(static_cast<unsigned>(s.T)), dim3(256),
                       0, st, static_cast<const uint16_t*>(x), s.T, s.k, s.d, pos,
                       static_cast<uint8_t*>(x_tok), row_scale, pa);
  } else {
    hipLaunchKernelGGL(disp_plan_tiles_kernel, dim3(static_cast<unsigned>(ceil_div(s.T, 4))), dim3(256),
                       0, st, s.T, s.k, pa);
  }
  return hipGetLastError();
}

}  // namespace moe
