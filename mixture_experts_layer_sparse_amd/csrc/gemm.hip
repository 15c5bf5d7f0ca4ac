// Grouped GEMMs of the expert FFNs ("moe communication costs" / "The core
// idea": each selected expert is a feed-forward network applied to its tokens;
// "Inference - why MoE is hard on hardware": small per-expert matrices).
//
//   up:   h[r][f] = act(sum_k A[r][k] W1[e][f][k], sum_k A[r][k] W3[e][f][k])
//   down: o[r][n] = sum_f h[r][f] W2[e][n][f]
// for every row r of expert e's segment [offsets[e], offsets[e+1]).  Both are
// "A times B-transposed" with K contiguous in both operands, which is the
// natural operand layout of the MFMA instructions.
//
// bf16 design (gfx950):
//   * one persistent workgroup per CU walks a device-side tile list: m-tiles of
//     every expert segment (counted from `offsets` on the device, so the host
//     never reads the routing) times n-tiles.  Consecutive tile ids share the
//     weight n-tile (GM m-tiles per n-tile) and each XCD owns contiguous runs
//     of tile ids, so the tiles running together on one XCD reuse the same
//     weight and activation tiles from that XCD's L2;
//   * 4 waves in a 2x2 grid, each computing a (BM/2)x(BN/2) block with
//     v_mfma_f32_32x32x16_bf16, float32 accumulation;
//   * K is streamed in 64-wide steps through two LDS stages (global -> registers
//     -> LDS, next step's loads in flight during this step's MFMAs); the 16-byte
//     chunks of each 128-byte LDS row are XOR-swizzled by the row index so that
//     fragment reads and tile writes are free of bank conflicts;
//   * fp8 activations (e4m3 codes) are widened to bf16 exactly on their way into
//     LDS and the per-row scale multiplies the float32 accumulator;
//   * SwiGLU: the B tile interleaves W1 and W3 rows of the same output columns
//     so that each wave holds both halves of its outputs; the activation runs
//     on the accumulators and h is written once, in bf16.
// The float32 path (small correctness shapes) is a plain dot-product kernel.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Epi { EPI_STORE = 0, EPI_SILU = 1, EPI_RELU = 2, EPI_SWIGLU = 3 };

struct GemmArgs {
  const void* a;           // [rows][K] bf16 bits, or e4m3 codes
  const float* a_scale;    // [rows] per-row scale (fp8 A) or null
  const int32_t* offsets;  // [n_seg + 1], or null: one dense segment of `rows`
  int64_t rows;
  int n_seg;
  int K;
  int n_out;               // output columns (F for up, d for down)
  const uint16_t* b0;      // [n_seg][n_out][K]  (W1 or W2)
  const uint16_t* b1;      // [n_seg][n_out][K]  (W3, SwiGLU only)
  int64_t b_stride;        // n_out * K
  uint16_t* out;           // [rows][n_out]
  int nt;                  // n-tiles
};

constexpr int GM = 4;      // m-tiles sharing one n-tile in the tile order

__device__ __forceinline__ int swz(int row) { return row & 7; }

__device__ __forceinline__ float silu(float u) { return u / (1.0f + __expf(-u)); }

__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 v) {
  // e4m3 -> float32 is exact, and every e4m3 value is a bf16 value, so the
  // upper half of the float32 bits is the exact bf16.
  uint32_t o[4];
  const uint32_t w[2] = {v.x, v.y};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[h]), false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[h]), true);
    o[2 * h] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
    o[2 * h + 1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int BM, int BN, int EPI, bool FP8A>
__global__ __launch_bounds__(256, 1) void gg_kernel(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TMI = WM / 32, TNI = WN / 32;
  constexpr int AR = BM / 32, BR = BN / 32;      // rows per thread per stage
  constexpr bool GATED = EPI == EPI_SWIGLU;
  static_assert(!GATED || (TNI % 2 == 0), "gated tile needs an even number of n-subtiles");

  __shared__ uint4 As[2][BM * 8];
  __shared__ uint4 Bs[2][BN * 8];
  __shared__ int mt_start[kMaxExperts + 2];
  __shared__ int seg_off[kMaxExperts + 2];
  __shared__ int scan_tmp[2][kMaxExperts + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_seg = g.offsets ? g.n_seg : 1;
  const int K = g.K, KT = K / BK;

  // m-tiles per segment and their exclusive scan (segments <= 256)
  {
    int ntile = 0, so = 0;
    if (tid < n_seg) {
      so = g.offsets ? g.offsets[tid] : 0;
      int eo = g.offsets ? g.offsets[tid + 1] : static_cast<int>(g.rows);
      ntile = (eo - so + BM - 1) / BM;
      seg_off[tid] = so;
      if (tid == n_seg - 1) seg_off[n_seg] = eo;
    }
    scan_tmp[0][tid] = ntile;
    __syncthreads();
    int cur = 0;
#pragma unroll
    for (int off = 1; off < 256; off <<= 1) {
      scan_tmp[cur ^ 1][tid] = scan_tmp[cur][tid] + (tid >= off ? scan_tmp[cur][tid - off] : 0);
      cur ^= 1;
      __syncthreads();
    }
    if (tid == 0) mt_start[0] = 0;
    if (tid < n_seg) mt_start[tid + 1] = scan_tmp[cur][tid];
    __syncthreads();
  }
  const int MT = mt_start[n_seg];
  const int NT = g.nt;
  const int total = MT * NT;

  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, S = gridDim.x >> 3;
  const int lc = tid & 7, lr = tid >> 3;         // load chunk / base row

  for (int round = 0;; ++round) {
    const int L = (round * 8 + xcd) * S + slot;
    if (L >= total) break;
    const int per_group = GM * NT;
    const int grp = L / per_group, rem = L - grp * per_group;
    const int m_base = grp * GM;
    const int gmn = min(GM, MT - m_base);
    const int mt = m_base + rem % gmn;
    const int ntile = rem / gmn;
    // expert of this m-tile: last e with mt_start[e] <= mt
    int lo = 0, hi = n_seg;                      // invariant: mt_start[lo] <= mt < mt_start[hi]
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (mt_start[mid] <= mt) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int row0 = seg_off[e] + (mt - mt_start[e]) * BM;
    const int row_end = seg_off[e + 1];

    // global row pointers for this thread's loads
    const uint8_t* a_base = static_cast<const uint8_t*>(g.a);
    const int64_t a_es = FP8A ? 1 : 2;
    const uint8_t* ap[AR];
#pragma unroll
    for (int i = 0; i < AR; ++i) {
      int r = row0 + lr + 32 * i;
      r = r < row_end ? r : row_end - 1;
      ap[i] = a_base + (static_cast<int64_t>(r) * K + lc * 8) * a_es;
    }
    const uint16_t* bp[BR];
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      const int n = lr + 32 * i;
      int f;
      const uint16_t* base;
      if (GATED) {
        const int wn_ = n / WN, q = n % WN, half = WN / 2;
        f = ntile * (BN / 2) + wn_ * half + (q % half);
        base = q < half ? g.b0 : g.b1;
      } else {
        f = ntile * BN + n;
        base = g.b0;
      }
      f = f < g.n_out ? f : g.n_out - 1;
      bp[i] = base + e * g.b_stride + static_cast<int64_t>(f) * K + lc * 8;
    }

    f32x16 acc[TMI][TNI];
#pragma unroll
    for (int i = 0; i < TMI; ++i)
#pragma unroll
      for (int j = 0; j < TNI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 ra[AR];
    uint2 ra8[AR];
    uint4 rb[BR];
    auto gload = [&](int kt) {
      const int64_t ko = static_cast<int64_t>(kt) * BK;
#pragma unroll
      for (int i = 0; i < AR; ++i) {
        if (FP8A) ra8[i] = *reinterpret_cast<const uint2*>(ap[i] + ko);
        else ra[i] = *reinterpret_cast<const uint4*>(ap[i] + ko * 2);
      }
#pragma unroll
      for (int i = 0; i < BR; ++i) rb[i] = *reinterpret_cast<const uint4*>(bp[i] + ko);
    };
    auto sstore = [&](int st) {
#pragma unroll
      for (int i = 0; i < AR; ++i) {
        const int r = lr + 32 * i;
        As[st][r * 8 + (lc ^ swz(r))] = FP8A ? fp8x8_to_bf16x8(ra8[i]) : ra[i];
      }
#pragma unroll
      for (int i = 0; i < BR; ++i) {
        const int r = lr + 32 * i;
        Bs[st][r * 8 + (lc ^ swz(r))] = rb[i];
      }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int st = kt & 1;
      if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int cc = kk * 2 + (lane >> 5);
        bf16x8 af[TMI], bfr[TNI];
#pragma unroll
        for (int i = 0; i < TMI; ++i) {
          const int r = wm * WM + i * 32 + (lane & 31);
          af[i] = *reinterpret_cast<const bf16x8*>(&As[st][r * 8 + (cc ^ swz(r))]);
        }
#pragma unroll
        for (int j = 0; j < TNI; ++j) {
          const int r = wn * WN + j * 32 + (lane & 31);
          bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[st][r * 8 + (cc ^ swz(r))]);
        }
#pragma unroll
        for (int i = 0; i < TMI; ++i)
#pragma unroll
          for (int j = 0; j < TNI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < KT) sstore(st ^ 1);
      __syncthreads();
    }

    // epilogue: acc[i][j][r] is row i*32 + 8*(r/4) + 4*(lane/32) + r%4, column j*32 + lane%32
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= row_end) continue;
        const float sc = FP8A ? g.a_scale[row] : 1.0f;
        uint16_t* orow = g.out + static_cast<int64_t>(row) * g.n_out;
        if (GATED) {
#pragma unroll
          for (int j = 0; j < TNI / 2; ++j) {
            const int col = ntile * (BN / 2) + wn * (WN / 2) + j * 32 + (lane & 31);
            if (col < g.n_out) {
              const float u = acc[i][j][r] * sc, gt = acc[i][j + TNI / 2][r] * sc;
              orow[col] = f32_to_bf16(silu(u) * gt);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < TNI; ++j) {
            const int col = ntile * BN + wn * WN + j * 32 + (lane & 31);
            if (col < g.n_out) {
              float v = acc[i][j][r] * sc;
              if (EPI == EPI_SILU) v = silu(v);
              if (EPI == EPI_RELU) v = fmaxf(v, 0.f);
              orow[col] = f32_to_bf16(v);
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------- float32 path --

__device__ __forceinline__ int seg_of(const int32_t* offsets, int n_seg, int r) {
  int lo = 0, hi = n_seg;                        // offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void f32_up_kernel(const float* __restrict__ a,
                                                     const int32_t* __restrict__ offsets,
                                                     int64_t rows, int n_seg, int K, int F,
                                                     const float* __restrict__ w1,
                                                     const float* __restrict__ w3,
                                                     float* __restrict__ h, int act) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t r = q / F;
  const int f = static_cast<int>(q % F);
  const int64_t R = offsets ? offsets[n_seg] : rows;
  if (r >= R) return;
  const int e = offsets ? seg_of(offsets, n_seg, static_cast<int>(r)) : 0;
  const float* ar = a + r * K;
  const float* u1 = w1 + (static_cast<int64_t>(e) * F + f) * K;
  float u = 0.f, gt = 0.f;
  for (int j = 0; j < K; ++j) u = fmaf(ar[j], u1[j], u);
  if (act == MOE_ACT_SWIGLU) {
    const float* u3 = w3 + (static_cast<int64_t>(e) * F + f) * K;
    for (int j = 0; j < K; ++j) gt = fmaf(ar[j], u3[j], gt);
  }
  float v;
  if (act == MOE_ACT_RELU) v = fmaxf(u, 0.f);
  else if (act == MOE_ACT_SILU) v = u / (1.0f + expf(-u));
  else v = u / (1.0f + expf(-u)) * gt;
  h[r * F + f] = v;
}

__global__ __launch_bounds__(256) void f32_down_kernel(const float* __restrict__ h,
                                                       const int32_t* __restrict__ offsets,
                                                       int64_t rows, int n_seg, int F, int d,
                                                       const float* __restrict__ w2,
                                                       float* __restrict__ o) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t r = q / d;
  const int n = static_cast<int>(q % d);
  const int64_t R = offsets ? offsets[n_seg] : rows;
  if (r >= R) return;
  const int e = offsets ? seg_of(offsets, n_seg, static_cast<int>(r)) : 0;
  const float* hr = h + r * F;
  const float* wr = w2 + (static_cast<int64_t>(e) * d + n) * F;
  float v = 0.f;
  for (int j = 0; j < F; ++j) v = fmaf(hr[j], wr[j], v);
  o[r * d + n] = v;
}

// ------------------------------------------------------------------- launch --

template <int BM, int BN, int EPI, bool FP8A>
hipError_t launch_gg_on(const GemmArgs& g, int tiles_upper, hipStream_t st) {
  int cus = device_cu_count();
  int grid = (cus / 8) * 8;
  int want = ((tiles_upper + 7) / 8) * 8;
  if (want < grid) grid = want;
  if (grid < 8) grid = 8;
  hipLaunchKernelGGL((gg_kernel<BM, BN, EPI, FP8A>), dim3(grid), dim3(256), 0, st, g);
  return hipGetLastError();
}

int pick_bm(int64_t rows, int n_seg) {
  const int64_t avg = n_seg > 0 ? rows / n_seg : rows;
  return avg >= 384 ? 256 : 128;
}

template <int EPI, bool FP8A>
hipError_t dispatch_up(int bm, const GemmArgs& g, int64_t rows, int n_seg, bool dense,
                       hipStream_t st) {
  const int nt = g.nt;
  if (bm == 256) {
    int mtu = static_cast<int>(ceil_div(rows, 256)) + (dense ? 0 : n_seg);
    return launch_gg_on<256, 256, EPI, FP8A>(g, mtu * nt, st);
  }
  int mtu = static_cast<int>(ceil_div(rows, 128)) + (dense ? 0 : n_seg);
  return launch_gg_on<128, 256, EPI, FP8A>(g, mtu * nt, st);
}

}  // namespace

hipError_t launch_expert_up(const moe_shape& s, const void* a, const float* row_scale,
                            const int32_t* offsets, int64_t rows, int n_seg, const void* w1,
                            const void* w3, void* h, hipStream_t st) {
  if (s.dtype == MOE_F32) {
    int64_t n = rows * s.F;
    dim3 grid(static_cast<unsigned>(ceil_div(n, 256)));
    hipLaunchKernelGGL(f32_up_kernel, grid, dim3(256), 0, st, static_cast<const float*>(a),
                       offsets, rows, n_seg, s.d, s.F, static_cast<const float*>(w1),
                       static_cast<const float*>(w3), static_cast<float*>(h), s.act);
    return hipGetLastError();
  }
  const bool fp8 = s.buf_dtype == MOE_FP8_E4M3 && row_scale != nullptr;
  const bool dense = offsets == nullptr;
  GemmArgs g{};
  g.a = a;
  g.a_scale = fp8 ? row_scale : nullptr;
  g.offsets = offsets;
  g.rows = rows;
  g.n_seg = n_seg;
  g.K = s.d;
  g.n_out = s.F;
  g.b0 = static_cast<const uint16_t*>(w1);
  g.b1 = static_cast<const uint16_t*>(w3);
  g.b_stride = static_cast<int64_t>(s.F) * s.d;
  g.out = static_cast<uint16_t*>(h);
  const bool gated = s.act == MOE_ACT_SWIGLU;
  g.nt = static_cast<int>(gated ? ceil_div(s.F, 128) : ceil_div(s.F, 256));
  const int bm = pick_bm(rows, dense ? 1 : n_seg);
  if (gated) return fp8 ? dispatch_up<EPI_SWIGLU, true>(bm, g, rows, n_seg, dense, st)
                        : dispatch_up<EPI_SWIGLU, false>(bm, g, rows, n_seg, dense, st);
  if (s.act == MOE_ACT_RELU) return fp8 ? dispatch_up<EPI_RELU, true>(bm, g, rows, n_seg, dense, st)
                                        : dispatch_up<EPI_RELU, false>(bm, g, rows, n_seg, dense, st);
  return fp8 ? dispatch_up<EPI_SILU, true>(bm, g, rows, n_seg, dense, st)
             : dispatch_up<EPI_SILU, false>(bm, g, rows, n_seg, dense, st);
}

hipError_t launch_expert_down(const moe_shape& s, const void* h, const int32_t* offsets,
                              int64_t rows, int n_seg, const void* w2, void* out,
                              hipStream_t st) {
  if (s.dtype == MOE_F32) {
    int64_t n = rows * s.d;
    dim3 grid(static_cast<unsigned>(ceil_div(n, 256)));
    hipLaunchKernelGGL(f32_down_kernel, grid, dim3(256), 0, st, static_cast<const float*>(h),
                       offsets, rows, n_seg, s.F, s.d, static_cast<const float*>(w2),
                       static_cast<float*>(out));
    return hipGetLastError();
  }
  const bool dense = offsets == nullptr;
  GemmArgs g{};
  g.a = h;
  g.a_scale = nullptr;
  g.offsets = offsets;
  g.rows = rows;
  g.n_seg = n_seg;
  g.K = s.F;
  g.n_out = s.d;
  g.b0 = static_cast<const uint16_t*>(w2);
  g.b1 = nullptr;
  g.b_stride = static_cast<int64_t>(s.d) * s.F;
  g.out = static_cast<uint16_t*>(out);
  g.nt = static_cast<int>(ceil_div(s.d, 256));
  const int bm = pick_bm(rows, dense ? 1 : n_seg);
  return dispatch_up<EPI_STORE, false>(bm, g, rows, n_seg, dense, st);
}

}  // namespace moe
