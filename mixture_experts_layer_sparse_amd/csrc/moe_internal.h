// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;
constexpr int kRouteTile = 16;     // tokens per router workgroup (at most; route_tile)
constexpr int kRouteTileMin = 8;   // the smaller router tile
constexpr int kDispatchBlock = 256;  // tokens per dispatch-plan block
constexpr int kSplitKMax = 16;       // K ranges per tile when a grouped GEMM has few tiles
constexpr size_t kSplitMetaBytes = 4096;  // header of the split-K scratch (tile count, tile rows)
// Router logits through the grouped GEMM: split-K partial tiles of this many
// token rows and expert columns, stored tile after tile in range-major order.
constexpr int kRouterTileRows = 128;
constexpr int kRouterTileCols = 256;

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// The combine's arithmetic on 8 bf16 values (the combine kernel and the
// combining epilogue of the down GEMM use these, so that both give the same
// bits): acc += w * v with one fused multiply-add per element, acc += v, and
// the float32 -> bf16 rounding of the sums.
__device__ __forceinline__ void combine_fma8(float* acc, uint4 v, float w) {
  const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, __uint_as_float(q[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, __uint_as_float(q[i] & 0xFFFF0000u), acc[2 * i + 1]);
  }
}
__device__ __forceinline__ void combine_add8(float* acc, uint4 v) {
  const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += __uint_as_float(q[i] << 16);
    acc[2 * i + 1] += __uint_as_float(q[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ uint4 combine_pack8(const float* acc) {
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = f32_to_bf16(acc[2 * i]) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// Columns of y per arrival counter of the combining down GEMM.
constexpr int kScatterCols = 128;

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) {
  return (a + b - 1) / b;
}

// Bytes of one MXFP4 matrix [rows][K]: the codes (two per byte), then one E8M0
// scale per 32 elements of a row.
constexpr inline size_t mxfp4_bytes(int64_t rows, int64_t K) {
  return static_cast<size_t>(rows * K / 2 + rows * K / 32);
}

// Workspace carving: offsets (bytes) of each region for one shape.
struct WsLayout {
  size_t route_psum;    // float   [nb_route][N]
  size_t route_hist;    // int32   [nb_route][N]
  size_t route_base;    // int32   [nb_route][N]
  size_t route_prod;    // double  [N], then the statistics kernel's arrival counter
  size_t route_lpart;   // partial logits: float [route_split_ranges(s)][T][N] (few tokens), or
                        // router_gemm_bytes(s) of split-K scratch (wide routers)
  size_t disp_hist;     // int32   [nb_disp][N]
  size_t x_codes;       // fp8 codes of x in token order [T][d] (fused layer with an fp8 buffer)
  size_t rscale;        // float   [T*k] row scales (fused layer with an fp8 buffer)
  size_t gemm_split;    // split-K tail scratch of the grouped GEMMs (gemm_split_bytes(s))
  size_t h;             // dtype   [T*k][F]
  size_t h_shared;      // dtype   [T][F]
  size_t sc_cnt;        // int32   [T][ceil(d / kScatterCols)] arrival counters (bf16 layers)
  size_t total;
};
WsLayout ws_layout(const moe_shape& s);

// ---------------------------------------------------------------- launchers --
// Each returns hipSuccess or the launch error; shapes are already validated.

// With few tokens (route_split_ranges(s) > 0) the logits are first computed as
// partial sums over that many d-ranges into lpart by a separate kernel spread
// over the experts, so that the router weights are read about once instead of
// once per 16-token tile; the router then adds the partials in range order
// (one range: whole dot products, for calls of one router tile).
int route_split_ranges(const moe_shape& s);
// The load statistics over all router tiles.  p, f, l_aux may be null;
// offsets (may be null): exclusive scan of the kept counts, N + 1 entries;
// base (may be null): [nb_route][N] assignments to each expert in earlier
// tiles; prod: [N] doubles of scratch (each expert's f p, for L_aux); done: a
// counter in the workspace that the router kernel zeroes.
struct RouteStats {
  int32_t* counts;
  int32_t* kept;
  float* p;
  float* f;
  float* l_aux;
  int32_t* offsets;
  int32_t* base;
  double* prod;
  int32_t* done;
};
// Tokens per router tile (workgroup) for this shape: 8 or 16 (every
// per-tile count and base, and the dispatch copy's ranks, use it).
int route_tile(const moe_shape& s);
// With one router tile (T <= kRouteTile) the router kernel writes the
// statistics itself; otherwise launch_route_finalize must follow launch_route.
bool route_folds_stats(const moe_shape& s);
// The fused layer's plan, written by the router itself for a call of one
// router tile with bf16 x (route_plans(s)): pos, src and drop as
// launch_dispatch_plan_fused writes them, and with an fp8 buffer (x_codes
// non-null) the codes of x in token order, the kept slots' row scales and the
// token scales (tscale: T floats of scratch; with one tile the per-tile partial
// sums' region is free, and every region holds at least 64 floats).  Such a
// call takes its logits
// from whole dot products, one workgroup per expert (two kernels in all).
struct RoutePlanOut {
  int32_t* pos;
  int32_t* src;
  uint8_t* drop;
  uint8_t* x_codes;
  float* row_scale;
  float* tscale;
};
bool route_plans(const moe_shape& s);
// plan (route_plans(s) and rs.offsets required, else hipErrorInvalidValue): see RoutePlanOut.
hipError_t launch_route(const moe_shape& s, const void* x, const void* wg, const float* bias,
                        int32_t* idx, float* w, float* logits, float* psum, int32_t* hist,
                        float* lpart, const RouteStats& rs, hipStream_t st,
                        const RoutePlanOut* plan = nullptr);
// With idx, pos, src and drop given, the statistics launch may also write
// the plan of the fused layer (launch_dispatch_plan_fused's pos, src and
// drop); *planned (may be null) says whether it did.
hipError_t launch_route_finalize(const moe_shape& s, const float* psum, const int32_t* hist,
                                 const RouteStats& rs, hipStream_t st, const int32_t* idx = nullptr,
                                 int32_t* pos = nullptr, int32_t* src = nullptr,
                                 uint8_t* drop = nullptr, bool* planned = nullptr);

hipError_t launch_dispatch_hist(const moe_shape& s, const int32_t* idx, int32_t* hist,
                                hipStream_t st);
hipError_t launch_dispatch_plan(const moe_shape& s, const int32_t* idx, const int32_t* hist,
                                int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                                hipStream_t st);
hipError_t launch_dispatch_copy(const moe_shape& s, const void* x, const int32_t* pos,
                                void* x_perm, float* row_scale, hipStream_t st);
// The copy with the plan folded in: positions from the router's per-tile
// counts (base, offsets from launch_route_finalize); writes pos, src, drop too.
hipError_t launch_dispatch_copy_planned(const moe_shape& s, const void* x, const int32_t* idx,
                                        const int32_t* base, const int32_t* offsets,
                                        int32_t* pos, int32_t* src, uint8_t* drop, void* x_perm,
                                        float* row_scale, hipStream_t st);

// The fused layer's plan: pos, src and drop as launch_dispatch_copy_planned
// writes them, without copying rows (the up GEMM gathers x through src).  For
// an fp8 buffer, each token's codes go once to row t of x_tok ([T][d]) and
// its scale to row_scale at each kept slot's position.
hipError_t launch_dispatch_plan_fused(const moe_shape& s, const void* x, const int32_t* idx,
                                      const int32_t* base, const int32_t* offsets, int32_t* pos,
                                      int32_t* src, uint8_t* drop, void* x_tok, float* row_scale,
                                      hipStream_t st);

// Grouped GEMMs.  `offsets` == nullptr means one dense segment of `rows` rows.
// `gather` (may be null): row r of the product reads row gather[r] of `a`,
// which then has `a_rows` rows (a_rows * d * element size < 4 GiB).
// `split` (may be null): gemm_split_bytes(s) of scratch for a split-K tail;
// without it a mostly idle last round runs as quarter tiles.
// Calls of at most four tokens with bf16 weights (gemv_fits) stream each
// weight row once with no tiles (the decode GEMV); there the up launch also
// takes an extra dense segment (x_rows > 0, with offsets): xout [x_rows][F]
// from xa [x_rows][d] (bf16) and xw1, xw3 (the shared expert's up GEMM);
// elsewhere x_rows must be 0.
bool gemv_fits(const moe_shape& s);
hipError_t launch_expert_up(const moe_shape& s, const void* a, const float* row_scale,
                            const int32_t* offsets, int64_t rows, int n_seg,
                            const void* w1, const void* w3, void* h, void* split, hipStream_t st,
                            const int32_t* gather = nullptr, int64_t a_rows = 0,
                            const void* xa = nullptr, const void* xw1 = nullptr,
                            const void* xw3 = nullptr, void* xout = nullptr, int64_t x_rows = 0);
// With x_rows > 0 (and offsets), the same launch also computes an extra dense
// segment after the routed ones: xout [x_rows][d] = xa [x_rows][F] times the one
// matrix xw2 (laid out as one of w2's), the shared expert's down GEMM.
//
// With `sc` (bf16 layers, no split-K scratch), the down GEMM also combines:
// cnt[t][c] starts at minus the number of rows of token t in the launch (its
// kept slots, plus its shared-expert row), every tile adds one per row for
// each kScatterCols-column group it covers after publishing its output rows,
// and the tile that brings a counter to zero writes those columns of y[t]
// from the token's rows as the combine kernel does (launch_scatter_init sets
// the counters and writes y of the tokens no row reaches).
struct ScatterArgs {
  const int32_t* src;   // [rows] token of each routed output row
  const int32_t* pos;   // [T][k]
  const float* w;       // [T][k]
  const void* x;        // [T][d] (dropped slots passed through)
  void* y;              // [T][d]
  int32_t* cnt;         // [T][ceil(d / kScatterCols)]
};
hipError_t launch_expert_down(const moe_shape& s, const void* h, const int32_t* offsets,
                              int64_t rows, int n_seg, const void* w2, void* out, void* split,
                              hipStream_t st, const void* xa = nullptr, const void* xw2 = nullptr,
                              void* xout = nullptr, int64_t x_rows = 0, const ScatterArgs* sc = nullptr);
hipError_t launch_scatter_init(const moe_shape& s, const int32_t* pos, const float* w, const void* x,
                               int32_t* cnt, void* y, hipStream_t st);
size_t gemm_split_bytes(const moe_shape& s);

// Wide routers (bf16, at least 64 experts, N d >= 2^19, 512 to 16384 tokens): the logits as
// one dense split-K GEMM of x [T][d] with W_g [N][d], so that each 128-token
// tile reads W_g once (instead of every 16-token router tile reading all of
// it).  The float32 partials stay in `scratch` (router_gemm_bytes(s)): a
// header whose words 0 and 1 hold the tile count and the K-range count,
// followed at kSplitMetaBytes by the partial tiles; the router adds the ranges
// in order.
bool router_gemm(const moe_shape& s);
size_t router_gemm_bytes(const moe_shape& s);
hipError_t launch_router_logits(const moe_shape& s, const void* x, const void* wg, void* scratch,
                                hipStream_t st);

hipError_t launch_combine(const moe_shape& s, const void* out, const void* out_shared,
                          const void* x, const int32_t* pos, const float* w, void* y,
                          hipStream_t st);

int device_cu_count();

}  // namespace moe
