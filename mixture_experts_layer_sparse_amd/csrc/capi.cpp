// C ABI: argument checks, workspace layout and kernel launches.  Every entry
// point validates on the host before touching the device, so the error
// conventions of include/moe.h hold without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <mutex>

#include "moe_internal.h"

namespace moe {

namespace {
constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
size_t elem_size(int dt) { return dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1); }
}  // namespace

// (a one-tile call keeps its T <= kRouteTile token scales in the smallest region)
static_assert(kRouteTile * 4 <= kAlign, "token scales fit any workspace region");

WsLayout ws_layout(const moe_shape& s) {
  WsLayout L{};
  const size_t T = static_cast<size_t>(s.T), N = static_cast<size_t>(s.N);
  const size_t nb_route = static_cast<size_t>(ceil_div(s.T, kRouteTileMin));
  const size_t nb_disp = static_cast<size_t>(ceil_div(s.T, kDispatchBlock));
  size_t off = 0;
  L.route_psum = off;
  off = align_up(off + nb_route * N * 4);
  L.route_hist = off;
  off = align_up(off + nb_route * N * 4);
  L.route_base = off;
  off = align_up(off + nb_route * N * 4);
  L.route_prod = off;
  off = align_up(off + N * 8 + 4);
  L.route_lpart = off;
  off = align_up(off + std::max(static_cast<size_t>(moe::route_split_ranges(s)) * T * N * 4,
                                moe::router_gemm_bytes(s)));
  L.disp_hist = off;
  off = align_up(off + nb_disp * N * 4);
  const bool fp8 = s.buf_dtype == MOE_FP8_E4M3;
  L.x_codes = off;
  if (fp8) off = align_up(off + T * static_cast<size_t>(s.d));
  L.rscale = off;
  if (fp8) off = align_up(off + T * static_cast<size_t>(s.k) * 4);
  L.gemm_split = off;
  off = align_up(off + moe::gemm_split_bytes(s));
  L.h = off;
  off = align_up(off + T * static_cast<size_t>(s.k) * static_cast<size_t>(s.F) * elem_size(s.dtype));
  L.h_shared = off;
  if (s.has_shared) off = align_up(off + T * static_cast<size_t>(s.F) * elem_size(s.dtype));
  L.sc_cnt = off;
  if (s.dtype == MOE_BF16) off = align_up(off + T * static_cast<size_t>(ceil_div(s.d, kScatterCols)) * 4);
  L.total = off;
  return L;
}

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace moe

using moe::WsLayout;

namespace {

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_ARG;
  if (s->T < 0 || s->d < 8 || s->d % 8 != 0 || s->N < 1 || s->N > moe::kMaxExperts || s->k < 1 ||
      s->k > s->N || s->F < 1)
    return MOE_ERR_ARG;
  if (s->k > moe::kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_ARG;
  if (s->buf_dtype != s->dtype && !(s->buf_dtype == MOE_FP8_E4M3 && s->dtype == MOE_BF16))
    return s->buf_dtype == MOE_FP8_E4M3 ? MOE_ERR_UNSUPPORTED : MOE_ERR_ARG;
  if (s->act < MOE_ACT_SILU || s->act > MOE_ACT_SWIGLU) return MOE_ERR_ARG;
  if (s->drop != MOE_DROP_PASSTHROUGH && s->drop != MOE_DROP_ZERO && s->drop != MOE_DROP_FALLBACK)
    return MOE_ERR_ARG;
  if (s->drop == MOE_DROP_FALLBACK && s->has_shared != 1) return MOE_ERR_ARG;
  if (s->n_groups > 1) {
    const int G = s->n_groups;
    if (G > 64 || s->N % G != 0) return MOE_ERR_ARG;
    if (s->topk_groups < 1 || s->topk_groups > G) return MOE_ERR_ARG;
    if (static_cast<int64_t>(s->topk_groups) * (s->N / G) < s->k) return MOE_ERR_ARG;
    if (s->group_score_k < 1 || s->group_score_k > s->N / G) return MOE_ERR_ARG;
    if (s->group_score_k > moe::kMaxTopK) return MOE_ERR_UNSUPPORTED;
  } else if (s->n_groups < 0) {
    return MOE_ERR_ARG;
  }
  if (s->has_shared != 0 && s->has_shared != 1) return MOE_ERR_ARG;
  if (s->gate != MOE_GATE_SPARSE && s->gate != MOE_GATE_FULL) return MOE_ERR_ARG;
  if (s->wfmt != MOE_W_DEFAULT && s->wfmt != MOE_W_MXFP4) return MOE_ERR_ARG;
  if (s->wfmt == MOE_W_MXFP4 && s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  // positions and row indices are int32
  if (s->T * static_cast<int64_t>(s->k) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (s->dtype == MOE_BF16 && (s->d % 64 != 0 || s->F % 64 != 0)) return MOE_ERR_UNSUPPORTED;
  // the grouped GEMMs read each expert matrix through a buffer resource with a
  // 32-bit byte range
  if (s->dtype == MOE_BF16 && static_cast<int64_t>(s->F) * s->d * 2 > static_cast<int64_t>(UINT32_MAX))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return moe::ws_layout(*s).total;
}

moe_status moe_check_shape(const moe_shape* s) { return check_shape(s); }

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or type combination";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch error";
    case MOE_ERR_TOO_LARGE: return "shape needs more scratch than the static buffer holds";
  }
  return "unknown status";
}

moe_status moe_route(const moe_shape* s, const void* x, const void* w_g, const float* bias,
                     int32_t* idx, float* w, int32_t* counts, int32_t* kept_counts, float* p,
                     float* f, float* l_aux, float* logits, void* ws, size_t ws_bytes,
                     void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!x || !w_g || !idx || !w || !counts || !kept_counts || !ws) return MOE_ERR_ARG;
  const WsLayout L = moe::ws_layout(*s);
  if (ws_bytes < L.disp_hist) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* psum = reinterpret_cast<float*>(base + L.route_psum);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.route_hist);
  float* lpart = reinterpret_cast<float*>(base + L.route_lpart);
  double* prod = reinterpret_cast<double*>(base + L.route_prod);
  const moe::RouteStats rs{counts, kept_counts, p, f, l_aux, nullptr, nullptr, prod,
                           reinterpret_cast<int32_t*>(prod + s->N)};
  hipError_t e = moe::launch_route(*s, x, w_g, bias, idx, w, logits, psum, hist, lpart, rs, st);
  if (e == hipSuccess && !moe::route_folds_stats(*s)) e = moe::launch_route_finalize(*s, psum, hist, rs, st);
  return hip_status(e);
}

moe_status moe_dispatch(const moe_shape* s, const void* x, const int32_t* idx, int32_t* offsets,
                        int32_t* pos, int32_t* src, uint8_t* drop, void* x_perm, float* row_scale,
                        void* ws, size_t ws_bytes, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!x || !idx || !offsets || !pos || !src || !drop || !x_perm || !ws) return MOE_ERR_ARG;
  if (s->buf_dtype == MOE_FP8_E4M3 && !row_scale) return MOE_ERR_ARG;
  const WsLayout L = moe::ws_layout(*s);
  if (ws_bytes < L.h) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* hist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.disp_hist);
  hipError_t e = moe::launch_dispatch_hist(*s, idx, hist, st);
  if (e == hipSuccess) e = moe::launch_dispatch_plan(*s, idx, hist, offsets, pos, src, drop, st);
  if (e == hipSuccess) e = moe::launch_dispatch_copy(*s, x, pos, x_perm, row_scale, st);
  return hip_status(e);
}

namespace {
// the split-K scratch inside a caller's workspace, or null (quarter-tile tail)
void* split_scratch(const moe_shape& s, void* ws, size_t ws_bytes, moe_status* err) {
  *err = MOE_OK;
  if (!ws || moe::gemm_split_bytes(s) == 0) return nullptr;
  const WsLayout L = moe::ws_layout(s);
  if (ws_bytes < L.gemm_split + moe::gemm_split_bytes(s)) {
    *err = MOE_ERR_WORKSPACE;
    return nullptr;
  }
  return static_cast<char*>(ws) + L.gemm_split;
}
}  // namespace

moe_status moe_expert_up(const moe_shape* s, const void* x_perm, const float* row_scale,
                         const int32_t* offsets, const void* w1, const void* w3, void* h,
                         void* ws, size_t ws_bytes, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!x_perm || !offsets || !w1 || !h) return MOE_ERR_ARG;
  if (s->act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_ARG;
  if (s->buf_dtype == MOE_FP8_E4M3 && !row_scale) return MOE_ERR_ARG;
  void* split = split_scratch(*s, ws, ws_bytes, &c);
  if (c != MOE_OK) return c;
  return hip_status(moe::launch_expert_up(*s, x_perm, row_scale, offsets, s->T * s->k, s->N, w1,
                                          w3, h, split, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_down(const moe_shape* s, const void* h, const int32_t* offsets,
                           const void* w2, void* out, void* ws, size_t ws_bytes, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!h || !offsets || !w2 || !out) return MOE_ERR_ARG;
  void* split = split_scratch(*s, ws, ws_bytes, &c);
  if (c != MOE_OK) return c;
  return hip_status(moe::launch_expert_down(*s, h, offsets, s->T * s->k, s->N, w2, out, split,
                                            static_cast<hipStream_t>(stream)));
}

moe_status moe_shared_expert(const moe_shape* s, const void* x, const void* ws1, const void* ws3,
                             const void* ws2, void* h_shared, void* out_shared, void* ws,
                             size_t ws_bytes, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!x || !ws1 || !ws2 || !h_shared || !out_shared) return MOE_ERR_ARG;
  if (s->act == MOE_ACT_SWIGLU && !ws3) return MOE_ERR_ARG;
  void* split = split_scratch(*s, ws, ws_bytes, &c);
  if (c != MOE_OK) return c;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the shared expert sees the unquantised input: same dtype as x
  moe_shape sd = *s;
  sd.buf_dtype = sd.dtype;
  hipError_t e = moe::launch_expert_up(sd, x, nullptr, nullptr, s->T, 1, ws1, ws3, h_shared,
                                       split, st);
  if (e == hipSuccess)
    e = moe::launch_expert_down(sd, h_shared, nullptr, s->T, 1, ws2, out_shared, split, st);
  return hip_status(e);
}

moe_status moe_shared_expert_up(const moe_shape* s, const void* x, const void* ws1, const void* ws3,
                                void* h_shared, void* ws, size_t ws_bytes, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!x || !ws1 || !h_shared) return MOE_ERR_ARG;
  if (s->act == MOE_ACT_SWIGLU && !ws3) return MOE_ERR_ARG;
  void* split = split_scratch(*s, ws, ws_bytes, &c);
  if (c != MOE_OK) return c;
  moe_shape sd = *s;
  sd.buf_dtype = sd.dtype;                     // the unquantised input
  return hip_status(moe::launch_expert_up(sd, x, nullptr, nullptr, s->T, 1, ws1, ws3, h_shared, split,
                                          static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_down_shared(const moe_shape* s, const void* h, const int32_t* offsets,
                                  const void* w2, void* out, const void* h_shared, const void* ws2,
                                  void* out_shared, void* ws, size_t ws_bytes, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!s->has_shared) return MOE_ERR_ARG;
  if (!h || !offsets || !w2 || !out || !h_shared || !ws2 || !out_shared) return MOE_ERR_ARG;
  void* split = split_scratch(*s, ws, ws_bytes, &c);
  if (c != MOE_OK) return c;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s->dtype != MOE_BF16) {
    // float32 layers: two launches
    hipError_t e = moe::launch_expert_down(*s, h, offsets, s->T * s->k, s->N, w2, out, split, st);
    if (e == hipSuccess) e = moe::launch_expert_down(*s, h_shared, nullptr, s->T, 1, ws2, out_shared, split, st);
    return hip_status(e);
  }
  return hip_status(moe::launch_expert_down(*s, h, offsets, s->T * s->k, s->N, w2, out, split, st, h_shared,
                                            ws2, out_shared, s->T));
}

moe_status moe_experts(const moe_shape* s, const void* x_perm, const float* row_scale,
                       const int32_t* offsets, const void* w1, const void* w3, const void* w2,
                       const void* x, const void* ws1, const void* ws3, const void* ws2,
                       void* out, void* out_shared, void* ws, size_t ws_bytes, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!ws || !out) return MOE_ERR_ARG;
  const WsLayout L = moe::ws_layout(*s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  moe_status r = moe_expert_up(s, x_perm, row_scale, offsets, w1, w3, base + L.h, ws, ws_bytes,
                               stream);
  if (r != MOE_OK) return r;
  if (!s->has_shared) return moe_expert_down(s, base + L.h, offsets, w2, out, ws, ws_bytes, stream);
  // the shared expert's up GEMM, then its down GEMM in the routed down launch
  r = moe_shared_expert_up(s, x, ws1, ws3, base + L.h_shared, ws, ws_bytes, stream);
  if (r != MOE_OK) return r;
  return moe_expert_down_shared(s, base + L.h, offsets, w2, out, base + L.h_shared, ws2, out_shared, ws,
                                ws_bytes, stream);
}

moe_status moe_combine(const moe_shape* s, const void* out, const void* out_shared, const void* x,
                       const int32_t* pos, const float* w, void* y, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!out || !x || !pos || !w || !y) return MOE_ERR_ARG;
  if (s->has_shared && !out_shared) return MOE_ERR_ARG;
  return hip_status(moe::launch_combine(*s, out, s->has_shared ? out_shared : nullptr, x, pos, w, y,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Argument checks of moe_route_dispatch (before the workspace), shared with
// its no-allocation variant.
moe_status route_dispatch_args(const moe_shape* s, const void* x, const void* w_g, int32_t* idx,
                               float* w, int32_t* counts, int32_t* kept_counts, int32_t* offsets,
                               int32_t* pos, int32_t* src, uint8_t* drop, void* x_perm,
                               float* row_scale) {
  if (!x || !w_g || !idx || !w || !counts || !kept_counts || !offsets || !pos || !src || !drop ||
      !x_perm)
    return MOE_ERR_ARG;
  if (s->buf_dtype == MOE_FP8_E4M3 && !row_scale) return MOE_ERR_ARG;
  return MOE_OK;
}

// Launches of moe_route_dispatch on a checked shape, with ws holding at least
// ws_layout(*s).disp_hist bytes.
moe_status route_dispatch_launch(const moe_shape* s, const void* x, const void* w_g,
                                 const float* bias, int32_t* idx, float* w, int32_t* counts,
                                 int32_t* kept_counts, float* p, float* f, float* l_aux,
                                 int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                                 void* x_perm, float* row_scale, void* ws, void* stream) {
  const WsLayout L = moe::ws_layout(*s);
  // the router's per-tile counts give every tile's base, so the row copy
  // places its token itself; the results equal moe_route then moe_dispatch
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* psum = reinterpret_cast<float*>(base + L.route_psum);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.route_hist);
  int32_t* tbase = reinterpret_cast<int32_t*>(base + L.route_base);
  float* lpart = reinterpret_cast<float*>(base + L.route_lpart);
  double* prod = reinterpret_cast<double*>(base + L.route_prod);
  const moe::RouteStats rs{counts, kept_counts, p, f, l_aux, offsets, tbase, prod,
                           reinterpret_cast<int32_t*>(prod + s->N)};
  hipError_t e = moe::launch_route(*s, x, w_g, bias, idx, w, nullptr, psum, hist, lpart, rs, st);
  if (e == hipSuccess && !moe::route_folds_stats(*s)) e = moe::launch_route_finalize(*s, psum, hist, rs, st);
  if (e == hipSuccess)
    e = moe::launch_dispatch_copy_planned(*s, x, idx, tbase, offsets, pos, src, drop, x_perm,
                                          row_scale, st);
  return hip_status(e);
}

// Scratch of moe_route_dispatch_noalloc: one array per GPU, held until the
// process ends.  Host code must not pass the array's name to a kernel (on the
// host it only stands in for the symbol); the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr int kMaxDevices = 64;
static_assert(MOE_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_route_dispatch(const moe_shape* s, const void* x, const void* w_g,
                              const float* bias, int32_t* idx, float* w, int32_t* counts,
                              int32_t* kept_counts, float* p, float* f, float* l_aux,
                              int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                              void* x_perm, float* row_scale, void* ws, size_t ws_bytes,
                              void* stream) {
  moe_status r = check_shape(s);
  if (r != MOE_OK) return r;
  if (s->T == 0) return MOE_OK;
  r = route_dispatch_args(s, x, w_g, idx, w, counts, kept_counts, offsets, pos, src, drop, x_perm,
                          row_scale);
  if (r != MOE_OK) return r;
  if (!ws) return MOE_ERR_ARG;
  if (ws_bytes < moe::ws_layout(*s).disp_hist) return MOE_ERR_WORKSPACE;
  return route_dispatch_launch(s, x, w_g, bias, idx, w, counts, kept_counts, p, f, l_aux, offsets,
                               pos, src, drop, x_perm, row_scale, ws, stream);
}

moe_status moe_route_dispatch_noalloc(const moe_shape* s, const void* x, const void* w_g,
                                      const float* bias, int32_t* idx, float* w, int32_t* counts,
                                      int32_t* kept_counts, float* p, float* f, float* l_aux,
                                      int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                                      void* x_perm, float* row_scale, void* stream) {
  moe_status r = check_shape(s);
  if (r != MOE_OK) return r;
  if (s->T == 0) return MOE_OK;
  r = route_dispatch_args(s, x, w_g, idx, w, counts, kept_counts, offsets, pos, src, drop, x_perm,
                          row_scale);
  if (r != MOE_OK) return r;
  if (moe::ws_layout(*s).disp_hist > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  void* ws = nullptr;
  r = static_scratch(&ws);
  if (r != MOE_OK) return r;
  // every scratch word the kernels read is written earlier in the same call
  // (per-tile partials, the split logits, the arrival counter zeroed by the
  // router kernel), so nothing is cleared here
  return route_dispatch_launch(s, x, w_g, bias, idx, w, counts, kept_counts, p, f, l_aux, offsets,
                               pos, src, drop, x_perm, row_scale, ws, stream);
}

moe_status moe_route_plan(const moe_shape* s, const void* x, const void* w_g, const float* bias,
                          int32_t* idx, float* w, int32_t* counts, int32_t* kept_counts, float* p,
                          float* f, float* l_aux, int32_t* offsets, int32_t* pos, int32_t* src,
                          uint8_t* drop, void* x_codes, float* row_scale, void* ws, size_t ws_bytes,
                          void* stream) {
  moe_status r = check_shape(s);
  if (r != MOE_OK) return r;
  if (s->T == 0) return MOE_OK;
  if (!x || !w_g || !idx || !w || !counts || !kept_counts || !offsets || !pos || !src || !drop || !ws)
    return MOE_ERR_ARG;
  const bool fp8 = s->buf_dtype == MOE_FP8_E4M3;
  if (fp8 && (!x_codes || !row_scale)) return MOE_ERR_ARG;
  const WsLayout L = moe::ws_layout(*s);
  if (ws_bytes < L.disp_hist) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* psum = reinterpret_cast<float*>(base + L.route_psum);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.route_hist);
  int32_t* tbase = reinterpret_cast<int32_t*>(base + L.route_base);
  float* lpart = reinterpret_cast<float*>(base + L.route_lpart);
  double* prod = reinterpret_cast<double*>(base + L.route_prod);
  const moe::RouteStats rs{counts, kept_counts, p, f, l_aux, offsets, tbase, prod,
                           reinterpret_cast<int32_t*>(prod + s->N)};
  // one router tile: the router writes the plan (and its logits kernel the
  // fp8 codes; the token scales go to the per-tile partial sums' region, which
  // a one-tile call does not use); with few tiles x experts the statistics
  // launch writes it (not for an fp8 buffer, whose quantising pass plans its
  // token itself)
  bool planned = moe::route_plans(*s);
  const moe::RoutePlanOut plan{pos, src, drop, fp8 ? static_cast<uint8_t*>(x_codes) : nullptr,
                               fp8 ? row_scale : nullptr, fp8 ? psum : nullptr};
  hipError_t e = moe::launch_route(*s, x, w_g, bias, idx, w, nullptr, psum, hist, lpart, rs, st,
                                   planned ? &plan : nullptr);
  if (e == hipSuccess && !moe::route_folds_stats(*s)) {
    if (fp8) e = moe::launch_route_finalize(*s, psum, hist, rs, st);
    else e = moe::launch_route_finalize(*s, psum, hist, rs, st, idx, pos, src, drop, &planned);
  }
  if (e == hipSuccess && !planned)
    e = moe::launch_dispatch_plan_fused(*s, x, idx, tbase, offsets, pos, src, drop, x_codes, row_scale, st);
  return hip_status(e);
}

namespace {
// The gathered up GEMM reads rows of a [T][d] operand through 32-bit offsets.
bool gather_fits(const moe_shape& s) {
  const int64_t es = s.buf_dtype == MOE_FP8_E4M3 ? 1 : (s.dtype == MOE_BF16 ? 2 : 4);
  return s.T * static_cast<int64_t>(s.d) * es <= static_cast<int64_t>(UINT32_MAX);
}
}  // namespace

moe_status moe_expert_up_gather(const moe_shape* s, const void* a, const float* row_scale,
                                const int32_t* offsets, const int32_t* src, const void* w1,
                                const void* w3, void* h, void* ws, size_t ws_bytes, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!a || !offsets || !src || !w1 || !h) return MOE_ERR_ARG;
  if (s->act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_ARG;
  if (s->buf_dtype == MOE_FP8_E4M3 && !row_scale) return MOE_ERR_ARG;
  if (!gather_fits(*s)) return MOE_ERR_UNSUPPORTED;
  void* split = split_scratch(*s, ws, ws_bytes, &c);
  if (c != MOE_OK) return c;
  return hip_status(moe::launch_expert_up(*s, a, row_scale, offsets, s->T * s->k, s->N, w1, w3, h,
                                          split, static_cast<hipStream_t>(stream), src, s->T));
}

moe_status moe_expert_up_gather_shared(const moe_shape* s, const void* a, const float* row_scale,
                                       const int32_t* offsets, const int32_t* src, const void* w1,
                                       const void* w3, void* h, const void* x, const void* ws1,
                                       const void* ws3, void* h_shared, void* ws, size_t ws_bytes,
                                       void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!s->has_shared) return MOE_ERR_ARG;
  if (!a || !offsets || !src || !w1 || !h || !x || !ws1 || !h_shared) return MOE_ERR_ARG;
  if (s->act == MOE_ACT_SWIGLU && (!w3 || !ws3)) return MOE_ERR_ARG;
  if (s->buf_dtype == MOE_FP8_E4M3 && !row_scale) return MOE_ERR_ARG;
  if (!gather_fits(*s)) return MOE_ERR_UNSUPPORTED;
  void* split = split_scratch(*s, ws, ws_bytes, &c);
  if (c != MOE_OK) return c;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (moe::gemv_fits(*s))
    return hip_status(moe::launch_expert_up(*s, a, row_scale, offsets, s->T * s->k, s->N, w1, w3, h, split,
                                            st, src, s->T, x, ws1, ws3, h_shared, s->T));
  hipError_t e = moe::launch_expert_up(*s, a, row_scale, offsets, s->T * s->k, s->N, w1, w3, h, split, st,
                                       src, s->T);
  if (e != hipSuccess) return hip_status(e);
  moe_shape sd = *s;
  sd.buf_dtype = sd.dtype;                     // the unquantised input
  return hip_status(moe::launch_expert_up(sd, x, nullptr, nullptr, s->T, 1, ws1, ws3, h_shared, split, st));
}

moe_status moe_expert_down_combine(const moe_shape* s, const void* h, const int32_t* offsets,
                                   const int32_t* src, const void* w2, void* out, const void* h_shared,
                                   const void* ws2, void* out_shared, const void* x, const int32_t* pos,
                                   const float* w, void* y, void* ws, size_t ws_bytes, void* stream) {
  moe_status c = check_shape(s);
  if (c != MOE_OK) return c;
  if (s->T == 0) return MOE_OK;
  if (!h || !offsets || !src || !w2 || !out || !x || !pos || !w || !y || !ws) return MOE_ERR_ARG;
  if (s->has_shared && (!h_shared || !ws2 || !out_shared)) return MOE_ERR_ARG;
  const WsLayout L = moe::ws_layout(*s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s->dtype != MOE_BF16 || moe::gemv_fits(*s)) {
    // float32 layers and decode-sized calls (the GEMV): the down GEMM, then the combine
    c = s->has_shared ? moe_expert_down_shared(s, h, offsets, w2, out, h_shared, ws2, out_shared, ws, ws_bytes,
                                               stream)
                      : moe_expert_down(s, h, offsets, w2, out, ws, ws_bytes, stream);
    if (c != MOE_OK) return c;
    return moe_combine(s, out, s->has_shared ? out_shared : nullptr, x, pos, w, y, stream);
  }
  int32_t* cnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.sc_cnt);
  hipError_t e = moe::launch_scatter_init(*s, pos, w, x, cnt, y, st);
  if (e != hipSuccess) return hip_status(e);
  const moe::ScatterArgs sc{src, pos, w, x, y, cnt};
  if (s->has_shared)
    return hip_status(moe::launch_expert_down(*s, h, offsets, s->T * s->k, s->N, w2, out, nullptr, st, h_shared,
                                              ws2, out_shared, s->T, &sc));
  return hip_status(moe::launch_expert_down(*s, h, offsets, s->T * s->k, s->N, w2, out, nullptr, st, nullptr,
                                            nullptr, nullptr, 0, &sc));
}

static moe_status forward_impl(const moe_shape* s, const void* x, const void* w_g, const float* bias,
                               const void* w1, const void* w3, const void* w2, const void* ws1,
                               const void* ws3, const void* ws2, int32_t* idx, float* w, int32_t* counts,
                               int32_t* kept_counts, float* p, float* f, float* l_aux, int32_t* offsets,
                               int32_t* pos, int32_t* src, uint8_t* drop, void* x_perm, float* row_scale,
                               void* out, void* out_shared, void* y, void* ws, size_t ws_bytes,
                               void* stream, bool scatter) {
  moe_status r = check_shape(s);
  if (r != MOE_OK) return r;
  if (s->T == 0) return MOE_OK;
  // every check of the three calls up front, so that nothing is launched on error
  if (!x || !w_g || !w1 || !w2 || !idx || !w || !counts || !kept_counts || !offsets || !pos ||
      !src || !drop || !out || !y || !ws)
    return MOE_ERR_ARG;
  const bool fused = x_perm == nullptr;
  if (s->act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_ARG;
  if (!fused && s->buf_dtype == MOE_FP8_E4M3 && !row_scale) return MOE_ERR_ARG;
  if (s->has_shared && (!ws1 || !ws2 || !out_shared || (s->act == MOE_ACT_SWIGLU && !ws3)))
    return MOE_ERR_ARG;
  if (fused && !gather_fits(*s)) return MOE_ERR_UNSUPPORTED;
  const WsLayout L = moe::ws_layout(*s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!fused) {
    r = moe_route_dispatch(s, x, w_g, bias, idx, w, counts, kept_counts, p, f, l_aux, offsets, pos,
                           src, drop, x_perm, row_scale, ws, ws_bytes, stream);
    if (r != MOE_OK) return r;
    r = moe_experts(s, x_perm, row_scale, offsets, w1, w3, w2, x, ws1, ws3, ws2, out, out_shared, ws,
                    ws_bytes, stream);
    if (r != MOE_OK) return r;
    return moe_combine(s, out, out_shared, x, pos, w, y, stream);
  }
  // fused dispatch: no expert-ordered copy of x; the up GEMM gathers its rows
  // through src from x (or from x's fp8 codes in token order)
  char* base = static_cast<char*>(ws);
  const bool fp8 = s->buf_dtype == MOE_FP8_E4M3;
  void* codes = fp8 ? base + L.x_codes : nullptr;
  float* rsc = fp8 ? (row_scale ? row_scale : reinterpret_cast<float*>(base + L.rscale)) : nullptr;
  r = moe_route_plan(s, x, w_g, bias, idx, w, counts, kept_counts, p, f, l_aux, offsets, pos, src, drop,
                     codes, rsc, ws, ws_bytes, stream);
  if (r != MOE_OK) return r;
  if (s->has_shared) {
    r = moe_expert_up_gather_shared(s, fp8 ? codes : x, rsc, offsets, src, w1, w3, base + L.h, x, ws1, ws3,
                                    base + L.h_shared, ws, ws_bytes, stream);
    if (r != MOE_OK) return r;
    if (scatter)
      return moe_expert_down_combine(s, base + L.h, offsets, src, w2, out, base + L.h_shared, ws2, out_shared, x,
                                     pos, w, y, ws, ws_bytes, stream);
    r = moe_expert_down_shared(s, base + L.h, offsets, w2, out, base + L.h_shared, ws2, out_shared, ws,
                               ws_bytes, stream);
  } else {
    r = moe_expert_up_gather(s, fp8 ? codes : x, rsc, offsets, src, w1, w3, base + L.h, ws, ws_bytes,
                             stream);
    if (r != MOE_OK) return r;
    if (scatter)
      return moe_expert_down_combine(s, base + L.h, offsets, src, w2, out, nullptr, nullptr, nullptr, x, pos, w,
                                     y, ws, ws_bytes, stream);
    r = moe_expert_down(s, base + L.h, offsets, w2, out, ws, ws_bytes, stream);
  }
  if (r != MOE_OK) return r;
  return moe_combine(s, out, out_shared, x, pos, w, y, stream);
}

moe_status moe_forward(const moe_shape* s, const void* x, const void* w_g, const float* bias,
                       const void* w1, const void* w3, const void* w2, const void* ws1,
                       const void* ws3, const void* ws2, int32_t* idx, float* w, int32_t* counts,
                       int32_t* kept_counts, float* p, float* f, float* l_aux, int32_t* offsets,
                       int32_t* pos, int32_t* src, uint8_t* drop, void* x_perm, float* row_scale,
                       void* out, void* out_shared, void* y, void* ws, size_t ws_bytes,
                       void* stream) {
  return forward_impl(s, x, w_g, bias, w1, w3, w2, ws1, ws3, ws2, idx, w, counts, kept_counts, p, f, l_aux,
                      offsets, pos, src, drop, x_perm, row_scale, out, out_shared, y, ws, ws_bytes, stream,
                      false);
}

moe_status moe_forward_scatter(const moe_shape* s, const void* x, const void* w_g, const float* bias,
                               const void* w1, const void* w3, const void* w2, const void* ws1,
                               const void* ws3, const void* ws2, int32_t* idx, float* w, int32_t* counts,
                               int32_t* kept_counts, float* p, float* f, float* l_aux, int32_t* offsets,
                               int32_t* pos, int32_t* src, uint8_t* drop, float* row_scale, void* out,
                               void* out_shared, void* y, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(s, x, w_g, bias, w1, w3, w2, ws1, ws3, ws2, idx, w, counts, kept_counts, p, f, l_aux,
                      offsets, pos, src, drop, nullptr, row_scale, out, out_shared, y, ws, ws_bytes, stream,
                      true);
}

}  // extern "C"
