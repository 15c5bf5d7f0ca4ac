/*
 * moe.h — C ABI of the sparse Mixture-of-Experts layer forward for AMD MI355X (gfx950).
 *
 * The layer, for T tokens x[t] of width d, N routed experts and k experts per token:
 *   route     l[t][e] = W_g[e] . x[t] (+ b[e]); optional group limit; the k largest
 *             logits (ties to the lower expert index); weights = softmax over only
 *             those k logits; load statistics f, p and L_aux.
 *   dispatch  permute the (token, slot) assignments into expert-contiguous order
 *             (histogram, prefix scan, stable rank, capacity drop, row copy or
 *             fp8 quantise).
 *   experts   per expert segment: h = act(W1 x, W3 x), o = W2 h (grouped GEMMs).
 *   combine   y[t] = sum_j w[t][j] * (o of slot j, or x[t] / 0 when dropped)
 *             (+ the shared expert's output).
 *
 * Sources (web pages, cited by title and section):
 *   "Advanced GPU Optimization: How to tech an LLM with CUDA and ROCm? - Part 5":
 *       "The Math"; "1.1 The Router Kernel (Top-k Gating)"; "1.2 Expert Parallelism
 *       with All-to-All Communication".
 *   "MoE: what it costs to train and serve": "Expert parallelism and two
 *       all-to-alls"; "Worked example: how many bytes does one token send?";
 *       "Limit how many machines a token touches"; "Numerical precision".
 *   "moe communication costs": "Router design"; "Load balancing - the critical
 *       auxiliary loss"; "Capacity factor and token dropping".
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed, owned by
 *     the caller.  The library never allocates, frees, or keeps state between
 *     calls.  Scratch memory comes from the caller through `ws`/`ws_bytes`
 *     (size from moe_workspace_bytes); its contents need no initialisation and
 *     carry nothing from one call to the next.  Calls that may run at the same
 *     time (on different streams) must use different workspaces: a call's
 *     kernels communicate through it (partial sums, counters, split-K tiles).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues kernels on it: no host synchronisation, no device-to-host read.
 *     Outputs are valid once the stream has reached that point.
 *   - Element types: `dtype` is the storage of x, W_g, the expert weights, the
 *     intermediate h, the expert outputs and y: MOE_F32 or MOE_BF16 (bit patterns
 *     of bfloat16).  Router logits, weights and statistics are always float32;
 *     all products accumulate in float32.
 *   - Errors are returned as moe_status; nothing is thrown.  Argument checks run
 *     on the host before any launch: MOE_ERR_ARG for invalid sizes or NULL
 *     required pointers, MOE_ERR_UNSUPPORTED for valid but unimplemented
 *     combinations, MOE_ERR_WORKSPACE when ws_bytes is too small, MOE_ERR_HIP
 *     when a launch fails.  T == 0 is a no-op returning MOE_OK.
 *   - Inputs must be finite; NaN/Inf inputs give undefined (but memory-safe)
 *     results.
 *   - Results are deterministic: repeated calls with the same inputs give
 *     bit-identical outputs (no floating-point atomics; fixed reduction orders).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4,
  MOE_ERR_TOO_LARGE = 5   /* moe_route_dispatch_noalloc: the shape's scratch exceeds
                             MOE_STATIC_SCRATCH_BYTES */
} moe_status;

/* Size of the library's static device scratch (one per GPU, held until the
 * process ends), used only by moe_route_dispatch_noalloc. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)48 << 20)

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;
typedef enum { MOE_ACT_SILU = 0, MOE_ACT_RELU = 1, MOE_ACT_SWIGLU = 2 } moe_act;
/* What a slot dropped by the capacity contributes ("moe communication costs" /
 * "Capacity factor and token dropping": overflow tokens either skip the layer
 * through the residual or go to a shared fallback expert).  PASSTHROUGH: w * x[t];
 * ZERO: nothing; FALLBACK: w * S(x[t]), S the shared expert (has_shared must be 1;
 * its always-on term is still added once). */
typedef enum { MOE_DROP_PASSTHROUGH = 0, MOE_DROP_ZERO = 1, MOE_DROP_FALLBACK = 2 } moe_drop;
/* Weights of the selected experts.  SPARSE: a softmax over the k selected logits
 * ("Part 5" / "The Math" and "1.1 The Router Kernel"); each token's weights sum
 * to 1.  FULL: the probability each selected expert has under the softmax over
 * all N logits, not renormalised ("moe communication costs" / "Router design":
 * y = sum over the top-k of G(x)_i E_i(x) with G(x) = softmax(W_g x); Switch's
 * single expert is weighted by its router probability); a token's weights sum
 * to at most 1. */
typedef enum { MOE_GATE_SPARSE = 0, MOE_GATE_FULL = 1 } moe_gate;
/* Storage of the expert weights (W1, W3, W2 and the shared expert's; the router
 * W_g keeps dtype).  DEFAULT: dtype.  MXFP4 ("MoE: what it costs to train and
 * serve" / "Memory: sparsity only helps once it fits": gpt-oss experts at about
 * 4.25 bits per weight), read as the OCP microscaling format: each matrix
 * [rows][K] (K the dimension the product sums over: d for W1/W3, F for W2) is
 * rows*K/2 bytes of FP4 E2M1 codes, row-major, element 2i in the low nibble of
 * byte i, followed by rows*K/32 E8M0 scales (2^(e-127); one per 32 elements of
 * a row, row-major); a weight is its code's value (0, 0.5, 1, 1.5, 2, 3, 4, 6,
 * signed) times its block's scale.  Stacked expert tensors hold N such
 * matrices back to back.  Needs dtype bf16; the weights are widened exactly
 * to bf16 inside the GEMMs (scale 255, NaN, is not supported, and scales
 * above 2^125 can overflow bf16). */
typedef enum { MOE_W_DEFAULT = 0, MOE_W_MXFP4 = 1 } moe_wfmt;

/* Shape and options of one layer.  Enumerations are stored as int32_t so that
 * the struct layout is fixed: 8 + 16 * 4 = 72 bytes, alpha at offset 60, gate
 * at offset 64, wfmt at offset 68. */
typedef struct moe_shape {
  int64_t T;             /* tokens, >= 0 */
  int32_t d;             /* hidden size */
  int32_t N;             /* routed experts, 1..256 */
  int32_t k;             /* experts per token, 1..min(N, 8) ("1.1 The Router Kernel": top-2;
                            "moe communication costs" table: k from 1 to 6) */
  int32_t F;             /* expert FFN width */
  int32_t capacity;      /* max kept assignments per expert; <= 0: unlimited
                            ("Capacity factor and token dropping": C = factor * T / N,
                            rounded by the caller) */
  int32_t n_groups;      /* 0 or 1: no group limit; else G contiguous groups of N/G
                            experts ("Limit how many machines a token touches") */
  int32_t topk_groups;   /* groups kept per token (G > 1) */
  int32_t group_score_k; /* a group's score is the sum of its group_score_k largest
                            logits, 1..8 */
  int32_t has_shared;    /* 1: one always-on shared expert (weight 1, unquantised x) */
  int32_t dtype;         /* moe_dtype: MOE_F32 or MOE_BF16 */
  int32_t buf_dtype;     /* dispatch buffer: == dtype, or MOE_FP8_E4M3 when dtype is bf16 */
  int32_t act;           /* moe_act */
  int32_t drop;          /* moe_drop: what a dropped slot contributes */
  float alpha;           /* L_aux coefficient ("Load balancing": typically 0.01-0.1) */
  int32_t gate;          /* moe_gate: how the selected experts are weighted */
  int32_t wfmt;          /* moe_wfmt: storage of the expert weights */
} moe_shape;

/* Bytes of device scratch needed by moe_route, moe_dispatch and moe_experts for
 * this shape (one buffer serves all of them; 256-byte aligned).  The largest
 * part is the expert intermediate h: T*k rows of F elements (+ T rows for the
 * shared expert).  Returns 0 for an invalid shape. */
size_t moe_workspace_bytes(const moe_shape* s);

/* Checks a shape; MOE_OK when every call supports it.  MOE_ERR_ARG for sizes
 * or fields out of their ranges (see moe_shape); MOE_ERR_UNSUPPORTED for valid
 * combinations this build does not run: k or group_score_k above 8, an fp8
 * dispatch buffer with float32 storage, T*k above INT32_MAX, and for bfloat16
 * d or F not a multiple of 64 or one expert matrix (F*d*2 bytes) above 4 GiB. */
moe_status moe_check_shape(const moe_shape* s);

/* Router.  "moe communication costs" / "Router design" (logits W_g x, no noise at
 * inference); "Part 5" / "1.1 The Router Kernel" (top-k scan with strict >, so
 * ties go to the lower index; softmax over only the selected logits, max
 * subtracted); "Load balancing" (f_i, p_i, L_aux = alpha N sum f_i p_i).
 *   x       [T][d] dtype          W_g [N][d] dtype (stored like x)
 *   bias    [N] float32 or NULL   added to the logits before every use
 *   idx     [T][k] int32 out      expert ids, slot 0 = largest logit
 *   w       [T][k] float32 out    gate weights: sparse softmax over the selection
 *                                 (each row sums to 1), or with gate = MOE_GATE_FULL
 *                                 each selected expert's full-softmax probability
 *   counts  [N] int32 out         assignments per expert before capacity drops
 *   kept_counts [N] int32 out     min(counts, capacity) (= counts if unlimited)
 *   p, f    [N] float32 out or NULL   mean full-softmax probability; counts/(T k)
 *   l_aux   [1] float32 out or NULL   alpha * N * sum(f * p)
 *   logits  [T][N] float32 out or NULL (debug: the biased logits)
 */
moe_status moe_route(const moe_shape* s, const void* x, const void* w_g, const float* bias,
                     int32_t* idx, float* w, int32_t* counts, int32_t* kept_counts,
                     float* p, float* f, float* l_aux, float* logits,
                     void* ws, size_t ws_bytes, void* stream);

/* Dispatch: the single-GPU form of the dispatch all-to-all ("Part 5" / "1.2
 * Expert Parallelism", step 1; "MoE: what it costs to train and serve" / "Expert
 * parallelism and two all-to-alls").  Assignment a = t*k + j goes to expert
 * e = idx[t][j]; its rank is the number of earlier assignments (smaller a) to e;
 * it is kept when capacity <= 0 or rank < capacity.
 *   idx       [T][k] int32 in (each row holds k distinct ids in [0, N))
 *   offsets   [N+1] int32 out   exclusive scan of the kept counts; R = offsets[N]
 *   pos       [T][k] int32 out  offsets[e] + rank, or -1 when dropped
 *   src       [T*k] int32 out   src[pos] = t for the R kept rows (rest untouched)
 *   drop      [T][k] uint8 out  1 when dropped
 *   x_perm    [T*k][d] out      row pos = x[t] (dtype), or fp8 e4m3 codes when
 *                               buf_dtype is FP8 ("Worked example: how many bytes
 *                               does one token send?": FP8 before dispatch);
 *                               rows >= R untouched.  Bytes written = R*d*s.
 *   row_scale [T*k] float32 out (FP8 only, else may be NULL): per-row scale;
 *             value = code * scale.  Per token: amax = max|x|, inv = 448/amax,
 *             code = e4m3(x*inv) rounded to nearest even, scale = amax/448
 *             (float32 IEEE arithmetic; amax < 2^-100, zero included, gives
 *             inv = scale = 1).
 */
moe_status moe_dispatch(const moe_shape* s, const void* x, const int32_t* idx,
                        int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                        void* x_perm, float* row_scale,
                        void* ws, size_t ws_bytes, void* stream);

/* Expert up-projection over the expert segments of x_perm (grouped GEMM 1 with
 * the activation fused): for row r of expert e, h[r] = act(W1[e] x_r, W3[e] x_r)
 * with x_r the (dequantised) dispatch row.  act: SiLU, ReLU, or SwiGLU
 * silu(W1 x) * (W3 x).  "moe communication costs" / "The core idea" (expert FFNs).
 *   x_perm [T*k][d] buf_dtype, row_scale [T*k] (FP8 only), offsets [N+1] from dispatch
 *   w1, w3 [N][F][d] dtype (w3 NULL unless SwiGLU)
 *   h      [T*k][F] dtype out (rows >= R untouched)
 *   ws     NULL, or a workspace of moe_workspace_bytes(s) bytes: with it, when the
 *          last round of 256x256 output tiles would leave most CUs idle, those
 *          tiles are split along K and their float32 partials added in a fixed
 *          order (deterministic); without it they run as 128x128 quarter tiles.
 *          The two give results that differ only in float32 rounding order.
 */
moe_status moe_expert_up(const moe_shape* s, const void* x_perm, const float* row_scale,
                         const int32_t* offsets, const void* w1, const void* w3, void* h,
                         void* ws, size_t ws_bytes, void* stream);

/* Expert down-projection (grouped GEMM 2): out[r] = W2[e] h[r].
 *   h [T*k][F] dtype, offsets [N+1], w2 [N][d][F] dtype, out [T*k][d] dtype;
 *   ws as for moe_expert_up. */
moe_status moe_expert_down(const moe_shape* s, const void* h, const int32_t* offsets,
                           const void* w2, void* out, void* ws, size_t ws_bytes, void* stream);

/* The always-on shared expert on the unquantised input ("moe communication
 * costs" / "Capacity factor and token dropping": a shared expert every token
 * passes through): h_shared = act(Ws1 x, Ws3 x), out_shared = Ws2 h_shared.
 *   x [T][d]; ws1, ws3 [F][d] (ws3 NULL unless SwiGLU); ws2 [d][F];
 *   h_shared [T][F] scratch; out_shared [T][d] out.  All dtype.
 *   ws     NULL, or a workspace of moe_workspace_bytes(s) bytes: with it, a
 *          GEMM of few output tiles (few tokens) is split along K over all CUs
 *          and its float32 partials added in a fixed order (results differ from
 *          the call without ws only in float32 rounding order). */
moe_status moe_shared_expert(const moe_shape* s, const void* x, const void* ws1,
                             const void* ws3, const void* ws2, void* h_shared,
                             void* out_shared, void* ws, size_t ws_bytes, void* stream);

/* The shared expert's first GEMM alone (the same passages as moe_shared_expert):
 * h_shared = act(Ws1 x, Ws3 x).  x [T][d]; ws1, ws3 [F][d] (ws3 NULL unless
 * SwiGLU); h_shared [T][F] out.  All dtype.  ws as for moe_shared_expert. */
moe_status moe_shared_expert_up(const moe_shape* s, const void* x, const void* ws1,
                                const void* ws3, void* h_shared, void* ws, size_t ws_bytes,
                                void* stream);

/* moe_expert_down and the shared expert's down GEMM (out_shared = Ws2 h_shared)
 * in one launch of the grouped GEMM, the shared expert as one more segment after
 * the routed ones (two launches for float32 layers).  Requires has_shared.
 *   h, offsets, w2, out as for moe_expert_down; h_shared [T][F], ws2 [d][F] (the
 *   layout of one of w2's matrices), out_shared [T][d] out; ws as for
 *   moe_expert_up.  Each output element is the one moe_expert_down or
 *   moe_shared_expert computes, up to float32 rounding order where the two
 *   forms split K differently (few tokens). */
moe_status moe_expert_down_shared(const moe_shape* s, const void* h, const int32_t* offsets,
                                  const void* w2, void* out, const void* h_shared,
                                  const void* ws2, void* out_shared, void* ws, size_t ws_bytes,
                                  void* stream);

/* All experts: moe_expert_up + moe_expert_down, or with has_shared
 * moe_expert_up + moe_shared_expert_up + moe_expert_down_shared (x, ws1, ws3,
 * ws2, out_shared required then, else ignored).  The intermediates live in the
 * workspace.  out [T*k][d], out_shared [T][d]. */
moe_status moe_experts(const moe_shape* s, const void* x_perm, const float* row_scale,
                       const int32_t* offsets, const void* w1, const void* w3, const void* w2,
                       const void* x, const void* ws1, const void* ws3, const void* ws2,
                       void* out, void* out_shared, void* ws, size_t ws_bytes, void* stream);

/* Combine: the single-GPU form of the return all-to-all ("Part 5" / "1.2", step 3)
 * and the mixture y = sum over the top-k of weight * expert output ("moe
 * communication costs" / "Router design").  Accumulates in float32 in slot order
 * j = 0..k-1, adds out_shared last, rounds once to dtype.
 *   out [T*k][d], out_shared [T][d] or NULL, x [T][d], pos [T][k], w [T][k] f32,
 *   y [T][d] dtype out.  A dropped slot contributes w * x[t] (pass-through) or 0. */
moe_status moe_combine(const moe_shape* s, const void* out, const void* out_shared,
                       const void* x, const int32_t* pos, const float* w, void* y,
                       void* stream);

/* Route then dispatch in one call, enqueued on one stream: the outputs of
 * moe_route (idx, w, counts, kept_counts, p, f, l_aux; no logits) and of
 * moe_dispatch (offsets, pos, src, drop, x_perm, row_scale), equal to those of
 * the two calls made one after the other.  The dispatch plan is folded into
 * the row copy: the router's per-tile expert counts give each 16-token tile's
 * base and the copy ranks its token inside its tile ("Part 5" / "1.2", step 1,
 * with every expert local), which saves two kernel launches.  Arguments,
 * layouts and errors as for the two calls; p, f, l_aux may be NULL. */
moe_status moe_route_dispatch(const moe_shape* s, const void* x, const void* w_g,
                              const float* bias, int32_t* idx, float* w, int32_t* counts,
                              int32_t* kept_counts, float* p, float* f, float* l_aux,
                              int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                              void* x_perm, float* row_scale, void* ws, size_t ws_bytes,
                              void* stream);

/* moe_route_dispatch without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Its kernels' scratch (router partials,
 * per-tile counts and bases, split logits) lives in a static device array of
 * MOE_STATIC_SCRATCH_BYTES (48 MiB) per GPU; the call allocates nothing.  The
 * caller still passes every input and output; arguments, layouts, results and
 * the other errors are those of moe_route_dispatch.  A shape whose scratch
 * (the router regions of moe_workspace_bytes' layout: about 12 bytes per
 * 8 tokens per expert, plus up to 32 MiB of partial logits for wide routers
 * or fewer than 512 tokens) exceeds the array returns MOE_ERR_TOO_LARGE
 * before any launch.  Every call on one GPU shares that GPU's array: calls
 * that may overlap in time on one GPU (different streams, or threads) race
 * and give undefined results; serialise them, or use moe_route_dispatch with
 * separate workspaces. */
moe_status moe_route_dispatch_noalloc(const moe_shape* s, const void* x, const void* w_g,
                                      const float* bias, int32_t* idx, float* w, int32_t* counts,
                                      int32_t* kept_counts, float* p, float* f, float* l_aux,
                                      int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                                      void* x_perm, float* row_scale, void* stream);

/* Route then plan, without the expert-ordered copy of x: the first phase of the
 * fused layer, whose up GEMM reads each row of x through src
 * (moe_expert_up_gather).  "MoE: what it costs to train and serve" / "In
 * short" and "Expert parallelism and two all-to-alls": the dispatch overlaps
 * with the expert computation instead of running as its own pass.  Outputs and
 * errors as moe_route_dispatch (idx, w, counts, kept_counts, p, f, l_aux,
 * offsets, pos, src, drop are identical), except:
 *   x_codes   [T][d] uint8 out (FP8 buffer only, else ignored): token t's e4m3
 *             codes in row t (moe_dispatch's quantiser, stored once per token)
 *   row_scale [T*k] float32 out (FP8 buffer only): the token's scale at each
 *             kept slot's position, as moe_dispatch writes it. */
moe_status moe_route_plan(const moe_shape* s, const void* x, const void* w_g, const float* bias,
                          int32_t* idx, float* w, int32_t* counts, int32_t* kept_counts, float* p,
                          float* f, float* l_aux, int32_t* offsets, int32_t* pos, int32_t* src,
                          uint8_t* drop, void* x_codes, float* row_scale, void* ws, size_t ws_bytes,
                          void* stream);

/* moe_expert_up with a gathered operand: row r of expert e's segment reads row
 * src[r] of a ([T][d]: x for a bf16/f32 buffer, the token-order codes of
 * moe_route_plan for an FP8 buffer, with row_scale [T*k] by position).  h and
 * the arithmetic are those of moe_expert_up on the dispatch buffer (bit for
 * bit the same).  MOE_ERR_UNSUPPORTED when T*d*element size exceeds 4 GiB - 1
 * (32-bit row offsets).  ws as for moe_expert_up. */
moe_status moe_expert_up_gather(const moe_shape* s, const void* a, const float* row_scale,
                                const int32_t* offsets, const int32_t* src, const void* w1,
                                const void* w3, void* h, void* ws, size_t ws_bytes, void* stream);

/* moe_expert_up_gather and moe_shared_expert_up in one call (has_shared must
 * be 1): h [T*k][F] from the routed rows of a, read through src as
 * moe_expert_up_gather reads them, and h_shared [T][F] from x [T][d] with
 * ws1, ws3, both bit for bit what the two calls write.  "MoE: what it costs to
 * train and serve" / "When decoding, batch size changes the arithmetic": a
 * decode step streams weights, and a call of at most four tokens with bf16
 * weights reads each weight row once in a single launch for both (no tiles);
 * otherwise the two GEMMs run one after the other.  Errors as the two calls. */
moe_status moe_expert_up_gather_shared(const moe_shape* s, const void* a, const float* row_scale,
                                       const int32_t* offsets, const int32_t* src, const void* w1,
                                       const void* w3, void* h, const void* x, const void* ws1,
                                       const void* ws3, void* h_shared, void* ws, size_t ws_bytes,
                                       void* stream);

/* The whole layer: moe_route_dispatch, moe_experts, moe_combine, enqueued on
 * one stream; results equal those of the four single-phase calls.  Every
 * output buffer is required except p, f, l_aux (may be NULL) and the
 * shared-expert buffers (ignored unless has_shared).  With x_perm == NULL the
 * layer runs fused: moe_route_plan, moe_expert_up_gather, moe_expert_down
 * (with has_shared: moe_expert_up_gather_shared and moe_expert_down_shared)
 * and moe_combine, with no dispatch buffer (row_scale may
 * then be NULL too; the fp8 codes and scales live in the workspace); every
 * other output is bit for bit that of the unfused call. */
moe_status moe_forward(const moe_shape* s, const void* x, const void* w_g, const float* bias,
                       const void* w1, const void* w3, const void* w2,
                       const void* ws1, const void* ws3, const void* ws2,
                       int32_t* idx, float* w, int32_t* counts, int32_t* kept_counts,
                       float* p, float* f, float* l_aux,
                       int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                       void* x_perm, float* row_scale, void* out, void* out_shared, void* y,
                       void* ws, size_t ws_bytes, void* stream);

/* The down GEMM with the combine in its epilogue: the scatter half of a fused
 * gather-GEMM-scatter ("MoE: what it costs to train and serve" / "In short":
 * dispatch and combine overlap with the expert computation; "Expert
 * parallelism and two all-to-alls": the return traffic).  Writes out (and,
 * with has_shared, out_shared) as moe_expert_down (moe_expert_down_shared)
 * called with ws = NULL, and y as moe_combine on those outputs, bit for bit.
 * Each tile of the down GEMM, once its output rows are written, counts them
 * per token and 128-column group; the tile that completes a token's group
 * (its kept slots and its shared-expert row) writes those columns of y in the
 * combine's order and arithmetic.  Tokens that no row reaches (every slot
 * dropped, no shared expert) get y before the GEMM.  No float atomics: results
 * are deterministic.  Float32 layers and calls of at most four tokens (the
 * decode GEMV) run moe_expert_down(_shared) with ws and moe_combine instead.
 *   h [T*k][F], offsets [N+1], src [T*k] (token of each kept row), w2, out as for
 *   moe_expert_down; h_shared, ws2, out_shared as for moe_expert_down_shared
 *   (required with has_shared, else ignored); x [T][d], pos [T][k], w [T][k]
 *   float32, y [T][d] as for moe_combine; ws required (its counters, no
 *   initialisation needed).  Errors as moe_expert_down and moe_combine. */
moe_status moe_expert_down_combine(const moe_shape* s, const void* h, const int32_t* offsets,
                                   const int32_t* src, const void* w2, void* out, const void* h_shared,
                                   const void* ws2, void* out_shared, const void* x, const int32_t* pos,
                                   const float* w, void* y, void* ws, size_t ws_bytes, void* stream);

/* The fused layer of moe_forward (x_perm = NULL) with moe_expert_down_combine
 * in place of the down GEMM and the combine: moe_route_plan, the gathering up
 * GEMM(s), moe_expert_down_combine.  Arguments as moe_forward without x_perm;
 * every output equals that of moe_route_plan, moe_expert_up_gather(_shared)
 * and moe_expert_down_combine called one after the other. */
moe_status moe_forward_scatter(const moe_shape* s, const void* x, const void* w_g, const float* bias,
                               const void* w1, const void* w3, const void* w2,
                               const void* ws1, const void* ws3, const void* ws2,
                               int32_t* idx, float* w, int32_t* counts, int32_t* kept_counts,
                               float* p, float* f, float* l_aux,
                               int32_t* offsets, int32_t* pos, int32_t* src, uint8_t* drop,
                               float* row_scale, void* out, void* out_shared, void* y,
                               void* ws, size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* moe_status_string(moe_status st);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
