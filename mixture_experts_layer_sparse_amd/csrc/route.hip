// Router: logits (skinny GEMM), group limit, top-k, sparse softmax and the
// per-tile load statistics, fused in one kernel; then the statistics over all
// tiles (counts, f, p, the per-tile prefix, the offsets and L_aux) in a kernel
// spread over the experts, or, with a single tile, in the router kernel itself.
//
// What it computes follows "moe communication costs" / "Router design" (logits
// W_g x; the top-k entries pick the experts), "Part 5" / "1.1 The Router Kernel"
// (strict > while scanning experts in index order, so equal logits go to the
// lower index; softmax over only the selected logits, max subtracted) and
// "Load balancing" (f_i, p_i, L_aux).  The group limit follows "MoE: what it
// costs to train and serve" / "Limit how many machines a token touches".
//
// Design (differs from the page's one-thread-per-token kernel): a workgroup of
// 8 waves owns 16 tokens.  For bf16 the logits come from 16x16x32 bf16 MFMAs:
// x staged through LDS (each element read once), W_g fragments from L2; the
// waves split the experts and the d-loop and their partial sums are added in a
// fixed order.  With few tokens the logits are first computed as partials
// spread over more waves, and for wide routers (many experts times a wide d)
// as one dense split-K GEMM; the router then adds the partials in order.  A
// call of at most 16 tokens (one router tile, e.g. a decode step) gets its
// logits from one workgroup per expert (whole dot products), and its router
// workgroup then also writes the fused layer's plan (and that kernel the fp8
// codes), so such a call is two kernels.
// Selection: with at most 32 experts a token's lanes hold one expert each (one
// lane per token under a group limit), with maximum reductions on keys (logit,
// ~index); with more, one wave handles one token, each lane four consecutive
// experts, by a float maximum over the wave and a ballot for the lowest expert
// index holding it.  Either way equal logits go to the lower index, and nothing
// depends on thread timing.
#include "fp8_quant.h"
#include "moe_internal.h"

// k-steps of loads each wave issues before their MFMAs (8 spills three
// registers under the four-waves-per-SIMD register budget)
#ifndef MOE_ROUTE_U
#define MOE_ROUTE_U 7
#endif

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRouteSplitMax = 64;     // K ranges of partial logits the router adds at most
constexpr int kLogitsSplitMax = 16;    // d-ranges of the few-token split logits at most
constexpr int kRouteSplitBatch = 16;   // ranges whose loads the router issues together
static_assert(kSplitKMax <= kRouteSplitMax, "the router adds every K range of the logits GEMM");

struct RouteArgs {
  const void* x;
  const void* wg;
  const float* bias;
  int32_t* idx;
  float* w;
  float* logits;
  float* psum;
  int32_t* hist;
  int64_t T;
  int d, N, k, n_groups, topk_groups, gsk;
  const float* lpart;   // partial logits (range kr, token t, expert e at kr * lrange + t * lld + e), or null
  int lsplit;
  int64_t lrange;
  int lld;
  const int32_t* lmeta; // non-null: the range count and the tile count come from this split-K header
  int gate;             // moe_gate
  RouteStats rs;        // rs.done: arrival counter of the statistics workgroups, zeroed here
  int fold;             // one tile: this kernel writes the final statistics (rs) itself
  int cap;
  float alpha;
  // with fold: the fused layer's plan (pos non-null: pos, src, drop; with
  // row_scale the kept slots' fp8 row scales, taken from tscale [T])
  int32_t* pos;
  int32_t* src;
  uint8_t* drop;
  float* row_scale;
  const float* tscale;
};

// Key ordering "larger logit first, then lower expert index"; 0 = no candidate.
__device__ __forceinline__ uint64_t sel_key(float v, int e) {
  v = v + 0.0f;                                   // -0 -> +0 so that zeros tie
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(0xFFFF - e);
}
__device__ __forceinline__ int key_index(uint64_t key) {
  return 0xFFFF - static_cast<int>(key & 0xFFFFFFFFu);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t u = static_cast<uint32_t>(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// Cross-lane steps on the DPP network (VALU, a few cycles each) instead of
// LDS permutes (a hundred or more cycles each, and the selection is a long
// chain of them): within each row of 16 lanes, swaps of lanes 1 and 2 apart
// (quad_perm) and the half-row and row mirrors, which pair every lane with one
// in the other half (8 or 16 lanes); the four rows then meet through lanes 0,
// 16, 32 and 48 (readlane).  Max, sum and the top-2 merge are symmetric in the
// pair, so every lane of a run ends with the same value.  Every lane must be
// active.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within 16
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xF, 0xF, false));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ float lanef(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// All-reduces over aligned runs of `width` lanes (a power of two up to 64).
__device__ __forceinline__ float run_max_f(float v, int width) {
  if (width > 1) v = fmaxf(v, dppf<kDppXor1>(v));
  if (width > 2) v = fmaxf(v, dppf<kDppXor2>(v));
  if (width > 4) v = fmaxf(v, dppf<kDppHalfMirror>(v));
  if (width > 8) v = fmaxf(v, dppf<kDppMirror>(v));
  if (width > 16) v = fmaxf(v, __shfl_xor(v, 16));
  if (width > 32) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float run_sum_f(float v, int width) {
  if (width > 1) v += dppf<kDppXor1>(v);
  if (width > 2) v += dppf<kDppXor2>(v);
  if (width > 4) v += dppf<kDppHalfMirror>(v);
  if (width > 8) v += dppf<kDppMirror>(v);
  if (width > 16) v += __shfl_xor(v, 16);
  if (width > 32) v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ uint64_t run_max_u64(uint64_t v, int width) {
  if (width > 1) v = umax64(v, dpp64<kDppXor1>(v));
  if (width > 2) v = umax64(v, dpp64<kDppXor2>(v));
  if (width > 4) v = umax64(v, dpp64<kDppHalfMirror>(v));
  if (width > 8) v = umax64(v, dpp64<kDppMirror>(v));
  if (width > 16) v = umax64(v, __shfl_xor(v, 16));
  if (width > 32) v = umax64(v, __shfl_xor(v, 32));
  return v;
}
// Whole wave: rows by DPP, then the four row results through readlane.
__device__ __forceinline__ float wave_max_f(float v) {
  v = run_max_f(v, 16);
  return fmaxf(fmaxf(lanef(v, 0), lanef(v, 16)), fmaxf(lanef(v, 32), lanef(v, 48)));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v = run_sum_f(v, 16);
  return (lanef(v, 0) + lanef(v, 16)) + (lanef(v, 32) + lanef(v, 48));
}

constexpr int RW = 8;                  // waves per router workgroup
constexpr int SMALL_N = 32;            // up to this many experts one lane selects for one token

// Logit tile [TM][ldl] in LDS, computed by the bf16 MFMA path.  The 8 waves
// split the experts into CG column groups of 16-expert blocks and d into KS
// slices (CG * KS = 8); each wave issues the loads of MOE_ROUTE_U (7) k-steps
// before their MFMAs, so that about 28 KB per wave are in flight.
template <int TM>
__device__ void logits_bf16(const RouteArgs& a, int64_t t0, float* part, float* lt, int ldl) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = a.N, d = a.d;
  const int NB = (N + 15) / 16;                       // 16-expert column blocks
  const int CG = NB >= 8 ? 8 : (NB >= 3 ? 4 : NB);    // column groups
  const int KS = RW / CG;                             // d-slices
  const int ks = wave / CG, cg = wave % CG;
  const int nsteps = d / 32;
  const int s0 = ks * nsteps / KS, s1 = (ks + 1) * nsteps / KS;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* wg = static_cast<const uint16_t*>(a.wg);
  int64_t t = t0 + lr;
  if (t > a.T - 1) t = a.T - 1;
  const uint16_t* xrow = x + t * d + lk;
  const uint16_t* wrow[2];
  bool wok[2];
  int nblk = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cb = cg + i * CG;
    const int e = cb * 16 + lr;
    wok[i] = cb < NB && e < N;
    wrow[i] = wg + static_cast<int64_t>(wok[i] ? e : 0) * d + lk;
    if (cb < NB) nblk = i + 1;
  }
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const bf16x8 zero = {};
  constexpr int U = MOE_ROUTE_U;
  int s = s0;
  for (; s + U <= s1; s += U) {
    bf16x8 av[U], bv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (s + u) * 32;
      av[u] = *reinterpret_cast<const bf16x8*>(xrow + k0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        bv[u][i] = (i < nblk && wok[i]) ? *reinterpret_cast<const bf16x8*>(wrow[i] + k0) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (i < nblk) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u][i], acc[i], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    const int k0 = s * 32;
    const bf16x8 av = *reinterpret_cast<const bf16x8*>(xrow + k0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i < nblk) {
        const bf16x8 bv = wok[i] ? *reinterpret_cast<const bf16x8*>(wrow[i] + k0) : zero;
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[i], 0, 0, 0);
      }
    }
  }
  // acc[i][r] = partial logit of token 4*(lane/16)+r, expert (cg+i*CG)*16 + lane%16
  const int NP = NB * 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i < nblk) {
      const int col = (cg + i * CG) * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if ((lane >> 4) * 4 + r < TM) part[(ks * TM + (lane >> 4) * 4 + r) * NP + col] = acc[i][r];
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < TM * N; q += RW * 64) {
    const int m = q / N, e = q % N;
    float v = 0.f;
    float pk[RW];
#pragma unroll
    for (int kk = 0; kk < RW; ++kk)             // (KS <= RW: the reads issued together, added in order)
      pk[kk] = part[((kk < KS ? kk : KS - 1) * TM + m) * NP + e];
#pragma unroll
    for (int kk = 0; kk < RW; ++kk)
      if (kk < KS) v += pk[kk];
    if (a.bias) v += a.bias[e];
    lt[m * ldl + e] = v;
  }
}

// 16 bytes per lane from a buffer straight into LDS (lane i writes lds + 16 * i).
typedef __attribute__((address_space(3))) void* lds_ptr;
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)lds, 16, voff, 0, 0, 0);
}

constexpr int SCH = 512;               // staged chunk: 512 elements (1 KB) of each token row
constexpr int SPH = 8;                 // chunks per staging phase (8 x 16 rows x 1 KB = 128 KB)

// The same logits with x staged through LDS (d a multiple of 512): every
// load is one token row's contiguous 1 KB, all of a phase's loads are issued
// at once (up to 128 KB in flight per workgroup), and the MFMA fragments are
// read from LDS.  Chunk ch of row r sits at buf + (ch * 16 + r) KB with its
// 16-byte pieces q stored at (q & ~15) | ((q & 15) ^ r): a fragment read (16
// rows, one piece each) then touches 16 different bank groups.  Rows past T
// read as zeros (buffer range).  part / lt live in buf once the loads are done.
template <int TM>
__device__ void logits_bf16_staged(const RouteArgs& a, int64_t t0, uint8_t* buf, float* part,
                                   float* lt, int ldl) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = a.N, d = a.d;
  const int NB = (N + 15) / 16;
  const int CG = NB >= 8 ? 8 : (NB >= 3 ? 4 : NB);
  const int KS = RW / CG;
  const int ks = wave / CG, cg = wave % CG;
  const int lr = lane & 15, kc = lane >> 4;
  const uint16_t* wg = static_cast<const uint16_t*>(a.wg);
  const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(static_cast<const uint16_t*>(a.x) + t0 * d), static_cast<short>(0),
      static_cast<int>((a.T - t0 < TM ? a.T - t0 : TM) * d * 2), 0x00020000);
  const uint16_t* wrow[2];
  bool wok[2];
  int nblk = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cb = cg + i * CG;
    const int e = cb * 16 + lr;
    wok[i] = cb < NB && e < N;
    wrow[i] = wg + static_cast<int64_t>(wok[i] ? e : 0) * d + kc * 8;
    if (cb < NB) nblk = i + 1;
  }
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const bf16x8 zero = {};
  const int nch_all = d / SCH;
  for (int c0 = 0; c0 < nch_all; c0 += SPH) {
    const int nch = nch_all - c0 < SPH ? nch_all - c0 : SPH;
    // loads: row-chunk i = ch * 16 + r, taken by the waves in turn
    for (int i = wave; i < nch * TM; i += RW) {
      const int ch = i / TM, r = i % TM;
      const int q = (lane & ~15) | ((lane & 15) ^ r);  // the piece this lane writes at lane * 16
      lds_dma16(rsx, buf + i * 1024,
                static_cast<uint32_t>(r * d * 2 + (c0 + ch) * 1024 + q * 16));
    }
    // this wave's k-steps (of 32) among the phase's nch * 16
    const int S = nch * (SCH / 32);
    const int s0 = ks * S / KS, s1 = (ks + 1) * S / KS;
    constexpr int U = 8;
    // W_g fragments of the first batch are loaded while x is still arriving
    bf16x8 bv[U][2];
    auto load_w = [&](int s) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int st = s + u < s1 ? s + u : s1 - 1;    // (repeats are not accumulated)
        const int k0 = (c0 * SCH) + st * 32;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          bv[u][i] = (i < nblk && wok[i]) ? *reinterpret_cast<const bf16x8*>(wrow[i] + k0) : zero;
      }
    };
    if (s0 < s1) load_w(s0);
    __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0): own loads landed
    __syncthreads();
    for (int s = s0; s < s1; s += U) {
      bf16x8 av[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int st = s + u < s1 ? s + u : s1 - 1;
        const int ch = st / (SCH / 32), q = (st % (SCH / 32)) * 4 + kc;
        // (with 8-token tiles the MFMA's rows 8-15 repeat rows 0-7; their results are dropped)
        const int lrow = lr % TM;
        av[u] = *reinterpret_cast<const bf16x8*>(buf + (ch * TM + lrow) * 1024 +
                                                 (((q & ~15) | ((q & 15) ^ lrow)) << 4));
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (s + u < s1) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
            if (i < nblk) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u][i], acc[i], 0, 0, 0);
        }
      if (s + U < s1) load_w(s + U);
    }
    __syncthreads();                                 // buf free for the next phase
  }
  const int NP = NB * 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i < nblk) {
      const int col = (cg + i * CG) * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kc * 4 + r < TM) part[(ks * TM + kc * 4 + r) * NP + col] = acc[i][r];
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < TM * N; q += RW * 64) {
    const int m = q / N, e = q % N;
    float v = 0.f;
    float pk[RW];
#pragma unroll
    for (int kk = 0; kk < RW; ++kk)             // (KS <= RW: the reads issued together, added in order)
      pk[kk] = part[((kk < KS ? kk : KS - 1) * TM + m) * NP + e];
#pragma unroll
    for (int kk = 0; kk < RW; ++kk)
      if (kk < KS) v += pk[kk];
    if (a.bias) v += a.bias[e];
    lt[m * ldl + e] = v;
  }
}

// Partial logits for few tokens: one wave per (16 tokens, 16 experts, d-range)
// unit, one 16x16x32 MFMA per 32-wide k-step (A = token rows, B = router rows,
// loaded straight from memory; rows past T or N read as zero).  Unit order is
// range-fastest, so the waves of a workgroup share token and router rows.
__global__ __launch_bounds__(256) void logits_split_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wg,
                                                           float* __restrict__ lpart, int64_t T,
                                                           int d, int N, int ks) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t TB = (T + 15) / 16;
  const int EB = (N + 15) / 16;
  if (unit >= TB * EB * ks) return;
  const int kr = static_cast<int>(unit % ks);
  const int64_t rest = unit / ks;
  const int eb = static_cast<int>(rest % EB);
  const int64_t tb = rest / EB;
  const int nst = d / 32;
  const int s0 = kr * nst / ks, s1 = (kr + 1) * nst / ks;
  const int r = lane & 15, kc = lane >> 4;
  const int64_t t = tb * 16 + r;
  const int e = eb * 16 + r;
  const bool tok = t < T, ex = e < N;
  const uint16_t* xr = x + (tok ? t : 0) * d + kc * 8;
  const uint16_t* wr = wg + static_cast<int64_t>(ex ? e : 0) * d + kc * 8;
  const bf16x8 zero = {};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;
  for (int st = s0; st < s1; st += U) {
    bf16x8 av[U], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (st + u < s1 ? st + u : s0) * 32;
      av[u] = tok ? *reinterpret_cast<const bf16x8*>(xr + k0) : zero;
      bv[u] = ex ? *reinterpret_cast<const bf16x8*>(wr + k0) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (st + u < s1) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u], acc, 0, 0, 0);
  }
  // acc[j]: token row 4 * kc + j, expert column r
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t2 = tb * 16 + 4 * kc + j;
    if (t2 < T && ex) lpart[(static_cast<int64_t>(kr) * T + t2) * N + e] = acc[j];
  }
}

// x . w over 8 bf16 pairs (the products are exact in float32), added to acc in element order
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
  const uint32_t xa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(xa[i] << 16), __uint_as_float(wb[i] << 16), acc);
    acc = fmaf(__uint_as_float(xa[i] & 0xFFFF0000u), __uint_as_float(wb[i] & 0xFFFF0000u), acc);
  }
  return acc;
}

// Logits of a call with at most 16 tokens: workgroup e computes x[t] . W_g[e]
// for every token, so that each router row is read once, by one CU.  The four
// waves split the tokens (TPW per wave) or, with fewer than four tokens, each
// token's d into P = 2 or 4 parts added in part order; a lane sums its 16-byte
// chunks in order and the wave adds its lanes by a fixed tree.  The result is
// the router's logits as one range of partials ([T][N]).  With x_codes the
// workgroups also quantise x to fp8 in token order (workgroup b: tokens b,
// b + gridDim.x, ...), codes and scales bit for bit those of the dispatch
// quantiser, the scales into tscale [T].
template <int TPW>
__global__ __launch_bounds__(256) void logits_dot_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wg,
                                                         float* __restrict__ out, int T, int d, int N,
                                                         uint8_t* __restrict__ x_codes,
                                                         float* __restrict__ tscale) {
  __shared__ float red[4][4];
  __shared__ float wmax[4];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P = T >= 4 ? 1 : (T >= 2 ? 2 : 4);       // d-parts per token
  const int G = 4 / P;                               // token groups
  const int tg = wave / P, part = wave % P;
  const int nch = d / 8;
  const int c0 = part * nch / P, c1 = (part + 1) * nch / P;
  const uint4* wr = reinterpret_cast<const uint4*>(wg + static_cast<int64_t>(e) * d);
  const uint4* xb = reinterpret_cast<const uint4*>(x);
  int tok[TPW];
  float acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    tok[j] = tg + G * j;
    acc[j] = 0.f;
  }
  // U chunks per lane per pass, their loads issued together (indices clamped
  // into range: loads under a condition were waited for one by one)
  constexpr int U = 4;
  for (int cb = c0 + lane; cb < c1; cb += 64 * U) {
    uint4 wv[U], xv[U][TPW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(cb + 64 * u, c1 - 1);
      wv[u] = wr[c];
#pragma unroll
      for (int j = 0; j < TPW; ++j) xv[u][j] = xb[static_cast<int64_t>(min(tok[j], T - 1)) * nch + c];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (cb + 64 * u < c1) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) acc[j] = dot8_bf16(xv[u][j], wv[u], acc[j]);
      }
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = wave_sum_f(acc[j]);
  if (P == 1) {
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < TPW; ++j)
        if (tok[j] < T) out[static_cast<int64_t>(tok[j]) * N + e] = acc[j];
    }
  } else {
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < TPW; ++j) red[wave][j] = acc[j];
    }
    __syncthreads();
    if (part == 0 && lane == 0) {
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        if (tok[j] >= T) continue;
        float v = red[wave][j];
        for (int q = 1; q < P; ++q) v += red[wave + q][j];
        out[static_cast<int64_t>(tok[j]) * N + e] = v;
      }
    }
  }
  if (!x_codes) return;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    const uint4* xr = xb + static_cast<int64_t>(t) * nch;
    float am = 0.f;
    for (int c = threadIdx.x; c < nch; c += 256) am = fmaxf(am, absmax8(xr[c]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    __syncthreads();                                // (the previous token's wmax reads are done)
    if (lane == 0) wmax[wave] = am;
    __syncthreads();
    am = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));   // (a max is exact in any order)
    float inv, scale;
    fp8_row_scale(am, &inv, &scale);
    uint2* dst = reinterpret_cast<uint2*>(x_codes + static_cast<int64_t>(t) * d);
    for (int c = threadIdx.x; c < nch; c += 256) dst[c] = quant8(xr[c], inv);
    if (threadIdx.x == 0) tscale[t] = scale;
  }
}

// Logits of a 16-token tile from the partials: the d-ranges added in order.
template <int TM>
__device__ void logits_from_partials(const RouteArgs& a, int ks, int64_t lrange, int64_t t0, float* lt,
                                     int ldl) {
  // only the tile's tokens (rows past T are never read); the ranges are added
  // in order, their loads issued kRouteSplitBatch at a time
  const int n_tok = static_cast<int>(a.T - t0 < TM ? a.T - t0 : TM);
  // (four entries' range loads in flight together: DeepSeek-V3 router 57.4 -> 55.4 us)
#pragma unroll 4
  for (int q = threadIdx.x; q < n_tok * a.N; q += RW * 64) {
    const int m = q / a.N, e = q % a.N;
    const int64_t t = t0 + m;
    float v = 0.f;
    for (int k0 = 0; k0 < ks; k0 += kRouteSplitBatch) {
      float pv[kRouteSplitBatch];
#pragma unroll
      for (int kr = 0; kr < kRouteSplitBatch; ++kr)
        pv[kr] = k0 + kr < ks ? a.lpart[(k0 + kr) * lrange + t * a.lld + e] : 0.f;
#pragma unroll
      for (int kr = 0; kr < kRouteSplitBatch; ++kr)
        if (k0 + kr < ks) v += pv[kr];
    }
    if (a.bias) v += a.bias[e];
    lt[m * ldl + e] = v;
  }
}

// fp32 path: plain dot products, one (token, expert) pair per thread at a time.
template <int TM>
__device__ void logits_f32(const RouteArgs& a, int64_t t0, float* lt, int ldl) {
  const float* x = static_cast<const float*>(a.x);
  const float* wg = static_cast<const float*>(a.wg);
  for (int q = threadIdx.x; q < TM * a.N; q += RW * 64) {
    const int m = q / a.N, e = q % a.N;
    int64_t t = t0 + m;
    if (t > a.T - 1) t = a.T - 1;
    const float* xr = x + t * a.d;
    const float* wr = wg + static_cast<int64_t>(e) * a.d;
    float v = 0.f;
    for (int j = 0; j < a.d; ++j) v = fmaf(xr[j], wr[j], v);
    if (a.bias) v += a.bias[e];
    lt[m * ldl + e] = v;
  }
}

// Exponentials of the routing weights and of p use the hardware exp2 (__expf,
// a few ulp for these arguments): both are float32 results checked to 1e-5
// relative, and no selection depends on them.

// Selection for one token by one lane (N <= SMALL_N): everything in order over
// the expert index, so a strictly larger value is needed to replace the
// current best and equal logits keep the lower index.  Writes the token's full
// softmax to prow (for p) and its k picks; counts go to the block histogram.
__device__ void select_lane(const RouteArgs& a, const float* row, float* prow, int64_t t, int* hl) {
  const int N = a.N, k = a.k;
  float mx = -INFINITY;
  for (int e = 0; e < N; ++e) mx = fmaxf(mx, row[e]);
  float zs = 0.f;
  for (int e = 0; e < N; ++e) zs += __expf(row[e] - mx);
  for (int e = 0; e < N; ++e) prow[e] = __expf(row[e] - mx) / zs;
  uint32_t allowed = N >= 32 ? 0xFFFFFFFFu : ((1u << N) - 1u);
  if (a.n_groups > 1) {
    const int G = a.n_groups, gsz = N / G;
    float gs[SMALL_N];
    for (int g = 0; g < G; ++g) {
      float top[kMaxTopK];
#pragma unroll
      for (int q = 0; q < kMaxTopK; ++q) top[q] = -INFINITY;
      for (int e = g * gsz; e < (g + 1) * gsz; ++e) {
        float val = row[e];
#pragma unroll
        for (int q = 0; q < kMaxTopK; ++q) {
          if (q < a.gsk && val > top[q]) {
            const float tmp = top[q];
            top[q] = val;
            val = tmp;
          }
        }
      }
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < kMaxTopK; ++q)
        if (q < a.gsk) sum += top[q];
      gs[g] = sum + 0.0f;
    }
    uint32_t gsel = 0u;
    for (int q = 0; q < a.topk_groups; ++q) {
      int best = -1;
      float bv = 0.f;
      for (int g = 0; g < G; ++g)
        if (!((gsel >> g) & 1u) && (best < 0 || gs[g] > bv)) { best = g; bv = gs[g]; }
      gsel |= 1u << best;
    }
    allowed = 0u;
    for (int e = 0; e < N; ++e)
      if ((gsel >> (e / gsz)) & 1u) allowed |= 1u << e;
  }
  int sel_e[kMaxTopK];
  float sel_v[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      int best = -1;
      float bv = 0.f;
      for (int e = 0; e < N; ++e) {
        const float v = row[e];
        if (((allowed >> e) & 1u) && (best < 0 || v > bv)) { best = e; bv = v; }
      }
      best = best < 0 ? 0 : best;                 // unreachable guard (k <= candidates)
      allowed &= ~(1u << best);
      sel_e[j] = best;
      sel_v[j] = row[best];
    }
  }
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) den += __expf(sel_v[j] - sel_v[0]);
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      a.idx[t * k + j] = sel_e[j];
      // full gate: the expert's probability in the softmax written to prow
      a.w[t * k + j] = a.gate == MOE_GATE_FULL ? __expf(sel_v[j] - mx) / zs
                                               : __expf(sel_v[j] - sel_v[0]) / den;
      atomicAdd(&hl[sel_e[j]], 1);
    }
  }
}

// Selection for N <= 32 experts without a group limit, all tokens of the tile
// at once: token m owns the NP lanes m * NP .. m * NP + NP - 1 (NP = N rounded
// up to a power of two, so a token's lanes never straddle a wave), lane e of
// them expert e.  The full softmax comes from butterflies over the token's
// lanes; top-k takes k rounds of a maximum over keys (logit, ~index), so equal
// logits go to the lower index as in an in-order scan with strict >.  Writes
// each token's p row to prow (for p) and its k picks; counts go to the block
// histogram.
template <int TM>
__device__ void select_lanes(const RouteArgs& a, const float* lt, int ldl, int64_t t0,
                             float (*prow)[SMALL_N + 1], int* hl) {
  const int N = a.N, k = a.k;
  int NP = 1;
  while (NP < N) NP <<= 1;
  const int m = threadIdx.x / NP, e = threadIdx.x % NP;   // (TM * NP <= 512 threads)
  const bool tok = m < TM && t0 + m < a.T;
  const bool live = tok && e < N;
  const float v = live ? lt[m * ldl + e] : -INFINITY;
  const float mx = run_max_f(v, NP);
  const float z = live ? __expf(v - mx) : 0.f;
  const float zs = run_sum_f(z, NP);
  if (m < TM && e < N) prow[m][e] = live ? z / zs : 0.f;
  uint64_t key = live ? sel_key(v, e) : 0ull;
  int sel_e[kMaxTopK];
  float sel_v[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      const uint64_t best = run_max_u64(key, NP);
      sel_e[j] = key_index(best);
      sel_v[j] = key_value(best);                // (the logit, with -0 read as +0)
      if (e == sel_e[j]) key = 0ull;
    }
  }
  if (!tok) return;
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) den += __expf(sel_v[j] - sel_v[0]);
  const int64_t t = t0 + m;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k && e == j) {
      a.idx[t * k + j] = sel_e[j];
      // full gate: the expert's probability in the softmax written to prow
      a.w[t * k + j] = a.gate == MOE_GATE_FULL ? __expf(sel_v[j] - mx) / zs
                                               : __expf(sel_v[j] - sel_v[0]) / den;
      atomicAdd(&hl[sel_e[j]], 1);
    }
  }
}

// The scan over the experts, by a whole workgroup (fixed orders): thread e <
// N holds expert e's kept count and f p; writes the exclusive scan of the kept
// counts into offsets and L_aux = alpha N sum f p.  A shuffle scan and a
// butterfly inside each wave, then the waves in order through LDS (xk, xp:
// one entry per wave).
__device__ void scan_experts(int kv, double pr, int N, float alpha, int32_t* offsets, float* l_aux,
                             int* xk, double* xp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (N + 63) / 64;
  int ki = kv;
  double tp = pr;
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(ki, off);
    if (lane >= off) ki += v;
    tp += __shfl_xor(tp, off);
  }
  if (wave < nw && lane == 63) xk[wave] = ki;
  if (wave < nw && lane == 0) xp[wave] = tp;
  __syncthreads();
  if (tid < N) {
    for (int w = 0; w < wave; ++w) ki += xk[w];
    if (offsets) {
      offsets[tid] = ki - kv;
      if (tid == N - 1) offsets[N] = ki;
    }
  }
  if (l_aux && tid == 0) {
    double acc = 0.0;
    for (int w = 0; w < nw; ++w) acc += xp[w];
    l_aux[0] = static_cast<float>(static_cast<double>(alpha) * N * acc);
  }
}

// End of a router workgroup, every thread with e = threadIdx.x (sum: the
// tile's p summed over its tokens, cnt: the tile's count, for e < N): the
// tile's partials for the statistics kernel, or, when the call has only this
// tile, the final statistics (the statistics kernel's formulas; no earlier
// tiles, so every base is 0).
__device__ void tile_stats(const RouteArgs& a, int e, float sum, int cnt, int* xk, double* xp) {
  const int N = a.N;
  if (!a.fold) {
    if (e < N) {
      a.psum[static_cast<int64_t>(blockIdx.x) * N + e] = sum;
      a.hist[static_cast<int64_t>(blockIdx.x) * N + e] = cnt;
    }
    return;
  }
  int kv = 0;
  double pr = 0.0;
  if (e < N) {
    const double pe = static_cast<double>(sum) / static_cast<double>(a.T);
    const double fe = static_cast<double>(cnt) / (static_cast<double>(a.T) * a.k);
    a.rs.counts[e] = cnt;
    kv = a.cap > 0 ? (cnt < a.cap ? cnt : a.cap) : cnt;
    a.rs.kept[e] = kv;
    if (a.rs.p) a.rs.p[e] = static_cast<float>(pe);
    if (a.rs.f) a.rs.f[e] = static_cast<float>(fe);
    if (a.rs.base) a.rs.base[e] = 0;
    pr = fe * pe;
  }
  scan_experts(kv, pr, N, a.alpha, a.rs.offsets, a.rs.l_aux, xk, xp);
}

// The fused layer's plan of a one-tile call, after tile_stats (every base is
// 0): slot j of token t goes to offsets[e] + the number of earlier tokens
// that chose e, or is dropped once that number reaches the capacity; the
// same positions as the dispatch plan's (token order, stable).  Writes pos,
// drop and src, and with an fp8 buffer the kept slots' row scales.
__device__ void tile_plan(const RouteArgs& a, int* sidx) {
  const int nk = static_cast<int>(a.T) * a.k;      // (one tile: T <= 16)
  __syncthreads();                                 // idx and offsets written by this workgroup
  for (int q = threadIdx.x; q < nk; q += RW * 64) sidx[q] = a.idx[q];
  __syncthreads();
  for (int q = threadIdx.x; q < nk; q += RW * 64) {
    const int e = sidx[q], t = q / a.k;
    int r = 0;
    for (int q2 = 0; q2 < t * a.k; ++q2) r += sidx[q2] == e ? 1 : 0;
    const int p = (a.cap > 0 && r >= a.cap) ? -1 : a.rs.offsets[e] + r;
    a.pos[q] = p;
    a.drop[q] = p < 0 ? 1 : 0;
    if (p >= 0) {
      a.src[p] = t;
      if (a.row_scale) a.row_scale[p] = a.tscale[t];
    }
  }
}

template <bool BF16, int TM>
__global__ __launch_bounds__(RW * 64) __attribute__((amdgpu_waves_per_eu(4))) void route_kernel(RouteArgs a) {
  // staging buffer of the x tile (bf16, d a multiple of 512); afterwards, and
  // on the other paths, it holds the d-split partials [KS][TM][NP] (16 KB) and
  // the logit tile [TM][kMaxExperts + 1].  Sized at launch (route_lds_bytes):
  // no larger than the shape needs, so that small d leaves room for more
  // workgroups per CU.
  extern __shared__ __attribute__((aligned(1024))) uint8_t sbuf[];
  float* part = reinterpret_cast<float*>(sbuf);
  float* lt = reinterpret_cast<float*>(sbuf + 16384);
  static_assert(16384 + TM * (kMaxExperts + 1) * 4 <= SPH * TM * 1024, "partials and logits fit");
  __shared__ float ps[RW][kMaxExperts];  // wave partial sums of p (large N)
  __shared__ float pl[TM][SMALL_N + 1];  // per-token p (small N)
  __shared__ int hl[kMaxExperts];
  __shared__ int xk[RW];
  __shared__ double xp[RW];
  __shared__ int sidx[TM * kMaxTopK];    // the tile's expert choices (one-tile plan)
  static_assert(RW * 64 >= kMaxExperts, "thread e ends expert e's statistics");
  const bool plan = a.fold && a.pos;
  const int ldl = kMaxExperts + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = a.N, k = a.k;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TM;

  for (int e = threadIdx.x; e < kMaxExperts; e += RW * 64) hl[e] = 0;
  // (the statistics kernel runs after this one on the same stream)
  if (blockIdx.x == 0 && threadIdx.x == 0 && !a.fold) *a.rs.done = 0;
  if (BF16) {
    if (a.lpart) {
      // range count and range stride: from the split-K header when the GEMM wrote the partials
      const int ks = a.lmeta ? a.lmeta[1] : a.lsplit;
      const int64_t lrange = a.lmeta ? static_cast<int64_t>(a.lmeta[0]) * (kRouterTileRows * kRouterTileCols)
                                     : a.lrange;
      logits_from_partials<TM>(a, ks, lrange, t0, lt, ldl);
    }
    else if (a.d % SCH == 0) logits_bf16_staged<TM>(a, t0, sbuf, part, lt, ldl);
    else logits_bf16<TM>(a, t0, part, lt, ldl);
  } else {
    logits_f32<TM>(a, t0, lt, ldl);
  }
  __syncthreads();

  if (a.logits) {
    for (int q = threadIdx.x; q < TM * N; q += RW * 64) {
      const int m = q / N, e = q % N;
      if (t0 + m < a.T) a.logits[(t0 + m) * N + e] = lt[m * ldl + e];
    }
  }

  if (N <= SMALL_N && a.n_groups <= 1) {
    select_lanes<TM>(a, lt, ldl, t0, pl, hl);
    __syncthreads();
    const int e = threadIdx.x;
    float sum = 0.f;
    if (e < N) {
#pragma unroll
      for (int m2 = 0; m2 < TM; ++m2) sum += pl[m2][e];
    }
    tile_stats(a, e, sum, e < N ? hl[e] : 0, xk, xp);
    if (plan) tile_plan(a, sidx);
    return;
  }
  if (N <= SMALL_N) {
    // group limit: one lane per token
    const int m = threadIdx.x;
    if (m < TM) {
      if (t0 + m < a.T) {
        select_lane(a, lt + m * ldl, pl[m], t0 + m, hl);
      } else {
        for (int e = 0; e < N; ++e) pl[m][e] = 0.f;
      }
    }
    __syncthreads();
    const int e = threadIdx.x;
    float sum = 0.f;
    if (e < N)
      for (int m2 = 0; m2 < TM; ++m2) sum += pl[m2][e];
    tile_stats(a, e, sum, e < N ? hl[e] : 0, xk, xp);
    if (plan) tile_plan(a, sidx);
    return;
  }

  // one wave per token; lane l holds experts 4l .. 4l + 3, so that a group of
  // gsz experts (gsz a multiple of 4, gsz / 4 a power of two) is an aligned
  // run of gsz / 4 lanes
  float psr[4] = {0.f, 0.f, 0.f, 0.f};    // this wave's sum of p over its tokens (expert 4 lane + i)
  const int G = a.n_groups > 1 ? a.n_groups : 1;
  const int gsz = N / G;
  const int GL = gsz / 4;
  const bool lane_groups = G > 1 && a.gsk <= 2 && gsz % 4 == 0 && (GL & (GL - 1)) == 0;
  int grp[4];                             // group of expert 4 lane + i
#pragma unroll
  for (int i = 0; i < 4; ++i) grp[i] = G > 1 && 4 * lane + i < N ? (4 * lane + i) / gsz : 0;
  for (int m = wave; m < TM; m += RW) {
    const int64_t t = t0 + m;
    if (t >= a.T) break;
    const float* row = lt + m * ldl;
    float v[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      ok[i] = e < N;
      v[i] = ok[i] ? row[e] : -INFINITY;
    }
    // full softmax over all N (bias included, no group mask) for p
    const float mx = wave_max_f(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    float z[4], zs = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = ok[i] ? __expf(v[i] - mx) : 0.f;
      zs += z[i];
    }
    zs = wave_sum_f(zs);
    const float rzs = 1.0f / zs;                  // (one division per token; p is a float32 mean)
#pragma unroll
    for (int i = 0; i < 4; ++i) psr[i] += z[i] * rzs;

    // group limit: a group scores the sum of its gsk largest logits, and the
    // topk_groups best groups (equal scores: the lower group) stay allowed
    uint64_t gsel = ~0ull;
    if (G > 1) {
      bool rep;                                   // this lane holds its group's score
      int rg;                                     // that group
      float gs = -INFINITY;
      if (lane_groups) {
        // the two largest of the lane's four, then merged over the group's lanes
        const float a0 = fmaxf(v[0], v[1]), b0 = fminf(v[0], v[1]);
        const float a1 = fmaxf(v[2], v[3]), b1 = fminf(v[2], v[3]);
        float t1 = fmaxf(a0, a1), t2 = fmaxf(fminf(a0, a1), fmaxf(b0, b1));
        auto merge = [&](float o1, float o2) {
          t2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
          t1 = fmaxf(t1, o1);
        };
        if (GL > 1) merge(dppf<kDppXor1>(t1), dppf<kDppXor1>(t2));
        if (GL > 2) merge(dppf<kDppXor2>(t1), dppf<kDppXor2>(t2));
        if (GL > 4) merge(dppf<kDppHalfMirror>(t1), dppf<kDppHalfMirror>(t2));
        if (GL > 8) merge(dppf<kDppMirror>(t1), dppf<kDppMirror>(t2));
        if (GL > 16) merge(__shfl_xor(t1, 16), __shfl_xor(t2, 16));
        if (GL > 32) merge(__shfl_xor(t1, 32), __shfl_xor(t2, 32));
        rep = (lane & (GL - 1)) == 0 && lane < G * GL;
        rg = lane / GL;
        if (rep) gs = a.gsk == 1 ? t1 : t1 + t2;
      } else {
        // lane g scores group g from the logit row
        rep = lane < G;
        rg = lane;
        if (rep) {
          float top[kMaxTopK];
#pragma unroll
          for (int q = 0; q < kMaxTopK; ++q) top[q] = -INFINITY;
          for (int e = lane * gsz; e < (lane + 1) * gsz; ++e) {
            float val = row[e];
            // insert into the descending list top[0..gsk)
#pragma unroll
            for (int q = 0; q < kMaxTopK; ++q) {
              if (q < a.gsk && val > top[q]) {
                const float tmp = top[q];
                top[q] = val;
                val = tmp;
              }
            }
          }
          gs = 0.f;
#pragma unroll
          for (int q = 0; q < kMaxTopK; ++q)
            if (q < a.gsk) gs += top[q];
        }
      }
      // rounds of: the best remaining score, the lowest lane holding it
      float cand = rep ? gs + 0.0f : -INFINITY;   // (-0 as +0)
      gsel = 0ull;
      for (int q = 0; q < a.topk_groups; ++q) {
        const float M = wave_max_f(cand);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(rep && cand == M);
        const int L0 = hit ? __builtin_ctzll(hit) : 0;
        const int g = __builtin_amdgcn_readlane(rg, L0);
        gsel |= 1ull << (g < G ? g : G - 1);
        if (lane == L0) cand = -INFINITY;
      }
    }
    // top-k over the allowed experts: rounds of the largest remaining logit
    // and the lowest expert index holding it (lowest lane, then lowest of its
    // four), which is then removed
    float cv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cv[i] = ok[i] && ((gsel >> grp[i]) & 1ull) ? v[i] + 0.0f : -INFINITY;
    int sel_e[kMaxTopK];
    float sel_v[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const float lm = fmaxf(fmaxf(cv[0], cv[1]), fmaxf(cv[2], cv[3]));
        const float M = wave_max_f(lm);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(lm == M);
        const int L0 = hit ? __builtin_ctzll(hit) : 0;
        const int fi = cv[0] == M ? 0 : (cv[1] == M ? 1 : (cv[2] == M ? 2 : 3));
        const int i0 = __builtin_amdgcn_readlane(fi, L0);
        const int e = 4 * L0 + i0;
        sel_e[j] = e < N ? e : N - 1;              // (unreachable guard: k <= candidates)
        sel_v[j] = M;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (lane == L0 && i == i0) cv[i] = -INFINITY;
      }
    }
    // softmax over the k selected logits, summed in slot order
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k) den += __expf(sel_v[j] - sel_v[0]);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k && lane == j) {
        a.idx[t * k + j] = sel_e[j];
        // full gate: the expert's probability in the softmax summed into p
        a.w[t * k + j] = a.gate == MOE_GATE_FULL ? __expf(sel_v[j] - mx) / zs
                                                 : __expf(sel_v[j] - sel_v[0]) / den;
        atomicAdd(&hl[sel_e[j]], 1);
      }
    }
  }
  // per-block partial statistics, combined over waves in wave order
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    if (e < N) ps[wave][e] = psr[i];
  }
  __syncthreads();
  {
    const int e = threadIdx.x;
    float sum = 0.f;
    if (e < N)
      for (int w = 0; w < RW; ++w) sum += ps[w][e];
    tile_stats(a, e, sum, e < N ? hl[e] : 0, xk, xp);
  }
  if (plan) tile_plan(a, sidx);
}

// Statistics over all router tiles, spread over the experts so that the
// per-tile partials (tiles x N values, 512 KB at 8192 tokens and 128 experts)
// are read by many CUs instead of one.  Workgroup b owns experts se*b ..
// se*b + se - 1 (se = 8 up to 8 experts, so that one workgroup of 1024 threads
// does all, else 4 per workgroup of 256).  Lane l of wave w handles expert
// l % se over tile range (part) w * 64 / se + l / se, summing its p partials
// and counts in increasing tile order; the parts are combined by shuffles
// inside each wave and then wave by wave in order (fixed orders, so the
// result does not depend on timing), and the expert's counts, kept count, p,
// f and f*p are written.  With `base`, the prefix over the parts (a shuffle
// scan inside the wave plus the earlier waves' totals) gives every tile the
// number of assignments to the expert in earlier tiles, from which the
// dispatch copy places each token without a separate plan step.  The last
// workgroup to arrive then scans the kept counts over the experts into
// offsets and sums L_aux.  (Reductions through LDS with a barrier per level
// cost 300-400 cycles a level at 16 waves.)
constexpr int ST = 256;                // threads per statistics workgroup, several workgroups (= kMaxExperts)
constexpr int ST1 = 1024;              // threads of a lone statistics workgroup
constexpr int SKEEP = 16;              // tiles per batch of loads issued together

int stats_experts_per_block(int N) { return N <= 8 ? 8 : 4; }

__global__ __launch_bounds__(ST1) void route_stats_kernel(const float* psum, const int32_t* hist,
                                                         int nb, int64_t T, int N, int k, int cap,
                                                         float alpha, RouteStats rs, int se) {
  int32_t* const counts = rs.counts;
  int32_t* const kept = rs.kept;
  float* const p = rs.p;
  float* const f = rs.f;
  double* const prod = rs.prod;
  int32_t* const base = rs.base;
  static_assert(ST == kMaxExperts && ST1 >= ST, "the last workgroup scans all experts, one per thread");
  __shared__ double wsum[ST1 / 64][8];   // per-wave totals of p and counts, per expert (se <= 8)
  __shared__ int wcnt[ST1 / 64][8];
  __shared__ int wpre[ST1 / 64][8];      // counts of the expert in earlier waves
  __shared__ int xk[ST1 / 64];           // the scan over the experts: per-wave totals
  __shared__ double xp[ST1 / 64];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = static_cast<int>(blockDim.x) >> 6;
  const int pw = 64 / se;                // parts per wave
  const int nparts = nw * pw;
  const int el = lane % se, part = wave * pw + lane / se;
  const int e = blockIdx.x * se + el;
  const bool ex = e < N;
  const int b0 = static_cast<int>(static_cast<int64_t>(part) * nb / nparts);
  const int b1 = static_cast<int>(static_cast<int64_t>(part + 1) * nb / nparts);
  // batches of SKEEP tiles whose loads are issued together; the first
  // batch's counts stay in registers for the tile prefix.  The loads are
  // unconditional (tile and expert clamped into the arrays; such values are
  // then dropped): under a condition the compiler waited for each in turn.
  const int ec = ex ? e : N - 1;
  int hv[SKEEP];
  double s = 0.0;
  int c = 0;
  for (int bb = b0; bb < b1; bb += SKEEP) {
    int hb[SKEEP];
    float pb[SKEEP];
#pragma unroll
    for (int i = 0; i < SKEEP; ++i) {
      const int64_t at = static_cast<int64_t>(min(bb + i, nb - 1)) * N + ec;
      hb[i] = hist[at];
      pb[i] = psum[at];
    }
#pragma unroll
    for (int i = 0; i < SKEEP; ++i) {
      const bool in = ex && bb + i < b1;
      hb[i] = in ? hb[i] : 0;
      pb[i] = in ? pb[i] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < SKEEP; ++i) {
      s += static_cast<double>(pb[i]);
      c += hb[i];
      if (bb == b0) hv[i] = hb[i];
    }
  }
  if (b0 >= b1) {
#pragma unroll
    for (int i = 0; i < SKEEP; ++i) hv[i] = 0;
  }
  // the wave's totals over its parts (lanes of one expert are se apart) and
  // the inclusive prefix of the counts over them
  double ts = s;
  int tc = c, inc = c;
  for (int off = se; off < 64; off <<= 1) {
    ts += __shfl_xor(ts, off);
    tc += __shfl_xor(tc, off);
    const int v = __shfl_up(inc, off);
    if (lane >= off) inc += v;
  }
  if (lane < se) {
    wsum[wave][el] = ts;
    wcnt[wave][el] = tc;
  }
  __syncthreads();
  // wave 0 combines the waves: lane (w, e) holds wave w's totals of expert e,
  // 64 / se waves per pass; a shuffle scan gives each wave's prefix and a
  // butterfly the pass total, the passes added in order (fixed orders)
  int kv = 0;
  double pr = 0.0;
  if (wave == 0) {
    const int per = 64 / se, wl = lane / se;
    double st = 0.0;
    int cnt = 0;
    for (int w0 = 0; w0 < nw; w0 += per) {
      const int w = w0 + wl;
      const double vs = w < nw ? wsum[w][el] : 0.0;
      const int vc = w < nw ? wcnt[w][el] : 0;
      int ic = vc, pc = vc;
      double ps = vs;
      for (int off = se; off < 64; off <<= 1) {
        const int v = __shfl_up(ic, off);
        if (lane >= off) ic += v;
        ps += __shfl_xor(ps, off);
        pc += __shfl_xor(pc, off);
      }
      if (w < nw) wpre[w][el] = cnt + ic - vc;
      st += ps;
      cnt += pc;
    }
    if (lane < se && ex) {                       // (part 0)
      const double pe = st / static_cast<double>(T);
      const double fe = static_cast<double>(cnt) / (static_cast<double>(T) * k);
      counts[e] = cnt;
      kv = cap > 0 ? (cnt < cap ? cnt : cap) : cnt;
      pr = fe * pe;
      kept[e] = kv;
      if (p) p[e] = static_cast<float>(pe);
      if (f) f[e] = static_cast<float>(fe);
      prod[e] = pr;
    }
  }
  __syncthreads();
  if (base && ex) {
    int run = inc - c + wpre[wave][el];          // earlier parts of this wave, then earlier waves
#pragma unroll
    for (int i = 0; i < SKEEP; ++i) {
      if (b0 + i < b1) {
        base[static_cast<int64_t>(b0 + i) * N + e] = run;
        run += hv[i];
      }
    }
    for (int bb = b0 + SKEEP; bb < b1; bb += SKEEP) {
      int hb[SKEEP];
#pragma unroll
      for (int i = 0; i < SKEEP; ++i) hb[i] = hist[static_cast<int64_t>(min(bb + i, nb - 1)) * N + e];
#pragma unroll
      for (int i = 0; i < SKEEP; ++i) {
        if (bb + i < b1) {
          base[static_cast<int64_t>(bb + i) * N + e] = run;
          run += hb[i];
        }
      }
    }
  }
  // The scan over the experts (fixed orders): the exclusive scan of the kept
  // counts into offsets and L_aux = alpha N sum f p.
  if (gridDim.x == 1) {
    // one workgroup, N <= se <= 8: wave 0's lanes e < N already hold expert e
    scan_experts(kv, pr, N, alpha, rs.offsets, rs.l_aux, xk, xp);
    return;
  }
  // Several workgroups: the last to arrive does it.  Each writer's stores are
  // made visible at device scope before its workgroup counts itself, and the
  // last one acquires them; which workgroup is last does not change the result.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(rs.done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
              static_cast<int>(gridDim.x) - 1;
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  kv = tid < N ? __hip_atomic_load(kept + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  pr = tid < N ? __hip_atomic_load(prod + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0;
  scan_experts(kv, pr, N, alpha, rs.offsets, rs.l_aux, xk, xp);
}

// Statistics over few (tiles x experts), in one launch spread over the router
// tiles: every workgroup re-adds the per-tile counts (at most kTileStats
// values, from L2) to get every expert's total and its own tile's base, scans
// the kept counts into the offsets, and, when asked, places its tile's
// assignments (the plan of the fused layer: rank = the tile's base + earlier
// tokens of the tile that chose the expert).  Workgroup 0 also writes the
// totals, kept counts, offsets, f, p and L_aux.  Thread i takes expert
// i % NP and tiles i / NP, i / NP + 256 / NP, ... (NP = N rounded up to a
// power of two), so each step of the loads reads whole rows of the per-tile
// arrays; integer sums are exact in any order, and p's float partials are
// added in double in a fixed order (tile order per thread, then thread order).
constexpr int kTileStats = 16384;      // tiles x experts up to which this kernel replaces the one above
constexpr int STS = 256;               // its threads

struct PlanOut {
  const int32_t* idx;    // null: statistics (and bases) only
  int32_t* pos;
  int32_t* src;
  uint8_t* drop;
};

__global__ __launch_bounds__(STS) void route_stats_tiles_kernel(const float* __restrict__ psum,
                                                               const int32_t* __restrict__ hist, int nb,
                                                               int TM, int64_t T, int N, int k, int cap,
                                                               float alpha, RouteStats rs, PlanOut po) {
  __shared__ int rb[STS], rt[STS];       // per-thread partial base and total
  __shared__ double rp[STS];             // per-thread partial sums of p (workgroup 0)
  __shared__ int ebase[kMaxExperts];     // this tile's base per expert
  __shared__ int eoff[kMaxExperts + 1];  // offsets
  __shared__ int tidx[kRouteTile * kMaxTopK];
  __shared__ int xk[RW];
  __shared__ double xp[RW];
  const int tid = threadIdx.x, b = blockIdx.x;
  int NP = 1;
  while (NP < N) NP <<= 1;
  const int e = tid % NP, q = tid / NP, nq = STS / NP;
  const bool ex = e < N;
  const bool first = b == 0;
  // this tile's entries, loaded early (used by the plan at the end)
  const int64_t t0 = static_cast<int64_t>(b) * TM;
  const int n_tok = static_cast<int>(T - t0 < TM ? T - t0 : TM);
  if (po.idx && tid < n_tok * k) tidx[tid] = po.idx[t0 * k + tid];
  int cb = 0, ct = 0;
  double ps = 0.0;
  if (ex) {
    // (8 rows' loads issued together; rows past nb are clamped and dropped)
    for (int t = q; t < nb; t += 8 * nq) {
      int hv[8];
      float pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int tt = min(t + u * nq, nb - 1);
        hv[u] = hist[static_cast<int64_t>(tt) * N + e];
        pv[u] = first ? psum[static_cast<int64_t>(tt) * N + e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int tt = t + u * nq;
        if (tt < nb) {
          ct += hv[u];
          if (tt < b) cb += hv[u];
          ps += static_cast<double>(pv[u]);
        }
      }
    }
  }
  rb[tid] = cb;
  rt[tid] = ct;
  rp[tid] = ps;
  __syncthreads();
  int kv = 0;
  double pr = 0.0;
  if (tid < N) {
    int sb = 0, st = 0;
    double sp = 0.0;
    for (int j = 0; j < nq; ++j) {
      sb += rb[j * NP + tid];
      st += rt[j * NP + tid];
      sp += rp[j * NP + tid];
    }
    ebase[tid] = sb;
    if (rs.base) rs.base[static_cast<int64_t>(b) * N + tid] = sb;
    kv = cap > 0 ? (st < cap ? st : cap) : st;
    if (first) {
      const double pe = sp / static_cast<double>(T);
      const double fe = static_cast<double>(st) / (static_cast<double>(T) * k);
      rs.counts[tid] = st;
      rs.kept[tid] = kv;
      if (rs.p) rs.p[tid] = static_cast<float>(pe);
      if (rs.f) rs.f[tid] = static_cast<float>(fe);
      pr = fe * pe;
    }
  }
  // the scan over the experts into this workgroup's offsets (and L_aux in workgroup 0)
  scan_experts(kv, pr, N, alpha, eoff, first ? rs.l_aux : nullptr, xk, xp);
  __syncthreads();
  // (N + 1 entries: with N = 256 the last one is past the workgroup's threads)
  if (first && rs.offsets)
    for (int i = tid; i <= N; i += STS) rs.offsets[i] = eoff[i];
  if (!po.idx) return;
  // the plan of this tile: entry a = (token m, slot j), ranked after the
  // earlier tokens' entries for the same expert (a token picks an expert once)
  if (tid < n_tok * k) {
    const int m = tid / k, j = tid - m * k;
    const int ee = tidx[tid];
    int p = -1;
    if (static_cast<unsigned>(ee) < static_cast<unsigned>(N)) {
      int r = ebase[ee];
      for (int a = 0; a < m * k; ++a) r += tidx[a] == ee ? 1 : 0;
      if (cap <= 0 || r < cap) p = eoff[ee] + r;
    }
    const int64_t t = t0 + m;
    po.pos[t * k + j] = p;
    po.drop[t * k + j] = p < 0 ? 1 : 0;
    if (p >= 0) po.src[p] = static_cast<int32_t>(t);
  }
}

}  // namespace

namespace {
// dynamic LDS of route_kernel: the staged x chunks of one phase, at least the
// partials and the logit tile
size_t route_lds_bytes(const moe_shape& s, int TM) {
  const size_t minimum = 16384 + static_cast<size_t>(TM) * (kMaxExperts + 1) * 4;
  size_t staged = 0;
  if (s.dtype == MOE_BF16 && s.d % SCH == 0) {
    const int nch = s.d / SCH;
    staged = static_cast<size_t>(nch < SPH ? nch : SPH) * TM * 1024;
  }
  return staged > minimum ? staged : minimum;
}
}  // namespace

// One router tile (at most 16 tokens) with bf16 x: whole dot products, one
// range (logits_dot_kernel), and the router writes the plan.  Above that and
// below 512 tokens (fewer than 32 router tiles, each of which would read all
// of W_g): d-ranges so that about 1024 waves (one four-wave workgroup per CU)
// stream W_g, at most kLogitsSplitMax, whose every tile re-adds its tokens'
// ranges (DeepSeek-V3 shape, route + plan: 128 tokens 37.9 -> 32.5 us with 8
// ranges instead of 4; 32 tokens measured 27.2 -> 28.2 us with 32 instead of
// 16, so it keeps 16).
bool route_plans(const moe_shape& s) {
  return s.dtype == MOE_BF16 && s.T > 0 && s.T <= kRouteTile && s.d % 8 == 0;
}

int route_split_ranges(const moe_shape& s) {
  if (route_plans(s)) return 1;                  // whole dot products: one range
  if (s.dtype != MOE_BF16 || s.T <= 0 || s.T >= 512 || s.d % 32 != 0) return 0;
  const int64_t units = ceil_div(s.T, 16) * ceil_div(s.N, 16);
  int64_t ks = ceil_div(1024, units);
  if (ks > kLogitsSplitMax) ks = kLogitsSplitMax;
  if (ks > s.d / 32) ks = s.d / 32;
  return static_cast<int>(ks < 1 ? 1 : ks);
}

// 8-token tiles where the logits come from partials (no x staging, no W_g
// re-reads): twice the workgroups, one token per wave, for the selection
// (DeepSeek-V3 shape: route + dispatch 122 -> 119 us).  Where the router
// kernel computes the logits, 16: 8-token tiles there re-read W_g twice as
// often and measured slower (Mixtral shape: router 17.4 -> 19.8 us, although
// two half-size staging buffers then share a CU).  A call with at most 16
// tokens keeps one tile.
int route_tile(const moe_shape& s) {
  if (s.dtype != MOE_BF16 || s.T <= kRouteTile) return kRouteTile;
  const bool partials = router_gemm(s) || route_split_ranges(s) > 0;
  return partials ? kRouteTileMin : kRouteTile;
}

bool route_folds_stats(const moe_shape& s) { return s.T <= kRouteTile; }

hipError_t launch_route(const moe_shape& s, const void* x, const void* wg, const float* bias,
                        int32_t* idx, float* w, float* logits, float* psum, int32_t* hist,
                        float* lpart, const RouteStats& rs, hipStream_t st, const RoutePlanOut* plan) {
  const int ks = route_split_ranges(s);
  const bool planning = plan != nullptr && route_plans(s) && rs.offsets != nullptr;
  if (plan != nullptr && !planning) return hipErrorInvalidValue;
  const bool codes = planning && plan->x_codes != nullptr;
  RouteArgs a{x, wg, bias, idx, w, logits, psum, hist, s.T, s.d, s.N, s.k,
              s.n_groups, s.topk_groups, s.group_score_k, ks > 0 ? lpart : nullptr, ks,
              s.T * s.N, s.N, nullptr, s.gate, rs, route_folds_stats(s) ? 1 : 0, s.capacity, s.alpha,
              planning ? plan->pos : nullptr, planning ? plan->src : nullptr,
              planning ? plan->drop : nullptr, codes ? plan->row_scale : nullptr,
              codes ? plan->tscale : nullptr};
  if (route_plans(s)) {
    // tokens per wave: the waves split 4 ways over tokens (T >= 4), else 2 or 1 way
    const int T = static_cast<int>(s.T);
    const int groups = T >= 4 ? 4 : (T >= 2 ? 2 : 1);
    const int tpw = (T + groups - 1) / groups;
    const auto xs = static_cast<const uint16_t*>(x);
    const auto ws = static_cast<const uint16_t*>(wg);
    uint8_t* xc = codes ? plan->x_codes : nullptr;
    float* ts = codes ? plan->tscale : nullptr;
    const dim3 grid(static_cast<unsigned>(s.N));
    if (tpw <= 1)
      hipLaunchKernelGGL(logits_dot_kernel<1>, grid, dim3(256), 0, st, xs, ws, lpart, T, s.d, s.N, xc, ts);
    else if (tpw <= 2)
      hipLaunchKernelGGL(logits_dot_kernel<2>, grid, dim3(256), 0, st, xs, ws, lpart, T, s.d, s.N, xc, ts);
    else
      hipLaunchKernelGGL(logits_dot_kernel<4>, grid, dim3(256), 0, st, xs, ws, lpart, T, s.d, s.N, xc, ts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (router_gemm(s)) {
    const hipError_t e = launch_router_logits(s, x, wg, lpart, st);
    if (e != hipSuccess) return e;
    a.lmeta = reinterpret_cast<const int32_t*>(lpart);
    a.lpart = reinterpret_cast<const float*>(reinterpret_cast<const char*>(lpart) + kSplitMetaBytes);
    a.lld = kRouterTileCols;
  } else if (ks > 0) {
    const int64_t units = ceil_div(s.T, 16) * ceil_div(s.N, 16) * ks;
    hipLaunchKernelGGL(logits_split_kernel, dim3(static_cast<unsigned>(ceil_div(units, 4))), dim3(256), 0,
                       st, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), lpart, s.T,
                       s.d, s.N, ks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int tm = route_tile(s);
  dim3 grid(static_cast<unsigned>(ceil_div(s.T, tm)));
  const size_t lds = route_lds_bytes(s, tm);
  // allow dynamic LDS above the default limit (the largest staging buffer)
  static const bool attr_set = [] {
    const int most = SPH * kRouteTile * 1024;
    auto set = [&](const void* f) {
      return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, most) == hipSuccess;
    };
    return set(reinterpret_cast<const void*>(route_kernel<true, kRouteTile>)) &&
           set(reinterpret_cast<const void*>(route_kernel<true, kRouteTileMin>)) &&
           set(reinterpret_cast<const void*>(route_kernel<false, kRouteTile>));
  }();
  if (!attr_set) return hipErrorInvalidValue;
  if (s.dtype != MOE_BF16)
    hipLaunchKernelGGL((route_kernel<false, kRouteTile>), grid, dim3(RW * 64), lds, st, a);
  else if (tm == kRouteTileMin)
    hipLaunchKernelGGL((route_kernel<true, kRouteTileMin>), grid, dim3(RW * 64), lds, st, a);
  else
    hipLaunchKernelGGL((route_kernel<true, kRouteTile>), grid, dim3(RW * 64), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_route_finalize(const moe_shape& s, const float* psum, const int32_t* hist,
                                 const RouteStats& rs, hipStream_t st, const int32_t* idx,
                                 int32_t* pos, int32_t* src, uint8_t* drop, bool* planned) {
  const int nb = static_cast<int>(ceil_div(s.T, route_tile(s)));
  if (planned) *planned = false;
  if (static_cast<int64_t>(nb) * s.N <= kTileStats) {
    const bool plan = idx && pos && src && drop;
    const PlanOut po{plan ? idx : nullptr, pos, src, drop};
    hipLaunchKernelGGL(route_stats_tiles_kernel, dim3(nb), dim3(STS), 0, st, psum, hist, nb,
                       route_tile(s), s.T, s.N, s.k, s.capacity, s.alpha, rs, po);
    if (planned) *planned = plan;
    return hipGetLastError();
  }
  const int se = stats_experts_per_block(s.N);
  const int blocks = static_cast<int>(ceil_div(s.N, se));
  hipLaunchKernelGGL(route_stats_kernel, dim3(blocks), dim3(blocks == 1 ? ST1 : ST), 0, st,
                     psum, hist, nb, s.T, s.N, s.k, s.capacity, s.alpha, rs, se);
  return hipGetLastError();
}

}  // namespace moe
