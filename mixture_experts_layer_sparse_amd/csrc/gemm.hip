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
//     never reads the routing) times n-tiles, expert-major and n-tile-major, so
//     that an expert's m-tiles consume each weight n-tile back to back; each XCD
//     owns runs of consecutive tile ids, so the tiles running together on one
//     XCD reuse the same weight and activation tiles from that XCD's L2;
//   * 8 waves (two per SIMD) in a WGM x WGN grid, each computing a block of
//     the tile with v_mfma_f32_32x32x16_bf16, float32 accumulation; a wave whose
//     rows all lie past the segment end skips its MFMAs;
//   * K is streamed in 64-wide steps through two LDS stages, by one of two
//     pipelines: (a) buffer loads straight into LDS (buffer_load ... lds),
//     double-buffered fragments, and the loads of step kt + 2 issued one per
//     MFMA right after the barrier that frees their stage; (b) buffer loads
//     into registers holding the next two steps, written to the free stage
//     halfway through each step (more bytes in flight).  (a) is faster on the
//     256-row tiles, (b) on the weight-streaming 128-row tiles;
//     the 16-byte chunks of each LDS row are XOR-swizzled by the row index so
//     that fragment reads are free of bank conflicts;
//   * fp8 activations (e4m3 codes) stay fp8 in LDS and are widened to bf16
//     exactly as fragments are read; the per-row scale multiplies the float32
//     accumulator;
//   * MXFP4 weights are widened to bf16 as they are written to LDS, except
//     with fp8 activations: then both operands stay in their codes and the
//     scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) applies the block scales;
//   * SwiGLU: the B tile interleaves W1 and W3 rows of the same output columns
//     so that each wave holds both halves of its outputs; the activation runs
//     on the accumulators and h is written once, in bf16.
// The float32 path (small correctness shapes) is a plain dot-product kernel.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "moe_internal.h"

// register buffers of staged loads: K steps in flight beyond the LDS stages (bf16
// and MXFP4 weights); 3 and 4 measured no faster than 2 on any shape
#ifndef MOE_GEMM_RBUF
#define MOE_GEMM_RBUF 2
#endif
#ifndef MOE_GEMM_RBUF_MX
#define MOE_GEMM_RBUF_MX 2
#endif
// 1: each XCD owns runs of consecutive tile ids; 0: tile id = round * grid + block
#ifndef MOE_GEMM_XCD_MAP
#define MOE_GEMM_XCD_MAP 1
#endif

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

enum Epi { EPI_STORE = 0, EPI_SILU = 1, EPI_RELU = 2, EPI_SWIGLU = 3 };

struct GemmArgs {
  const void* a;           // [rows][K] bf16 bits, or e4m3 codes; with `gather`, [a_total][K]
  const float* a_scale;    // [rows] per-row scale (fp8 A) or null
  const int32_t* gather;   // null, or [rows]: row r of the product reads A row gather[r]
  int64_t a_total;         // rows of A when gathering
  const int32_t* offsets;  // [n_seg + 1], or null: one dense segment of `rows`
  int64_t rows;
  int n_seg;
  int K;
  int n_out;               // output columns (F for up, d for down)
  const uint16_t* b0;      // [n_seg][n_out][K]  (W1 or W2)
  const uint16_t* b1;      // [n_seg][n_out][K]  (W3, SwiGLU only)
  int64_t b_stride;        // n_out * K (elements); MXFP4 B: bytes of one matrix (codes, then scales)
  int64_t mx_scale_off;    // MXFP4 B: byte offset of the scales within a matrix (n_out * K / 2)
  uint16_t* out;           // [rows][n_out]
  int nt;                  // n-tiles of the tile list
  int split_slots;         // > 0: tail split over this many workgroup slots (see below)
  float* part;             // split-K tail: [units][256][256] float32 partial tiles
  int32_t* part_meta;      // split-K tail: [0] = tail tiles, then (row0, row_end, ntile) per tile
  int split_k_max;         // > 0: the tail is split along K (up to this many ranges per tile)
  // An extra dense segment after the routed ones (the shared expert's down GEMM
  // in the launch of the routed one): A [x_rows][K] at xa, B one matrix at xb0
  // (laid out as one of b0's), output [x_rows][n_out] at xout.  No gather, no
  // row scale, no gated epilogue.
  const void* xa;
  const uint16_t* xb0;
  uint16_t* xout;
  int64_t x_rows;          // 0: none
  // Combining epilogue (EPI_STORE, not split-K; sc_cnt null: off): after a tile
  // has written its output rows it counts them per token and kScatterCols-column
  // group, and the tile that completes a group writes those columns of y.
  const int32_t* sc_src;   // [rows] token of each routed row (the extra segment's row r is token r)
  const int32_t* sc_pos;   // [T][k]
  const float* sc_w;       // [T][k]
  const uint16_t* sc_x;    // [T][n_out]
  uint16_t* sc_y;          // [T][n_out]
  int32_t* sc_cnt;         // [T][ceil(n_out / kScatterCols)], set by launch_scatter_init
  int sc_k;
  int sc_drop;
};

// silu(u) = u / (1 + e^-u) with the hardware reciprocal (about 1 ulp): the result is rounded to
// bf16 (8 significant bits) right after, so the exact quotient buys nothing
__device__ __forceinline__ float silu_fast(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}
// float32 -> bf16 bits, round to nearest even (the gfx950 conversion instruction)
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from a buffer into registers (reads past the end return zero).
// Kept in a device function: the host compilation pass only needs the kernel stub.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
}

// 16 bytes per lane from a buffer straight into LDS (lane i writes lds + 16 * i).
typedef __attribute__((address_space(3))) void* lds_ptr;
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff,
                                          uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)lds, 16, voff, soff, 0, 0);
}

// 4 bytes per lane from a buffer straight into LDS (lane i writes lds + 4 * i).
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff,
                                         uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)lds, 4, voff, soff, 0, 0);
}

// s_waitcnt on the LDS counter only (lgkmcnt = 0), leaving vector loads in flight.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// s_waitcnt on the vector-memory counter only (vmcnt = 0).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }



// Scheduling pattern for the machine scheduler: for q = 0 .. NMM - 1, one MFMA
// followed by the vector-memory loads that fall to it when LPW loads are spread
// evenly over NMM MFMAs.
template <int CNT>
__device__ __forceinline__ void sched_mfma_then_loads() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
  if constexpr (CNT > 0) __builtin_amdgcn_sched_group_barrier(0x020, CNT, 0);   // VMEM read
}
template <int NMM, int LPW, int... Q>
__device__ __forceinline__ void sched_mfma_loads(std::integer_sequence<int, Q...>) {
  (sched_mfma_then_loads<(Q + 1) * LPW / NMM - Q * LPW / NMM>(), ...);
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), unrolled.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// f(integral_constant<int, min(n, N)>) for a wave-uniform 0 <= n: one code
// path per count of live 32-row blocks.
template <int N, typename F>
__device__ __forceinline__ void with_blocks(int n, F&& f) {
  if constexpr (N == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (n >= N) f(std::integral_constant<int, N>{});
    else with_blocks<N - 1>(n, f);
  }
}

// Buffer resource over [base, base + bytes): loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(n), 0x00020000);
}

// LDS holds 64 banks of 4 bytes and a 16-byte-per-lane read is served 16 lanes
// (256 bytes) at a time.  Fragment reads hit 16 consecutive rows at the same
// logical 16-byte chunk, so the chunk is XOR-swizzled by the row: with RB-byte
// rows, 256/RB rows share one 256-byte bank line (the row's place in the line
// picks the bank group) and (row / (256/RB)) % (RB/16) picks the chunk.
template <int RB>
__device__ __forceinline__ int swz(int row) {
  return (row / (256 / RB)) % (RB / 16);
}

// Tail split.  With split_slots = S > 0 the tile list (m-tiles of height MBM,
// n-tiles of g.nt) is cut at total - r, r = total % S, when 0 < r <= S / 4: the
// main launch (TAIL = false, tile BM x BN = MBM x BN) runs the tiles before the
// cut, whole rounds of S workgroups; the tail launch (TAIL = true, tile of half
// height and half width) runs each of the r remaining tiles as four quarters,
// so that the last round is not left mostly idle.  A quarter streams twice
// the bytes per FLOP of a whole tile and runs at about half its rate, so the
// split pays only while all quarters fit in one round (4 r <= S).  When the
// caller provides scratch (part), the tail launch instead splits each of the r
// tiles along K into ksplit = min(split_k_max, S / r) ranges (SPLITK = true,
// whole 256x256 tiles, so at the main kernel's rate), and when the whole list has at most S / 2 tiles
// (a decode step, a small dense call) every tile goes to the tail, split into
// min(split_k_max, S / tiles) ranges, so that all CUs stream its weights.  The
// float32 partial tiles are then added in range order by gg_splitk_reduce,
// which applies the epilogue.  The launches count the same tile list from
// `offsets`; without split-K every output element is computed by one workgroup
// over the whole K.
//
// MX: B (the weights) is MXFP4: per matrix [n_out][K], FP4 E2M1 codes (two per
// byte, element 2i in the low nibble) then one E8M0 scale per 32 elements of
// a row.  Register-staged pipeline only: each wave loads 32 rows x 64 K of
// codes (16 bytes per lane, one 32-element block) and the block's scale, and
// widens them exactly to bf16 (v_cvt_scalef32_pk_bf16_fp4) as it writes the
// stage, so the LDS tile and the MFMA loop are those of a bf16 B.
//
// MXS (MXFP4 B with fp8 A, K a multiple of 128): no widening at all.  The
// stage holds the e4m3 codes of A, the FP4 codes of B and B's E8M0 scales as
// they are in memory, and v_mfma_scale_f32_32x32x64_f8f6f4 multiplies them
// (A scale 1, the per-row scale on the accumulator as for every fp8 A).  In
// that instruction a lane of the B operand holds 32 consecutive K (one MX
// block, with its scale) and the lane half h of column n holds K 32h ..
// 32h + 31 of the 64; the A lane half h holds K 16h .. 16h + 15 in its first
// 16 bytes and K 32 + 16h .. 32 + 16h + 15 in the next 16.  Register-staged,
// a step is 128 K (two MFMA slices); on the LDS-DMA pipeline (K a multiple of
// 256) a step is 256 K, four MFMA slices as in the bf16 pipeline, the codes
// and scales landing in LDS straight from memory (the scales by 4-byte loads,
// one wave-load per 32 B rows).
template <int BM, int BN, int WGM, int WGN, int EPI, bool FP8A, bool REG, bool TAIL, bool SPLITK,
          bool MX = false, bool MXS = false>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gg_kernel(GemmArgs g) {
  static_assert(!SPLITK || TAIL, "split-K is a tail mode");
  static_assert(!MX || ((REG || MXS) && BN == 32 * WGM * WGN), "MXFP4 B: 32 B rows per wave");
  static_assert(!MXS || (MX && FP8A), "scaled MFMA: fp8 A, MXFP4 B");
  constexpr bool MXD = MXS && !REG;                // scaled MFMA on the LDS-DMA pipeline
  constexpr int NW = WGM * WGN;                    // waves; WGM x WGN grid of wave tiles
  constexpr int BK = MXS ? (REG ? 128 : 256) : 64;
  constexpr int SA = FP8A ? 1 : 2;                 // bytes per A element
  constexpr int ROWA = BK * SA;                    // bytes per tile row per stage: A,
  constexpr int ROWB = MXS ? BK / 2 : BK * 2;      // B (FP4 codes with MXS, else bf16)
  constexpr int A_BYTES = BM * ROWA, B_BYTES = BN * ROWB;
  constexpr int SCR = BK / 32;                     // MXS: B's block scales per row and step
  constexpr int SC_BYTES = MXS ? BN * SCR : 0;
  constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
  constexpr int A_PW = A_BYTES / 1024 / NW;        // 1 KB wave-loads per wave per stage
  constexpr int B_PW = B_BYTES / 1024 / NW;
  constexpr int B_PWS = B_PW + (MXD ? 1 : 0);      // B pieces with MXD's scale load
  constexpr int LPW = A_PW + B_PWS;                // loads per wave per stage
  constexpr int KB_STEP = MXS ? BK / 2 : BK * 2;   // B bytes per row and step
  // LDS-DMA loads of one step in two bursts: B (weights) right after the step
  // barrier, A in the first K slice of the next step (see fstep).  Only for
  // the gate/up GEMMs, whose A (the dispatch buffer) every n-tile re-reads, so
  // it comes from the caches and needs less time in flight; the down GEMM's A
  // (h) streams, and there the later A loads measured slower.
  constexpr bool SPLIT_AB = !REG && EPI != EPI_STORE;
  constexpr int A_CPR = ROWA / 16, B_CPR = ROWB / 16;   // 16-byte chunks per row
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TMI = WM / 32, TNI = WN / 32;
  constexpr bool GATED = EPI == EPI_SWIGLU;
  static_assert(!GATED || (TNI % 2 == 0), "gated tile needs an even number of n-subtiles");
  static_assert(A_PW >= 1 && B_PW >= 1, "tile too small for the load split");
  static_assert(A_PW * NW * 1024 == A_BYTES && B_PW * NW * 1024 == B_BYTES, "load split");
  static_assert(!GATED || (WN / 2) % (1024 / ROWB) == 0, "a wave-load must not straddle W1 and W3");
  static_assert(2 * STAGE <= 144 * 1024, "LDS budget");
  static_assert(!MXD || BN * SCR == NW * 256, "MXD: one 4-byte wave-load of scales per wave");

  // two LDS stages, each its own array: step kt computes from one while step
  // kt + 1 is written to the other
  __shared__ __attribute__((aligned(1024))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sm1[STAGE];
  __shared__ int mt_start[kMaxExperts + 2];
  __shared__ int seg_off[kMaxExperts + 2];
  __shared__ int scan_tmp[2][kMaxExperts + 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave / WGN, wn = wave % WGN;
  const int n_seg = g.offsets ? g.n_seg : 1;
  const int K = g.K, KT = K / BK;
  constexpr bool QUARTERS = TAIL && !SPLITK;
  constexpr int MBM = QUARTERS ? 2 * BM : BM;    // m-tile height of the tile list

  // m-tiles per segment and their exclusive scan (segments <= 256)
  {
    int ntile = 0;
    if (tid < n_seg) {
      // (segment bounds clamped into [0, rows]: valid offsets pass unchanged,
      // and no other value can index past the row buffers)
      const int rows_i = static_cast<int>(g.rows);
      const int so = g.offsets ? min(max(g.offsets[tid], 0), rows_i) : 0;
      const int eo = g.offsets ? min(max(g.offsets[tid + 1], so), rows_i) : rows_i;
      ntile = (eo - so + MBM - 1) / MBM;
      seg_off[tid] = so;
      if (tid == n_seg - 1) seg_off[n_seg] = eo;
    }
    if (tid < 256) scan_tmp[0][tid] = ntile;
    __syncthreads();
    int cur = 0;
#pragma unroll
    for (int off = 1; off < 256; off <<= 1) {
      if (tid < 256)
        scan_tmp[cur ^ 1][tid] = scan_tmp[cur][tid] + (tid >= off ? scan_tmp[cur][tid - off] : 0);
      cur ^= 1;
      __syncthreads();
    }
    if (tid == 0) mt_start[0] = 0;
    if (tid < n_seg) mt_start[tid + 1] = scan_tmp[cur][tid];
    // the extra segment's m-tiles after the routed ones
    if (tid == n_seg - 1) mt_start[n_seg + 1] = scan_tmp[cur][tid] + static_cast<int>((g.x_rows + MBM - 1) / MBM);
    __syncthreads();
  }
  const int n_all = n_seg + (g.x_rows > 0 ? 1 : 0);  // segments, the extra one included
  const int MT = __builtin_amdgcn_readfirstlane(mt_start[n_all]);
  const int NT = g.nt;
  const int total = MT * NT;
  int cut = total;                               // main tiles [0, cut), tail tiles [cut, total)
  int ksplit = 1;                                // K ranges per tail tile (split-K tail)
  if (g.split_slots > 0 && total > 0) {
    const int S_ = g.split_slots;
    if (g.split_k_max > 0 && 2 * total <= S_) {
      // few tiles (a decode step, a small dense call): all of them split
      cut = 0;
      ksplit = S_ / total < g.split_k_max ? S_ / total : g.split_k_max;
    } else if (!REG && !MX) {
      // (MXFP4 kernels make no cut: their split-K tail launch is register-staged)
      const int r = total % S_;
      if (r > 0 && 4 * r <= S_) {
        cut = total - r;
        // with split-K, as many K ranges as fill the S slots (Mixtral-shaped
        // down GEMM, r = 48: 5 ranges, 0.847 -> 0.840 ms)
        if (g.split_k_max > 0) ksplit = S_ / r < g.split_k_max ? S_ / r : g.split_k_max;
      }
    }
  }
  const int items = TAIL ? (SPLITK ? ksplit : 4) * (total - cut) : cut;
  if (SPLITK && blockIdx.x == 0 && tid == 0) {
    g.part_meta[0] = total - cut;
    g.part_meta[1] = ksplit;
  }
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, S = gridDim.x >> 3;

  // segment of tile-list entry Lm: mt_start[e] * NT <= Lm < mt_start[e + 1] * NT
  auto seg_of_tile = [&](int Lm) {
    int lo = 0, hi = n_all;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (mt_start[mid] * NT <= Lm) lo = mid; else hi = mid;
    }
    return __builtin_amdgcn_readfirstlane(lo);
  };
  // per-lane LDS fragment offsets (rows i*32 + lane%32 share the swizzle)
  const int fr = lane & 31, fk = lane >> 5;

  // per-lane source offsets of this wave's A loads (the K step is added as
  // soffset): relative to the tile's first row, so the same for every tile,
  // or, when gathering, from the base of A through the tile's row indices
  // (set by bind_tile)
  uint32_t a_off[A_PW];
#pragma unroll
  for (int j = 0; j < A_PW; ++j) {
    const int r = (wave * A_PW + j) * (1024 / ROWA) + lane / A_CPR;
    const int c = (lane % A_CPR) ^ swz<ROWA>(r);
    a_off[j] = static_cast<uint32_t>(r * K * SA + c * 16);
  }
  const bool gather = g.gather != nullptr;

  // The current tile (wave-uniform values).  Tile order: expert-major, then
  // n-tile, then the expert's m-tiles, so the m-tiles of an expert consume
  // each weight n-tile back to back (one HBM read, the rest from L2); each XCD
  // takes S consecutive tile ids per round.
  int round = -1, row0 = 0, row_end = 0, ntile = 0, e = 0;
  bool xseg = false;                             // the current tile is the extra segment's
  int kbeg = 0, kend = KT, unit = 0;             // K steps of the current tile (a range for split-K)
  auto next_tile = [&]() -> bool {
    for (;;) {
      ++round;
      const int L = MOE_GEMM_XCD_MAP ? (round * 8 + xcd) * S + slot
                                     : round * static_cast<int>(gridDim.x) + static_cast<int>(blockIdx.x);
      if (L >= items) return false;
      // tile of the list (quarter L & 3, or K range L / r, in the tail; the
      // split-K units are range-major, so that the units running together on
      // an XCD share A and B ranges through its L2 as whole tiles do)
      const int Lm = TAIL ? cut + (SPLITK ? L % (total - cut) : (L >> 2)) : L;
      // values read from LDS are the same in every lane: make that explicit so
      // that the buffer descriptors live in scalar registers
      e = seg_of_tile(Lm);
      const int mte = __builtin_amdgcn_readfirstlane(mt_start[e + 1] - mt_start[e]);
      const int local = Lm - __builtin_amdgcn_readfirstlane(mt_start[e]) * NT;
      const int nt_list = local / mte;
      const int mloc = local - nt_list * mte;
      xseg = e == n_seg;
      // (the extra segment's rows count from 0 in its own buffers)
      row0 = (xseg ? 0 : __builtin_amdgcn_readfirstlane(seg_off[e])) + mloc * MBM +
             (QUARTERS ? ((L >> 1) & 1) * BM : 0);
      row_end = xseg ? static_cast<int>(g.x_rows) : __builtin_amdgcn_readfirstlane(seg_off[e + 1]);
      ntile = QUARTERS ? 2 * nt_list + (L & 1) : nt_list;
      // a tail quarter wholly past the segment end or the last column has no work
      if (QUARTERS && (row0 >= row_end || ntile * (GATED ? BN / 2 : BN) >= g.n_out)) continue;
      if (SPLITK) {
        const int sp = L / (total - cut);
        kbeg = sp * KT / ksplit;
        kend = (sp + 1) * KT / ksplit;
        unit = L;
        if (sp == 0 && tid == 0) {
          int32_t* m = g.part_meta + 2 + 3 * (Lm - cut);
          m[0] = row0;
          m[1] = row_end;
          m[2] = ntile | (xseg ? (1 << 30) : 0);
        }
      }
      return true;
    }
  };

  // buffer resources of the current tile: A from its first row (reads past
  // the buffer return zero), B per expert matrix; per-lane B offsets
  __amdgpu_buffer_rsrc_t rsB0 = make_rsrc(g.b0, 0), rsB1 = rsB0;
  uint32_t b_off[B_PW];
  uint32_t mx_code = 0, mx_scale = 0;            // MXFP4 B: this lane's code and scale offsets (K step 0)
  // gated: B tile row n interleaves W1 and W3 rows in runs of WN / 2; the weight row it holds
  auto b_row = [&](int n) {
    if (GATED) {
      const int wn_ = n / WN, q = n % WN, half = WN / 2;
      return ntile * (BN / 2) + wn_ * half + (q % half);
    }
    return ntile * BN + n;
  };
  bool wave_rows = false;                        // a wave whose rows all lie past the segment end skips its MFMAs
  int wave_blocks = TMI;                         // 32-row blocks of the wave's rows inside the segment
  int a_rows = 0;                                // rows of the tile inside its segment
  const uint8_t* a_tile = static_cast<const uint8_t*>(g.a);
  uint32_t a_nrec = 0;
  // Loads of A rows past the segment end go through a descriptor with no
  // records (every lane out of range: zeros, no memory access), so a
  // segment's partial last m-tile moves only the A bytes it uses.  The
  // choice is uniform per load and is made on the record count, a scalar:
  // choosing between two whole descriptors puts them in a stack array.
  const __amdgpu_buffer_rsrc_t rs_null = make_rsrc(g.b0, 0);
  auto rs_a = [&](int j, bool live = true) {
    const bool in = live && (wave * A_PW + j) * (1024 / ROWA) < a_rows;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a_tile), static_cast<short>(0),
                                             static_cast<int>(in ? a_nrec : 0u), 0x00020000);
  };
  // The register-staged path reads whole tiles: there, skipping the rows past
  // the segment end measured about 12% slower at 128-row segments.
  __amdgpu_buffer_rsrc_t rs_a_whole = rs_null;
  auto bind_tile = [&]() {
    uint64_t a_bytes;
    if (gather) {
      // A rows of the tile through the row indices (rows past the segment end
      // read row 0: loaded, never stored); the host keeps a_total * K * SA
      // within the 32-bit range of the offsets
      a_tile = static_cast<const uint8_t*>(g.a);
      a_bytes = static_cast<uint64_t>(g.a_total) * K * SA;
      int tok[A_PW];
#pragma unroll
      for (int j = 0; j < A_PW; ++j) {
        const int r = (wave * A_PW + j) * (1024 / ROWA) + lane / A_CPR;
        tok[j] = g.gather[min(row0 + r, row_end - 1)];      // (loads issued together)
      }
#pragma unroll
      for (int j = 0; j < A_PW; ++j) {
        const int r = (wave * A_PW + j) * (1024 / ROWA) + lane / A_CPR;
        const int c = (lane % A_CPR) ^ swz<ROWA>(r);
        const int t = row0 + r < row_end ? tok[j] : 0;
        a_off[j] = static_cast<uint32_t>(t) * static_cast<uint32_t>(K * SA) + static_cast<uint32_t>(c * 16);
      }
    } else {
      a_tile = static_cast<const uint8_t*>(xseg ? g.xa : g.a) + static_cast<int64_t>(row0) * K * SA;
      a_bytes = static_cast<uint64_t>((xseg ? g.x_rows : g.rows) - row0) * K * SA;
    }
    a_nrec = a_bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(a_bytes);
    if constexpr (MX) {
      // lane: row n = wave * 32 + lane / 2 of the B tile, the half (32 elements
      // of the step's 64) lane % 2; the tile's rows interleave W1 and W3 in
      // runs of WN / 2 >= 32 (gated), so a wave's rows come from one matrix
      const uint8_t* m0 = xseg ? reinterpret_cast<const uint8_t*>(g.xb0)
                               : reinterpret_cast<const uint8_t*>(g.b0) + e * g.b_stride;
      const uint8_t* m1 = GATED ? reinterpret_cast<const uint8_t*>(g.b1) + e * g.b_stride : m0;
      rsB0 = make_rsrc(m0, static_cast<uint64_t>(g.b_stride));
      rsB1 = GATED ? make_rsrc(m1, static_cast<uint64_t>(g.b_stride)) : rsB0;
      if constexpr (MXD) {
        // codes: as a bf16 B's wave-loads, 8 rows of 128 bytes per 1 KB; scales:
        // row wave * 32 + lane / 2, the step's 8 bytes as two words
#pragma unroll
        for (int j = 0; j < B_PW; ++j) {
          const int n = (wave * B_PW + j) * (1024 / ROWB) + lane / B_CPR;
          const int c = (lane % B_CPR) ^ swz<ROWB>(n);
          b_off[j] = static_cast<uint32_t>(b_row(n)) * static_cast<uint32_t>(K / 2) + static_cast<uint32_t>(c * 16);
        }
        mx_scale = static_cast<uint32_t>(g.mx_scale_off) +
                   static_cast<uint32_t>(b_row(wave * 32 + (lane >> 1))) * static_cast<uint32_t>(K / 32) + (lane & 1) * 4;
      } else if constexpr (MXS) {
        // codes: rows wave * 32 + 16 j + lane / 4, 16-byte chunk lane % 4 of the
        // step's 64 bytes (piece j adds 16 weight rows, as the soffset); scales:
        // lane % 32's row, the step's 4 bytes as one word
        const int fc = b_row(wave * 32 + (lane >> 2)), fs = b_row(wave * 32 + (lane & 31));
        mx_code = static_cast<uint32_t>(fc) * static_cast<uint32_t>(K / 2) + (lane & 3) * 16;
        mx_scale = static_cast<uint32_t>(g.mx_scale_off) + static_cast<uint32_t>(fs) * static_cast<uint32_t>(K / 32);
      } else {
        const int f = b_row(wave * 32 + (lane >> 1));
        mx_code = static_cast<uint32_t>(f) * static_cast<uint32_t>(K / 2) + (lane & 1) * 16;
        mx_scale = static_cast<uint32_t>(g.mx_scale_off) + static_cast<uint32_t>(f) * static_cast<uint32_t>(K / 32) +
                   (lane & 1);
      }
    } else {
    const uint64_t b_bytes = static_cast<uint64_t>(g.n_out) * K * 2;
    rsB0 = make_rsrc(xseg ? g.xb0 : g.b0 + e * g.b_stride, b_bytes);
    rsB1 = GATED ? make_rsrc(g.b1 + e * g.b_stride, b_bytes) : rsB0;
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
      const int n = (wave * B_PW + j) * (1024 / ROWB) + lane / B_CPR;
      const int c = (lane % B_CPR) ^ swz<ROWB>(n);
      b_off[j] = static_cast<uint32_t>((b_row(n) * K) * 2 + c * 16);
    }
    }
    wave_rows = row0 + wm * WM < row_end;
    a_rows = __builtin_amdgcn_readfirstlane(row_end - row0);
    rs_a_whole = make_rsrc(a_tile, a_bytes);
    const int live = a_rows - wm * WM;
    wave_blocks = live <= 0 ? 0 : (live >= TMI * 32 ? TMI : (live + 31) >> 5);
  };

  f32x16 acc[TMI][TNI];

  // K steps of this wave's loads, staged in registers: A_PW + B_PW pieces of
  // 16 bytes per lane, each landing at lane * 16 of its 1 KB block in LDS.
  // RB register buffers keep RB steps of loads in flight.
  constexpr int RB = REG ? (MX ? MOE_GEMM_RBUF_MX : MOE_GEMM_RBUF) : 1;
  static_assert(RB >= 1 && RB <= 4, "register buffers");
  u32x4 ra[RB][A_PW], rb[RB][MX && !MXS ? 1 : B_PW];
  uint32_t rsc[RB];                              // MXFP4 B: the lane's block scale(s) (E8M0)
  auto load_regs = [&](int kt, auto Q) {
    constexpr int q = decltype(Q)::value;
    const uint32_t ka = static_cast<uint32_t>(kt * BK * SA), kb = static_cast<uint32_t>(kt * BK * 2);
#pragma unroll
    for (int j = 0; j < A_PW; ++j) ra[q][j] = buf_load16(rs_a_whole, a_off[j], ka);
    if constexpr (MXS) {
      const bool w3 = GATED && ((wave * 32) % WN) >= WN / 2;
      const __amdgpu_buffer_rsrc_t r = w3 ? rsB1 : rsB0;
#pragma unroll
      for (int j = 0; j < B_PW; ++j)
        rb[q][j] = buf_load16(r, mx_code, static_cast<uint32_t>(kt * (BK / 2) + j * 16 * (K / 2)));
      rsc[q] = __builtin_amdgcn_raw_buffer_load_b32(r, mx_scale, static_cast<uint32_t>(kt * (BK / 32)), 0);
    } else if constexpr (MX) {
      // gated: the wave's 32 rows are W1 rows in the first half of each WN-wide column group
      const bool w3 = GATED && ((wave * 32) % WN) >= WN / 2;
      const __amdgpu_buffer_rsrc_t r = w3 ? rsB1 : rsB0;
      rb[q][0] = buf_load16(r, mx_code, static_cast<uint32_t>(kt * (BK / 2)));
      rsc[q] = __builtin_amdgcn_raw_buffer_load_b8(r, mx_scale, static_cast<uint32_t>(kt * (BK / 32)), 0);
    } else {
#pragma unroll
      for (int j = 0; j < B_PW; ++j) {
        const int gi = wave * B_PW + j;
        // gated: B rows q < WN/2 of each wave column group come from W1, the rest from W3
        const bool w3 = GATED && ((gi * (1024 / ROWB)) % WN) >= WN / 2;
        rb[q][j] = buf_load16(w3 ? rsB1 : rsB0, b_off[j], kb);
      }
    }
  };
  auto store_regs = [&](uint8_t* stg, auto Q) {
    constexpr int q = decltype(Q)::value;
#pragma unroll
    for (int j = 0; j < A_PW; ++j)
      *reinterpret_cast<u32x4*>(stg + (wave * A_PW + j) * 1024 + lane * 16) = ra[q][j];
    if constexpr (MXS) {
      // codes as loaded (row n, chunk lane % 4, swizzled), the scale word of row wave * 32 + lane
#pragma unroll
      for (int j = 0; j < B_PW; ++j) {
        const int n = wave * 32 + j * 16 + (lane >> 2);
        *reinterpret_cast<u32x4*>(stg + A_BYTES + n * ROWB + (((lane & 3) ^ swz<ROWB>(n)) << 4)) = rb[q][j];
      }
      if (lane < 32) *reinterpret_cast<uint32_t*>(stg + A_BYTES + B_BYTES + (wave * 32 + lane) * SCR) = rsc[q];
    } else if constexpr (MX) {
      // 32 codes -> 32 bf16 (4 chunks of 16 bytes) at row n, chunks 4 * (lane % 2) ..,
      // swizzled like every bf16 B row; scale 2^(e - 127) (e = 0: 2^-127)
      const int n = wave * 32 + (lane >> 1);
      const uint32_t e8 = rsc[q] & 0xFFu;
      const float sf = __uint_as_float(e8 == 0 ? 0x00400000u : (e8 << 23));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = rb[q][0][i];
        u32x4 o;
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 0));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 1));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 2));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 3));
        const int c = (lane & 1) * 4 + i;
        *reinterpret_cast<u32x4*>(stg + A_BYTES + n * ROWB + ((c ^ swz<ROWB>(n)) << 4)) = o;
      }
    } else {
#pragma unroll
      for (int j = 0; j < B_PW; ++j)
        *reinterpret_cast<u32x4*>(stg + A_BYTES + (wave * B_PW + j) * 1024 + lane * 16) = rb[q][j];
    }
  };
  // MXS: MFMA slice kk (64 K) of the stage
  auto compute_mxs = [&](const uint8_t* sA, int kk) {
    const uint8_t* sB = sA + A_BYTES;
    i32x8 af[TMI], bfr[TNI];
    int sc[TNI];
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
      const int r = wm * WM + i * 32 + fr;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(sA + r * ROWA + (((kk * 4 + fk) ^ swz<ROWA>(r)) << 4));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(sA + r * ROWA + (((kk * 4 + 2 + fk) ^ swz<ROWA>(r)) << 4));
      af[i] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int j = 0; j < TNI; ++j) {
      const int n = wn * WN + j * 32 + fr;
      const u32x4 b = *reinterpret_cast<const u32x4*>(sB + n * ROWB + (((kk * 2 + fk) ^ swz<ROWB>(n)) << 4));
      // (FP4 B reads the first four registers of the operand)
      bfr[j] = __builtin_bit_cast(i32x8, __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1));
      sc[j] = sB[B_BYTES + n * SCR + kk * 2 + fk];
    }
#pragma unroll
    for (int i = 0; i < TMI; ++i)
#pragma unroll
      for (int j = 0; j < TNI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j], 0 /* A e4m3 */,
                                                                     4 /* B e2m1 */, 0, 127, 0, sc[j]);
  };
  auto compute = [&](const uint8_t* sA, int kk) {
    if constexpr (MXS) {
      compute_mxs(sA, kk);
      return;
    }
    const uint8_t* sB = sA + A_BYTES;
    const int cc = kk * 2 + fk;                 // 8-element k chunk of this lane
    bf16x8 af[TMI], bfr[TNI];
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
      const int r = wm * WM + i * 32 + fr;
      if (FP8A) {
        const uint2 v = *reinterpret_cast<const uint2*>(
            sA + r * ROWA + (((cc >> 1) ^ swz<ROWA>(r)) << 4) + ((cc & 1) << 3));
        const uint4 w = fp8x8_to_bf16x8(v);
        af[i] = *reinterpret_cast<const bf16x8*>(&w);
      } else {
        af[i] = *reinterpret_cast<const bf16x8*>(sA + r * ROWA + ((cc ^ swz<ROWA>(r)) << 4));
      }
    }
#pragma unroll
    for (int j = 0; j < TNI; ++j) {
      const int n = wn * WN + j * 32 + fr;
      bfr[j] = *reinterpret_cast<const bf16x8*>(sB + n * ROWB + ((cc ^ swz<ROWB>(n)) << 4));
    }
#pragma unroll
    for (int i = 0; i < TMI; ++i)
#pragma unroll
      for (int j = 0; j < TNI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };

  // Register-staged pipeline (RB register buffers, 2 by default; MXFP4 weights
  // MOE_GEMM_RBUF_MX): while step kt computes from one LDS stage,
  // registers hold the loads of the next RB steps; halfway through step kt
  // the registers of step kt + 1 are written to the other stage and refilled
  // with the loads of step kt + 1 + RB, so RB steps of global loads stay in
  // flight.  One barrier per step publishes the written stage and frees the
  // one just read.  Register buffer q holds steps congruent to q mod RB.
  using I0 = std::integral_constant<int, 0>;
  constexpr int NSL = MXS ? BK / 64 : BK / 16;     // MFMA K slices per step
  auto step = [&](int kt, const uint8_t* cur, uint8_t* nxt, auto Q) {
    if (wave_rows) {
#pragma unroll
      for (int kk = 0; kk < NSL / 2; ++kk) compute(cur, kk);
    }
    if (kt + 1 < kend) store_regs(nxt, Q);
    if (kt + 1 + RB < kend) load_regs(kt + 1 + RB, Q);
    if (wave_rows) {
#pragma unroll
      for (int kk = NSL / 2; kk < NSL; ++kk) compute(cur, kk);
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
  };
  // LDS-DMA pipeline: buffer loads write straight into LDS (no registers),
  // each stage its own array so that the compiler can tell the stage being
  // read from the one being filled and adds no wait before fragment reads.
  // Fragments are double-buffered in registers: the reads of slice kk + 1
  // are in flight while slice kk's MFMAs run.  The last slice's fragments
  // are read before the step barrier, so its MFMAs run after it, with the
  // loads of step kt + 2 (into the stage just freed) issued one after each
  // MFMA: a wave that issues them all at once stalls on the full load
  // queue with its MFMAs unissued.
  // MXD: the step's scale bytes of the wave's 32 B rows (W1 or W3 as the rows)
  auto dma_scales = [&](__amdgpu_buffer_rsrc_t r0, __amdgpu_buffer_rsrc_t r1, uint8_t* stg, uint32_t ks) {
    const bool w3 = GATED && ((wave * 32) % WN) >= WN / 2;
    lds_dma4(w3 ? r1 : r0, stg + A_BYTES + B_BYTES + wave * 256, mx_scale, ks);
  };
  auto dma = [&](int kt, uint8_t* stg, bool with_a) {
    const uint32_t ka = static_cast<uint32_t>(kt * BK * SA), kb = static_cast<uint32_t>(kt * KB_STEP);
    if (with_a) {
#pragma unroll
      for (int j = 0; j < A_PW; ++j) lds_dma16(rs_a(j), stg + (wave * A_PW + j) * 1024, a_off[j], ka);
    }
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
      const int gi = wave * B_PW + j;
      const bool w3 = GATED && ((gi * (1024 / ROWB)) % WN) >= WN / 2;
      lds_dma16(w3 ? rsB1 : rsB0, stg + A_BYTES + gi * 1024, b_off[j], kb);
    }
    if constexpr (MXD) dma_scales(rsB0, rsB1, stg, static_cast<uint32_t>(kt * SCR));
  };
  bf16x8 fa[2][TMI], fb[2][TNI];
  i32x8 xa[2][TMI];                              // MXD fragments: A as the instruction's two halves,
  u32x4 xb[2][TNI];                              // B as the lane's MX block,
  int xs[2][TNI];                                // and its scale
  auto ldfr = [&](const uint8_t* sA, int kk, auto P, auto NI) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value, ni = decltype(NI)::value;
    if constexpr (ni == 0) return;
    const uint8_t* sB = sA + A_BYTES;
    if constexpr (MXD) {
#pragma unroll
      for (int i = 0; i < ni; ++i) {
        const int r = wm * WM + i * 32 + fr;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sA + r * ROWA + (((kk * 4 + fk) ^ swz<ROWA>(r)) << 4));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sA + r * ROWA + (((kk * 4 + 2 + fk) ^ swz<ROWA>(r)) << 4));
        xa[p][i] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int j = 0; j < TNI; ++j) {
        const int n = wn * WN + j * 32 + fr;
        xb[p][j] = *reinterpret_cast<const u32x4*>(sB + n * ROWB + (((kk * 2 + fk) ^ swz<ROWB>(n)) << 4));
        xs[p][j] = sB[B_BYTES + n * SCR + kk * 2 + fk];
      }
      return;
    }
    const int cc = kk * 2 + fk;
#pragma unroll
    for (int i = 0; i < ni; ++i) {
      const int r = wm * WM + i * 32 + fr;
      if (FP8A) {
        const uint2 v = *reinterpret_cast<const uint2*>(
            sA + r * ROWA + (((cc >> 1) ^ swz<ROWA>(r)) << 4) + ((cc & 1) << 3));
        const uint4 w = fp8x8_to_bf16x8(v);
        fa[p][i] = *reinterpret_cast<const bf16x8*>(&w);
      } else {
        fa[p][i] = *reinterpret_cast<const bf16x8*>(sA + r * ROWA + ((cc ^ swz<ROWA>(r)) << 4));
      }
    }
#pragma unroll
    for (int j = 0; j < TNI; ++j) {
      const int n = wn * WN + j * 32 + fr;
      fb[p][j] = *reinterpret_cast<const bf16x8*>(sB + n * ROWB + ((cc ^ swz<ROWB>(n)) << 4));
    }
  };
  // one MFMA of fragment buffer p: row block i, column block j
  auto mfma1 = [&](auto P, int i, int j) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    if constexpr (MXD) {
      // (FP4 B reads the first four registers of the operand)
      const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(xb[p][j], xb[p][j], 0, 1, 2, 3, -1, -1, -1, -1));
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa[p][i], b, acc[i][j], 0 /* A e4m3 */,
                                                                   4 /* B e2m1 */, 0, 127, 0, xs[p][j]);
    } else {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[p][i], fb[p][j], acc[i][j], 0, 0, 0);
    }
  };
  auto mm = [&](auto P, auto NI) __attribute__((always_inline)) {
    constexpr int ni = decltype(NI)::value;
#pragma unroll
    for (int i = 0; i < ni; ++i)
#pragma unroll
      for (int j = 0; j < TNI; ++j) mfma1(P, i, j);
  };
  // MFMAs of fragment buffer P (the NI live row blocks) with the loads of
  // step kt2 into stg spread between them: A and B pieces, only A (WHAT = 1)
  // or only B (WHAT = 2).  Past the last step the loads go through an empty
  // descriptor (every lane out of range: no memory access) rather than a
  // branch: a branch would duplicate the loads, and the compiler then no
  // longer tells the two stages apart and waits for all loads before every
  // fragment read.
  auto mm_dma = [&](auto P, auto NI, int kt2, uint8_t* stg, auto WHAT) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    constexpr int NMM = decltype(NI)::value * TNI;
    constexpr int what = decltype(WHAT)::value;
    constexpr int U0 = what == 2 ? A_PW : 0;                  // first piece (A pieces first)
    constexpr int NL = what == 1 ? A_PW : (what == 2 ? B_PWS : LPW);
    const bool live = kt2 < kend;

    const __amdgpu_buffer_rsrc_t rb0 = live ? rsB0 : rs_null;
    const __amdgpu_buffer_rsrc_t rb1 = live ? rsB1 : rs_null;
    const uint32_t ka = live ? static_cast<uint32_t>(kt2 * BK * SA) : 0u;
    const uint32_t kb = live ? static_cast<uint32_t>(kt2 * KB_STEP) : 0u;
    auto issue = [&](int u) {
      if (u < A_PW) {
        lds_dma16(rs_a(u, live), stg + (wave * A_PW + u) * 1024, a_off[u], ka);
      } else if (u < A_PW + B_PW) {
        const int j = u - A_PW, gi = wave * B_PW + j;
        const bool w3 = GATED && ((gi * (1024 / ROWB)) % WN) >= WN / 2;
        lds_dma16(w3 ? rb1 : rb0, stg + A_BYTES + gi * 1024, b_off[j], kb);
      } else if constexpr (MXD) {
        dma_scales(rb0, rb1, stg, live ? static_cast<uint32_t>(kt2 * SCR) : 0u);
      }
    };
    if constexpr (NMM == 0) {
#pragma unroll
      for (int u = 0; u < NL; ++u) issue(U0 + u);
    } else {
#pragma unroll
      for (int q = 0; q < NMM; ++q) {
        mfma1(P, q / TNI, q % TNI);
#pragma unroll
        for (int u = q * NL / NMM; u < (q + 1) * NL / NMM; ++u) issue(U0 + u);
      }
      // keep that order through scheduling: one MFMA, then its loads
      sched_mfma_loads<NMM, NL>(std::make_integer_sequence<int, NMM>{});
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  static_assert(REG || (MXD ? BK / 64 : BK / 16) == 4, "four K slices per step");
  // invariant at step entry: fragments of (cur, slice 0) issued into buffer 0.
  // NI = the wave's live 32-row blocks: fragment reads and MFMAs of blocks
  // wholly past the segment end are left out, so that a segment's partial
  // last m-tile costs about its share of rows; every NI runs the same loads
  // and barriers.
  // With SPLIT_AB the first slice's MFMAs carry the A loads of step kt + 1
  // into nxt (its B came with the previous step; nxt's last readers passed
  // that step's barrier), and the last slice's only the B loads of step kt + 2.
  using W_AB = std::integral_constant<int, 0>;
  using W_A = std::integral_constant<int, 1>;
  using W_B = std::integral_constant<int, 2>;
  auto fstep = [&](int kt, uint8_t* cur, uint8_t* nxt, auto NI) __attribute__((always_inline)) {
    ldfr(cur, 1, P1{}, NI);
    if constexpr (SPLIT_AB) mm_dma(P0{}, NI, kt + 1, nxt, W_A{});
    else mm(P0{}, NI);
    ldfr(cur, 2, P0{}, NI);
    mm(P1{}, NI);
    ldfr(cur, 3, P1{}, NI);
    mm(P0{}, NI);
    wait_vm0();                               // own loads of step kt + 1 landed
    wait_lgkm0();                             // own reads of cur done
    __builtin_amdgcn_s_barrier();
    ldfr(nxt, 0, P0{}, NI);
    if constexpr (SPLIT_AB) mm_dma(P1{}, NI, kt + 2, cur, W_B{});
    else mm_dma(P1{}, NI, kt + 2, cur, W_AB{});
  };

  // Combining epilogue of tile rows [r0, r_end), n-tile nt_ (extra segment: xs).
  // After the workgroup barrier (the tile's output stores are complete), every
  // thread publishes them at agent scope (a release fence: the XCDs' L2 caches
  // are not coherent with each other) before its counter updates, so each
  // update is ordered after all of the tile's stores; each (row, column group)
  // pair adds one to its token's counter, and a pair that brings the counter to
  // zero (the token's other rows in these columns are all written and
  // published) is queued.  After an agent-scope acquire the workgroup writes
  // those columns of y: sum over the slots in slot order of w * (the slot's
  // output row, or for a dropped slot x or the shared output), then the shared
  // output, float32, one rounding, the arithmetic of the combine kernel.
  __shared__ int sc_tok[EPI == EPI_STORE ? BM * BN / kScatterCols : 1];
  __shared__ int sc_grp[EPI == EPI_STORE ? BM * BN / kScatterCols : 1];
  __shared__ int sc_n;
  auto scatter_combine = [&](int r0, int r_end, int nt_, bool xs) {
    constexpr int CG = kScatterCols;
    const int n_out = g.n_out;
    const int G = (n_out + CG - 1) / CG;
    const int c0 = nt_ * BN;
    const int ncol = min(BN, n_out - c0);
    const int ngrp = ncol > 0 ? (ncol + CG - 1) / CG : 0;
    const int nrow = max(0, min(BM, r_end - r0));
    if (tid == 0) sc_n = 0;
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    for (int q = tid; q < nrow * ngrp; q += NW * 64) {
      const int r = r0 + q / ngrp, grp = c0 / CG + q % ngrp;
      const int t = xs ? r : g.sc_src[r];
      const int old = __hip_atomic_fetch_add(g.sc_cnt + static_cast<int64_t>(t) * G + grp, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      if (old == -1) {
        const int i = atomicAdd(&sc_n, 1);
        sc_tok[i] = t;
        sc_grp[i] = grp;
      }
    }
    __syncthreads();
    const int n_own = __builtin_amdgcn_readfirstlane(sc_n);
    if (n_own > 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const int k = g.sc_k;
      const bool shared = g.x_rows > 0;
      const bool fallback = g.sc_drop == MOE_DROP_FALLBACK && shared;
      const bool pass = g.sc_drop == MOE_DROP_PASSTHROUGH;
      for (int q = tid; q < n_own * (CG / 8); q += NW * 64) {
        const int it = q / (CG / 8);
        const int64_t t = sc_tok[it];
        const int col = sc_grp[it] * CG + (q % (CG / 8)) * 8;
        if (col < n_out) {
          float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          for (int j = 0; j < k; ++j) {
            const int p = g.sc_pos[t * k + j];
            const float wj = g.sc_w[t * k + j];
            const uint16_t* row = p >= 0 ? g.out + static_cast<int64_t>(p) * n_out
                                         : (fallback ? g.xout + t * n_out : g.sc_x + t * n_out);
            if (p >= 0 || pass || fallback) combine_fma8(acc, *reinterpret_cast<const uint4*>(row + col), wj);
          }
          if (shared) combine_add8(acc, *reinterpret_cast<const uint4*>(g.xout + t * n_out + col));
          *reinterpret_cast<uint4*>(g.sc_y + t * n_out + col) = combine_pack8(acc);
        }
      }
    }
    __syncthreads();
  };

  if (!next_tile()) return;
  bind_tile();
  if constexpr (!REG) {
    dma(kbeg, sm0, true);
    dma(kbeg + 1, sm1, !SPLIT_AB);               // (past the range: unused bytes, in range or zero)
  }
  for (;;) {
#pragma unroll
    for (int i = 0; i < TMI; ++i)
#pragma unroll
      for (int j = 0; j < TNI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if constexpr (REG) {
      load_regs(kbeg, I0{});
      store_regs(sm0, I0{});
      // steps kbeg + 1 .. kbeg + RB into buffers 1, .., RB - 1, 0
      static_for<RB>([&](auto I) {
        constexpr int i = decltype(I)::value + 1;
        if (kend - kbeg > i) load_regs(kbeg + i, std::integral_constant<int, i % RB>{});
      });
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      // step kt stores the registers of step kt + 1: buffer (kt + 1 - kbeg) % RB;
      // the LDS stages alternate, so the loop is unrolled by lcm(2, RB)
      constexpr int U = RB % 2 == 0 ? RB : 2 * RB;
      for (int kt = kbeg; kt < kend; kt += U) {
        static_for<U>([&](auto J) {
          constexpr int j = decltype(J)::value;
          if (j == 0 || kt + j < kend)
            step(kt + j, j % 2 ? sm1 : sm0, j % 2 ? sm0 : sm1, std::integral_constant<int, (j + 1) % RB>{});
        });
      }
    } else {
      // the tile's first two steps were issued before the previous epilogue
      wait_vm0();
      __builtin_amdgcn_s_barrier();
      // (steps in pairs, the odd last one after the loop: a conditional step
      // inside the loop merges a path with loads pending into the stage the
      // loop head reads, and the compiler then waits for them there)
      with_blocks<TMI>(wave_blocks, [&](auto NI) __attribute__((always_inline)) {
        ldfr(sm0, 0, P0{}, NI);
        int kt = kbeg;
        for (; kt + 1 < kend; kt += 2) {
          fstep(kt, sm0, sm1, NI);
          fstep(kt + 1, sm1, sm0, NI);
        }
        if (kt < kend) fstep(kt, sm0, sm1, NI);
      });
      wait_vm0();                                 // (the last steps' empty loads included)
      __builtin_amdgcn_s_barrier();               // every wave is done with the stages
    }

    // Next tile first: its first two steps load while this tile's epilogue
    // runs (the stages are free, the epilogue does not use LDS).
    const int erow0 = row0, erow_end = row_end, entile = ntile, eunit = unit;
    const bool exseg = xseg;
    uint16_t* const eout = xseg ? g.xout : g.out;
    const bool more = next_tile();
    if (more) {
      bind_tile();
      if constexpr (!REG) {
        dma(kbeg, sm0, true);
        dma(kbeg + 1, sm1, !SPLIT_AB);
      }
    }

    if constexpr (SPLITK) {
      // the raw float32 partial tile, rows and columns in tile order; rows past
      // the segment end are left out (the reduction never reads them; a
      // decode step's one-row tiles would otherwise write 128x the bytes).
      // The lane index is made opaque here so that the compiler computes the
      // store offsets now instead of keeping all of them live across the tile
      // loop (which spills).
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int live = erow_end - erow0 - wm * WM;          // rows of this wave's part in the segment
      const int lrow = 4 * (ln >> 5);
      float* pt = g.part + static_cast<int64_t>(eunit) * (BM * BN) + (wm * WM + lrow) * BN + wn * WN + (ln & 31);
#pragma unroll
      for (int i = 0; i < TMI; ++i) {
        if (i * 32 < live) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = i * 32 + 8 * (r >> 2) + (r & 3);
            if (lr + lrow < live) {
#pragma unroll
              for (int j = 0; j < TNI; ++j) pt[lr * BN + j * 32] = acc[i][j][r];
            }
          }
        }
      }
      if (!more) break;
      continue;
    }

    // epilogue: acc[i][j][r] is row i*32 + 8*(r/4) + 4*(lane/32) + r%4, column j*32 + lane%32.
    // Rows r, r + 1 (r even) and the columns of lanes L, L + 1 (L even) form 2x2
    // blocks: lane L gives its row-(r + 1) value to lane L + 1 and takes that lane's
    // row-r value (one DPP swap), so that lane L writes both outputs of row r and
    // lane L + 1 both of row r + 1, each as one 32-bit store.
    const bool odd = lane & 1;
    auto store_pair = [&](int i, int r, int col_lane, float v0, float v1) {
      const uint32_t b0 = to_bf16(v0), b1 = to_bf16(v1);
      const uint32_t got = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(
          static_cast<int>(odd ? b0 : b1), 0xB1 /* quad_perm [1,0,3,2] */, 0xF, 0xF, false));
      const uint32_t word = odd ? (got | (b1 << 16)) : (b0 | (got << 16));
      const int row = erow0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) + (odd ? 1 : 0);
      const int col = col_lane - (odd ? 1 : 0);
      if (row < erow_end && col < g.n_out)
        *reinterpret_cast<uint32_t*>(eout + static_cast<int64_t>(row) * g.n_out + col) = word;
    };
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float sc0 = 1.0f, sc1 = 1.0f;
        if (FP8A) {
          const int row0 = erow0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          sc0 = row0 < erow_end ? g.a_scale[row0] : 0.f;
          sc1 = row0 + 1 < erow_end ? g.a_scale[row0 + 1] : 0.f;
        }
        if (GATED) {
#pragma unroll
          for (int j = 0; j < TNI / 2; ++j) {
            const int col = entile * (BN / 2) + wn * (WN / 2) + j * 32 + (lane & 31);
            const float v0 = silu_fast(acc[i][j][r] * sc0) * (acc[i][j + TNI / 2][r] * sc0);
            const float v1 = silu_fast(acc[i][j][r + 1] * sc1) * (acc[i][j + TNI / 2][r + 1] * sc1);
            store_pair(i, r, col, v0, v1);
          }
        } else {
#pragma unroll
          for (int j = 0; j < TNI; ++j) {
            const int col = entile * BN + wn * WN + j * 32 + (lane & 31);
            float v0 = acc[i][j][r] * sc0, v1 = acc[i][j][r + 1] * sc1;
            if (EPI == EPI_SILU) v0 = silu_fast(v0), v1 = silu_fast(v1);
            if (EPI == EPI_RELU) v0 = fmaxf(v0, 0.f), v1 = fmaxf(v1, 0.f);
            store_pair(i, r, col, v0, v1);
          }
        }
      }
    }
    if constexpr (EPI == EPI_STORE) {
      if (g.sc_cnt != nullptr) scatter_combine(erow0, erow_end, entile, exseg);
    }
    if (!more) break;
  }
}

// Split-K tail: adds the ksplit float32 partials of each tail tile in range
// order (fixed, so the result does not depend on timing) and applies the
// epilogue.  Unit sp * tiles + t holds range sp of tail tile t.  Grid (tail
// tiles at most, BM / 16): block y covers 16 of the tile's rows.  SwiGLU pairs
// output column c < 128 with the W1 column (c / 32) * 64 + c % 32 and the W3
// column 32 further.
template <int EPI, bool FP8A, int BM>
__global__ __launch_bounds__(256) void gg_splitk_reduce(GemmArgs g) {
  constexpr int TB = 256;                        // tile columns (BM rows)
  constexpr bool GATED = EPI == EPI_SWIGLU;
  const int t = blockIdx.x, ntail = g.part_meta[0], ksplit = g.part_meta[1];
  if (t >= ntail) return;
  const int32_t* m = g.part_meta + 2 + 3 * t;
  const int row0 = m[0], row_end = m[1], ntile = m[2] & ((1 << 30) - 1);
  uint16_t* const outp = (m[2] >> 30) & 1 ? g.xout : g.out;   // the extra segment's tile
  // A thread owns 4 adjacent output columns (16-byte partial loads, one 8-byte
  // store): 64 threads cover a tile row (gated: 32, each reading 4 up and the
  // 4 gate columns 32 further on), and the 4 waves take every 4th of the
  // workgroup's 16 rows.
  const int q = threadIdx.x & 63, sub = threadIdx.x >> 6;
  if (GATED && q >= TB / 8) return;
  const int pc = GATED ? (q >> 3) * 64 + (q & 7) * 4 : 4 * q;      // first partial column
  const int col = ntile * (GATED ? TB / 2 : TB) + 4 * q;           // first output column
  const bool vec = (g.n_out & 3) == 0 && col + 3 < g.n_out;
  const float* pt = g.part + static_cast<int64_t>(t) * (BM * TB) + pc;
  const int64_t range_stride = static_cast<int64_t>(ntail) * (BM * TB);
#pragma unroll 2
  for (int rr = sub; rr < 16; rr += 4) {
    const int lr = blockIdx.y * 16 + rr;
    const int row = row0 + lr;
    if (row >= row_end) break;
    const float sc = FP8A ? g.a_scale[row] : 1.0f;
    const float* pr = pt + lr * TB;
    // (the ranges' loads issued together, then added in range order)
    f32x4 pv[kSplitKMax], pg[kSplitKMax];
#pragma unroll
    for (int sp = 0; sp < kSplitKMax; ++sp) {
      pv[sp] = sp < ksplit ? *reinterpret_cast<const f32x4*>(pr + sp * range_stride) : f32x4{};
      if (GATED) pg[sp] = sp < ksplit ? *reinterpret_cast<const f32x4*>(pr + sp * range_stride + 32) : f32x4{};
    }
    f32x4 u{}, gt{};
#pragma unroll
    for (int sp = 0; sp < kSplitKMax; ++sp) {
      if (sp < ksplit) {
        u += pv[sp];
        if (GATED) gt += pg[sp];
      }
    }
    uint16_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v;
      if (GATED) {
        v = silu_fast(u[i] * sc) * (gt[i] * sc);
      } else {
        v = u[i] * sc;
        if (EPI == EPI_SILU) v = silu_fast(v);
        if (EPI == EPI_RELU) v = fmaxf(v, 0.f);
      }
      o[i] = to_bf16(v);
    }
    uint16_t* dst = outp + static_cast<int64_t>(row) * g.n_out + col;
    if (vec) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                                                  o[2] | (static_cast<uint32_t>(o[3]) << 16));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (col + i < g.n_out) dst[i] = o[i];
    }
  }
}

// ------------------------------------------------------------- decode GEMV --
// Calls of at most four tokens (a decode step) with bf16 weights: every
// segment holds at most four rows, so a tile of 128 or 256 rows would be
// nearly empty and the GEMM becomes weight streaming.  Here each weight row is
// read once and multiplied with the segment's rows (two at a time), with no
// tiles, no LDS staging and no split-K scratch: one work item is JB output
// columns of one segment (for the gated up GEMM the W1 and W3 rows of each),
// its four waves each take a quarter of K, a lane sums its 16-byte chunks in
// order, the wave adds its lanes by a fixed tree and the quarters are added
// in wave order.  The arithmetic (float32 sums of exact bf16 products, the
// fp8 codes widened exactly, the row scale then the activation) is that of
// the tiled kernels; only the order of the additions differs.  Nonempty
// segments only: an expert no token chose costs nothing.  An extra dense
// segment (the shared expert: its own A, weights and output) can join the
// launch.
struct GemvArgs {
  const void* a;            // routed A rows (bf16, or e4m3 codes with fp8): by position, or through gather
  const float* a_scale;     // [positions] row scales (fp8 A), else null
  const int32_t* gather;    // position -> A row, or null
  const int32_t* offsets;   // [n_seg + 1] segment bounds over the positions, or null: one segment
  int64_t rows;             // positions
  int n_seg;
  int K, n_out;
  const uint16_t* b0;       // segment e's matrix [n_out][K] at b0 + e * b_stride
  const uint16_t* b1;       // (gated: the W3 matrices, same layout)
  int64_t b_stride;
  uint16_t* out;            // [positions][n_out]
  const uint16_t* xa;       // the extra segment: A [x_rows][K] (bf16), B at xb0 (xb1), out [x_rows][n_out]
  const uint16_t* xb0;
  const uint16_t* xb1;
  uint16_t* xout;
  int x_rows;               // 0: none
  int epi;                  // Epi
  int fp8;                  // routed A are e4m3 codes (scaled by a_scale)
};

constexpr int kGemvRowsMax = 4;    // tokens of a call that takes this path

// x . w over 8 bf16 pairs (exact products), added to acc in element order
__device__ __forceinline__ float gemv_dot8(uint4 a, uint4 b, float acc) {
  const uint32_t xa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(xa[i] << 16), __uint_as_float(wb[i] << 16), acc);
    acc = fmaf(__uint_as_float(xa[i] & 0xFFFF0000u), __uint_as_float(wb[i] & 0xFFFF0000u), acc);
  }
  return acc;
}

template <int CTRL>
__device__ __forceinline__ float gemv_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// the sum over the wave's lanes, in a fixed order (rows of 16 by DPP, then the four rows)
__device__ __forceinline__ float gemv_wave_sum(float v) {
  v += gemv_dpp<0xB1>(v);     // quad_perm [1, 0, 3, 2]
  v += gemv_dpp<0x4E>(v);     // quad_perm [2, 3, 0, 1]
  v += gemv_dpp<0x141>(v);    // lane i <-> 7 - i within 8
  v += gemv_dpp<0x140>(v);    // lane i <-> 15 - i within 16
  auto ln = [](float u, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u), l)); };
  return (ln(v, 0) + ln(v, 16)) + (ln(v, 32) + ln(v, 48));
}

// One pass of an item: rows r0 .. r0 + nr - 1 (nr <= 2) of a segment times JB
// output columns from j0 (w0 = the first column's W1 row, w1 its W3 row).
template <int JB, int U, bool GATED, bool FP8>
__device__ __forceinline__ void gemv_pass(const GemvArgs& g, const uint8_t* a, const int32_t* gather,
                                          const float* a_scale, int64_t r0, int nr,
                                          const uint16_t* w0, const uint16_t* w1, uint16_t* out,
                                          int j0, float (*red)[JB * 2 * 2]) {
  constexpr int MATS = GATED ? 2 : 1;
  constexpr int R = 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = g.K, nch = K / 8;
  const int c0 = wave * nch / 4, c1 = (wave + 1) * nch / 4;
  const size_t arow = FP8 ? static_cast<size_t>(K) : static_cast<size_t>(K) * 2;   // A row bytes
  const uint8_t* ar[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t pos = r0 + (r < nr ? r : nr - 1);
    ar[r] = a + static_cast<size_t>(gather ? gather[pos] : pos) * arow;
  }
  const uint4* wr[JB][MATS];
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int col = j0 + j < g.n_out ? j0 + j : g.n_out - 1;
    wr[j][0] = reinterpret_cast<const uint4*>(w0 + static_cast<int64_t>(col) * K);
    if (GATED) wr[j][MATS - 1] = reinterpret_cast<const uint4*>(w1 + static_cast<int64_t>(col) * K);
  }
  float acc[JB][MATS][R];
#pragma unroll
  for (int j = 0; j < JB; ++j)
#pragma unroll
    for (int m = 0; m < MATS; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][m][r] = 0.f;
  // U chunks per lane per round, every load of the round issued first
  // (indices clamped into range: loads under a condition are waited for one by one)
  for (int cb = c0 + lane; cb < c1; cb += 64 * U) {
    uint4 wv[U][JB][MATS], av[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = cb + 64 * u < c1 ? cb + 64 * u : c1 - 1;
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int m = 0; m < MATS; ++m) wv[u][j][m] = wr[j][m][c];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (FP8) av[u][r] = fp8x8_to_bf16x8(reinterpret_cast<const uint2*>(ar[r])[c]);
        else av[u][r] = reinterpret_cast<const uint4*>(ar[r])[c];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (cb + 64 * u < c1) {
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
          for (int m = 0; m < MATS; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[j][m][r] = gemv_dot8(av[u][r], wv[u][j][m], acc[j][m][r]);
      }
  }
#pragma unroll
  for (int j = 0; j < JB; ++j)
#pragma unroll
    for (int m = 0; m < MATS; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = gemv_wave_sum(acc[j][m][r]);
        if (lane == 0) red[wave][(j * MATS + m) * R + r] = v;
      }
  __syncthreads();
  if (threadIdx.x < JB * R) {
    const int j = threadIdx.x / R, r = threadIdx.x % R;
    if (j0 + j < g.n_out && r < nr) {
      float v[MATS];
#pragma unroll
      for (int m = 0; m < MATS; ++m) {
        const int q = (j * MATS + m) * R + r;
        v[m] = ((red[0][q] + red[1][q]) + red[2][q]) + red[3][q];
      }
      const float sc = a_scale ? a_scale[r0 + r] : 1.0f;
      float o;
      if (GATED) {
        o = silu_fast(v[0] * sc) * (v[MATS - 1] * sc);
      } else {
        o = v[0] * sc;
        if (g.epi == EPI_SILU) o = silu_fast(o);
        if (g.epi == EPI_RELU) o = fmaxf(o, 0.f);
      }
      out[static_cast<int64_t>(r0 + r) * g.n_out + j0 + j] = to_bf16(o);
    }
  }
  __syncthreads();                                // (red is read before the next pass writes it)
}

template <int JB, int U, bool GATED>
__global__ __launch_bounds__(256, 4) void gemv_kernel(GemvArgs g) {
  __shared__ int segs[kMaxExperts + 1];
  __shared__ int wcnt[4];
  __shared__ float red[4][JB * 2 * 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the nonempty segments in index order (the same list in every workgroup)
  const int n_seg = g.offsets ? g.n_seg : 1;
  auto bounds = [&](int e, int64_t* p0, int64_t* p1) {
    if (!g.offsets) {
      *p0 = 0;
      *p1 = g.rows;
      return;
    }
    int64_t a = g.offsets[e], b = g.offsets[e + 1];
    a = a < 0 ? 0 : (a > g.rows ? g.rows : a);     // (valid offsets pass unchanged)
    b = b < a ? a : (b > g.rows ? g.rows : b);
    *p0 = a;
    *p1 = b;
  };
  bool live = false;
  if (tid < n_seg) {
    int64_t p0, p1;
    bounds(tid, &p0, &p1);
    live = p1 > p0;
  }
  const uint64_t mask = __ballot(live);
  if (lane == 0) wcnt[wave] = __popcll(mask);
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wcnt[w];
  if (live) segs[base + __popcll(mask & ((1ull << lane) - 1))] = tid;
  const int nsegs = (wcnt[0] + wcnt[1]) + (wcnt[2] + wcnt[3]);
  __syncthreads();
  const int jbs = (g.n_out + JB - 1) / JB;                    // items per segment
  const int items = (nsegs + (g.x_rows > 0 ? 1 : 0)) * jbs;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int si = it / jbs, j0 = (it - si * jbs) * JB;
    if (si == nsegs) {                                        // the extra segment (bf16 A, no scale)
      for (int64_t r0 = 0; r0 < g.x_rows; r0 += 2)
        gemv_pass<JB, U, GATED, false>(g, reinterpret_cast<const uint8_t*>(g.xa), nullptr, nullptr, r0,
                                       g.x_rows - r0 < 2 ? static_cast<int>(g.x_rows - r0) : 2, g.xb0,
                                       g.xb1, g.xout, j0, red);
    } else {
      const int e = segs[si];
      int64_t p0, p1;
      bounds(e, &p0, &p1);
      const uint16_t* w0 = g.b0 + (g.offsets ? e * g.b_stride : 0);
      const uint16_t* w1 = GATED ? g.b1 + (g.offsets ? e * g.b_stride : 0) : nullptr;
      for (int64_t r0 = p0; r0 < p1; r0 += 2) {
        const int nr = p1 - r0 < 2 ? static_cast<int>(p1 - r0) : 2;
        if (g.fp8)
          gemv_pass<JB, U, GATED, true>(g, static_cast<const uint8_t*>(g.a), g.gather, g.a_scale, r0, nr,
                                        w0, w1, g.out, j0, red);
        else
          gemv_pass<JB, U, GATED, false>(g, static_cast<const uint8_t*>(g.a), g.gather, nullptr, r0, nr,
                                         w0, w1, g.out, j0, red);
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
                                                     const int32_t* __restrict__ gather,
                                                     int64_t rows, int n_seg, int K, int F,
                                                     const float* __restrict__ w1,
                                                     const float* __restrict__ w3,
                                                     float* __restrict__ h, int act) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t r = q / F;
  const int f = static_cast<int>(q % F);
  const int64_t R = offsets ? min(static_cast<int64_t>(offsets[n_seg]), rows) : rows;
  if (r >= R) return;
  const int e = offsets ? seg_of(offsets, n_seg, static_cast<int>(r)) : 0;
  const float* ar = a + (gather ? static_cast<int64_t>(gather[r]) : r) * K;
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
  const int64_t R = offsets ? min(static_cast<int64_t>(offsets[n_seg]), rows) : rows;
  if (r >= R) return;
  const int e = offsets ? seg_of(offsets, n_seg, static_cast<int>(r)) : 0;
  const float* hr = h + r * F;
  const float* wr = w2 + (static_cast<int64_t>(e) * d + n) * F;
  float v = 0.f;
  for (int j = 0; j < F; ++j) v = fmaf(hr[j], wr[j], v);
  o[r * d + n] = v;
}

// ------------------------------------------------------------------- launch --

template <int BM, int BN, int WGM, int WGN, int EPI, bool FP8A, bool REG, bool TAIL, bool SPLITK = false,
          bool MX = false, bool MXS = false>
hipError_t launch_gg_on(const GemmArgs& g, int tiles_upper, hipStream_t st) {
  int cus = device_cu_count();
  int grid = (cus / 8) * 8;
  int want = ((tiles_upper + 7) / 8) * 8;
  if (want < grid) grid = want;
  if (grid < 8) grid = 8;
  hipLaunchKernelGGL((gg_kernel<BM, BN, WGM, WGN, EPI, FP8A, REG, TAIL, SPLITK, MX, MXS>), dim3(grid),
                     dim3(64 * WGM * WGN), 0, st, g);
  return hipGetLastError();
}

// Tile height: 256 rows read each weight n-tile once per 256 rows of an
// expert, 128 rows waste less on short segments.  The taller tile pays from
// this many rows per expert on average: 96 with fp8 activations (A rows cost
// half as much; measured at the DeepSeek-V3-shaped gate/up, ~128 rows per
// expert, 4.18 -> 3.96 ms) and for the down GEMM (1.84 -> 1.80 ms there), 384
// for the gate/up GEMM with bf16 activations (the change to 96 lost 6%).
constexpr int kBm256RowsFp8 = 96, kBm256RowsUp = 384, kBm256RowsDown = 96;
int split_slots() { return (device_cu_count() / 8) * 8; }

// Few tiles (a decode step, a small dense call): at most S / 2 tiles of 128
// rows, each of at most min(rows, segments) segments holding fewer than 128
// rows.  With split-K scratch these run as 128-row register-staged tiles (the
// pipeline with the most bytes in flight, which weight streaming needs), every
// tile split along K so that all CUs stream its weights.
bool skinny(int64_t rows, int n_seg, int64_t nt) {
  const int64_t segs = rows < n_seg ? rows : n_seg;
  const int64_t mt = ceil_div(rows, 128) > segs ? ceil_div(rows, 128) : segs;
  return 2 * mt * nt <= split_slots();
}

int pick_bm(int64_t rows, int n_seg, int min_avg_256, int64_t nt, bool split, bool mx = false) {
  if (mx || (split && skinny(rows, n_seg, nt))) return 128;
  const int64_t avg = n_seg > 0 ? rows / n_seg : rows;
  return avg >= min_avg_256 ? 256 : 128;
}


// 8 waves (two per SIMD, so one wave's MFMAs cover the other's waits) in a
// 2 x 4 grid: 128x64 per wave at BM = 256, 64x64 at BM = 128.  Measured choice of
// load path: LDS-DMA for the MFMA-bound 256-row tiles, the register-staged
// pipeline (more bytes in flight) for the weight-streaming 128-row tiles.  The
// 256-row tile list is tail-split; its 128x128 quarters run on 4 waves of 64x64.
template <int EPI, bool FP8A, bool MX = false>
hipError_t dispatch_up(int bm, GemmArgs g, int64_t rows, int n_seg, bool dense, void* split,
                       hipStream_t st) {
  const int nt = g.nt;
  if (MX && bm == 256) return hipErrorInvalidValue;          // (MXFP4 weights: 128-row tiles only)
  if (!MX && bm == 256) {
    const int mtu = static_cast<int>(ceil_div(rows, 256)) + (dense ? 0 : n_seg);
    g.split_slots = split_slots();
    // the scratch header holds the tail's tile count, range count and up to S / 2 tiles' rows
    if (2 + 3 * (g.split_slots / 2) > static_cast<int>(kSplitMetaBytes / 4)) split = nullptr;
    g.split_k_max = split != nullptr ? kSplitKMax : 0;
    hipError_t err = launch_gg_on<256, 256, 2, 4, EPI, FP8A, false, false>(g, mtu * nt, st);
    if (err != hipSuccess) return err;
    if (split == nullptr)
      return launch_gg_on<128, 128, 2, 2, EPI, FP8A, false, true>(g, 4 * mtu * nt, st);
    // split-K tail (scratch from the caller): whole tiles, K ranges each
    g.part_meta = static_cast<int32_t*>(split);
    g.part = reinterpret_cast<float*>(static_cast<char*>(split) + kSplitMetaBytes);
    err = launch_gg_on<256, 256, 2, 4, EPI, FP8A, false, true, true>(g, kSplitKMax * mtu * nt, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((gg_splitk_reduce<EPI, FP8A, 256>), dim3(g.split_slots / 2, 16), dim3(256), 0,
                       st, g);
    return hipGetLastError();
  }
  // 128-row tiles; with scratch (given only when the list is expected to hold
  // at most S / 2 tiles) every tile is split along K over all CUs.  The
  // whole-tile launch takes the list when it turns out longer (the kernel
  // counts it); it is left out when the list is short for certain: every
  // m-tile holds a row and every nonempty segment adds at most one partial
  // m-tile, so there are at most min(rows, (rows + 127 s) / 128) of them, s =
  // min(rows, segments) (an empty launch still costs ~4.5 us).
  const int mtu = static_cast<int>(ceil_div(rows, 128)) + (dense ? 0 : n_seg);
  g.split_slots = split != nullptr ? split_slots() : 0;
  if (2 + 3 * (g.split_slots / 2) > static_cast<int>(kSplitMetaBytes / 4)) split = nullptr, g.split_slots = 0;
  g.split_k_max = split != nullptr ? kSplitKMax : 0;
  const int64_t segs = dense ? 1 : (rows < n_seg ? rows : n_seg);
  const int64_t mt_most = dense ? ceil_div(rows, 128) : std::min<int64_t>(rows, (rows + 127 * segs) / 128);
  const bool all_split = split != nullptr && 2 * mt_most * nt <= g.split_slots;
  // fp8 A with MXFP4 B: the scaled MFMA on the codes as stored; whole tiles on
  // the LDS-DMA pipeline (256-K steps), else register-staged (128-K steps)
  constexpr bool MXS_OK = MX && FP8A;
  const bool mxs = MXS_OK && g.K % 128 == 0;
  hipError_t err = hipSuccess;
  if (!all_split) {
    if constexpr (MXS_OK) {
      if (g.K % 256 == 0)
        err = launch_gg_on<128, 256, 2, 4, EPI, FP8A, false, false, false, MX, true>(g, mtu * nt, st);
      else if (mxs)
        err = launch_gg_on<128, 256, 2, 4, EPI, FP8A, true, false, false, MX, true>(g, mtu * nt, st);
      else
        err = launch_gg_on<128, 256, 2, 4, EPI, FP8A, true, false, false, MX>(g, mtu * nt, st);
    } else {
      err = launch_gg_on<128, 256, 2, 4, EPI, FP8A, true, false, false, MX>(g, mtu * nt, st);
    }
    if (err != hipSuccess || split == nullptr) return err;
  }
  g.part_meta = static_cast<int32_t*>(split);
  g.part = reinterpret_cast<float*>(static_cast<char*>(split) + kSplitMetaBytes);
  err = mxs ? launch_gg_on<128, 256, 2, 4, EPI, FP8A, true, true, true, MX, MXS_OK>(g, kSplitKMax * mtu * nt, st)
            : launch_gg_on<128, 256, 2, 4, EPI, FP8A, true, true, true, MX>(g, kSplitKMax * mtu * nt, st);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((gg_splitk_reduce<EPI, FP8A, 128>), dim3(g.split_slots / 2, 8), dim3(256), 0, st, g);
  return hipGetLastError();
}

// The decode GEMV launch: four workgroups per CU (at most 128 VGPRs), each
// lane with 8 to 16 weight loads of one round in flight: U chunks per lane
// per round (a quarter of K in one or a few rounds) times JB columns (times
// W1 and W3 when gated).  Measured at the DeepSeek-V3 decode shape (graph
// replay of the whole layer, 1 / 2 / 4 tokens): against the tiled split-K
// GEMMs 191.5 / 285.8 / 531.6 -> 168.9 / 273.1 / 523.9 us; two workgroups per
// CU with 16-24 loads lost (194.8 us at 1 token), and so did 8 loads per
// lane (175.3) or 6 and 8 workgroups per CU (229.1, 220.3: spills).
template <bool GATED>
hipError_t launch_gemv_on(const GemvArgs& g, hipStream_t st) {
  const int cpl = static_cast<int>(ceil_div(ceil_div(g.K / 8, 4), 64));   // chunks per lane
  const dim3 grid(static_cast<unsigned>(4 * device_cu_count())), block(256);
  if constexpr (GATED) {
    if (cpl >= 4) hipLaunchKernelGGL((gemv_kernel<2, 4, GATED>), grid, block, 0, st, g);
    else if (cpl >= 2) hipLaunchKernelGGL((gemv_kernel<4, 2, GATED>), grid, block, 0, st, g);
    else hipLaunchKernelGGL((gemv_kernel<4, 1, GATED>), grid, block, 0, st, g);
  } else {
    if (cpl >= 4) hipLaunchKernelGGL((gemv_kernel<3, 4, GATED>), grid, block, 0, st, g);
    else if (cpl >= 2) hipLaunchKernelGGL((gemv_kernel<8, 2, GATED>), grid, block, 0, st, g);
    else hipLaunchKernelGGL((gemv_kernel<8, 1, GATED>), grid, block, 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace

// Scratch of the split-K tails of this shape's grouped GEMMs (routed, and the
// shared expert's dense ones): none when none uses 256-row tiles or few tiles,
// else one float32 partial tile (at most 256x256) per tail work unit, at most S
// of them (a tail of r <= S / 4 tiles in 4 ranges, or t <= S / 2 tiles in at
// most S / t ranges).
size_t gemm_split_bytes(const moe_shape& s) {
  if (s.dtype != MOE_BF16) return 0;
  const int64_t rows = s.T * s.k;
  const int64_t nt_up = s.act == MOE_ACT_SWIGLU ? ceil_div(s.F, 128) : ceil_div(s.F, 256);
  const int64_t nt_down = ceil_div(s.d, 256);
  const bool fp8 = s.buf_dtype == MOE_FP8_E4M3;
  int64_t tiles = 0;
  const bool mx = s.wfmt == MOE_W_MXFP4;
  auto add = [&](int64_t r, int n_seg, int min_avg_256, int64_t nt) {
    if (skinny(r, n_seg, nt) || pick_bm(r, n_seg, min_avg_256, nt, false, mx) == 256)
      tiles = std::max(tiles, (ceil_div(r, 128) + (n_seg > 1 ? n_seg : 0)) * nt);
  };
  add(rows, s.N, fp8 ? kBm256RowsFp8 : kBm256RowsUp, nt_up);
  add(rows, s.N, kBm256RowsDown, nt_down);
  if (s.has_shared) {
    add(s.T, 1, kBm256RowsUp, nt_up);
    add(s.T, 1, kBm256RowsDown, nt_down);
    add(rows + s.T, s.N + 1, kBm256RowsDown, nt_down);   // the routed and shared down in one launch
  }
  if (tiles == 0) return 0;
  const int64_t units = std::min<int64_t>(split_slots(), kSplitKMax * tiles);
  return kSplitMetaBytes + static_cast<size_t>(units) * 256 * 256 * 4;
}

// The router kernel's own logits re-read W_g (N d bf16) per 16 tokens; the GEMM
// instead writes and re-reads float32 partials of 1 KB per token and K range.
// Measured: the GEMM pays at N = 256, d = 7168 (router 142 -> 76 us at 4096
// tokens) and not at N = 128, d = 1024 (43 -> 60 us at 8192 tokens).
bool router_gemm(const moe_shape& s) {
  return s.dtype == MOE_BF16 && s.N >= 64 && s.N <= kRouterTileCols &&
         static_cast<int64_t>(s.N) * s.d >= (1 << 19) && s.T >= 512 && s.d % 64 == 0 &&
         skinny(s.T, 1, 1);
}

size_t router_gemm_bytes(const moe_shape& s) {
  if (!router_gemm(s)) return 0;
  return kSplitMetaBytes + static_cast<size_t>(split_slots()) * kRouterTileRows * kRouterTileCols * 4;
}

// The split-K tail alone (few tiles: every tile in min(8, S / tiles) K
// ranges), register-staged 128 x 256 tiles; no reduction, the router reads
// the partials.
hipError_t launch_router_logits(const moe_shape& s, const void* x, const void* wg, void* scratch,
                                hipStream_t st) {
  GemmArgs g{};
  g.a = x;
  g.a_scale = nullptr;
  g.offsets = nullptr;
  g.rows = s.T;
  g.n_seg = 1;
  g.K = s.d;
  g.n_out = s.N;
  g.b0 = static_cast<const uint16_t*>(wg);
  g.b1 = nullptr;
  g.b_stride = static_cast<int64_t>(s.N) * s.d;
  g.out = nullptr;
  g.nt = 1;
  g.split_slots = split_slots();
  g.split_k_max = kSplitKMax;
  g.part_meta = static_cast<int32_t*>(scratch);
  g.part = reinterpret_cast<float*>(static_cast<char*>(scratch) + kSplitMetaBytes);
  const int mtu = static_cast<int>(ceil_div(s.T, kRouterTileRows));
  return launch_gg_on<kRouterTileRows, kRouterTileCols, 2, 4, EPI_STORE, false, true, true, true>(
      g, kSplitKMax * mtu, st);
}

bool gemv_fits(const moe_shape& s) {
  return s.dtype == MOE_BF16 && s.wfmt != MOE_W_MXFP4 && s.T > 0 && s.T <= kGemvRowsMax && s.d % 8 == 0 &&
         s.F % 8 == 0;
}

hipError_t launch_expert_up(const moe_shape& s, const void* a, const float* row_scale,
                            const int32_t* offsets, int64_t rows, int n_seg, const void* w1,
                            const void* w3, void* h, void* split, hipStream_t st,
                            const int32_t* gather, int64_t a_rows, const void* xa, const void* xw1,
                            const void* xw3, void* xout, int64_t x_rows) {
  if (gemv_fits(s)) {
    GemvArgs g{};
    const bool fp8 = s.buf_dtype == MOE_FP8_E4M3 && row_scale != nullptr;
    g.a = a;
    g.a_scale = fp8 ? row_scale : nullptr;
    g.gather = gather;
    g.offsets = offsets;
    g.rows = rows;
    g.n_seg = n_seg;
    g.K = s.d;
    g.n_out = s.F;
    g.b0 = static_cast<const uint16_t*>(w1);
    g.b1 = static_cast<const uint16_t*>(w3);
    g.b_stride = static_cast<int64_t>(s.F) * s.d;
    g.out = static_cast<uint16_t*>(h);
    const bool extra = x_rows > 0 && offsets != nullptr;
    g.xa = extra ? static_cast<const uint16_t*>(xa) : nullptr;
    g.xb0 = extra ? static_cast<const uint16_t*>(xw1) : nullptr;
    g.xb1 = extra ? static_cast<const uint16_t*>(xw3) : nullptr;
    g.xout = extra ? static_cast<uint16_t*>(xout) : nullptr;
    g.x_rows = extra ? static_cast<int>(x_rows) : 0;
    g.epi = s.act == MOE_ACT_SWIGLU ? EPI_SWIGLU : (s.act == MOE_ACT_RELU ? EPI_RELU : EPI_SILU);
    g.fp8 = fp8 ? 1 : 0;
    return s.act == MOE_ACT_SWIGLU ? launch_gemv_on<true>(g, st) : launch_gemv_on<false>(g, st);
  }
  if (x_rows > 0) return hipErrorInvalidValue;       // (the tiled path takes the extra segment only for down)
  if (s.dtype == MOE_F32) {
    int64_t n = rows * s.F;
    dim3 grid(static_cast<unsigned>(ceil_div(n, 256)));
    hipLaunchKernelGGL(f32_up_kernel, grid, dim3(256), 0, st, static_cast<const float*>(a),
                       offsets, gather, rows, n_seg, s.d, s.F, static_cast<const float*>(w1),
                       static_cast<const float*>(w3), static_cast<float*>(h), s.act);
    return hipGetLastError();
  }
  const bool fp8 = s.buf_dtype == MOE_FP8_E4M3 && row_scale != nullptr;
  const bool dense = offsets == nullptr;
  GemmArgs g{};
  g.a = a;
  g.a_scale = fp8 ? row_scale : nullptr;
  g.gather = gather;
  g.a_total = a_rows;
  g.offsets = offsets;
  g.rows = rows;
  g.n_seg = n_seg;
  g.K = s.d;
  g.n_out = s.F;
  g.b0 = static_cast<const uint16_t*>(w1);
  g.b1 = static_cast<const uint16_t*>(w3);
  const bool mx = s.wfmt == MOE_W_MXFP4;
  g.b_stride = mx ? static_cast<int64_t>(mxfp4_bytes(s.F, s.d)) : static_cast<int64_t>(s.F) * s.d;
  g.mx_scale_off = static_cast<int64_t>(s.F) * s.d / 2;
  g.out = static_cast<uint16_t*>(h);
  const bool gated = s.act == MOE_ACT_SWIGLU;
  g.nt = static_cast<int>(gated ? ceil_div(s.F, 128) : ceil_div(s.F, 256));
  const bool sk = split != nullptr && skinny(rows, dense ? 1 : n_seg, g.nt);
  const int bm = pick_bm(rows, dense ? 1 : n_seg, fp8 ? kBm256RowsFp8 : kBm256RowsUp, g.nt, sk, mx);
  if (bm != 256 && !sk) split = nullptr;        // (128-row tiles use the scratch only when few)
#define MOE_UP(EPI_)                                                                                   \
  return mx ? (fp8 ? dispatch_up<EPI_, true, true>(bm, g, rows, n_seg, dense, split, st)               \
                   : dispatch_up<EPI_, false, true>(bm, g, rows, n_seg, dense, split, st))             \
            : (fp8 ? dispatch_up<EPI_, true>(bm, g, rows, n_seg, dense, split, st)                     \
                   : dispatch_up<EPI_, false>(bm, g, rows, n_seg, dense, split, st));
  if (gated) MOE_UP(EPI_SWIGLU)
  if (s.act == MOE_ACT_RELU) MOE_UP(EPI_RELU)
  MOE_UP(EPI_SILU)
#undef MOE_UP
}

hipError_t launch_expert_down(const moe_shape& s, const void* h, const int32_t* offsets,
                              int64_t rows, int n_seg, const void* w2, void* out, void* split,
                              hipStream_t st, const void* xa, const void* xw2, void* xout, int64_t x_rows,
                              const ScatterArgs* sc) {
  // (the combining epilogue runs in the tiled bf16 kernels only)
  if (sc != nullptr && (gemv_fits(s) || s.dtype != MOE_BF16)) return hipErrorInvalidValue;
  if (gemv_fits(s)) {
    GemvArgs g{};
    g.a = h;
    g.offsets = offsets;
    g.rows = rows;
    g.n_seg = n_seg;
    g.K = s.F;
    g.n_out = s.d;
    g.b0 = static_cast<const uint16_t*>(w2);
    g.b_stride = static_cast<int64_t>(s.d) * s.F;
    g.out = static_cast<uint16_t*>(out);
    const bool extra = x_rows > 0 && offsets != nullptr;
    g.xa = extra ? static_cast<const uint16_t*>(xa) : nullptr;
    g.xb0 = extra ? static_cast<const uint16_t*>(xw2) : nullptr;
    g.xout = extra ? static_cast<uint16_t*>(xout) : nullptr;
    g.x_rows = extra ? static_cast<int>(x_rows) : 0;
    g.epi = EPI_STORE;
    return launch_gemv_on<false>(g, st);
  }
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
  const bool mx = s.wfmt == MOE_W_MXFP4;
  g.b_stride = mx ? static_cast<int64_t>(mxfp4_bytes(s.d, s.F)) : static_cast<int64_t>(s.d) * s.F;
  g.mx_scale_off = static_cast<int64_t>(s.d) * s.F / 2;
  g.out = static_cast<uint16_t*>(out);
  g.nt = static_cast<int>(ceil_div(s.d, 256));
  // the extra dense segment (offsets given; its rows and m-tiles count in the estimates)
  const bool extra = x_rows > 0 && !dense;
  g.xa = extra ? xa : nullptr;
  g.xb0 = extra ? static_cast<const uint16_t*>(xw2) : nullptr;
  g.xout = extra ? static_cast<uint16_t*>(xout) : nullptr;
  g.x_rows = extra ? x_rows : 0;
  if (sc != nullptr) {
    // every output element from one workgroup's epilogue: no split-K tail
    split = nullptr;
    g.sc_src = sc->src;
    g.sc_pos = sc->pos;
    g.sc_w = sc->w;
    g.sc_x = static_cast<const uint16_t*>(sc->x);
    g.sc_y = static_cast<uint16_t*>(sc->y);
    g.sc_cnt = sc->cnt;
    g.sc_k = s.k;
    g.sc_drop = s.drop;
  }
  const int64_t rows_all = rows + g.x_rows;
  const int segs_all = dense ? 1 : n_seg + (extra ? 1 : 0);
  const bool sk = split != nullptr && skinny(rows_all, segs_all, g.nt);
  const int bm = pick_bm(rows_all, segs_all, kBm256RowsDown, g.nt, sk, mx);
  if (bm != 256 && !sk) split = nullptr;        // (128-row tiles use the scratch only when few)
  return mx ? dispatch_up<EPI_STORE, false, true>(bm, g, rows_all, segs_all, dense, split, st)
            : dispatch_up<EPI_STORE, false>(bm, g, rows_all, segs_all, dense, split, st);
}

}  // namespace moe
