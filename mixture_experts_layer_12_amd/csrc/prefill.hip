// Prefill path: grouped GEMMs over the expert-sorted token order on the bf16
// matrix cores, for large batches where the layer is compute-bound.
//
// Sources: "Fused MoE kernel on Triton: 5 launches vs 24" (ai-manual.ru),
// section "Fused kernel: one operation instead of twenty-four" -- the expert
// computation takes two launches over all engaged experts at once, and the
// weighted aggregation is fused (no per-operation intermediate buffers,
// section "Megablocks? It has been obsolete for two years").  Here:
//   gate/up GEMM  one launch for every routed expert segment and every shared
//                 expert; x rows are gathered through the sorted order while
//                 they are staged into LDS; the epilogue applies silu(g) * u
//                 and stores bf16 activations;
//   down GEMM     one launch; its epilogue multiplies by the routing weight
//                 and stores fp32 partial rows (one per sorted row and k
//                 range);
//   combine       each token's routed and shared rows added in one fixed
//                 order and cast to the output dtype (deterministic: no
//                 float atomics, so the bits do not depend on which tile
//                 finished first).
//
// Both GEMMs run one work-group per 256 x 256 output tile (256 sorted token
// rows by 256 weight rows: for gate/up 128 gate + 128 up rows of the same
// intermediate columns, for down 256 hidden columns) on the same pipeline:
//  * four waves, one per SIMD, each accumulating a 128 x 128 block in 16
//    32x32 MFMA tiles held in the accumulation registers (two MFMAs per
//    16-byte LDS operand read).  The 32x32x16 form is the one a single wave
//    per SIMD issues at the full matrix rate (the 16x16x32 form reaches
//    about 60 % that way), and a 256 x 256 tile is the largest those
//    registers allow: it moves the fewest bytes per flop through the load
//    path, which is what limits these kernels;
//  * operands move global -> LDS with the gfx950 direct-to-LDS loads, one
//    wave instruction = 8 rows x 128 bytes (the load path moves 64-byte row
//    pieces at well under half the rate), in stages of 64 values of k; the
//    weight operand (from HBM) has three ring slots and the other two
//    (5 x 32 KiB), so weight loads are issued about two stages ahead;
//  * a stage is multiplied in four MFMA k-steps; while one k-step is
//    multiplied the operands of the next are read from LDS (interleaved one
//    read per MFMA), and the refills are spread over the k-steps (a few
//    loads between MFMAs) so the matrix cores never wait behind a burst of
//    load issues;
//  * the 16-byte chunks of each staged row are XOR-permuted so the 16 rows
//    one operand read touches fall on distinct LDS banks.
// Row tiles follow the dispatch padding of this path (256 rows per expert
// segment), so a tile never spans two experts.  An expert's last tile with
// at most 128 rows in use is a half tile: only those 128 token rows are
// staged and the four waves split the weight rows instead (each 2 x 4 or
// 4 x 2 MFMA blocks), half the work of a full tile.
#include "common.hpp"

namespace moe {

// Calls f(std::integral_constant<int, i>) for i = B .. E - 1 (compile-time loop).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int MM_TM = 256;                    // token rows per tile (the dispatch padding of this path)
constexpr int MM_TN = 256;                    // weight rows per tile
constexpr int MM_BK = 64;                     // k per LDS stage: 128-byte staged rows
constexpr int MM_WAVES = 4;
constexpr int MM_RPI = 8;                     // staged rows per load instruction (1 KiB)
constexpr int MM_NS = 256 / MM_RPI / MM_WAVES;   // load instructions per wave per stage for 256 rows (8)
constexpr int MM_DMA = 2 * MM_NS;             // at most: two operands of 256 rows
// The ring: three slots for the operand that streams from HBM and two for
// the other, 5 x 32 KiB, the whole LDS of a CU.
constexpr int MM_HALF = MM_TM * MM_BK;        // bf16 elements of one operand's slot
constexpr size_t MM_LDS = size_t(5) * MM_HALF * sizeof(uint16_t);   // 160 KiB

// Wait until at most N vector-memory operations of this wave are outstanding
// (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Work-group barrier for the ring: this wave's LDS reads are complete
// (lgkmcnt 0) and the caller has already waited for its own stage loads.  A
// plain __syncthreads() would also wait for every load still in flight
// (vmcnt 0).  The asm statement clobbers memory, so the compiler moves no
// memory access across it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | (0x0 << 8) | ((0x3F >> 4) << 14));   // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Chunk c of staged row r is stored at position c ^ mm_swz(r): the 16 rows
// that 16 consecutive lanes of an operand read touch (one chunk each) then
// fall on distinct banks, whether the LDS serves 8 or 16 lanes per cycle.
// The swizzle depends on bits 0-3 of r only, so it is the same for a row's
// index within any block that starts at a multiple of 16 rows.
__device__ __forceinline__ int mm_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Tile order.  The work is the list of (k range, column group, row tile,
// column) items over the row tiles in use only: the routed tiles up to the
// dispatch's padded total (the capacity's worst case leaves several unused)
// and the shared experts' tiles.  Column groups are MM_CG column tiles; in
// a group the row tiles go in order and the columns inner, so consecutive
// items share a weight tile (same columns, same expert) or a token tile.
// Each XCD (hardware places work-group b on XCD b % 8) takes one contiguous
// eighth of the list, in order: the XCDs get equal work whatever the number
// of row tiles, the work-groups resident on one XCD at a time cover a block
// of about 32 / MM_CG row tiles by MM_CG columns and share its operands in
// that XCD's L2, and each weight column is read by one or two XCDs only.
#ifndef MOE_PF_CG
#define MOE_PF_CG 4
#endif
constexpr int MM_CG = MOE_PF_CG;
struct TileList {
  int n_real;      // routed row tiles in use
  int n_routed;    // routed row tiles of the capacity
  int n_rows;      // row tiles in the list: n_real + the shared experts' tiles
  int n_ct;        // column tiles
  long n_items;    // k ranges x n_rows x n_ct
};
__device__ __forceinline__ TileList tile_list(const PrefillArgs& a, int n_ct, int k_ranges) {
  TileList L;
  L.n_routed = a.capacity / MM_TM;
  L.n_real = min(max(a.offsets[a.E], 0) / MM_TM, L.n_routed);
  L.n_rows = L.n_real + (a.n_row_tiles - L.n_routed);
  L.n_ct = n_ct;
  L.n_items = long(k_ranges) * L.n_rows * n_ct;
  return L;
}
// Item of work-group `bid`: false past the end of its XCD's share.
__device__ __forceinline__ bool tile_item(int bid, const TileList& L, int& kr, int& rt, int& ct) {
  const int x = bid & 7;
  const long item = x * L.n_items / 8 + (bid >> 3);
  if (item >= (x + 1) * L.n_items / 8) return false;
  const long per_k = long(L.n_rows) * L.n_ct;
  kr = int(item / per_k);
  const int in_k = int(item - kr * per_k);
  const int g = in_k / (L.n_rows * MM_CG);
  const int in_g = in_k - g * L.n_rows * MM_CG;
  const int ncg = min(MM_CG, L.n_ct - g * MM_CG);
  const int j = in_g / ncg;
  ct = g * MM_CG + in_g % ncg;
  rt = j < L.n_real ? j : L.n_routed + (j - L.n_real);
  return true;
}
// Work-groups for up to n_items items: every XCD's share fits.
__host__ __device__ inline int tile_grid(long n_items) { return int(8 * ((n_items + 7) / 8)); }

// What one wave stages per k stage: load instruction q (8 rows x 128 bytes)
// reads matrix base[q] (wave-uniform) at this lane's element offset off[q]
// (row offset plus the lane's chunk) and fills staged rows row[q] ..
// row[q] + 7 (wave-uniform).  Bit q of `upper`: this lane's chunk is one of
// the upper 32 values of a stage.
struct TileLoads {
  const uint16_t* base[MM_DMA];
  uint32_t off[MM_DMA];
  int row[MM_DMA];
  unsigned upper;
};

// Fills entry q of `ld` for staged row block `row0` (a multiple of 8) of a
// matrix with row `src_row` for this lane's staged row and `stride`
// elements per row.
__device__ __forceinline__ void set_load(TileLoads& ld, int q, const uint16_t* base, int row0, int src_row,
                                         int stride, int lane) {
  const int chunk = (lane & 7) ^ mm_swz(row0 + (lane >> 3));
  ld.base[q] = base;
  ld.off[q] = uint32_t(src_row) * uint32_t(stride) + uint32_t(chunk << 3);
  ld.row[q] = row0;
  ld.upper |= unsigned(chunk >= 4) << q;
}

template <int NI, int NJ>
struct MMFrags { u32x4_t a[2][NI], b[2][NJ]; };   // [k-step parity][32-row block]

// One wave's share of the work-group's MFMA tile over K (a multiple of 32).
// Staged rows [0, 256) are the A operand, [256, 512) the B operand.  This
// wave has NI A blocks of 32 rows, at a0 + (i & 1) * 32 + (i >> 1) * a_step
// (NI = 4) or a0 + i * a_step (NI = 2), and NJ B blocks at 256 + b0 + 32 j;
// acc[i][j] accumulates A block i x B block j: register q of lane l holds
// row 8 (q / 4) + 4 (l / 32) + q % 4 of A block i and row l % 32 of B
// block j.  A full tile is NI = NJ = 4 in every wave (256 x 256); a half
// tile stages only 128 rows of one operand and gives each wave 2 x 4 or
// 4 x 2 blocks.
//
// The ring (`smem`, MM_LDS bytes) has three slots for the SLOW
// operand (1: A, 2: B), the one that streams from HBM, and two for the
// other; the slow operand's rows are load instructions q < MM_NS of `ld`,
// the fast operand's the next NF.  After the barrier of stage kt the fast
// operand of stage kt + 2 is issued first (k-steps 3 and 0) and then the
// slow operand of stage kt + 3 (k-steps 1 and 2 of the next stage), so the
// barrier of stage kt + 1 waits for everything but those last loads (loads
// complete in issue order): slow loads get about two stages to arrive,
// fast loads one.
template <int SLOW, int NI, int NJ, int NF>
__device__ __forceinline__ void mm_tile(uint16_t* smem, const TileLoads& ld, int K, int a0, int a_step, int b0,
                                        f32x16_t (&acc)[NI][NJ]) {
  static_assert(SLOW == 1 || SLOW == 2, "slow operand");
  static_assert((NI == 4 || NI == 2) && (NJ == 4 || NJ == 2) && (NF == 8 || NF == 4), "tile shape");
  constexpr int NQ = MM_NS + NF;               // load instructions per wave per stage
  static_assert(NQ <= MM_DMA, "load table");
  const int lane = threadIdx.x & 63;
  const int nk = (K + MM_BK - 1) / MM_BK;     // stages; K % 64 == 32 leaves a half-full last one
  const int nk_full = K / MM_BK;
  // Element offsets of stage kt's A and B slots; a staged row r is at
  // offset + r * MM_BK (B rows are r = 256 .. 511).
  auto slow = [](int kt) { return (kt % 3) * MM_HALF; };        // slots 0 .. 2
  auto fast = [](int kt) { return (3 + kt % 2) * MM_HALF; };    // slots 3, 4
  auto a_slot = [&](int kt) { return SLOW == 1 ? slow(kt) : fast(kt); };
  auto b_slot = [&](int kt) { return (SLOW == 1 ? fast(kt) : slow(kt)) - MM_HALF; };
  // In a half-full last stage, lanes whose chunk lies past K load the chunk
  // 32 values lower instead (in bounds), and the k-steps past K multiply a
  // zero B operand.
  auto issue = [&](int kt, auto q0, auto q1) {   // load instructions q0 .. q1 - 1 of stage kt
    const int k0 = kt * MM_BK;
    const bool part = k0 + MM_BK > K;
    const int os = SLOW == 1 ? a_slot(kt) : b_slot(kt), of = SLOW == 1 ? b_slot(kt) : a_slot(kt);
    static_for<decltype(q0)::value, decltype(q1)::value>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      const int back = (part && ((ld.upper >> q) & 1)) ? 32 : 0;
      uint16_t* d = smem + (q < MM_NS ? os : of);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(ld.base[q] + (ld.off[q] + uint32_t(k0 - back))),
                                       (lds_void_t*)(d + ld.row[q] * MM_BK), 16, 0, 0);
    });
  };
  using Q0 = std::integral_constant<int, 0>;
  using QS2 = std::integral_constant<int, MM_NS / 2>;
  using QS = std::integral_constant<int, MM_NS>;
  using QF2 = std::integral_constant<int, MM_NS + NF / 2>;
  using QALL = std::integral_constant<int, NQ>;

  // Operand reads: row (block base + l % 32), chunk 2 * kstep + l / 32.
  const int l32 = lane & 31, hi = lane >> 5;
  MMFrags<NI, NJ> f;
  auto read_step = [&](int kt, int ks, auto steady) {   // the operands of one MFMA k-step
    const int h = ks & 1;
    const uint16_t* sh = smem + l32 * MM_BK + (((2 * ks + hi) ^ mm_swz(l32)) << 3);
    const uint16_t* sa = sh + a_slot(kt);
    const uint16_t* sb = sh + b_slot(kt);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = NI == 4 ? a0 + (i & 1) * 32 + (i >> 1) * a_step : a0 + i * a_step;
      f.a[h][i] = *reinterpret_cast<const u32x4_t*>(sa + r * MM_BK);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) f.b[h][j] = *reinterpret_cast<const u32x4_t*>(sb + (MM_TM + b0 + j * 32) * MM_BK);
    if (!steady && kt * MM_BK + ks * 16 >= K) {     // past K in a half-full last stage
#pragma unroll
      for (int j = 0; j < NJ; ++j) f.b[h][j] = u32x4_t{0, 0, 0, 0};
    }
  };
  auto multiply = [&](int h) {   // one MFMA k-step
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32_bf16(f.a[h][i], f.b[h][j], acc[i][j]);
  };
  // Full tile: the 8 operand reads of one k-step go between the first 8 of
  // the 16 MFMAs of the previous k-step, so at most 8 reads are in flight
  // and they have landed by the time their own MFMAs start; `nv` loads from
  // memory go between the last 8 MFMAs (after the reads: the compiler keeps
  // LDS reads and LDS-writing loads in program order).  Half tile: 6 reads
  // over the first 6 of 8 MFMAs and the loads over the last `nv`.
  auto interleave = [](auto nv) {
    constexpr int NV = decltype(nv)::value;
    constexpr int NM = NI * NJ, NR = NI + NJ;
    if constexpr (NM == 16) {
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      }
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // one load
      }
      if constexpr (NR + NV < NM) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR - NV, 0);
    } else {
      static_assert(NV <= NM, "one load per MFMA");
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // one MFMA
        if (q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // one LDS read
        if (q >= NM - NV) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one load
      }
    }
  };
  using fast_loads = std::integral_constant<int, NF / 2>;
  using slow_loads = std::integral_constant<int, MM_NS / 2>;

  // Stage kt with every stage it issues (up to kt + 2) full: straight-line
  // code.  With S the slow operand and F the fast one: k-step 0 issues the
  // second half of F(kt + 1), k-steps 1 and 2 S(kt + 2); the barrier leaves
  // S(kt + 2) in flight; k-step 3 issues the first half of F(kt + 2).
  auto step_steady = [&](int kt) {
    multiply(0);
    read_step(kt, 1, std::true_type{});
    issue(kt + 1, QF2{}, QALL{});
    interleave(fast_loads{});
    __builtin_amdgcn_sched_barrier(0);
    multiply(1);
    read_step(kt, 2, std::true_type{});
    issue(kt + 2, Q0{}, QS2{});
    interleave(slow_loads{});
    __builtin_amdgcn_sched_barrier(0);
    multiply(0);
    read_step(kt, 3, std::true_type{});
    issue(kt + 2, QS2{}, QS{});
    interleave(slow_loads{});
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<MM_NS>();     // all but S(kt + 2): stage kt + 1 landed (this wave's part)
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
    multiply(1);
    read_step(kt + 1, 0, std::true_type{});
    issue(kt + 2, QS{}, QF2{});
    interleave(fast_loads{});
    __builtin_amdgcn_sched_barrier(0);
  };
  // The same issue pattern with guards (last stages, short k loops).
  auto step_tail = [&](int kt) {
    multiply(0);
    read_step(kt, 1, std::false_type{});
    if (kt + 1 < nk) issue(kt + 1, QF2{}, QALL{});
    multiply(1);
    read_step(kt, 2, std::false_type{});
    if (kt + 2 < nk) issue(kt + 2, Q0{}, QS{});
    multiply(0);
    read_step(kt, 3, std::false_type{});
    const bool more = kt + 1 < nk;
    if (more) {
      if (kt + 2 < nk) wait_vmcnt<MM_NS>();
      else wait_vmcnt<0>();
      ring_barrier();
    }
    multiply(1);
    if (more) {
      read_step(kt + 1, 0, std::false_type{});
      if (kt + 2 < nk) issue(kt + 2, QS{}, QF2{});
    }
  };
  // Prologue: stage 0, S(1), the first half of F(1); wait for stage 0.
  issue(0, Q0{}, QALL{});
  if (1 < nk) {
    issue(1, Q0{}, QF2{});
    wait_vmcnt<QF2::value>();
  } else {
    wait_vmcnt<0>();
  }
  ring_barrier();
  read_step(0, 0, std::false_type{});
  int kt = 0;
  for (; kt + 2 < nk_full; ++kt) step_steady(kt);
  for (; kt < nk; ++kt) step_tail(kt);
}

template <int NI, int NJ>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[NI][NJ]) {
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
}

// --------------------------------------------------------------- gate/up --
// Tile: 256 sorted rows (tokens) x 128 intermediate columns.  Staged A rows
// [0, 128) are gate rows, [128, 256) the up rows of the same columns; B rows
// are the gathered token rows.  Full tile: wave (wm, wn) = (w / 2, w % 2)
// multiplies tokens [128 wm, +128) with columns [64 wn, +64) of gate and up
// (A blocks: gate 2, up 2).  Half tile (tokens [0, 128) only): wave w
// multiplies them with columns [32 w, +32) of gate and up (A blocks: gate
// 1, up 1).  Either way a lane holds matching gate and up sums: 4
// consecutive intermediate columns of one token per register group.  Each
// wave stages a quarter of the gate rows, the same up rows and a quarter of
// the tokens.

constexpr int GU_BN = MM_TN / 2;              // intermediate columns per tile

template <bool HALF>
__device__ __forceinline__ void gateup_tile(const PrefillArgs& a, uint16_t* smem, bool routed, int local, int N,
                                            const uint16_t* Wg, const uint16_t* Wu, int n0, int hrow0) {
  constexpr int NI = HALF ? 2 : 4, NJ = 4, NF = HALF ? 4 : 8;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int H = a.H;
  TileLoads ld;
  ld.upper = 0;
  const int lrow = lane >> 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {                 // instructions 0..7: gate / up rows, 8 at a time
    const int r = wv * 32 + j * 8;              // first row within the gate (or up) block
    const int n = n0 + r + lrow;
    const int src = n < N ? n : n0;             // rows past N are read but never stored
    set_load(ld, 2 * j, Wg, r, src, H, lane);
    set_load(ld, 2 * j + 1, Wu, GU_BN + r, src, H, lane);
  }
  const uint16_t* const xb = reinterpret_cast<const uint16_t*>(a.x);
  constexpr int TPW = HALF ? 32 : 64;           // token rows staged per wave
#pragma unroll
  for (int j = 0; j < NF; ++j) {                // instructions 8..: token rows
    const int m = wv * TPW + j * 8 + lrow;
    int tok;
    if (routed) {
      const int fl = a.sorted_ids[hrow0 + m];
      tok = fl < a.T * a.k ? fl / a.k : 0;      // padding rows read a real row; their outputs are never used
    } else {
      tok = local * MM_TM + m;
      tok = tok < a.T ? tok : 0;
    }
    set_load(ld, MM_NS + j, xb, MM_TN + wv * TPW + j * 8, tok, H, lane);
  }

  const int wm = HALF ? 0 : wv >> 1, wn = HALF ? wv : wv & 1;
  constexpr int WC = HALF ? 32 : 64;            // columns of gate (and of up) per wave
  f32x16_t acc[NI][NJ];
  zero_acc(acc);
  mm_tile<1, NI, NJ, NF>(smem, ld, H, wn * WC, GU_BN, wm * 128, acc);

  // epilogue: h[row][n] = bf16(silu(g) * u); A blocks [0, NI/2) are gate, the rest up
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < NI / 2; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + wn * WC + i * 32 + g * 8 + hi * 4;
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int m = wm * 128 + j * 32 + l32;
        float hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[q] = silu_f(acc[i][j][4 * g + q]) * acc[i + NI / 2][j][4 * g + q];
        *reinterpret_cast<u32x2_t*>(a.h + size_t(hrow0 + m) * a.h_stride + n) =
            u32x2_t{pack_bf16(hv[0], hv[1]), pack_bf16(hv[2], hv[3])};
      }
    }
}

// Whether row tile rt has at most 128 rows in use (rows 128 .. 255 are all
// dispatch padding, or past the tokens of a shared expert).
__device__ __forceinline__ bool half_tile(const PrefillArgs& a, int rt, int n_routed_tiles) {
  if (rt < n_routed_tiles) return a.sorted_ids[rt * MM_TM + 128] >= a.T * a.k;
  return (rt - n_routed_tiles) % (a.t_pad / MM_TM) * MM_TM + 128 >= a.T;
}

__global__ void __launch_bounds__(64 * MM_WAVES) prefill_gateup_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const TileList L = tile_list(a, a.n_col_tiles, 1);
  int kr, rt, ct;
  if (!tile_item(blockIdx.x, L, kr, rt, ct)) return;

  const int n_routed_tiles = L.n_routed;
  const int H = a.H;
  int N, local = 0;
  const uint16_t *Wg, *Wu;
  const bool routed = rt < n_routed_tiles;
  if (routed) {
    const int e = a.tile_expert[rt];
    if (e < 0) return;
    N = a.I;
    Wg = a.wg + size_t(e) * a.I * H;
    Wu = a.wu + size_t(e) * a.I * H;
  } else {
    const int tiles_per_shared = a.t_pad / MM_TM;
    const int s = (rt - n_routed_tiles) / tiles_per_shared;
    local = (rt - n_routed_tiles) % tiles_per_shared;
    N = a.Is;
    Wg = a.sg + size_t(s) * a.Is * H;
    Wu = a.su + size_t(s) * a.Is * H;
  }
  const int n0 = ct * GU_BN;
  if (n0 >= N) return;
  if (half_tile(a, rt, n_routed_tiles)) gateup_tile<true>(a, smem, routed, local, N, Wg, Wu, n0, rt * MM_TM);
  else gateup_tile<false>(a, smem, routed, local, N, Wg, Wu, n0, rt * MM_TM);
}

// ------------------------------------------------------------------ down --

// k per range when a reduction of K is cut into ks ranges: whole 64-deep
// stages except maybe at the end; ranges that start at or past K are empty.
__host__ __device__ inline int down_k_chunk(int K, int ks) { return (K + 64 * ks - 1) / (64 * ks) * 64; }

// Tile: 256 sorted rows x 256 hidden columns.  Staged A rows are activation
// rows (sorted order, contiguous), B rows the down-projection rows of the
// hidden outputs.  Full tile: wave (wm, wn) multiplies rows [128 wm, +128)
// with columns [128 wn, +128).  Half tile (rows [0, 128) only): wave w
// multiplies them with columns [64 w, +64).  Register q of a lane holds one
// hidden column of 16 sorted rows, which it scales by the routing weight
// and stores into the sorted row of this k range's partial plane (lanes
// 0-31 cover 32 consecutive columns of one row).  Each wave stages a
// quarter of each operand.

template <bool HALF>
__device__ __forceinline__ void down_tile(const PrefillArgs& a, uint16_t* smem, const uint16_t* Wd, int K, int rt,
                                          int n_routed_tiles, int n0, int kr, int k_begin, int k_len) {
  constexpr int NI = 4, NJ = HALF ? 2 : 4, NF = HALF ? 4 : 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(int(tid >> 6));
  const int H = a.H, hrow0 = rt * MM_TM;
  TileLoads ld;
  ld.upper = 0;
  const int lrow = lane >> 3;
  // The weight rows (B, from HBM) are the slow operand: load instructions
  // 0..7, the activation rows the next NF.
#pragma unroll
  for (int j = 0; j < 8; ++j) {                 // down-projection rows
    const int r = wv * 64 + j * 8;
    const int n = n0 + r + lrow;
    set_load(ld, j, Wd + k_begin, MM_TM + r, n < H ? n : n0, K, lane);   // columns past H are never stored
  }
  constexpr int RPW = HALF ? 32 : 64;           // activation rows staged per wave
#pragma unroll
  for (int j = 0; j < NF; ++j) {                // activation rows
    const int r = wv * RPW + j * 8;
    set_load(ld, MM_NS + j, a.h + k_begin, r, hrow0 + r + lrow, a.h_stride, lane);
  }

  const int wm = HALF ? 0 : wv >> 1, wn = HALF ? wv : wv & 1;
  constexpr int WC = HALF ? 64 : 128;           // hidden columns per wave
  f32x16_t acc[NI][NJ];
  zero_acc(acc);
  mm_tile<2, NI, NJ, NF>(smem, ld, k_len, wm * 128, 64, wn * WC, acc);

  // The tile's token ids (-1: padding) and routing weights of this wave's
  // rows go to the slow operand's slot nk % 3, which no wave reads or fills
  // any more: its last stage (nk - 3) was read before the barrier of stage
  // nk - 2, which every wave has passed, and stage nk is never loaded.  Each
  // wave writes the rows it reads (waves with the same rows write the same
  // values), so no barrier is needed.
  const int nk = (k_len + MM_BK - 1) / MM_BK;
  int* tok_s = reinterpret_cast<int*>(smem + (nk % 3) * MM_HALF);
  float* w_s = reinterpret_cast<float*>(tok_s + MM_TM);
  const int n_asg = a.T * a.k;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int m = wm * 128 + u * 64 + lane;
    if (rt < n_routed_tiles) {
      const int fl = a.sorted_ids[hrow0 + m];
      const bool ok = fl < n_asg;
      tok_s[m] = ok ? fl / a.k : -1;
      w_s[m] = ok ? a.topk_w[fl] : 0.f;
    } else {
      const int t = (rt - n_routed_tiles) % (a.t_pad / MM_TM) * MM_TM + m;
      tok_s[m] = t < a.T ? t : -1;
      w_s[m] = 1.0f;
    }
  }

  // epilogue: partial row (plane kr, sorted row) = w * y
  const int l32 = lane & 31, hi = lane >> 5;
  float* const prow = a.partials + size_t(kr) * a.part_plane + size_t(hrow0) * H;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn * WC + j * 32 + l32;
    if (n >= H) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = wm * 128 + i * 32 + (q >> 2) * 8 + hi * 4 + (q & 3);
        if (tok_s[m] >= 0) prow[size_t(m) * H + n] = w_s[m] * acc[i][j][q];
      }
  }
}

__global__ void __launch_bounds__(64 * MM_WAVES) prefill_down_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  // work-group = (k range, tile)
  const TileList L = tile_list(a, a.n_col_tiles, a.k_split);
  int kr, rt, ct;
  if (!tile_item(blockIdx.x, L, kr, rt, ct)) return;
  const int n_routed_tiles = L.n_routed;
  const int H = a.H;
  int K;
  const uint16_t* Wd;
  if (rt < n_routed_tiles) {
    const int e = a.tile_expert[rt];
    if (e < 0) return;
    K = a.I;
    Wd = a.wd + size_t(e) * H * a.I;
  } else {
    const int tiles_per_shared = a.t_pad / MM_TM;
    const int s = (rt - n_routed_tiles) / tiles_per_shared;
    K = a.Is;
    Wd = a.sd + size_t(s) * H * a.Is;
  }
  const int n0 = ct * MM_TN;
  // this work-group's k range [k_begin, k_begin + k_len): whole 64-deep stages except maybe the end
  const int k_chunk = down_k_chunk(K, a.k_split);
  const int k_begin = kr * k_chunk;
  const int k_len = min(k_chunk, K - k_begin);
  if (k_len <= 0) return;
  if (half_tile(a, rt, n_routed_tiles)) down_tile<true>(a, smem, Wd, K, rt, n_routed_tiles, n0, kr, k_begin, k_len);
  else down_tile<false>(a, smem, Wd, K, rt, n_routed_tiles, n0, kr, k_begin, k_len);
}

// --------------------------------------------------------------- combine --
// out[t] = the k routed partial rows of token t (located through the
// dispatch's inverse permutation), each summed over its k-range planes in
// order, then its shared-expert rows the same way; one fixed order, so the
// output does not depend on the order in which the down tiles finished.
// Planes of k ranges that start past a matrix's own K (a short shared or
// routed reduction) are never written and are not read.  A thread per 4
// outputs.
template <int OT>
__global__ void __launch_bounds__(256) combine_kernel(PrefillArgs a) {
  const long i4 = long(blockIdx.x) * blockDim.x + threadIdx.x;
  const int H4 = a.H / 4;
  if (i4 >= long(a.T) * H4) return;
  const int t = int(i4 / H4), h = int(i4 - long(t) * H4) * 4;
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  auto add_row = [&](long row, int planes) {
    const float* p = a.partials + row * a.H + h;
    for (int q = 0; q < planes; ++q) v += *reinterpret_cast<const f32x4_t*>(p + q * a.part_plane);
  };
  const int pr = (a.I + down_k_chunk(a.I, a.k_split) - 1) / down_k_chunk(a.I, a.k_split);
  for (int j = 0; j < a.k; ++j) add_row(a.inv[t * a.k + j], pr);
  if (a.S > 0) {
    const int ps = (a.Is + down_k_chunk(a.Is, a.k_split) - 1) / down_k_chunk(a.Is, a.k_split);
    for (int s = 0; s < a.S; ++s) add_row(long(a.capacity) + long(s) * a.t_pad + t, ps);
  }
  if constexpr (OT == DT_F32) reinterpret_cast<f32x4_t*>(a.out)[i4] = v;
  else reinterpret_cast<u32x2_t*>(a.out)[i4] = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}

// ---------------------------------------------------------------- launch --

#ifndef MOE_PF_DN_SPLIT
#define MOE_PF_DN_SPLIT 0
#endif
// k ranges per down-projection tile: 1, 2 or 4, enough for about four
// rounds of 256 work-groups, each range at least 1024 deep.
int down_k_split(int tiles, int K) {
  if (MOE_PF_DN_SPLIT > 0) return MOE_PF_DN_SPLIT;
  int s = 1;
  while (s < 4 && tiles * s < 4 * 256 && K / (2 * s) >= 1024) s *= 2;
  return s;
}

// k ranges of the down GEMM for a shape (the host sizes the partial planes by it).
int prefill_k_split(int capacity, int S, int t_pad, int H, int nmax) {
  const int n_rt = capacity / MM_TM + S * (t_pad / MM_TM);
  return down_k_split(n_rt * ((H + MM_TN - 1) / MM_TN), nmax);
}

hipError_t launch_prefill(const PrefillArgs& a, int out_dt, hipStream_t st, StageMarker* mark) {
  // dynamic LDS above 64 KiB must be allowed per kernel (thread-safe one-time set-up)
  static const hipError_t attr_rc = [] {
    hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_gateup_kernel),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, int(MM_LDS));
    hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_down_kernel),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, int(MM_LDS));
    return e1 != hipSuccess ? e1 : e2;
  }();
  if (attr_rc != hipSuccess) return attr_rc;
  if (a.tile_m != MM_TM) return hipErrorInvalidValue;
  const int n_rt = a.capacity / MM_TM + a.S * (a.t_pad / MM_TM);
  PrefillArgs g = a;
  const int nmax = a.I > a.Is ? a.I : a.Is;
  g.n_row_tiles = n_rt;
  g.n_col_tiles = (nmax + GU_BN - 1) / GU_BN;
  hipLaunchKernelGGL(prefill_gateup_kernel, dim3(tile_grid(long(n_rt) * g.n_col_tiles)), dim3(64 * MM_WAVES), MM_LDS, st,
                     g);
  if (mark) mark->mark(st);
  PrefillArgs d = a;
  d.n_row_tiles = n_rt;
  d.n_col_tiles = (a.H + MM_TN - 1) / MM_TN;
  // A few hundred output tiles leave the last round of work-groups mostly
  // idle (one work-group per CU): split k so there are at least ~4 rounds.
  d.k_split = down_k_split(n_rt * d.n_col_tiles, nmax);
  hipLaunchKernelGGL(prefill_down_kernel, dim3(tile_grid(long(n_rt) * d.n_col_tiles * d.k_split)), dim3(64 * MM_WAVES),
                     MM_LDS, st, d);
  if (mark) mark->mark(st);
  const long n = long(a.T) * a.H;
  const int blocks = int((n / 4 + 255) / 256);
  if (out_dt == DT_F32) hipLaunchKernelGGL(combine_kernel<DT_F32>, dim3(blocks), dim3(256), 0, st, d);
  else hipLaunchKernelGGL(combine_kernel<DT_BF16>, dim3(blocks), dim3(256), 0, st, d);
  if (mark) mark->mark(st);
  return hipGetLastError();
}

}  // namespace moe
