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
//                 and adds into an fp32 [T, H] accumulator (the combine);
//   cast          fp32 accumulator -> output dtype.
//
// Tiles: 128 sorted rows x 128 output columns per work-group (for gate/up:
// 128 gate and 128 up columns), 8 waves in a 2 x 4 arrangement (two waves
// per SIMD hide each other's LDS and barrier stalls), k staged 64 at a time.
// Operands move global -> LDS with the gfx950 direct-to-LDS loads (one wave
// instruction = 8 rows x 128 bytes, no register staging) into a ring of LDS
// stages filled ahead of the MFMAs that consume them: 3 stages (144 KiB, one
// work-group per CU) for gate/up, 2 stages (64 KiB, two work-groups per CU)
// for down.
// Because those loads write each row contiguously, rows cannot be padded;
// instead the 16-byte chunks of row r are XOR-permuted by (r >> 1) & 7 so
// that the 16 rows one MFMA operand read touches fall on distinct LDS banks.
// A partial last k stage (K % 64 == 32) is staged through registers with
// zero fill.  Work-group ids are remapped so that the groups resident on one
// XCD (one L2) work on neighbouring tiles.
#include "common.hpp"

namespace moe {

#ifndef MOE_PF_GROUP
#define MOE_PF_GROUP 8
#endif
// Calls f(std::integral_constant<int, i>) for i = B .. E - 1 (compile-time loop).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int PF_BM = 128;     // sorted rows per down-projection tile (divides the dispatch padding)
constexpr int PF_BN = 128;     // output columns per tile
constexpr int PF_BK = 64;      // k per LDS stage: a staged row is 128 bytes = 8 chunks
#ifndef MOE_PF_DN_STAGES
#define MOE_PF_DN_STAGES 2
#endif
constexpr int DN_STAGES = MOE_PF_DN_STAGES;   // down ring depth
constexpr int PF_GROUP = MOE_PF_GROUP;   // row tiles per scheduling group

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// XCD-aware tile order: hardware places work-group b on XCD b % 8.  Give each
// XCD a contiguous range of logical tiles, then walk them in groups of
// PF_GROUP row tiles so that concurrently resident groups share A and B tiles
// in that XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int n_rt, int n_ct, int& rt, int& ct) {
  const int total = n_rt * n_ct;
  const int per = total / 8;
  const int xcd = bid % 8, local = bid / 8;
  const int L = local < per ? xcd * per + local : 8 * per + xcd;   // leftovers when total % 8 != 0
  const int group = L / (PF_GROUP * n_ct);
  const int first = group * PF_GROUP;
  const int gsz = min(PF_GROUP, n_rt - first);
  const int in = L - group * PF_GROUP * n_ct;
  rt = first + in % gsz;
  ct = in / gsz;
}

// Tile order for the gate/up GEMM.  Each XCD (hardware places work-group b
// on XCD b % 8) owns a contiguous range of row tiles, so its resident
// work-groups mostly serve one expert and share that expert's weight tiles
// in its L2.  All XCDs walk the output columns in the same order, in groups
// of GU_CG column tiles (outer) over their row tiles (inner), so the XCDs
// that serve one expert read the same weight columns at about the same time:
// HBM delivers them about once and the
// memory-side cache serves the other XCDs.  Returns false for the padding
// work-groups of a grid of 8 * ceil(n_rt / 8) * n_ct.
#ifndef MOE_PF_GU_CG
#define MOE_PF_GU_CG 4
#endif
constexpr int GU_CG = MOE_PF_GU_CG;
__device__ __forceinline__ bool tile_colgroups(int bid, int n_rt, int n_ct, int& rt, int& ct) {
  const int x = bid & 7, local = bid >> 3;
  const int r8 = (n_rt + 7) >> 3;
  const int g = local / (r8 * GU_CG);
  const int in = local - g * r8 * GU_CG;
  const int ncg = min(GU_CG, n_ct - g * GU_CG);
  ct = g * GU_CG + in % ncg;
  rt = x * r8 + in / ncg;
  return rt < n_rt && ct < n_ct;
}

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Element offset of logical 16-byte chunk c of staged row r.
__device__ __forceinline__ int lds_off(int r, int c) { return r * PF_BK + ((c ^ swz(r)) << 3); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Work-group barrier for the k-stage ring: this wave's LDS reads are complete
// (lgkmcnt 0) and the caller has already waited for its own stage loads.  A
// plain __syncthreads() would also wait for every load still in flight
// (vmcnt 0), which would serialise the ring.  The asm statement clobbers
// memory, so the compiler moves no memory access across it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | (0x0 << 8) | ((0x3F >> 4) << 14));   // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// One wave instruction: 8 staged rows x 128 bytes.  Lane l fills row
// (first row of the group) + l/8, physical chunk l%8, with the logical chunk
// (l%8) ^ swz(row) of its source row.  `src` is this lane's source row at the
// stage's first k; `dst` is the group's first staged row (wave-uniform).
__device__ __forceinline__ void dma_group(const uint16_t* src, int row, int lane, uint16_t* dst) {
  const int c = (lane & 7) ^ swz(row);
  __builtin_amdgcn_global_load_lds((glb_void_t*)(src + c * 8), (lds_void_t*)dst, 16, 0, 0);
}

// Register path for a partial k stage: the same lane -> (row, chunk) mapping,
// zero fill where k >= K.
__device__ __forceinline__ void reg_group(const uint16_t* src, int row, int lane, uint16_t* dst, int k0, int K) {
  const int p = lane & 7, c = p ^ swz(row);
  u32x4_t v = {0, 0, 0, 0};
  if (k0 + c * 8 < K) v = ldg16(src + c * 8);
  *reinterpret_cast<u32x4_t*>(dst + (lane >> 3) * PF_BK + p * 8) = v;
}

// --------------------------------------------------------------- gate/up --
// Tile: 256 sorted rows (tokens) x 128 intermediate columns, i.e. 128 gate
// rows and 128 up rows of the weights.  Four waves, one per SIMD, in a
// 2 x 2 arrangement; each wave accumulates a 128 x 128 block (64 gate + 64 up
// rows x 128 tokens) in 16 32x32 MFMA tiles held in the accumulation
// registers: two MFMAs per 16-byte LDS operand read.  The square 256 x 256
// MFMA tile per work-group is the largest those registers allow and moves
// the fewest bytes per flop through the load path, which limits this
// kernel.  The 32x32x16 form is the one a single wave per SIMD issues at the
// full matrix rate (the 16x16x32 form reaches about 60 % that way).  An LDS
// stage holds GU_BK values of k for all 512 rows (128-byte rows: the load
// path moves 64-byte rows at well under half the rate); the stage is
// multiplied in GU_BK / 16 MFMA k-steps, and while one k-step is multiplied
// the operands of the next are read into the other half of a two-k-step
// register set.
// MFMA A operand = weight rows, B operand = token rows, so a lane's
// accumulator holds groups of 4 consecutive intermediate columns of one
// token.

constexpr int GU_BM = 256;                    // tokens per tile (the dispatch padding of this path)
constexpr int GU_BN = 128;                    // intermediate columns per tile
constexpr int GU_WAVES = 4;
constexpr int GU_ROWS = 2 * GU_BN + GU_BM;    // 512 staged rows: gate, up, tokens
#ifndef MOE_PF_GU_BK
#define MOE_PF_GU_BK 64
#endif
constexpr int GU_BK = MOE_PF_GU_BK;           // k per stage
static_assert(GU_BK == 32 || GU_BK == 64, "gate/up stage depth");
constexpr int GU_KS = GU_BK / 16;             // MFMA k-steps per stage
constexpr int GU_CH = GU_BK / 8;              // 16-byte chunks per staged row
constexpr int GU_RPI = 64 / GU_CH;            // staged rows per load instruction (1 KiB)
constexpr int GU_DMA = GU_ROWS / GU_RPI / GU_WAVES;   // load instructions per wave per stage
constexpr int GU_STAGE = GU_ROWS * GU_BK;     // bf16 elements per stage
#ifndef MOE_PF_GU_STAGES
#define MOE_PF_GU_STAGES (GU_BK == 64 ? 2 : 4)
#endif
constexpr int GU_S = MOE_PF_GU_STAGES;
static_assert(GU_S >= 2 && GU_S * GU_STAGE * 2 <= 163840, "gate/up ring fits LDS");
static_assert((GU_S - 2) * GU_DMA <= 63, "vmcnt range");

// Chunk c of staged row r is stored at position c ^ gu_swz(r): the 16 rows
// that 16 consecutive lanes of an operand read touch (one chunk each) then
// fall on distinct banks, whether the LDS serves 8 or 16 lanes per cycle.
// The swizzle depends on bits 0-3 of r only, so it is the same for a row's
// index within any block that starts at a multiple of 16 rows.
__device__ __forceinline__ int gu_swz(int r) {
  if constexpr (GU_CH == 4) return (((r >> 1) ^ (r >> 3)) & 1) | ((r >> 1) & 2);
  else return (r & 7) ^ ((r >> 3) & 1);
}

struct GUFrags { u32x4_t a[2][4], b[2][4]; };   // [k-step parity][32-row block]

__global__ void __launch_bounds__(64 * GU_WAVES) prefill_gateup_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int rt, ct;
  if (!tile_colgroups(blockIdx.x, a.n_row_tiles, a.n_col_tiles, rt, ct)) return;

  const int n_routed_tiles = a.capacity / GU_BM;
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
    const int tiles_per_shared = a.t_pad / GU_BM;
    const int s = (rt - n_routed_tiles) / tiles_per_shared;
    local = (rt - n_routed_tiles) % tiles_per_shared;
    N = a.Is;
    Wg = a.sg + size_t(s) * a.Is * H;
    Wu = a.su + size_t(s) * a.Is * H;
  }
  const int n0 = ct * GU_BN;
  if (n0 >= N) return;
  const int hrow0 = rt * GU_BM;

  // Each wave stages a quarter of the gate rows, the same up rows and a
  // quarter of the token rows; every wave reads all of them from LDS.  One load instruction stages GU_RPI rows: lane l
  // writes position l % GU_CH of row l / GU_CH with chunk (position ^
  // swizzle) of its source row.  Source addresses are a wave-uniform matrix
  // base plus a 32-bit per-lane element offset (chunk included); gate and up
  // rows share their offsets.
  constexpr int WI = GU_BN / 4 / GU_RPI, TI = GU_BM / 4 / GU_RPI;   // instructions per weight matrix / for tokens
  static_assert(2 * WI + TI == GU_DMA, "staging split");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lrow = lane / GU_CH;
  uint32_t woff[WI], toff[TI];
  unsigned upper = 0;     // bit j: weight (j < WI) or token (WI + j) instruction stages an upper-half chunk
#pragma unroll
  for (int j = 0; j < WI; ++j) {
    const int r = wv * (GU_BN / 4) + j * GU_RPI + lrow;   // row within the gate (or up) block
    const int n = n0 + r;
    const int chunk = (lane % GU_CH) ^ gu_swz(r);
    woff[j] = uint32_t(n < N ? n : n0) * uint32_t(H) + uint32_t(chunk << 3);   // rows past N are never stored
    upper |= unsigned(chunk >= 4) << j;
  }
#pragma unroll
  for (int j = 0; j < TI; ++j) {
    const int m = wv * (GU_BM / 4) + j * GU_RPI + lrow;   // token row within the tile
    int tok;
    if (routed) {
      const int f = a.sorted_ids[hrow0 + m];
      tok = f < a.T * a.k ? f / a.k : 0;      // padding rows read a real row; their outputs are never used
    } else {
      tok = local * GU_BM + m;
      tok = tok < a.T ? tok : 0;
    }
    const int chunk = (lane % GU_CH) ^ gu_swz(2 * GU_BN + m);
    toff[j] = uint32_t(tok) * uint32_t(H) + uint32_t(chunk << 3);
    upper |= unsigned(chunk >= 4) << (WI + j);
  }
  const uint16_t* const xb = reinterpret_cast<const uint16_t*>(a.x);
  // H is a multiple of 32, so with 64-deep stages the last one may hold 32
  // values: there, lanes whose chunk lies past H load the chunk 32 values
  // lower instead (in bounds), and the k-steps past H multiply zeros.
  const int nk = (H + GU_BK - 1) / GU_BK;
  const int nk_full = H / GU_BK;
  // The stage's load instructions, numbered q = 0 .. GU_DMA - 1: gate and up
  // rows alternate, then the token rows.  issue(kt, Q0, Q1) issues Q0..Q1-1.
  auto issue = [&](int kt, auto q0, auto q1) {
    uint16_t* d = smem + (kt % GU_S) * GU_STAGE;
    const int k0 = kt * GU_BK;
    const bool part = k0 + GU_BK > H;
    static_for<decltype(q0)::value, decltype(q1)::value>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      constexpr bool w = q < 2 * WI;
      constexpr int j = w ? q >> 1 : q - 2 * WI;
      const uint16_t* base = w ? ((q & 1) ? Wu : Wg) : xb;
      const uint32_t off = w ? woff[w ? j : 0] : toff[w ? 0 : j];
      constexpr int bit = w ? j : WI + j;
      const int row = w ? (q & 1) * GU_BN + wv * (GU_BN / 4) + j * GU_RPI : 2 * GU_BN + wv * (GU_BM / 4) + j * GU_RPI;
      const int back = (part && ((upper >> bit) & 1)) ? 32 : 0;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(base + (off + uint32_t(k0 - back))),
                                       (lds_void_t*)(d + row * GU_BK), 16, 0, 0);
    });
  };
  using Q0 = std::integral_constant<int, 0>;
  using QALL = std::integral_constant<int, GU_DMA>;
  // In steady state a stage's loads are spread over GU_NP MFMA k-steps: the
  // first part starts right after the barrier that frees its slot, the others
  // go into the next stage's first k-steps, one load between MFMAs, so the
  // matrix cores never wait behind a burst of load issues.  With a 2-deep
  // ring the last part must land before the next barrier, one k-step later.
  constexpr int GU_NP = GU_S == 2 ? GU_KS - 1 : GU_KS;
  constexpr int GU_PQ = (GU_DMA + GU_NP - 1) / GU_NP;      // loads per part
  static_assert(GU_PQ <= 8, "one load per MFMA pair");
  // Operand reads: row (block base + l%32), chunk 2 * kstep + l/32.  Blocks
  // start at multiples of 32 rows, so the lane's offset inside a block
  // depends on the lane and the k-step only.
  // Wave (wm, wn) = (wv / 2, wv % 2) multiplies tokens [128 wm, 128 wm + 128)
  // with intermediate columns [64 wn, 64 wn + 64) of gate and up.
  const int l32 = lane & 31, hi = lane >> 5;
  const int wm = wv >> 1, wn = wv & 1;
  const int a_row = wn * 64 * GU_BK, b_row = (2 * GU_BN + wm * 128) * GU_BK;
  auto read_step = [&](int kt, int ks, GUFrags& f, auto steady) {   // the operands of one MFMA k-step
    const int h = ks & 1;
    const uint16_t* sh = smem + (kt % GU_S) * GU_STAGE + l32 * GU_BK + (((2 * ks + hi) ^ gu_swz(l32)) << 3);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f.a[h][i] = *reinterpret_cast<const u32x4_t*>(sh + a_row + i * 32 * GU_BK);
      f.a[h][i + 2] = *reinterpret_cast<const u32x4_t*>(sh + a_row + (GU_BN + i * 32) * GU_BK);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[h][j] = *reinterpret_cast<const u32x4_t*>(sh + b_row + j * 32 * GU_BK);
    if (!steady && kt * GU_BK + ks * 16 >= H) {     // past H in a partial last stage
#pragma unroll
      for (int j = 0; j < 4; ++j) f.b[h][j] = u32x4_t{0, 0, 0, 0};
    }
  };

  f32x16_t acc[4][4];   // [weight block: gate 0-1, up 2-3][token block]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  auto multiply = [&](const GUFrags& f, int h) {   // one MFMA k-step
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32_bf16(f.a[h][i], f.b[h][j], acc[i][j]);
  };
  // The 8 operand reads of one k-step go between the first 8 of the 16 MFMAs
  // of the previous k-step, so at most 8 reads are in flight and they have
  // landed by the time their own MFMAs start; `nv` loads from memory go
  // between the last 8 MFMAs (after the reads: the compiler keeps LDS reads
  // and LDS-writing loads in program order).
  auto interleave = [](auto nv) {
    constexpr int NV = decltype(nv)::value;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // one load
    }
    if constexpr (NV < 8) __builtin_amdgcn_sched_group_barrier(0x008, 8 - NV, 0);
  };
  using no_loads = std::integral_constant<int, 0>;
  using part_loads = std::integral_constant<int, GU_PQ>;
  auto wait_newer = [&](int newer) {   // this wave's loads of all but the `newer` latest stages landed
    if (newer >= 2) wait_vmcnt<2 * GU_DMA>();
    else if (newer == 1) wait_vmcnt<GU_DMA>();
    else wait_vmcnt<0>();
  };
  // One stage.  Before its last k-step every read of stage kt has been
  // issued; the barrier there (which also waits for this wave's reads) makes
  // the slot of stage kt free and stage kt + 1 visible, so the slot is
  // refilled with stage kt + GU_S while the last k-step is multiplied and
  // the first operands of stage kt + 1 are read.
  // Steady state (kt + GU_S < nk_full): straight-line code; the refill of a
  // slot is spread: part 0 of stage kt + GU_S goes into the last k-step of
  // stage kt, parts 1 .. GU_NP - 1 into the first k-steps of stage kt + 1.
  GUFrags f;
  auto step_steady = [&](int kt) {
    static_for<0, GU_KS - 1>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      multiply(f, ks & 1);
      read_step(kt, ks + 1, f, std::true_type{});
      if constexpr (ks + 1 < GU_NP) {
        issue(kt - 1 + GU_S, std::integral_constant<int, (ks + 1) * GU_PQ>{},
              std::integral_constant<int, ((ks + 2) * GU_PQ < GU_DMA ? (ks + 2) * GU_PQ : GU_DMA)>{});
        interleave(part_loads{});
      } else {
        interleave(no_loads{});
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    wait_vmcnt<(GU_S - 2) * GU_DMA>();     // stage kt + 1 landed; kt + 2 .. kt + S - 1 may be in flight
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
    multiply(f, (GU_KS - 1) & 1);
    read_step(kt + 1, 0, f, std::true_type{});
    issue(kt + GU_S, Q0{}, std::integral_constant<int, GU_PQ>{});
    interleave(part_loads{});
    __builtin_amdgcn_sched_barrier(0);
  };
  // The last stages (and every stage of a short k loop): loads are issued
  // whole; `pend` says the previous (steady) stage left refill parts 1.. of
  // stage kt - 1 + GU_S to this one.
  auto step_tail = [&](int kt, bool pend) {
    if (pend) issue(kt - 1 + GU_S, std::integral_constant<int, GU_PQ>{}, QALL{});
    static_for<0, GU_KS - 1>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      multiply(f, ks & 1);
      read_step(kt, ks + 1, f, std::false_type{});
    });
    const bool more = kt + 1 < nk;
    if (more) {
      wait_newer(min(kt + GU_S - 1, nk - 1) - (kt + 1));
      ring_barrier();
    }
    multiply(f, (GU_KS - 1) & 1);
    if (more) {
      read_step(kt + 1, 0, f, std::false_type{});
      if (kt + GU_S < nk) issue(kt + GU_S, Q0{}, QALL{});
    }
  };

  // Prologue: stages 0 .. GU_S - 1 (the last one only its part 0 when a
  // steady step follows), then wait for stage 0.
  const bool piped = GU_S < nk_full;
#pragma unroll
  for (int p = 0; p < GU_S - 1; ++p)
    if (p < nk) issue(p, Q0{}, QALL{});
  if (GU_S - 1 < nk) {
    if (piped) issue(GU_S - 1, Q0{}, std::integral_constant<int, GU_PQ>{});
    else issue(GU_S - 1, Q0{}, QALL{});
  }
  if (piped) wait_vmcnt<(GU_S - 2) * GU_DMA + GU_PQ>();
  else wait_newer(min(GU_S, nk) - 1);
  ring_barrier();
  read_step(0, 0, f, std::false_type{});
  int kt = 0;
  for (; kt + GU_S < nk_full; ++kt) step_steady(kt);
  bool pend = piped;
  for (; kt < nk; ++kt) {
    step_tail(kt, pend);
    pend = false;
  }

  // epilogue: h[row][n] = bf16(silu(g) * u); register q of a tile holds
  // column n = 8 (q / 4) + 4 (l / 32) + q % 4 of the 32-row weight block
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + wn * 64 + i * 32 + g * 8 + hi * 4;
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = wm * 128 + j * 32 + l32;
        float hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[q] = silu_f(acc[i][j][4 * g + q]) * acc[i + 2][j][4 * g + q];
        *reinterpret_cast<u32x2_t*>(a.h + size_t(hrow0 + m) * a.h_stride + n) =
            u32x2_t{pack_bf16(hv[0], hv[1]), pack_bf16(hv[2], hv[3])};
      }
    }
}

// ------------------------------------------------------------------ down --
// Staged rows per k stage: [0,128) activation rows (sorted order), [128,256)
// down-projection rows (hidden outputs).  MFMA A operand = activation rows,
// B operand = down rows; a lane's accumulator holds 4 sorted rows of one
// hidden column, which it scales by the routing weight and adds into the fp32
// accumulator with hardware float atomics.

#ifndef MOE_PF_DN_WAVES
#define MOE_PF_DN_WAVES 8
#endif
constexpr int DN_WAVES = MOE_PF_DN_WAVES;            // 4: 2x2 wave grid, 8: 2x4
constexpr int DN_ROWS = PF_BM + PF_BN;               // 256
constexpr int DN_GROUPS_PER_WAVE = DN_ROWS / 8 / DN_WAVES;
constexpr int DN_WN = DN_WAVES / 2;
constexpr int DN_NF = PF_BN / DN_WN / 16;            // 16-column fragments per wave

__global__ void __launch_bounds__(64 * DN_WAVES) prefill_down_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ int tok_s[PF_BM];
  __shared__ float w_s[PF_BM];
  constexpr int STAGE = DN_ROWS * PF_BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int rt, ct;
  tile_of(blockIdx.x, a.n_row_tiles, a.n_col_tiles, rt, ct);
  const int n_routed_tiles = a.capacity / PF_BM;
  const int H = a.H;
  int K;
  const uint16_t* Wd;
  if (rt < n_routed_tiles) {
    const int e = a.tile_expert[rt * PF_BM / a.tile_m];   // expert segments are padded to whole tile_m rows
    if (e < 0) return;
    K = a.I;
    Wd = a.wd + size_t(e) * H * a.I;
    if (tid < PF_BM) {
      const int f = a.sorted_ids[rt * PF_BM + tid];
      const bool ok = f < a.T * a.k;
      tok_s[tid] = ok ? f / a.k : -1;
      w_s[tid] = ok ? a.topk_w[f] : 0.f;
    }
  } else {
    const int tiles_per_shared = a.t_pad / PF_BM;
    const int s = (rt - n_routed_tiles) / tiles_per_shared;
    const int local = (rt - n_routed_tiles) % tiles_per_shared;
    K = a.Is;
    Wd = a.sd + size_t(s) * H * a.Is;
    if (tid < PF_BM) {
      const int t = local * PF_BM + tid;
      tok_s[tid] = t < a.T ? t : -1;
      w_s[tid] = 1.0f;
    }
  }
  const int n0 = ct * PF_BN;
  const int hrow0 = rt * PF_BM;

  const uint16_t* src[DN_GROUPS_PER_WAVE];
  int srow[DN_GROUPS_PER_WAVE];
#pragma unroll
  for (int j = 0; j < DN_GROUPS_PER_WAVE; ++j) {
    const int r = (wave * DN_GROUPS_PER_WAVE + j) * 8 + (lane >> 3);
    srow[j] = r;
    if (r < PF_BM) {
      src[j] = a.h + size_t(hrow0 + r) * a.h_stride;
    } else {
      const int n = n0 + r - PF_BM;
      src[j] = Wd + size_t(n < H ? n : n0) * K;     // H % 128 may leave a partial tile
    }
  }
  const int nk = (K + PF_BK - 1) / PF_BK;
  const bool k_tail = (K % PF_BK) != 0;
  auto stage_in = [&](int kt) {
    uint16_t* s = smem + (kt % DN_STAGES) * STAGE;
    const int k0 = kt * PF_BK;
    if (!(k_tail && kt == nk - 1)) {
#pragma unroll
      for (int j = 0; j < DN_GROUPS_PER_WAVE; ++j)
        dma_group(src[j] + k0, srow[j], lane, s + (wave * DN_GROUPS_PER_WAVE + j) * 8 * PF_BK);
    } else {
#pragma unroll
      for (int j = 0; j < DN_GROUPS_PER_WAVE; ++j)
        reg_group(src[j] + k0, srow[j], lane, s + (wave * DN_GROUPS_PER_WAVE + j) * 8 * PF_BK, k0, K);
    }
  };
  const int wm = wave / DN_WN, wn = wave % DN_WN;
  const int g = lane >> 4, l16 = lane & 15;
  f32x4_t acc[4][DN_NF];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < DN_NF; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // ring of DN_STAGES slots, loads issued DN_STAGES - 1 stages ahead
  constexpr int AHEAD = DN_STAGES - 1;
#pragma unroll
  for (int p = 0; p < AHEAD; ++p)
    if (p < nk) stage_in(p);
  static_assert(AHEAD >= 1 && AHEAD <= 3, "ring depth 2..4");
  for (int kt = 0; kt < nk; ++kt) {
    const int newer = min(kt + AHEAD - 1, nk - 1) - kt;   // stages issued after stage kt, still allowed in flight
    if (newer >= 2) wait_vmcnt<2 * DN_GROUPS_PER_WAVE>();
    else if (newer == 1) wait_vmcnt<DN_GROUPS_PER_WAVE>();
    else wait_vmcnt<0>();
    ring_barrier();
    if (kt + AHEAD < nk) stage_in(kt + AHEAD);
    const uint16_t* s = smem + (kt % DN_STAGES) * STAGE;
#pragma unroll
    for (int ks = 0; ks < PF_BK / 32; ++ks) {
      const int c = ks * 4 + g;
      u32x4_t ha[4], wb[DN_NF];
#pragma unroll
      for (int i = 0; i < 4; ++i) ha[i] = *reinterpret_cast<const u32x4_t*>(s + lds_off(wm * 64 + i * 16 + l16, c));
#pragma unroll
      for (int j = 0; j < DN_NF; ++j)
        wb[j] = *reinterpret_cast<const u32x4_t*>(s + lds_off(PF_BM + wn * (DN_NF * 16) + j * 16 + l16, c));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < DN_NF; ++j) acc[i][j] = mfma_bf16(ha[i], wb[j], acc[i][j]);
    }
  }

  // epilogue: acc[t][n] += w * y
#pragma unroll
  for (int j = 0; j < DN_NF; ++j) {
    const int n = n0 + wn * (DN_NF * 16) + j * 16 + l16;
    if (n >= H) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wm * 64 + i * 16 + g * 4 + q;
        const int t = tok_s[m];
        if (t >= 0) unsafeAtomicAdd(a.acc + size_t(t) * H + n, w_s[m] * acc[i][j][q]);
      }
    }
  }
}

// ------------------------------------------------------------------ cast --

template <int OT>
__global__ void __launch_bounds__(256) cast_kernel(const float* __restrict__ acc, void* out, long n) {
  const long i4 = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i4 * 4 >= n) return;
  f32x4_t v = reinterpret_cast<const f32x4_t*>(acc)[i4];
  if constexpr (OT == DT_F32) reinterpret_cast<f32x4_t*>(out)[i4] = v;
  else reinterpret_cast<u32x2_t*>(out)[i4] = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}

// ---------------------------------------------------------------- launch --

size_t prefill_gateup_lds() { return size_t(GU_S) * GU_STAGE * sizeof(uint16_t); }
size_t prefill_down_lds() { return size_t(DN_STAGES) * DN_ROWS * PF_BK * sizeof(uint16_t); }

hipError_t launch_prefill(const PrefillArgs& a, int out_dt, hipStream_t st, StageMarker* mark) {
  // dynamic LDS above 64 KiB must be allowed per kernel (thread-safe one-time set-up)
  static const hipError_t attr_rc = [] {
    hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_gateup_kernel),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, int(prefill_gateup_lds()));
    hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_down_kernel),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, int(prefill_down_lds()));
    return e1 != hipSuccess ? e1 : e2;
  }();
  if (attr_rc != hipSuccess) return attr_rc;
  PrefillArgs g = a;
  const int nmax = a.I > a.Is ? a.I : a.Is;
  g.n_row_tiles = a.capacity / GU_BM + a.S * (a.t_pad / GU_BM);
  g.n_col_tiles = (nmax + GU_BN - 1) / GU_BN;
  hipLaunchKernelGGL(prefill_gateup_kernel, dim3(8 * ((g.n_row_tiles + 7) / 8) * g.n_col_tiles), dim3(64 * GU_WAVES),
                     prefill_gateup_lds(), st, g);
  if (mark) mark->mark(st);
  PrefillArgs d = a;
  d.n_row_tiles = a.capacity / PF_BM + a.S * (a.t_pad / PF_BM);
  d.n_col_tiles = (a.H + PF_BN - 1) / PF_BN;
  hipLaunchKernelGGL(prefill_down_kernel, dim3(d.n_row_tiles * d.n_col_tiles), dim3(64 * DN_WAVES),
                     prefill_down_lds(), st, d);
  if (mark) mark->mark(st);
  const long n = long(a.T) * a.H;
  const int blocks = int((n / 4 + 255) / 256);
  if (out_dt == DT_F32) hipLaunchKernelGGL(cast_kernel<DT_F32>, dim3(blocks), dim3(256), 0, st, a.acc, a.out, n);
  else hipLaunchKernelGGL(cast_kernel<DT_BF16>, dim3(blocks), dim3(256), 0, st, a.acc, a.out, n);
  if (mark) mark->mark(st);
  return hipGetLastError();
}

}  // namespace moe
