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
constexpr int PF_BM = 128;     // sorted rows per tile (== dispatch padding tile)
constexpr int PF_BN = 128;     // output columns per tile
constexpr int PF_BK = 64;      // k per LDS stage: a staged row is 128 bytes = 8 chunks
constexpr int PF_STAGES = 3;   // gate/up ring depth (144 KiB of LDS)
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
// Staged rows per k stage: [0,128) gate rows, [128,256) up rows, [256,384)
// gathered x rows.  MFMA A operand = weight rows, B operand = token rows, so
// a lane's accumulator holds 4 consecutive intermediate columns of one token.

#ifndef MOE_PF_GU_WAVES
#define MOE_PF_GU_WAVES 8
#endif
constexpr int GU_WAVES = MOE_PF_GU_WAVES;            // 4: 2x2 wave grid, 8: 2x4
constexpr int GU_ROWS = 2 * PF_BN + PF_BM;           // 384
constexpr int GU_GROUPS_PER_WAVE = GU_ROWS / 8 / GU_WAVES;
constexpr int GU_WN = GU_WAVES / 2;                  // waves across the columns
constexpr int GU_NF = PF_BN / GU_WN / 16;            // 16-column fragments per wave (gate and up each)

__global__ void __launch_bounds__(64 * GU_WAVES) prefill_gateup_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr int STAGE = GU_ROWS * PF_BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int rt, ct;
  tile_of(blockIdx.x, a.n_row_tiles, a.n_col_tiles, rt, ct);

  const int n_routed_tiles = a.capacity / PF_BM;
  const int H = a.H;
  int N, e_or_s;
  const uint16_t *Wg, *Wu;
  const bool routed = rt < n_routed_tiles;
  int local = 0;
  if (routed) {
    e_or_s = a.tile_expert[rt];
    if (e_or_s < 0) return;
    N = a.I;
    Wg = a.wg + size_t(e_or_s) * a.I * H;
    Wu = a.wu + size_t(e_or_s) * a.I * H;
  } else {
    const int tiles_per_shared = a.t_pad / PF_BM;
    e_or_s = (rt - n_routed_tiles) / tiles_per_shared;
    local = (rt - n_routed_tiles) % tiles_per_shared;
    N = a.Is;
    Wg = a.sg + size_t(e_or_s) * a.Is * H;
    Wu = a.su + size_t(e_or_s) * a.Is * H;
  }
  const int n0 = ct * PF_BN;
  if (n0 >= N) return;
  const int hrow0 = rt * PF_BM;

  // this lane's source row for each of its wave's 12 staged 8-row groups
  const uint16_t* src[GU_GROUPS_PER_WAVE];
  int srow[GU_GROUPS_PER_WAVE];
#pragma unroll
  for (int j = 0; j < GU_GROUPS_PER_WAVE; ++j) {
    const int r = (wave * GU_GROUPS_PER_WAVE + j) * 8 + (lane >> 3);
    srow[j] = r;
    if (r < 2 * PF_BN) {
      const int n = n0 + (r & (PF_BN - 1));
      src[j] = (r < PF_BN ? Wg : Wu) + size_t(n < N ? n : n0) * H;
    } else {
      const int m = r - 2 * PF_BN;
      int tok;
      if (routed) {
        const int f = a.sorted_ids[hrow0 + m];
        tok = f < a.T * a.k ? f / a.k : 0;        // padding rows read a real row; their outputs are never used
      } else {
        tok = local * PF_BM + m;
        tok = tok < a.T ? tok : 0;
      }
      src[j] = reinterpret_cast<const uint16_t*>(a.x) + size_t(tok) * H;
    }
  }
  const int nk = (H + PF_BK - 1) / PF_BK;
  const bool k_tail = (H % PF_BK) != 0;
  auto stage_in = [&](int kt) {
    uint16_t* s = smem + (kt % PF_STAGES) * STAGE;
    const int k0 = kt * PF_BK;
    if (!(k_tail && kt == nk - 1)) {
#pragma unroll
      for (int j = 0; j < GU_GROUPS_PER_WAVE; ++j)
        dma_group(src[j] + k0, srow[j], lane, s + (wave * GU_GROUPS_PER_WAVE + j) * 8 * PF_BK);
    } else {
#pragma unroll
      for (int j = 0; j < GU_GROUPS_PER_WAVE; ++j)
        reg_group(src[j] + k0, srow[j], lane, s + (wave * GU_GROUPS_PER_WAVE + j) * 8 * PF_BK, k0, H);
    }
  };

  const int wn = wave % GU_WN, wm = wave / GU_WN;
  const int g = lane >> 4, l16 = lane & 15;
  f32x4_t accg[GU_NF][4], accu[GU_NF][4];
#pragma unroll
  for (int i = 0; i < GU_NF; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) accg[i][j] = accu[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  stage_in(0);
  if (nk > 1) stage_in(1);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) wait_vmcnt<GU_GROUPS_PER_WAVE>();   // stage kt landed; kt+1 may be in flight
    else wait_vmcnt<0>();
    ring_barrier();                                       // every wave's part of stage kt landed,
    if (kt + 2 < nk) stage_in(kt + 2);                    // and every wave is done with stage kt-1
    const uint16_t* s = smem + (kt % PF_STAGES) * STAGE;
#pragma unroll
    for (int ks = 0; ks < PF_BK / 32; ++ks) {
      const int c = ks * 4 + g;
      u32x4_t ga[GU_NF], ua[GU_NF], xb[4];
#pragma unroll
      for (int i = 0; i < GU_NF; ++i) {
        const int rg = wn * (GU_NF * 16) + i * 16 + l16;
        ga[i] = *reinterpret_cast<const u32x4_t*>(s + lds_off(rg, c));
        ua[i] = *reinterpret_cast<const u32x4_t*>(s + lds_off(PF_BN + rg, c));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xb[j] = *reinterpret_cast<const u32x4_t*>(s + lds_off(2 * PF_BN + wm * 64 + j * 16 + l16, c));
#pragma unroll
      for (int i = 0; i < GU_NF; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          accg[i][j] = mfma_bf16(ga[i], xb[j], accg[i][j]);
          accu[i][j] = mfma_bf16(ua[i], xb[j], accu[i][j]);
        }
    }
  }

  // epilogue: h[row][n] = bf16(silu(g) * u)
#pragma unroll
  for (int i = 0; i < GU_NF; ++i) {
    const int n = n0 + wn * (GU_NF * 16) + i * 16 + g * 4;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = wm * 64 + j * 16 + l16;
      float hv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[q] = silu_f(accg[i][j][q]) * accu[i][j][q];
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
    const int e = a.tile_expert[rt];
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

size_t prefill_gateup_lds() { return size_t(PF_STAGES) * GU_ROWS * PF_BK * sizeof(uint16_t); }
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
  g.n_col_tiles = (nmax + PF_BN - 1) / PF_BN;
  hipLaunchKernelGGL(prefill_gateup_kernel, dim3(g.n_row_tiles * g.n_col_tiles), dim3(64 * GU_WAVES),
                     prefill_gateup_lds(), st, g);
  if (mark) mark->mark(st);
  PrefillArgs d = a;
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
