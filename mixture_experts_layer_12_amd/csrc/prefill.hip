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
// Tiles: 128 sorted rows x 128 output columns per work-group, 4 waves in a
// 2 x 2 arrangement, k staged 64 at a time through double-buffered LDS with
// the next stage's global loads in flight during the current stage's MFMAs.
// Rows are padded to 72 bf16 (144 bytes) in LDS so that the 16 rows read by
// one 16-lane group land on distinct banks.  Work-group ids are remapped so
// that the groups resident on one XCD (one L2) work on neighbouring tiles.
#include "common.hpp"

namespace moe {

constexpr int PF_BM = 128;     // sorted rows per tile (== dispatch padding tile)
constexpr int PF_BN = 128;     // output columns per tile
constexpr int PF_BK = 64;      // k per LDS stage
constexpr int PF_LD = PF_BK + 8;   // LDS row stride in bf16 elements
constexpr int PF_GROUP = 8;    // row tiles per scheduling group

// XCD-aware tile order: hardware places work-group b on XCD b % 8.  Give each
// XCD a contiguous range of logical tiles, then walk them in groups of
// PF_GROUP row tiles so that concurrently resident groups share A and B tiles
// in that XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int n_rt, int n_ct, int& rt, int& ct) {
  const int total = n_rt * n_ct;
  const int per = total / 8, extra = total % 8;
  const int xcd = bid % 8, local = bid / 8;
  int L;
  if (local < per) L = xcd * per + local;
  else L = 8 * per + xcd;                 // leftovers (only when extra > 0)
  (void)extra;
  const int group = L / (PF_GROUP * n_ct);
  const int first = group * PF_GROUP;
  const int gsz = min(PF_GROUP, n_rt - first);
  const int in = L - group * PF_GROUP * n_ct;
  rt = first + in % gsz;
  ct = in / gsz;
}

// --------------------------------------------------------------- gate/up --
// MFMA A operand = weight rows (gate rows 0..127 and up rows 128..255 of the
// stage), B operand = gathered token rows, so the accumulator of a lane holds
// 4 consecutive intermediate columns of one token row.

__global__ void __launch_bounds__(256) prefill_gateup_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr int ROWS = 2 * PF_BN + PF_BM;      // gate, up, x rows per stage
  constexpr int STAGE = ROWS * PF_LD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int rt, ct;
  tile_of(blockIdx.x, a.n_row_tiles, a.n_col_tiles, rt, ct);

  const int n_routed_tiles = a.capacity / PF_BM;
  const int H = a.H;
  int N;
  const uint16_t *Wg, *Wu;
  int hrow0 = rt * PF_BM;
  int tokrow[4];                      // token of this thread's 4 staged x rows (-1 = padding)
  const int kc = tid & 7, r0 = tid >> 3;
  if (rt < n_routed_tiles) {
    const int e = a.tile_expert[rt];
    if (e < 0) return;
    N = a.I;
    Wg = a.wg + size_t(e) * a.I * H;
    Wu = a.wu + size_t(e) * a.I * H;
    const int n = a.T * a.k;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = a.sorted_ids[rt * PF_BM + r0 + 32 * j];
      tokrow[j] = f < n ? f / a.k : -1;
    }
  } else {
    const int tiles_per_shared = a.t_pad / PF_BM;
    const int s = (rt - n_routed_tiles) / tiles_per_shared;
    const int local = (rt - n_routed_tiles) % tiles_per_shared;
    N = a.Is;
    Wg = a.sg + size_t(s) * a.Is * H;
    Wu = a.su + size_t(s) * a.Is * H;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = local * PF_BM + r0 + 32 * j;
      tokrow[j] = t < a.T ? t : -1;
    }
  }
  const int n0 = ct * PF_BN;
  if (n0 >= N) return;

  // global -> register staging: 8 weight chunks + 4 x chunks of 16 bytes
  const uint16_t* xptr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    xptr[j] = reinterpret_cast<const uint16_t*>(a.x) + size_t(tokrow[j] < 0 ? 0 : tokrow[j]) * H + kc * 8;
  const uint16_t* wptr[8];
  bool wok[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = r0 + 32 * (j & 3);
    const int n = n0 + r;
    wok[j] = n < N;
    wptr[j] = (j < 4 ? Wg : Wu) + size_t(wok[j] ? n : n0) * H + kc * 8;
  }
  const int nk = (H + PF_BK - 1) / PF_BK;
  u32x4_t stg[12];
  const u32x4_t z4 = {0, 0, 0, 0};
  auto gload = [&](int kt) {
    const int k = kt * PF_BK + kc * 8;
    const bool kok = k < H;
#pragma unroll
    for (int j = 0; j < 8; ++j) stg[j] = (wok[j] && kok) ? ldg16(wptr[j] + size_t(kt) * PF_BK) : z4;
#pragma unroll
    for (int j = 0; j < 4; ++j) stg[8 + j] = (tokrow[j] >= 0 && kok) ? ldg16(xptr[j] + size_t(kt) * PF_BK) : z4;
  };
  auto sstore = [&](int buf) {
    uint16_t* s = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = (j < 4 ? 0 : PF_BN) + r0 + 32 * (j & 3);
      *reinterpret_cast<u32x4_t*>(s + row * PF_LD + kc * 8) = stg[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4_t*>(s + (2 * PF_BN + r0 + 32 * j) * PF_LD + kc * 8) = stg[8 + j];
  };

  // wave tile: 64 intermediate columns (gate and up) x 64 token rows
  const int wn = wave & 1, wm = wave >> 1;
  const int g = lane >> 4, l16 = lane & 15;
  f32x4_t accg[4][4], accu[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) accg[i][j] = accu[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* s = smem + buf * STAGE;
#pragma unroll
    for (int ks = 0; ks < PF_BK / 32; ++ks) {
      const int ko = ks * 32 + g * 8;
      u32x4_t ga[4], ua[4], xb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ga[i] = *reinterpret_cast<const u32x4_t*>(s + (wn * 64 + i * 16 + l16) * PF_LD + ko);
        ua[i] = *reinterpret_cast<const u32x4_t*>(s + (PF_BN + wn * 64 + i * 16 + l16) * PF_LD + ko);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xb[j] = *reinterpret_cast<const u32x4_t*>(s + (2 * PF_BN + wm * 64 + j * 16 + l16) * PF_LD + ko);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          accg[i][j] = mfma_bf16(ga[i], xb[j], accg[i][j]);
          accu[i][j] = mfma_bf16(ua[i], xb[j], accu[i][j]);
        }
    }
    if (kt + 1 < nk) {
      sstore(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: h[row][n] = bf16(silu(g) * u)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + wn * 64 + i * 16 + g * 4;
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
// MFMA A operand = activation rows (sorted order), B operand = down-projection
// rows (hidden outputs); a lane's accumulator holds 4 sorted rows of one
// hidden column, which it scales by the routing weight and adds into the fp32
// accumulator with hardware float atomics.

__global__ void __launch_bounds__(256) prefill_down_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ int tok_s[PF_BM];
  __shared__ float w_s[PF_BM];
  constexpr int ROWS = 2 * PF_BM;
  constexpr int STAGE = ROWS * PF_LD;
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
  const int kc = tid & 7, r0 = tid >> 3;
  const uint16_t* hptr[4];
  const uint16_t* wptr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hptr[j] = a.h + size_t(hrow0 + r0 + 32 * j) * a.h_stride + kc * 8;
    wptr[j] = Wd + size_t(n0 + r0 + 32 * j) * K + kc * 8;   // H % 128 may leave a partial tile
  }
  bool wok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wok[j] = n0 + r0 + 32 * j < H;
  const int nk = (K + PF_BK - 1) / PF_BK;
  u32x4_t stg[8];
  const u32x4_t z4 = {0, 0, 0, 0};
  auto gload = [&](int kt) {
    const int k = kt * PF_BK + kc * 8;
    const bool kok = k < K;
#pragma unroll
    for (int j = 0; j < 4; ++j) stg[j] = kok ? ldg16(hptr[j] + size_t(kt) * PF_BK) : z4;
#pragma unroll
    for (int j = 0; j < 4; ++j) stg[4 + j] = (kok && wok[j]) ? ldg16(wptr[j] + size_t(kt) * PF_BK) : z4;
  };
  auto sstore = [&](int buf) {
    uint16_t* s = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4_t*>(s + (r0 + 32 * j) * PF_LD + kc * 8) = stg[j];
      *reinterpret_cast<u32x4_t*>(s + (PF_BM + r0 + 32 * j) * PF_LD + kc * 8) = stg[4 + j];
    }
  };
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, l16 = lane & 15;
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* s = smem + buf * STAGE;
#pragma unroll
    for (int ks = 0; ks < PF_BK / 32; ++ks) {
      const int ko = ks * 32 + g * 8;
      u32x4_t ha[4], wb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ha[i] = *reinterpret_cast<const u32x4_t*>(s + (wm * 64 + i * 16 + l16) * PF_LD + ko);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wb[j] = *reinterpret_cast<const u32x4_t*>(s + (PF_BM + wn * 64 + j * 16 + l16) * PF_LD + ko);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(ha[i], wb[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      sstore(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: acc[t][n] += w * y
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + j * 16 + l16;
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

size_t prefill_gateup_lds() { return size_t(2) * (2 * PF_BN + PF_BM) * PF_LD * sizeof(uint16_t); }
size_t prefill_down_lds() { return size_t(2) * (2 * PF_BM) * PF_LD * sizeof(uint16_t); }

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
  hipLaunchKernelGGL(prefill_gateup_kernel, dim3(g.n_row_tiles * g.n_col_tiles), dim3(256),
                     prefill_gateup_lds(), st, g);
  if (mark) mark->mark(st);
  PrefillArgs d = a;
  d.n_col_tiles = (a.H + PF_BN - 1) / PF_BN;
  hipLaunchKernelGGL(prefill_down_kernel, dim3(d.n_row_tiles * d.n_col_tiles), dim3(256),
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
