// Router: logits GEMV/GEMM on MFMA, then (in the last work-group to finish)
// softmax, top-k with renormalisation and the dispatch into expert-sorted
// order.
//
// Sources: "Fused MoE kernel on Triton: 5 launches vs 24" (ai-manual.ru),
// section "Fused kernel: one operation instead of twenty-four": routing
// (top-k weights) and dispatch each take one launch in the fused design; here
// both sit in one launch.  "Why MoE on RTX 5090 falls short: a bandwidth
// measurement" (news.malakhovai.ru), paragraph on the kernel-time split:
// top-k plus row gathering are a small share of decode time, so this kernel
// favours few launches and full-chip parallelism for the logits read over
// cleverness in the top-k.
//
// Logits: rows = experts (A operand, router weights), columns = tokens
// (B operand, x).  One work-group owns a 16-expert x 16-token tile; its waves
// split H and reduce through LDS.  Accumulation is fp32: bf16 x bf16 products
// are exact in fp32; fp32 activations against bf16 weights are split into a
// bf16 hi + lo pair (two MFMAs); fp32 x fp32 uses the fp32 MFMA.
#include "common.hpp"

namespace moe {

constexpr int kRouterIdsLds = 16384;   // flat ids kept in LDS for the dispatch (64 KiB)

// ------------------------------------------------------------- logits ----

template <int RT, int XT>
__device__ __forceinline__ f32x4_t router_dot(const RouterArgs& a, int rtile, int ctile, int wave, int NW,
                                              int lane) {
  const int H = a.H;
  const int row = rtile * 16 + (lane & 15);
  const int tok = ctile * 16 + (lane & 15);
  const int g = lane >> 4;
  const bool arow = row < a.E;
  const bool btok = tok < a.T;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (RT == DT_F32) {
    // 16x16x4 fp32 MFMA; one 16-byte load = 4 k values; step covers 16 k.
    const int nsteps = H / 16;
    const int s0 = wave * nsteps / NW, s1 = (wave + 1) * nsteps / NW;
    const float* wrow = reinterpret_cast<const float*>(a.wr) + size_t(row) * H;
    for (int sb = s0; sb < s1; sb += 8) {
      u32x4_t av[8];
      float bv[8][4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = sb + u;
        const int k0 = s * 16 + g * 4;
        const bool in = s < s1;
        av[u] = (arow && in) ? ldg16(wrow + k0) : u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < 4; ++m) bv[u][m] = 0.f;
        if (btok && in) {
          if constexpr (XT == DT_F32) {
            u32x4_t t = ldg16(reinterpret_cast<const float*>(a.x) + size_t(tok) * H + k0);
#pragma unroll
            for (int m = 0; m < 4; ++m) bv[u][m] = __uint_as_float(t[m]);
          } else {
            u32x2_t t = ldg8(reinterpret_cast<const uint16_t*>(a.x) + size_t(tok) * H + k0);
            bv[u][0] = bf16_lo(t[0]); bv[u][1] = bf16_hi(t[0]); bv[u][2] = bf16_lo(t[1]); bv[u][3] = bf16_hi(t[1]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc = mfma_f32(__uint_as_float(av[u][m]), bv[u][m], acc);
    }
  } else {
    // 16x16x32 bf16 MFMA; one 16-byte load = 8 k values; step covers 32 k.
    const int nsteps = H / 32;
    const int s0 = wave * nsteps / NW, s1 = (wave + 1) * nsteps / NW;
    const uint16_t* wrow = reinterpret_cast<const uint16_t*>(a.wr) + size_t(row) * H;
    for (int sb = s0; sb < s1; sb += 8) {
      u32x4_t av[8];
      float v[8][8];
      u32x4_t bx[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = sb + u;
        const int k0 = s * 32 + g * 8;
        const bool in = s < s1;
        av[u] = (arow && in) ? ldg16(wrow + k0) : u32x4_t{0, 0, 0, 0};
        if constexpr (XT == DT_BF16) {
          bx[u] = (btok && in) ? ldg16(reinterpret_cast<const uint16_t*>(a.x) + size_t(tok) * H + k0)
                               : u32x4_t{0, 0, 0, 0};
        } else {
#pragma unroll
          for (int m = 0; m < 8; ++m) v[u][m] = 0.f;
          if (btok && in) {
            const float* xp = reinterpret_cast<const float*>(a.x) + size_t(tok) * H + k0;
            u32x4_t t0 = ldg16(xp), t1 = ldg16(xp + 4);
#pragma unroll
            for (int m = 0; m < 4; ++m) { v[u][m] = __uint_as_float(t0[m]); v[u][m + 4] = __uint_as_float(t1[m]); }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if constexpr (XT == DT_BF16) {
          acc = mfma_bf16(av[u], bx[u], acc);
        } else {
          u32x4_t hi, lo;
          split_bf16x8(v[u], hi, lo);
          acc = mfma_bf16(av[u], hi, acc);
          acc = mfma_bf16(av[u], lo, acc);
        }
      }
    }
  }
  return acc;
}

// ------------------------------------------------------------- top-k -----

// Candidate order: larger logit first; equal logits -> lower expert index.
// NaN logits are treated as -inf so every selected index is a real expert.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ float sanitize(float v) { return v != v ? -__builtin_inff() : v; }

// One thread selects the top-k of one token (E <= EMAX <= 32, k <= 8).  Logits,
// selections and weights stay in registers (loops fully unrolled and
// predicated); ids and weights are written once.  `ids_lds` (or null)
// receives a copy of the ids for the dispatch.
template <int EMAX>
__device__ void topk_thread(const float* l, int E, int k, int32_t* ids, float* w, int32_t* ids_lds) {
  constexpr int KMAX = 8;
  float lv[EMAX], zv[KMAX];
  int iv[KMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) lv[e] = e < E ? sanitize(l[e]) : -__builtin_inff();
  uint32_t taken = 0;
  float lmax = 0.f, denom = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    zv[j] = 0.f;
    iv[j] = 0;
    if (j < k) {
      int bi = 0x7fffffff;
      float bv = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (e < E && !(taken & (1u << e)) && better(lv[e], e, bv, bi)) { bv = lv[e]; bi = e; }
      }
      taken |= 1u << bi;
      if (j == 0) lmax = bv;
      // weights: softmax over the selected logits (the full-softmax denominator cancels)
      const float z = (bv == -__builtin_inff()) ? 0.f : __expf(bv - lmax);
      zv[j] = z;
      iv[j] = bi;
      denom += z;
    }
  }
  const float r = denom > 0.f ? 1.0f / denom : 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      ids[j] = iv[j];
      if (ids_lds) ids_lds[j] = iv[j];
      w[j] = denom > 0.f ? zv[j] * r : 1.0f / float(k);   // all selected logits -inf/NaN: equal weights
    }
  }
}

// (value, index) maximum over the 16 lanes of a DPP row: rotations by 8, 4, 2
// and 1 lanes leave every lane of the row holding the row's best candidate.
template <int ROT>
__device__ __forceinline__ void dpp_row_best(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), 0x120 + ROT, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_mov_dpp(bi, 0x120 + ROT, 0xF, 0xF, false);
  if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
}

// One wave selects the top-k of one token (any E <= 256, k <= E).  Each
// round takes the best remaining candidate of every lane (4 per lane), the
// best of every 16-lane row with DPP rotations, and the best of the 4 rows
// with lane reads.  Selection j is kept by lane j % 64 (slot j / 64) and
// written once at the end.
__device__ void topk_wave(const float* l, int E, int k, int32_t* ids, float* w, int32_t* ids_lds, int lane) {
  float v[4], zk[4];
  bool taken[4];
  int ik[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    v[m] = e < E ? sanitize(l[e]) : -__builtin_inff();
    taken[m] = e >= E;
    zk[m] = 0.f;
    ik[m] = 0;
  }
  float lmax = 0.f, denom = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * m;
      if (!taken[m] && better(v[m], e, bv, bi)) { bv = v[m]; bi = e; }
    }
    dpp_row_best<8>(bv, bi);
    dpp_row_best<4>(bv, bi);
    dpp_row_best<2>(bv, bi);
    dpp_row_best<1>(bv, bi);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
      const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), r));
      const int oi = __builtin_amdgcn_readlane(bi, r);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    // every lane of row 0 now holds the wave's best; broadcast it
    bv = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bv)));
    bi = __builtin_amdgcn_readfirstlane(bi);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (lane + 64 * m == bi) taken[m] = true;
    if (j == 0) lmax = bv;
    const float z = (bv == -__builtin_inff()) ? 0.f : __expf(bv - lmax);
    denom += z;
    if (lane == (j & 63)) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if ((j >> 6) == m) { zk[m] = z; ik[m] = bi; }
    }
  }
  const float r = denom > 0.f ? 1.0f / denom : 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int j = lane + 64 * m;
    if (j < k) {
      ids[j] = ik[m];
      if (ids_lds) ids_lds[j] = ik[m];
      w[j] = denom > 0.f ? zk[m] * r : 1.0f / float(k);
    }
  }
}

// ------------------------------------------------------------ dispatch ---

// Expert-sorted order, built by one work-group.  Deterministic: the rank of an
// assignment inside its expert's segment is the number of smaller flat ids
// routed to the same expert (stable counting sort); no atomics decide order.
__device__ void dispatch_wg(const RouterArgs& a, int* lds, const int32_t* ids) {
  const RouteBufs& rb = a.rb;
  const int E = a.E, n = a.T * a.k, M = a.tile_m;
  const int tid = threadIdx.x, NT = blockDim.x, lane = tid & 63, wave = tid >> 6, NW = NT >> 6;
  int* hist = lds;                 // [NW][E]: per-wave counts, then per-wave rank bases
  int* cnt = hist + NW * E;        // [E]
  int* off = cnt + E;              // [E+1]

  for (int i = tid; i < NW * E; i += NT) hist[i] = 0;
  __syncthreads();
  const int chunk = (n + NW - 1) / NW;
  const int f0 = min(n, wave * chunk), f1 = min(n, f0 + chunk);
  for (int f = f0 + lane; f < f1; f += 64) atomicAdd(&hist[wave * E + ids[f]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int s = 0;
    for (int w = 0; w < NW; ++w) {
      int c = hist[w * E + e];
      hist[w * E + e] = s;
      s += c;
    }
    cnt[e] = s;
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scans over experts (padded offsets, unpadded prefix) and the
    // compact active list; experts 4*lane .. 4*lane+3 belong to this lane
    int c[4], pad[4], act = 0, sp = 0, sc = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane * 4 + m;
      c[m] = e < E ? cnt[e] : 0;
      pad[m] = (c[m] + M - 1) / M * M;
      sp += pad[m];
      sc += c[m];
      act += c[m] > 0;
    }
    int ip = sp, ic = sc, ia = act;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(ip, d), uc = __shfl_up(ic, d), ua = __shfl_up(ia, d);
      if (lane >= d) { ip += up; ic += uc; ia += ua; }
    }
    int bp = ip - sp, bc = ic - sc, ba = ia - act;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane * 4 + m;
      if (e < E) {
        off[e] = bp;
        rb.offsets[e] = bp;
        rb.cprefix[e] = bc;
        rb.counts[e] = c[m];
        if (c[m] > 0) rb.active[1 + ba++] = e;
      }
      bp += pad[m];
      bc += c[m];
    }
    if (lane == 63) {
      off[E] = ip;
      rb.offsets[E] = ip;
      rb.cprefix[E] = ic;
      rb.active[0] = ia;
    }
  }
  __syncthreads();
  for (int c0 = f0; c0 < f1; c0 += 64) {
    const int f = c0 + lane;
    const bool valid = f < f1;
    const int e = valid ? ids[f] : 0;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    int base = 0;
    if (valid) base = hist[wave * E + e];
    if (valid) {
      const int rank = __popcll(m & ((1ull << lane) - 1ull));
      const int pos = off[e] + base + rank;
      rb.sorted_ids[pos] = f;
      rb.inv[f] = pos;
    }
    if (valid && (m >> lane) == 1ull) hist[wave * E + e] = base + __popcll(m);
  }
  __syncthreads();
  for (int e = wave; e < E; e += NW)
    for (int p = off[e] + cnt[e] + lane; p < off[e + 1]; p += 64) rb.sorted_ids[p] = n;
  for (int p = off[E] + tid; p < a.capacity; p += NT) rb.sorted_ids[p] = n;
  const int n_tiles = rb.tile_expert ? a.capacity / M : 0;   // the decode path reads no tile table
  for (int i = tid; i < n_tiles; i += NT) {
    const int r = i * M;
    int e = -1;
    if (r < off[E]) {
      int lo = 0, hi = E;          // largest e with off[e] <= r
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (off[mid] <= r) lo = mid; else hi = mid;
      }
      e = lo;
    }
    rb.tile_expert[i] = e;
  }
}

// --------------------------------------------------------------- kernel --

// One 16-expert x 16-token logits tile: the waves split H, partial sums meet
// in LDS, wave 0 adds the bias and stores to `dst` ([T, E], row stride E).
template <int RT, int XT>
__device__ __forceinline__ void logits_tile(const RouterArgs& a, float* red, float* dst) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, NW = blockDim.x >> 6;
  const int rtile = blockIdx.x % a.n_row_tiles, ctile = blockIdx.x / a.n_row_tiles;
  // side job of the prefill path: clear the fp32 combine accumulator
  if (a.zero_f32) {
    const long n4 = a.zero_n / 4;
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    for (long i = long(blockIdx.x) * blockDim.x + tid; i < n4; i += long(gridDim.x) * blockDim.x)
      reinterpret_cast<f32x4_t*>(a.zero_f32)[i] = z;
  }
  f32x4_t acc = router_dot<RT, XT>(a, rtile, ctile, wave, NW, lane);
  *reinterpret_cast<f32x4_t*>(red + (wave * 64 + lane) * 4) = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t s = *reinterpret_cast<f32x4_t*>(red + lane * 4);
    for (int w = 1; w < NW; ++w) s += *reinterpret_cast<f32x4_t*>(red + (w * 64 + lane) * 4);
    const int tok = ctile * 16 + (lane & 15);
    if (tok < a.T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = rtile * 16 + (lane >> 4) * 4 + i;
        if (e < a.E) dst[size_t(tok) * a.E + e] = s[i] + (a.bias ? a.bias[e] : 0.f);
      }
    }
  }
}

// Top-k of every token from logits `l` ([T, E]), then the dispatch.  One
// work-group.  The ids are also kept in LDS (after the dispatch scratch) when
// T*k fits, so the dispatch does not read them back from memory.
__device__ __forceinline__ void select_and_dispatch(const RouterArgs& a, const float* l, int* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, NW = blockDim.x >> 6;
  const int T = a.T, E = a.E, k = a.k, n = T * k;
  int* ids_lds = (n <= kRouterIdsLds) ? lds + NW * E + 2 * E + 1 : nullptr;
  if (E <= 32 && k <= 8) {
    for (int t = tid; t < T; t += blockDim.x) {
      const float* lt = l + size_t(t) * E;
      int32_t* it = a.rb.topk_ids + size_t(t) * k;
      float* wt = a.rb.topk_w + size_t(t) * k;
      int32_t* il = ids_lds ? ids_lds + t * k : nullptr;
      if (E <= 8) topk_thread<8>(lt, E, k, it, wt, il);
      else if (E <= 16) topk_thread<16>(lt, E, k, it, wt, il);
      else topk_thread<32>(lt, E, k, it, wt, il);
    }
  } else {
    for (int t = wave; t < T; t += NW)
      topk_wave(l + size_t(t) * E, E, k, a.rb.topk_ids + size_t(t) * k, a.rb.topk_w + size_t(t) * k,
                ids_lds ? ids_lds + t * k : nullptr, lane);
  }
  __threadfence_block();
  __syncthreads();
  dispatch_wg(a, lds, ids_lds ? ids_lds : a.rb.topk_ids);
}

// Single work-group (at most 16 experts x 16 tokens): logits stay in LDS.
template <int RT, int XT>
__global__ void __launch_bounds__(1024) router_fused_kernel(RouterArgs a) {
  extern __shared__ int lds[];
  __shared__ float lg[256];
  logits_tile<RT, XT>(a, reinterpret_cast<float*>(lds), lg);
  __syncthreads();
  select_and_dispatch(a, lg, lds);
}

// Larger grids: the logits go to the workspace; the selection and dispatch run
// in a second launch (the kernel boundary orders them, no device-wide fences).
template <int RT, int XT>
__global__ void __launch_bounds__(1024) router_logits_kernel(RouterArgs a) {
  extern __shared__ int lds[];
  logits_tile<RT, XT>(a, reinterpret_cast<float*>(lds), a.rb.logits);
}

__global__ void __launch_bounds__(1024) router_select_kernel(RouterArgs a) {
  extern __shared__ int lds[];
  select_and_dispatch(a, a.rb.logits, lds);
}

// --------------------------------------------------------------- launch --

size_t router_lds_bytes(int NW, int E, int n) {
  size_t red = size_t(NW) * 64 * 4 * sizeof(float);
  size_t disp = (size_t(NW) * E + 2 * E + 1 + (n <= kRouterIdsLds ? n : 0)) * sizeof(int);
  return red > disp ? red : disp;
}

template <int RT, int XT>
static void launch_router_t(const RouterArgs& a, int NW, hipStream_t st) {
  const int nblocks = a.n_row_tiles * a.n_col_tiles;
  if (nblocks == 1) {
    hipLaunchKernelGGL((router_fused_kernel<RT, XT>), dim3(1), dim3(NW * 64), router_lds_bytes(NW, a.E, a.T * a.k),
                       st, a);
  } else {
    hipLaunchKernelGGL((router_logits_kernel<RT, XT>), dim3(nblocks), dim3(NW * 64),
                       size_t(NW) * 64 * 4 * sizeof(float), st, a);
    hipLaunchKernelGGL(router_select_kernel, dim3(1), dim3(1024), router_lds_bytes(16, a.E, a.T * a.k), st, a);
  }
}

hipError_t launch_router(const RouterArgs& a, int rdt, int xdt, int NW, hipStream_t st) {
  if (rdt == DT_F32 && xdt == DT_F32) launch_router_t<DT_F32, DT_F32>(a, NW, st);
  else if (rdt == DT_F32) launch_router_t<DT_F32, DT_BF16>(a, NW, st);
  else if (xdt == DT_F32) launch_router_t<DT_BF16, DT_F32>(a, NW, st);
  else launch_router_t<DT_BF16, DT_BF16>(a, NW, st);
  return hipGetLastError();
}

}  // namespace moe
