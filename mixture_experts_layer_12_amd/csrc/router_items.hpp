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
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kRouterIdsLds = 8192;    // flat ids kept in LDS for the dispatch (32 KiB)
constexpr int kRouterStage = 8192;     // logits staged in LDS per chunk of tokens (32 KiB)

// ------------------------------------------------------------- logits ----

// The reduction over H is cut into kLogitChunks chunks of steps, each with its
// own accumulator, and the chunk sums are added in one fixed order (groups of
// four chunks left to right, then the groups left to right, then the bias),
// whatever the number of waves or work-groups that computed them: the
// multi-launch and the single-launch paths produce the same bits.
constexpr int kLogitChunks = 16;

template <int RT>
__host__ __device__ __forceinline__ int logit_steps(int H) { return RT == DT_F32 ? H / 16 : H / 32; }

// Accumulators of chunks c0 .. c0+CPW-1 of the 16-expert x 16-token tile;
// each batch issues 8 loads of A (and of B) per lane across the CPW chunks.
template <int RT, int XT, int CPW>
__device__ __forceinline__ void router_dot(const RouterArgs a, int rtile, int ctile, int c0, int lane, f32x4_t* acc) {
  // fp32 activations against bf16 router rows hold 8 floats per step: half the batch
  constexpr int U = (RT == DT_BF16 && XT == DT_F32) ? (CPW >= 4 ? 1 : 4 / CPW) : 8 / CPW;
  const int H = a.H, nsteps = logit_steps<RT>(H);
  const int row = rtile * 16 + (lane & 15);
  const int tok = ctile * 16 + (lane & 15);
  const int g = lane >> 4;
  const bool arow = row < a.E;
  const bool btok = tok < a.T;
  int s0[CPW], s1[CPW], len = 0;
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    s0[j] = (c0 + j) * nsteps / kLogitChunks;
    s1[j] = (c0 + j + 1) * nsteps / kLogitChunks;
    len = max(len, s1[j] - s0[j]);
    acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int sb = 0; sb < len; sb += U) {
    if constexpr (RT == DT_F32) {
      // 16x16x4 fp32 MFMA; one 16-byte load = 4 k values; a step covers 16 k.
      const float* wrow = reinterpret_cast<const float*>(a.wr) + size_t(row) * H;
      u32x4_t av[CPW][U];
      float bv[CPW][U][4];
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int s = s0[j] + sb + u;
          const int k0 = s * 16 + g * 4;
          const bool in = s < s1[j];
          av[j][u] = (arow && in) ? ldg16(wrow + k0) : u32x4_t{0, 0, 0, 0};
#pragma unroll
          for (int m = 0; m < 4; ++m) bv[j][u][m] = 0.f;
          if (btok && in) {
            if constexpr (XT == DT_F32) {
              const u32x4_t t = ldg16(reinterpret_cast<const float*>(a.x) + size_t(tok) * H + k0);
#pragma unroll
              for (int m = 0; m < 4; ++m) bv[j][u][m] = __uint_as_float(t[m]);
            } else {
              const u32x2_t t = ldg8(reinterpret_cast<const uint16_t*>(a.x) + size_t(tok) * H + k0);
              bv[j][u][0] = bf16_lo(t[0]); bv[j][u][1] = bf16_hi(t[0]);
              bv[j][u][2] = bf16_lo(t[1]); bv[j][u][3] = bf16_hi(t[1]);
            }
          }
        }
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[j] = mfma_f32(__uint_as_float(av[j][u][m]), bv[j][u][m], acc[j]);
    } else {
      // 16x16x32 bf16 MFMA; one 16-byte load = 8 k values; a step covers 32 k.
      const uint16_t* wrow = reinterpret_cast<const uint16_t*>(a.wr) + size_t(row) * H;
      u32x4_t av[CPW][U], bx[CPW][U];
      float v[CPW][U][8];
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int s = s0[j] + sb + u;
          const int k0 = s * 32 + g * 8;
          const bool in = s < s1[j];
          av[j][u] = (arow && in) ? ldg16(wrow + k0) : u32x4_t{0, 0, 0, 0};
          if constexpr (XT == DT_BF16) {
            bx[j][u] = (btok && in) ? ldg16(reinterpret_cast<const uint16_t*>(a.x) + size_t(tok) * H + k0)
                                    : u32x4_t{0, 0, 0, 0};
          } else {
#pragma unroll
            for (int m = 0; m < 8; ++m) v[j][u][m] = 0.f;
            if (btok && in) {
              const float* xp = reinterpret_cast<const float*>(a.x) + size_t(tok) * H + k0;
              const u32x4_t t0 = ldg16(xp), t1 = ldg16(xp + 4);
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                v[j][u][m] = __uint_as_float(t0[m]);
                v[j][u][m + 4] = __uint_as_float(t1[m]);
              }
            }
          }
        }
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if constexpr (XT == DT_BF16) {
            acc[j] = mfma_bf16(av[j][u], bx[j][u], acc[j]);
          } else {
            u32x4_t hi, lo;
            split_bf16x8(v[j][u], hi, lo);
            acc[j] = mfma_bf16(av[j][u], hi, acc[j]);
            acc[j] = mfma_bf16(av[j][u], lo, acc[j]);
          }
        }
    }
  }
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
template <int EMAX, bool COH>
__device__ __forceinline__ void topk_thread(const float* l, int E, int k, int32_t* ids, float* w, int32_t* ids_lds) {
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
      st_i32<COH>(ids + j, iv[j]);
      if (ids_lds) ids_lds[j] = iv[j];
      st_f32<COH>(w + j, denom > 0.f ? zv[j] * r : 1.0f / float(k));   // all selected logits -inf/NaN: equal weights
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
template <bool COH>
__device__ __forceinline__ void topk_wave(const float* l, int E, int k, int32_t* ids, float* w, int32_t* ids_lds, int lane) {
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
      st_i32<COH>(ids + j, ik[m]);
      if (ids_lds) ids_lds[j] = ik[m];
      st_f32<COH>(w + j, denom > 0.f ? zk[m] * r : 1.0f / float(k));
    }
  }
}

// One 16-lane DPP row selects the top-k of one token (E <= 64, k <= 16), so a
// wave serves 4 tokens at once: lane r of the row holds experts r, r+16, r+32
// and r+48, rotations within the row find each round's best, and selection j
// is kept by lane j of the row.  A row with `valid` false still takes part
// (its lanes hold -inf) and writes nothing.
template <bool COH>
__device__ __forceinline__ void topk_row16(const float* l, int E, int k, bool valid, int32_t* ids, float* w, int32_t* ids_lds,
                           int r) {
  float v[4];
  bool taken[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = r + 16 * m;
    v[m] = (valid && e < E) ? sanitize(l[e]) : -__builtin_inff();
    taken[m] = e >= E;
  }
  float lmax = 0.f, denom = 0.f, zk = 0.f;
  int ik = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = r + 16 * m;
      if (!taken[m] && better(v[m], e, bv, bi)) { bv = v[m]; bi = e; }
    }
    dpp_row_best<8>(bv, bi);
    dpp_row_best<4>(bv, bi);
    dpp_row_best<2>(bv, bi);
    dpp_row_best<1>(bv, bi);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (r + 16 * m == bi) taken[m] = true;
    if (j == 0) lmax = bv;
    const float z = (bv == -__builtin_inff()) ? 0.f : __expf(bv - lmax);
    denom += z;
    if (r == j) { zk = z; ik = bi; }
  }
  if (valid && r < k) {
    st_i32<COH>(ids + r, ik);
    if (ids_lds) ids_lds[r] = ik;
    st_f32<COH>(w + r, denom > 0.f ? zk * (1.0f / denom) : 1.0f / float(k));
  }
}

// ------------------------------------------------------------ dispatch ---

// Lanes of the wave whose (valid) expert id equals this lane's: 8 ballots, one
// per bit of the id (E <= 256).
__device__ __forceinline__ uint64_t same_expert_mask(int e, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Expert-sorted order, built by one work-group.  Deterministic: the rank of an
// assignment inside its expert's segment is the number of smaller flat ids
// routed to the same expert (stable counting sort); no atomics decide order.
template <bool COH>
__device__ __forceinline__ void dispatch_wg(const RouterArgs a, int* lds, const int32_t* ids) {
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
  // per-wave counts without atomics: the first lane of each group of equal ids adds the group size
  for (int c0 = f0; c0 < f1; c0 += 64) {
    const int f = c0 + lane;
    const bool valid = f < f1;
    const int e = valid ? ids[f] : 0;
    const uint64_t m = same_expert_mask(e, valid);
    if (valid && (m & ((1ull << lane) - 1ull)) == 0) hist[wave * E + e] += __popcll(m);
  }
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
        st_i32<COH>(rb.offsets + e, bp);
        st_i32<COH>(rb.cprefix + e, bc);
        st_i32<COH>(rb.counts + e, c[m]);
        if (c[m] > 0) st_i32<COH>(rb.active + 1 + ba++, e);
      }
      bp += pad[m];
      bc += c[m];
    }
    if (lane == 63) {
      off[E] = ip;
      st_i32<COH>(rb.offsets + E, ip);
      st_i32<COH>(rb.cprefix + E, ic);
      st_i32<COH>(rb.active, ia);
    }
  }
  __syncthreads();
  for (int c0 = f0; c0 < f1; c0 += 64) {
    const int f = c0 + lane;
    const bool valid = f < f1;
    const int e = valid ? ids[f] : 0;
    const uint64_t m = same_expert_mask(e, valid);
    int base = 0;
    if (valid) base = hist[wave * E + e];
    if (valid) {
      const int rank = __popcll(m & ((1ull << lane) - 1ull));
      const int pos = off[e] + base + rank;
      st_i32<COH>(rb.sorted_ids + pos, f);
      st_i32<COH>(rb.inv + f, pos);
    }
    if (valid && (m >> lane) == 1ull) hist[wave * E + e] = base + __popcll(m);
  }
  __syncthreads();
  for (int e = wave; e < E; e += NW)
    for (int p = off[e] + cnt[e] + lane; p < off[e + 1]; p += 64) st_i32<COH>(rb.sorted_ids + p, n);
  for (int p = off[E] + tid; p < a.capacity; p += NT) st_i32<COH>(rb.sorted_ids + p, n);
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
    st_i32<COH>(rb.tile_expert + i, e);
  }
}

// --------------------------------------------------------------- kernel --

// One 16-expert x 16-token logits tile: the waves split H, partial sums meet
// in LDS, wave 0 adds the bias and stores to `dst` ([T, E], row stride E).
// Logits of one 16-expert x 16-token tile from chunks [cb, cb + n) with n =
// 4 * (number of groups): each wave computes CPW = n / NW chunks into `red` (LDS,
// n x 64 x 4 floats), then wave 0 adds them in the fixed order.  final: n is
// all 16 chunks, the bias is added and dst is the [T, E] logits; otherwise
// the group sum goes to dst as one partial [T, E] plane (bias added by the
// reader, after the planes, in the same order).
template <int RT, int XT, bool COH, int CPW>
__device__ __forceinline__ void logits_tile(const RouterArgs a, int rtile, int ctile, int cb, int n, float* red,
                                            float* dst) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c0 = cb + wave * CPW;
  f32x4_t acc[CPW];
  router_dot<RT, XT, CPW>(a, rtile, ctile, c0, lane, acc);
#pragma unroll
  for (int j = 0; j < CPW; ++j) *reinterpret_cast<f32x4_t*>(red + ((wave * CPW + j) * 64 + lane) * 4) = acc[j];
  __syncthreads();
  if (wave == 0) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < n / 4; ++q) {
      f32x4_t gsum = *reinterpret_cast<f32x4_t*>(red + (4 * q * 64 + lane) * 4);
      for (int c = 1; c < 4; ++c) gsum += *reinterpret_cast<f32x4_t*>(red + ((4 * q + c) * 64 + lane) * 4);
      s = q == 0 ? gsum : s + gsum;
    }
    const bool final = n == kLogitChunks;
    const int tok = ctile * 16 + (lane & 15);
    if (tok < a.T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = rtile * 16 + (lane >> 4) * 4 + i;
        if (e < a.E) st_f32<COH>(dst + size_t(tok) * a.E + e, final ? s[i] + (a.bias ? a.bias[e] : 0.f) : s[i]);
      }
    }
  }
}

// LDS of the selection and dispatch, in ints: dispatch scratch, then the flat
// ids (when T*k fits), then the logits staging area (select kernel only).
// A multiple of 4 ints, so that what follows stays 16-byte aligned.
__host__ __device__ inline int router_disp_ints(int NW, int E) {
  const int d = NW * E + 2 * E + 1 > kSmallDispInts ? NW * E + 2 * E + 1 : kSmallDispInts;
  return (d + 3) & ~3;
}

// Selection strategies of the general path; each kernel is built for one of
// them, so that its code holds only the loops it runs.
enum : int { kTopkT8 = 0, kTopkT16 = 1, kTopkT32 = 2, kTopkRow16 = 3, kTopkWave = 4 };

__host__ __device__ inline int topk_mode(int E, int k) {
  if (E <= 32 && k <= 8) return E <= 8 ? kTopkT8 : (E <= 16 ? kTopkT16 : kTopkT32);
  return (E <= 64 && k <= 16) ? kTopkRow16 : kTopkWave;
}

// Top-k of tokens [t0, t0 + nt) whose logit rows start at `l` (row stride E,
// LDS): a thread per token (E <= 32, k <= 8), a 16-lane row per token
// (E <= 64, k <= 16), else a wave per token; MODE is topk_mode(E, k).
template <bool COH, int MODE>
__device__ __forceinline__ void topk_chunk(const RouterArgs a, const float* l, int t0, int nt, int32_t* ids_lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, NT = blockDim.x, NW = NT >> 6;
  const int E = a.E, k = a.k;
  if constexpr (MODE <= kTopkT32) {
    constexpr int EMAX = MODE == kTopkT8 ? 8 : (MODE == kTopkT16 ? 16 : 32);
    for (int i = tid; i < nt; i += NT) {
      const size_t t = size_t(t0 + i);
      topk_thread<EMAX, COH>(l + size_t(i) * E, E, k, a.rb.topk_ids + t * k, a.rb.topk_w + t * k,
                             ids_lds ? ids_lds + t * k : nullptr);
    }
  } else if constexpr (MODE == kTopkRow16) {
    for (int i0 = wave * 4; i0 < nt; i0 += NW * 4) {        // wave-uniform loop
      const int i = i0 + (lane >> 4);
      const bool valid = i < nt;
      const int ic = valid ? i : 0;
      const size_t t = size_t(t0 + ic);
      topk_row16<COH>(l + size_t(ic) * E, E, k, valid, a.rb.topk_ids + t * k, a.rb.topk_w + t * k,
                 ids_lds ? ids_lds + t * k : nullptr, lane & 15);
    }
  } else {
    for (int i = wave; i < nt; i += NW) {
      const size_t t = size_t(t0 + i);
      topk_wave<COH>(l + size_t(i) * E, E, k, a.rb.topk_ids + t * k, a.rb.topk_w + t * k,
                ids_lds ? ids_lds + t * k : nullptr, lane);
    }
  }
}

// Logits [0, cnt) of the [T, E] block at `src` into LDS.  With partial planes
// (logit_parts 4, `plane` floats apart) the four group sums are added in
// order and then the bias.  Every load of a batch is issued before the first
// store: the loads use a clamped index and the stores are predicated.
template <bool COH>
__device__ __forceinline__ void stage_logits(const RouterArgs a, const float* src, int cnt, size_t plane, float* stage) {
  const int tid = threadIdx.x, NT = blockDim.x, E = a.E;
  for (int b = 0; b < cnt; b += 8 * NT) {
    float v[8];
    if (a.logit_parts == 1) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ld_f32<COH>(src + min(b + u * NT + tid, cnt - 1));
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = min(b + u * NT + tid, cnt - 1);
        float acc = ld_f32<COH>(src + idx);
        acc += ld_f32<COH>(src + plane + idx);
        acc += ld_f32<COH>(src + 2 * plane + idx);
        acc += ld_f32<COH>(src + 3 * plane + idx);
        acc += a.bias ? a.bias[idx % E] : 0.f;
        v[u] = acc;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = b + u * NT + tid;
      if (idx < cnt) stage[idx] = v[u];
    }
  }
}

// Candidate order as one unsigned key (larger key = earlier candidate): the
// order-preserving bits of the logit (NaN read as -inf, -0 as +0) above the
// complemented expert index, so equal logits go to the lower index.
__device__ __forceinline__ uint64_t cand_key(float v, int j) {
  v = sanitize(v) + 0.f;
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(o) << 32) | uint32_t(~uint32_t(j));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = uint32_t(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Selection and dispatch of few assignments (small_route), in five phases:
//  1. the logits of every token become candidate keys in LDS (rows padded to
//     E4 = E rounded up to 4 with key 0, which precedes nothing);
//  2. the rank of an expert is the number of keys above its own; experts of
//     rank < k are the selection, in rank order (the list the round-by-round
//     selections produce).  Ranks are counted inside groups of 64 experts
//     (a wave per group, a lane per expert);
//  3. with more than one group per token, the keys ranked below k in their
//     group are ranked again among themselves;
//  4. wave 0, lane f = flat id t * k + j: the weight of selection j (softmax
//     over the selected logits, the denominator summed in selection order, as
//     in the other strategies) and, with ballots over the 8 bits of the
//     expert ids, each assignment's group of equal experts, its rank in the
//     group (smaller flat id first), and the assignments and active experts
//     with a smaller expert id; active experts' segments follow in expert
//     order, each padded to a multiple of tile_m;
//  5. the work-group writes the per-expert tables, the padding and the tile
//     table.  The results are those of dispatch_wg.
// Phases 1-3 are small_select, 4 small_place and 5 small_tables, so that a
// consumer can keep the routing in LDS (see the decode gate/up launch).
// The phases share one LDS region (16-byte aligned), laid out here.
struct SmallRoute {
  int* s_e;                        // [64]: expert of active slot j (slots in expert order)
  int* s_cnt;                      // [64]: its assignments
  int* s_pad;                      // [64]: its padded length
  int* s_off;                      // [65]: start of its segment; [A]: end of the last segment
  int* s_cpre;                     // [65]: assignments with a smaller expert; [A]: n
  int* s_na;                       // [1]: A, the number of active experts
  int32_t* ids;                    // [n]: selected experts, flat order
  float* wts;                      // [n]: their weights
  int* sorted;                     // [n]: flat ids in expert-sorted order (tile_m 1)
  float* selv;                     // [n]: selected logits, flat order
  uint64_t* keys;                  // [T][E4]
  int* part;                       // survivors of the group ranks: [T][ceil(E / 64) * k] 64-bit keys
  __device__ __forceinline__ SmallRoute(int* lds, int T, int E, int k) {
    const int n = T * k, E4 = (E + 3) & ~3;
    s_e = lds; s_cnt = s_e + 64; s_pad = s_cnt + 64; s_off = s_pad + 64; s_cpre = s_off + 65; s_na = s_cpre + 65;
    ids = lds + ((kSmallDispInts + 3) & ~3);
    wts = reinterpret_cast<float*>(ids + n);
    sorted = reinterpret_cast<int*>(wts + n);
    selv = reinterpret_cast<float*>(sorted + n);
    keys = reinterpret_cast<uint64_t*>(ids + ((4 * n + 3) & ~3));
    part = reinterpret_cast<int*>(keys + T * E4);
  }
};

// Ints of the region for a work-group of NT threads (at most: the survivors
// take 2 * T * ceil(E / 64) * k <= 512 <= 4 * NT ints).
__host__ __device__ inline int small_route_ints(int NT, int T, int E, int k) {
  return ((kSmallDispInts + 3) & ~3) + ((4 * T * k + 3) & ~3) + 2 * T * ((E + 3) & ~3) + 4 * NT;
}

// Upper bound of small_route_ints over every shape small_route admits.
__host__ __device__ constexpr int small_route_max_ints(int NT) {
  return ((kSmallDispInts + 3) & ~3) + 4 * kSmallN + 2 * (1024 + 3 * kSmallN) + 4 * NT;
}

// Phases 1-3: the selection into R.ids and R.selv (ends with a barrier).
template <bool COH>
__device__ __forceinline__ void small_select(const RouterArgs a, const float* l, bool l_in_lds, const SmallRoute& R) {
  const int tid = threadIdx.x, NT = blockDim.x;
  const int T = a.T, E = a.E, k = a.k;
  const int E4 = (E + 3) & ~3;
  int32_t* ids_lds = R.ids;
  float* selv = R.selv;
  uint64_t* keys = R.keys;

  // 1. keys (and the survivor slots of step 2 cleared)
  if (E > 64)
    for (int p = tid; p < T * ((E + 63) >> 6) * k; p += NT) reinterpret_cast<uint64_t*>(R.part)[p] = 0ull;
  const size_t plane = size_t(T) * E;
  const bool four = !l_in_lds && a.logit_parts != 1;
  const bool with_bias = four && a.bias;
  for (int b = 0; b < T * E4; b += 4 * NT) {
    int idx[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = min(b + u * NT + tid, T * E4 - 1);
      const int i = p / E4;
      idx[u] = i * E + min(p - i * E4, E - 1);
    }
    // Every load of the batch is issued before the first sum (the branches
    // only decide which loads exist), so the batch costs one round trip; the
    // sums then follow the fixed order of the other readers of the planes.
    float v[4], q1[4], q2[4], q3[4], bs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = l_in_lds ? l[idx[u]] : ld_f32<COH>(l + idx[u]);
    if (four) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        q1[u] = ld_f32<COH>(l + plane + idx[u]);
        q2[u] = ld_f32<COH>(l + 2 * plane + idx[u]);
        q3[u] = ld_f32<COH>(l + 3 * plane + idx[u]);
      }
    }
    if (with_bias) {
#pragma unroll
      for (int u = 0; u < 4; ++u) bs[u] = a.bias[idx[u] % E];
    }
    if (four) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float acc = v[u];
        acc += q1[u];
        acc += q2[u];
        acc += q3[u];
        acc += with_bias ? bs[u] : 0.f;
        v[u] = acc;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = b + u * NT + tid;
      if (p < T * E4) {
        const int j = p % E4;
        keys[p] = j < E ? cand_key(v[u], j) : 0ull;
      }
    }
  }
  __syncthreads();

  // 2. rank of each key inside its group of 64 experts (a wave per token and
  //    group, a lane per expert, every lane reading the group's keys in the
  //    same order).  A key with k or more larger keys in its own group is out;
  //    the selection is among the rest: for one group the local rank is the
  //    rank, else the survivors (at most k per group) go to `cand` and
  //    3. each survivor's rank among the survivors of its token is its rank:
  //    every key above a selected key is itself a survivor, and a survivor
  //    outside the selection has the k selected keys above it.
  const int lane = tid & 63, wave = tid >> 6, NW = NT >> 6;
  const int GP = (E + 63) >> 6, C = GP * k;
  uint64_t* cand = reinterpret_cast<uint64_t*>(R.part);    // [T][GP * k] survivors (0: none)
  for (int w = wave; w < T * GP; w += NW) {                // wave-uniform loop
    const int i = w / GP, g = w - i * GP;
    const uint64_t* row = keys + i * E4 + 64 * g;
    const int len = min(64, E4 - 64 * g);                 // keys of the group, padding (key 0) included
    const bool valid = 64 * g + lane < E;
    const uint64_t mine = valid ? row[lane] : 0ull;
    int c0 = 0, c1 = 0;
#pragma unroll 8
    for (int j = 0; j < len; j += 2) {
      const u32x4_t t = *reinterpret_cast<const u32x4_t*>(row + j);
      c0 += (uint64_t(t[0]) | (uint64_t(t[1]) << 32)) > mine;
      c1 += (uint64_t(t[2]) | (uint64_t(t[3]) << 32)) > mine;
    }
    const int r = c0 + c1;
    if (valid && r < k) {
      if (GP == 1) {
        ids_lds[i * k + r] = 64 * g + lane;
        selv[i * k + r] = key_value(mine);
      } else {
        cand[i * C + g * k + r] = mine;
      }
    }
  }
  __syncthreads();
  if (GP > 1) {
    for (int p = tid; p < T * C; p += NT) {
      const int i = p / C;
      const uint64_t* ci = cand + i * C;
      const uint64_t mine = ci[p - i * C];
      int r = 0;
      for (int j = 0; j < C; ++j) r += ci[j] > mine;
      if (mine != 0ull && r < k) {
        ids_lds[i * k + r] = int(~uint32_t(mine));
        selv[i * k + r] = key_value(mine);
      }
    }
    __syncthreads();
  }
}

// Phase 4 (wave 0): weights into R.wts (and the top-k outputs when `store`),
// the slot tables, and for tile_m 1 the expert-sorted flat ids into
// R.sorted; returns each assignment's rank in its group and its slot (lanes
// of wave 0).  Ends with a barrier.
template <bool COH>
__device__ __forceinline__ void small_place(const RouterArgs a, const SmallRoute& R, bool store, int& rk, int& slot) {
  const RouteBufs& rb = a.rb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int T = a.T, k = a.k, n = T * k, M = a.tile_m;
  int* s_e = R.s_e; int* s_cnt = R.s_cnt; int* s_pad = R.s_pad; int* s_off = R.s_off; int* s_cpre = R.s_cpre;
  int* s_na = R.s_na;
  const int32_t* ids_lds = R.ids;
  const float* selv = R.selv;
  rk = 0;
  slot = 0;
  if (tid < 64) {
    const bool valid = lane < n;
    const int f = valid ? lane : 0;
    const int i = f / k;
    const float* si = selv + i * k;
    const float lmax = si[0];
    float denom = 0.f, zf = 0.f;
    for (int j = 0; j < k; ++j) {
      const float z = (si[j] == -__builtin_inff()) ? 0.f : __expf(si[j] - lmax);
      denom += z;
      if (j == f - i * k) zf = z;
    }
    const int e = valid ? ids_lds[f] : 0;
    const float wf = denom > 0.f ? zf * (1.0f / denom) : 1.0f / float(k);   // see topk_thread
    if (valid) {
      R.wts[f] = wf;
      if (store) {
        st_i32<COH>(rb.topk_ids + f, e);
        st_f32<COH>(rb.topk_w + f, wf);
      }
    }
    uint64_t same = __ballot(valid), lt = 0;     // same expert / smaller expert (valid lanes)
#pragma unroll
    for (int bt = 7; bt >= 0; --bt) {
      const bool bit = (e >> bt) & 1;
      const uint64_t bb = __ballot(bit);
      if (bit) { lt |= same & ~bb; same &= bb; }
      else same &= ~bb;
    }
    const uint64_t below = (1ull << lane) - 1ull;
    const bool leader = valid && (same & below) == 0;
    const uint64_t lead = __ballot(leader);
    const int A = __popcll(lead);
    rk = __popcll(same & below);
    slot = __popcll(lt & lead);
    if (M == 1 && valid) R.sorted[__popcll(lt) + rk] = f;
    if (leader) {
      const int c = __popcll(same);
      s_e[slot] = e;
      s_cnt[slot] = c;
      s_pad[slot] = (c + M - 1) / M * M;
      s_cpre[slot] = __popcll(lt);
      if (M == 1) s_off[slot] = __popcll(lt);
    }
    if (lane == 0) {
      s_na[0] = A;
      s_cpre[A] = n;
      if (M == 1) s_off[A] = n;
    }
    if (M != 1) {
      // padded starts: exclusive scan of the pads over the slots
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int v = lane < A ? s_pad[lane] : 0;
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d);
        if (lane >= d) incl += u;
      }
      if (lane < A) s_off[lane] = incl - v;
      if (lane == 63) s_off[A] = incl;
    }
  }
  __syncthreads();
}

// Phase 5: the routing tables in memory.
template <bool COH>
__device__ __forceinline__ void small_tables(const RouterArgs a, const SmallRoute& R, int rk, int slot) {
  const RouteBufs& rb = a.rb;
  const int tid = threadIdx.x, NT = blockDim.x;
  const int E = a.E, n = a.T * a.k, M = a.tile_m;
  const int* s_e = R.s_e; const int* s_cnt = R.s_cnt; const int* s_off = R.s_off; const int* s_cpre = R.s_cpre;
  const int A = R.s_na[0];
  const int total = s_off[A];
  if (tid < n) {
    const int pos = s_off[slot] + rk;
    st_i32<COH>(rb.sorted_ids + pos, tid);
    st_i32<COH>(rb.inv + tid, pos);
  }
  for (int e = tid; e < E; e += NT) {
    int lo = 0, hi = A;            // first slot whose expert is >= e
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_e[mid] < e) lo = mid + 1; else hi = mid;
    }
    st_i32<COH>(rb.counts + e, (lo < A && s_e[lo] == e) ? s_cnt[lo] : 0);
    st_i32<COH>(rb.offsets + e, s_off[lo]);
    st_i32<COH>(rb.cprefix + e, s_cpre[lo]);
  }
  if (tid < A) st_i32<COH>(rb.active + 1 + tid, s_e[tid]);
  if (tid == 0) {
    st_i32<COH>(rb.offsets + E, total);
    st_i32<COH>(rb.cprefix + E, n);
    st_i32<COH>(rb.active, A);
  }
  if (M != 1) {                    // padding rows inside the segments, then past the last one
    for (int w = tid; w < A * M; w += NT) {
      const int j = w / M, p = s_off[j] + s_cnt[j] + (w - j * M);
      if (p < s_off[j + 1]) st_i32<COH>(rb.sorted_ids + p, n);
    }
    for (int p = total + tid; p < a.capacity; p += NT) st_i32<COH>(rb.sorted_ids + p, n);
  }
  const int n_tiles = rb.tile_expert ? a.capacity / M : 0;
  for (int i = tid; i < n_tiles; i += NT) {
    const int r = i * M;
    int e = -1;
    if (r < total) {
      int lo = 0, hi = A;          // last slot starting at or before r
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= r) lo = mid; else hi = mid;
      }
      e = s_e[lo];
    }
    st_i32<COH>(rb.tile_expert + i, e);
  }
}

// Phases 1-4 into R (small_select, then `between` -- work of the caller that
// needs no routing, placed where it overlaps the selection's barriers --
// then small_place, which ends with a barrier).
template <bool COH, class F>
__device__ __forceinline__ void route_select_place(const RouterArgs a, const float* l, bool l_in_lds, const SmallRoute& R,
                                                   bool store, int& rk, int& slot, F between) {
  small_select<COH>(a, l, l_in_lds, R);
  between();
  small_place<COH>(a, R, store, rk, slot);
}

template <bool COH>
__device__ __forceinline__ void route_small(const RouterArgs a, const float* l, bool l_in_lds, int* lds) {
  const SmallRoute R(lds, a.T, a.E, a.k);
  int rk, slot;
  route_select_place<COH>(a, l, l_in_lds, R, true, rk, slot, [] {});
  small_tables<COH>(a, R, rk, slot);
}

// Top-k of every token, then the dispatch; one work-group.  Few assignments
// take route_small.  Otherwise logits in global
// memory are staged into LDS a chunk of tokens at a time, and the selection
// and dispatch_wg follow.
template <bool COH, int MODE>
__device__ __forceinline__ void select_and_dispatch(const RouterArgs a, const float* l, bool l_in_lds, int* lds) {
  const int NW = blockDim.x >> 6;
  const int T = a.T, E = a.E, n = T * a.k;
  const bool ids_fit = n <= kRouterIdsLds;
  int* ids_lds = ids_fit ? lds + router_disp_ints(NW, E) : nullptr;
  if (small_route(T, E, a.k)) {
    route_small<COH>(a, l, l_in_lds, lds);
    return;
  }
  if (l_in_lds) {
    topk_chunk<COH, MODE>(a, l, 0, T, ids_lds);
  } else {
    float* stage = reinterpret_cast<float*>(lds + router_disp_ints(NW, E) + (ids_fit ? n : 0));
    const int ch = max(1, kRouterStage / E);
    for (int t0 = 0; t0 < T; t0 += ch) {
      stage_logits<COH>(a, l + size_t(t0) * E, min(ch, T - t0) * E, size_t(T) * E, stage);
      __syncthreads();
      topk_chunk<COH, MODE>(a, stage, t0, min(ch, T - t0), ids_lds);
      __syncthreads();
    }
  }
  __threadfence_block();
  __syncthreads();
  dispatch_wg<COH>(a, lds, ids_lds ? ids_lds : a.rb.topk_ids);
}

}  // namespace moe
