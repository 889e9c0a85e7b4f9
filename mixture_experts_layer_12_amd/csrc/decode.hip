// Decode path: the expert FFNs for small batches (T <= 64 per pass), where the
// layer is bound by reading each engaged expert's weights once from HBM.
//
// Sources: "Why MoE on RTX 5090 falls short: a bandwidth measurement"
// (news.malakhovai.ru): mat-vec work dominates decode kernel time while
// routing is a small share (kernel-time split paragraph), and kernels that
// read little per launch do not reach full DRAM bandwidth (bandwidth versus
// bytes-per-kernel measurement) -- so each launch here covers every engaged
// expert at once and streams its rows with 16-byte loads.  "llama.cpp:
// fusing shared experts into MMVQ" (ai-manual.ru), sections "What MMVQ is and
// what CUDA has to do with it" (quantised weights are read once without being
// expanded to full precision in memory) and "How fusing shared experts into
// MMVQ can speed up inference" (shared experts in the same pass): the shared
// experts are extra slots of the same grid, and Q4_0 blocks are expanded in
// registers only.
//
// Two launches:
//   gate/up:  grid (row tile of 16 intermediate rows, expert slot).  Slots are
//             the active routed experts (compact list built by the router)
//             followed by the shared experts.  The 4 waves of a work-group
//             split the hidden dimension; partial sums meet in LDS.  The
//             epilogue applies silu(g) * u and the routing weight and writes
//             the activation rows in the format the down launch consumes.
//   down:     grid (row tile of 16 hidden outputs, split).  The waves of all
//             splits of one row tile share the (slot, k) space of that row
//             tile evenly; each wave folds its partial outputs into a private
//             LDS accumulator indexed by token and the work-group sums its
//             waves in a fixed order.  With one split the work-group writes
//             `out`; otherwise it writes its split's partial and a small
//             combine launch sums the splits in a fixed order.  The combine is
//             deterministic, needs no atomics, and needs no device-wide fence
//             (the kernel boundary orders the partials and their sum).
//
// Matrix cores do the dot products: weights are the A operand (16 rows per
// wave tile), tokens the B operand (16 per column tile).  bf16 weights use the
// bf16 MFMA with fp32 activations split into hi + lo bf16 parts; Q4_0 weights
// are dequantised in registers to fp16 and use the fp16 MFMA against fp16
// activations; fp32 weights use the fp32 MFMA.
#include "common.hpp"

namespace moe {

template <int WT> struct KPL;
template <> struct KPL<DT_F32> { static constexpr int v = 4; };
template <> struct KPL<DT_BF16> { static constexpr int v = 8; };
template <> struct KPL<DT_Q4> { static constexpr int v = 32; };

// Number of 4-lane-group steps along a reduction of length K.
template <int WT>
__host__ __device__ __forceinline__ int n_steps(int K) {
  if constexpr (WT == DT_Q4) return (K / 32 + 3) / 4;
  else return K / (4 * KPL<WT>::v);
}

// Row r of matrix `e` in a stack [n_mat, N, K].
template <int WT>
struct RowPtr {
  const uint8_t* p;        // first byte of the row (nibbles for Q4_0)
  const uint16_t* sc;      // Q4_0 scales of the row
  __device__ __forceinline__ void init(const uint8_t* base, long n_mat, long N, long K, long e, long r) {
    if constexpr (WT == DT_F32) p = base + (size_t(e) * N + r) * K * 4;
    else if constexpr (WT == DT_BF16) p = base + (size_t(e) * N + r) * K * 2;
    else {
      p = base + (size_t(e) * N + r) * (K / 2);
      sc = reinterpret_cast<const uint16_t*>(base + q4_scale_offset(n_mat, N, K)) + (size_t(e) * N + r) * (K / 32);
    }
  }
};

// A operand fragments of one step.
template <int WT> struct AFrag;
template <> struct AFrag<DT_F32> { u32x4_t v; };
template <> struct AFrag<DT_BF16> { u32x4_t v; };
template <> struct AFrag<DT_Q4> { u32x4_t raw; uint16_t d; };

template <int WT>
__device__ __forceinline__ AFrag<WT> load_a(const RowPtr<WT>& r, int s, int g, int K) {
  AFrag<WT> f;
  if constexpr (WT == DT_F32) f.v = ldg16(r.p + size_t(s * 16 + g * 4) * 4);
  else if constexpr (WT == DT_BF16) f.v = ldg16(r.p + size_t(s * 32 + g * 8) * 2);
  else {
    const int nblk = K / 32;
    int blk = 4 * s + g;
    const bool ok = blk < nblk;
    blk = ok ? blk : nblk - 1;
    f.raw = ldg16(r.p + size_t(blk) * 16);
    f.d = ok ? r.sc[blk] : uint16_t(0);
  }
  return f;
}

// -------------------------------------------------- B operand: activations --
// x rows (gate/up) in fp32 or bf16; for each weight type the lane supplies the
// k positions that its A fragment covers.

template <int WT, int XT> struct XFrag;
template <int XT> struct XFrag<DT_F32, XT> { float v[4]; };
template <> struct XFrag<DT_BF16, DT_BF16> { u32x4_t v; };
template <> struct XFrag<DT_BF16, DT_F32> { u32x4_t hi, lo; };
template <int XT> struct XFrag<DT_Q4, XT> { u32x4_t v[4]; };

template <int WT, int XT>
__device__ __forceinline__ XFrag<WT, XT> load_x(const uint8_t* xrow, bool ok, int s, int g, int K) {
  XFrag<WT, XT> b;
  if constexpr (WT == DT_F32) {
    const int k0 = s * 16 + g * 4;
    if constexpr (XT == DT_F32) {
      u32x4_t t = ldg16(xrow + size_t(k0) * 4);
#pragma unroll
      for (int m = 0; m < 4; ++m) b.v[m] = ok ? __uint_as_float(t[m]) : 0.f;
    } else {
      u32x2_t t = ldg8(xrow + size_t(k0) * 2);
      b.v[0] = ok ? bf16_lo(t[0]) : 0.f; b.v[1] = ok ? bf16_hi(t[0]) : 0.f;
      b.v[2] = ok ? bf16_lo(t[1]) : 0.f; b.v[3] = ok ? bf16_hi(t[1]) : 0.f;
    }
  } else if constexpr (WT == DT_BF16) {
    const int k0 = s * 32 + g * 8;
    if constexpr (XT == DT_BF16) {
      u32x4_t t = ldg16(xrow + size_t(k0) * 2);
      const u32x4_t z = {0, 0, 0, 0};
      b.v = ok ? t : z;
    } else {
      const float* xp = reinterpret_cast<const float*>(xrow) + k0;
      u32x4_t t0 = ldg16(xp), t1 = ldg16(xp + 4);
      float v[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        v[m] = ok ? __uint_as_float(t0[m]) : 0.f;
        v[m + 4] = ok ? __uint_as_float(t1[m]) : 0.f;
      }
      split_bf16x8(v, b.hi, b.lo);
    }
  } else {
    const int nblk = K / 32;
    int blk = 4 * s + g;
    ok = ok && blk < nblk;
    blk = blk < nblk ? blk : nblk - 1;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int k0 = blk * 32 + f * 8;
      if constexpr (XT == DT_F32) {
        const float* xp = reinterpret_cast<const float*>(xrow) + k0;
        u32x4_t t0 = ldg16(xp), t1 = ldg16(xp + 4);
        b.v[f][0] = pack_f16(__uint_as_float(t0[0]), __uint_as_float(t0[1]));
        b.v[f][1] = pack_f16(__uint_as_float(t0[2]), __uint_as_float(t0[3]));
        b.v[f][2] = pack_f16(__uint_as_float(t1[0]), __uint_as_float(t1[1]));
        b.v[f][3] = pack_f16(__uint_as_float(t1[2]), __uint_as_float(t1[3]));
      } else {
        u32x4_t t = ldg16(xrow + size_t(k0) * 2);
#pragma unroll
        for (int m = 0; m < 4; ++m) b.v[f][m] = bf16x2_to_f16x2(t[m]);
      }
      if (!ok) b.v[f] = u32x4_t{0, 0, 0, 0};
    }
  }
  return b;
}

template <int WT, int XT>
__device__ __forceinline__ f32x4_t mma(const AFrag<WT>& a, const XFrag<WT, XT>& b, f32x4_t c) {
  if constexpr (WT == DT_F32) {
#pragma unroll
    for (int m = 0; m < 4; ++m) c = mfma_f32(__uint_as_float(a.v[m]), b.v[m], c);
  } else if constexpr (WT == DT_BF16) {
    if constexpr (XT == DT_BF16) c = mfma_bf16(a.v, b.v, c);
    else {
      c = mfma_bf16(a.v, b.hi, c);
      c = mfma_bf16(a.v, b.lo, c);
    }
  } else {
    u32x4_t fr[4];
    q4_dequant_block(a.raw, a.d, fr);
#pragma unroll
    for (int f = 0; f < 4; ++f) c = mfma_f16(fr[f], b.v[f], c);
  }
  return c;
}

// Q4_0 A fragments are dequantised once and used for every column tile.
template <int WT>
struct AReady { AFrag<WT> a; };
template <>
struct AReady<DT_Q4> { u32x4_t fr[4]; };

template <int WT>
__device__ __forceinline__ AReady<WT> prep_a(const AFrag<WT>& a) {
  AReady<WT> r;
  if constexpr (WT == DT_Q4) q4_dequant_block(a.raw, a.d, r.fr);
  else r.a = a;
  return r;
}

template <int WT, int XT>
__device__ __forceinline__ f32x4_t mma_ready(const AReady<WT>& a, const XFrag<WT, XT>& b, f32x4_t c) {
  if constexpr (WT == DT_Q4) {
#pragma unroll
    for (int f = 0; f < 4; ++f) c = mfma_f16(a.fr[f], b.v[f], c);
    return c;
  } else {
    return mma<WT, XT>(a.a, b, c);
  }
}

// Unroll depth: keep several 16-byte weight loads in flight per lane.
#ifndef MOE_GU_UNROLL_BF16
#define MOE_GU_UNROLL_BF16 8
#endif
#ifndef MOE_DN_UNROLL_BF16
#define MOE_DN_UNROLL_BF16 8
#endif
template <int WT, int NCT>
struct Unroll {
  static constexpr int v = (WT == DT_BF16) ? (NCT == 1 ? MOE_GU_UNROLL_BF16 : 2) : (NCT == 1 ? 4 : 1);
};
template <int WT, int NCT>
struct UnrollDown {
  static constexpr int v = (WT == DT_BF16) ? (NCT == 1 ? MOE_DN_UNROLL_BF16 : 4) : (NCT == 1 ? 8 : 2);
};

// ------------------------------------------------------------- gate/up --

template <int WT, int XT, int NCT>
__global__ void __launch_bounds__(256) decode_gateup_kernel(DecodeArgs a) {
  __shared__ f32x4_t red[4][2 * NCT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rt = blockIdx.x, slot = blockIdx.y;
  const bool routed = slot < a.n_routed_slots;
  int e, n_e, hrow0, N, seg = 0;
  long n_mat;
  const uint8_t *bg, *bu;
  if (routed) {
    if (slot >= a.active[0]) return;
    e = a.active[1 + slot];
    n_e = a.counts[e];
    seg = a.offsets[e];
    hrow0 = a.cprefix[e];
    N = a.I; bg = a.wg; bu = a.wu; n_mat = a.E;
  } else {
    e = slot - a.n_routed_slots;
    n_e = a.T;
    hrow0 = a.T * a.k + e * a.T;
    N = a.Is; bg = a.sg; bu = a.su; n_mat = a.S;
  }
  if (rt * 16 >= N) return;
  const int K = a.H, g = lane >> 4;
  RowPtr<WT> rg, ru;
  rg.init(bg, n_mat, N, K, e, rt * 16 + (lane & 15));
  ru.init(bu, n_mat, N, K, e, rt * 16 + (lane & 15));

  constexpr int xb = XT == DT_F32 ? 4 : 2;
  const uint8_t* xrow[NCT];
  bool xok[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int c = ct * 16 + (lane & 15);
    xok[ct] = c < n_e;
    int tok = 0;
    if (xok[ct]) tok = routed ? a.sorted_ids[seg + c] / a.k : c;
    xrow[ct] = reinterpret_cast<const uint8_t*>(a.x) + size_t(tok) * K * xb;
  }
  const int nct = (n_e + 15) >> 4;

  const int nsteps = n_steps<WT>(K);
  const int s0 = wave * nsteps / 4, s1 = (wave + 1) * nsteps / 4;
  f32x4_t accg[NCT], accu[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) accg[ct] = accu[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int U = Unroll<WT, NCT>::v;
  auto body = [&](int s, const AFrag<WT>& fa_g, const AFrag<WT>& fa_u) {
    const AReady<WT> ag = prep_a<WT>(fa_g), au = prep_a<WT>(fa_u);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (NCT == 1 || ct < nct) {
        XFrag<WT, XT> b = load_x<WT, XT>(xrow[ct], xok[ct], s, g, K);
        accg[ct] = mma_ready<WT, XT>(ag, b, accg[ct]);
        accu[ct] = mma_ready<WT, XT>(au, b, accu[ct]);
      }
    }
  };
  int s = s0;
  for (; s + U <= s1; s += U) {
    AFrag<WT> fg[U], fu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      fg[u] = load_a<WT>(rg, s + u, g, K);
      fu[u] = load_a<WT>(ru, s + u, g, K);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) body(s + u, fg[u], fu[u]);
  }
  for (; s < s1; ++s) body(s, load_a<WT>(rg, s, g, K), load_a<WT>(ru, s, g, K));

#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    red[wave][ct][lane] = accg[ct];
    red[wave][NCT + ct][lane] = accu[ct];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    if (!(NCT == 1 || ct < nct)) continue;
    f32x4_t gs = red[0][ct][lane], us = red[0][NCT + ct][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      gs += red[w][ct][lane];
      us += red[w][NCT + ct][lane];
    }
    const int c = ct * 16 + (lane & 15);
    if (c >= n_e) continue;
    const float wr = routed ? a.topk_w[a.sorted_ids[seg + c]] : 1.0f;
    float hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu_f(gs[i]) * us[i] * wr;
    const size_t off = size_t(hrow0 + c) * a.h_stride + rt * 16 + (lane >> 4) * 4;
    if constexpr (WT == DT_F32) {
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.h) + off) = f32x4_t{hv[0], hv[1], hv[2], hv[3]};
    } else if constexpr (WT == DT_BF16) {
      uint32_t h0 = f32_to_bf16(hv[0]), h1 = f32_to_bf16(hv[1]), h2 = f32_to_bf16(hv[2]), h3 = f32_to_bf16(hv[3]);
      float r0 = hv[0] - __uint_as_float(h0 << 16), r1 = hv[1] - __uint_as_float(h1 << 16);
      float r2 = hv[2] - __uint_as_float(h2 << 16), r3 = hv[3] - __uint_as_float(h3 << 16);
      uint16_t* hp = reinterpret_cast<uint16_t*>(a.h);
      *reinterpret_cast<u32x2_t*>(hp + off) = u32x2_t{h0 | (h1 << 16), h2 | (h3 << 16)};
      *reinterpret_cast<u32x2_t*>(hp + a.h_plane + off) = u32x2_t{pack_bf16(r0, r1), pack_bf16(r2, r3)};
    } else {
      uint16_t* hp = reinterpret_cast<uint16_t*>(a.h);
      *reinterpret_cast<u32x2_t*>(hp + off) = u32x2_t{pack_f16(hv[0], hv[1]), pack_f16(hv[2], hv[3])};
    }
  }
}

// ---------------------------------------------------------------- down --

// B operand of the down projection: activation rows written by gate/up.
template <int WT> struct HFrag;
template <> struct HFrag<DT_F32> { float v[4]; };
template <> struct HFrag<DT_BF16> { u32x4_t hi, lo; };
template <> struct HFrag<DT_Q4> { u32x4_t v[4]; };

template <int WT>
__device__ __forceinline__ HFrag<WT> load_h(const DecodeArgs& a, size_t row_off, bool ok, int s, int g, int K) {
  HFrag<WT> b;
  const u32x4_t z = {0, 0, 0, 0};
  if constexpr (WT == DT_F32) {
    u32x4_t t = ldg16(reinterpret_cast<const float*>(a.h) + row_off + s * 16 + g * 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) b.v[m] = ok ? __uint_as_float(t[m]) : 0.f;
  } else if constexpr (WT == DT_BF16) {
    const uint16_t* hp = reinterpret_cast<const uint16_t*>(a.h) + row_off + s * 32 + g * 8;
    u32x4_t t0 = ldg16(hp), t1 = ldg16(hp + a.h_plane);
    b.hi = ok ? t0 : z;
    b.lo = ok ? t1 : z;
  } else {
    const int nblk = K / 32;
    int blk = 4 * s + g;
    ok = ok && blk < nblk;
    blk = blk < nblk ? blk : nblk - 1;
    const uint16_t* hp = reinterpret_cast<const uint16_t*>(a.h) + row_off + blk * 32;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      u32x4_t t = ldg16(hp + f * 8);
      b.v[f] = ok ? t : z;
    }
  }
  return b;
}

template <int WT>
__device__ __forceinline__ f32x4_t mma_h(const AReady<WT>& a, const HFrag<WT>& b, f32x4_t c) {
  if constexpr (WT == DT_F32) {
#pragma unroll
    for (int m = 0; m < 4; ++m) c = mfma_f32(__uint_as_float(a.a.v[m]), b.v[m], c);
  } else if constexpr (WT == DT_BF16) {
    c = mfma_bf16(a.a.v, b.hi, c);
    c = mfma_bf16(a.a.v, b.lo, c);
  } else {
#pragma unroll
    for (int f = 0; f < 4; ++f) c = mfma_f16(a.fr[f], b.v[f], c);
  }
  return c;
}

template <int WT, int OT, int NCT>
__global__ void __launch_bounds__(256) decode_down_kernel(DecodeArgs a) {
  extern __shared__ float acc_lds[];     // [4 waves][16 rows][T]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int rt = blockIdx.x, split = blockIdx.y;
  const int T = a.T, g = lane >> 4, H = a.H;
  float* myacc = acc_lds + wave * 16 * T;
  for (int i = lane; i < 16 * T; i += 64) myacc[i] = 0.f;

  const int n_act = a.active[0];
  const int SR = n_steps<WT>(a.I), SS = n_steps<WT>(a.Is);
  const long routed_steps = long(n_act) * SR;
  const long total = routed_steps + long(a.S) * SS;
  const long G = long(a.nsplit) * 4, gw = long(split) * 4 + wave;
  long pos = total * gw / G;
  const long r1 = total * (gw + 1) / G;
  const int row = rt * 16 + (lane & 15);
  constexpr int U = UnrollDown<WT, NCT>::v;

  while (pos < r1) {
    int e, n_e, hrow0, seg = 0, K, sstep, sl_steps;
    long n_mat;
    const uint8_t* base;
    bool routed;
    if (pos < routed_steps) {
      const int slot = int(pos / SR);
      sstep = int(pos % SR);
      sl_steps = SR;
      e = a.active[1 + slot];
      n_e = a.counts[e];
      seg = a.offsets[e];
      hrow0 = a.cprefix[e];
      K = a.I; base = a.wd; n_mat = a.E; routed = true;
    } else {
      const long q = pos - routed_steps;
      e = int(q / SS);
      sstep = int(q % SS);
      sl_steps = SS;
      n_e = T;
      hrow0 = T * a.k + e * T;
      K = a.Is; base = a.sd; n_mat = a.S; routed = false;
    }
    const int cnt = int(min(long(sl_steps - sstep), r1 - pos));
    RowPtr<WT> rw;
    rw.init(base, n_mat, H, K, e, row);
    size_t hoff[NCT];
    bool hok[NCT];
    int tok[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int c = ct * 16 + (lane & 15);
      hok[ct] = c < n_e;
      const int cc = hok[ct] ? c : 0;
      hoff[ct] = size_t(hrow0 + cc) * a.h_stride;
      tok[ct] = routed ? a.sorted_ids[seg + cc] / a.k : cc;
    }
    const int nct = (n_e + 15) >> 4;
    f32x4_t acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto body = [&](int s, const AFrag<WT>& fa) {
      const AReady<WT> ar = prep_a<WT>(fa);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if (NCT == 1 || ct < nct) {
          HFrag<WT> b = load_h<WT>(a, hoff[ct], hok[ct], s, g, K);
          acc[ct] = mma_h<WT>(ar, b, acc[ct]);
        }
      }
    };
    int s = sstep;
    const int s_end = sstep + cnt;
    for (; s + U <= s_end; s += U) {
      AFrag<WT> fa[U];
#pragma unroll
      for (int u = 0; u < U; ++u) fa[u] = load_a<WT>(rw, s + u, g, K);
#pragma unroll
      for (int u = 0; u < U; ++u) body(s + u, fa[u]);
    }
    for (; s < s_end; ++s) body(s, load_a<WT>(rw, s, g, K));

    // fold into this wave's accumulator (distinct (row, token) per lane)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if ((NCT == 1 || ct < nct) && hok[ct]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) myacc[((lane >> 4) * 4 + i) * T + tok[ct]] += acc[ct][i];
      }
    }
    pos += cnt;
  }
  __syncthreads();

  // waves -> work-group sum, in wave order (region of wave 0 reused)
  for (int idx = tid; idx < 16 * T; idx += 256) {
    float v = acc_lds[idx];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += acc_lds[w * 16 * T + idx];
    acc_lds[idx] = v;
  }
  __syncthreads();
  for (int j = tid; j < 16 * T; j += 256) {
    const int t = j >> 4, r = j & 15;
    const float v = acc_lds[r * T + t];
    const size_t o = size_t(t) * H + rt * 16 + r;
    if (a.nsplit > 1) {
      a.partials[size_t(split) * T * H + o] = v;      // summed by decode_combine_kernel
    } else if constexpr (OT == DT_F32) {
      reinterpret_cast<float*>(a.out)[o] = v;
    } else {
      reinterpret_cast<uint16_t*>(a.out)[o] = uint16_t(f32_to_bf16(v));
    }
  }
}

// Sum of the split partials [nsplit][T*H] in split order -> out (4 outputs per thread).
template <int OT>
__global__ void __launch_bounds__(256) decode_combine_kernel(const float* __restrict__ partials, void* out,
                                                             int nsplit, long n) {
  const long i4 = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i4 * 4 >= n) return;
  f32x4_t v = reinterpret_cast<const f32x4_t*>(partials)[i4];
  for (int sp = 1; sp < nsplit; ++sp) v += reinterpret_cast<const f32x4_t*>(partials + size_t(sp) * n)[i4];
  if constexpr (OT == DT_F32) reinterpret_cast<f32x4_t*>(out)[i4] = v;
  else reinterpret_cast<u32x2_t*>(out)[i4] = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}

// -------------------------------------------------------------- launch --

template <int WT, int XT, int NCT>
static void launch_decode_t(const DecodeArgs& a, int n_gu_row_tiles, hipStream_t st, StageMarker* mark) {
  dim3 g1(n_gu_row_tiles, a.n_routed_slots + a.S), b(256);
  hipLaunchKernelGGL((decode_gateup_kernel<WT, XT, NCT>), g1, b, 0, st, a);
  if (mark) mark->mark(st);
  dim3 g2(a.H / 16, a.nsplit);
  const size_t lds = size_t(4) * 16 * a.T * sizeof(float);
  hipLaunchKernelGGL((decode_down_kernel<WT, XT, NCT>), g2, b, lds, st, a);
  if (a.nsplit > 1) {
    const long n = long(a.T) * a.H;
    hipLaunchKernelGGL((decode_combine_kernel<XT>), dim3(int((n / 4 + 255) / 256)), b, 0, st, a.partials, a.out,
                       a.nsplit, n);
  }
  if (mark) mark->mark(st);
}

template <int WT, int XT>
static void launch_decode_x(const DecodeArgs& a, int n_gu_row_tiles, hipStream_t st, StageMarker* mark) {
  if (a.T <= 16) launch_decode_t<WT, XT, 1>(a, n_gu_row_tiles, st, mark);
  else launch_decode_t<WT, XT, 4>(a, n_gu_row_tiles, st, mark);
}

hipError_t launch_decode(const DecodeArgs& a, int wdt, int xdt, int n_gu_row_tiles, hipStream_t st,
                         StageMarker* mark) {
  if (wdt == DT_F32) {
    if (xdt == DT_F32) launch_decode_x<DT_F32, DT_F32>(a, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_F32, DT_BF16>(a, n_gu_row_tiles, st, mark);
  } else if (wdt == DT_BF16) {
    if (xdt == DT_F32) launch_decode_x<DT_BF16, DT_F32>(a, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_BF16, DT_BF16>(a, n_gu_row_tiles, st, mark);
  } else {
    if (xdt == DT_F32) launch_decode_x<DT_Q4, DT_F32>(a, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_Q4, DT_BF16>(a, n_gu_row_tiles, st, mark);
  }
  return hipGetLastError();
}

}  // namespace moe
