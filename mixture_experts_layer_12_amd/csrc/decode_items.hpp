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
// Three launches:
//   gate/up:  grid (row tile of 16 intermediate rows, expert slot).  Slots are
//             the active routed experts (compact list built by the router)
//             followed by the shared experts.  The 4 waves of a work-group
//             split the hidden dimension; partial sums meet in LDS.  The
//             epilogue applies silu(g) * u and the routing weight and writes
//             the activation rows in the format the down launch consumes.
//   down:     grid (row tile of 16 hidden outputs, expert slot), the same
//             shape as gate/up: the 4 waves split the slot's intermediate
//             dimension and meet in LDS; the work-group writes the slot's
//             routing-weighted output rows (one row per assignment) once.
//   combine:  out[t] = the k assignment rows of token t (located through the
//             dispatch's inverse permutation) plus its shared-expert rows,
//             summed in a fixed order.  Deterministic, no atomics, and no
//             device-wide fence (the kernel boundary orders the handoff).
//
// Matrix cores do the dot products: weights are the A operand (16 rows per
// wave tile), tokens the B operand (16 per column tile).  bf16 weights use the
// bf16 MFMA with fp32 activations split into hi + lo bf16 parts; Q4_0 weights
// are dequantised in registers to fp16 and use the fp16 MFMA against fp16
// activations; fp32 weights use the fp32 MFMA.
#pragma once
#include "common.hpp"
#include "router_items.hpp"

namespace moe {

// Operand family of a stored weight type: the MFMA it feeds, the activation
// (B operand) layout and the format of the activation rows between gate/up
// and down.  Q8_0 shares Q4_0's (one 32-value block per lane group, fp16);
// fp8 has its own (16 codes per lane group, two fp16 k-slices of 8, fp16
// activation rows).
template <int WT> struct Fam { static constexpr int v = WT; };
template <> struct Fam<DT_Q8> { static constexpr int v = DT_Q4; };

// Number of 4-lane-group steps along a reduction of length K.
template <int WT>
__host__ __device__ __forceinline__ int n_steps(int K) {
  if constexpr (WT == DT_F32) return K / 16;
  else if constexpr (WT == DT_BF16) return K / 32;
  else if constexpr (WT == DT_FP8) return (K + 63) / 64;
  else return (K / 32 + 3) / 4;                    // Q4_0, Q8_0
}

// Row r of matrix `e` in a stack [n_mat, N, K].
template <int WT>
struct RowPtr {
  const uint8_t* p;        // first byte of the row (codes for the quantised types)
  const uint16_t* sc;      // Q4_0 / Q8_0 block scales of the row
  __device__ __forceinline__ void init(const uint8_t* base, long n_mat, long N, long K, long e, long r) {
    const size_t row = size_t(e) * N + r;
    if constexpr (WT == DT_F32) p = base + row * K * 4;
    else if constexpr (WT == DT_BF16) p = base + row * K * 2;
    else if constexpr (WT == DT_Q4) {
      p = base + row * (K / 2);
      sc = reinterpret_cast<const uint16_t*>(base + q4_scale_offset(n_mat, N, K)) + row * (K / 32);
    } else if constexpr (WT == DT_Q8) {
      p = base + row * K;
      sc = reinterpret_cast<const uint16_t*>(base + byte_code_scale_offset(n_mat, N, K)) + row * (K / 32);
    } else {
      p = base + row * K;
    }
  }
};

// fp8 row scales of output rows r0 .. r0+3 of matrix e (one 16-byte load).
__device__ __forceinline__ f32x4_t fp8_row_scales(const uint8_t* base, long n_mat, long N, long K, long e, long r0) {
  return *(const __attribute__((address_space(1))) f32x4_t*)(base + byte_code_scale_offset(n_mat, N, K) +
                                                             (size_t(e) * N + r0) * 4);
}

// A operand fragments of one step, as loaded.
template <int WT> struct AFrag;
template <> struct AFrag<DT_F32> { u32x4_t v; };
template <> struct AFrag<DT_BF16> { u32x4_t v; };
template <> struct AFrag<DT_Q4> { u32x4_t raw; uint16_t d; };
template <> struct AFrag<DT_Q8> { u32x4_t raw0, raw1; uint16_t d; };
template <> struct AFrag<DT_FP8> { u32x4_t raw; bool ok; };

template <int WT>
__device__ __forceinline__ AFrag<WT> load_a(const RowPtr<WT>& r, int s, int g, int K) {
  AFrag<WT> f;
  if constexpr (WT == DT_F32) f.v = ldg16(r.p + size_t(s * 16 + g * 4) * 4);
  else if constexpr (WT == DT_BF16) f.v = ldg16(r.p + size_t(s * 32 + g * 8) * 2);
  else if constexpr (WT == DT_FP8) {
    const int k0 = s * 64 + g * 16;
    f.ok = k0 < K;
    f.raw = ldg16(r.p + (f.ok ? k0 : K - 16));     // past the end: a valid address, zeroed in prep_a
  } else {
    const int nblk = K / 32;
    int blk = 4 * s + g;
    const bool ok = blk < nblk;
    blk = ok ? blk : nblk - 1;
    if constexpr (WT == DT_Q4) {
      f.raw = ldg16(r.p + size_t(blk) * 16);
    } else {
      f.raw0 = ldg16(r.p + size_t(blk) * 32);
      f.raw1 = ldg16(r.p + size_t(blk) * 32 + 16);
    }
    f.d = ok ? *(const __attribute__((address_space(1))) uint16_t*)(r.sc + blk) : uint16_t(0);
  }
  return f;
}

// A operand ready for the MFMA of its family (quantised codes expanded once
// per step and used for every column tile).
template <int F> struct AReady;
template <> struct AReady<DT_F32> { u32x4_t v; };
template <> struct AReady<DT_BF16> { u32x4_t v; };
template <> struct AReady<DT_Q4> { u32x4_t fr[4]; };
template <> struct AReady<DT_FP8> { u32x4_t v[2]; };       // fp16x8 each

template <int WT>
__device__ __forceinline__ AReady<Fam<WT>::v> prep_a(const AFrag<WT>& a) {
  AReady<Fam<WT>::v> r;
  if constexpr (WT == DT_F32 || WT == DT_BF16) r.v = a.v;
  else if constexpr (WT == DT_Q4) q4_dequant_block(a.raw, a.d, r.fr);
  else if constexpr (WT == DT_Q8) q8_dequant_block(a.raw0, a.raw1, a.d, r.fr);
  else fp8x16_to_f16(a.ok ? a.raw : u32x4_t{0, 0, 0, 0}, r.v);
  return r;
}

// -------------------------------------------------- B operand: activations --
// x rows (gate/up) in fp32 or bf16; for each family the lane supplies the k
// positions that its A fragment covers.

template <int F, int XT> struct XFrag;
template <int XT> struct XFrag<DT_F32, XT> { float v[4]; };
template <> struct XFrag<DT_BF16, DT_BF16> { u32x4_t v; };
template <> struct XFrag<DT_BF16, DT_F32> { u32x4_t hi, lo; };
template <int XT> struct XFrag<DT_Q4, XT> { u32x4_t v[4]; };
template <int XT> struct XFrag<DT_FP8, XT> { u32x4_t v[2]; };       // fp16x8 each

// Raw activation words of one step, loaded with the step's weights and only
// turned into MFMA operands (cook_x) when the step is computed, so that no
// wait for them is placed where the loads are issued.
template <int F, int XT> struct XRaw;
template <> struct XRaw<DT_F32, DT_F32> { u32x4_t t; };
template <> struct XRaw<DT_F32, DT_BF16> { u32x2_t t; };
template <> struct XRaw<DT_BF16, DT_BF16> { u32x4_t t; };
template <> struct XRaw<DT_BF16, DT_F32> { u32x4_t t0, t1; };
template <> struct XRaw<DT_Q4, DT_F32> { u32x4_t t[8]; };
template <> struct XRaw<DT_Q4, DT_BF16> { u32x4_t t[4]; };
template <> struct XRaw<DT_FP8, DT_F32> { u32x4_t t[4]; };
template <> struct XRaw<DT_FP8, DT_BF16> { u32x4_t t[2]; };

// 8 activations from k0 as one bf16-family operand.
template <int XT>
__device__ __forceinline__ XRaw<DT_BF16, XT> load_x8(const uint8_t* xrow, int k0) {
  XRaw<DT_BF16, XT> r;
  if constexpr (XT == DT_BF16) {
    r.t = ldg16(xrow + size_t(k0) * 2);
  } else {
    const float* xp = reinterpret_cast<const float*>(xrow) + k0;
    r.t0 = ldg16(xp);
    r.t1 = ldg16(xp + 4);
  }
  return r;
}

template <int F, int XT>
__device__ __forceinline__ XRaw<F, XT> load_x_raw(const uint8_t* xrow, int s, int g, int K) {
  XRaw<F, XT> r;
  if constexpr (F == DT_F32) {
    const int k0 = s * 16 + g * 4;
    if constexpr (XT == DT_F32) r.t = ldg16(xrow + size_t(k0) * 4);
    else r.t = ldg8(xrow + size_t(k0) * 2);
  } else if constexpr (F == DT_BF16) {
    r = load_x8<XT>(xrow, s * 32 + g * 8);
  } else if constexpr (F == DT_FP8) {
    int k0 = s * 64 + g * 16;
    k0 = k0 < K ? k0 : K - 16;
    if constexpr (XT == DT_F32) {
      const float* xp = reinterpret_cast<const float*>(xrow) + k0;
#pragma unroll
      for (int q = 0; q < 4; ++q) r.t[q] = ldg16(xp + 4 * q);
    } else {
      r.t[0] = ldg16(xrow + size_t(k0) * 2);
      r.t[1] = ldg16(xrow + size_t(k0 + 8) * 2);
    }
  } else {
    const int nblk = K / 32;
    int blk = 4 * s + g;
    blk = blk < nblk ? blk : nblk - 1;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int k0 = blk * 32 + f * 8;
      if constexpr (XT == DT_F32) {
        const float* xp = reinterpret_cast<const float*>(xrow) + k0;
        r.t[2 * f] = ldg16(xp);
        r.t[2 * f + 1] = ldg16(xp + 4);
      } else {
        r.t[f] = ldg16(xrow + size_t(k0) * 2);
      }
    }
  }
  return r;
}

template <int XT>
__device__ __forceinline__ XFrag<DT_BF16, XT> cook_x8(const XRaw<DT_BF16, XT>& r, bool ok) {
  XFrag<DT_BF16, XT> b;
  if constexpr (XT == DT_BF16) {
    const u32x4_t z = {0, 0, 0, 0};
    b.v = ok ? r.t : z;
  } else {
    float v[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v[m] = ok ? __uint_as_float(r.t0[m]) : 0.f;
      v[m + 4] = ok ? __uint_as_float(r.t1[m]) : 0.f;
    }
    split_bf16x8(v, b.hi, b.lo);
  }
  return b;
}

template <int F, int XT>
__device__ __forceinline__ XFrag<F, XT> cook_x(const XRaw<F, XT>& r, bool ok, int s, int g, int K) {
  XFrag<F, XT> b;
  if constexpr (F == DT_F32) {
    if constexpr (XT == DT_F32) {
#pragma unroll
      for (int m = 0; m < 4; ++m) b.v[m] = ok ? __uint_as_float(r.t[m]) : 0.f;
    } else {
      b.v[0] = ok ? bf16_lo(r.t[0]) : 0.f; b.v[1] = ok ? bf16_hi(r.t[0]) : 0.f;
      b.v[2] = ok ? bf16_lo(r.t[1]) : 0.f; b.v[3] = ok ? bf16_hi(r.t[1]) : 0.f;
    }
  } else if constexpr (F == DT_BF16) {
    b = cook_x8<XT>(r, ok);
  } else if constexpr (F == DT_FP8) {
    ok = ok && s * 64 + g * 16 < K;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (XT == DT_F32) {
        const u32x4_t t0 = r.t[2 * i], t1 = r.t[2 * i + 1];
        b.v[i][0] = pack_f16(__uint_as_float(t0[0]), __uint_as_float(t0[1]));
        b.v[i][1] = pack_f16(__uint_as_float(t0[2]), __uint_as_float(t0[3]));
        b.v[i][2] = pack_f16(__uint_as_float(t1[0]), __uint_as_float(t1[1]));
        b.v[i][3] = pack_f16(__uint_as_float(t1[2]), __uint_as_float(t1[3]));
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) b.v[i][m] = bf16x2_to_f16x2(r.t[i][m]);
      }
      if (!ok) b.v[i] = u32x4_t{0, 0, 0, 0};
    }
  } else {
    ok = ok && (4 * s + g) < K / 32;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if constexpr (XT == DT_F32) {
        const u32x4_t t0 = r.t[2 * f], t1 = r.t[2 * f + 1];
        b.v[f][0] = pack_f16(__uint_as_float(t0[0]), __uint_as_float(t0[1]));
        b.v[f][1] = pack_f16(__uint_as_float(t0[2]), __uint_as_float(t0[3]));
        b.v[f][2] = pack_f16(__uint_as_float(t1[0]), __uint_as_float(t1[1]));
        b.v[f][3] = pack_f16(__uint_as_float(t1[2]), __uint_as_float(t1[3]));
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) b.v[f][m] = bf16x2_to_f16x2(r.t[f][m]);
      }
      if (!ok) b.v[f] = u32x4_t{0, 0, 0, 0};
    }
  }
  return b;
}

template <int F, int XT>
__device__ __forceinline__ f32x4_t mma_ready(const AReady<F>& a, const XFrag<F, XT>& b, f32x4_t c) {
  if constexpr (F == DT_F32) {
#pragma unroll
    for (int m = 0; m < 4; ++m) c = mfma_f32(__uint_as_float(a.v[m]), b.v[m], c);
  } else if constexpr (F == DT_BF16) {
    if constexpr (XT == DT_BF16) c = mfma_bf16(a.v, b.v, c);
    else {
      c = mfma_bf16(a.v, b.hi, c);
      c = mfma_bf16(a.v, b.lo, c);
    }
  } else if constexpr (F == DT_FP8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) c = mfma_f16(a.v[i], b.v[i], c);
  } else {
#pragma unroll
    for (int f = 0; f < 4; ++f) c = mfma_f16(a.fr[f], b.v[f], c);
  }
  return c;
}

// Unroll depth: keep several 16-byte weight loads in flight per lane.
#ifndef MOE_GU_UNROLL_BF16
#define MOE_GU_UNROLL_BF16 4
#endif
// fp8 holds its raw codes and their fp16 expansion: two steps in flight keep
// more waves resident (Mixtral-shaped batch of 8: 4 steps 162 us, 3 159, 2 155)
#ifndef MOE_GU_UNROLL_FP8
#define MOE_GU_UNROLL_FP8 2
#endif
#ifndef MOE_DN_UNROLL_BF16
#define MOE_DN_UNROLL_BF16 2
#endif
// bf16 and fp8 load one 16-byte word per matrix and step, the others more.
template <int WT, int NCT>
struct Unroll {
  static constexpr bool one_word = WT == DT_BF16 || WT == DT_FP8;
  static constexpr int v = one_word ? (NCT == 1 ? (WT == DT_FP8 ? MOE_GU_UNROLL_FP8 : MOE_GU_UNROLL_BF16) : 2)
                                    : (NCT == 1 ? 2 : 1);
};
template <int WT, int NCT>
struct UnrollDown {
  static constexpr bool one_word = WT == DT_BF16 || WT == DT_FP8;
  static constexpr int v = one_word ? (NCT == 1 ? MOE_DN_UNROLL_BF16 : 1) : (NCT == 1 ? 2 : 1);
};

// Steps [s0, s1) in groups of U with the weight loads of group i+1 issued
// before the MFMAs of group i, so the wave keeps weight bytes in flight
// across group boundaries (a plain unrolled loop drains them at every group).
// `load(s)` returns the A fragments of step s, `body(s, frag)` consumes them.
// Masked B: lanes of token columns past the slot's count issue no activation
// loads (their operand is zeroed anyway).  Pays off in gate/up, not in down.
#ifndef MOE_GU_MASKED_B
#define MOE_GU_MASKED_B 1
#endif
#ifndef MOE_DN_MASKED_B
#define MOE_DN_MASKED_B 0
#endif
#ifndef MOE_DECODE_PIPELINE
#define MOE_DECODE_PIPELINE 1
#endif
template <int U, class Load, class Body>
__device__ __forceinline__ void stream_steps(int s0, int s1, Load load, Body body) {
  using F = decltype(load(0));
  int s = s0;
  if (!MOE_DECODE_PIPELINE) {
    for (; s + U <= s1; s += U) {
      F cur[U];
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = load(s + u);
#pragma unroll
      for (int u = 0; u < U; ++u) body(s + u, cur[u]);
    }
    for (; s < s1; ++s) body(s, load(s));
    return;
  }
  if (s + U <= s1) {
    F cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = load(s + u);
    for (; s + 2 * U <= s1; s += U) {
      F nxt[U];
#pragma unroll
      for (int u = 0; u < U; ++u) nxt[u] = load(s + U + u);
#pragma unroll
      for (int u = 0; u < U; ++u) body(s + u, cur[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) body(s + u, cur[u]);
    s += U;
  }
  for (; s < s1; ++s) body(s, load(s));
}

template <int WT, int XT, int NCT>
struct GUStep { AFrag<WT> g, u; XRaw<Fam<WT>::v, XT> x[NCT]; };

// Activations staged once per work-group as fp16 rows [T, K] in LDS, for the
// fp16-operand families (Q4_0, Q8_0) of small latency-bound batches: the
// weight loads of a step then need no activation loads beside them, so a
// wave can keep all of its steps' weight loads in flight at once.  The fp16
// values are the ones cook_x forms (same rounding), so the results are the
// same bits.  stage_x_load issues a thread's loads, stage_x_store converts
// and stores them (8 values per thread and round; T * K / 8 <= kStageX8 *
// blockDim.x).
constexpr int kStageX8 = 4;
template <int XT> struct XStage { u32x4_t t[kStageX8][XT == DT_F32 ? 2 : 1]; };

template <int XT>
__device__ __forceinline__ XStage<XT> stage_x_load(const void* x, int n8) {
  XStage<XT> r;
#pragma unroll
  for (int q = 0; q < kStageX8; ++q) {
    const int i = min(int(threadIdx.x) + q * int(blockDim.x), n8 - 1);
    if constexpr (XT == DT_F32) {
      r.t[q][0] = ldg16(reinterpret_cast<const float*>(x) + size_t(i) * 8);
      r.t[q][1] = ldg16(reinterpret_cast<const float*>(x) + size_t(i) * 8 + 4);
    } else {
      r.t[q][0] = ldg16(reinterpret_cast<const uint16_t*>(x) + size_t(i) * 8);
    }
  }
  return r;
}

template <int XT>
__device__ __forceinline__ void stage_x_store(const XStage<XT>& r, int n8, uint16_t* xs) {
#pragma unroll
  for (int q = 0; q < kStageX8; ++q) {
    const int i = int(threadIdx.x) + q * int(blockDim.x);
    if (i >= n8) continue;
    u32x4_t v;
    if constexpr (XT == DT_F32) {
      const u32x4_t t0 = r.t[q][0], t1 = r.t[q][1];
      v = u32x4_t{pack_f16(__uint_as_float(t0[0]), __uint_as_float(t0[1])),
                  pack_f16(__uint_as_float(t0[2]), __uint_as_float(t0[3])),
                  pack_f16(__uint_as_float(t1[0]), __uint_as_float(t1[1])),
                  pack_f16(__uint_as_float(t1[2]), __uint_as_float(t1[3]))};
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) v[m] = bf16x2_to_f16x2(r.t[q][0][m]);
    }
    *reinterpret_cast<u32x4_t*>(xs + size_t(i) * 8) = v;
  }
}

// The fp16 B operand of one step read from the staged rows (Q4_0 family
// layout, as load_x_raw + cook_x): zero past K or for an empty column.
__device__ __forceinline__ XFrag<DT_Q4, DT_F32> lds_x_frag(const uint16_t* xrow, bool ok, int s, int g, int K) {
  XFrag<DT_Q4, DT_F32> b;
  const int nblk = K / 32;
  const int blk = 4 * s + g;
  ok = ok && blk < nblk;
  const uint16_t* p = xrow + (ok ? blk : 0) * 32;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p + f * 8);
    b.v[f] = ok ? v : u32x4_t{0, 0, 0, 0};
  }
  return b;
}


// ------------------------------------------------------------- gate/up --

// One work-group: 16 intermediate rows (gate and up) of one expert slot, for
// the slot's token columns [c0, c0 + 16 * NCT); `red` is LDS for the
// cross-wave sums.  Returns whether the slot has columns past these (the
// caller then runs another pass after a barrier); every thread returns the
// same value.
// PRO: the routing of routed slots comes from the work-group's own selection
// in LDS (`R`, tile_m 1) instead of the tables in memory.
// XS: the activations come from fp16 rows staged in LDS at `xs` ([T, K],
// Q4_0 / Q8_0 families, one column tile), and a wave issues the weight loads
// of up to 4 steps at once.
template <int WT, int XT, int NCT, bool COH, bool PRO = false, bool XS = false>
__device__ __forceinline__ bool gateup_item(const DecodeArgs a, int rt, int slot, f32x4_t (*red)[2 * NCT][64],
                                            int c0 = 0, const SmallRoute* R = nullptr,
                                            const uint16_t* xs = nullptr) {
  static_assert(!XS || (Fam<WT>::v == DT_Q4 && NCT == 1), "staged activations: fp16-operand families, one tile");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool routed = slot < a.n_routed_slots;
  // the matrices of the slot's family: selects on a uniform flag (a branch per field lets the
  // compiler turn the pointers into a private lookup table)
  const uint8_t* bg = routed ? a.wg : a.sg;
  const uint8_t* bu = routed ? a.wu : a.su;
  const int N = routed ? a.I : a.Is;
  long n_mat = routed ? a.E : a.S;
  int e, ew, n_e, hrow0, seg = 0;     // ew: the matrix of expert e in its stacks
  if (routed) {
    if constexpr (PRO) {
      if (slot >= R->s_na[0]) return false;
      e = R->s_e[slot];
      n_e = R->s_cnt[slot];
      seg = hrow0 = R->s_cpre[slot];
    } else {
      if (slot >= ld_i32<COH>(a.active)) return false;
      e = ld_i32<COH>(a.active + 1 + slot);
      n_e = ld_i32<COH>(a.counts + e);
      seg = ld_i32<COH>(a.offsets + e);
      hrow0 = ld_i32<COH>(a.cprefix + e);
    }
    const RoutedAt w = routed_at<COH>(a, e);    // an expert cache's slot, or the host stacks
    ew = w.idx;
    n_mat = w.n_mat;
    bg = w.host ? a.wg_h : bg;
    bu = w.host ? a.wu_h : bu;
  } else {
    e = ew = slot - a.n_routed_slots;
    n_e = a.T;
    hrow0 = a.T * a.k + e * a.T;
  }
  if (rt * 16 >= N) return false;
  constexpr int F = Fam<WT>::v;
  const int K = a.H, g = lane >> 4;
  RowPtr<WT> rg, ru;
  rg.init(bg, n_mat, N, K, ew, rt * 16 + (lane & 15));
  ru.init(bu, n_mat, N, K, ew, rt * 16 + (lane & 15));
  // fp8: the row scales of this lane's output rows, fetched early and applied to the sums
  f32x4_t sg_rows = {1.f, 1.f, 1.f, 1.f}, su_rows = {1.f, 1.f, 1.f, 1.f};
  if constexpr (WT == DT_FP8) {
    if (wave == 0) {
      sg_rows = fp8_row_scales(bg, n_mat, N, K, ew, rt * 16 + (lane >> 4) * 4);
      su_rows = fp8_row_scales(bu, n_mat, N, K, ew, rt * 16 + (lane >> 4) * 4);
    }
  }

  constexpr int xb = XT == DT_F32 ? 4 : 2;
  const uint8_t* xrow[NCT];
  bool xok[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int c = c0 + ct * 16 + (lane & 15);
    xok[ct] = c < n_e;
    int tok = 0;
    if (xok[ct]) {
      if constexpr (PRO) tok = routed ? R->sorted[seg + c] / a.k : c;
      else tok = routed ? ld_i32<COH>(a.sorted_ids + seg + c) / a.k : c;
    }
    xrow[ct] = XS ? reinterpret_cast<const uint8_t*>(xs + size_t(tok) * K)
                  : reinterpret_cast<const uint8_t*>(a.x) + size_t(tok) * K * xb;
  }
  const int nct = (n_e - c0 + 15) >> 4;

  const int nsteps = n_steps<WT>(K);
  const int s0 = wave * nsteps / 4, s1 = (wave + 1) * nsteps / 4;
  f32x4_t accg[NCT], accu[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) accg[ct] = accu[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int U = XS ? 4 : Unroll<WT, NCT>::v;
  auto load = [&](int s) {
    GUStep<WT, XT, NCT> st;
    st.g = load_a<WT>(rg, s, g, K);
    st.u = load_a<WT>(ru, s, g, K);
    if constexpr (!XS) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        if (NCT == 1 || ct < nct) {
          if (!MOE_GU_MASKED_B || xok[ct]) st.x[ct] = load_x_raw<F, XT>(xrow[ct], s, g, K);
        }
    }
    return st;
  };
  auto body = [&](int s, const GUStep<WT, XT, NCT>& st) {
    const AReady<F> ag = prep_a<WT>(st.g), au = prep_a<WT>(st.u);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (NCT == 1 || ct < nct) {
        XFrag<F, XT> b;
        if constexpr (XS) {
          const XFrag<DT_Q4, DT_F32> bl = lds_x_frag(reinterpret_cast<const uint16_t*>(xrow[ct]), xok[ct], s, g, K);
#pragma unroll
          for (int f = 0; f < 4; ++f) b.v[f] = bl.v[f];
        } else {
          b = cook_x<F, XT>(st.x[ct], xok[ct], s, g, K);
        }
        accg[ct] = mma_ready<F, XT>(ag, b, accg[ct]);
        accu[ct] = mma_ready<F, XT>(au, b, accu[ct]);
      }
    }
  };
  stream_steps<U>(s0, s1, load, body);

#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    red[wave][ct][lane] = accg[ct];
    red[wave][NCT + ct][lane] = accu[ct];
  }
  __syncthreads();
  const bool more = c0 + 16 * NCT < n_e;
  if (wave != 0) return more;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    if (!(NCT == 1 || ct < nct)) continue;
    f32x4_t gs = red[0][ct][lane], us = red[0][NCT + ct][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      gs += red[w][ct][lane];
      us += red[w][NCT + ct][lane];
    }
    const int c = c0 + ct * 16 + (lane & 15);
    if (c >= n_e) continue;
    float wr = 1.0f;
    if constexpr (PRO) {
      if (routed) wr = R->wts[R->sorted[seg + c]];
    } else {
      if (routed) wr = ld_f32<COH>(a.topk_w + ld_i32<COH>(a.sorted_ids + seg + c));
    }
    float hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu_f(gs[i] * sg_rows[i]) * (us[i] * su_rows[i]) * wr;
    const size_t off = size_t(hrow0 + c) * a.h_stride + rt * 16 + (lane >> 4) * 4;
    if constexpr (F == DT_F32) {
      st_f32x4<COH>(reinterpret_cast<float*>(a.h) + off, f32x4_t{hv[0], hv[1], hv[2], hv[3]});
    } else if constexpr (F == DT_BF16) {
      uint32_t h0 = f32_to_bf16(hv[0]), h1 = f32_to_bf16(hv[1]), h2 = f32_to_bf16(hv[2]), h3 = f32_to_bf16(hv[3]);
      float r0 = hv[0] - __uint_as_float(h0 << 16), r1 = hv[1] - __uint_as_float(h1 << 16);
      float r2 = hv[2] - __uint_as_float(h2 << 16), r3 = hv[3] - __uint_as_float(h3 << 16);
      uint16_t* hp = reinterpret_cast<uint16_t*>(a.h);
      st_u32x2<COH>(hp + off, u32x2_t{h0 | (h1 << 16), h2 | (h3 << 16)});
      st_u32x2<COH>(hp + a.h_plane + off, u32x2_t{pack_bf16(r0, r1), pack_bf16(r2, r3)});
    } else {
      uint16_t* hp = reinterpret_cast<uint16_t*>(a.h);
      st_u32x2<COH>(hp + off, u32x2_t{pack_f16(hv[0], hv[1]), pack_f16(hv[2], hv[3])});
    }
  }
  return more;
}

// ---------------------------------------------------------------- down --

// B operand of the down projection: activation rows written by gate/up, in
// the format of the weight family (fp32; bf16 hi + lo planes; fp16 for the
// Q4_0 / Q8_0 and the fp8 families).
template <int F> struct HFrag;
template <> struct HFrag<DT_F32> { float v[4]; };
template <> struct HFrag<DT_BF16> { u32x4_t hi, lo; };
template <> struct HFrag<DT_Q4> { u32x4_t v[4]; };
template <> struct HFrag<DT_FP8> { u32x4_t v[2]; };

__device__ __forceinline__ HFrag<DT_BF16> load_h8(const void* h, long h_plane, size_t row_off, int k0) {
  const uint16_t* hp = reinterpret_cast<const uint16_t*>(h) + row_off + k0;
  return HFrag<DT_BF16>{ldg16(hp), ldg16(hp + h_plane)};
}

template <int F>
__device__ __forceinline__ HFrag<F> load_h_raw(const DecodeArgs a, size_t row_off, int s, int g, int K) {
  HFrag<F> b;
  if constexpr (F == DT_F32) {
    const u32x4_t t = ldg16(reinterpret_cast<const float*>(a.h) + row_off + s * 16 + g * 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) b.v[m] = __uint_as_float(t[m]);
  } else if constexpr (F == DT_BF16) {
    b = load_h8(a.h, a.h_plane, row_off, s * 32 + g * 8);
  } else if constexpr (F == DT_FP8) {
    int k0 = s * 64 + g * 16;
    k0 = k0 < K ? k0 : K - 16;
    const uint16_t* hp = reinterpret_cast<const uint16_t*>(a.h) + row_off + k0;
    b.v[0] = ldg16(hp);
    b.v[1] = ldg16(hp + 8);
  } else {
    const int nblk = K / 32;
    int blk = 4 * s + g;
    blk = blk < nblk ? blk : nblk - 1;
    const uint16_t* hp = reinterpret_cast<const uint16_t*>(a.h) + row_off + blk * 32;
#pragma unroll
    for (int f = 0; f < 4; ++f) b.v[f] = ldg16(hp + f * 8);
  }
  return b;
}

template <int F>
__device__ __forceinline__ HFrag<F> cook_h(HFrag<F> b, bool ok, int s, int g, int K) {
  const u32x4_t z = {0, 0, 0, 0};
  if constexpr (F == DT_F32) {
#pragma unroll
    for (int m = 0; m < 4; ++m) b.v[m] = ok ? b.v[m] : 0.f;
  } else if constexpr (F == DT_BF16) {
    b.hi = ok ? b.hi : z;
    b.lo = ok ? b.lo : z;
  } else if constexpr (F == DT_FP8) {
    ok = ok && s * 64 + g * 16 < K;
    b.v[0] = ok ? b.v[0] : z;
    b.v[1] = ok ? b.v[1] : z;
  } else {
    ok = ok && (4 * s + g) < K / 32;
#pragma unroll
    for (int f = 0; f < 4; ++f) b.v[f] = ok ? b.v[f] : z;
  }
  return b;
}

template <int F>
__device__ __forceinline__ f32x4_t mma_h(const AReady<F>& a, const HFrag<F>& b, f32x4_t c) {
  if constexpr (F == DT_F32) {
#pragma unroll
    for (int m = 0; m < 4; ++m) c = mfma_f32(__uint_as_float(a.v[m]), b.v[m], c);
  } else if constexpr (F == DT_BF16) {
    c = mfma_bf16(a.v, b.hi, c);
    c = mfma_bf16(a.v, b.lo, c);
  } else if constexpr (F == DT_FP8) {
    c = mfma_f16(a.v[0], b.v[0], c);
    c = mfma_f16(a.v[1], b.v[1], c);
  } else {
#pragma unroll
    for (int f = 0; f < 4; ++f) c = mfma_f16(a.fr[f], b.v[f], c);
  }
  return c;
}

template <int WT, int NCT, int RPW>
struct DNStep { AFrag<WT> a[RPW]; HFrag<Fam<WT>::v> h[NCT]; };

// One work-group: RPW x 16 hidden outputs (rows of the down projection) of
// one expert slot, for the slot's token columns [c0, c0 + 16 * NCT) (returns
// whether more follow, as gateup_item), over k range kr of ks: the steps of
// the reduction over the slot's intermediate dimension are cut into ks equal
// ranges, and this work-group's partial rows go to plane kr of `partials`.
// Its 4 waves split the range; partial sums meet in LDS.  A wave's RPW row
// tiles share each activation fragment it loads, which cuts the activation
// loads per weight byte by RPW (they otherwise add a fifth of the weight
// stream's load instructions).  The result rows are the routing-weighted
// expert outputs; they go to `partials` at the same row the activations use
// (one row per routed assignment, then the shared tokens).  `red` holds
// [4 waves][RPW * NCT][64] accumulators.
// CST: the partial rows are stored with device-scope stores (read by another
// work-group of the same launch); COH implies it.
template <int WT, int NCT, bool COH, int RPW = 1, bool CST = COH, int NW = 4>
__device__ __forceinline__ bool down_item(const DecodeArgs a, int rt, int slot, f32x4_t (*red)[RPW * NCT][64],
                                          int c0 = 0, int kr = 0, int ks = 1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool routed = slot < a.n_routed_slots;
  const uint8_t* base = routed ? a.wd : a.sd;     // selects, as in gateup_item
  const int K = routed ? a.I : a.Is;
  long n_mat = routed ? a.E : a.S;
  int e, ew, n_e, hrow0;              // ew: the matrix of expert e in its stacks
  if (routed) {
    if (slot >= ld_i32<COH>(a.active)) return false;
    e = ld_i32<COH>(a.active + 1 + slot);
    n_e = ld_i32<COH>(a.counts + e);
    hrow0 = ld_i32<COH>(a.cprefix + e);
    const RoutedAt w = routed_at<COH>(a, e);    // an expert cache's slot, or the host stacks
    ew = w.idx;
    n_mat = w.n_mat;
    base = w.host ? a.wd_h : base;
  } else {
    e = ew = slot - a.n_routed_slots;
    n_e = a.T;
    hrow0 = a.T * a.k + e * a.T;
  }
  constexpr int F = Fam<WT>::v;
  const int H = a.H, g = lane >> 4;
  const int row0 = rt * RPW * 16;               // first output row of this work-group
  RowPtr<WT> rw[RPW];
  f32x4_t sd_rows[RPW];                         // fp8: row scales of this lane's output rows
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    rw[r].init(base, n_mat, H, K, ew, row0 + r * 16 + (lane & 15));
    sd_rows[r] = f32x4_t{1.f, 1.f, 1.f, 1.f};
    if constexpr (WT == DT_FP8) {
      if (wave == 0) sd_rows[r] = fp8_row_scales(base, n_mat, H, K, ew, row0 + r * 16 + (lane >> 4) * 4);
    }
  }
  size_t hoff[NCT];
  bool hok[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int c = c0 + ct * 16 + (lane & 15);
    hok[ct] = c < n_e;
    hoff[ct] = size_t(hrow0 + (hok[ct] ? c : 0)) * a.h_stride;
  }
  const int nct = (n_e - c0 + 15) >> 4;
  const int nsteps = n_steps<WT>(K);
  const int kb = kr * nsteps / ks, ke = (kr + 1) * nsteps / ks;
  const int s0 = kb + wave * (ke - kb) / NW, s1 = kb + (wave + 1) * (ke - kb) / NW;
  f32x4_t acc[RPW][NCT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[r][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int U = UnrollDown<WT, NCT>::v;
  auto load = [&](int s) {
    DNStep<WT, NCT, RPW> st;
#pragma unroll
    for (int r = 0; r < RPW; ++r) st.a[r] = load_a<WT>(rw[r], s, g, K);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      if (NCT == 1 || ct < nct) {
        if (!MOE_DN_MASKED_B || hok[ct]) st.h[ct] = load_h_raw<F>(a, hoff[ct], s, g, K);
      }
    return st;
  };
  auto body = [&](int s, const DNStep<WT, NCT, RPW>& st) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (NCT == 1 || ct < nct) {
        const auto hc = cook_h<F>(st.h[ct], hok[ct], s, g, K);
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[r][ct] = mma_h<F>(prep_a<WT>(st.a[r]), hc, acc[r][ct]);
      }
    }
  };
  stream_steps<U>(s0, s1, load, body);

#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) red[wave][r * NCT + ct][lane] = acc[r][ct];
  __syncthreads();
  const bool more = c0 + 16 * NCT < n_e;
  if (wave != 0) return more;
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (!(NCT == 1 || ct < nct)) continue;
      f32x4_t v = red[0][r * NCT + ct][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += red[w][r * NCT + ct][lane];
      const int c = c0 + ct * 16 + (lane & 15);
      if (c >= n_e) continue;
      // lane holds rows 4*(lane/16) + 0..3 of row tile r for token column c
      st_f32x4<COH || CST>(a.partials + size_t(kr) * a.part_plane + size_t(hrow0 + c) * H + row0 + r * 16 +
                               (lane >> 4) * 4, v * sd_rows[r]);
    }
  return more;
}

// One output row of one expert slot: the sum of its k-range planes in order.
template <bool COH>
__device__ __forceinline__ f32x4_t partial_row(const DecodeArgs& a, size_t row, int h) {
  const float* p = a.partials + row * a.H + h;
  f32x4_t r = ld_f32x4<COH>(p);
  for (int q = 1; q < a.dn_ksplit; ++q) r += ld_f32x4<COH>(p + size_t(q) * a.part_plane);
  return r;
}

// ------------------------------------------------------ down, one token --
// A batch of one token: its k routed experts are distinct, so its activation
// rows are rows 0 .. k-1 (expert order) followed by the S shared rows, one
// per slot.  One work-group covers 16 output rows for every slot and adds the
// slots itself -- no partial rows, no arrival counter, no second round trip
// for a combine.  The activation rows are staged into LDS (every plane of the
// family's format); each wave issues the weight loads of all its (slot, step)
// pairs at once (at most kDownOneLoads), then multiplies them into one
// accumulator in slot order, and the waves are added in order (deterministic).
// Needs every slot to share one K (no shared experts, or I_shared == I).
constexpr int kDownOneLoads = 16;

template <int WT> constexpr int h_elem_bytes() { return Fam<WT>::v == DT_F32 ? 4 : 2; }
template <int WT> constexpr int h_planes() { return Fam<WT>::v == DT_BF16 ? 2 : 1; }

// B fragment of step s from the staged activations (layout as load_h_raw's,
// planes plane_bytes apart).
template <int F>
__device__ __forceinline__ HFrag<F> lds_h_frag(const uint8_t* hs, size_t plane_bytes, size_t row_off, int s, int g,
                                               int K) {
  HFrag<F> b;
  if constexpr (F == DT_F32) {
    const u32x4_t t = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const float*>(hs) + row_off + s * 16 + g * 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) b.v[m] = __uint_as_float(t[m]);
  } else if constexpr (F == DT_BF16) {
    const uint16_t* hp = reinterpret_cast<const uint16_t*>(hs) + row_off + s * 32 + g * 8;
    b.hi = *reinterpret_cast<const u32x4_t*>(hp);
    b.lo = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(hp) + plane_bytes);
  } else {
    static_assert(F == DT_Q4, "fp8 rows take per-slot scales");
    const int nblk = K / 32;
    int blk = 4 * s + g;
    blk = blk < nblk ? blk : nblk - 1;
    const uint16_t* hp = reinterpret_cast<const uint16_t*>(hs) + row_off + blk * 32;
#pragma unroll
    for (int f = 0; f < 4; ++f) b.v[f] = *reinterpret_cast<const u32x4_t*>(hp + f * 8);
  }
  return b;
}

template <int WT, int OT>
__device__ __forceinline__ void down_one_item(const DecodeArgs a, int rt, uint8_t* hs, f32x4_t (*red)[64]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4;
  constexpr int F = Fam<WT>::v;
  constexpr int EB = h_elem_bytes<WT>(), NP = h_planes<WT>();
  const int K = a.I, H = a.H;
  const int n_slots = a.k + a.S;
  // every routed slot's expert and activation row, one per lane (a vector
  // load each, in bounds for any slot count): slot j < k is the j-th active
  // expert, whose row is its prefix count; slot k + s is the shared expert s,
  // row k + s.  Lanes are read back with readlane (uniform slot index).
  const int A = ld_i32<false>(a.active);
  const int jl = lane < a.k ? lane : a.k - 1;
  int el = ld_i32<false>(a.active + 1 + jl);
  el = el < 0 ? 0 : (el >= a.E ? a.E - 1 : el);   // entries past A are stale
  const int hl = ld_i32<false>(a.cprefix + el);
  const int sl = a.slot_of ? ld_i32<false>(a.slot_of + el) : el;   // an expert cache's slot (-1: host stacks)
  // this wave's steps of every slot, all loads in flight at once
  const int nsteps = n_steps<WT>(K);
  const int s0 = wave * nsteps / 4, len = (wave + 1) * nsteps / 4 - s0;
  const int n_pairs = n_slots * len;
  AFrag<WT> af[kDownOneLoads];
#pragma unroll
  for (int i = 0; i < kDownOneLoads; ++i) {
    if (i < n_pairs) {
      const int j = i / len, st = s0 + i % len;
      const bool routed = j < a.k;
      if (routed && j >= A) continue;
      const int ej = __builtin_amdgcn_readlane(el, j), sj = __builtin_amdgcn_readlane(sl, j);
      const bool host = a.slot_of && sj < 0, cached = a.slot_of && sj >= 0;
      RowPtr<WT> rw;
      rw.init(routed ? (host ? a.wd_h : a.wd) : a.sd, routed ? (cached ? long(a.E_w) : long(a.E)) : long(a.S), H, K,
              routed ? (cached ? sj : ej) : j - a.k, rt * 16 + (lane & 15));
      af[i] = load_a<WT>(rw, st, g, K);
    }
  }
  // then stage every plane of rows [0, k + S) of the activations, four
  // 16-byte chunks per thread in flight
  const size_t plane_bytes = size_t(n_slots) * a.h_stride * EB;
  const int n16 = int(plane_bytes / 16), tot16 = n16 * NP;
  constexpr int kChunks = 4;
  for (int base = 0; base < tot16; base += 256 * kChunks) {
    u32x4_t v[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int idx = base + c * 256 + tid, p = idx >= n16, i = idx - p * n16;
      if (idx < tot16) v[c] = ldg16(reinterpret_cast<const uint8_t*>(a.h) + (size_t(p) * a.h_plane * EB + size_t(i) * 16));
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int idx = base + c * 256 + tid;
      if (idx < tot16) *reinterpret_cast<u32x4_t*>(hs + size_t(idx) * 16) = v[c];
    }
  }
  __syncthreads();                               // staged activations visible
  const bool hok = (lane & 15) == 0;             // the token is column 0
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kDownOneLoads; ++i) {
    if (i < n_pairs) {
      const int j = i / len, st = s0 + i % len;
      if (j < a.k && j >= A) continue;
      const int hrow = j < a.k ? __builtin_amdgcn_readlane(hl, j) : j;
      const auto hr = lds_h_frag<F>(hs, plane_bytes, size_t(hrow) * a.h_stride, st, g, K);
      acc = mma_h<F>(prep_a<WT>(af[i]), cook_h<F>(hr, hok, st, g, K), acc);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4_t v = red[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) v += red[w][lane];
  if (!hok) return;
  const long o = (long(rt) * 16 + g * 4) / 4;   // this lane's four outputs of the one token
  if constexpr (OT == DT_F32) reinterpret_cast<f32x4_t*>(a.out)[o] = v;
  else reinterpret_cast<u32x2_t*>(a.out)[o] = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}

// out[t] = sum over j of the partial row of assignment t*k + j (found through
// inv), then the shared experts' rows, in that fixed order; 4 outputs per thread.
template <int OT, bool COH>
__device__ __forceinline__ void combine_item(const DecodeArgs a, long i4) {
  const int H4 = a.H / 4;
  if (i4 >= long(a.T) * H4) return;
  const int t = int(i4 / H4), h4 = int(i4 % H4);
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < a.k; j0 += 8) {     // the rows of 8 assignments located first, then added in order
    int row[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) row[u] = j0 + u < a.k ? ld_i32<COH>(a.inv + t * a.k + j0 + u) : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < a.k) v += partial_row<false>(a, size_t(row[u]), 4 * h4);
  }
  for (int s = 0; s < a.S; ++s) v += partial_row<false>(a, size_t(a.T * a.k + s * a.T + t), 4 * h4);
  if constexpr (OT == DT_F32) reinterpret_cast<f32x4_t*>(a.out)[i4] = v;
  else reinterpret_cast<u32x2_t*>(a.out)[i4] = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}

// Combine epilogue of the down projection.  The work-groups writing partial
// rows into output row group rt (`rows` outputs wide) are the A active
// routed slots and the S shared ones; each counts in once its device-scope
// stores of the partials have completed, and the last to count in sums, for
// every token, the k routed rows and the S shared rows in the order of
// combine_item (same bits) and writes the outputs.  The rows are read with
// device-scope loads: with 16-output row groups two groups share a 128-byte
// line, and the last work-group of the neighbouring group may already have
// pulled that line into this XCD's L2 before this group's writers finished.
// dn_count[rt] is zeroed by the router launch of the same pass.
template <int OT>
__device__ __forceinline__ void down_combine(const DecodeArgs a, int rt, int slot, int rows) {
  __shared__ int last;
  const int tid = threadIdx.x;
  const int A = ld_i32<false>(a.active);                    // written by an earlier launch
  if (slot < a.n_routed_slots && slot >= A) return;          // this work-group wrote nothing
  if (tid < 64) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // wave 0 stored the partials
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(a.dn_count + rt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           unsigned((A + a.S) * a.dn_ksplit - 1);
  __syncthreads();
  if (!last) return;
  const int H = a.H, r4 = rows / 4;
  for (int i = tid; i < a.T * r4; i += blockDim.x) {
    const int t = i / r4, h = rt * rows + 4 * (i - t * r4);
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.k; ++j) v += partial_row<true>(a, size_t(a.inv[t * a.k + j]), h);
    for (int s = 0; s < a.S; ++s) v += partial_row<true>(a, size_t(a.T * a.k + s * a.T + t), h);
    const long o = (long(t) * H + h) / 4;
    if constexpr (OT == DT_F32) reinterpret_cast<f32x4_t*>(a.out)[o] = v;
    else reinterpret_cast<u32x2_t*>(a.out)[o] = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  }
}

}  // namespace moe
