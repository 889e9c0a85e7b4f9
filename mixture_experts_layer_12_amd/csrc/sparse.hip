// Budgeted top-c channel-sparse routed experts (decode, small batches).
//
// Source: "KAIST removed calibration from MoE decoding and sped up blocks up
// to 2.69x over vLLM" (news.hamidun.com), sections "A threshold promises a
// budget but does not keep it" and "Top-k instead of a threshold": per token
// only a fixed number c of each engaged expert's intermediate channels is
// read -- the c with the highest selector scores -- so the bytes read per
// token are known in advance.  Given the kept set the expert FFN runs on those
// channels only: rows of the gate and up matrices and columns of the down
// matrix.  The down matrix is taken transposed ([E, I, H]), so that one kept
// channel is one contiguous row of H values.  Shared experts stay dense.
//
// Launches of one pass (T <= 64 tokens): router (+ dispatch), channel
// selection, sparse gate/up and the shared experts' gate/up, sparse down and
// the shared experts' down, combine.  When the router is one work-group
// (E <= 16 experts, T <= 16 tokens) the selection runs in the router's
// launch, for every (token, expert): it needs only the scores, so it no
// longer waits for the routing, and the engaged rows are picked through
// topk_ids afterwards (E / k times the selection work, all in parallel).
//
//   select:  one work-group of 16 waves per (token, engaged expert).  Scores
//            become order-preserving 32-bit keys in LDS; a radix select over 4
//            bytes (per-wave histograms, one update per distinct byte per wave)
//            finds the c-th largest key, then a stable compaction in index
//            order keeps the keys above it and the first equal ones.
//   gate/up: the decode gate/up operand code with gathered rows: a work-group
//            takes 16 kept channels (A rows) against the one token (B column),
//            its 8 waves split H, and writes silu(g) * u * (routing weight).
//   down:    y = sum over kept channels q of h_q * WdT[q, :].  Each lane owns 8
//            consecutive outputs (one 16-byte row slice per channel), a wave
//            512, a work-group 2048; the kept channels are split R ways over
//            work-groups, and the R partial rows are summed in a fixed order
//            by the combine.  Plain FMAs: the work is a weighted sum of rows.
#include "decode_items.hpp"

namespace moe {


// ------------------------------------------------------------- select ----

// Order-preserving key of a score: larger score, larger key; -0 and +0 are
// one value; NaN is below every number.
__device__ __forceinline__ uint32_t score_key(float v) {
  if (v != v) return 0u;
  if (v == 0.f) v = 0.f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelWaves = 16;

// Exclusive prefix sum over the threads of the work-group (in thread order).
__device__ __forceinline__ int wg_exclusive_scan(int v, int* lds_nw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) lds_nw[wave] = incl;
  __syncthreads();
  // the totals of the waves before this one: one read per lane, then a
  // reduction over the first 16 lanes (integer sums: order does not matter)
  int base = lane < wave ? lds_nw[lane] : 0;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) base += __shfl_xor(base, d);
  base = __shfl(base, 0);
  __syncthreads();
  return base + incl - v;
}

// Radix digits of the selection: 11, 11 and 10 bits from the top of the key.
__host__ __device__ constexpr int sel_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__host__ __device__ constexpr int sel_bits(int pass) { return pass == 2 ? 10 : 11; }
constexpr int kSelBins = 2048;
static_assert(kSelBins <= 2 * kSelWaves * 64 && (1 << 10) >= kSelWaves * 64, "two bins or one per thread");

// One work-group of 16 waves per (token, engaged expert): an exact radix
// select of the c-th largest key in three passes (11, 11, 10 bits), each a
// histogram of the keys that match the digits chosen so far, counted with LDS
// atomics (a wave's lanes rarely share a bin once 11 bits are used), then one
// ordered compaction.  Keys stay in LDS.
// Channels of token t, expert e into `out` (c ints); `keys` is LDS of
// sparse_select_lds_bytes(I) bytes.
__device__ __forceinline__ void select_channels(const SparseArgs& a, int t, int e, int32_t* out, uint32_t* keys) {
  const int tid = threadIdx.x;
  constexpr int NT = kSelWaves * 64;
  const int I = a.d.I, c = a.c;
  const float* s = a.scores + (size_t(t) * a.d.E + e) * I;
  uint32_t* hist = keys + I;
  int* misc = reinterpret_cast<int*>(hist + kSelBins);   // [0] bin, [1] remaining, [4..20) scan scratch
  {
    // all score loads first (I <= 16 * NT), so their latencies overlap
    static_assert(16 * NT >= 16384, "one batch of loads covers the largest I");
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = tid + u * NT;
      v[u] = i < I ? s[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = tid + u * NT;
      if (i < I) keys[i] = score_key(v[u]);
    }
  }
  uint32_t prefix = 0, pmask = 0;
  int remaining = c;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = sel_shift(pass), nb = 1 << sel_bits(pass);
    for (int i = tid; i < kSelBins; i += NT) hist[i] = 0;
    __syncthreads();
    uint32_t kv[16];              // all reads of the pass first, then the counts
#pragma unroll
    for (int u = 0; u < 16; ++u) kv[u] = tid + u * NT < I ? keys[tid + u * NT] : 0u;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (tid + u * NT < I && (kv[u] & pmask) == prefix) atomicAdd(&hist[(kv[u] >> shift) & uint32_t(nb - 1)], 1u);
    __syncthreads();
    {
      // thread t holds bins nb-1-per*t .. nb-per*(t+1) (highest first); a
      // work-group scan in thread order counts the keys in higher bins
      const int per = nb / NT;
      uint32_t cnt[2] = {0u, 0u}, sum = 0;
#pragma unroll
      for (int m = 0; m < 2; ++m)
        if (m < per) { cnt[m] = hist[nb - 1 - per * tid - m]; sum += cnt[m]; }
      uint32_t before = uint32_t(wg_exclusive_scan(int(sum), misc + 4));
      if (before < uint32_t(remaining) && before + sum >= uint32_t(remaining)) {
        const int m = before + cnt[0] >= uint32_t(remaining) ? 0 : 1;
        misc[0] = nb - 1 - per * tid - m;
        misc[1] = remaining - int(before + (m ? cnt[0] : 0u));
      }
    }
    __syncthreads();
    prefix |= uint32_t(misc[0]) << shift;
    pmask |= uint32_t(nb - 1) << shift;
    remaining = misc[1];
    __syncthreads();
  }
  // prefix is now the c-th largest key; keep every larger key and the first
  // `remaining` equal ones in index order.  Thread tid owns a contiguous chunk.
  const int ch = (I + NT - 1) / NT;     // at most 16
  const int i0 = min(I, tid * ch), i1 = min(I, i0 + ch);
  uint32_t kc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) kc[j] = i0 + j < i1 ? keys[i0 + j] : 0u;
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    n_gt += i0 + j < i1 && kc[j] > prefix;
    n_eq += i0 + j < i1 && kc[j] == prefix;
  }
  const int eq_base = wg_exclusive_scan(n_eq, misc + 4);
  const int take_eq = min(max(remaining - eq_base, 0), n_eq);
  int pos = wg_exclusive_scan(n_gt + take_eq, misc + 4);
  int eq_seen = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (i0 + j >= i1) break;
    const uint32_t kk = kc[j];
    bool keep = kk > prefix;
    if (kk == prefix) keep = eq_seen++ < take_eq;
    if (keep && pos < c) out[pos++] = i0 + j;      // exactly c are kept; the bound only guards the buffer
  }
}

__global__ void __launch_bounds__(kSelWaves * 64) sparse_select_kernel(SparseArgs a) {
  extern __shared__ uint32_t keys[];                 // [I], then hist [2048], then scratch
  const int f = blockIdx.x;
  select_channels(a, f / a.d.k, a.topk_ids[f], a.sel + size_t(f) * a.c, keys);
}

// Router and channel selection in one launch, for a single-work-group
// router: work-group 0 routes (logits, top-k, dispatch, as the router's
// fused kernel), work-groups 1 .. T*E select the channels of every
// (token, expert), which needs only the scores; the selection no longer
// waits for the routing.  The engaged experts' rows are picked up later
// through topk_ids.
template <int RT, int XT, int MODE>
__global__ void __launch_bounds__(kSelWaves * 64) sparse_route_select_kernel(RouterArgs ra, SparseArgs a) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  if (blockIdx.x == 0) {
    __shared__ float lg[256];
    logits_tile<RT, XT, false, 1>(ra, 0, 0, 0, kLogitChunks, reinterpret_cast<float*>(lds), lg);
    __syncthreads();
    select_and_dispatch<false, MODE>(ra, lg, true, lds);
    return;
  }
  const int f = blockIdx.x - 1;
  select_channels(a, f / a.d.E, f % a.d.E, a.sel + size_t(f) * a.c, reinterpret_cast<uint32_t*>(lds));
}

// Row of `sel` with the kept channels of assignment f.
__device__ __forceinline__ size_t sel_row(const SparseArgs& a, int f) {
  return a.sel_all ? size_t(f / a.d.k) * a.d.E + a.topk_ids[f] : size_t(f);
}

// ------------------------------------------------------------- gate/up ---

constexpr int kGuWaves = 8;

template <int WT, int XT>
__global__ void __launch_bounds__(kGuWaves * 64) sparse_gateup_kernel(SparseArgs a) {
  __shared__ f32x4_t red[kGuWaves][2][64];
  const DecodeArgs d = a.d;
  constexpr int F = Fam<WT>::v;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;
  const int rt = blockIdx.x, f = blockIdx.y, c = a.c, K = d.H;
  const int t = f / d.k, e = a.topk_ids[f];
  const int r = rt * 16 + (lane & 15);
  const int chan = a.sel[sel_row(a, f) * c + (r < c ? r : c - 1)];     // past the end: a kept row, output dropped
  RowPtr<WT> rg, ru;
  rg.init(d.wg, d.E, d.I, K, e, chan);
  ru.init(d.wu, d.E, d.I, K, e, chan);
  constexpr int xb = XT == DT_F32 ? 4 : 2;
  const uint8_t* xrow = reinterpret_cast<const uint8_t*>(d.x) + size_t(t) * K * xb;
  const bool xok = (lane & 15) == 0;                                // one token: B column 0
  const int nsteps = n_steps<WT>(K);
  const int s0 = wave * nsteps / kGuWaves, s1 = (wave + 1) * nsteps / kGuWaves;
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = accg;
  auto load = [&](int s) {
    GUStep<WT, XT, 1> st;
    st.g = load_a<WT>(rg, s, g, K);
    st.u = load_a<WT>(ru, s, g, K);
    if (xok) st.x[0] = load_x_raw<F, XT>(xrow, s, g, K);
    return st;
  };
  auto body = [&](int s, const GUStep<WT, XT, 1>& st) {
    const AReady<F> ag = prep_a<WT>(st.g), au = prep_a<WT>(st.u);
    const XFrag<F, XT> b = cook_x<F, XT>(st.x[0], xok, s, g, K);
    accg = mma_ready<F, XT>(ag, b, accg);
    accu = mma_ready<F, XT>(au, b, accu);
  };
  stream_steps<Unroll<WT, 1>::v>(s0, s1, load, body);
  red[wave][0][lane] = accg;
  red[wave][1][lane] = accu;
  __syncthreads();
  if (wave != 0 || !xok) return;
  f32x4_t gs = red[0][0][lane], us = red[0][1][lane];
  for (int w = 1; w < kGuWaves; ++w) {
    gs += red[w][0][lane];
    us += red[w][1][lane];
  }
  const float wr = d.topk_w[f];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = rt * 16 + g * 4 + i;            // D rows of this lane: 4g .. 4g+3
    if (rr < c) a.hs[size_t(f) * c + rr] = silu_f(gs[i]) * us[i] * wr;
  }
}

// --------------------------------------------------------------- down ----

template <int WT>
__global__ void __launch_bounds__(256) sparse_down_kernel(SparseArgs a) {
  __shared__ int qsel[kSparseMaxRows];
  __shared__ float qh[kSparseMaxRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int f = blockIdx.z, r = blockIdx.y, c = a.c, H = a.d.H, I = a.d.I;
  const int e = a.topk_ids[f];
  const int q0 = int(long(r) * c / a.R), q1 = int(long(r + 1) * c / a.R);
  for (int q = q0 + threadIdx.x; q < q1; q += 256) {
    qsel[q - q0] = a.sel[sel_row(a, f) * c + q];
    qh[q - q0] = a.hs[size_t(f) * c + q];
  }
  __syncthreads();
  const int col = (blockIdx.x * 4 + wave) * 512 + lane * 8;
  if (col >= H) return;
  constexpr int eb = WT == DT_F32 ? 4 : 2;
  const uint8_t* base = a.wdt + (size_t(e) * I) * size_t(H) * eb + size_t(col) * eb;
  float acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = 0.f;
  constexpr int U = 8;
  for (int q = q0; q < q1; q += U) {
    u32x4_t w[U][eb / 2];
    float hv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = q + u < q1;
      const int qi = in ? q + u - q0 : 0;
      hv[u] = in ? qh[qi] : 0.f;
      const uint8_t* rowp = base + size_t(qsel[qi]) * H * eb;
#pragma unroll
      for (int p = 0; p < eb / 2; ++p) w[u][p] = ldg16(rowp + 16 * p);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (WT == DT_F32) {
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m] = fmaf(hv[u], __uint_as_float(w[u][m >> 2][m & 3]), acc[m]);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc[2 * m] = fmaf(hv[u], bf16_lo(w[u][0][m]), acc[2 * m]);
          acc[2 * m + 1] = fmaf(hv[u], bf16_hi(w[u][0][m]), acc[2 * m + 1]);
        }
      }
    }
  }
  float* dst = a.spart + (size_t(f) * a.R + r) * H + col;
  *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
  *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
}

// ------------------------------------------------------------ combine ----

// out[t]: the routed partial rows (all j, all splits r) and the shared
// experts' rows.  A work-group takes 32 column quads; its 8 row groups each sum
// a fixed share of the k*R partial rows with 8 loads in flight, and the group
// sums and the shared rows are added in a fixed order.
constexpr int kCmbCols = 32, kCmbGroups = 8;

template <int OT>
__global__ void __launch_bounds__(kCmbCols * kCmbGroups) sparse_combine_kernel(SparseArgs a) {
  __shared__ f32x4_t red[kCmbGroups][kCmbCols];
  const DecodeArgs d = a.d;
  const int H4 = d.H / 4;
  const int q = threadIdx.x % kCmbCols, grp = threadIdx.x / kCmbCols;
  const long i4 = long(blockIdx.x) * kCmbCols + q;
  const bool ok = i4 < long(d.T) * H4;
  const int t = ok ? int(i4 / H4) : 0, h4 = ok ? int(i4 % H4) : 0;
  const f32x4_t* sp = reinterpret_cast<const f32x4_t*>(a.spart);
  const int nrows = d.k * a.R;                                    // rows (j, r) of token t, j-major
  const int n0 = grp * nrows / kCmbGroups, n1 = (grp + 1) * nrows / kCmbGroups;
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  for (int n = n0; n < n1; n += 8) {
    f32x4_t b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      b[u] = (ok && n + u < n1) ? sp[(size_t(t) * nrows + n + u) * H4 + h4] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) v += b[u];
  }
  red[grp][q] = v;
  __syncthreads();
  if (grp != 0 || !ok) return;
  v = red[0][q];
  for (int g = 1; g < kCmbGroups; ++g) v += red[g][q];
  const f32x4_t* p = reinterpret_cast<const f32x4_t*>(d.partials);
  for (int s = 0; s < d.S; ++s) v += p[size_t(d.T * d.k + s * d.T + t) * H4 + h4];
  if constexpr (OT == DT_F32) reinterpret_cast<f32x4_t*>(d.out)[i4] = v;
  else reinterpret_cast<u32x2_t*>(d.out)[i4] = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}

// ------------------------------------------------------------- launch ----

hipError_t launch_decode_shared(const DecodeArgs& a, int wdt, int xdt, hipStream_t st);

size_t sparse_select_lds_bytes(int I) { return (size_t(I) + kSelBins + 4 + kSelWaves) * 4; }

size_t router_lds_bytes(int NW, int E, int n, bool stage);

template <int RT, int XT, int MODE>
static void launch_route_select_m(const RouterArgs& ra, const SparseArgs& a, hipStream_t st) {
  const size_t lds_max = std::max(router_lds_bytes(16, 16, 16 * 16, false), sparse_select_lds_bytes(16384));
  static const bool attr = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_route_select_kernel<RT, XT, MODE>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_max));
    return true;
  }();
  (void)attr;
  const size_t lds = std::max(router_lds_bytes(16, ra.E, ra.T * ra.k, false), sparse_select_lds_bytes(a.d.I));
  hipLaunchKernelGGL((sparse_route_select_kernel<RT, XT, MODE>), dim3(1 + a.d.T * a.d.E), dim3(kSelWaves * 64), lds,
                     st, ra, a);
}

template <int RT, int XT>
static void launch_route_select_t(const RouterArgs& ra, const SparseArgs& a, hipStream_t st) {
  const int mode = topk_mode(ra.E, ra.k);
  if (mode == kTopkT8) launch_route_select_m<RT, XT, kTopkT8>(ra, a, st);
  else if (mode == kTopkT16) launch_route_select_m<RT, XT, kTopkT16>(ra, a, st);
  else launch_route_select_m<RT, XT, kTopkRow16>(ra, a, st);
}

// The router of a single routing tile (E <= 16 experts, T <= 16 tokens) and
// the channel selection of every (token, expert) in one launch; a.sel_all
// must be set and a.sel must hold T*E rows.
hipError_t launch_sparse_route_select(const RouterArgs& ra, const SparseArgs& a, int rdt, int xdt, hipStream_t st) {
  if (!a.sel_all || ra.n_row_tiles * ra.n_col_tiles != 1 || ra.E > 16 || ra.T > 16) return hipErrorInvalidValue;
  if (rdt == DT_F32 && xdt == DT_F32) launch_route_select_t<DT_F32, DT_F32>(ra, a, st);
  else if (rdt == DT_F32) launch_route_select_t<DT_F32, DT_BF16>(ra, a, st);
  else if (xdt == DT_F32) launch_route_select_t<DT_BF16, DT_F32>(ra, a, st);
  else launch_route_select_t<DT_BF16, DT_BF16>(ra, a, st);
  return hipGetLastError();
}

// With a.sel_all the selection already ran (launch_sparse_route_select).
template <int WT, int XT>
static hipError_t launch_sparse_t(const SparseArgs& a, hipStream_t st, StageMarker* mark) {
  const int n = a.d.T * a.d.k;
  static const bool attr = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_select_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(sparse_select_lds_bytes(16384)));
    return true;
  }();
  (void)attr;
  if (!a.sel_all)
    hipLaunchKernelGGL(sparse_select_kernel, dim3(n), dim3(kSelWaves * 64), sparse_select_lds_bytes(a.d.I), st, a);
  if (mark) mark->mark(st);
  hipLaunchKernelGGL((sparse_gateup_kernel<WT, XT>), dim3((a.c + 15) / 16, n), dim3(kGuWaves * 64), 0, st, a);
  if (hipError_t e = launch_decode_shared(a.d, WT, XT, st)) return e;     // shared experts: dense
  if (mark) mark->mark(st);
  hipLaunchKernelGGL((sparse_down_kernel<WT>), dim3((a.d.H + 2047) / 2048, a.R, n), dim3(256), 0, st, a);
  const long n4 = long(a.d.T) * a.d.H / 4;
  hipLaunchKernelGGL((sparse_combine_kernel<XT>), dim3(int((n4 + kCmbCols - 1) / kCmbCols)),
                     dim3(kCmbCols * kCmbGroups), 0, st, a);
  if (mark) mark->mark(st);
  return hipGetLastError();
}

hipError_t launch_sparse(const SparseArgs& a, int wdt, int xdt, hipStream_t st, StageMarker* mark) {
  if (wdt == DT_F32) return xdt == DT_F32 ? launch_sparse_t<DT_F32, DT_F32>(a, st, mark)
                                          : launch_sparse_t<DT_F32, DT_BF16>(a, st, mark);
  if (wdt == DT_BF16) return xdt == DT_F32 ? launch_sparse_t<DT_BF16, DT_F32>(a, st, mark)
                                           : launch_sparse_t<DT_BF16, DT_BF16>(a, st, mark);
  return hipErrorInvalidValue;
}

}  // namespace moe
