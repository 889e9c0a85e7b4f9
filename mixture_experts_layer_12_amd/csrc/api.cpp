// C ABI of the MoE layer forward: argument validation, workspace layout, path
// choice and kernel launches.  Host code only; the kernels live in
// router.hip, decode.hip, decode_fused.hip and prefill.hip.  See include/moe.h
// for the contract.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdlib>
#include <random>

#include "common.hpp"

namespace moe {
hipError_t launch_router(const RouterArgs& a, int rdt, int xdt, int NW, hipStream_t st, bool logits_only = false);
hipError_t launch_decode(const DecodeArgs& a, int wdt, int xdt, int rdt, int n_gu_row_tiles, hipStream_t st,
                         StageMarker* mark);
hipError_t launch_prefill(const PrefillArgs& a, int out_dt, hipStream_t st, StageMarker* mark);
int prefill_k_split(int capacity, int S, int t_pad, int H, int nmax);
hipError_t launch_decode_fused(const FusedArgs& f, int wdt, int xdt, hipStream_t st);
hipError_t launch_sparse(const SparseArgs& a, int wdt, int xdt, hipStream_t st, StageMarker* mark);
hipError_t launch_sparse_route_select(const RouterArgs& ra, const SparseArgs& a, int rdt, int xdt, hipStream_t st);
}  // namespace moe

namespace {

#ifndef MOE_EPILOGUE_MAX_SLOTS
#define MOE_EPILOGUE_MAX_SLOTS 16
#endif
constexpr int kEpilogueMaxSlots = MOE_EPILOGUE_MAX_SLOTS;   // decode: expert slots per output row group for the combine epilogue
// decode: gate/up grids that select in their own prologue -- up to 1024
// work-groups, or up to 8192 with bf16 or fp32 weights when the selection is
// tiny (tokens * experts <= 128: the Mixtral-shaped batches of 1 and 8 gain
// 2.5-3 us per layer; with fp8 weights the batch of 8 loses 48 us, and a
// DeepSeek-shaped batch of 8 over 64 experts loses 12 us at 4400 work-groups)
constexpr long kRouteInGateUpMaxGroups = 1024;
constexpr long kRouteInGateUpMaxGroupsTiny = 8192;
constexpr long kTinySelection = 128;
constexpr int kTileM = 128;          // padding multiple of the expert-sorted order (moe_route, decode)
constexpr int kPrefillTileM = 256;   // padding multiple of the prefill path (its GEMM row tile)
constexpr int kDecodeMaxT = 64;      // tokens per decode pass
constexpr int kFusedMaxK = 16;       // top_k limit of the single-launch decode
constexpr int kHRowAlign = 64;       // decode activation rows padded to 64 elements (whole 128-byte lines)
constexpr size_t kAlign = 256;

size_t al(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }
long roundup(long n, long m) { return (n + m - 1) / m * m; }

struct Layout {
  int path;            // MOE_PATH_DECODE | MOE_PATH_PREFILL | MOE_PATH_DECODE_FUSED
  int Tr;              // tokens per routing pass
  int tile_m;          // padding multiple of the expert-sorted order
  int cap, n_tiles;    // sorted-order capacity and tiles for Tr tokens
  size_t logits, topk_ids, topk_w, counts, offsets, cprefix, active, sorted_ids, tile_expert, inv;
  size_t h, partials;
  int pf_ksplit;        // prefill: k ranges of the down GEMM (partial planes)
  size_t dn_count;     // multi-launch decode: down arrival counters [H / 16, rounded up to 4]
  size_t flags, error;  // single-launch decode: completion flags [n_items]; status pair (also the decode
                        // path's, for a selection inside the logits launch)
  size_t sel_flags;     // multi-launch decode: completion flags of the logit work-groups
  long n_items;
  long h_plane;
  int h_stride;
  int t_pad;
  size_t total;
};

// The prefill kernels address one weight matrix, x and the activation rows
// with 32-bit element offsets from a per-matrix base.
bool prefill_fits(const moe_shape_t* s) {
  const long n = std::max(s->I, s->n_shared > 0 ? s->I_shared : 0);
  const long rows = roundup(long(s->T) * s->top_k + long(s->E) * (kPrefillTileM - 1), kPrefillTileM) +
                    long(s->n_shared) * roundup(s->T, kPrefillTileM);   // activation rows
  return n * s->H < (1L << 31) && long(s->T) * s->H < (1L << 31) && rows * n < (1L << 31);
}

int check_shape(const moe_shape_t* s) {
  if (!s) return MOE_ERR_NULL;
  const long T = s->T, H = s->H, E = s->E, I = s->I, k = s->top_k, S = s->n_shared, Is = s->I_shared;
  if (T < 0 || T > 1048576) return MOE_ERR_SHAPE;
  if (H < 32 || H > 65536 || H % 32) return MOE_ERR_SHAPE;
  if (E < 1 || E > 256) return MOE_ERR_SHAPE;
  if (I < 32 || I > 1048576 || I % 32) return MOE_ERR_SHAPE;
  if (k < 1 || k > E || T * k > 16777216) return MOE_ERR_SHAPE;
  if (S < 0 || S > 16) return MOE_ERR_SHAPE;
  if (S > 0 && (Is < 32 || Is > 1048576 || Is % 32)) return MOE_ERR_SHAPE;
  if (s->x_dtype != MOE_F32 && s->x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (s->router_dtype != MOE_F32 && s->router_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (s->w_dtype < MOE_F32 || s->w_dtype > MOE_FP8_E4M3) return MOE_ERR_DTYPE;
  if (s->path < MOE_PATH_AUTO || s->path > MOE_PATH_DECODE_FUSED) return MOE_ERR_SHAPE;
  if (s->path == MOE_PATH_DECODE_FUSED && (s->router_dtype != s->x_dtype || s->w_dtype > MOE_Q4_0))
    return MOE_ERR_DTYPE;
  if (s->path == MOE_PATH_DECODE_FUSED && s->top_k > kFusedMaxK) return MOE_ERR_SHAPE;
  if (s->path == MOE_PATH_PREFILL && (s->x_dtype != MOE_BF16 || s->w_dtype != MOE_BF16)) return MOE_ERR_DTYPE;
  if (s->path == MOE_PATH_PREFILL && !prefill_fits(s)) return MOE_ERR_SHAPE;
  // index arithmetic of the largest buffers stays in 32-bit ranges
  if (roundup(T * k + E * (kPrefillTileM - 1), kPrefillTileM) + S * roundup(T, kPrefillTileM) > 2147483647L / 8)
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

int choose_path(const moe_shape_t* s) {
  if (s->path != MOE_PATH_AUTO) return s->path;
  if (s->x_dtype == MOE_BF16 && s->w_dtype == MOE_BF16 && s->T > kDecodeMaxT && prefill_fits(s))
    return MOE_PATH_PREFILL;
  // The single-launch decode is measured slower than the multi-launch kernels on every benchmarked
  // shape (its resident grid runs items one after another per work-group), so AUTO does not pick it.
  return MOE_PATH_DECODE;
}

// Work list of one single-launch decode pass of Tc tokens (see decode_fused.hip).
moe::FusedArgs fused_plan(const moe_shape_t* s, int Tc) {
  moe::FusedArgs f{};
  const int S = s->n_shared, Is = S > 0 ? s->I_shared : 0;
  const int n_slots = std::min(s->E, Tc * s->top_k);
  f.gu_rt_routed = s->I / 16;
  f.gu_rt_shared = Is / 16;
  f.n_logit = 4 * ((s->E + 15) / 16) * ((Tc + 15) / 16);   // 4 partial planes per tile
  f.end_shared_gu = f.n_logit + S * f.gu_rt_shared;
  // routing in the routed gate/up items: few assignments and few such items (each repeats it)
  f.route_in_gu = moe::small_route(Tc, s->E, s->top_k) && long(n_slots) * f.gu_rt_routed <= 512 ? 1 : 0;
  f.end_select = f.end_shared_gu + (f.route_in_gu ? 0 : 1);
  f.end_gu = f.end_select + n_slots * f.gu_rt_routed;
  f.end_down = f.end_gu + (n_slots + S) * (s->H / (Tc <= 16 ? moe::kFusedDownRows<1> : moe::kFusedDownRows<4>));
  f.n_items = f.end_down + int((long(Tc) * s->H / 4 + 255) / 256);
  return f;
}

// Completion tags of the single-launch decode: a process-wide counter started
// at a random 64-bit value, so that no tag matches leftover workspace contents.
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> ctr{[] {
    std::random_device rd;
    const unsigned long long t = uint64_t(std::chrono::steady_clock::now().time_since_epoch().count());
    return ((uint64_t(rd()) << 32) ^ uint64_t(rd()) ^ (t * 0x9E3779B97F4A7C15ull)) | 1ull;
  }()};
  return ctr.fetch_add(1, std::memory_order_relaxed) + 1;
}

// Polling rounds before a wait of the single-launch decode gives up (each
// round is one pass over up to 512 flags and a short sleep): about a second
// of waiting.  MOE_FUSED_WAIT_ROUNDS overrides it, read on every call, so
// that a test can force every wait to give up (0) and check that the failure
// is reported while every work-group still exits.
int fused_spin_rounds() {
  const char* v = std::getenv("MOE_FUSED_WAIT_ROUNDS");
  if (v && *v) {
    char* end = nullptr;
    const long r = std::strtol(v, &end, 10);
    if (end && *end == '\0' && r >= 0 && r <= (1L << 30)) return int(r);
  }
  return 1 << 21;
}

// MFMA steps of the decode kernels along a reduction of length K (one step =
// the K one 16-byte load per lane group covers), as n_steps in decode_items.hpp.
int decode_steps(int w_dtype, int K) {
  switch (w_dtype) {
    case MOE_F32: return K / 16;
    case MOE_BF16: return K / 32;
    case MOE_FP8_E4M3: return (K + 63) / 64;
    default: return (K / 32 + 3) / 4;     // Q4_0, Q8_0
  }
}

// Down-projection shape of a multi-launch decode pass of Tc tokens.
moe::DownShape pass_down_shape(const moe_shape_t* s, int Tc) {
  const int S = s->n_shared, Is = S > 0 ? s->I_shared : 0;
  const int n_slots = std::min(s->E, Tc * s->top_k) + S;
  return moe::decode_down_shape(moe::decode_one_col_tile(Tc, s->top_k, s->E), s->H, n_slots,
                                decode_steps(s->w_dtype, std::max(s->I, Is)));
}

// route_only: buffers for moe_route over all T tokens.
Layout make_layout(const moe_shape_t* s, bool route_only) {
  Layout L{};
  L.path = route_only ? MOE_PATH_DECODE : choose_path(s);
  const int T = s->T, H = s->H, E = s->E, k = s->top_k, S = s->n_shared;
  const int I = s->I, Is = S > 0 ? s->I_shared : 0;
  L.Tr = (route_only || L.path == MOE_PATH_PREFILL) ? T : std::min(T, kDecodeMaxT);
  const int Tr = std::max(L.Tr, 1);
  L.tile_m = (!route_only && L.path == MOE_PATH_PREFILL) ? kPrefillTileM : kTileM;
  L.cap = int(roundup(long(Tr) * k + long(E) * (L.tile_m - 1), L.tile_m));
  L.n_tiles = L.cap / L.tile_m;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += al(bytes); return o; };
  L.logits = take(size_t(Tr) * E * 4 * (route_only || L.path == MOE_PATH_PREFILL ? 1 : 4));   // decode: 4 planes
  L.topk_ids = take(size_t(Tr) * k * 4);
  L.topk_w = take(size_t(Tr) * k * 4);
  L.counts = take(size_t(E) * 4);
  L.offsets = take(size_t(E + 1) * 4);
  L.cprefix = take(size_t(E + 1) * 4);
  L.active = take(size_t(E + 1) * 4);
  L.sorted_ids = take(size_t(L.cap) * 4);
  L.tile_expert = take(size_t(L.n_tiles) * 4);
  L.inv = take(size_t(Tr) * k * 4);
  L.h_stride = std::max(I, Is);
  if (!route_only && (L.path == MOE_PATH_DECODE || L.path == MOE_PATH_DECODE_FUSED)) {
    L.h_stride = int(roundup(L.h_stride, kHRowAlign));
    const long rows = long(Tr) * k + long(S) * Tr;
    L.h_plane = rows * L.h_stride;
    // fp16 (Q4_0, Q8_0, fp8) | fp32 | bf16 hi + lo planes
    const size_t elem = (s->w_dtype == MOE_F32 || s->w_dtype == MOE_BF16) ? 4 : 2;
    L.h = take(size_t(L.h_plane) * elem);
    // partial rows: one plane per k range of the down projection (the passes' largest count)
    int planes = 1;
    if (L.path == MOE_PATH_DECODE && T > 0) {
      planes = pass_down_shape(s, Tr).ks;
      if (T % kDecodeMaxT) planes = std::max(planes, pass_down_shape(s, T % kDecodeMaxT).ks);
    }
    L.partials = take(size_t(planes) * rows * H * 4);
    L.dn_count = take(size_t(roundup(H / 16, 4)) * 4);
    if (L.path == MOE_PATH_DECODE) {
      L.sel_flags = take(size_t(4) * ((E + 15) / 16) * ((Tr + 15) / 16) * 8);
      L.error = take(16);
    }
    if (L.path == MOE_PATH_DECODE_FUSED) {
      L.n_items = fused_plan(s, Tr).n_items;
      L.flags = take(size_t(L.n_items) * 8);
      L.error = take(16);          // status pair: this call's tag, the tag of the last call that gave up
    }
  }
  if (!route_only && L.path == MOE_PATH_PREFILL) {
    L.t_pad = int(roundup(T, L.tile_m));
    const long rows = long(L.cap) + long(S) * L.t_pad;
    L.h_plane = rows * L.h_stride;
    L.h = take(size_t(L.h_plane) * 2);
    // routing-weighted rows of the down GEMM: one plane per k range
    L.pf_ksplit = moe::prefill_k_split(L.cap, S, L.t_pad, H, std::max(I, Is));
    L.partials = take(size_t(L.pf_ksplit) * rows * H * 4);
  }
  L.total = off;
  return L;
}

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

thread_local int g_last_hip_error = 0;
}  // namespace

namespace moe {
void set_last_hip_error(int e) { g_last_hip_error = e; }
}  // namespace moe

namespace {

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = int(e);
  return MOE_ERR_HIP;
}

int router_waves(int nblocks) { return nblocks < 64 ? 16 : (nblocks < 256 ? 8 : 4); }

moe::RouteBufs route_bufs(uint8_t* ws, const Layout& L) {
  moe::RouteBufs rb;
  rb.logits = reinterpret_cast<float*>(ws + L.logits);
  rb.topk_ids = reinterpret_cast<int32_t*>(ws + L.topk_ids);
  rb.topk_w = reinterpret_cast<float*>(ws + L.topk_w);
  rb.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  rb.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  rb.cprefix = reinterpret_cast<int32_t*>(ws + L.cprefix);
  rb.active = reinterpret_cast<int32_t*>(ws + L.active);
  rb.sorted_ids = reinterpret_cast<int32_t*>(ws + L.sorted_ids);
  rb.tile_expert = reinterpret_cast<int32_t*>(ws + L.tile_expert);
  rb.inv = reinterpret_cast<int32_t*>(ws + L.inv);
  return rb;
}

moe::RouterArgs router_args(const moe_shape_t* s, int T, const void* x, const void* wr, const float* b,
                            const moe::RouteBufs& rb, int tile_m = kTileM) {
  moe::RouterArgs a{};
  a.x = x; a.wr = wr; a.bias = b;
  a.T = T; a.H = s->H; a.E = s->E; a.k = s->top_k;
  a.tile_m = tile_m;
  a.capacity = int(roundup(long(T) * s->top_k + long(s->E) * (tile_m - 1), tile_m));
  a.n_row_tiles = (s->E + 15) / 16;
  a.n_col_tiles = (T + 15) / 16;
  a.logit_parts = 1;
  a.zero_f32 = nullptr; a.zero_n = 0;
  a.rb = rb;
  return a;
}

// Launch plan of one multi-launch decode pass of Tc tokens.
//  route_in_gu: few assignments and a small gate/up grid (or a tiny
//    selection): the router launch computes the logits only, and every routed
//    gate/up work-group selects and dispatches in its prologue (one launch
//    fewer on the critical path; larger grids would repeat a costly selection
//    too often).
//  logit_parts: few logit tiles are split over 4 work-groups each (partial
//    planes) to spread the router read.
//  shared_in_router: with route_in_gu and split logits, the shared experts'
//    gate/up runs in the logits launch (it needs no routing).
struct PassPlan {
  bool route_in_gu, shared_in_router;
  int logit_parts;
};
PassPlan pass_plan(const moe_shape_t* s, int Tc) {
  const int n_routed_slots = std::min(s->E, Tc * s->top_k);
  const int S = s->n_shared, Is = S > 0 ? s->I_shared : 0;
  const long n_gu_rt = (std::max(s->I, Is) + 15) / 16;
  const long gu_groups = n_gu_rt * (n_routed_slots + S);
  const int nblocks = ((s->E + 15) / 16) * ((Tc + 15) / 16);
  PassPlan p{};
  const bool tiny = long(Tc) * s->E <= kTinySelection && (s->w_dtype == MOE_BF16 || s->w_dtype == MOE_F32);
  p.route_in_gu = Tc <= 16 && moe::small_route(Tc, s->E, s->top_k) &&
                  gu_groups <= (tiny ? kRouteInGateUpMaxGroupsTiny : kRouteInGateUpMaxGroups);
  p.logit_parts = (nblocks < 64 && (p.route_in_gu || nblocks > 1)) ? 4 : 1;
  // shared experts' gate/up in the logits launch: with the routing in the gate/up prologue, or, for
  // one column tile per routed slot, with the selection in one more work-group of that launch
  // (DeepSeek-shaped batch of 8: 5 launches -> 4, about 1 us less; batch of 64: 266.8 -> 262.5 us)
  p.shared_in_router = S > 0 && p.logit_parts == 4 &&
                       (p.route_in_gu || moe::decode_one_col_tile(Tc, s->top_k, s->E));
  return p;
}

}  // namespace

extern "C" {

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "required pointer is NULL (or a pointer that must be NULL is not)";
    case MOE_ERR_SHAPE: return "shape out of range";
    case MOE_ERR_DTYPE: return "unsupported dtype or dtype/path combination";
    case MOE_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failure";
    case MOE_ERR_TOO_LARGE: return "shape needs more workspace than the static scratch of moe_forward_noalloc";
    case MOE_ERR_NOT_PINNED: return "host expert stack is not pinned host memory";
    case MOE_ERR_HOST_ALLOC: return "host memory for the expert cache's bookkeeping could not be allocated";
    default: return "unknown error code";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int moe_resolve_path(const moe_shape_t* s) {
  if (int rc = check_shape(s)) return rc;
  return choose_path(s);
}

int moe_workspace_size(const moe_shape_t* s, size_t* bytes) {
  if (!s || !bytes) return MOE_ERR_NULL;
  int rc = check_shape(s);
  if (rc) return rc;
  const Layout a = make_layout(s, false), b = make_layout(s, true);
  *bytes = std::max(a.total, b.total);
  return MOE_OK;
}

int moe_route_workspace_size(const moe_shape_t* s, size_t* bytes) {
  if (!s || !bytes) return MOE_ERR_NULL;
  if (int rc = check_shape(s)) return rc;
  *bytes = make_layout(s, true).total;
  return MOE_OK;
}

int moe_forward_tables(const moe_shape_t* s, moe_forward_tables_t* t) {
  if (!s || !t) return MOE_ERR_NULL;
  if (int rc = check_shape(s)) return rc;
  const Layout L = make_layout(s, false);
  const bool prefill = L.path == MOE_PATH_PREFILL;
  const int last = s->T == 0 ? 0 : (prefill ? s->T : s->T - (s->T - 1) / kDecodeMaxT * kDecodeMaxT);
  t->path = L.path;
  t->tokens = last;
  t->tile_m = prefill ? L.tile_m : 1;       // decode passes route with tile_m 1 (no padding)
  t->capacity = prefill ? L.cap : last * s->top_k;
  t->n_tiles = prefill ? L.n_tiles : 0;
  t->topk_ids = L.topk_ids;
  t->topk_w = L.topk_w;
  t->counts = L.counts;
  t->offsets = L.offsets;
  t->sorted_ids = L.sorted_ids;
  t->tile_expert = prefill ? L.tile_expert : 0;
  t->inv = L.inv;
  t->active = L.active;
  const PassPlan plan = pass_plan(s, last);
  const bool sel = L.path == MOE_PATH_DECODE && last > 0 && plan.shared_in_router && !plan.route_in_gu;
  t->status = (L.path == MOE_PATH_DECODE_FUSED || sel) ? L.error : 0;
  t->route_in_gateup = L.path == MOE_PATH_DECODE && last > 0 && plan.route_in_gu;
  t->shared_in_router = L.path == MOE_PATH_DECODE && last > 0 && plan.shared_in_router;
  return MOE_OK;
}

int moe_dispatch_dims(const moe_shape_t* s, int32_t* tile_m, int32_t* capacity, int32_t* n_tiles) {
  int rc = check_shape(s);
  if (rc) return rc;
  const long cap = roundup(long(s->T) * s->top_k + long(s->E) * (kTileM - 1), kTileM);
  if (tile_m) *tile_m = kTileM;
  if (capacity) *capacity = int32_t(cap);
  if (n_tiles) *n_tiles = int32_t(cap / kTileM);
  return MOE_OK;
}

int moe_route(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
              const moe_route_out_t* out, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!out || !out->topk_ids || !out->topk_w) return MOE_ERR_NULL;
  if (s->T == 0) return MOE_OK;
  if (!x || !router_w || !workspace) return MOE_ERR_NULL;
  const void* ptrs[] = {x, router_w, router_b, out->topk_ids, out->topk_w, out->counts, out->offsets,
                        out->sorted_ids, out->tile_expert, out->inv, out->active, workspace};
  for (const void* p : ptrs)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  const Layout L = make_layout(s, true);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  moe::RouteBufs rb = route_bufs(ws, L);
  rb.topk_ids = out->topk_ids;
  rb.topk_w = out->topk_w;
  if (out->counts) rb.counts = out->counts;
  if (out->offsets) rb.offsets = out->offsets;
  if (out->sorted_ids) rb.sorted_ids = out->sorted_ids;
  if (out->tile_expert) rb.tile_expert = out->tile_expert;
  if (out->inv) rb.inv = out->inv;
  if (out->active) rb.active = out->active;
  moe::RouterArgs a = router_args(s, s->T, x, router_w, router_b, rb);
  const int nblocks = a.n_row_tiles * a.n_col_tiles;
  return hip_status(moe::launch_router(a, s->router_dtype, s->x_dtype, router_waves(nblocks),
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Records events[i] after launch i of a pass (events[0] before the first launch).
struct StageEvents : moe::StageMarker {
  void* const* ev;
  int n;
  int next = 0;
  StageEvents(void* const* e, int k) : ev(e), n(k) {}
  void mark(hipStream_t st) override {
    if (ev && next < n && ev[next]) (void)hipEventRecord(static_cast<hipEvent_t>(ev[next]), st);
    ++next;
  }
};

int forward_impl(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                 const void* w_gate, const void* w_up, const void* w_down,
                 const void* ws_gate, const void* ws_up, const void* ws_down,
                 void* out, void* workspace, size_t ws_bytes, void* stream, void* const* events, int n_events,
                 moe::DecodeHook* hook = nullptr) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (hook && s->path != MOE_PATH_DECODE) return MOE_ERR_SHAPE;   // the hook runs between decode launches
  if (s->T == 0) return MOE_OK;
  if (!x || !router_w || !w_gate || !w_up || !w_down || !out || !workspace) return MOE_ERR_NULL;
  const bool has_shared = s->n_shared > 0;
  if (has_shared != (ws_gate != nullptr) || has_shared != (ws_up != nullptr) || has_shared != (ws_down != nullptr))
    return MOE_ERR_NULL;
  const void* ptrs[] = {x, router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, out, workspace};
  for (const void* p : ptrs)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  size_t need = 0;
  moe_workspace_size(s, &need);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const Layout L = make_layout(s, false);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int xb = s->x_dtype == MOE_F32 ? 4 : 2;
  const moe::RouteBufs rb = route_bufs(ws, L);

  if (L.path == MOE_PATH_PREFILL) {
    StageEvents sev{events, n_events};
    sev.mark(st);
    moe::RouterArgs ra = router_args(s, s->T, x, router_w, router_b, rb, L.tile_m);
    const int nblocks = ra.n_row_tiles * ra.n_col_tiles;
    if (int e = hip_status(moe::launch_router(ra, s->router_dtype, s->x_dtype, router_waves(nblocks), st))) return e;
    sev.mark(st);
    moe::PrefillArgs p{};
    p.x = x;
    p.wg = static_cast<const uint16_t*>(w_gate); p.wu = static_cast<const uint16_t*>(w_up);
    p.wd = static_cast<const uint16_t*>(w_down);
    p.sg = static_cast<const uint16_t*>(ws_gate); p.su = static_cast<const uint16_t*>(ws_up);
    p.sd = static_cast<const uint16_t*>(ws_down);
    p.T = s->T; p.H = s->H; p.E = s->E; p.I = s->I; p.k = s->top_k; p.S = s->n_shared;
    p.Is = has_shared ? s->I_shared : 0;
    p.capacity = L.cap; p.tile_m = L.tile_m; p.t_pad = L.t_pad;
    p.tile_expert = rb.tile_expert; p.sorted_ids = rb.sorted_ids; p.topk_w = rb.topk_w; p.offsets = rb.offsets;
    p.h = reinterpret_cast<uint16_t*>(ws + L.h);
    p.h_stride = L.h_stride;
    p.partials = reinterpret_cast<float*>(ws + L.partials);
    p.part_plane = (long(L.cap) + long(p.S) * L.t_pad) * s->H;
    p.inv = rb.inv;
    p.out = out;
    return hip_status(moe::launch_prefill(p, s->x_dtype, st, events ? &sev : nullptr));
  }

  // decode: passes of at most kDecodeMaxT tokens (each token's output depends on that token only).
  // The single-launch form is not captured into graphs: a replay would reuse the capture's tags.
  // The same holds for the selection inside the logits launch (its waits compare epochs).
  bool fused = L.path == MOE_PATH_DECODE_FUSED;
  bool capturing = false;
  {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
      (void)hipGetLastError();
      cs = hipStreamCaptureStatusActive;
    }
    capturing = cs != hipStreamCaptureStatusNone;
  }
  fused = fused && !capturing;
  for (int t0 = 0; t0 < s->T; t0 += kDecodeMaxT) {
    const int Tc = std::min(kDecodeMaxT, s->T - t0);
    const uint8_t* xc = static_cast<const uint8_t*>(x) + size_t(t0) * s->H * xb;
    uint8_t* oc = static_cast<uint8_t*>(out) + size_t(t0) * s->H * xb;
    StageEvents sev{events, n_events};
    // decode uses no padding, so the tile table would hold one entry per row: it is not written
    moe::RouteBufs rbd = rb;
    rbd.tile_expert = nullptr;
    moe::RouterArgs ra = router_args(s, Tc, xc, router_w, router_b, rbd, 1);
    moe::DecodeArgs d{};
    d.x = xc;
    d.wg = static_cast<const uint8_t*>(w_gate); d.wu = static_cast<const uint8_t*>(w_up);
    d.wd = static_cast<const uint8_t*>(w_down);
    d.sg = static_cast<const uint8_t*>(ws_gate); d.su = static_cast<const uint8_t*>(ws_up);
    d.sd = static_cast<const uint8_t*>(ws_down);
    d.T = Tc; d.H = s->H; d.E = s->E; d.I = s->I; d.k = s->top_k; d.S = s->n_shared;
    d.Is = has_shared ? s->I_shared : 0;
    d.n_routed_slots = std::min(s->E, Tc * s->top_k);
    d.active = rb.active; d.counts = rb.counts; d.offsets = rb.offsets; d.cprefix = rb.cprefix;
    d.sorted_ids = rb.sorted_ids; d.topk_w = rb.topk_w; d.inv = rb.inv;
    d.h = ws + L.h;
    d.h_plane = long(Tc * s->top_k + s->n_shared * Tc) * L.h_stride;
    d.h_stride = L.h_stride;
    d.partials = reinterpret_cast<float*>(ws + L.partials);
    d.part_plane = long(Tc * s->top_k + s->n_shared * Tc) * s->H;
    if (fused) {                   // the single-launch items use one k range and their own row groups
      d.dn_ksplit = 1;
      d.dn_rpw = 1;
    } else {
      const moe::DownShape ds = pass_down_shape(s, Tc);
      d.dn_ksplit = ds.ks;
      d.dn_rpw = ds.rpw;
      d.dn_waves = ds.waves;
    }
    d.out = oc;
    // combine in the down launch's epilogue when few work-groups write each output row group
    // (their arrival counts serialise on one counter per group); else in a launch of its own
    d.dn_count = d.n_routed_slots + d.S <= kEpilogueMaxSlots ? reinterpret_cast<unsigned*>(ws + L.dn_count) : nullptr;
    const int n_gu_rt = (std::max(s->I, d.Is) + 15) / 16;
    d.n_row_tiles = n_gu_rt;
    if (hook)
      if (int e = hook->before_pass(d, st)) return e;
    sev.mark(st);
    if (fused) {
      moe::FusedArgs f = fused_plan(s, Tc);
      f.r = ra;
      f.r.logit_parts = 4;
      f.d = d;
      f.epoch = next_epoch();
      f.flags = reinterpret_cast<unsigned long long*>(ws + L.flags);
      f.call_tag = reinterpret_cast<unsigned long long*>(ws + L.error);
      f.error = f.call_tag + 1;
      f.spin_rounds = fused_spin_rounds();
      if (int e = hip_status(moe::launch_decode_fused(f, s->w_dtype, s->x_dtype, st))) return e;
      sev.mark(st);
      continue;
    }
    const int nblocks = ra.n_row_tiles * ra.n_col_tiles;
    const PassPlan plan = pass_plan(s, Tc);
    const bool pro = plan.route_in_gu;
    ra.logit_parts = plan.logit_parts;
    if (d.dn_count) {             // the router launch clears the down launch's arrival counters
      ra.zero_f32 = reinterpret_cast<float*>(d.dn_count);
      ra.zero_n = roundup(s->H / 16, 4);
    }
    if (pro) d.route_in_gu = 1;
    if (pro || plan.shared_in_router) {
      d.route = ra;
      d.shared_in_router = plan.shared_in_router;
    }
    if (plan.shared_in_router && !pro && !capturing && L.path == MOE_PATH_DECODE) {
      d.sel_flags = reinterpret_cast<unsigned long long*>(ws + L.sel_flags);
      d.sel_status = reinterpret_cast<unsigned long long*>(ws + L.error);
      d.sel_epoch = next_epoch();
      d.sel_spin = fused_spin_rounds();
    }
    if (!d.shared_in_router) {
      if (int e = hip_status(moe::launch_router(ra, s->router_dtype, s->x_dtype, router_waves(nblocks), st, pro)))
        return e;
      sev.mark(st);
    }
    if (int e = hip_status(moe::launch_decode(d, s->w_dtype, s->x_dtype, s->router_dtype, n_gu_rt, st,
                                              events ? &sev : nullptr)))
      return e;
    if (hook)
      if (int e = hook->after_pass(d, st)) return e;
  }
  return MOE_OK;
}

// ------------------------------------------------ channel-sparse experts --

constexpr int kSparseMaxI = 16384;   // the channel selection keeps one expert's scores in LDS

int sparse_check(const moe_shape_t* s, int budget) {
  if (int rc = check_shape(s)) return rc;
  if (s->w_dtype != MOE_F32 && s->w_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (budget < 1 || budget > s->I || s->I > kSparseMaxI) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// Splits of the kept channels in the down projection for a pass of Tc tokens:
// enough work-groups to fill the chip, few enough that the partial rows stay
// near a tenth of the weight bytes, and each split small enough for LDS.
int sparse_splits(const moe_shape_t* s, int Tc, int c) {
  const int ctiles = (s->H + 2047) / 2048, n = Tc * s->top_k;
  int R = std::min(std::max(1, c / 40), std::max(1, (1024 + ctiles * n - 1) / (ctiles * n)));
  return std::max(R, (c + moe::kSparseMaxRows - 1) / moe::kSparseMaxRows);
}

struct SparseLayout {
  Layout L;            // routing, and h / partials of the shared experts (decode layout)
  size_t sel, hs, spart, total;
};

SparseLayout make_sparse_layout(const moe_shape_t* s0, int c) {
  moe_shape_t s = *s0;
  s.path = MOE_PATH_DECODE;
  SparseLayout S{};
  S.L = make_layout(&s, false);
  const int Tr = std::max(S.L.Tr, 1);
  size_t off = S.L.total;
  auto take = [&](size_t bytes) { size_t o = off; off += al(bytes); return o; };
  // kept channels: [T*k, c], or [T*E, c] when the selection runs for every
  // expert next to a single-tile router (E <= 16, passes of <= 16 tokens)
  size_t sel_rows = size_t(Tr) * s.top_k;
  if (s.E <= 16) sel_rows = std::max(sel_rows, size_t(std::min(Tr, 16)) * s.E);
  S.sel = take(sel_rows * c * 4);
  S.hs = take(size_t(Tr) * s.top_k * c * 4);
  size_t rows = 0;
  for (int Tc = 1; Tc <= Tr; ++Tc) rows = std::max(rows, size_t(Tc) * s.top_k * sparse_splits(&s, Tc, c));
  S.spart = take(rows * s.H * 4);
  S.total = off;
  return S;
}

}  // namespace

extern "C" {

int moe_sparse_workspace_size(const moe_shape_t* s, int32_t budget, size_t* bytes) {
  if (!s || !bytes) return MOE_ERR_NULL;
  if (int rc = sparse_check(s, budget)) return rc;
  *bytes = make_sparse_layout(s, budget).total;
  return MOE_OK;
}

int moe_forward_channel_sparse(const moe_shape_t* s, int32_t budget, const float* channel_scores,
                               const void* x, const void* router_w, const float* router_b,
                               const void* w_gate, const void* w_up, const void* w_down_t,
                               const void* ws_gate, const void* ws_up, const void* ws_down,
                               void* out, void* workspace, size_t ws_bytes, void* stream) {
  if (!s) return MOE_ERR_NULL;
  if (int rc = sparse_check(s, budget)) return rc;
  if (s->T == 0) return MOE_OK;
  if (!channel_scores || !x || !router_w || !w_gate || !w_up || !w_down_t || !out || !workspace) return MOE_ERR_NULL;
  const bool has_shared = s->n_shared > 0;
  if (has_shared != (ws_gate != nullptr) || has_shared != (ws_up != nullptr) || has_shared != (ws_down != nullptr))
    return MOE_ERR_NULL;
  const void* ptrs[] = {channel_scores, x, router_w, router_b, w_gate, w_up, w_down_t, ws_gate, ws_up, ws_down,
                        out, workspace};
  for (const void* p : ptrs)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  const SparseLayout SL = make_sparse_layout(s, budget);
  if (ws_bytes < SL.total) return MOE_ERR_WORKSPACE;
  const Layout& L = SL.L;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int xb = s->x_dtype == MOE_F32 ? 4 : 2;
  const moe::RouteBufs rb = route_bufs(ws, L);
  for (int t0 = 0; t0 < s->T; t0 += kDecodeMaxT) {
    const int Tc = std::min(kDecodeMaxT, s->T - t0);
    const uint8_t* xc = static_cast<const uint8_t*>(x) + size_t(t0) * s->H * xb;
    moe::RouteBufs rbd = rb;
    rbd.tile_expert = nullptr;
    moe::RouterArgs ra = router_args(s, Tc, xc, router_w, router_b, rbd, 1);
    const int nblocks = ra.n_row_tiles * ra.n_col_tiles;
    // one routing tile: the channel selection runs for every expert in the
    // router's launch instead of waiting for it
    const bool sel_all = nblocks == 1;
    if (!sel_all)
      if (int e = hip_status(moe::launch_router(ra, s->router_dtype, s->x_dtype, router_waves(nblocks), st))) return e;
    moe::SparseArgs a{};
    moe::DecodeArgs& d = a.d;
    d.x = xc;
    d.wg = static_cast<const uint8_t*>(w_gate); d.wu = static_cast<const uint8_t*>(w_up);
    d.sg = static_cast<const uint8_t*>(ws_gate); d.su = static_cast<const uint8_t*>(ws_up);
    d.sd = static_cast<const uint8_t*>(ws_down);
    d.T = Tc; d.H = s->H; d.E = s->E; d.I = s->I; d.k = s->top_k; d.S = s->n_shared;
    d.Is = has_shared ? s->I_shared : 0;
    d.n_routed_slots = 0;                     // the decode kernels run the shared experts only
    d.active = rb.active; d.counts = rb.counts; d.offsets = rb.offsets; d.cprefix = rb.cprefix;
    d.sorted_ids = rb.sorted_ids; d.topk_w = rb.topk_w; d.inv = rb.inv;
    d.h = ws + L.h;
    d.h_plane = long(Tc * s->top_k + s->n_shared * Tc) * L.h_stride;
    d.h_stride = L.h_stride;
    d.partials = reinterpret_cast<float*>(ws + L.partials);
    d.part_plane = long(Tc * s->top_k + s->n_shared * Tc) * s->H;
    d.dn_ksplit = 1;             // the shared experts' down writes one plane (read by the sparse combine)
    d.dn_rpw = moe::decode_down_shape(Tc <= 16, s->H, s->n_shared, 0).rpw;
    d.n_row_tiles = (std::max(s->I, d.Is) + 15) / 16;
    d.out = static_cast<uint8_t*>(out) + size_t(t0) * s->H * xb;
    a.topk_ids = rb.topk_ids;
    a.scores = channel_scores + size_t(t0) * s->E * s->I;
    a.wdt = static_cast<const uint8_t*>(w_down_t);
    a.c = budget;
    a.R = sparse_splits(s, Tc, budget);
    a.sel = reinterpret_cast<int32_t*>(ws + SL.sel);
    a.hs = reinterpret_cast<float*>(ws + SL.hs);
    a.spart = reinterpret_cast<float*>(ws + SL.spart);
    a.sel_all = sel_all ? 1 : 0;
    if (sel_all)
      if (int e = hip_status(moe::launch_sparse_route_select(ra, a, s->router_dtype, s->x_dtype, st))) return e;
    if (int e = hip_status(moe::launch_sparse(a, s->w_dtype, s->x_dtype, st, nullptr))) return e;
  }
  return MOE_OK;
}

}  // extern "C"

namespace moe {
// moe_forward on the decode path with a hook around each pass's expert launches.
int forward_hooked(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                   const void* w_gate, const void* w_up, const void* w_down,
                   const void* ws_gate, const void* ws_up, const void* ws_down,
                   void* out, void* workspace, size_t ws_bytes, void* stream, DecodeHook* hook) {
  return forward_impl(s, x, router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, out, workspace,
                      ws_bytes, stream, nullptr, 0, hook);
}
}  // namespace moe

extern "C" {

int moe_forward(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                const void* w_gate, const void* w_up, const void* w_down,
                const void* ws_gate, const void* ws_up, const void* ws_down,
                void* out, void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(s, x, router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, out, workspace,
                      ws_bytes, stream, nullptr, 0);
}

int moe_forward_profiled(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                         const void* w_gate, const void* w_up, const void* w_down,
                         const void* ws_gate, const void* ws_up, const void* ws_down,
                         void* out, void* workspace, size_t ws_bytes, void* stream,
                         void* const* events, int n_events) {
  if (!events || n_events < 1) return MOE_ERR_NULL;
  return forward_impl(s, x, router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, out, workspace,
                      ws_bytes, stream, events, n_events);
}

}  // extern "C"
