// Host-resident routed experts with a GPU expert cache and predictive
// prefetching ("FATE: how to speed up MoE inference in llama.cpp with an
// expert cache and prefetching", ai-manual.ru, sections "How the expert cache
// works" and "Predictive prefetching: guessing the future").  Host code only:
// the bookkeeping of which (layer, expert) sits in which slot, the copies on
// the caller's copy stream and the event edges between that stream and the
// compute stream.  The expert kernels are the decode path's; they read the
// routed matrices from the slot stacks through DecodeArgs::active_w.
//
// Region layout (device, caller-allocated):
//   [0, 256 * ceil((E + 1) * 4 / 256))    active_w: count, then the slot of each active expert
//   then three stacks of n_slots matrices in w_dtype's layout (gate, up, down),
//   each starting at a multiple of 256 bytes.
// Copying expert e of a layer into slot s copies matrix e of each host stack
// to matrix s of the slot stack: its codes, and for the quantised formats its
// scales, which sit after all codes of a stack.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "common.hpp"

namespace moe {
int forward_hooked(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                   const void* w_gate, const void* w_up, const void* w_down,
                   const void* ws_gate, const void* ws_up, const void* ws_down,
                   void* out, void* workspace, size_t ws_bytes, void* stream, DecodeHook* hook);
hipError_t launch_put_i32(int32_t* dst, const int32_t* v, int n, hipStream_t st);
void set_last_hip_error(int e);
}  // namespace moe

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxSlots = 65536;
constexpr int kPassMaxT = 64;   // tokens per decode pass (as moe_forward's decode path)

size_t roundup(size_t v, size_t a) { return (v + a - 1) / a * a; }

// One matrix [N, K] of a stack in a weight format: its code bytes, its scale
// bytes, and where the scales of a stack of n matrices start.
struct Geom {
  int wdt;
  long N, K;
  size_t code() const {
    switch (wdt) {
      case MOE_F32: return size_t(N) * K * 4;
      case MOE_BF16: return size_t(N) * K * 2;
      case MOE_Q4_0: return size_t(N) * K / 2;
      default: return size_t(N) * K;                    // Q8_0, FP8: one byte per value
    }
  }
  size_t scale() const {
    switch (wdt) {
      case MOE_Q4_0:
      case MOE_Q8_0: return size_t(N) * (K / 32) * 2;   // fp16 per block of 32
      case MOE_FP8_E4M3: return size_t(N) * 4;          // fp32 per row
      default: return 0;
    }
  }
  size_t scale_offset(long n) const {
    if (wdt == MOE_Q4_0) return moe::q4_scale_offset(n, N, K);
    if (wdt == MOE_Q8_0 || wdt == MOE_FP8_E4M3) return moe::byte_code_scale_offset(n, N, K);
    return size_t(n) * code();
  }
  size_t stack(long n) const { return scale() ? scale_offset(n) + size_t(n) * scale() : size_t(n) * code(); }
};

struct Geoms {
  Geom m[3];   // gate, up, down
  size_t head, off[3], total;
  Geoms(const moe_shape_t* s, long n_slots)
      : m{{s->w_dtype, s->I, s->H}, {s->w_dtype, s->I, s->H}, {s->w_dtype, s->H, s->I}} {
    head = roundup(size_t(s->E + 1) * 4, kAlign);
    size_t o = head;
    for (int i = 0; i < 3; ++i) {
      off[i] = o;
      o = roundup(o + m[i].stack(n_slots), kAlign);
    }
    total = o;
  }
};

bool same_layer_shape(const moe_shape_t* a, const moe_shape_t* b) {
  return a->H == b->H && a->E == b->E && a->I == b->I && a->top_k == b->top_k && a->n_shared == b->n_shared &&
         (a->n_shared == 0 || a->I_shared == b->I_shared) && a->x_dtype == b->x_dtype &&
         a->w_dtype == b->w_dtype && a->router_dtype == b->router_dtype;
}

int hip_fail(hipError_t e) {
  moe::set_last_hip_error(int(e));
  return MOE_ERR_HIP;
}

}  // namespace

struct moe_expert_cache : moe::DecodeHook {
  moe_shape_t shape;
  int n_layers, n_slots, depth, shift;
  std::vector<moe_host_experts_t> host;
  uint8_t* region;
  Geoms geo;
  hipStream_t copy;
  // per slot
  std::vector<int> key;              // layer * E + expert held (or being copied in), -1 if none
  std::vector<uint64_t> stamp;       // last use or fill, for least-recently-used replacement
  std::vector<char> prefetched;      // filled by a prefetch and not used since
  std::vector<char> wait_ready;      // a copy into the slot that the compute stream has not waited for
  std::vector<char> wait_release;    // reads of the slot that the copy stream has not waited for
  std::vector<char> in_pass;         // needed by the current pass
  std::vector<hipEvent_t> ready;     // recorded on the copy stream after the slot's last fill
  std::vector<hipEvent_t> released;  // recorded on the compute stream after the slot's last reader
  std::vector<int> where;            // [n_layers * E]: slot of (layer, expert), -1 if not resident
  std::vector<int32_t> act;          // host copy of a pass's active list
  std::vector<int32_t> slot_list;    // count, then the slot of each active expert
  std::vector<int> pass_slots;
  uint64_t clock = 0;
  int layer = 0;                     // layer of the call in progress
  moe_cache_stats_t stats{};

  moe_expert_cache(const moe_shape_t* s, int L, const moe_host_experts_t* layers, void* reg, int C, int d, int sh,
                   hipStream_t cs)
      : shape(*s), n_layers(L), n_slots(C), depth(d), shift(sh), host(layers, layers + L),
        region(static_cast<uint8_t*>(reg)), geo(s, C), copy(cs), key(C, -1), stamp(C, 0), prefetched(C, 0),
        wait_ready(C, 0), wait_release(C, 0), in_pass(C, 0), ready(C, nullptr), released(C, nullptr),
        where(size_t(L) * s->E, -1), act(s->E + 1), slot_list(s->E + 1) {}

  int32_t* active_w() const { return reinterpret_cast<int32_t*>(region); }
  const uint8_t* stack(int m) const { return region + geo.off[m]; }

  // Least recently used slot outside the current pass (and, for prefetches,
  // outside the experts this round already placed); -1 if every slot is taken.
  int victim(const std::vector<char>& taken) const {
    int best = -1;
    for (int i = 0; i < n_slots; ++i) {
      if (in_pass[i] || taken[i]) continue;
      if (key[i] < 0) return i;
      if (best < 0 || stamp[i] < stamp[best]) best = i;
    }
    return best;
  }

  // Copy expert e of layer l into slot s on the copy stream, after every read
  // of the slot's previous contents.
  int fill(int l, int e, int s) {
    if (key[s] >= 0) where[key[s]] = -1;
    key[s] = l * shape.E + e;
    where[key[s]] = s;
    if (wait_release[s]) {
      if (hipError_t r = hipStreamWaitEvent(copy, released[s], 0)) return hip_fail(r);
      wait_release[s] = 0;
    }
    const void* src[3] = {host[l].w_gate, host[l].w_up, host[l].w_down};
    for (int m = 0; m < 3; ++m) {
      const Geom& g = geo.m[m];
      const uint8_t* h = static_cast<const uint8_t*>(src[m]);
      uint8_t* dst = region + geo.off[m];
      if (hipError_t r = hipMemcpyAsync(dst + size_t(s) * g.code(), h + size_t(e) * g.code(), g.code(),
                                        hipMemcpyHostToDevice, copy))
        return hip_fail(r);
      if (g.scale()) {
        if (hipError_t r = hipMemcpyAsync(dst + g.scale_offset(n_slots) + size_t(s) * g.scale(),
                                          h + g.scale_offset(shape.E) + size_t(e) * g.scale(), g.scale(),
                                          hipMemcpyHostToDevice, copy))
          return hip_fail(r);
      }
      stats.bytes_copied += g.code() + g.scale();
    }
    if (hipError_t r = hipEventRecord(ready[s], copy)) return hip_fail(r);
    wait_ready[s] = 1;
    stamp[s] = ++clock;
    return MOE_OK;
  }

  int before_experts(moe::DecodeArgs& d, hipStream_t st) override {
    const int E = shape.E;
    if (hipError_t r = hipMemcpyAsync(act.data(), d.active, size_t(E + 1) * 4, hipMemcpyDeviceToHost, st))
      return hip_fail(r);
    if (hipError_t r = hipStreamSynchronize(st)) return hip_fail(r);
    const int A = act[0];
    if (A < 0 || A > E || A > n_slots) return MOE_ERR_TOO_LARGE;   // not reached: checked per call
    pass_slots.clear();
    // hits first, so that a miss never evicts an expert this pass needs
    for (int j = 0; j < A; ++j) {
      const int e = act[1 + j];
      if (e < 0 || e >= E) return MOE_ERR_HIP;
      const int s = where[size_t(layer) * E + e];
      slot_list[1 + j] = s;
      if (s >= 0) in_pass[s] = 1;
    }
    std::vector<char> none(n_slots, 0);
    for (int j = 0; j < A; ++j) {
      ++stats.lookups;
      int s = slot_list[1 + j];
      if (s >= 0) {
        ++stats.hits;
        if (prefetched[s]) ++stats.prefetch_hits;
      } else {
        ++stats.misses;
        s = victim(none);
        if (s < 0) return MOE_ERR_TOO_LARGE;
        if (int rc = fill(layer, act[1 + j], s)) return rc;
        in_pass[s] = 1;
        slot_list[1 + j] = s;
      }
      prefetched[s] = 0;
      stamp[s] = ++clock;
      pass_slots.push_back(s);
    }
    slot_list[0] = A;
    if (hipError_t r = moe::launch_put_i32(active_w(), slot_list.data(), A + 1, st)) return hip_fail(r);
    for (int s : pass_slots) {
      if (!wait_ready[s]) continue;
      if (hipError_t r = hipStreamWaitEvent(st, ready[s], 0)) return hip_fail(r);
      wait_ready[s] = 0;
    }
    d.wg = stack(0);
    d.wu = stack(1);
    d.wd = stack(2);
    d.active_w = active_w();
    d.E_w = n_slots;
    return MOE_OK;
  }

  int after_experts(hipStream_t st) override {
    for (int s : pass_slots) {
      if (hipError_t r = hipEventRecord(released[s], st)) return hip_fail(r);
      wait_release[s] = 1;
    }
    // prefetch the predicted experts of the next layers into slots this pass does not use
    const int E = shape.E, A = act[0];
    std::vector<char> taken(n_slots, 0);
    for (int dd = 1; dd <= depth; ++dd) {
      const int l = (layer + dd) % n_layers;
      const int off = int(((long(dd) * shift) % E + E) % E);
      for (int j = 0; j < A; ++j) {
        const int e = (act[1 + j] + off) % E;
        const int cur = where[size_t(l) * E + e];
        if (cur >= 0) {
          taken[cur] = 1;          // already resident or on its way: keep it
          continue;
        }
        const int s = victim(taken);
        if (s < 0) break;
        if (int rc = fill(l, e, s)) return rc;
        prefetched[s] = 1;
        taken[s] = 1;
        ++stats.prefetches;
      }
    }
    for (int s : pass_slots) in_pass[s] = 0;
    pass_slots.clear();
    return MOE_OK;
  }
};

extern "C" {

int moe_cache_region_bytes(const moe_shape_t* s, int32_t n_slots, size_t* bytes) {
  if (!s || !bytes) return MOE_ERR_NULL;
  moe_shape_t t = *s;
  t.T = 1;
  t.path = MOE_PATH_DECODE;
  size_t ws = 0;
  if (int rc = moe_workspace_size(&t, &ws)) return rc;
  if (n_slots < 1 || n_slots > kMaxSlots) return MOE_ERR_SHAPE;
  *bytes = Geoms(s, n_slots).total;
  return MOE_OK;
}

int moe_cache_create(const moe_shape_t* s, int32_t n_layers, const moe_host_experts_t* layers, void* region,
                     size_t region_bytes, int32_t n_slots, int32_t prefetch_depth, int32_t prefetch_shift,
                     void* copy_stream, moe_expert_cache_t** out) {
  if (!s || !layers || !region || !out) return MOE_ERR_NULL;
  *out = nullptr;
  size_t need = 0;
  if (int rc = moe_cache_region_bytes(s, n_slots, &need)) return rc;
  if (n_layers < 1 || prefetch_depth < 0 || prefetch_depth >= n_layers) return MOE_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(region) % kAlign) return MOE_ERR_ALIGN;
  if (region_bytes < need) return MOE_ERR_WORKSPACE;
  if (!copy_stream) return MOE_ERR_NULL;
  for (int l = 0; l < n_layers; ++l) {
    const void* p[3] = {layers[l].w_gate, layers[l].w_up, layers[l].w_down};
    for (const void* q : p) {
      if (!q) return MOE_ERR_NULL;
      hipPointerAttribute_t at{};
      const hipError_t r = hipPointerGetAttributes(&at, q);
      if (r != hipSuccess || at.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return MOE_ERR_NOT_PINNED;
      }
    }
  }
  auto* c = new moe_expert_cache(s, n_layers, layers, region, n_slots, prefetch_depth, prefetch_shift,
                                 static_cast<hipStream_t>(copy_stream));
  for (int i = 0; i < n_slots; ++i) {
    hipError_t r = hipEventCreateWithFlags(&c->ready[i], hipEventDisableTiming);
    if (r == hipSuccess) r = hipEventCreateWithFlags(&c->released[i], hipEventDisableTiming);
    if (r != hipSuccess) {
      moe_cache_destroy(c);
      return hip_fail(r);
    }
  }
  *out = c;
  return MOE_OK;
}

int moe_cache_destroy(moe_expert_cache_t* c) {
  if (!c) return MOE_ERR_NULL;
  const hipError_t r = hipStreamSynchronize(c->copy);
  for (hipEvent_t e : c->ready)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->released)
    if (e) (void)hipEventDestroy(e);
  delete c;
  return r == hipSuccess ? MOE_OK : hip_fail(r);
}

int moe_forward_cached(moe_expert_cache_t* c, int32_t layer, const moe_shape_t* s, const void* x,
                       const void* router_w, const float* router_b,
                       const void* ws_gate, const void* ws_up, const void* ws_down,
                       void* out, void* workspace, size_t ws_bytes, void* stream) {
  if (!c || !s) return MOE_ERR_NULL;
  if (!same_layer_shape(s, &c->shape)) return MOE_ERR_SHAPE;
  if (layer < 0 || layer >= c->n_layers) return MOE_ERR_SHAPE;
  moe_shape_t t = *s;
  t.path = MOE_PATH_DECODE;
  const long pass_t = std::min<long>(t.T, kPassMaxT);
  if (std::min<long>(t.E, pass_t * t.top_k) > c->n_slots) return MOE_ERR_TOO_LARGE;
  c->layer = layer;
  return moe::forward_hooked(&t, x, router_w, router_b, c->stack(0), c->stack(1), c->stack(2), ws_gate, ws_up,
                             ws_down, out, workspace, ws_bytes, stream, c);
}

int moe_cache_stats(moe_expert_cache_t* c, moe_cache_stats_t* out, int32_t reset) {
  if (!c || !out) return MOE_ERR_NULL;
  *out = c->stats;
  if (reset) c->stats = moe_cache_stats_t{};
  return MOE_OK;
}

int moe_cache_flush(moe_expert_cache_t* c) {
  if (!c) return MOE_ERR_NULL;
  std::fill(c->where.begin(), c->where.end(), -1);
  std::fill(c->key.begin(), c->key.end(), -1);
  std::fill(c->prefetched.begin(), c->prefetched.end(), 0);
  return MOE_OK;
}

}  // extern "C"
