// Host-resident routed experts with a GPU expert cache and predictive
// prefetching ("FATE: how to speed up MoE inference in llama.cpp with an
// expert cache and prefetching", ai-manual.ru, sections "How the expert cache
// works" and "Predictive prefetching: guessing the future").  Host code only:
// the bookkeeping of which (layer, expert) sits in which slot, the copies on
// the caller's copy stream and the event edges between that stream and the
// compute stream.  The expert kernels are the decode path's; they read the
// routed matrices from the slot stacks through DecodeArgs::active_w.
//
// Region layout (device, caller-allocated): three stacks of n_slots matrices
// in w_dtype's layout (gate, up, down), each starting at a multiple of 256
// bytes.  The slot of each active expert (DecodeArgs::active_w) lives in the
// cache's pinned host buffer: the host writes it before the expert launches
// and they read it through its device mapping.
// Copying expert e of a layer into slot s copies matrix e of each host stack
// to matrix s of the slot stack: its codes, and for the quantised formats its
// scales, which sit after all codes of a stack.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdint>
#include <cstring>
#include <vector>

#include "common.hpp"

namespace moe {
int forward_hooked(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                   const void* w_gate, const void* w_up, const void* w_down,
                   const void* ws_gate, const void* ws_up, const void* ws_down,
                   void* out, void* workspace, size_t ws_bytes, void* stream, DecodeHook* hook);
hipError_t launch_gather_copy(const void* const* src, void* const* dst, const size_t* bytes, int n, hipStream_t st);
hipError_t launch_export_list(const int32_t* src, int n, int32_t* dst, unsigned long long* flag,
                              unsigned long long tag, hipStream_t st);
void set_last_hip_error(int e);
}  // namespace moe

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxSlots = 65536;
constexpr int kPassMaxT = 64;   // tokens per decode pass (as moe_forward's decode path)
constexpr size_t kPinListOffset = 64;                 // pinned host buffer: tag, active list, slot list
constexpr double kSpinSeconds = 0.2;                  // then the wait for a pass's routing blocks on the stream

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
  size_t off[3], total;
  Geoms(const moe_shape_t* s, long n_slots)
      : m{{s->w_dtype, s->I, s->H}, {s->w_dtype, s->I, s->H}, {s->w_dtype, s->H, s->I}} {
    size_t o = 0;
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
  std::vector<moe_host_experts_t> host;  // device-mapped addresses of the pinned host stacks
  uint8_t* pin = nullptr;                // pinned, fine-grained host buffer: tag, then a pass's active list
  uint8_t* pin_dev = nullptr;            // ... as the device addresses it
  unsigned long long tag = 0;
  // copies enqueued by fill and not yet launched (launch_copies)
  std::vector<const void*> seg_src;
  std::vector<void*> seg_dst;
  std::vector<size_t> seg_bytes;
  std::vector<int> seg_slots;
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
  std::vector<char> taken;           // scratch of after_experts (slots placed by this prefetch round)
  std::vector<char> none;            // all zero: no slot excluded beyond the pass's own
  uint64_t clock = 0;
  int layer = 0;                     // layer of the call in progress
  moe_cache_stats_t stats{};

  moe_expert_cache(const moe_shape_t* s, int L, const moe_host_experts_t* layers, void* reg, int C, int d, int sh,
                   hipStream_t cs)
      : shape(*s), n_layers(L), n_slots(C), depth(d), shift(sh), host(layers, layers + L),
        region(static_cast<uint8_t*>(reg)), geo(s, C), copy(cs), key(C, -1), stamp(C, 0), prefetched(C, 0),
        wait_ready(C, 0), wait_release(C, 0), in_pass(C, 0), ready(C, nullptr), released(C, nullptr),
        where(size_t(L) * s->E, -1), act(s->E + 1), slot_list(s->E + 1), taken(C, 0), none(C, 0) {
    pass_slots.reserve(size_t(s->E));
    const size_t segs = size_t(C) * 6;
    seg_src.reserve(segs);
    seg_dst.reserve(segs);
    seg_bytes.reserve(segs);
    seg_slots.reserve(size_t(C));
  }

  size_t pin_slot_offset() const { return kPinListOffset + roundup(size_t(shape.E + 1) * 4, 64); }
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
      add_seg(h + size_t(e) * g.code(), dst + size_t(s) * g.code(), g.code());
      if (g.scale())
        add_seg(h + g.scale_offset(shape.E) + size_t(e) * g.scale(), dst + g.scale_offset(n_slots) +
                size_t(s) * g.scale(), g.scale());
      stats.bytes_copied += g.code() + g.scale();
    }
    seg_slots.push_back(s);
    wait_ready[s] = 1;
    stamp[s] = ++clock;
    return MOE_OK;
  }

  void add_seg(const void* src, void* dst, size_t bytes) {
    seg_src.push_back(src);
    seg_dst.push_back(dst);
    seg_bytes.push_back(bytes);
  }

  // Launch the pending copies on the copy stream (kCopyMaxSegs segments a
  // launch), then mark each filled slot ready after them.
  int launch_copies() {
    for (size_t i = 0; i < seg_src.size(); i += moe::kCopyMaxSegs) {
      const int n = int(std::min<size_t>(moe::kCopyMaxSegs, seg_src.size() - i));
      if (hipError_t r = moe::launch_gather_copy(&seg_src[i], &seg_dst[i], &seg_bytes[i], n, copy))
        return hip_fail(r);
    }
    for (int s : seg_slots)
      if (hipError_t r = hipEventRecord(ready[s], copy)) return hip_fail(r);
    seg_src.clear();
    seg_dst.clear();
    seg_bytes.clear();
    seg_slots.clear();
    return MOE_OK;
  }

  // The pass's active list, read back through the pinned buffer: a kernel
  // writes it there after the routing, and the host polls the tag (then, past
  // kSpinSeconds, blocks on the stream).
  int read_active(const int32_t* active, hipStream_t st) {
    const int n = shape.E + 1;
    auto* flag = reinterpret_cast<unsigned long long*>(pin);
    const unsigned long long want = ++tag;
    if (hipError_t r = moe::launch_export_list(active, n, reinterpret_cast<int32_t*>(pin_dev + kPinListOffset),
                                               reinterpret_cast<unsigned long long*>(pin_dev), want, st))
      return hip_fail(r);
    const auto t0 = std::chrono::steady_clock::now();
    for (long it = 0; __atomic_load_n(flag, __ATOMIC_ACQUIRE) != want; ++it) {
      if ((it & 1023) == 1023 &&
          std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() > kSpinSeconds) {
        if (hipError_t r = hipStreamSynchronize(st)) return hip_fail(r);
        if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) != want) return hip_fail(hipErrorLaunchFailure);
        break;
      }
    }
    std::memcpy(act.data(), pin + kPinListOffset, size_t(n) * 4);
    return MOE_OK;
  }

  int before_experts(moe::DecodeArgs& d, hipStream_t st) override {
    const int E = shape.E;
    if (int rc = read_active(d.active, st)) return rc;
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
    if (int rc = launch_copies()) return rc;
    // the previous pass's launches, the last readers of the list, finished before its routing did
    slot_list[0] = A;
    std::memcpy(pin + pin_slot_offset(), slot_list.data(), size_t(A + 1) * 4);
    for (int s : pass_slots) {
      if (!wait_ready[s]) continue;
      if (hipError_t r = hipStreamWaitEvent(st, ready[s], 0)) return hip_fail(r);
      wait_ready[s] = 0;
    }
    d.wg = stack(0);
    d.wu = stack(1);
    d.wd = stack(2);
    d.active_w = reinterpret_cast<const int32_t*>(pin_dev + pin_slot_offset());
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
    std::fill(taken.begin(), taken.end(), 0);
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
    return launch_copies();
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
  std::vector<moe_host_experts_t> mapped;
  try {
    mapped.assign(layers, layers + n_layers);
  } catch (...) {
    return MOE_ERR_HOST_ALLOC;
  }
  for (int l = 0; l < n_layers; ++l) {
    const void** p[3] = {&mapped[l].w_gate, &mapped[l].w_up, &mapped[l].w_down};
    for (const void** q : p) {
      if (!*q) return MOE_ERR_NULL;
      if (reinterpret_cast<uintptr_t>(*q) % 16) return MOE_ERR_ALIGN;
      hipPointerAttribute_t at{};
      void* dp = nullptr;
      hipError_t r = hipPointerGetAttributes(&at, *q);
      if (r == hipSuccess && at.type == hipMemoryTypeHost) r = hipHostGetDevicePointer(&dp, const_cast<void*>(*q), 0);
      if (r != hipSuccess || at.type != hipMemoryTypeHost || !dp) {
        (void)hipGetLastError();
        return MOE_ERR_NOT_PINNED;
      }
      *q = dp;
    }
  }
  moe_expert_cache* c = nullptr;
  try {       // no exception crosses the C ABI: host allocation failure is reported as MOE_ERR_HOST_ALLOC
    c = new moe_expert_cache(s, n_layers, mapped.data(), region, n_slots, prefetch_depth, prefetch_shift,
                             static_cast<hipStream_t>(copy_stream));
  } catch (...) {
    return MOE_ERR_HOST_ALLOC;
  }
  {
    void* pin = nullptr;
    void* pin_dev = nullptr;
    hipError_t r = hipHostMalloc(&pin, c->pin_slot_offset() + size_t(s->E + 1) * 4, hipHostMallocCoherent);
    if (r == hipSuccess) r = hipHostGetDevicePointer(&pin_dev, pin, 0);
    if (r != hipSuccess) {
      if (pin) (void)hipHostFree(pin);
      delete c;
      return hip_fail(r);
    }
    c->pin = static_cast<uint8_t*>(pin);
    c->pin_dev = static_cast<uint8_t*>(pin_dev);
    *reinterpret_cast<unsigned long long*>(c->pin) = 0;
  }
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
  if (c->pin) (void)hipHostFree(c->pin);
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
