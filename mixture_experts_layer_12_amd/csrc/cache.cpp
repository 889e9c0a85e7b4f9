// Host-resident routed experts with a GPU expert cache and predictive
// prefetching ("FATE: how to speed up MoE inference in llama.cpp with an
// expert cache and prefetching", ai-manual.ru, sections "How the expert cache
// works" and "Predictive prefetching: guessing the future").  Host code only:
// the bookkeeping of which (layer, expert) sits in which slot, the copies on
// the caller's copy stream, and the slot map the expert kernels read.
//
// Region layout (device, caller-allocated): the slot map, int32 [n_layers][E]
// (the slot of each (layer, expert), -1 when not resident), then three stacks
// of n_slots matrices in w_dtype's layout (gate, up, down), each starting at a
// multiple of 256 bytes.  Copying expert e of a layer into slot s copies
// matrix e of each host stack to matrix s of the slot stack: its codes, and
// for the quantised formats its scales, which sit after all codes of a stack.
//
// The expert kernels look each engaged expert up in the map: a resident one
// is read from its slot, any other straight from the pinned host stacks
// through their device mapping (the same bytes, so the result never depends
// on the cache).  No call waits for its own routing.  After each pass a kernel
// writes the pass's active list into a ring of pinned host buffers; the host
// reads it (at once when prefetching, else whenever it has arrived) to count
// hits and misses, to copy in the experts missed a second time and to
// prefetch the predicted experts of the next layers.
//
// Every change of the map is a kernel on the compute stream, so each expert
// launch sees one fixed map:
//  * eviction: the entry of the slot's old expert becomes -1; the copy
//    stream waits for an event recorded after that kernel, so no launch that
//    could still read the old contents runs while the slot is overwritten;
//  * publication: once a slot's copy has completed, its entry is set.  A
//    pass waits for the copies of its own layer's experts and publishes them;
//    other copies are published when they are found complete.
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
hipError_t launch_map_update(int32_t* map, const int32_t* idx, const int32_t* val, int n, hipStream_t st);
hipError_t launch_map_clear(int32_t* map, long n, hipStream_t st);
void set_last_hip_error(int e);
}  // namespace moe

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxSlots = 65536;
constexpr int kMaxLayers = 65536;
constexpr int kRing = 64;                 // passes whose active lists the host has not read yet
constexpr double kSpinSeconds = 0.2;      // then a wait for an active list blocks on the stream
constexpr int kPrefetchBit = 1 << 30;     // marks a prefetch request

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
  Geoms(const moe_shape_t* s, long n_layers, long n_slots)
      : m{{s->w_dtype, s->I, s->H}, {s->w_dtype, s->I, s->H}, {s->w_dtype, s->H, s->I}} {
    size_t o = roundup(size_t(n_layers) * s->E * 4, kAlign);   // the slot map
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

enum SlotState : char { kFree = 0, kFilling = 1, kResident = 2 };

}  // namespace

struct moe_expert_cache : moe::DecodeHook {
  moe_shape_t shape;
  int n_layers, n_slots, depth, shift;
  std::vector<moe_host_experts_t> host;  // device-mapped addresses of the pinned host stacks
  uint8_t* region;
  int32_t* map;                          // device slot map [n_layers][E]
  Geoms geo;
  hipStream_t copy;
  // pinned, fine-grained host ring of kRing entries: a tag, then a pass's active list
  uint8_t* pin = nullptr;
  uint8_t* pin_dev = nullptr;
  size_t entry_bytes = 0;
  unsigned long long tag = 0;
  // passes whose lists are not read yet, oldest first
  struct Rec {
    unsigned long long tag;
    int layer;
    int entry;
  };
  std::vector<Rec> recs;                 // at most kRing
  std::vector<int32_t> snaps;            // [kRing][E]: the map of the pass's layer as the pass saw it
  int next_entry = 0;
  // per slot
  std::vector<int> key;                  // layer * E + expert held or being copied in, -1 if none
  std::vector<char> state;
  std::vector<uint64_t> stamp;           // last use or fill, for least-recently-used replacement
  std::vector<char> prefetched;          // filled by a prefetch and not used since
  std::vector<char> wait_release;        // unmapped since the copy stream last waited for the compute stream
  std::vector<char> busy;                // scratch: chosen or published in the current round
  std::vector<hipEvent_t> ready;         // recorded on the copy stream after the slot's last fill
  hipEvent_t released = nullptr;         // recorded on the compute stream after map changes
  // per (layer, expert)
  std::vector<int> pub;                  // slot in the map as enqueued on the compute stream, or -1
  std::vector<int> filling;              // slot being filled, or -1
  std::vector<char> requested;           // in `req`
  std::vector<uint8_t> missed;           // misses since the expert was last copied in (saturating)
  std::vector<int> req;                  // keys to copy in (kPrefetchBit marks a prefetch)
  // scratch
  std::vector<int32_t> act, map_idx, map_val;
  std::vector<const void*> seg_src;
  std::vector<void*> seg_dst;
  std::vector<size_t> seg_bytes;
  std::vector<int> seg_slots;
  uint64_t clock = 0;
  int layer = 0;                         // layer of the call in progress
  bool flush_pending = false;
  moe_cache_stats_t stats{};

  moe_expert_cache(const moe_shape_t* s, int L, const moe_host_experts_t* layers, void* reg, int C, int d, int sh,
                   hipStream_t cs)
      : shape(*s), n_layers(L), n_slots(C), depth(d), shift(sh), host(layers, layers + L),
        region(static_cast<uint8_t*>(reg)), map(static_cast<int32_t*>(reg)), geo(s, L, C), copy(cs),
        snaps(size_t(kRing) * s->E), key(C, -1), state(C, kFree), stamp(C, 0), prefetched(C, 0),
        wait_release(C, 0), busy(C, 0), ready(C, nullptr), pub(size_t(L) * s->E, -1),
        filling(size_t(L) * s->E, -1), requested(size_t(L) * s->E, 0), missed(size_t(L) * s->E, 0),
        act(s->E + 1) {
    recs.reserve(kRing);
    req.reserve(size_t(L) * s->E);
    map_idx.reserve(size_t(2) * C);
    map_val.reserve(size_t(2) * C);
    const size_t segs = size_t(C) * 6;
    seg_src.reserve(segs);
    seg_dst.reserve(segs);
    seg_bytes.reserve(segs);
    seg_slots.reserve(size_t(C));
    entry_bytes = roundup(8 + size_t(s->E + 1) * 4, 64);
  }

  uint8_t* stack(int m) const { return region + geo.off[m]; }
  const unsigned long long* entry_tag(int i) const {
    return reinterpret_cast<const unsigned long long*>(pin + size_t(i) * entry_bytes);
  }

  // ------------------------------------------------------------ reading --
  // Whether pass record r's list has arrived; with `wait`, waits for it
  // (spinning, then blocking on `st`).  Sets rc on a HIP failure.
  bool arrived(const Rec& r, bool wait, hipStream_t st, int& rc) {
    const unsigned long long* f = entry_tag(r.entry);
    if (__atomic_load_n(f, __ATOMIC_ACQUIRE) == r.tag) return true;
    if (!wait) return false;
    const auto t0 = std::chrono::steady_clock::now();
    for (long it = 0; __atomic_load_n(f, __ATOMIC_ACQUIRE) != r.tag; ++it) {
      if ((it & 1023) == 1023 &&
          std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() > kSpinSeconds) {
        if (hipError_t e = hipStreamSynchronize(st)) {
          rc = hip_fail(e);
          return false;
        }
        if (__atomic_load_n(f, __ATOMIC_ACQUIRE) != r.tag) {
          rc = hip_fail(hipErrorLaunchFailure);
          return false;
        }
        break;
      }
    }
    return true;
  }

  void request(int k, bool pre) {
    if (pub[k] >= 0 || filling[k] >= 0 || requested[k]) return;
    requested[k] = 1;
    req.push_back(pre ? (k | kPrefetchBit) : k);
  }

  // Counts one arrived pass: hits and misses against the map the pass saw;
  // requests the missed experts and, for each of the next `depth` layers,
  // the experts the prefetch rule predicts from this pass's.
  void account(const Rec& r) {
    const int E = shape.E;
    std::memcpy(act.data(), pin + size_t(r.entry) * entry_bytes + 8, size_t(E + 1) * 4);
    const int A = std::min(std::max(int(act[0]), 0), E);
    const int32_t* snap = &snaps[size_t(r.entry) * E];
    for (int j = 0; j < A; ++j) {
      const int e = act[1 + j];
      if (e < 0 || e >= E) continue;
      ++stats.lookups;
      const int k = r.layer * E + e;
      const int s = snap[e];
      if (s >= 0) {
        ++stats.hits;
        if (key[s] == k) {
          if (prefetched[s]) ++stats.prefetch_hits;
          prefetched[s] = 0;
          stamp[s] = ++clock;
        }
      } else {
        // a miss was read from host memory; the expert is copied in from its second miss on
        // (the frequently used experts stay resident, an expert met once costs no copy)
        ++stats.misses;
        if (missed[k] < 255) ++missed[k];
        if (missed[k] >= 2) request(k, false);
      }
    }
    for (int dd = 1; dd <= depth; ++dd) {
      const int l = (r.layer + dd) % n_layers;
      const int off = int(((long(dd) * shift) % E + E) % E);
      for (int j = 0; j < A; ++j) {
        const int e = act[1 + j];
        if (e >= 0 && e < E) request(l * E + (e + off) % E, true);
      }
    }
  }

  // Reads the arrived passes, oldest first; with `wait_all`, waits for all.
  int drain(bool wait_all, hipStream_t st) {
    size_t done = 0;
    for (; done < recs.size(); ++done) {
      int rc = MOE_OK;
      if (!arrived(recs[done], wait_all, st, rc)) {
        if (rc) return rc;
        break;
      }
      account(recs[done]);
    }
    recs.erase(recs.begin(), recs.begin() + long(done));
    return MOE_OK;
  }

  // ------------------------------------------------------------- slots --
  int victim() const {
    int best = -1;
    for (int i = 0; i < n_slots; ++i) {
      if (busy[i] || state[i] == kFilling) continue;
      if (state[i] == kFree) return i;
      if (best < 0 || stamp[i] < stamp[best]) best = i;
    }
    return best;
  }

  void add_seg(const void* src, void* dst, size_t bytes) {
    seg_src.push_back(src);
    seg_dst.push_back(dst);
    seg_bytes.push_back(bytes);
  }

  // Enqueues, in this order: a pending flush; the publication of completed
  // copies (on `st` the copies of layer `layer_now`'s experts are waited for
  // and published too); the requested copies, each into the least recently
  // used slot (unmapping its old expert); the map changes on `st`; the copies
  // on the copy stream, after every launch that could still read an unmapped slot.
  int update(hipStream_t st, int layer_now) {
    const int E = shape.E;
    map_idx.clear();
    map_val.clear();
    std::fill(busy.begin(), busy.end(), 0);
    if (flush_pending) {
      flush_pending = false;
      if (hipError_t e = moe::launch_map_clear(map, long(n_layers) * E, st)) return hip_fail(e);
      for (int i = 0; i < n_slots; ++i) {
        if (key[i] >= 0) {
          pub[key[i]] = -1;
          filling[key[i]] = -1;
        }
        if (state[i] != kFree) wait_release[i] = 1;
        key[i] = -1;
        state[i] = kFree;
        prefetched[i] = 0;
      }
    }
    for (int i = 0; i < n_slots; ++i) {
      if (state[i] != kFilling) continue;
      hipError_t q = hipEventQuery(ready[i]);
      if (q == hipErrorNotReady && key[i] / E == layer_now) {
        if (hipError_t e = hipStreamWaitEvent(st, ready[i], 0)) return hip_fail(e);
        q = hipSuccess;
      }
      if (q == hipErrorNotReady) continue;
      if (q != hipSuccess) return hip_fail(q);
      state[i] = kResident;
      filling[key[i]] = -1;
      pub[key[i]] = i;
      busy[i] = 1;
      map_idx.push_back(key[i]);
      map_val.push_back(i);
    }
    size_t taken = 0;
    for (; taken < req.size(); ++taken) {
      const int k = req[taken] & ~kPrefetchBit;
      const bool pre = (req[taken] & kPrefetchBit) != 0;
      if (pub[k] >= 0 || filling[k] >= 0) {
        requested[k] = 0;
        continue;
      }
      const int s = victim();
      if (s < 0) break;          // every slot is being filled or was just published: the rest waits
      requested[k] = 0;
      if (state[s] == kResident) {
        pub[key[s]] = -1;
        map_idx.push_back(key[s]);
        map_val.push_back(-1);
        wait_release[s] = 1;
      }
      key[s] = k;
      state[s] = kFilling;
      filling[k] = s;
      missed[k] = 0;
      prefetched[s] = pre;
      busy[s] = 1;
      stamp[s] = ++clock;
      if (pre) ++stats.prefetches;
      const int l = k / E, e = k % E;
      const void* src[3] = {host[l].w_gate, host[l].w_up, host[l].w_down};
      for (int m = 0; m < 3; ++m) {
        const Geom& g = geo.m[m];
        const uint8_t* h = static_cast<const uint8_t*>(src[m]);
        uint8_t* dst = stack(m);
        add_seg(h + size_t(e) * g.code(), dst + size_t(s) * g.code(), g.code());
        if (g.scale())
          add_seg(h + g.scale_offset(shape.E) + size_t(e) * g.scale(),
                  dst + g.scale_offset(n_slots) + size_t(s) * g.scale(), g.scale());
        stats.bytes_copied += g.code() + g.scale();
      }
      seg_slots.push_back(s);
    }
    req.erase(req.begin(), req.begin() + long(taken));
    for (size_t i = 0; i < map_idx.size(); i += moe::kMapMaxPairs) {
      const int n = int(std::min<size_t>(moe::kMapMaxPairs, map_idx.size() - i));
      if (hipError_t e = moe::launch_map_update(map, &map_idx[i], &map_val[i], n, st)) return hip_fail(e);
    }
    if (!seg_slots.empty()) {
      bool need = false;
      for (int s : seg_slots) need = need || wait_release[s];
      if (need) {
        if (hipError_t e = hipEventRecord(released, st)) return hip_fail(e);
        if (hipError_t e = hipStreamWaitEvent(copy, released, 0)) return hip_fail(e);
        for (int s : seg_slots) wait_release[s] = 0;
      }
      for (size_t i = 0; i < seg_src.size(); i += moe::kCopyMaxSegs) {
        const int n = int(std::min<size_t>(moe::kCopyMaxSegs, seg_src.size() - i));
        if (hipError_t e = moe::launch_gather_copy(&seg_src[i], &seg_dst[i], &seg_bytes[i], n, copy))
          return hip_fail(e);
      }
      for (int s : seg_slots)
        if (hipError_t e = hipEventRecord(ready[s], copy)) return hip_fail(e);
    }
    seg_src.clear();
    seg_dst.clear();
    seg_bytes.clear();
    seg_slots.clear();
    return MOE_OK;
  }

  // -------------------------------------------------------------- hooks --
  int before_pass(moe::DecodeArgs& d, hipStream_t st) override {
    if (int rc = drain(false, st)) return rc;
    if (recs.size() >= size_t(kRing)) {        // the ring is full: wait for the oldest pass
      int rc = MOE_OK;
      if (!arrived(recs.front(), true, st, rc)) return rc ? rc : hip_fail(hipErrorLaunchFailure);
      if (int rc2 = drain(false, st)) return rc2;
    }
    if (int rc = update(st, layer)) return rc;
    const int E = shape.E;
    const int entry = next_entry;
    next_entry = (next_entry + 1) % kRing;
    std::memcpy(&snaps[size_t(entry) * E], &pub[size_t(layer) * E], size_t(E) * 4);
    recs.push_back(Rec{++tag, layer, entry});
    d.wg = stack(0);
    d.wu = stack(1);
    d.wd = stack(2);
    d.slot_of = map + size_t(layer) * E;
    d.wg_h = static_cast<const uint8_t*>(host[layer].w_gate);
    d.wu_h = static_cast<const uint8_t*>(host[layer].w_up);
    d.wd_h = static_cast<const uint8_t*>(host[layer].w_down);
    d.E_w = n_slots;
    return MOE_OK;
  }

  int after_pass(const moe::DecodeArgs& d, hipStream_t st) override {
    const Rec& r = recs.back();
    uint8_t* ent = pin_dev + size_t(r.entry) * entry_bytes;
    if (hipError_t e = moe::launch_export_list(d.active, shape.E + 1, reinterpret_cast<int32_t*>(ent + 8),
                                               reinterpret_cast<unsigned long long*>(ent), r.tag, st))
      return hip_fail(e);
    if (depth > 0) {
      // prefetching: read this pass's experts now (the host waits while the GPU finishes the
      // pass) and start the copies they predict, so the copies overlap with what follows
      if (int rc = drain(true, st)) return rc;
      if (int rc = update(st, -1)) return rc;
    }
    return MOE_OK;
  }
};

extern "C" {

int moe_cache_region_bytes(const moe_shape_t* s, int32_t n_layers, int32_t n_slots, size_t* bytes) {
  if (!s || !bytes) return MOE_ERR_NULL;
  moe_shape_t t = *s;
  t.T = 1;
  t.path = MOE_PATH_DECODE;
  size_t ws = 0;
  if (int rc = moe_workspace_size(&t, &ws)) return rc;
  if (n_slots < 1 || n_slots > kMaxSlots || n_layers < 1 || n_layers > kMaxLayers) return MOE_ERR_SHAPE;
  *bytes = Geoms(s, n_layers, n_slots).total;
  return MOE_OK;
}

int moe_cache_create(const moe_shape_t* s, int32_t n_layers, const moe_host_experts_t* layers, void* region,
                     size_t region_bytes, int32_t n_slots, int32_t prefetch_depth, int32_t prefetch_shift,
                     void* copy_stream, moe_expert_cache_t** out) {
  if (!s || !layers || !region || !out) return MOE_ERR_NULL;
  *out = nullptr;
  size_t need = 0;
  if (int rc = moe_cache_region_bytes(s, n_layers, n_slots, &need)) return rc;
  if (prefetch_depth < 0 || prefetch_depth >= n_layers) return MOE_ERR_SHAPE;
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
  hipError_t r = hipHostMalloc(reinterpret_cast<void**>(&c->pin), size_t(kRing) * c->entry_bytes,
                               hipHostMallocCoherent);
  if (r == hipSuccess) r = hipHostGetDevicePointer(reinterpret_cast<void**>(&c->pin_dev), c->pin, 0);
  if (r == hipSuccess) {
    std::memset(c->pin, 0, size_t(kRing) * c->entry_bytes);
    r = hipEventCreateWithFlags(&c->released, hipEventDisableTiming);
  }
  for (int i = 0; i < n_slots && r == hipSuccess; ++i) r = hipEventCreateWithFlags(&c->ready[i], hipEventDisableTiming);
  // an empty map: every expert is read from the host until it has been copied in
  if (r == hipSuccess) r = moe::launch_map_clear(c->map, long(n_layers) * s->E, c->copy);
  if (r == hipSuccess) r = hipStreamSynchronize(c->copy);
  if (r != hipSuccess) {
    moe_cache_destroy(c);
    return hip_fail(r);
  }
  *out = c;
  return MOE_OK;
}

int moe_cache_destroy(moe_expert_cache_t* c) {
  if (!c) return MOE_ERR_NULL;
  const hipError_t r = hipStreamSynchronize(c->copy);
  for (hipEvent_t e : c->ready)
    if (e) (void)hipEventDestroy(e);
  if (c->released) (void)hipEventDestroy(c->released);
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
  c->layer = layer;
  return moe::forward_hooked(&t, x, router_w, router_b, c->stack(0), c->stack(1), c->stack(2), ws_gate, ws_up,
                             ws_down, out, workspace, ws_bytes, stream, c);
}

int moe_cache_stats(moe_expert_cache_t* c, moe_cache_stats_t* out, int32_t reset) {
  if (!c || !out) return MOE_ERR_NULL;
  if (int rc = c->drain(false, nullptr)) return rc;     // the passes whose lists have arrived
  *out = c->stats;
  if (reset) c->stats = moe_cache_stats_t{};
  return MOE_OK;
}

int moe_cache_flush(moe_expert_cache_t* c) {
  if (!c) return MOE_ERR_NULL;
  c->flush_pending = true;        // applied in stream order before the next call's launches
  for (int k : c->req) c->requested[k & ~kPrefetchBit] = 0;
  c->req.clear();
  return MOE_OK;
}

}  // extern "C"
