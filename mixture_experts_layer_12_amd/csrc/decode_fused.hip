// Single-launch decode: router logits, top-k and dispatch, shared and routed
// gate/up, down and the combine in one launch.
//
// Sources: "Fused MoE kernel on Triton: 5 launches vs 24" (ai-manual.ru),
// section "Fused kernel: one operation instead of twenty-four" (routing,
// dispatch, the expert computation and the aggregation as few launches with
// no intermediate round trips through the host); "Why MoE on RTX 5090 falls
// short: a bandwidth measurement" (news.malakhovai.ru), paragraphs on kernel
// launch overhead and on kernels that move too little per launch to reach
// full bandwidth -- a batch-1 layer reads only tens of MB, so every extra
// launch and every serial round trip is a visible share of its time.
// "llama.cpp: fusing shared experts into MMVQ" (ai-manual.ru), section "How
// fusing shared experts into MMVQ can speed up inference": the shared experts
// run in the same pass; here their gate/up tiles come before the top-k in the
// work list, so their weights stream while the routing is still being decided.
//
// Work list (fixed order, item i taken by work-group i mod G; G is at most
// what the GPU holds at once, see launch_fused_t):
//   [0, n_logit)                 router logits: 16 experts x 16 tokens x a quarter of H
//   [n_logit, end_shared_gu)     shared-expert gate/up row tiles
//   end_shared_gu                top-k, renormalisation, dispatch (one item)
//   [end_select, end_gu)         routed gate/up row tiles, slot-major
// With few assignments (route_in_gu) there is no selection item: each routed
// gate/up item waits for the logits and runs the few-assignment route itself
// (the first one also writes the routing tables, on which the routed down
// items then wait), so the routing latency is paid in parallel, not in
// series with one item's handoff.
//   [end_gu, end_down)           down row groups of kFusedDownRows outputs, slot-major (routed, then shared)
//   [end_down, n_items)          combine, 1024 outputs per item
// An item waits only on items of lower index, and every work-group takes its
// items in increasing order, so the lowest unfinished item can always run.
// Each item ends by storing the call's epoch into its flag after its own
// device-scope stores have completed; waits poll flags with device-scope
// loads and give up after a bounded number of rounds.  A wait that gives up
// stores the epoch into the error tag before its item signals; an item whose
// wait gave up, or that finds the error tag at this call's epoch after its
// waits, skips its body (it would read routing tables or activations that
// were never written in this call) and only signals.  Every item is an
// ancestor of every combine item, so once any wait has given up the combine
// writes NaN over the whole output, and the status pair in the workspace
// (this call's tag, stored by item 0; the error tag) holds two equal words
// after the call.  The same item functions serve the multi-launch kernels
// with ordinary memory accesses.
#include <algorithm>

#include "decode_items.hpp"
#include "router_items.hpp"

namespace moe {

constexpr int kFusedThreads = 256;

// Every flag in [lo, hi) equal to the epoch.  Wave 0 polls, 8 flags per lane
// per round from the first one it has not yet seen set (flags only move to
// the epoch during a call), for at most f.spin_rounds rounds.  Returns, the
// same for every thread, whether the item may run: its waits completed and
// no wait of this call has given up.
__device__ __forceinline__ bool wait_items(const FusedArgs& f, int lo, int hi) {
  __shared__ int s_run;
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    int cur = lo + lane;
    bool done = lo >= hi;
    for (int it = 0; !done && it < f.spin_rounds; ++it) {
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = cur + 64 * u;
        ok[u] = idx >= hi || __hip_atomic_load(f.flags + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == f.epoch;
      }
      int adv = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) adv += (adv == u && ok[u]) ? 1 : 0;
      cur += 64 * adv;
      done = __all(cur >= hi);
      if (done) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (!done && lane == 0) __hip_atomic_store(f.error, f.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // read after the flags: an item that gave up stored the tag before its flag
    const bool failed = __hip_atomic_load(f.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == f.epoch;
    if (lane == 0) s_run = (done && !failed) ? 1 : 0;
  }
  __syncthreads();
  const bool run = s_run != 0;
  __syncthreads();          // every wave has read s_run before a later wait rewrites it
  asm volatile("" ::: "memory");
  return run;
}

// Item i is complete: this thread's stores have reached memory (vmcnt counts
// stores on this architecture), then one thread publishes the flag.
__device__ __forceinline__ void signal_item(const FusedArgs& f, int i) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(f.flags + i, f.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Ints of the gate/up cross-wave sums (the few-assignment route of a routed
// gate/up item lives past them).
template <int NCT>
constexpr int kFusedGuInts = (kFusedThreads / 64) * 2 * NCT * 64 * 4;

template <int WT, int XT, int NCT>
__global__ void __launch_bounds__(kFusedThreads) decode_fused_kernel(FusedArgs f) {
  extern __shared__ __attribute__((aligned(16))) int smem[];
  const DecodeArgs a = f.d;
  auto* red_gu = reinterpret_cast<f32x4_t(*)[2 * NCT][64]>(smem);
  constexpr int RPW = kFusedDownRows<NCT> / 16;
  auto* red_dn = reinterpret_cast<f32x4_t(*)[RPW * NCT][64]>(smem);
  const int nrt_down = a.H / (16 * RPW);
  for (int i = blockIdx.x; i < f.n_items; i += gridDim.x) {
    if (i == 0 && threadIdx.x == 0) __hip_atomic_store(f.call_tag, f.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (i < f.n_logit) {      // one group of 4 chunks of one tile -> its partial plane
      const int tile = i >> 2, q = i & 3;
      logits_tile<XT, XT, true, 1>(f.r, tile % f.r.n_row_tiles, tile / f.r.n_row_tiles, 4 * q, 4,
                                reinterpret_cast<float*>(smem), f.r.rb.logits + size_t(q) * a.T * a.E);
    } else if (i < f.end_shared_gu) {
      const int j = i - f.n_logit;
      gateup_item<WT, XT, NCT, true>(a, j % f.gu_rt_shared, a.n_routed_slots + j / f.gu_rt_shared, red_gu);
    } else if (i < f.end_select) {
      if (wait_items(f, 0, f.n_logit)) switch (topk_mode(a.E, a.k)) {
        case kTopkT8: select_and_dispatch<true, kTopkT8>(f.r, f.r.rb.logits, false, smem); break;
        case kTopkT16: select_and_dispatch<true, kTopkT16>(f.r, f.r.rb.logits, false, smem); break;
        case kTopkT32: select_and_dispatch<true, kTopkT32>(f.r, f.r.rb.logits, false, smem); break;
        case kTopkRow16: select_and_dispatch<true, kTopkRow16>(f.r, f.r.rb.logits, false, smem); break;
        default: select_and_dispatch<true, kTopkWave>(f.r, f.r.rb.logits, false, smem); break;
      }
    } else if (i < f.end_gu) {
      const int j = i - f.end_select;
      if (f.route_in_gu) {
        // the item selects and dispatches from the logits into LDS past the cross-wave sums; the
        // first one (slot 0, row tile 0) also publishes the routing tables for the down items
        if (wait_items(f, 0, f.n_logit)) {
          const SmallRoute R(smem + kFusedGuInts<NCT>, a.T, a.E, a.k);
          int rk, fs;
          route_select_place<true>(f.r, f.r.rb.logits, false, R, j == 0, rk, fs, [] {});
          if (j == 0) small_tables<true>(f.r, R, rk, fs);
          gateup_item<WT, XT, NCT, true, true>(a, j % f.gu_rt_routed, j / f.gu_rt_routed, red_gu, 0, &R);
        }
      } else if (wait_items(f, f.end_shared_gu, f.end_select)) {
        gateup_item<WT, XT, NCT, true>(a, j % f.gu_rt_routed, j / f.gu_rt_routed, red_gu);
      }
    } else if (i < f.end_down) {
      const int j = i - f.end_gu;
      const int slot = j / nrt_down, rt = j % nrt_down;
      bool run;
      if (slot < a.n_routed_slots) {
        const int b = f.end_select + slot * f.gu_rt_routed;
        // the routing tables (with route_in_gu, published by the first routed gate/up item)
        const bool tables = f.route_in_gu ? wait_items(f, f.end_select, f.end_select + 1) : true;
        run = wait_items(f, b, b + f.gu_rt_routed) && tables;
      } else {
        const int b = f.n_logit + (slot - a.n_routed_slots) * f.gu_rt_shared;
        run = wait_items(f, b, b + f.gu_rt_shared);
      }
      if (run) down_item<WT, NCT, true, RPW>(a, rt, slot, red_dn);
    } else {
      const bool run = wait_items(f, f.end_gu, f.end_down);
      const long i4 = long(i - f.end_down) * kFusedThreads + threadIdx.x;
      if (!run) {
        if (i4 < long(a.T) * (a.H / 4)) {
          const float nan = __builtin_nanf("");
          if constexpr (XT == DT_F32) reinterpret_cast<f32x4_t*>(a.out)[i4] = f32x4_t{nan, nan, nan, nan};
          else reinterpret_cast<u32x2_t*>(a.out)[i4] = u32x2_t{0x7fc07fc0u, 0x7fc07fc0u};
        }
      } else {
        combine_item<XT, true>(a, i4);
      }
    }
    signal_item(f, i);
  }
}

// LDS of one work-group: the largest of the logits reduction, the selection
// and dispatch scratch, and the gate/up and down cross-wave sums.
size_t fused_lds_bytes(int E, int T, int k, int nct) {
  const int NW = kFusedThreads / 64;
  const size_t logits = size_t(NW) * 64 * 4 * sizeof(float);
  const int n = T * k;
  const int ch = std::max(1, kRouterStage / E);
  const size_t select = (size_t(router_disp_ints(NW, E)) + (n <= kRouterIdsLds ? n : 0) + size_t(std::min(T, ch)) * E) *
                        sizeof(int);
  const size_t gu = size_t(NW) * 2 * nct * 64 * sizeof(f32x4_t);
  const size_t route = gu + size_t(small_route_max_ints(kFusedThreads)) * sizeof(int);   // route_in_gu items
  return std::max(std::max(logits, select), route);
}

template <int WT, int XT, int NCT>
static hipError_t launch_fused_t(FusedArgs f, hipStream_t st) {
  const void* kern = reinterpret_cast<const void*>(decode_fused_kernel<WT, XT, NCT>);
  // One fixed LDS size per instantiation (the largest any shape of the
  // single-launch path needs), so the resident grid is computed once.
  static const size_t lds = fused_lds_bytes(256, 64, 16, NCT);
  static int resident = [&] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFusedThreads, lds) != hipSuccess) return 0;
    return cus * std::min(per_cu, 2);
  }();
  if (resident <= 0) return hipErrorInvalidConfiguration;
  const int grid = std::min(resident, f.n_items);
  // An ordinary launch: a cooperative one guarantees the co-residency that
  // the waits rely on but costs about 19 us per call here (measured on the
  // Qwen-A3B shape: 61.6 -> 42.4 us), a third of the layer.  The grid never
  // exceeds what the GPU holds at once, so an otherwise idle GPU dispatches
  // all of it immediately; work-groups held back by other kernels start as
  // those finish (which never wait on this one); and every wait is bounded,
  // after which the call marks its output NaN instead of hanging.
  hipLaunchKernelGGL((decode_fused_kernel<WT, XT, NCT>), dim3(grid), dim3(kFusedThreads), lds, st, f);
  return hipGetLastError();
}

template <int WT, int XT>
static hipError_t launch_fused_x(const FusedArgs& f, hipStream_t st) {
  return f.d.T <= 16 ? launch_fused_t<WT, XT, 1>(f, st) : launch_fused_t<WT, XT, 4>(f, st);
}

// Router and activations share one dtype on this path (x_dtype == router dtype).
hipError_t launch_decode_fused(const FusedArgs& f, int wdt, int xdt, hipStream_t st) {
  if (wdt == DT_F32) return xdt == DT_F32 ? launch_fused_x<DT_F32, DT_F32>(f, st) : launch_fused_x<DT_F32, DT_BF16>(f, st);
  if (wdt == DT_BF16)
    return xdt == DT_F32 ? launch_fused_x<DT_BF16, DT_F32>(f, st) : launch_fused_x<DT_BF16, DT_BF16>(f, st);
  if (wdt == DT_Q4)
    return xdt == DT_F32 ? launch_fused_x<DT_Q4, DT_F32>(f, st) : launch_fused_x<DT_Q4, DT_BF16>(f, st);
  return hipErrorInvalidValue;       // the 8-bit weight types run the multi-launch decode only
}

}  // namespace moe
