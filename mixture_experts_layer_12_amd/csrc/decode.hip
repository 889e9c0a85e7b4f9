// Decode path: the multi-launch kernels (gate/up, down, combine) built from
// the work items of decode_items.hpp.
#include "decode_items.hpp"

namespace moe {

void launch_router_select(const RouterArgs& a, hipStream_t st);   // router.hip
size_t router_lds_bytes(int NW, int E, int n, bool stage);         // router.hip

// ------------------------------------------------------------- kernels --

// Slot of a work-group row: the shared experts' rows of the grid come first,
// so that their work-groups (every token, hence the most columns) start with
// the first wave of the grid instead of forming its tail.
__device__ __forceinline__ int grid_slot(const DecodeArgs& a) {
  const int y = blockIdx.y;
  return y < a.S ? a.n_routed_slots + y : y - a.S;
}

// Slot of a gate/up work-group row: as grid_slot, or the routed slots only
// when the shared experts' gate/up ran in the logits launch.
__device__ __forceinline__ int gu_slot(const DecodeArgs& a) {
  return a.shared_in_router ? int(blockIdx.y) : grid_slot(a);
}

// PASSES: slots with more tokens than the NCT column tiles take further
// passes over the same weight rows (served from cache); without, one pass
// (every slot fits: the loop would only cost registers).
// PRO: a.route_in_gu; every routed work-group first selects and dispatches
// from the logits in LDS (dynamic LDS of small_route_ints(256, ...) ints) and
// takes its slot's routing from there; the one of slot 0, row tile 0 also
// writes the routing tables for the down launch.  One pass.  Here the routed
// slots' rows of the grid come first: a grid slightly larger than the CU
// count puts its last rows on CUs that already hold a work-group, and two
// routing prologues sharing a CU take twice as long (the shared experts'
// work-groups, which do not route, absorb that instead).
// XS (with PRO, fp16-operand families): the activations [T, H] are staged
// into LDS as fp16 past the routing region, their loads issued before the
// routing's (they do not depend on it) and stored once the selection is done.
template <int WT, int XT, int NCT, bool PASSES, bool PRO, bool XS = false>
__global__ void __launch_bounds__(256) decode_gateup_kernel(DecodeArgs a) {
  __shared__ f32x4_t red[4][2 * NCT][64];
  const int slot = PRO ? int(blockIdx.y) : gu_slot(a);
  if constexpr (PRO) {
    extern __shared__ __attribute__((aligned(16))) int lds[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds + small_route_ints(256, a.route.T, a.route.E, a.route.k));
    const int n8 = a.T * a.H / 8;
    XStage<XT> xst;
    if constexpr (XS) xst = stage_x_load<XT>(a.x, n8);
    if (slot < a.n_routed_slots) {
      const SmallRoute R(lds, a.route.T, a.route.E, a.route.k);
      const bool writer = blockIdx.x == 0 && slot == 0;
      int rk, fslot;
      route_select_place<false>(a.route, a.route.rb.logits, false, R, writer, rk, fslot, [&] {
        if constexpr (XS) stage_x_store<XT>(xst, n8, xs);
      });
      if (writer) small_tables<false>(a.route, R, rk, fslot);
      gateup_item<WT, XT, NCT, false, true, XS>(a, blockIdx.x, slot, red, 0, &R, xs);
      return;
    }
    if constexpr (XS) {
      stage_x_store<XT>(xst, n8, xs);
      __syncthreads();
      gateup_item<WT, XT, NCT, false, false, XS>(a, blockIdx.x, slot, red, 0, nullptr, xs);
      return;
    }
  }
  if constexpr (PASSES) {
    for (int c0 = 0; gateup_item<WT, XT, NCT, false>(a, blockIdx.x, slot, red, c0); c0 += 16 * NCT) __syncthreads();
  } else {
    gateup_item<WT, XT, NCT, false>(a, blockIdx.x, slot, red);
  }
}

// Router logits and the shared experts' gate/up in one launch (route_in_gu
// with shared experts): the shared rows do not depend on the routing, so
// they stream while the logits are computed, and the routed gate/up launch
// that follows needs one work-group per routed row tile only.  Work-groups
// [0, 4 * tiles) compute the logits (four partial planes per 16 x 16 tile,
// as router_logits_kernel), the rest one shared row tile each; the grid also
// clears route.zero_f32.  XS: the shared work-groups stage the activations.
// SNCT: 16-token column tiles of the shared rows (4 for more than 16 tokens:
// the shared weight rows are read once for every token).  SEL: the last
// work-group selects and dispatches once every logit work-group has
// published its planes (device-scope stores, then its flag at the call's
// epoch); it waits at most a.sel_spin polling rounds, and after a wait that
// gave up it stores the epoch into the error word and still selects from the
// logits as they are (the routing tables stay well formed, the output is then
// not valid).
template <int RT, int WT, int XT, bool XS, int SNCT = 1, bool SEL = false>
__global__ void __launch_bounds__(256) decode_router_shared_kernel(DecodeArgs a) {
  __shared__ f32x4_t red[4][2 * SNCT][64];
  extern __shared__ __attribute__((aligned(16))) int lds[];
  const RouterArgs& r = a.route;
  if (r.zero_f32) {
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < r.zero_n / 4; i += long(gridDim.x) * blockDim.x)
      reinterpret_cast<f32x4_t*>(r.zero_f32)[i] = z;
  }
  const int n_logit = 4 * r.n_row_tiles * r.n_col_tiles;
  if (int(blockIdx.x) < n_logit) {
    const int tile = blockIdx.x >> 2, q = blockIdx.x & 3;
    logits_tile<RT, XT, SEL, 1>(r, tile % r.n_row_tiles, tile / r.n_row_tiles, 4 * q, 4,
                                reinterpret_cast<float*>(lds), r.rb.logits + size_t(q) * r.T * r.E);
    if constexpr (SEL) {          // the planes have reached memory, then the flag
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_store(a.sel_flags + blockIdx.x, a.sel_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if constexpr (SEL) {
    if (blockIdx.x == gridDim.x - 1) {
      __shared__ int s_ok;
      if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        if (lane == 0) __hip_atomic_store(a.sel_status, a.sel_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bool done = false;
        for (int it = 0; it < a.sel_spin && !done; ++it) {
          bool mine = true;
          for (int i = lane; i < n_logit; i += 64)
            mine = mine && __hip_atomic_load(a.sel_flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.sel_epoch;
          done = __all(mine);
          if (!done) __builtin_amdgcn_s_sleep(2);
        }
        if (lane == 0) {
          s_ok = done ? 1 : 0;
          if (!done) __hip_atomic_store(a.sel_status + 1, a.sel_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
      (void)s_ok;
      switch (topk_mode(r.E, r.k)) {
        case kTopkT8: select_and_dispatch<true, kTopkT8>(r, r.rb.logits, false, lds); break;
        case kTopkT16: select_and_dispatch<true, kTopkT16>(r, r.rb.logits, false, lds); break;
        case kTopkT32: select_and_dispatch<true, kTopkT32>(r, r.rb.logits, false, lds); break;
        case kTopkRow16: select_and_dispatch<true, kTopkRow16>(r, r.rb.logits, false, lds); break;
        default: select_and_dispatch<true, kTopkWave>(r, r.rb.logits, false, lds); break;
      }
      return;
    }
  }
  const int j = blockIdx.x - n_logit, gu_rt = (a.Is + 15) / 16;
  const int slot = a.n_routed_slots + j / gu_rt, rt = j % gu_rt;
  if constexpr (XS) {
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
    const int n8 = a.T * a.H / 8;
    stage_x_store<XT>(stage_x_load<XT>(a.x, n8), n8, xs);
    __syncthreads();
    gateup_item<WT, XT, 1, false, false, true>(a, rt, slot, red, 0, nullptr, xs);
  } else {
    for (int c0 = 0; gateup_item<WT, XT, SNCT, false>(a, rt, slot, red, c0); c0 += 16 * SNCT) __syncthreads();
  }
}

// OT >= 0: with the combine epilogue, outputs of dtype OT (partials stored
// with device-scope stores); OT < 0: partials only.
// Work-group (x, slot): k range x / n_rt of row group x % n_rt.
// NW waves split each k range (4, or 8 for large grids of two-row-tile
// work-groups).
template <int WT, int NCT, int RPW, int OT, bool PASSES, int NW = 4>
__global__ void __launch_bounds__(64 * NW) decode_down_kernel(DecodeArgs a) {
  __shared__ f32x4_t red[NW][RPW * NCT][64];
  const int slot = grid_slot(a);
  const int n_rt = a.H / (16 * RPW);
  const int rt = blockIdx.x % n_rt, kr = blockIdx.x / n_rt;
  if constexpr (PASSES) {
    for (int c0 = 0; down_item<WT, NCT, false, RPW, (OT >= 0), NW>(a, rt, slot, red, c0, kr, a.dn_ksplit);
         c0 += 16 * NCT)
      __syncthreads();
  } else {
    down_item<WT, NCT, false, RPW, (OT >= 0), NW>(a, rt, slot, red, 0, kr, a.dn_ksplit);
  }
  if constexpr (OT >= 0) down_combine<OT>(a, rt, slot, RPW * 16);
}

// Row tiles per work-group and k ranges come with the arguments
// (decode_down_shape, chosen by the host, which sizes the partial planes).
// The launch also requests MOE_DN_LDS_PAD bytes of LDS it does not use:
// with at most 16 KiB of its own that caps the kernel at 3 work-groups per
// CU.  Fewer concurrent weight streams per CU read HBM faster here (the
// Mixtral-shaped batch of 8: 4 per CU 179 us, 3 per CU 176, 2 per CU 171,
// 1 per CU 200, before the other down settings above).  Eight-wave
// work-groups (dn_waves 8) are capped at two per CU (three: 160 us, two:
// 159, one: 167, against 164 with four waves).
#ifndef MOE_DN_LDS_PAD
#define MOE_DN_LDS_PAD 36864
#endif
#ifndef MOE_DN_W8_LDS_PAD
#define MOE_DN_W8_LDS_PAD 61440            // eight-wave work-groups: 16 KiB of their own, two per CU
#endif
template <int WT, int NCT, int OT, bool PASSES>
static void launch_down(const DecodeArgs& a, int n_slots, hipStream_t st) {
  const dim3 b(256);
  const size_t pad = MOE_DN_LDS_PAD;
  if constexpr (NCT == 1) {
    if (a.dn_rpw == 2 && a.dn_waves == 8) {   // eight waves; the padding keeps two work-groups per CU
      hipLaunchKernelGGL((decode_down_kernel<WT, 1, 2, OT, PASSES, 8>), dim3(a.H / 32 * a.dn_ksplit, n_slots), dim3(512),
                         size_t(MOE_DN_W8_LDS_PAD), st, a);
      return;
    }
  }
  if (NCT == 1 && a.dn_rpw == 4)
    hipLaunchKernelGGL((decode_down_kernel<WT, NCT, 4, OT, PASSES>), dim3(a.H / 64 * a.dn_ksplit, n_slots), b, pad, st, a);
  else if (NCT == 1 && a.dn_rpw == 2)
    hipLaunchKernelGGL((decode_down_kernel<WT, NCT, 2, OT, PASSES>), dim3(a.H / 32 * a.dn_ksplit, n_slots), b, pad, st, a);
  else
    hipLaunchKernelGGL((decode_down_kernel<WT, NCT, 1, OT, PASSES>), dim3(a.H / 16 * a.dn_ksplit, n_slots), b, pad, st, a);
}

// One token: a work-group per 16 output rows over every slot (down_one_item),
// the activation rows staged in dynamic LDS.
template <int WT, int OT>
__global__ void __launch_bounds__(256) decode_down_one_kernel(DecodeArgs a) {
  __shared__ f32x4_t red[4][64];
  extern __shared__ __attribute__((aligned(16))) uint8_t hs[];
  down_one_item<WT, OT>(a, blockIdx.x, hs, red);
}

// Whether the one-token down (decode_down_one_kernel) applies, and its LDS.
template <int WT>
static bool down_one_fits(const DecodeArgs& a, size_t& lds) {
  if constexpr (WT == DT_FP8) {
    return false;
  } else {
    if (a.T != 1 || a.H % 16 || (a.S > 0 && a.Is != a.I)) return false;
    const int len = (n_steps<WT>(a.I) + 3) / 4;
    lds = size_t(a.k + a.S) * a.h_stride * h_elem_bytes<WT>() * h_planes<WT>();
    return (a.k + a.S) * len <= kDownOneLoads && lds <= 48 * 1024;
  }
}

template <int OT>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeArgs a) {
  combine_item<OT, false>(a, long(blockIdx.x) * blockDim.x + threadIdx.x);
}

// -------------------------------------------------------------- launch --

// With a.dn_count the combine runs in the down launch's epilogue; without,
// in a launch of its own.
template <int RT, int WT, int XT>
static void launch_router_shared(const DecodeArgs& a, bool stage, hipStream_t st) {
  const int grid = 4 * a.route.n_row_tiles * a.route.n_col_tiles + a.S * ((a.Is + 15) / 16);
  const size_t logit_lds = size_t(4) * 64 * 4 * sizeof(float);
  const size_t x_lds = size_t(a.T) * a.H * 2;
  if (a.T > 16) {
    if (a.sel_flags) {            // one more work-group selects and dispatches
      static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(decode_router_shared_kernel<RT, WT, XT, false, 4, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  int(router_lds_bytes(4, 256, kRouterIdsLds, true)));
        return true;
      }();
      (void)attr;
      const size_t sel_lds = router_lds_bytes(4, a.E, a.T * a.k, true);
      hipLaunchKernelGGL((decode_router_shared_kernel<RT, WT, XT, false, 4, true>), dim3(grid + 1), dim3(256),
                         sel_lds > logit_lds ? sel_lds : logit_lds, st, a);
    } else {
      hipLaunchKernelGGL((decode_router_shared_kernel<RT, WT, XT, false, 4>), dim3(grid), dim3(256), logit_lds, st, a);
    }
    return;
  }
  if (a.sel_flags) {              // one column tile per shared row, one more work-group selects
    static const bool attr = [] {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(decode_router_shared_kernel<RT, WT, XT, false, 1, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(router_lds_bytes(4, 256, kRouterIdsLds, true)));
      return true;
    }();
    (void)attr;
    const size_t sel_lds = router_lds_bytes(4, a.E, a.T * a.k, true);
    hipLaunchKernelGGL((decode_router_shared_kernel<RT, WT, XT, false, 1, true>), dim3(grid + 1), dim3(256),
                       sel_lds > logit_lds ? sel_lds : logit_lds, st, a);
    return;
  }
  if constexpr (Fam<WT>::v == DT_Q4) {
    if (stage) {
      hipLaunchKernelGGL((decode_router_shared_kernel<RT, WT, XT, true>), dim3(grid), dim3(256),
                         logit_lds > x_lds ? logit_lds : x_lds, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((decode_router_shared_kernel<RT, WT, XT, false>), dim3(grid), dim3(256), logit_lds, st, a);
}

template <int WT, int XT, int NCT, bool PASSES>
static void launch_decode_t(const DecodeArgs& a, int rdt, int n_gu_row_tiles, hipStream_t st, StageMarker* mark) {
  constexpr bool fp16_family = Fam<WT>::v == DT_Q4;
  // activations staged in LDS: at most kStageX8 rounds of 8 values per thread
  const bool stage = fp16_family && long(a.T) * a.H <= long(kStageX8) * 256 * 8;
  // the shared experts' gate/up in the logits launch; without the routing in
  // the gate/up prologue the selection and dispatch follow in a launch of
  // their own
  const bool srouter = NCT == 1 && a.shared_in_router;
  if (srouter) {
    if (rdt == DT_F32) launch_router_shared<DT_F32, WT, XT>(a, stage && a.route_in_gu, st);
    else launch_router_shared<DT_BF16, WT, XT>(a, stage && a.route_in_gu, st);
    if (!a.route_in_gu && !a.sel_flags) launch_router_select(a.route, st);
    if (mark) mark->mark(st);
  }
  dim3 g1(n_gu_row_tiles, a.n_routed_slots + (srouter ? 0 : a.S)), b(256);
  const size_t route_lds = size_t(small_route_ints(256, a.T, a.E, a.k)) * 4;
  if (NCT == 1 && !PASSES && a.route_in_gu && stage)
    hipLaunchKernelGGL((decode_gateup_kernel<WT, XT, 1, false, true, fp16_family>), g1, b,
                       route_lds + size_t(a.T) * a.H * 2, st, a);
  else if (NCT == 1 && !PASSES && a.route_in_gu)
    hipLaunchKernelGGL((decode_gateup_kernel<WT, XT, 1, false, true>), g1, b, route_lds, st, a);
  else
    hipLaunchKernelGGL((decode_gateup_kernel<WT, XT, NCT, PASSES, false>), g1, b, 0, st, a);
  if (mark) mark->mark(st);
  size_t one_lds = 0;
  bool one = false;
  if constexpr (NCT == 1 && !PASSES && WT != DT_FP8) {
    if (down_one_fits<WT>(a, one_lds)) {
      hipLaunchKernelGGL((decode_down_one_kernel<WT, XT>), dim3(a.H / 16), b, one_lds, st, a);
      one = true;
    }
  }
  if (one) {
  } else if (a.dn_count) {
    launch_down<WT, NCT, XT, PASSES>(a, a.n_routed_slots + a.S, st);
  } else {
    launch_down<WT, NCT, -1, PASSES>(a, a.n_routed_slots + a.S, st);
    const long n4 = long(a.T) * a.H / 4;
    hipLaunchKernelGGL((decode_combine_kernel<XT>), dim3(int((n4 + 255) / 256)), b, 0, st, a);
  }
  if (mark) mark->mark(st);
}

// One 16-token column tile per pass unless the routed slots average more than
// 8 tokens (decode_one_col_tile): the one-tile kernels keep more weight bytes
// in flight per wave, and the rare slot with more tokens takes another pass.
template <int WT, int XT>
static void launch_decode_x(const DecodeArgs& a, int rdt, int n_gu_row_tiles, hipStream_t st, StageMarker* mark) {
  if (a.T <= 16) launch_decode_t<WT, XT, 1, false>(a, rdt, n_gu_row_tiles, st, mark);
  else if (decode_one_col_tile(a.T, a.k, a.E)) launch_decode_t<WT, XT, 1, true>(a, rdt, n_gu_row_tiles, st, mark);
  else launch_decode_t<WT, XT, 4, false>(a, rdt, n_gu_row_tiles, st, mark);
}

// Gate/up and down of the shared experts only (a.n_routed_slots must be 0):
// rows T*k + s*T + t of h and of the partials, as in the full decode pass.
template <int WT, int XT, int NCT>
static void launch_shared_t(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_gateup_kernel<WT, XT, NCT, false, false>), dim3(a.n_row_tiles, a.S), dim3(256), 0, st, a);
  launch_down<WT, NCT, -1, false>(a, a.S, st);
}

template <int WT, int XT>
static void launch_shared_x(const DecodeArgs& a, hipStream_t st) {
  if (a.T <= 16) launch_shared_t<WT, XT, 1>(a, st);
  else launch_shared_t<WT, XT, 4>(a, st);
}

hipError_t launch_decode_shared(const DecodeArgs& a, int wdt, int xdt, hipStream_t st) {
  if (a.S == 0) return hipSuccess;
  if (a.n_routed_slots != 0 || a.dn_count || a.route_in_gu) return hipErrorInvalidValue;
  if (wdt == DT_F32) {
    if (xdt == DT_F32) launch_shared_x<DT_F32, DT_F32>(a, st);
    else launch_shared_x<DT_F32, DT_BF16>(a, st);
  } else if (wdt == DT_BF16) {
    if (xdt == DT_F32) launch_shared_x<DT_BF16, DT_F32>(a, st);
    else launch_shared_x<DT_BF16, DT_BF16>(a, st);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int wdt, int xdt, int rdt, int n_gu_row_tiles, hipStream_t st,
                         StageMarker* mark) {
  if (a.route_in_gu && (a.T > 16 || !small_route(a.T, a.E, a.k) || a.route.tile_m != 1)) return hipErrorInvalidValue;
  if (a.slot_of && (a.E_w < 1 || !a.wg_h || !a.wu_h || !a.wd_h)) return hipErrorInvalidValue;
  if (a.shared_in_router &&
      (a.S == 0 || a.route.logit_parts != 4 || !decode_one_col_tile(a.T, a.k, a.E) || (a.route_in_gu && a.T > 16)))
    return hipErrorInvalidValue;
  if (a.sel_flags && (!a.shared_in_router || a.route_in_gu || !a.sel_status)) return hipErrorInvalidValue;
  if (a.dn_ksplit < 1 || a.dn_ksplit > kDownMaxKs || (a.dn_rpw != 1 && a.dn_rpw != 2 && a.dn_rpw != 4) ||
      a.H % (16 * a.dn_rpw) != 0)
    return hipErrorInvalidValue;
  if (wdt == DT_F32) {
    if (xdt == DT_F32) launch_decode_x<DT_F32, DT_F32>(a, rdt, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_F32, DT_BF16>(a, rdt, n_gu_row_tiles, st, mark);
  } else if (wdt == DT_BF16) {
    if (xdt == DT_F32) launch_decode_x<DT_BF16, DT_F32>(a, rdt, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_BF16, DT_BF16>(a, rdt, n_gu_row_tiles, st, mark);
  } else if (wdt == DT_Q4) {
    if (xdt == DT_F32) launch_decode_x<DT_Q4, DT_F32>(a, rdt, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_Q4, DT_BF16>(a, rdt, n_gu_row_tiles, st, mark);
  } else if (wdt == DT_Q8) {
    if (xdt == DT_F32) launch_decode_x<DT_Q8, DT_F32>(a, rdt, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_Q8, DT_BF16>(a, rdt, n_gu_row_tiles, st, mark);
  } else if (wdt == DT_FP8) {
    if (xdt == DT_F32) launch_decode_x<DT_FP8, DT_F32>(a, rdt, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_FP8, DT_BF16>(a, rdt, n_gu_row_tiles, st, mark);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Host-to-device copies of expert matrices by the GPU itself: work-group b
// copies 64 KiB chunk b of the concatenated segments (16-byte loads from
// device-mapped pinned host memory, 16 in flight per thread), so one launch
// keeps PCIe busy however small each segment is.
struct CopySeg {
  const uint8_t* src;   // device-mapped pinned host memory
  uint8_t* dst;
  unsigned long long bytes;   // multiple of 16; src and dst 16-byte aligned
  unsigned long long chunk0;  // first chunk of this segment
};
struct CopyList {
  int n;
  CopySeg s[kCopyMaxSegs];
};

constexpr int kCopyChunk = 65536;

__global__ void __launch_bounds__(256) gather_copy_kernel(CopyList l) {
  const unsigned long long b = blockIdx.x;
  int i = 0;
  while (i + 1 < l.n && l.s[i + 1].chunk0 <= b) ++i;
  const CopySeg sg = l.s[i];
  const unsigned long long off = (b - sg.chunk0) * kCopyChunk;
  if (off >= sg.bytes) return;
  const unsigned long long len = sg.bytes - off < kCopyChunk ? sg.bytes - off : kCopyChunk;
  const int n16 = int(len / 16);
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(sg.src + off);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(sg.dst + off);
  u32x4_t v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int q = j * 256 + int(threadIdx.x);
    if (q < n16) v[j] = __builtin_nontemporal_load(src + q);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int q = j * 256 + int(threadIdx.x);
    if (q < n16) dst[q] = v[j];
  }
}

hipError_t launch_gather_copy(const void* const* src, void* const* dst, const size_t* bytes, int n, hipStream_t st) {
  if (n < 1 || n > kCopyMaxSegs) return hipErrorInvalidValue;
  CopyList l;
  l.n = n;
  unsigned long long chunks = 0;
  for (int i = 0; i < n; ++i) {
    if (bytes[i] % 16 || reinterpret_cast<uintptr_t>(src[i]) % 16 || reinterpret_cast<uintptr_t>(dst[i]) % 16)
      return hipErrorInvalidValue;
    l.s[i] = CopySeg{static_cast<const uint8_t*>(src[i]), static_cast<uint8_t*>(dst[i]), bytes[i], chunks};
    chunks += (bytes[i] + kCopyChunk - 1) / kCopyChunk;
  }
  if (chunks == 0) return hipSuccess;
  if (chunks > 0x7fffffffull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_copy_kernel, dim3(unsigned(chunks)), dim3(256), 0, st, l);
  return hipGetLastError();
}

// A pass's active list written to (device-mapped, fine-grained) pinned host
// memory, then `tag` into *flag once every element is visible to the host.
__global__ void __launch_bounds__(256) export_list_kernel(const int32_t* src, int n, int32_t* dst,
                                                          unsigned long long* flag, unsigned long long tag) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_export_list(const int32_t* src, int n, int32_t* dst, unsigned long long* flag,
                              unsigned long long tag, hipStream_t st) {
  hipLaunchKernelGGL(export_list_kernel, dim3(1), dim3(256), 0, st, src, n, dst, flag, tag);
  return hipGetLastError();
}

// Slot-map updates of the expert cache, in stream order: entry idx[i] of
// `map` becomes val[i] (indices distinct within one launch), or every entry
// becomes -1.
struct MapPairs {
  int n;
  int32_t idx[kMapMaxPairs];
  int32_t val[kMapMaxPairs];
};

__global__ void __launch_bounds__(256) map_update_kernel(int32_t* map, MapPairs p) {
  for (int i = threadIdx.x; i < p.n; i += blockDim.x) map[p.idx[i]] = p.val[i];
}

__global__ void __launch_bounds__(256) map_clear_kernel(int32_t* map, long n) {
  for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += long(gridDim.x) * blockDim.x) map[i] = -1;
}

hipError_t launch_map_update(int32_t* map, const int32_t* idx, const int32_t* val, int n, hipStream_t st) {
  if (n < 0 || n > kMapMaxPairs) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  MapPairs p;
  p.n = n;
  for (int i = 0; i < n; ++i) {
    p.idx[i] = idx[i];
    p.val[i] = val[i];
  }
  hipLaunchKernelGGL(map_update_kernel, dim3(1), dim3(256), 0, st, map, p);
  return hipGetLastError();
}

hipError_t launch_map_clear(int32_t* map, long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long blocks = std::min<long>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(map_clear_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, map, n);
  return hipGetLastError();
}

}  // namespace moe
