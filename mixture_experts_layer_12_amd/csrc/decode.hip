// Decode path: the multi-launch kernels (gate/up, down, combine) built from
// the work items of decode_items.hpp.
#include "decode_items.hpp"

namespace moe {

// ------------------------------------------------------------- kernels --

// Slot of a work-group row: the shared experts' rows of the grid come first,
// so that their work-groups (every token, hence the most columns) start with
// the first wave of the grid instead of forming its tail.
__device__ __forceinline__ int grid_slot(const DecodeArgs& a) {
  const int y = blockIdx.y;
  return y < a.S ? a.n_routed_slots + y : y - a.S;
}

// PASSES: slots with more tokens than the NCT column tiles take further
// passes over the same weight rows (served from cache); without, one pass
// (every slot fits: the loop would only cost registers).
// PRO: a.route_in_gu; every routed work-group first selects and dispatches
// from the logits in LDS (dynamic LDS of small_route_ints(256, ...) ints) and
// takes its slot's routing from there; the one of slot 0, row tile 0 also
// writes the routing tables for the down launch.  One pass.
template <int WT, int XT, int NCT, bool PASSES, bool PRO>
__global__ void __launch_bounds__(256) decode_gateup_kernel(DecodeArgs a) {
  __shared__ f32x4_t red[4][2 * NCT][64];
  const int slot = grid_slot(a);
  if constexpr (PRO) {
    extern __shared__ __attribute__((aligned(16))) int lds[];
    if (slot < a.n_routed_slots) {
      const SmallRoute R(lds, a.route.T, a.route.E, a.route.k);
      const bool writer = blockIdx.x == 0 && slot == 0;
      int rk, fslot;
      small_select<false>(a.route, a.route.rb.logits, false, R);
      small_place<false>(a.route, R, writer, rk, fslot);
      if (writer) small_tables<false>(a.route, R, rk, fslot);
      gateup_item<WT, XT, NCT, false, true>(a, blockIdx.x, slot, red, 0, &R);
      return;
    }
  }
  if constexpr (PASSES) {
    for (int c0 = 0; gateup_item<WT, XT, NCT, false>(a, blockIdx.x, slot, red, c0); c0 += 16 * NCT) __syncthreads();
  } else {
    gateup_item<WT, XT, NCT, false>(a, blockIdx.x, slot, red);
  }
}

// OT >= 0: with the combine epilogue, outputs of dtype OT (partials stored
// with device-scope stores); OT < 0: partials only.
template <int WT, int NCT, int RPW, int OT, bool PASSES>
__global__ void __launch_bounds__(256) decode_down_kernel(DecodeArgs a) {
  __shared__ f32x4_t red[4][RPW * NCT][64];
  const int slot = grid_slot(a);
  if constexpr (PASSES) {
    for (int c0 = 0; down_item<WT, NCT, false, RPW, (OT >= 0)>(a, blockIdx.x, slot, red, c0); c0 += 16 * NCT)
      __syncthreads();
  } else {
    down_item<WT, NCT, false, RPW, (OT >= 0)>(a, blockIdx.x, slot, red);
  }
  if constexpr (OT >= 0) down_combine<OT>(a, blockIdx.x, slot, RPW * 16);
}

// Row tiles of 16 outputs per down-projection work-group when the token
// columns fit one MFMA tile (the tiles share every activation load): four
// while that still leaves at least 2048 work-groups, else two (fewer
// work-groups starve the memory stream).
#ifndef MOE_DN_RPW
#define MOE_DN_RPW 4
#endif
template <int WT, int NCT, int OT, bool PASSES>
static void launch_down(const DecodeArgs& a, int n_slots, hipStream_t st) {
  constexpr int R = NCT == 1 ? MOE_DN_RPW : 1;
  if (R >= 4 && a.H % 64 == 0 && (a.H / 64) * n_slots >= 2048)
    hipLaunchKernelGGL((decode_down_kernel<WT, NCT, R, OT, PASSES>), dim3(a.H / 64, n_slots), dim3(256), 0, st, a);
  else if (R >= 2 && a.H % 32 == 0)
    hipLaunchKernelGGL((decode_down_kernel<WT, NCT, (R >= 2 ? 2 : 1), OT, PASSES>), dim3(a.H / 32, n_slots), dim3(256),
                       0, st, a);
  else
    hipLaunchKernelGGL((decode_down_kernel<WT, NCT, 1, OT, PASSES>), dim3(a.H / 16, n_slots), dim3(256), 0, st, a);
}

template <int OT>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeArgs a) {
  combine_item<OT, false>(a, long(blockIdx.x) * blockDim.x + threadIdx.x);
}

// -------------------------------------------------------------- launch --

// With a.dn_count the combine runs in the down launch's epilogue; without,
// in a launch of its own.
template <int WT, int XT, int NCT, bool PASSES>
static void launch_decode_t(const DecodeArgs& a, int n_gu_row_tiles, hipStream_t st, StageMarker* mark) {
  dim3 g1(n_gu_row_tiles, a.n_routed_slots + a.S), b(256);
  if (NCT == 1 && !PASSES && a.route_in_gu)
    hipLaunchKernelGGL((decode_gateup_kernel<WT, XT, 1, false, true>), g1, b,
                       size_t(small_route_ints(256, a.T, a.E, a.k)) * 4, st, a);
  else
    hipLaunchKernelGGL((decode_gateup_kernel<WT, XT, NCT, PASSES, false>), g1, b, 0, st, a);
  if (mark) mark->mark(st);
  if (a.dn_count) {
    launch_down<WT, NCT, XT, PASSES>(a, a.n_routed_slots + a.S, st);
  } else {
    launch_down<WT, NCT, -1, PASSES>(a, a.n_routed_slots + a.S, st);
    const long n4 = long(a.T) * a.H / 4;
    hipLaunchKernelGGL((decode_combine_kernel<XT>), dim3(int((n4 + 255) / 256)), b, 0, st, a);
  }
  if (mark) mark->mark(st);
}

// One 16-token column tile per pass unless the routed slots average more than
// 8 tokens: the one-tile kernels keep more weight bytes in flight per wave,
// and the rare slot with more tokens takes another pass.
template <int WT, int XT>
static void launch_decode_x(const DecodeArgs& a, int n_gu_row_tiles, hipStream_t st, StageMarker* mark) {
  if (a.T <= 16) launch_decode_t<WT, XT, 1, false>(a, n_gu_row_tiles, st, mark);
  else if (a.T * a.k <= 8 * a.E) launch_decode_t<WT, XT, 1, true>(a, n_gu_row_tiles, st, mark);
  else launch_decode_t<WT, XT, 4, false>(a, n_gu_row_tiles, st, mark);
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

hipError_t launch_decode(const DecodeArgs& a, int wdt, int xdt, int n_gu_row_tiles, hipStream_t st,
                         StageMarker* mark) {
  if (a.route_in_gu && (a.T > 16 || !small_route(a.T, a.E, a.k) || a.route.tile_m != 1)) return hipErrorInvalidValue;
  if (wdt == DT_F32) {
    if (xdt == DT_F32) launch_decode_x<DT_F32, DT_F32>(a, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_F32, DT_BF16>(a, n_gu_row_tiles, st, mark);
  } else if (wdt == DT_BF16) {
    if (xdt == DT_F32) launch_decode_x<DT_BF16, DT_F32>(a, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_BF16, DT_BF16>(a, n_gu_row_tiles, st, mark);
  } else if (wdt == DT_Q4) {
    if (xdt == DT_F32) launch_decode_x<DT_Q4, DT_F32>(a, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_Q4, DT_BF16>(a, n_gu_row_tiles, st, mark);
  } else if (wdt == DT_Q8) {
    if (xdt == DT_F32) launch_decode_x<DT_Q8, DT_F32>(a, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_Q8, DT_BF16>(a, n_gu_row_tiles, st, mark);
  } else if (wdt == DT_FP8) {
    if (xdt == DT_F32) launch_decode_x<DT_FP8, DT_F32>(a, n_gu_row_tiles, st, mark);
    else launch_decode_x<DT_FP8, DT_BF16>(a, n_gu_row_tiles, st, mark);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
