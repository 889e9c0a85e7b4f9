// Router kernels: single-work-group (fused) and two-launch (logits, then
// selection and dispatch) forms of the items in router_items.hpp.
#include "router_items.hpp"

namespace moe {

// Side job: clear a buffer the later launches of the same pass need zeroed
// (the decode down launch's arrival counters), spread over the router's grid.
__device__ __forceinline__ void clear_accumulator(const RouterArgs& a) {
  if (!a.zero_f32) return;
  const long n4 = a.zero_n / 4;
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += long(gridDim.x) * blockDim.x)
    reinterpret_cast<f32x4_t*>(a.zero_f32)[i] = z;
}

// Single work-group (at most 16 experts x 16 tokens) of 16 waves, a chunk of
// the logits reduction each: logits stay in LDS.
template <int RT, int XT, int MODE>
__global__ void __launch_bounds__(1024) router_fused_kernel(RouterArgs a) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  __shared__ float lg[256];
  clear_accumulator(a);
  logits_tile<RT, XT, false, 1>(a, 0, 0, 0, kLogitChunks, reinterpret_cast<float*>(lds), lg);
  __syncthreads();
  select_and_dispatch<false, MODE>(a, lg, true, lds);
}

// Larger grids: the logits go to the workspace; the selection and dispatch run
// in a second launch (the kernel boundary orders them, no device-wide fences).
// With a.logit_parts == 4 (grids of few tiles) each tile is split over four
// work-groups, one per group of 4 chunks, which write partial planes; the
// selection adds the planes in order and then the bias, the same sums in the
// same order as the single-plane form.
// CPW chunks per wave: 1 for the partial-plane form (4 waves, 4 chunks), else
// 16 / waves.
template <int RT, int XT, int CPW>
__global__ void __launch_bounds__(1024) router_logits_kernel(RouterArgs a) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  clear_accumulator(a);
  if (a.logit_parts == 4) {
    const int tile = blockIdx.x >> 2, q = blockIdx.x & 3;
    logits_tile<RT, XT, false, CPW>(a, tile % a.n_row_tiles, tile / a.n_row_tiles, 4 * q, 4,
                                    reinterpret_cast<float*>(lds), a.rb.logits + size_t(q) * a.T * a.E);
  } else {
    logits_tile<RT, XT, false, CPW>(a, blockIdx.x % a.n_row_tiles, blockIdx.x / a.n_row_tiles, 0, kLogitChunks,
                                    reinterpret_cast<float*>(lds), a.rb.logits);
  }
}

template <int MODE>
__global__ void __launch_bounds__(1024) router_select_kernel(RouterArgs a) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  select_and_dispatch<false, MODE>(a, a.rb.logits, false, lds);
}

// --------------------------------------------------------------- launch --

size_t router_lds_bytes(int NW, int E, int n, bool stage) {
  const size_t red = size_t(kLogitChunks) * 64 * 4 * sizeof(float);
  const size_t disp = (size_t(router_disp_ints(NW, E)) + (n <= kRouterIdsLds ? n : 0) + (stage ? kRouterStage : 0)) *
                      sizeof(int);
  return red > disp ? red : disp;
}

template <int MODE>
static void launch_select(const RouterArgs& a, hipStream_t st) {
  static const bool attr = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(router_select_kernel<MODE>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              int(router_lds_bytes(16, 256, kRouterIdsLds, true)));
    return true;
  }();
  (void)attr;
  hipLaunchKernelGGL(router_select_kernel<MODE>, dim3(1), dim3(1024), router_lds_bytes(16, a.E, a.T * a.k, true), st, a);
}

// The selection and dispatch alone, from logits already in rb.logits (one
// plane, or four partial planes with logit_parts 4).
void launch_router_select(const RouterArgs& a, hipStream_t st) {
  switch (topk_mode(a.E, a.k)) {
    case kTopkT8: launch_select<kTopkT8>(a, st); break;
    case kTopkT16: launch_select<kTopkT16>(a, st); break;
    case kTopkT32: launch_select<kTopkT32>(a, st); break;
    case kTopkRow16: launch_select<kTopkRow16>(a, st); break;
    default: launch_select<kTopkWave>(a, st); break;
  }
}

template <int RT, int XT, int CPW>
static void launch_logits(const RouterArgs& a, int grid, int NW, hipStream_t st) {
  hipLaunchKernelGGL((router_logits_kernel<RT, XT, CPW>), dim3(grid), dim3(NW * 64),
                     size_t(kLogitChunks) * 64 * 4 * sizeof(float), st, a);
}

template <int RT, int XT>
static void launch_router_t(const RouterArgs& a, int NW, bool logits_only, hipStream_t st) {
  const int nblocks = a.n_row_tiles * a.n_col_tiles;
  const int mode = topk_mode(a.E, a.k);
  if (logits_only) {
    if (a.logit_parts == 4) launch_logits<RT, XT, 1>(a, 4 * nblocks, 4, st);
    else if (NW == 16) launch_logits<RT, XT, 1>(a, nblocks, 16, st);
    else if (NW == 8) launch_logits<RT, XT, 2>(a, nblocks, 8, st);
    else launch_logits<RT, XT, 4>(a, nblocks, 4, st);
  } else if (nblocks == 1) {
    // E <= 16: a thread per token, or a 16-lane row when k > 8
    const size_t lds = router_lds_bytes(16, a.E, a.T * a.k, false);
    if (mode == kTopkT8) hipLaunchKernelGGL((router_fused_kernel<RT, XT, kTopkT8>), dim3(1), dim3(1024), lds, st, a);
    else if (mode == kTopkT16) hipLaunchKernelGGL((router_fused_kernel<RT, XT, kTopkT16>), dim3(1), dim3(1024), lds, st, a);
    else hipLaunchKernelGGL((router_fused_kernel<RT, XT, kTopkRow16>), dim3(1), dim3(1024), lds, st, a);
  } else {
    if (a.logit_parts == 4) launch_logits<RT, XT, 1>(a, 4 * nblocks, 4, st);   // a wave per chunk of each group
    else if (NW == 16) launch_logits<RT, XT, 1>(a, nblocks, 16, st);
    else if (NW == 8) launch_logits<RT, XT, 2>(a, nblocks, 8, st);
    else launch_logits<RT, XT, 4>(a, nblocks, 4, st);
    switch (mode) {
      case kTopkT8: launch_select<kTopkT8>(a, st); break;
      case kTopkT16: launch_select<kTopkT16>(a, st); break;
      case kTopkT32: launch_select<kTopkT32>(a, st); break;
      case kTopkRow16: launch_select<kTopkRow16>(a, st); break;
      default: launch_select<kTopkWave>(a, st); break;
    }
  }
}

hipError_t launch_router(const RouterArgs& a, int rdt, int xdt, int NW, hipStream_t st, bool logits_only) {
  if (rdt == DT_F32 && xdt == DT_F32) launch_router_t<DT_F32, DT_F32>(a, NW, logits_only, st);
  else if (rdt == DT_F32) launch_router_t<DT_F32, DT_BF16>(a, NW, logits_only, st);
  else if (xdt == DT_F32) launch_router_t<DT_BF16, DT_F32>(a, NW, logits_only, st);
  else launch_router_t<DT_BF16, DT_BF16>(a, NW, logits_only, st);
  return hipGetLastError();
}

}  // namespace moe
