// Router kernels: single-work-group (fused) and two-launch (logits, then
// selection and dispatch) forms of the items in router_items.hpp.
#include "router_items.hpp"

namespace moe {

// Side job of the prefill path: clear the fp32 combine accumulator, spread
// over the router's grid.
__device__ __forceinline__ void clear_accumulator(const RouterArgs& a) {
  if (!a.zero_f32) return;
  const long n4 = a.zero_n / 4;
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += long(gridDim.x) * blockDim.x)
    reinterpret_cast<f32x4_t*>(a.zero_f32)[i] = z;
}

// Single work-group (at most 16 experts x 16 tokens): logits stay in LDS.
template <int RT, int XT>
__global__ void __launch_bounds__(1024) router_fused_kernel(RouterArgs a) {
  extern __shared__ int lds[];
  __shared__ float lg[256];
  clear_accumulator(a);
  logits_tile<RT, XT, false>(a, 0, 0, 0, kLogitChunks, reinterpret_cast<float*>(lds), lg);
  __syncthreads();
  select_and_dispatch<false>(a, lg, true, lds);
}

// Larger grids: the logits go to the workspace; the selection and dispatch run
// in a second launch (the kernel boundary orders them, no device-wide fences).
// With a.logit_parts == 4 (grids of few tiles) each tile is split over four
// work-groups, one per group of 4 chunks, which write partial planes; the
// selection adds the planes in order and then the bias, the same sums in the
// same order as the single-plane form.
template <int RT, int XT>
__global__ void __launch_bounds__(1024) router_logits_kernel(RouterArgs a) {
  extern __shared__ int lds[];
  clear_accumulator(a);
  if (a.logit_parts == 4) {
    const int tile = blockIdx.x >> 2, q = blockIdx.x & 3;
    logits_tile<RT, XT, false>(a, tile % a.n_row_tiles, tile / a.n_row_tiles, 4 * q, 4, reinterpret_cast<float*>(lds),
                               a.rb.logits + size_t(q) * a.T * a.E);
  } else {
    logits_tile<RT, XT, false>(a, blockIdx.x % a.n_row_tiles, blockIdx.x / a.n_row_tiles, 0, kLogitChunks,
                               reinterpret_cast<float*>(lds), a.rb.logits);
  }
}

__global__ void __launch_bounds__(1024) router_select_kernel(RouterArgs a) {
  extern __shared__ int lds[];
  select_and_dispatch<false>(a, a.rb.logits, false, lds);
}

// --------------------------------------------------------------- launch --

size_t router_lds_bytes(int NW, int E, int n, bool stage) {
  const size_t red = size_t(kLogitChunks) * 64 * 4 * sizeof(float);
  const size_t disp = (size_t(router_disp_ints(NW, E)) + (n <= kRouterIdsLds ? n : 0) + (stage ? kRouterStage : 0)) *
                      sizeof(int);
  return red > disp ? red : disp;
}

template <int RT, int XT>
static void launch_router_t(const RouterArgs& a, int NW, hipStream_t st) {
  const int nblocks = a.n_row_tiles * a.n_col_tiles;
  if (nblocks == 1) {
    hipLaunchKernelGGL((router_fused_kernel<RT, XT>), dim3(1), dim3(NW * 64),
                       router_lds_bytes(NW, a.E, a.T * a.k, false), st, a);
  } else {
    static const bool attr = [] {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(router_select_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(router_lds_bytes(16, 256, kRouterIdsLds, true)));
      return true;
    }();
    (void)attr;
    if (a.logit_parts == 4)      // a wave per chunk of each group
      hipLaunchKernelGGL((router_logits_kernel<RT, XT>), dim3(4 * nblocks), dim3(4 * 64),
                         size_t(kLogitChunks) * 64 * 4 * sizeof(float), st, a);
    else
      hipLaunchKernelGGL((router_logits_kernel<RT, XT>), dim3(nblocks), dim3(NW * 64),
                         size_t(kLogitChunks) * 64 * 4 * sizeof(float), st, a);
    hipLaunchKernelGGL(router_select_kernel, dim3(1), dim3(1024), router_lds_bytes(16, a.E, a.T * a.k, true), st, a);
  }
}

hipError_t launch_router(const RouterArgs& a, int rdt, int xdt, int NW, hipStream_t st) {
  if (rdt == DT_F32 && xdt == DT_F32) launch_router_t<DT_F32, DT_F32>(a, NW, st);
  else if (rdt == DT_F32) launch_router_t<DT_F32, DT_BF16>(a, NW, st);
  else if (xdt == DT_F32) launch_router_t<DT_BF16, DT_F32>(a, NW, st);
  else launch_router_t<DT_BF16, DT_BF16>(a, NW, st);
  return hipGetLastError();
}

}  // namespace moe
