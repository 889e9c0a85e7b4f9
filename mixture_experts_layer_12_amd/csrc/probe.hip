// Measurement probes: what this GPU reaches on a plain streaming read and on
// back-to-back bf16 MFMAs.  They give the measured peaks the layer's kernels
// are reported against next to the published ones ("Why MoE on RTX 5090
// falls short: a bandwidth measurement", news.malakhovai.ru: bandwidth
// measured against the data-sheet figure, and bandwidth as a function of the
// bytes one kernel reads on cold data).  Not part of the layer.
#include "moe_probe.h"

#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.hpp"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;            // 16-byte loads in flight per lane
constexpr int kProbeMaxGrid = 8192;

// Work-group b reads the 16-byte words [b * per_wg, (b + 1) * per_wg) of
// the buffer (clamped to n16), kProbeUnroll loads per lane in flight, and
// folds them into one word it stores to sink[b] (so no load is dead).
__global__ void __launch_bounds__(kProbeThreads) probe_read_kernel(const u32x4_t* __restrict__ buf, long n16,
                                                                   long per_wg, uint32_t* __restrict__ sink) {
  const long begin = long(blockIdx.x) * per_wg;
  const long end = begin + per_wg < n16 ? begin + per_wg : n16;
  uint32_t acc = 0;
  long i = begin + threadIdx.x;
  constexpr long step = long(kProbeThreads) * kProbeUnroll;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += step) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = ldg16(buf + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += kProbeThreads) {
    const u32x4_t v = ldg16(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // fold the wave, one word per work-group
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d);
  __shared__ uint32_t w[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int q = 0; q < kProbeThreads / 64; ++q) s ^= w[q];
    sink[blockIdx.x] = s;
  }
}

// Each wave issues `iters` rounds of 8 independent 32x32x16 bf16 MFMAs on
// register operands (8 accumulator chains, so each MFMA's result is not
// needed again until 7 others have issued); one work-group per CU, one wave
// per SIMD.
constexpr int kMfmaChains = 8;
__global__ void __launch_bounds__(kProbeThreads) probe_mfma_kernel(int iters, float* __restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63;
  u32x4_t a = {0x3f803f80u ^ lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  u32x4_t b = {0x3c003c00u, 0x3c003c00u ^ (lane << 1), 0x3c003c00u, 0x3c003c00u};
  f32x16_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[c][q] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = mfma32_bf16(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int q = 0; q < 16; ++q) s += acc[c][q];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace moe

extern "C" {

int moe_probe_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink) return -1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 15u)) return -4;
  if (bytes < 16 || bytes % 16) return -2;
  const long n16 = long(bytes / 16);
  // about 64 KiB per work-group, at most kProbeMaxGrid of them
  long grid = std::min<long>(moe::kProbeMaxGrid, std::max<long>(1, (n16 + 4095) / 4096));
  const long per_wg = (n16 + grid - 1) / grid;
  grid = (n16 + per_wg - 1) / per_wg;
  hipLaunchKernelGGL(moe::probe_read_kernel, dim3(unsigned(grid)), dim3(moe::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const moe::u32x4_t*>(buf), n16, per_wg,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int moe_probe_mfma_bf16(int32_t iters, void* sink, double* flops, void* stream) {
  if (!sink || !flops) return -1;
  if (reinterpret_cast<uintptr_t>(sink) & 15u) return -4;
  if (iters < 1) return -2;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -6;
  const int grid = std::min(cus, moe::kProbeMaxGrid);
  hipLaunchKernelGGL(moe::probe_mfma_kernel, dim3(grid), dim3(moe::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), int(iters), static_cast<float*>(sink));
  *flops = double(grid) * (moe::kProbeThreads / 64) * double(iters) * moe::kMfmaChains * (2.0 * 32 * 32 * 16);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
