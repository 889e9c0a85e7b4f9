// Device helpers shared by the MoE kernels: vector types, bf16/fp16
// conversions, CDNA4 MFMA wrappers, Q4_0 dequantisation, and the argument
// blocks the host passes to each kernel.
//
// MFMA operand layout used everywhere (16x16 tiles, wave64):
//   A operand: lane l supplies row (l % 16) and a k-group g = l / 16;
//   B operand: lane l supplies column (l % 16) and the same k-group g;
//   D (4 floats): lane l holds column (l % 16), rows 4*(l/16) + i, i = 0..3.
// Within one MFMA the k positions a lane supplies are the same for A and B,
// so any assignment of physical k indices to (g, element) works as long as
// both operands use it; the kernels pick assignments that keep global loads
// 16 bytes wide and contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_Q4 = 2, DT_Q8 = 3, DT_FP8 = 4 };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// ------------------------------------------------------------ conversions --

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// float -> fp16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// 8 floats -> two bf16x8 operands hi + lo with hi + lo == v to ~2^-17 relative.
__device__ __forceinline__ void split_bf16x8(const float* v, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h0 = f32_to_bf16(v[2 * i]), h1 = f32_to_bf16(v[2 * i + 1]);
    float r0 = v[2 * i] - __uint_as_float(h0 << 16);
    float r1 = v[2 * i + 1] - __uint_as_float(h1 << 16);
    hi[i] = h0 | (h1 << 16);
    lo[i] = f32_to_bf16(r0) | (f32_to_bf16(r1) << 16);
  }
}

// bf16 pair word -> fp16 pair word (exact for |v| within fp16 range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16(bf16_lo(w), bf16_hi(w));
}

// ------------------------------------------------------------------ MFMA --

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// 32x32x16 bf16: A lane l = row l%32, k 8*(l/32)..+7; B lane l = column l%32,
// same k; D lane l register q = column l%32, row 8*(q/4) + 4*(l/32) + q%4.
// One wave per SIMD issues these at the full matrix rate.
__device__ __forceinline__ f32x16_t mfma32_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ Q4_0 --
// One 16-byte block (32 codes, value j < 16 in the low nibble of byte j, value
// j + 16 in the high nibble) and its fp16 scale d -> four fp16x8 operands:
// frag 0 = values 0..7, 1 = 8..15, 2 = 16..23, 3 = 24..31, each d * (q - 8).
// (1024 + q) is formed exactly in fp16 by OR-ing q into the mantissa of 1024;
// subtracting 1032 then gives q - 8 exactly, and one fp16 multiply by d
// rounds once.

__device__ __forceinline__ uint32_t q4_pair(uint32_t v) {       // v holds the two codes at bits 0-3, 16-19
  return (v & 0x000F000Fu) | 0x64006400u;
}

__device__ __forceinline__ uint32_t q4_scale_pair(uint32_t magic, f16x2_t d2) {
  const f16x2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  f16x2_t v = __builtin_bit_cast(f16x2_t, magic) - off;
  return __builtin_bit_cast(uint32_t, v * d2);
}

__device__ __forceinline__ void q4_dequant_block(u32x4_t raw, uint16_t d_bits, u32x4_t frag[4]) {
  _Float16 d = __builtin_bit_cast(_Float16, d_bits);
  f16x2_t d2 = {d, d};
#pragma unroll
  for (int half = 0; half < 2; ++half) {           // bytes 0..7 -> frags 0/2, bytes 8..15 -> frags 1/3
#pragma unroll
    for (int wi = 0; wi < 2; ++wi) {
      // reorder bytes [b0 b1 b2 b3] -> [b0 b2 b1 b3] so that the low nibbles of
      // b0,b1 sit at bits 0-3 / 16-19 and those of b2,b3 at bits 8-11 / 24-27
      uint32_t w = __builtin_amdgcn_perm(raw[2 * half + wi], raw[2 * half + wi], 0x03010200u);
      frag[half][2 * wi + 0] = q4_scale_pair(q4_pair(w), d2);
      frag[half][2 * wi + 1] = q4_scale_pair(q4_pair(w >> 8), d2);
      frag[half + 2][2 * wi + 0] = q4_scale_pair(q4_pair(w >> 4), d2);
      frag[half + 2][2 * wi + 1] = q4_scale_pair(q4_pair(w >> 12), d2);
    }
  }
}

// ------------------------------------------------------------------ Q8_0 --
// One block of 32 signed codes (two 16-byte loads) and its fp16 scale d ->
// four fp16x8 operands (frag f = values 8f .. 8f+7), each d * q.  Flipping the
// sign bit turns q into q + 128 in 0..255, which is OR-ed into the mantissa of
// 1024 exactly; subtracting 1152 gives q exactly and one multiply rounds once.

__device__ __forceinline__ uint32_t q8_scale_pair(uint32_t magic, f16x2_t d2) {
  const f16x2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
  f16x2_t v = __builtin_bit_cast(f16x2_t, magic) - off;
  return __builtin_bit_cast(uint32_t, v * d2);
}

__device__ __forceinline__ void q8_dequant_block(u32x4_t raw0, u32x4_t raw1, uint16_t d_bits, u32x4_t frag[4]) {
  _Float16 d = __builtin_bit_cast(_Float16, d_bits);
  f16x2_t d2 = {d, d};
#pragma unroll
  for (int w = 0; w < 8; ++w) {                 // word w holds values 4w .. 4w+3
    const uint32_t t = (w < 4 ? raw0[w] : raw1[w - 4]) ^ 0x80808080u;
    // bytes [t0 0x64 t1 0x64] and [t2 0x64 t3 0x64]: two fp16 pairs 1024 + u
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, t, 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, t, 0x04030402u);
    frag[w >> 1][2 * (w & 1) + 0] = q8_scale_pair(lo, d2);
    frag[w >> 1][2 * (w & 1) + 1] = q8_scale_pair(hi, d2);
  }
}

// ------------------------------------------------------------ fp8 E4M3 --
// 16 E4M3 codes -> two fp16x8 operands (codes 0..7, 8..15).  The hardware
// conversion reads the OCP E4M3 encoding on this architecture; every E4M3
// value (at most 448, at least 2^-9 in magnitude) is exact in fp16, and the
// scale 1.0 leaves it unchanged.

__device__ __forceinline__ void fp8x16_to_f16(u32x4_t raw, u32x4_t out[2]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    out[w >> 1][2 * (w & 1) + 0] =
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(int(raw[w]), 1.0f, false));
    out[w >> 1][2 * (w & 1) + 1] =
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(int(raw[w]), 1.0f, true));
  }
}

// Byte offset of the scale array of a one-byte-code stack (Q8_0, fp8) [n_mat, N, K].
__host__ __device__ __forceinline__ size_t byte_code_scale_offset(long n_mat, long N, long K) {
  return (size_t(n_mat) * size_t(N) * size_t(K) + 255) / 256 * 256;
}

// Byte offset of the scale array of a Q4_0 stack [n_mat, N, K].
__host__ __device__ __forceinline__ size_t q4_scale_offset(long n_mat, long N, long K) {
  size_t nib = size_t(n_mat) * size_t(N) * size_t(K / 2);
  return (nib + 255) / 256 * 256;
}

// ------------------------------------------------------------ utilities --

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Loads from global memory, stated as such: the pointer may reach here
// through a path the compiler cannot see into (a base picked among several
// at run time can end up in a private lookup table), and a generic load
// would also wait on LDS traffic.
typedef const __attribute__((address_space(1))) u32x4_t g_u32x4_t;
typedef const __attribute__((address_space(1))) u32x2_t g_u32x2_t;
__device__ __forceinline__ u32x4_t ldg16(const void* p) { return *(g_u32x4_t*)(p); }
__device__ __forceinline__ u32x2_t ldg8(const void* p) { return *(g_u32x2_t*)(p); }

// Handoffs between work-groups of one launch (the single-launch decode).  The
// L2 of each XCD is not coherent with the others, so data that another
// work-group reads later in the same launch is written with device-scope
// stores (written through to memory) and flags and small routing values are
// read with device-scope loads.  COH false: ordinary accesses, for launches
// whose consumers run in a later kernel.
template <bool COH>
__device__ __forceinline__ void st_i32(int32_t* p, int32_t v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ void st_f32(float* p, float v) {
  if constexpr (COH) __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ void st_u32x2(void* p, u32x2_t v) {
  if constexpr (COH) {
    const uint64_t w = uint64_t(v[0]) | (uint64_t(v[1]) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *reinterpret_cast<u32x2_t*>(p) = v;
  }
}
template <bool COH>
__device__ __forceinline__ void st_f32x4(float* p, f32x4_t v) {
  if constexpr (COH) {
    st_u32x2<true>(p, u32x2_t{__float_as_uint(v[0]), __float_as_uint(v[1])});
    st_u32x2<true>(p + 2, u32x2_t{__float_as_uint(v[2]), __float_as_uint(v[3])});
  } else {
    *reinterpret_cast<f32x4_t*>(p) = v;
  }
}
template <bool COH>
__device__ __forceinline__ int32_t ld_i32(const int32_t* p) {
  if constexpr (COH) return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COH>
__device__ __forceinline__ f32x4_t ld_f32x4(const float* p) {
  if constexpr (COH) {
    uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(p));
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4_t{__uint_as_float(uint32_t(lo)), __uint_as_float(uint32_t(lo >> 32)), __uint_as_float(uint32_t(hi)),
                   __uint_as_float(uint32_t(hi >> 32))};
  } else {
    return *reinterpret_cast<const f32x4_t*>(p);
  }
}
template <bool COH>
__device__ __forceinline__ float ld_f32(const float* p) {
  if constexpr (COH)
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
  else return *p;
}

// Host-side hook called after each kernel launch (stage timing).
struct StageMarker {
  virtual void mark(hipStream_t st) = 0;
  virtual ~StageMarker() = default;
};

// Few assignments (decode): at most kSmallN of them (T * k), T * E <= 1024 and
// T * E * E <= kRankWork take the few-assignment route (route_small).
constexpr int kSmallN = 64;
constexpr int kRankWork = 65536;
constexpr int kSmallDispInts = 3 * 64 + 2 * 65 + 1;    // slot tables of the one-wave dispatch

__host__ __device__ inline bool small_route(int T, int E, int k) {
  return T * k <= kSmallN && T * E <= 1024 && long(T) * E * E <= kRankWork;
}

// Multi-launch decode: one 16-token column tile per pass (NCT = 1) unless the
// routed slots average more than 8 tokens (then 4 tiles, NCT = 4).
__host__ __device__ inline bool decode_one_col_tile(int T, int k, int E) { return T <= 16 || T * k <= 8 * E; }

// Multi-launch decode down projection: row tiles of 16 outputs per work-group
// (rpw) and k ranges (ks) per output row group.  With one column tile a
// work-group covers 4 row tiles while that still leaves >= 2048 work-groups,
// else 2 (H % 32 == 0) or 1.  The reduction over the intermediate dimension
// is then cut into 2 ranges, one work-group each, while the grid stays below
// 4096 work-groups and each wave keeps at least 8 steps of its range: a
// single round of large work-groups leaves the chip idle behind its slowest
// CU (measured on the Mixtral-shaped batch of 8: one range 190 us, two 166,
// four 171-179, eight 188-198).  `steps` is the number of MFMA steps along
// the longest K.
#ifndef MOE_DN_GRID_TARGET
#define MOE_DN_GRID_TARGET 4096
#endif
#ifndef MOE_DN_MAX_KS
#define MOE_DN_MAX_KS 2
#endif
#ifndef MOE_DN_RPW4_MIN_GRID
#define MOE_DN_RPW4_MIN_GRID 2048
#endif
#ifndef MOE_DN_MIN_WAVE_STEPS
#define MOE_DN_MIN_WAVE_STEPS 8
#endif
constexpr int kDownMaxKs = MOE_DN_MAX_KS;
#ifndef MOE_DN_W8_MIN_GRID
#define MOE_DN_W8_MIN_GRID 2048
#endif
// waves: 8 (each range cut over eight waves, two work-groups per CU) for
// grids of two-row-tile work-groups with at least MOE_DN_W8_MIN_GRID of them
// (Mixtral-shaped batch of 8: down 164 -> 159 us), else 4; smaller grids
// lose with eight (batch of 1: 46.6 -> 48.7 us).
struct DownShape { int rpw, ks, waves; };
__host__ inline DownShape decode_down_shape(bool one_col_tile, int H, int n_slots, int steps) {
  DownShape d{1, 1, 4};
  if (!one_col_tile) return d;
  if (H % 64 == 0 && (H / 64) * n_slots >= MOE_DN_RPW4_MIN_GRID) d.rpw = 4;
  else if (H % 32 == 0) d.rpw = 2;
  const long grid = long(H / (16 * d.rpw)) * n_slots;
  while (d.ks < kDownMaxKs && grid * d.ks * 2 <= MOE_DN_GRID_TARGET && steps / (4 * d.ks * 2) >= MOE_DN_MIN_WAVE_STEPS)
    d.ks *= 2;
  if (d.rpw == 2 && grid * d.ks >= MOE_DN_W8_MIN_GRID) d.waves = 8;
  return d;
}

// ------------------------------------------------------ kernel arguments --

// Routing state inside the workspace (or caller buffers for moe_route).
struct RouteBufs {
  float* logits;        // [T, E]
  int32_t* topk_ids;    // [T*k]
  float* topk_w;        // [T*k]
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E+1] padded
  int32_t* cprefix;     // [E+1] unpadded prefix of counts
  int32_t* active;      // [E+1]
  int32_t* sorted_ids;  // [capacity]
  int32_t* tile_expert; // [n_tiles]; nullptr: not written
  int32_t* inv;         // [T*k]
};

struct RouterArgs {
  const void* x;
  const void* wr;
  const float* bias;
  int T, H, E, k;
  int tile_m, capacity;
  int n_row_tiles, n_col_tiles;
  int logit_parts;      // 1: rb.logits holds the logits; 4: four group planes [4][T][E] without the bias
  float* zero_f32;      // optional buffer to clear (the decode down launch's arrival counters), or null
  long zero_n;          // its length in floats (multiple of 4)
  RouteBufs rb;
};

struct DecodeArgs {
  const void* x;        // [T, H]
  const uint8_t* wg; const uint8_t* wu; const uint8_t* wd;     // routed stacks
  const uint8_t* sg; const uint8_t* su; const uint8_t* sd;     // shared stacks
  int T, H, E, I, k, S, Is;
  int n_routed_slots;   // min(E, T*k)
  int n_row_tiles;      // gate/up: ceil(max(I, Is) / 16); down: H / 16
  const int32_t* active; const int32_t* counts; const int32_t* offsets; const int32_t* cprefix;
  const int32_t* sorted_ids; const float* topk_w; const int32_t* inv;
  void* h;              // activations between the two launches
  long h_plane;         // elements per plane (bf16 hi/lo planes)
  int h_stride;         // elements per h row
  float* partials;      // down: [dn_ksplit][T*k + S*T][H] weighted expert output rows, one plane per k range
  long part_plane;      // floats per plane of partials
  int dn_ksplit;        // down: ranges the reduction over I is cut into (1 or 2), one work-group each
  int dn_rpw;           // down: row tiles of 16 outputs per work-group (1, 2 or 4; 1 with NCT 4)
  int dn_waves;         // down: waves per work-group splitting each k range (8 with dn_rpw 2 only; else 4)
  void* out;            // [T, H]
  unsigned* dn_count;   // down with the combine epilogue: arrivals per output row group [H / 16]; else null
  int route_in_gu;      // 1: the routed gate/up work-groups select and dispatch from the logits themselves
  RouterArgs route;     // ... with these arguments (logits in route.rb.logits)
  int shared_in_router; // the decode launches start with one for the router logits and the shared
                        // experts' gate/up together; the gate/up launch covers routed slots only
  // shared_in_router without route_in_gu, outside graph capture (else null): the selection and
  // dispatch run in one more work-group of that launch, which waits for the logit work-groups'
  // completion flags (the call's epoch) for at most sel_spin polling rounds
  unsigned long long* sel_flags;    // [logit work-groups]
  unsigned long long* sel_status;   // status pair: this call's tag, the tag of the last call whose wait gave up
  unsigned long long sel_epoch;
  int sel_spin;
  // Expert cache: null, or the slot of each routed expert e in the cache's stacks wg/wu/wd
  // (E_w matrices each), -1 for an expert that is not resident, whose matrices are then read
  // from the host stacks wg_h/wu_h/wd_h (E matrices, device-mapped pinned host memory).
  const int32_t* slot_of;
  const uint8_t* wg_h; const uint8_t* wu_h; const uint8_t* wd_h;
  int E_w;
};

// Segments of one launch_gather_copy (sixteen experts of three quantised
// matrices; the list is a kernel argument of 3 KiB).
constexpr int kCopyMaxSegs = 96;
// Slot-map entries one launch_map_update writes.
constexpr int kMapMaxPairs = 240;

// Where routed expert e's matrices are: matrix `idx` of stacks of `n_mat`
// matrices, in the host stacks when `host`.
struct RoutedAt {
  int idx;
  long n_mat;
  bool host;
};
template <bool COH>
__device__ __forceinline__ RoutedAt routed_at(const DecodeArgs& a, int e) {
  if (!a.slot_of) return RoutedAt{e, a.E, false};
  const int s = ld_i32<COH>(a.slot_of + e);
  return s >= 0 ? RoutedAt{s, a.E_w, false} : RoutedAt{e, a.E, true};
}

// Host callbacks of an expert cache around each decode pass: before_pass
// runs before the pass's first launch and points the routed stacks at the
// cache (DecodeArgs wg/wu/wd, slot_of, wg_h/wu_h/wd_h, E_w), enqueueing its
// slot-map updates on the stream first; after_pass runs once the pass's
// launches are enqueued (d.active then holds the pass's active list in stream
// order).  A nonzero return ends the call with that code.
struct DecodeHook {
  virtual int before_pass(DecodeArgs& d, hipStream_t st) = 0;
  virtual int after_pass(const DecodeArgs& d, hipStream_t st) = 0;
  virtual ~DecodeHook() = default;
};

// Output rows per down item of the single-launch decode: two row tiles when
// the tokens fit one column tile (H is a multiple of 32), else one.
template <int NCT>
constexpr int kFusedDownRows = NCT == 1 ? 32 : 16;

// Single-launch decode: one work list of items in a fixed order, taken
// round-robin by a co-resident grid; an item waits only on items of lower
// index (completion flags carry the call's epoch).
struct FusedArgs {
  RouterArgs r;
  DecodeArgs d;
  int n_logit;          // [0, n_logit): router logit tiles
  int end_shared_gu;    // [n_logit, end_shared_gu): shared-expert gate/up row tiles
  int end_select;       // end_shared_gu: top-k and dispatch (one item; none with route_in_gu)
  int route_in_gu;      // 1: every routed gate/up item selects and dispatches from the logits itself
  int end_gu;           // [end_select, end_gu): routed gate/up row tiles, slot-major
  int end_down;         // [end_gu, end_down): down row groups (kFusedDownRows), slot-major, routed then shared
  int n_items;          // [end_down, n_items): combine blocks of 1024 outputs
  int gu_rt_routed, gu_rt_shared;   // gate/up row tiles per routed / shared slot
  unsigned long long epoch;
  unsigned long long* flags;        // [n_items]
  unsigned long long* call_tag;     // status pair, word 0: the epoch of this call (stored by item 0)
  unsigned long long* error;        // status pair, word 1: the epoch of the last call in which a wait gave up
  int spin_rounds;                  // polling rounds before a wait gives up
};

// Budgeted channel-sparse routed experts (decode).
constexpr int kSparseMaxRows = 2048;      // kept channels of one down split (staged in LDS)

struct SparseArgs {
  DecodeArgs d;               // x, routed gate/up stacks, shared stacks, routing, h / partials of the shared experts
  const int32_t* topk_ids;    // [T*k]
  const float* scores;        // [T, E, I] of this pass
  const uint8_t* wdt;         // routed down, transposed: [E, I, H]
  int c;                      // channels kept per (token, engaged expert)
  int R;                      // splits of the kept channels in the down projection
  int32_t* sel;               // [T*k, c] kept channels, ascending; with sel_all [T*E, c], every expert
  int sel_all;                // 1: the selection ran for every (token, expert), alongside the router
  float* hs;                  // [T*k, c] routing-weighted activations of the kept channels
  float* spart;               // [T*k, R, H] down partial rows
};

struct PrefillArgs {
  const void* x;
  const uint16_t* wg; const uint16_t* wu; const uint16_t* wd;
  const uint16_t* sg; const uint16_t* su; const uint16_t* sd;
  int T, H, E, I, k, S, Is;
  int capacity, tile_m, t_pad;        // routed rows, padding tile, shared rows per expert
  int n_row_tiles, n_col_tiles;
  int k_split;           // down projection: k ranges per output tile (one partial plane each)
  const int32_t* tile_expert; const int32_t* sorted_ids; const float* topk_w; const int32_t* offsets;
  uint16_t* h;           // [capacity + S*t_pad, h_stride] bf16
  int h_stride;
  float* partials;       // [k_split][capacity + S*t_pad, H] fp32 routing-weighted rows of the down GEMM
  long part_plane;       // elements per partial plane
  const int32_t* inv;    // [T*k] position of each assignment in the sorted order
  void* out;
};

}  // namespace moe
