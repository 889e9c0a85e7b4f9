/*
 * moe.h -- C ABI of the fused Mixture-of-Experts layer forward for AMD
 * Instinct MI355X (gfx950).
 *
 * What the layer computes, per token t (row of x):
 *   logits  l[t,e] = sum_h x[t,h] * router_w[e,h] + router_b[e]
 *   probs   p[t,:] = softmax(l[t,:])
 *   top-k   S_t    = the top_k experts with the largest logits (descending;
 *                    equal logits go to the lower expert index)
 *   weights w[t,j] = p[t,S_tj] / sum_j' p[t,S_tj']
 *   expert  FFN_e(v) = w_down[e] (silu(w_gate[e] v) * (w_up[e] v)),
 *           silu(z) = z / (1 + exp(-z))
 *   out[t]  = sum_j w[t,j] FFN_{S_tj}(x[t]) + sum_s FFN^shared_s(x[t])
 *
 * Sources: "Fused MoE kernel on Triton: 5 launches vs 24" (ai-manual.ru),
 * section "Fused kernel: one operation instead of twenty-four" (the four
 * fused steps: top-k routing weights, dispatch, engaged-expert compute,
 * weighted aggregation) and section "Megablocks? It has been obsolete for two
 * years" (top-k chosen at run time); "llama.cpp: fusing shared experts into
 * MMVQ" (ai-manual.ru), sections "Shared experts in MoE: what they are and
 * why they exist" (router + top-k experts; always-on shared experts) and
 * "How fusing shared experts into MMVQ can speed up inference" (shared experts
 * computed in the same pass as the routed ones, weights untouched).  The FFN
 * form (SwiGLU), the softmax scoring, the renormalisation, the weight 1 of
 * shared experts and the optional router bias are readings: the pages name
 * the steps but never write their formulas.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns
 *     every buffer; the library allocates no device memory.  Its only state
 *     is process-wide and does not carry data from one call to the next:
 *     one-time kernel attributes set on first use, the last HIP error of
 *     each thread (moe_last_hip_error) and the completion-tag counter of the
 *     single-launch decode (MOE_PATH_DECODE_FUSED).
 *   - Every device pointer must be 16-byte aligned (MOE_ERR_ALIGN otherwise).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  No call synchronises or copies device data to the
 *     host.  Results are valid once the caller has synchronised the stream.
 *   - Arguments are validated before anything is enqueued: on any error code
 *     other than MOE_ERR_HIP nothing has been launched.
 *   - The workspace is scratch for one call: no initial contents are
 *     required and nothing in it survives a call.  Calls that share one
 *     workspace must not overlap in time (use one workspace per stream).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types (MOE_Q8_0 and MOE_FP8_E4M3: expert weights of the decode path only) */
enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_Q4_0 = 2, MOE_Q8_0 = 3, MOE_FP8_E4M3 = 4 };

/* execution path (moe_shape_t.path) */
enum {
  MOE_PATH_AUTO = 0,    /* decode path when T <= 64, the dtypes need it or the sizes exceed
                           the prefill limits below, else prefill */
  MOE_PATH_DECODE = 1,  /* weight-streaming mat-vec kernels, any supported dtype, any T */
  MOE_PATH_PREFILL = 2, /* bf16 MFMA grouped GEMMs; needs x, experts bf16, and (32-bit element
                           offsets inside one matrix) max(I, I_shared) * H, T * H and
                           (roundup(T*top_k + E*255, 256) + n_shared*roundup(T, 256)) *
                           max(I, I_shared) all below 2^31; its expert segments are padded
                           to multiples of 256 rows */
  MOE_PATH_DECODE_FUSED = 3  /* the decode kernels as one launch (a resident grid) per pass of
                           at most 64 tokens; needs router_dtype == x_dtype and
                           top_k <= 16.  While `stream` is being captured into a
                           graph the call runs path 1 instead (a captured launch
                           would replay the completion tags of the capture).
                           Opt-in only: it measures slower than path 1, and a
                           wait that gives up is reported through the status
                           words of moe_forward_tables_t, not the return code. */
};

/* return codes */
enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,       /* a required pointer is NULL, or a forbidden one is not */
  MOE_ERR_SHAPE = -2,      /* sizes out of range (see moe_shape_t) */
  MOE_ERR_DTYPE = -3,      /* unsupported dtype or dtype/path combination */
  MOE_ERR_ALIGN = -4,      /* a device pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = -5,  /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = -6,        /* a HIP launch failed (hipGetLastError) */
  MOE_ERR_TOO_LARGE = -7,  /* moe_forward_noalloc: the shape needs more workspace than its
                              static scratch array holds (MOE_NOALLOC_SCRATCH_BYTES) */
  MOE_ERR_NOT_PINNED = -8, /* moe_cache_create: a host expert stack is not pinned host memory */
  MOE_ERR_HOST_ALLOC = -9  /* moe_cache_create: its host bookkeeping could not be allocated */
};

/*
 * Layer shape and dtypes.
 *   T         tokens (rows of x), 0 <= T <= 1048576; T == 0 is a no-op.
 *   H         hidden size, 32 <= H <= 65536, H % 32 == 0.
 *   E         routed experts, 1 <= E <= 256.
 *   I         routed-expert intermediate size, 32 <= I <= 1048576, I % 32 == 0.
 *   top_k     experts per token, 1 <= top_k <= E, T * top_k <= 16777216.
 *   n_shared  always-on shared experts, 0 <= n_shared <= 16.
 *   I_shared  shared-expert intermediate size (same rules as I); ignored
 *             when n_shared == 0.
 *   x_dtype   MOE_F32 | MOE_BF16; `out` has the same dtype.
 *   w_dtype   MOE_F32 | MOE_BF16 | MOE_Q4_0 | MOE_Q8_0 | MOE_FP8_E4M3, for routed
 *             and shared experts (the two 8-bit types on MOE_PATH_DECODE only).
 *   router_dtype  MOE_F32 | MOE_BF16.
 *   path      MOE_PATH_*.
 *
 * Weight layouts (row-major, K contiguous):
 *   router_w [E, H]; router_b f32 [E] (optional);
 *   w_gate, w_up [E, I, H]; w_down [E, H, I];
 *   ws_gate, ws_up [n_shared, I_shared, H]; ws_down [n_shared, H, I_shared].
 * A MOE_Q4_0 stack [E, N, K] (K % 32 == 0) is one buffer: all nibble bytes
 * [E, N, K/2] first, then, starting at the next multiple of 256 bytes from
 * the buffer start, all fp16 scales [E, N, K/32].  In each block of 32 values
 * along K, value j < 16 is the low nibble of byte j and value j + 16 the high
 * nibble of byte j; the value is d * (q - 8).  The stored d must satisfy
 * 8 * |d| <= 65504.
 * A MOE_Q8_0 stack [E, N, K] (K % 32 == 0): all int8 codes [E, N, K] first,
 * then from the next multiple of 256 bytes all fp16 scales [E, N, K/32];
 * the value of code q in block b is d_b * q (|d_b| * 128 <= 65504).
 * A MOE_FP8_E4M3 stack [E, N, K]: all codes [E, N, K] in the OCP E4M3
 * encoding first, then from the next multiple of 256 bytes the fp32 scales
 * [E, N], one per row; the value is scale[e][n] * E4M3(code).
 */
typedef struct {
  int32_t T, H, E, I, top_k;
  int32_t n_shared, I_shared;
  int32_t x_dtype, w_dtype, router_dtype;
  int32_t path;
} moe_shape_t;

/*
 * Routing outputs of moe_route.  Flat assignment id f = t * top_k + j.
 *   topk_ids    int32 [T*top_k]   required; expert of assignment f
 *   topk_w      f32   [T*top_k]   required; renormalised weight of f
 *   counts      int32 [E]         or NULL; assignments per expert
 *   offsets     int32 [E+1]       or NULL; start of each expert's segment in
 *               the expert-sorted order; segments are padded to multiples of
 *               tile_m (moe_dispatch_dims)
 *   sorted_ids  int32 [capacity]  or NULL; flat ids in expert-sorted order,
 *               ascending f inside a segment; padding and the tail up to
 *               capacity hold the sentinel T*top_k
 *   tile_expert int32 [n_tiles]   or NULL; expert owning rows
 *               [i*tile_m, (i+1)*tile_m) of the sorted order, -1 past offsets[E]
 *   inv         int32 [T*top_k]   or NULL; position of f in sorted_ids
 *   active      int32 [E+1]       or NULL; active[0] = number of experts with
 *               counts > 0, followed by those experts in ascending order
 */
typedef struct {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_ids;
  int32_t* tile_expert;
  int32_t* inv;
  int32_t* active;
} moe_route_out_t;

/* Bytes of workspace moe_forward / moe_route need for shape *s (host call,
 * no GPU access).  Returns MOE_OK and writes *bytes, or a validation error. */
int moe_workspace_size(const moe_shape_t* s, size_t* bytes /* host */);

/* The path moe_forward takes for shape *s when the stream is not being
 * captured: s->path itself, or what MOE_PATH_AUTO resolves to (host call).
 * Returns the MOE_PATH_* value (1, 2 or 3) or a validation error (< 0). */
int moe_resolve_path(const moe_shape_t* s);

/* Dimensions of the expert-sorted order for shape *s (host call):
 * tile_m (padding multiple), capacity = roundup(T*top_k + E*(tile_m-1), tile_m),
 * n_tiles = capacity / tile_m.  Any output pointer may be NULL. */
int moe_dispatch_dims(const moe_shape_t* s, int32_t* tile_m /* host */,
                      int32_t* capacity /* host */, int32_t* n_tiles /* host */);

/* Router and dispatch only: logits, softmax, top-k, renormalisation, and the
 * expert-sorted order.  x [T,H] (x_dtype), router_w [E,H] (router_dtype),
 * router_b f32 [E] or NULL.  The expert weights and `path` are not used.
 * The workspace needs moe_route_workspace_size(s) bytes (any workspace sized
 * for moe_forward also serves). */
int moe_route(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
              const moe_route_out_t* out /* host struct of device pointers */,
              void* workspace, size_t ws_bytes, void* stream);

/* The whole layer forward.  x [T,H] (x_dtype); out [T,H] (x_dtype), which
 * must not overlap x; router_b may be NULL; ws_gate/ws_up/ws_down must be
 * NULL exactly when n_shared == 0. */
int moe_forward(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                const void* w_gate, const void* w_up, const void* w_down,
                const void* ws_gate, const void* ws_up, const void* ws_down,
                void* out, void* workspace, size_t ws_bytes, void* stream);

/* moe_forward that also records caller-created HIP events (hipEvent_t,
 * passed as void*) on `stream` at the stage boundaries of each pass:
 * events[0] before the first launch, events[i] after launch i.  Launches of
 * one pass: decode path 1 router+dispatch, 2 gate/up, 3 down+combine;
 * single-launch decode 1 the whole pass;
 * prefill path 1 router+dispatch, 2 gate/up GEMM, 3 down GEMM (weighted
 * partial rows), 4 combine (fixed-order sum per token, cast to the output
 * dtype).  A decode call with T > 64 makes several passes; the events then
 * hold the last pass.  Entries beyond n_events, or NULL entries, are skipped.
 * Returns MOE_ERR_NULL when events is NULL or n_events < 1; otherwise as
 * moe_forward.  Meant for stage timing (hipEventElapsedTime). */
int moe_forward_profiled(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                         const void* w_gate, const void* w_up, const void* w_down,
                         const void* ws_gate, const void* ws_up, const void* ws_down,
                         void* out, void* workspace, size_t ws_bytes, void* stream,
                         void* const* events /* host array of hipEvent_t */, int n_events);

/*
 * Budgeted channel-sparse routed experts ("KAIST removed calibration from MoE
 * decoding and sped up blocks up to 2.69x over vLLM", news.hamidun.com,
 * sections "A threshold promises a budget but does not keep it" and "Top-k
 * instead of a threshold"): for every token and each of its top_k experts,
 * only the `budget` intermediate channels with the highest scores are used --
 * rows of that expert's gate and up matrices and the matching columns of its
 * down matrix -- so the bytes read per token are fixed in advance.  Equal
 * scores keep the lower channel index; NaN scores rank below every number.
 * Routing, renormalisation and the shared experts are as in moe_forward
 * (shared experts stay dense).  The scorer is the caller's.
 *
 *   channel_scores f32 [T, E, I]: score of channel i of expert e for token t
 *   budget         channels kept per (token, engaged expert), 1 <= budget <= I
 *   w_down_t       routed down stack transposed: [E, I, H] (row i = channel i)
 *   ws_down        shared down stack as in moe_forward: [n_shared, H, I_shared]
 * Requirements: w_dtype MOE_F32 or MOE_BF16; I <= 16384; `path` is ignored
 * (the decode kernels run the routing and the shared experts, in passes of
 * at most 64 tokens).  Workspace: moe_sparse_workspace_size bytes, no initial
 * contents required.  Errors as moe_forward.
 */
int moe_sparse_workspace_size(const moe_shape_t* s, int32_t budget, size_t* bytes /* host */);
int moe_forward_channel_sparse(const moe_shape_t* s, int32_t budget, const float* channel_scores,
                               const void* x, const void* router_w, const float* router_b,
                               const void* w_gate, const void* w_up, const void* w_down_t,
                               const void* ws_gate, const void* ws_up, const void* ws_down,
                               void* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * Where moe_forward leaves the routing of its last pass inside its workspace,
 * as byte offsets from the workspace start (host call, no GPU access).  After
 * a moe_forward call with shape *s has completed on its stream, the workspace
 * holds, for the tokens of the last pass ([T - tokens, T)), the arrays of
 * moe_route_out_t in the expert-sorted order of the path the forward took:
 * flat ids f = t * top_k + j count from the first token of that pass, and
 * segments are padded to multiples of tile_m (256 on the prefill path, 1 on
 * the decode paths, which pad nothing).  tile_expert is written only when
 * n_tiles > 0 (prefill); its offset is 0 otherwise.  The offsets describe a
 * layout; they stay valid until the next call that uses the workspace.
 * Meant for callers that want the routing the forward used (expert load
 * statistics) without a second routing call.
 */
typedef struct {
  int32_t path;        /* MOE_PATH_DECODE, MOE_PATH_PREFILL or MOE_PATH_DECODE_FUSED */
  int32_t tokens;      /* tokens of the last pass (T for prefill; decode passes take at most 64) */
  int32_t tile_m;      /* padding multiple of the sorted order */
  int32_t capacity;    /* entries of sorted_ids */
  int32_t n_tiles;     /* entries of tile_expert (0: not written) */
  size_t topk_ids, topk_w, counts, offsets, sorted_ids, tile_expert, inv, active;
  /* MOE_PATH_DECODE_FUSED, and MOE_PATH_DECODE when the last pass selects
   * inside its logits launch (shared_in_router without route_in_gateup; not
   * in a captured graph, which takes a separate selection launch); 0
   * otherwise: two uint64 words.  These forms rely on work-groups of one
   * launch running at the same time; every wait between them is bounded
   * (about a second; the environment variable MOE_FUSED_WAIT_ROUNDS, read on
   * each call, sets the number of polling rounds).  After the call has
   * completed on its stream the two words are equal exactly when some wait
   * of the last pass gave up: `out` is then not valid (on the single-launch
   * decode its affected elements hold NaN) although the call returned
   * MOE_OK. */
  size_t status;
  /* MOE_PATH_DECODE, last pass: route_in_gateup 1 when the routed gate/up
   * work-groups select and dispatch in their own prologue (the router launch
   * computes logits only); shared_in_router 1 when the shared experts'
   * gate/up runs in the logits launch (with the routing in the gate/up
   * prologue, or, for one column tile per routed slot, with the selection in
   * one more work-group of that launch). */
  int32_t route_in_gateup, shared_in_router;
} moe_forward_tables_t;
int moe_forward_tables(const moe_shape_t* s, moe_forward_tables_t* t /* host */);

/* Bytes of workspace moe_route needs for shape *s (host call); at most
 * moe_workspace_size(s). */
int moe_route_workspace_size(const moe_shape_t* s, size_t* bytes /* host */);

/*
 * moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments, layouts, paths and results are those of
 * moe_forward; the workspace is a static device array of the library
 * (MOE_NOALLOC_SCRATCH_BYTES bytes, held by every GPU the library runs on
 * from its first call there until the process ends).  Shapes whose
 * moe_workspace_size exceeds it are rejected with MOE_ERR_TOO_LARGE before
 * anything else happens.  The call allocates nothing.  All calls on one GPU
 * share the array, which keeps the last call's contents: calls that overlap
 * in time on one GPU (several streams or threads) race and must not be
 * issued; calls ordered on one stream are fine.  The first call on a device
 * looks the array's address up with that device current (HIP's current
 * device must be the device of `stream`).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                        const void* w_gate, const void* w_up, const void* w_down,
                        const void* ws_gate, const void* ws_up, const void* ws_down,
                        void* out, void* stream);

/*
 * Host-resident routed experts with a GPU expert cache and predictive
 * prefetching ("FATE: how to speed up MoE inference in llama.cpp with an
 * expert cache and prefetching", ai-manual.ru, sections "How the expert cache
 * works" and "Predictive prefetching: guessing the future").
 *
 * The routed experts of n_layers layers stay in pinned host memory (in the
 * layouts above, one stack per matrix and layer).  A device region the caller
 * allocates holds n_slots expert slots shared by all layers and a slot map.
 * In moe_forward_cached the expert kernels look each engaged expert up in the
 * map: a resident expert is read from its slot (HBM), any other straight from
 * the host stacks over PCIe -- the same bytes, so the output never depends on
 * what is resident.  The host learns each pass's engaged experts from a list
 * the GPU writes into pinned memory after the pass; it counts hits and misses,
 * copies an expert missed a second time (since it was last resident) into the
 * least recently used slot on copy_stream, and, for each of the next
 * prefetch_depth layers d (cyclically: after the
 * last layer comes layer 0 of the next token), copies in the experts
 * (e + d * prefetch_shift) mod E of every engaged e.  The page's example
 * predicts, from experts 3 and 7 in one layer, experts 4 and 8 in the next
 * (shift 1).  With prefetch_depth 0 no call waits for anything on the host;
 * with prefetching each call waits, after enqueueing its launches, for its
 * own engaged experts (the GPU finishes the pass meanwhile) and starts the
 * predicted copies at once, and a pass waits for the copies of its own
 * layer's experts that are in flight.  Slot-map changes run on the compute
 * stream, so no launch sees a slot change under it; a slot is overwritten
 * only after every launch that could read its old contents has finished.
 *
 * Results equal moe_forward on the decode path (MOE_PATH_DECODE) with the
 * same weights on the device up to the order of fp32 sums (bit for bit when
 * both take the same launch structure).  Shared experts and router weights
 * stay device-resident and are passed per call.  A cache is used from one
 * host thread and one compute stream at a time.  The library allocates no
 * device memory; moe_cache_create allocates the host bookkeeping, HIP events
 * and a pinned host ring of 64 active lists, which moe_cache_destroy frees.
 */
typedef struct {
  const void* w_gate;   /* (host, pinned) [E, I, H] in w_dtype's layout */
  const void* w_up;     /* (host, pinned) [E, I, H] */
  const void* w_down;   /* (host, pinned) [E, H, I] */
} moe_host_experts_t;

typedef struct {
  uint64_t lookups;        /* engaged (pass, expert) pairs looked up */
  uint64_t hits;           /* ... found resident (prefetched ones included) */
  uint64_t misses;         /* ... not resident: read from host memory by the kernels */
  uint64_t prefetches;     /* experts copied in ahead of time */
  uint64_t prefetch_hits;  /* hits on a prefetched expert, its first use */
  uint64_t bytes_copied;   /* host-to-device bytes enqueued (copies after misses, and prefetches) */
} moe_cache_stats_t;

typedef struct moe_expert_cache moe_expert_cache_t;

/* Device bytes of a cache region for n_layers layers and n_slots slots of
 * the shape's routed experts (its T and path are ignored); 1 <= n_layers <=
 * 65536, 1 <= n_slots <= 65536. Host call. */
int moe_cache_region_bytes(const moe_shape_t* s, int32_t n_layers, int32_t n_slots, size_t* bytes /* (host) */);

/* Creates a cache over `layers` (host array of n_layers entries, each stack
 * pinned and 16-byte aligned: MOE_ERR_NOT_PINNED / MOE_ERR_ALIGN otherwise)
 * in `region` (device, 256-byte aligned, at least moe_cache_region_bytes; it
 * must outlive the cache).  0 <= prefetch_depth < n_layers (0: no prefetch);
 * prefetch_shift is any integer (taken mod E).  copy_stream: a hipStream_t
 * of default priority, not the compute stream.  The map starts empty (the
 * call waits until it is cleared); nothing is copied yet.  *out receives the
 * handle (host). */
int moe_cache_create(const moe_shape_t* s, int32_t n_layers, const moe_host_experts_t* layers,
                     void* region, size_t region_bytes, int32_t n_slots, int32_t prefetch_depth,
                     int32_t prefetch_shift, void* copy_stream, moe_expert_cache_t** out);

/* Waits for the cache's copies, then frees its bookkeeping, events and
 * pinned ring.  The caller must have synchronised the compute stream that
 * ran moe_forward_cached (its last launches write into the ring). */
int moe_cache_destroy(moe_expert_cache_t* c);

/* Layer `layer`'s forward, as moe_forward with the routed experts read from
 * the cache or from host memory.  s must equal the shape given to
 * moe_cache_create except for T and path (the call always takes the decode
 * path); workspace as moe_workspace_size for s with path MOE_PATH_DECODE.
 * Any cache size works (a pass may engage more experts than there are
 * slots).  With prefetch_depth > 0 the call returns once its pass's engaged
 * experts are known (after the pass has finished on the GPU). */
int moe_forward_cached(moe_expert_cache_t* c, int32_t layer, const moe_shape_t* s, const void* x,
                       const void* router_w, const float* router_b,
                       const void* ws_gate, const void* ws_up, const void* ws_down,
                       void* out, void* workspace, size_t ws_bytes, void* stream);

/* Counters since creation or the last reset (reset != 0 zeroes them after
 * the read), over the passes whose engaged experts have reached the host
 * (all of them once the compute stream has been synchronised). */
int moe_cache_stats(moe_expert_cache_t* c, moe_cache_stats_t* out /* (host) */, int32_t reset);

/* Forgets every resident expert: the next call's launches find none (the map
 * is cleared on its stream first); copies in flight still complete. */
int moe_cache_flush(moe_expert_cache_t* c);

/* The hipError_t value behind the most recent MOE_ERR_HIP returned to the
 * calling thread (0 if there was none).  Host call. */
int moe_last_hip_error(void);

/* Static description of a return code. */
const char* moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
