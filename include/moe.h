/*
 * moe.h -- C ABI of an MI355X (gfx950) Mixture-of-Experts FFN layer forward.
 *
 * One call evaluates, for T tokens,
 *     out[t] = sum over token t's k chosen experts e of w[t,e] * FFN_e(x[t]),
 *     FFN_e(x) = Wd_e (silu(Wg_e x) * (Wu_e x)),
 * with the expert weights stored as integer codes plus fp16 scales and
 * zero-points (W = (q - z) * s) and read through an expert-to-slot table.
 * Weight formats: int4 or 8-bit codes, with one (s, z) per output row or per
 * output row and group of 128 inputs.
 * Optional shared experts are added for every token with weight 1:
 *     out[t] += sum over s < num_shared of FFN_{E+s}(x[t]).
 *
 * Where each step comes from (three web pages on expert offloading for MoE
 * inference; the "Strata" page is titled "125B MoE at 100+ tok/s on an
 * RTX 3090: a full-pipeline inference tuning record"):
 *   routing       Strata page, section 1.1 (top-2 or top-1 experts per token);
 *                 Co-inference page, section 5.1 (router kept at full precision)
 *   regrouping    Strata page, section 4.2 (tokens reordered by expert id)
 *   int4 experts  Strata page, section 3.1 (per-expert scale and zero-point,
 *                 dequantised on the load path, not in a kernel of its own)
 *   8-bit, groups Co-inference page, section 5.1 (8-bit expert weights, the
 *                 router in full precision, grouped quantisation)
 *   group GEMM    Strata page, section 3.2 (one batched product over the
 *                 experts' contiguous token groups)
 *   slots         Co-inference page, section 2.2 (experts held in GPU cache
 *                 slots); Strata page, section 2.1 (hot-expert pool)
 *   shared expert Strata page, section 2.1 (the shared expert of MoE models,
 *                 kept resident with the layers every token uses)
 *   graph replay  Strata page, section 3.4 (the decode step captured once and
 *                 replayed, with a fixed batch and buffers allocated first)
 *
 * Conventions shared by every entry point
 *   - Every function returns a moe_status; no C++ exception crosses the ABI.
 *     On failure moe_last_error() holds a message for the calling thread.
 *   - Argument checks happen before anything is enqueued: a call that fails
 *     validation has not touched the stream or device memory.
 *   - Device pointers are caller-owned, must be 16-byte aligned, and must stay
 *     valid until the enqueued work completes.  The library allocates no
 *     device memory; all intermediates live in the caller's workspace.
 *   - A workspace must be zero-filled once before its first use, and the
 *     fill must be complete, or ordered on `stream`, when that first call's
 *     work starts (a fill on another stream needs an event or a
 *     synchronisation).  Its first bytes hold control words (completion
 *     tickets of fused kernels) that every call leaves zero again, so later
 *     calls need no clearing.
 *   - moe_forward and moe_graph_launch only enqueue work on `stream` (a
 *     hipStream_t; NULL means the null stream): no host synchronisation.
 *   - Calls that share one workspace must not overlap in time.
 *   - bf16 and fp16 values are passed as their 16-bit patterns (uint16_t).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,          /* null pointer, bad handle, misaligned pointer */
  MOE_ERR_UNSUPPORTED_SHAPE = 2,    /* a shape outside the supported set (see moe_create) */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < moe_workspace_size(T) */
  MOE_ERR_HIP = 4,                  /* a HIP runtime call failed; detail in moe_last_error() */
  MOE_ERR_BAD_STATE = 5             /* e.g. moe_graph_launch before a successful capture */
} moe_status;

/* Device error bits, reported by moe_device_flags. */
#define MOE_FLAG_BAD_SLOT 0x1u      /* slot_table[e] outside [0, num_slots) for an expert with rows;
                                       that expert contributed zero */

typedef struct moe_config {
  int32_t d_model;      /* hidden width d; multiple of 128 */
  int32_t d_ff;         /* expert inner width; multiple of 128 */
  int32_t num_experts;  /* E, routed experts (rows of the router), 1..256 */
  int32_t top_k;        /* k, routed experts per token, 1..min(E, 8) */
  int32_t num_slots;    /* slots in the weight pool, >= 1 */
  int32_t max_tokens;   /* largest T a call may pass, 1..65536 */
  uint32_t flags;       /* reserved, must be 0 */
  int32_t num_shared;   /* shared experts, 0 <= S with k + S <= 8 and E + S <= 256.  Shared
                           expert s has id E + s and the shape of a routed expert; every
                           token takes it with weight exactly 1, after its k routed ones.
                           Its weights are in pool slot slot_table[E + s]. */
  int32_t weight_bits;  /* code width: 4 (int4; 0 also means 4) or 8 */
  int32_t group_size;   /* 0: one (s, z) per output row; 128: one per output row and group of
                           128 consecutive inputs (k) */
} moe_config;

/* Per-slot weight pool (device pointers, caller-owned).  Slot s of a matrix
 * with N output rows and K inputs occupies N*K*B/8 bytes (B = weight_bits):
 * row n holds K codes in 0..2^B-1, int4 two per byte with the even k in the
 * low nibble, 8-bit one per byte.  Scales and zero-points are fp16 (the
 * zero-points integers), indexed by slot: [N] per slot with group_size 0,
 * [K/128][N] per slot (group-major) with group_size 128.  Below, P(N, K)
 * stands for that per-slot shape. */
typedef struct moe_weights {
  const uint8_t *w_gate;   /* [num_slots][d_ff][d_model*B/8] */
  const uint8_t *w_up;     /* [num_slots][d_ff][d_model*B/8] */
  const uint8_t *w_down;   /* [num_slots][d_model][d_ff*B/8] */
  const uint16_t *s_gate, *z_gate;  /* [num_slots] P(d_ff, d_model) */
  const uint16_t *s_up, *z_up;      /* [num_slots] P(d_ff, d_model) */
  const uint16_t *s_down, *z_down;  /* [num_slots] P(d_model, d_ff) */
} moe_weights;

/* Device pointers into a workspace after a forward with T tokens.  With S
 * shared experts every token has K = k + S columns (R = T*K rows, E + S
 * groups): columns 0..k-1 are its routed experts, column k + s is shared
 * expert E + s with weight 1, so each shared group holds all T tokens. */
typedef struct moe_routing {
  const int32_t *topk_idx;  /* [T][K]  routed: logit descending, ties to lower id; then E..E+S-1 */
  const float *topk_w;      /* [T][K]  softmax over the k chosen logits; 1 for shared columns */
  const int32_t *counts;    /* [E+S]   rows per expert */
  const int32_t *offsets;   /* [E+S+1] exclusive prefix sum of counts */
  const int32_t *perm;      /* [R]     grouped position p -> assignment a = t*K + j */
  const int32_t *inv_perm;  /* [R]     assignment a -> grouped position p */
} moe_routing;

typedef struct moe_layer *moe_handle;
typedef void *moe_stream; /* a hipStream_t */

/* Creates a handle for one layer shape.  Host only: no device call, no device
 * allocation.  Returns MOE_ERR_UNSUPPORTED_SHAPE for shapes outside:
 * d_model % 128 == 0, d_ff % 128 == 0, 1 <= E <= 256, 1 <= k <= min(E, 8),
 * num_slots >= 1, 1 <= max_tokens <= 65536, flags == 0, num_shared >= 0,
 * k + num_shared <= 8, E + num_shared <= 256, weight_bits in {0, 4, 8},
 * group_size in {0, 128}. */
moe_status moe_create(const moe_config *cfg, moe_handle *out);

/* Frees the handle and any captured graph.  NULL is ignored. */
void moe_destroy(moe_handle h);

/* Bytes of workspace a forward with T tokens needs (0 <= T <= max_tokens). */
moe_status moe_workspace_size(moe_handle h, int32_t T, size_t *bytes);

/* Bytes at the start of every workspace of this handle that hold control
 * words (completion tickets): the same for every T, zero before first use and
 * left zero by every call. */
moe_status moe_control_bytes(moe_handle h, size_t *bytes);

/* Enqueues the layer forward for T tokens (0 <= T <= max_tokens; T = 0 is a
 * no-op returning MOE_OK).
 *   hidden       bf16 [T][d_model]
 *   router_w     fp32 [E][d_model]
 *   router_bias  fp32 [E], or NULL for none
 *   slot_table   int32 [E + num_shared], device memory, read when the kernels run
 *   w            the slot-indexed weight pool
 *   out          bf16 [T][d_model]
 *   workspace    at least moe_workspace_size(T) bytes, zero-filled before its
 *                first use; holds the routing (see moe_routing_view) and the
 *                device error flags after the call. */
moe_status moe_forward(moe_handle h, int32_t T, const uint16_t *hidden, const float *router_w,
                       const float *router_bias, const int32_t *slot_table, const moe_weights *w,
                       uint16_t *out, void *workspace, size_t workspace_bytes, moe_stream stream);

/* moe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The intermediates live in a fixed 16 MiB device
 * array of the library instead, one copy per device, held until the process
 * ends; the library allocates nothing, and the first call on a device only
 * looks up that array's address and clears its control words with a kernel
 * on `stream`.  Every call on one device shares the array, which keeps the
 * last call's contents: calls that overlap in time on one device (other
 * streams, other threads, other handles) race and must be serialised by the
 * caller.  Arguments as for moe_forward; a shape whose moe_workspace_size(T)
 * exceeds 16 MiB returns MOE_ERR_WORKSPACE_TOO_SMALL before anything is
 * enqueued (all decode shapes up to T = 64 at d_model 4096 and d_ff 14336
 * fit).  The routing and the device error flags of such a call stay in the
 * library's array and are not readable through moe_routing_view or
 * moe_device_flags; a bad slot still makes its expert contribute zero. */
moe_status moe_forward_noalloc(moe_handle h, int32_t T, const uint16_t *hidden, const float *router_w,
                               const float *router_bias, const int32_t *slot_table, const moe_weights *w,
                               uint16_t *out, moe_stream stream);

/* Fills `view` with device pointers to the routing a forward with T tokens
 * left in `workspace`.  Pointer arithmetic only. */
moe_status moe_routing_view(moe_handle h, const void *workspace, int32_t T, moe_routing *view);

/* Captures the enqueue sequence of moe_forward (same arguments) into a HIP
 * graph held by the handle, replacing any earlier capture.  The graph bakes
 * in T and every pointer; the contents of hidden, router weights, the slot
 * table and the weight pool are read at each replay, so the caller may
 * rewrite them between launches.  `stream` must not be NULL. */
moe_status moe_graph_capture(moe_handle h, int32_t T, const uint16_t *hidden, const float *router_w,
                             const float *router_bias, const int32_t *slot_table, const moe_weights *w,
                             uint16_t *out, void *workspace, size_t workspace_bytes, moe_stream stream);

/* Replays the captured graph on `stream`.  MOE_ERR_BAD_STATE without a capture,
 * or when the current device is not the one the graph was captured on (its
 * kernels and pointers belong to that device). */
moe_status moe_graph_launch(moe_handle h, moe_stream stream);

/* Waits for `stream`, then reads the MOE_FLAG_* bits the last forward on
 * `workspace` raised.  Each forward clears the bits when it starts. */
moe_status moe_device_flags(moe_handle h, const void *workspace, int32_t T, moe_stream stream,
                            uint32_t *flags);

/* Optional stage timing for measurement.  With max_forwards > 0 the handle
 * creates HIP events for that many forwards (a setup step: call it outside
 * any timed or captured region), and each eager moe_forward records an event
 * on its stream before the first and after every stage: router, regroup,
 * gate/up GEMM, down GEMM, combine.  0 releases the events.  Graph captures
 * never record stage events. */
moe_status moe_set_stage_timing(moe_handle h, int32_t max_forwards);

/* Waits for the last recorded forward, writes the summed milliseconds of each
 * of the MOE_NUM_STAGES stages over the recorded forwards to ms[] and their
 * number to *forwards, then starts a new recording.  n_stages must be
 * >= MOE_NUM_STAGES. */
#define MOE_NUM_STAGES 5
moe_status moe_stage_times(moe_handle h, float *ms, int32_t n_stages, int32_t *forwards);

/* Static text for a status code. */
const char *moe_status_string(moe_status s);

/* Detail of the calling thread's last failing call ("" if none). */
const char *moe_last_error(void);

/* ---- Expert slot cache and slot refill ------------------------------------
 * Co-inference page, section 2.2: the weight pool's slots form an N-way
 * set-associative cache of (layer, expert) weights -- M ways per set,
 * N = S / M sets -- with LRU replacement.  Section 3.1 and the Strata page,
 * section 2.2: the experts a layer will need are copied host -> device on a
 * second stream while the GPU computes.  The cache only decides which slot
 * holds which expert (host bookkeeping, no device call); the caller enqueues
 * the copies it asks for with moe_expert_upload, orders them before the
 * forward that uses them (an event between the streams), and writes the slot
 * table the request returns to the device. */
typedef struct moe_cache *moe_cache_handle;

/* A cache of num_sets x ways slots (slot = set * ways + way) over experts
 * 0 .. num_experts - 1 of any number of layers.  MOE_ERR_INVALID_ARG unless
 * all three are positive and there are at most 2^24 slots. */
moe_status moe_cache_create(int32_t num_sets, int32_t ways, int32_t num_experts, moe_cache_handle *out);

/* Frees the cache.  NULL is ignored. */
void moe_cache_destroy(moe_cache_handle c);

/* Makes the n experts in `experts` (duplicates allowed) of layer `layer`
 * (>= 0) resident in the layer's set, layer mod num_sets.  Resident ones are
 * hits.  Each missing one takes an empty way of the set (lowest first), else
 * the least recently used way that holds no expert of this request (lowest
 * way among equals), evicting its expert; then every expert of the request
 * counts as used now.
 *   slots         [n] receives the slot of experts[i]
 *   load_experts,
 *   load_slots    [n] receive the experts that were not resident and their
 *                 new slots (*n_loads of them): copy those before use
 *   slot_table    [num_experts] or NULL: receives the layer's slot table, the
 *                 slot of every resident expert and -1 elsewhere (a forward
 *                 treats -1 as missing: the expert contributes zero and
 *                 MOE_FLAG_BAD_SLOT is raised)
 * MOE_ERR_INVALID_ARG for an expert out of range or more distinct experts
 * than ways; the cache is then unchanged. */
moe_status moe_cache_request(moe_cache_handle c, int32_t layer, const int32_t *experts, int32_t n, int32_t *slots,
                             int32_t *load_experts, int32_t *load_slots, int32_t *n_loads, int32_t *slot_table);

/* Hits and misses over all requests so far. */
moe_status moe_cache_stats(moe_cache_handle c, int64_t *hits, int64_t *misses);

/* Pool geometry, Co-inference page, section 2.2: num_slots = floor(free_bytes
 * / expert_bytes) slots in num_sets = floor(num_slots / ways) sets of `ways`
 * (the remaining slots are left out of the cache).  Host arithmetic only.
 * MOE_ERR_INVALID_ARG for a zero expert size, ways < 1 or more than 2^24
 * slots. */
moe_status moe_cache_geometry(uint64_t free_bytes, uint64_t expert_bytes, int32_t ways, int32_t *num_slots,
                              int32_t *num_sets);

/* Bytes of one expert's weights in the handle's format: the codes of gate, up
 * and down plus their fp16 scales and zero-points (one pool slot). */
moe_status moe_expert_bytes(moe_handle h, uint64_t *bytes);

/* Enqueues on `stream` the copies of one expert's weights into pool slot
 * `slot` (0 <= slot < num_slots): `src` holds that expert alone, in the
 * moe_weights layout with a single slot, in host memory (page-locked, for the
 * copies to run asynchronously) or device memory.  Nothing is allocated; the
 * source must stay valid until the copies complete.  The caller orders the
 * copies before any forward that reads the slot (and after any still
 * reading the expert it replaces). */
moe_status moe_expert_upload(moe_handle h, const moe_weights *pool, int32_t slot, const moe_weights *src,
                             moe_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
