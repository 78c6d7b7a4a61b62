// C ABI of the MoE FFN layer forward: argument checks, the workspace plan,
// the launch sequence, HIP-graph capture and replay, status reporting.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "moe.h"
#include "plan.h"

namespace moe {

void launch_gateup(const moe_config& c, const Plan& p, const uint16_t* hidden, const int32_t* slot_table,
                   const moe_weights& w, char* ws, hipStream_t s) {
  if (p.family == GemmFamily::kStream)
    launch_gateup_stream(c, p, hidden, slot_table, w, ws, s);
  else
    launch_gateup_prefill(c, p, hidden, w, ws, s);
}

void launch_down(const moe_config& c, const Plan& p, const int32_t* slot_table, const moe_weights& w, uint16_t* out,
                 char* ws, hipStream_t s) {
  if (p.family == GemmFamily::kStream)
    launch_down_stream(c, p, slot_table, w, out, ws, s);
  else
    launch_down_prefill(c, p, w, ws, s);
}

}  // namespace moe

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr uint32_t kMagic = 0x4d6f4531u;  // "MoE1"

thread_local std::string g_last_error;

moe_status vfail(moe_status st, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_last_error = buf;
  return st;
}

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int largest_divisor_at_most(int n, int cap) {
  cap = std::max(1, std::min(cap, n));
  for (int q = cap; q >= 1; --q)
    if (n % q == 0) return q;
  return 1;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

struct moe_layer {
  uint32_t magic = kMagic;
  moe_config cfg{};   // as created
  // the shape every kernel after the router sees: shared experts are groups
  // E .. E+S-1 and token columns k .. k+S-1 (num_experts = E + S, top_k = k + S)
  moe_config ecfg{};
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int graph_device = -1;  // the device current when the graph was captured
  int graph_T = 0;        // its token count
  // stage timing: (MOE_NUM_STAGES + 1) events per recorded forward
  std::vector<hipEvent_t> events;
  int timing_capacity = 0;
  int timing_recorded = 0;
};

namespace moe {
// Error reporting and handle checks shared with the library's other host sources.
moe_status api_fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}
bool api_check_handle(moe_handle h, const moe_config** cfg) {
  if (!h || h->magic != kMagic) return false;
  *cfg = &h->ecfg;  // the normalised shape (weight_bits 4 or 8)
  return true;
}
}  // namespace moe

#ifndef MOE_DENSE_IDLE_MAX
#define MOE_DENSE_IDLE_MAX 0.02  // dense tiles while an expert without routed rows is at most this likely
#endif
#ifndef MOE_ROUTER_SMALL_K
#define MOE_ROUTER_SMALL_K 2048  // few-token router: k per block (each wave one 512-k pass)
#endif
#ifndef MOE_FUSED_COMBINE_MAX_T
// Up to this T the down kernel's last blocks run the combine; above it a
// kernel of its own (after a launch gap) beats them: the last block of a
// column slice gathers T x 64 outputs through coherent loads, one round trip
// past the L2 each (T = 64 layer steps: 178 -> 166 us Mixtral-shaped).
#define MOE_FUSED_COMBINE_MAX_T 8
#endif

namespace moe {

void make_plan(const moe_config& c, int T, Plan* p) {
  *p = Plan{};
  p->T = T;
  p->R = T * c.top_k;
  const int E = c.num_experts;                  // groups: routed + shared experts
  const int Er = c.num_experts - c.num_shared;  // rows of the router
  if (T <= kStreamMaxTokens) {
    p->family = GemmFamily::kStream;
    // tiles of 16 rows; of 32 once an expert can have more than 16 rows (each
    // token picks an expert at most once), so that its weights are streamed
    // once for up to 32 of them
    p->tile_rows = T > kStreamTileRows * MOE_STREAM_RG2_MIN_T_FACTOR ? 2 * kStreamTileRows : kStreamTileRows;
  } else {
    p->family = GemmFamily::kPrefill;
    p->tile_rows = kPrefillTileRows;
  }
  p->fused_small = T <= kStreamMaxTokens;
  p->fused_combine = p->fused_small && T <= MOE_FUSED_COMBINE_MAX_T;
  if (T <= kStreamMaxTokens) {
    p->router_split = 0;
    // one 512-k pass per wave (k-split in multiples of 128, up to
    // kRouterSmallMaxSplit); with several token groups, two passes and half the
    // blocks, whose finish then reloads half the partial logits (phi35_skew
    // router 13.5 -> 12.5 us; with one token group, fine_decode, 12.7 -> 13.2)
    const int kblock = MOE_ROUTER_SMALL_K * (T > kRouterTokTile ? 2 : 1);
    p->small_split = largest_divisor_at_most(c.d_model / 128, std::max(1, std::min(kRouterSmallMaxSplit, c.d_model / kblock)));
  } else {
    // 64-token x router_tile_experts(E) tiles; split k (in multiples of 32) until about
    // MOE_ROUTER_BLOCKS blocks
    const int tiles = ((T + kRouterMfmaTokens - 1) / kRouterMfmaTokens) *
                      ((Er + router_tile_experts(Er) - 1) / router_tile_experts(Er));
    p->router_split = largest_divisor_at_most(c.d_model / kRouterMfmaK,
                                              std::max(1, (MOE_ROUTER_BLOCKS + tiles - 1) / tiles));
  }
  // GEMM row tiles: sum_e ceil(c_e / rows) <= ceil(R / rows) + (non-empty experts)
  p->max_tiles = (p->R + p->tile_rows - 1) / p->tile_rows + std::min(E, p->R);
  // Dense tiles: with at most 16 tokens an expert's rows fit one 16-row tile,
  // whose matrix-core work is the same whichever tokens fill it, so every
  // expert can take all T tokens: the gate/up GEMM then needs no routing and
  // runs beside the router; the down GEMM, after it, takes the routed rows.  Worth
  // it when an expert without routed rows -- whose gate/up weights are then
  // streamed for nothing -- is rare: each token picks k of Er experts, so an
  // expert gets no row with probability about (1 - k/Er)^T under even routing.
  {
    const int kr = c.top_k - c.num_shared;
    const double idle = std::pow(1.0 - (double)kr / Er, (double)T);
    // (per-row int4 only: the fused kernel of the other formats spills registers)
    const bool fits = T <= kStreamTileRows && T <= kStreamMaxTokens && T * Er <= 1024 && c.weight_bits == 4 &&
                      c.group_size == 0;
    p->dense = fits && idle <= MOE_DENSE_IDLE_MAX;
  }
  // split the down projection's k range until the grid has enough blocks
  if (p->family == GemmFamily::kStream) {
    p->gateup_ncw = (kStreamMaxNCW >= 2 && c.d_ff % 128 == 0) ? 2 : 1;
    p->down_ncw = (kStreamMaxNCWDown >= 2 && c.d_model % 128 == 0) ? 2 : 1;
    const int blocks = std::max(1, p->max_tiles * (c.d_model / (64 * p->down_ncw)));
    p->down_split = largest_divisor_at_most(c.d_ff / kGemmKStep, (kDownStreamBlocks + blocks - 1) / blocks);
  } else {
    p->down_split = 1;
  }

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  const size_t R = (size_t)p->R;
  // control words, laid out the same for every T: [0] router ticket,
  // [1 + i] combine ticket of output column slice i, then per expert the
  // token mask the router publishes for dense gate/up tiles
  p->tmask = 4 * (1 + (size_t)c.d_model / kStreamCols);
  p->ctrl = take(p->tmask + 4 * (size_t)E);
  p->ctrl_bytes = off;  // aligned end of the control words (they start at offset 0)
  p->flags = take(4);
  p->logits = take(sizeof(double) * (size_t)std::max({1, p->router_split, p->small_split}) * T * Er);
  p->topk_idx = take(4 * R);
  p->topk_w = take(4 * R);
  p->counts = take(4 * (size_t)E);
  p->offsets = take(4 * (size_t)(E + 1));
  p->perm = take(4 * R);
  p->inv = take(4 * R);
  p->tiles = take(16 * (size_t)p->max_tiles);
  p->xsum = take(4 * (size_t)T);
  p->hsum_part = take(4 * R * (size_t)(c.d_ff / 128));
  p->num_tiles = take(4);
  // dense tiles: h holds every expert's rows for all T tokens
  p->h = take(2 * (p->dense ? (size_t)E * T : R) * (size_t)c.d_ff);
  p->y = take(4 * (size_t)p->down_split * R * (size_t)c.d_model);
  // prefill: x in the GEMMs' fragment k-order
  p->xperm = take(p->family == GemmFamily::kPrefill ? 2 * (size_t)T * c.d_model : 0);
  // prefill: per k-split fp64 row sums of x (the router's logits kernel writes them)
  p->xsum_part = take(p->family == GemmFamily::kPrefill ? 8 * (size_t)p->router_split * T : 0);
  // prefill, grouped int4 weights: sums of x per token and group of 128 k
  p->xgsum = take(p->family == GemmFamily::kPrefill && c.group_size && c.weight_bits == 4
                      ? 4 * (size_t)T * (c.d_model / 128)
                      : 0);
  // many rows: per-chunk expert histograms of the regroup
  p->rhist = take(p->family == GemmFamily::kPrefill ? 4 * (size_t)((p->R + kPermuteThreads - 1) / kPermuteThreads) * E : 0);
  p->total = off;
}

}  // namespace moe

namespace {

moe_status check_handle(moe_handle h) {
  if (!h || h->magic != kMagic) return fail(MOE_ERR_INVALID_ARG, "invalid handle");
  return MOE_OK;
}

moe_status check_T(const moe_layer* h, int32_t T) {
  if (T < 0 || T > h->cfg.max_tokens)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T=%d outside [0, max_tokens=%d]", T, h->cfg.max_tokens);
  return MOE_OK;
}

// workspace_bytes value for checking every argument but the workspace
constexpr size_t kNoWorkspace = ~size_t(0);

moe_status check_forward_args(moe_handle h, int32_t T, const uint16_t* hidden, const float* router_w,
                              const float* router_bias, const int32_t* slot_table, const moe_weights* w,
                              uint16_t* out, void* workspace, size_t workspace_bytes, moe::Plan* plan) {
  moe_status st = check_handle(h);
  if (st != MOE_OK) return st;
  if ((st = check_T(h, T)) != MOE_OK) return st;
  moe::make_plan(h->ecfg, T, plan);
  if (T == 0) return MOE_OK;
  if (!hidden || !router_w || !slot_table || !w || !out || (!workspace && workspace_bytes != kNoWorkspace))
    return fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  if (!w->w_gate || !w->w_up || !w->w_down || !w->s_gate || !w->z_gate || !w->s_up || !w->z_up ||
      !w->s_down || !w->z_down)
    return fail(MOE_ERR_INVALID_ARG, "null pointer in moe_weights");
  const void* a16[] = {hidden, router_w, out, workspace, w->w_gate, w->w_up, w->w_down};
  for (const void* p : a16)
    if (!aligned(p, 16)) return fail(MOE_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
  const void* a4[] = {slot_table, router_bias};
  for (const void* p : a4)
    if (p && !aligned(p, 4)) return fail(MOE_ERR_INVALID_ARG, "pointer %p is not 4-byte aligned", p);
  const void* a2[] = {w->s_gate, w->z_gate, w->s_up, w->z_up, w->s_down, w->z_down};
  for (const void* p : a2)
    if (!aligned(p, 2)) return fail(MOE_ERR_INVALID_ARG, "pointer %p is not 2-byte aligned", p);
  if (workspace_bytes == kNoWorkspace) return MOE_OK;  // the caller supplies the workspace later
  if (workspace_bytes < plan->total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, T=%d needs %zu", workspace_bytes, T,
                plan->total);
  return MOE_OK;
}

moe_status enqueue(moe_layer* h, const moe::Plan& p, const uint16_t* hidden, const float* router_w,
                   const float* router_bias, const int32_t* slot_table, const moe_weights* w, uint16_t* out,
                   void* workspace, hipStream_t s, bool capturing) {
  char* ws = static_cast<char*>(workspace);
  hipEvent_t* ev = nullptr;
  if (!capturing && h->timing_recorded < h->timing_capacity)
    ev = &h->events[(size_t)h->timing_recorded++ * (MOE_NUM_STAGES + 1)];
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], s);
  };
  // with few tokens the regroup runs inside the router kernel and the
  // combine inside the down kernel (their stages then time as empty)
  // with dense tiles the router runs in the gate/up launch (its stages then
  // time as empty too)
  const moe_config& c = h->ecfg;
  mark(0);
  if (!p.dense) moe::launch_router(c, p, hidden, router_w, router_bias, slot_table, ws, s);
  mark(1);
  if (!p.fused_small) moe::launch_permute(c, p, slot_table, ws, s);
  mark(2);
  if (p.dense)
    moe::launch_gateup_router_stream(c, p, hidden, router_w, router_bias, slot_table, *w, ws, s);
  else
    moe::launch_gateup(c, p, hidden, slot_table, *w, ws, s);
  mark(3);
  moe::launch_down(c, p, slot_table, *w, out, ws, s);
  mark(4);
  if (!p.fused_small)
    moe::launch_combine(c, p, out, ws, s);
  else if (!p.fused_combine)
    moe::launch_combine_partials(c, p, out, ws, s);
  mark(5);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return MOE_OK;
}

void drop_events(moe_layer* h) {
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  h->events.clear();
  h->timing_capacity = h->timing_recorded = 0;
}

void drop_graph(moe_layer* h) {
  if (h->exec) (void)hipGraphExecDestroy(h->exec);
  if (h->graph) (void)hipGraphDestroy(h->graph);
  h->exec = nullptr;
  h->graph = nullptr;
}

}  // namespace

MOE_EXPORT moe_status moe_create(const moe_config* cfg, moe_handle* out) {
  if (!cfg || !out) return fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  *out = nullptr;
  const moe_config& c = *cfg;
  if (c.flags != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "flags must be 0");
  if (c.d_model <= 0 || c.d_model % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "d_model=%d must be a positive multiple of 128", c.d_model);
  if (c.d_ff <= 0 || c.d_ff % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "d_ff=%d must be a positive multiple of 128", c.d_ff);
  if (c.num_experts < 1 || c.num_experts > 256)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "num_experts=%d outside [1, 256]", c.num_experts);
  if (c.top_k < 1 || c.top_k > std::min(c.num_experts, 8))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "top_k=%d outside [1, min(E, 8)]", c.top_k);
  if (c.num_slots < 1) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "num_slots=%d must be >= 1", c.num_slots);
  if (c.max_tokens < 1 || c.max_tokens > 65536)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "max_tokens=%d outside [1, 65536]", c.max_tokens);
  if (c.num_shared < 0 || c.top_k + c.num_shared > 8 || c.num_experts + c.num_shared > 256)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "num_shared=%d: need >= 0, top_k + num_shared <= 8 and "
                "num_experts + num_shared <= 256", c.num_shared);
  if (c.weight_bits != 0 && c.weight_bits != 4 && c.weight_bits != 8)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "weight_bits=%d must be 0, 4 or 8", c.weight_bits);
  if (c.group_size != 0 && c.group_size != 128)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "group_size=%d must be 0 or 128", c.group_size);
  moe_layer* h = new (std::nothrow) moe_layer;
  if (!h) return fail(MOE_ERR_INVALID_ARG, "out of host memory");
  h->cfg = c;
  h->ecfg = c;
  h->ecfg.num_experts = c.num_experts + c.num_shared;
  h->ecfg.top_k = c.top_k + c.num_shared;
  if (h->ecfg.weight_bits == 0) h->ecfg.weight_bits = 4;
  *out = h;
  return MOE_OK;
}

MOE_EXPORT void moe_destroy(moe_handle h) {
  if (!h || h->magic != kMagic) return;
  drop_graph(h);
  drop_events(h);
  h->magic = 0;
  delete h;
}

MOE_EXPORT moe_status moe_control_bytes(moe_handle h, size_t* bytes) {
  moe_status st = check_handle(h);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  moe::Plan p;
  moe::make_plan(h->ecfg, 0, &p);
  *bytes = p.ctrl_bytes;
  return MOE_OK;
}

MOE_EXPORT moe_status moe_workspace_size(moe_handle h, int32_t T, size_t* bytes) {
  moe_status st = check_handle(h);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  if ((st = check_T(h, T)) != MOE_OK) return st;
  moe::Plan p;
  moe::make_plan(h->ecfg, T, &p);
  *bytes = p.total;
  return MOE_OK;
}

MOE_EXPORT moe_status moe_forward(moe_handle h, int32_t T, const uint16_t* hidden, const float* router_w,
                                  const float* router_bias, const int32_t* slot_table, const moe_weights* w,
                                  uint16_t* out, void* workspace, size_t workspace_bytes, moe_stream stream) {
  moe::Plan p;
  moe_status st = check_forward_args(h, T, hidden, router_w, router_bias, slot_table, w, out, workspace,
                                     workspace_bytes, &p);
  if (st != MOE_OK || T == 0) return st;
  return enqueue(h, p, hidden, router_w, router_bias, slot_table, w, out, workspace,
                 static_cast<hipStream_t>(stream), false);
}

MOE_EXPORT moe_status moe_routing_view(moe_handle h, const void* workspace, int32_t T, moe_routing* view) {
  moe_status st = check_handle(h);
  if (st != MOE_OK) return st;
  if (!workspace || !view) return fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  if ((st = check_T(h, T)) != MOE_OK) return st;
  moe::Plan p;
  moe::make_plan(h->ecfg, T, &p);
  const char* ws = static_cast<const char*>(workspace);
  view->topk_idx = reinterpret_cast<const int32_t*>(ws + p.topk_idx);
  view->topk_w = reinterpret_cast<const float*>(ws + p.topk_w);
  view->counts = reinterpret_cast<const int32_t*>(ws + p.counts);
  view->offsets = reinterpret_cast<const int32_t*>(ws + p.offsets);
  view->perm = reinterpret_cast<const int32_t*>(ws + p.perm);
  view->inv_perm = reinterpret_cast<const int32_t*>(ws + p.inv);
  return MOE_OK;
}

MOE_EXPORT moe_status moe_graph_capture(moe_handle h, int32_t T, const uint16_t* hidden, const float* router_w,
                                        const float* router_bias, const int32_t* slot_table,
                                        const moe_weights* w, uint16_t* out, void* workspace,
                                        size_t workspace_bytes, moe_stream stream) {
  moe::Plan p;
  moe_status st = check_forward_args(h, T, hidden, router_w, router_bias, slot_table, w, out, workspace,
                                     workspace_bytes, &p);
  if (st != MOE_OK) return st;
  if (!stream) return fail(MOE_ERR_INVALID_ARG, "graph capture needs a non-null stream");
  if (T == 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "graph capture needs T > 0");
  int device = -1;
  hipError_t err = hipGetDevice(&device);
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
  // The new graph replaces the held one only once it is instantiated: a
  // failed capture leaves the handle's earlier graph (if any) in place.
  hipStream_t s = static_cast<hipStream_t>(stream);
  err = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(err));
  const moe_status est = enqueue(h, p, hidden, router_w, router_bias, slot_table, w, out, workspace, s, true);
  hipGraph_t graph = nullptr;
  err = hipStreamEndCapture(s, &graph);
  if (est != MOE_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return est;
  }
  if (err != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return fail(MOE_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(err));
  }
  hipGraphExec_t exec = nullptr;
  err = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (err != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(MOE_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(err));
  }
  drop_graph(h);
  h->graph = graph;
  h->exec = exec;
  h->graph_device = device;
  h->graph_T = T;
  return MOE_OK;
}

MOE_EXPORT moe_status moe_graph_launch(moe_handle h, moe_stream stream) {
  moe_status st = check_handle(h);
  if (st != MOE_OK) return st;
  if (!h->exec) return fail(MOE_ERR_BAD_STATE, "no captured graph");
  int device = -1;
  hipError_t err = hipGetDevice(&device);
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
  // the graph's kernels and pointers belong to the device it was captured on
  if (device != h->graph_device)
    return fail(MOE_ERR_BAD_STATE, "graph (T=%d) was captured on device %d, device %d is current", h->graph_T,
                h->graph_device, device);
  err = hipGraphLaunch(h->exec, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGraphLaunch: %s", hipGetErrorString(err));
  return MOE_OK;
}

MOE_EXPORT moe_status moe_device_flags(moe_handle h, const void* workspace, int32_t T, moe_stream stream,
                                       uint32_t* flags) {
  moe_status st = check_handle(h);
  if (st != MOE_OK) return st;
  if (!workspace || !flags) return fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  if ((st = check_T(h, T)) != MOE_OK) return st;
  moe::Plan p;
  moe::make_plan(h->ecfg, T, &p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t err = hipMemcpyAsync(&v, static_cast<const char*>(workspace) + p.flags, sizeof v,
                                  hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "reading device flags: %s", hipGetErrorString(err));
  *flags = v;
  return MOE_OK;
}

MOE_EXPORT moe_status moe_set_stage_timing(moe_handle h, int32_t max_forwards) {
  moe_status st = check_handle(h);
  if (st != MOE_OK) return st;
  if (max_forwards < 0 || max_forwards > 100000)
    return fail(MOE_ERR_INVALID_ARG, "max_forwards=%d outside [0, 100000]", max_forwards);
  drop_events(h);
  const size_t n = (size_t)max_forwards * (MOE_NUM_STAGES + 1);
  h->events.reserve(n);
  for (size_t i = 0; i < n; ++i) {
    hipEvent_t e = nullptr;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      drop_events(h);
      return fail(MOE_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    }
    h->events.push_back(e);
  }
  h->timing_capacity = max_forwards;
  return MOE_OK;
}

MOE_EXPORT moe_status moe_stage_times(moe_handle h, float* ms, int32_t n_stages, int32_t* forwards) {
  moe_status st = check_handle(h);
  if (st != MOE_OK) return st;
  if (!ms || !forwards) return fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  if (n_stages < MOE_NUM_STAGES) return fail(MOE_ERR_INVALID_ARG, "n_stages=%d < %d", n_stages, MOE_NUM_STAGES);
  for (int i = 0; i < MOE_NUM_STAGES; ++i) ms[i] = 0.0f;
  const int n = h->timing_recorded;
  if (n > 0) {
    hipError_t err = hipEventSynchronize(h->events[(size_t)n * (MOE_NUM_STAGES + 1) - 1]);
    for (int f = 0; f < n && err == hipSuccess; ++f) {
      const hipEvent_t* ev = &h->events[(size_t)f * (MOE_NUM_STAGES + 1)];
      for (int i = 0; i < MOE_NUM_STAGES && err == hipSuccess; ++i) {
        float t = 0.0f;
        err = hipEventElapsedTime(&t, ev[i], ev[i + 1]);
        ms[i] += t;
      }
    }
    if (err != hipSuccess) return fail(MOE_ERR_HIP, "reading stage events: %s", hipGetErrorString(err));
  }
  *forwards = n;
  h->timing_recorded = 0;
  return MOE_OK;
}

MOE_EXPORT const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_BAD_STATE: return "MOE_ERR_BAD_STATE";
  }
  return "MOE_ERR_UNKNOWN";
}

MOE_EXPORT const char* moe_last_error(void) { return g_last_error.c_str(); }

// ---- Allocation-free forward -------------------------------------------------
// moe_forward with the workspace taken from a fixed device array of this
// library instead of the caller: for callers that cannot allocate device
// memory.  Each device holds its own copy of the array until the process
// ends; its address on a device comes from hipGetSymbolAddress, called once
// per device with that device current, and only that address is handed to
// the kernels.  Every call on a device shares the array.
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
size_t g_scratch_clear[kMaxDevices] = {};  // leading bytes of the array cleared by a launched kernel

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's copy of the scratch array; the first call on a device
// looks its address up.
moe_status scratch_of_current_device(void** ptr, int* device) {
  hipError_t err = hipGetDevice(device);
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
  if (*device < 0 || *device >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "device %d outside [0, %d)", *device, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[*device]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(err));
    g_scratch_ptr[*device] = p;
  }
  *ptr = g_scratch_ptr[*device];
  return MOE_OK;
}

}  // namespace

MOE_EXPORT moe_status moe_forward_noalloc(moe_handle h, int32_t T, const uint16_t* hidden, const float* router_w,
                                          const float* router_bias, const int32_t* slot_table,
                                          const moe_weights* w, uint16_t* out, moe_stream stream) {
  moe_status st = check_handle(h);
  if (st != MOE_OK) return st;
  if ((st = check_T(h, T)) != MOE_OK) return st;
  moe::Plan p;
  moe::make_plan(h->ecfg, T, &p);
  if (T == 0) return MOE_OK;
  if (p.total > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "T=%d needs %zu bytes of workspace; the static scratch holds %zu (use moe_forward with a "
                "caller workspace)", T, p.total, kScratchBytes);
  // every argument is checked before the first device call
  if ((st = check_forward_args(h, T, hidden, router_w, router_bias, slot_table, w, out, nullptr, kNoWorkspace,
                               &p)) != MOE_OK)
    return st;
  void* ws = nullptr;
  int device = -1;
  if ((st = scratch_of_current_device(&ws, &device)) != MOE_OK) return st;
  if ((st = check_forward_args(h, T, hidden, router_w, router_bias, slot_table, w, out, ws, kScratchBytes, &p)) !=
      MOE_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  {
    // The control words at the start of the array must be zero before their
    // first use (every call leaves them zero): clear them once per device, by
    // a kernel on the caller's stream.
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_clear[device] < p.ctrl_bytes) {
      clear_words_kernel<<<1, 256, 0, s>>>(static_cast<uint32_t*>(ws), (int)(p.ctrl_bytes / 4));
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return fail(MOE_ERR_HIP, "clearing the scratch control words: %s", hipGetErrorString(err));
      g_scratch_clear[device] = p.ctrl_bytes;
    }
  }
  return enqueue(h, p, hidden, router_w, router_bias, slot_table, w, out, ws, s, false);
}
