// Host-side plan of one forward: launch shapes and the carve-up of the
// caller's workspace.  Shared by moe_forward, moe_workspace_size and
// moe_routing_view so that all three agree on every offset.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kRouterTokTile = 16;     // tokens per router wave
constexpr int kRouterSmallMaxSplit = 4;  // few-token router: at most this many k-splits
constexpr int kRouterMfmaTokens = 64;  // many-token router: tokens per block tile (16 per wave)
constexpr int kRouterMfmaK = 32;       // many-token router: k per LDS chunk
#ifndef MOE_ROUTER_BLOCKS
#define MOE_ROUTER_BLOCKS 512          // many-token router: k-split until about this many blocks
#endif
// many-token router: experts per block tile (a multiple of 16, the MFMA width)
inline int router_tile_experts(int E) { return E > 32 ? 64 : (E > 16 ? 32 : 16); }
constexpr int kPrefillTileRows = 128;  // prefill family: rows of an expert group per GEMM tile
constexpr int kGemmKStep = 128;        // granularity of the decode down GEMM's k-split
constexpr int kPermuteThreads = 1024;
constexpr int kStreamMaxTokens = 64;   // up to this T the decode (weight-streaming) family runs

#ifndef MOE_DOWN_BLOCKS
#define MOE_DOWN_BLOCKS 1024
#endif
#ifndef MOE_STREAM_NCW
#define MOE_STREAM_NCW 1
#endif
constexpr int kStreamCols = 64;                     // decode family: narrowest block (64 output columns)
constexpr int kStreamMaxNCW = MOE_STREAM_NCW;       // decode family: widest block, 64 x this many columns
constexpr int kStreamTileRows = 16;                 // decode family: rows of an expert group per tile
#ifndef MOE_STREAM_RG2_MIN_T_FACTOR
#define MOE_STREAM_RG2_MIN_T_FACTOR 1                   // 32-row decode tiles once T exceeds 16 x this
#endif
constexpr int kDownStreamBlocks = MOE_DOWN_BLOCKS;  // k-split the decode down GEMM up to about this many blocks
#ifndef MOE_STREAM_NCW_DOWN
#define MOE_STREAM_NCW_DOWN MOE_STREAM_NCW
#endif
constexpr int kStreamMaxNCWDown = MOE_STREAM_NCW_DOWN;  // decode-family down GEMM: widest block, 64 x this

enum class GemmFamily { kStream, kPrefill };

struct Plan {
  int T = 0, R = 0;
  GemmFamily family = GemmFamily::kPrefill;
  int router_split = 0;       // 0: few-token router; else k-splits of the tiled router
  int small_split = 1;        // few-token router: k-splits (blocks per expert and token group)
  int gateup_ncw = 1, down_ncw = 1;  // decode family: blocks of 64 x ncw output columns
  int tile_rows = kPrefillTileRows;  // rows of an expert group per GEMM row tile
  int down_split = 1;         // k-split of the down projection
  int max_tiles = 0;          // upper bound on GEMM row tiles
  bool fused_small = false;   // few tokens: router + top-k + regroup in one kernel
  // few tokens: the combine runs in the down kernel (the last block of each
  // column slice); otherwise, with fused_small, a kernel of its own sums the
  // down kernel's fp32 partials
  bool fused_combine = false;
  // few tokens and nearly every expert routed to: dense tiles (every expert
  // with all T tokens), the router launched beside the gate/up GEMM
  bool dense = false;
  // byte offsets into the workspace; [ctrl, ctrl + ctrl_bytes) are control
  // words that must be zero before first use and are left zero by every call
  size_t ctrl = 0, ctrl_bytes = 0, tmask = 0, flags = 0, logits = 0, topk_idx = 0, topk_w = 0, counts = 0,
         offsets = 0, perm = 0, inv = 0, tiles = 0, num_tiles = 0, xsum = 0, hsum_part = 0, h = 0, y = 0,
         xperm = 0, xsum_part = 0, xgsum = 0, rhist = 0, total = 0;
};

// Fills `p` for T tokens.  Pure host arithmetic.
void make_plan(const moe_config& c, int T, Plan* p);

struct RegroupArgs;
RegroupArgs regroup_args(const moe_config& c, const Plan& p, const int32_t* slot_table, char* ws);
struct RouterSmallArgs;
RouterSmallArgs router_small_args(const moe_config& c, const Plan& p, const uint16_t* hidden, const float* router_w,
                                  const float* router_bias, const int32_t* slot_table, char* ws);

// Kernel launchers (enqueue only).
void launch_router(const moe_config& c, const Plan& p, const uint16_t* hidden, const float* router_w,
                   const float* router_bias, const int32_t* slot_table, char* ws, hipStream_t s);
void launch_permute(const moe_config& c, const Plan& p, const int32_t* slot_table, char* ws, hipStream_t s);
void launch_gateup(const moe_config& c, const Plan& p, const uint16_t* hidden, const int32_t* slot_table,
                   const moe_weights& w, char* ws, hipStream_t s);
void launch_down(const moe_config& c, const Plan& p, const int32_t* slot_table, const moe_weights& w, uint16_t* out,
                 char* ws, hipStream_t s);
// decode family (stream_gemm.hip); with p.fused_small the down launch also writes out
void launch_gateup_stream(const moe_config& c, const Plan& p, const uint16_t* hidden, const int32_t* slot_table,
                          const moe_weights& w, char* ws, hipStream_t s);
// p.dense: the router and the gate/up GEMM in one launch
void launch_gateup_router_stream(const moe_config& c, const Plan& p, const uint16_t* hidden, const float* router_w,
                                 const float* router_bias, const int32_t* slot_table, const moe_weights& w,
                                 char* ws, hipStream_t s);
void launch_down_stream(const moe_config& c, const Plan& p, const int32_t* slot_table, const moe_weights& w,
                        uint16_t* out, char* ws, hipStream_t s);
// prefill family (prefill_gemm.hip)
void launch_gateup_prefill(const moe_config& c, const Plan& p, const uint16_t* hidden, const moe_weights& w,
                           char* ws, hipStream_t s);
void launch_down_prefill(const moe_config& c, const Plan& p, const moe_weights& w, char* ws, hipStream_t s);
void launch_combine(const moe_config& c, const Plan& p, uint16_t* out, char* ws, hipStream_t s);
// fused_small without fused_combine: out from the down kernel's fp32 partials
void launch_combine_partials(const moe_config& c, const Plan& p, uint16_t* out, char* ws, hipStream_t s);

}  // namespace moe
