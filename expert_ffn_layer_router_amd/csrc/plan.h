// Host-side plan of one forward: launch shapes and the carve-up of the
// caller's workspace.  Shared by moe_forward, moe_workspace_size and
// moe_routing_view so that all three agree on every offset.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kRouterTokTile = 16;     // tokens per router block
constexpr int kRouterExpTile = 64;     // experts per router block
constexpr int kRouterKChunk = 64;      // k per router LDS stage
constexpr int kTileRows = 64;          // rows of an expert group per GEMM tile
constexpr int kGemmColsPerBlock = 128; // output columns per GEMM block (4 waves x 32)
constexpr int kGemmKStep = 128;        // k per GEMM load step
constexpr int kPermuteThreads = 1024;

struct Plan {
  int T = 0, R = 0;
  int router_split = 1;   // k-split of the router GEMV
  int down_split = 1;     // k-split of the down projection
  int max_tiles = 0;      // upper bound on GEMM row tiles
  // byte offsets into the workspace
  size_t flags = 0, logit_part = 0, topk_idx = 0, topk_w = 0, counts = 0, offsets = 0,
         perm = 0, inv = 0, tile_e = 0, tile_r0 = 0, num_tiles = 0, h = 0, y = 0, total = 0;
};

// Fills `p` for T tokens.  Pure host arithmetic.
void make_plan(const moe_config& c, int T, Plan* p);

// Kernel launchers (enqueue only).
void launch_router(const moe_config& c, const Plan& p, const uint16_t* hidden, const float* router_w,
                   const float* router_bias, char* ws, hipStream_t s);
void launch_permute(const moe_config& c, const Plan& p, char* ws, hipStream_t s);
void launch_gemms(const moe_config& c, const Plan& p, const uint16_t* hidden, const int32_t* slot_table,
                  const moe_weights& w, char* ws, hipStream_t s);
void launch_combine(const moe_config& c, const Plan& p, uint16_t* out, char* ws, hipStream_t s);

}  // namespace moe
