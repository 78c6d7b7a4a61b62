// Regroup routed rows by expert id.
//
// Strata page, section 4.2: after routing, tokens are reordered by expert id
// so that each expert's tokens are contiguous and its weights are loaded once
// for all of them; section 3.2 runs the group GEMM over these groups.
//
// One workgroup: an LDS histogram of the expert ids, an exclusive scan, then
// a stable counting-sort scatter.  Rows keep ascending assignment order
// a = t*k + j inside each expert's group: NT assignments are placed per
// round; inside a wave a lane's rank among same-expert lanes comes from
// ballots over the bits of the id, and across waves from per-wave counts in
// LDS.  Also emits the GEMM row-tile list: one descriptor (expert, slot,
// first grouped row, rows) for every tile_rows rows of every non-empty group,
// in expert order.
#include "device_common.h"
#include "plan.h"
#include "regroup.h"

namespace moe {

__global__ __launch_bounds__(kPermuteThreads) void permute_kernel(RegroupArgs a) {
  regroup_block<kPermuteThreads>(a);
}

RegroupArgs regroup_args(const moe_config& c, const Plan& p, const int32_t* slot_table, char* ws) {
  RegroupArgs a;
  a.topk_idx = reinterpret_cast<const int32_t*>(ws + p.topk_idx);
  a.slot_table = slot_table;
  a.R = p.R;
  a.E = c.num_experts;
  a.tile_rows = p.tile_rows;
  a.counts = reinterpret_cast<int32_t*>(ws + p.counts);
  a.offsets = reinterpret_cast<int32_t*>(ws + p.offsets);
  a.perm = reinterpret_cast<int32_t*>(ws + p.perm);
  a.inv = reinterpret_cast<int32_t*>(ws + p.inv);
  a.tiles = reinterpret_cast<int4*>(ws + p.tiles);
  a.num_tiles = reinterpret_cast<int32_t*>(ws + p.num_tiles);
  return a;
}

void launch_permute(const moe_config& c, const Plan& p, const int32_t* slot_table, char* ws, hipStream_t s) {
  permute_kernel<<<1, kPermuteThreads, 0, s>>>(regroup_args(c, p, slot_table, ws));
}

}  // namespace moe
