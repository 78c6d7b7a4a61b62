// Regroup routed rows by expert id.
//
// Strata page, section 4.2: after routing, tokens are reordered by expert id
// so that each expert's tokens are contiguous and its weights are loaded once
// for all of them; section 3.2 runs the group GEMM over these groups.
//
// One workgroup: an LDS histogram of the expert ids, an exclusive scan, then
// a stable counting-sort scatter.  Rows keep ascending assignment order
// a = t*k + j inside each expert's group: 1024 assignments are placed per
// round; inside a wave a lane's rank among same-expert lanes comes from
// ballots over the bits of the id, and across waves from per-wave counts in
// LDS.  Also emits the GEMM row-tile list: (expert, first row) for every
// kTileRows rows of every non-empty group, in expert order.
#include "device_common.h"
#include "plan.h"

namespace moe {

constexpr int kPermWaves = kPermuteThreads / 64;

__global__ __launch_bounds__(kPermuteThreads) void permute_kernel(
    const int32_t* __restrict__ topk_idx, int R, int E, int tile_rows, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_r0, int32_t* __restrict__ num_tiles) {
  __shared__ int cnt[256];
  __shared__ int base[256];
  __shared__ int wc[kPermWaves][256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  for (int e = tid; e < E; e += kPermuteThreads) cnt[e] = 0;
  __syncthreads();
  for (int a = tid; a < R; a += kPermuteThreads) atomicAdd(&cnt[topk_idx[a]], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0, nt = 0;
    for (int e = 0; e < E; ++e) {
      const int c = cnt[e];
      base[e] = run;
      offsets[e] = run;
      counts[e] = c;
      for (int r0 = 0; r0 < c; r0 += tile_rows) {
        tile_e[nt] = e;
        tile_r0[nt] = r0;
        ++nt;
      }
      run += c;
    }
    offsets[E] = run;
    *num_tiles = nt;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int chunk = 0; chunk < R; chunk += kPermuteThreads) {
    for (int i = tid; i < kPermWaves * 256; i += kPermuteThreads) (&wc[0][0])[i] = 0;
    __syncthreads();
    const int a = chunk + tid;
    const bool valid = a < R;
    const int e = valid ? topk_idx[a] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wc[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wc[w][e];
      perm[pos] = a;
      inv[a] = pos;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kPermuteThreads) {
      int s = 0;
      for (int w = 0; w < kPermWaves; ++w) s += wc[w][x];
      base[x] += s;
    }
    __syncthreads();
  }
}

void launch_permute(const moe_config& c, const Plan& p, char* ws, hipStream_t s) {
  permute_kernel<<<1, kPermuteThreads, 0, s>>>(
      reinterpret_cast<const int32_t*>(ws + p.topk_idx), p.R, c.num_experts, kTileRows,
      reinterpret_cast<int32_t*>(ws + p.counts), reinterpret_cast<int32_t*>(ws + p.offsets),
      reinterpret_cast<int32_t*>(ws + p.perm), reinterpret_cast<int32_t*>(ws + p.inv),
      reinterpret_cast<int32_t*>(ws + p.tile_e), reinterpret_cast<int32_t*>(ws + p.tile_r0),
      reinterpret_cast<int32_t*>(ws + p.num_tiles));
}

}  // namespace moe
