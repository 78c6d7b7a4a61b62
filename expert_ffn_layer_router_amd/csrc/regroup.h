// Block-level stable regroup of routed rows by expert id (device code shared
// by the stand-alone regroup kernel and the fused few-token router).
#pragma once

#include "device_common.h"

namespace moe {

struct RegroupArgs {
  const int32_t* topk_idx;   // [R] expert id of assignment a = t*k + j
  const int32_t* slot_table; // [E]
  int R, E, tile_rows;
  int32_t* counts;           // [E]
  int32_t* offsets;          // [E+1]
  int32_t* perm;             // [R] grouped position -> assignment
  int32_t* inv;              // [R] assignment -> grouped position
  int4* tiles;               // [max_tiles] (expert, slot, first grouped row, rows)
  int32_t* num_tiles;
};

// LDS bytes regroup_block<NT> works in.
template <int NT>
constexpr int regroup_lds_bytes() { return (3 + NT / 64) * 256 * 4; }

// Runs on one workgroup of NT threads (a multiple of 64, <= 1024).  Callers
// make earlier global writes of topk_idx visible to the block first.  lds:
// regroup_lds_bytes<NT>() bytes of LDS the block does not otherwise use
// meanwhile, 4-byte aligned.
template <int NT>
__device__ void regroup_block(const RegroupArgs& a, char* lds) {
  constexpr int NW = NT / 64;
  int* cnt = reinterpret_cast<int*>(lds);  // [256] rows per expert
  int* base = cnt + 256;                   // [256] running grouped position per expert
  int* tstart = base + 256;                // [256] first row tile per expert
  int (*wc)[256] = reinterpret_cast<int (*)[256]>(tstart + 256);  // [NW][256] per-wave counts
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int R = a.R, E = a.E;

  for (int e = tid; e < E; e += NT) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < R; i += NT) atomicAdd(&cnt[a.topk_idx[i]], 1);
  __syncthreads();
  if (wave == 0) {
    // exclusive scans over experts of the row counts and of the row-tile
    // counts; lane l owns experts 4l .. 4l+3 (E <= 256)
    int c[4], nt[4], sc = 0, st = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      c[j] = e < E ? cnt[e] : 0;
      nt[j] = (c[j] + a.tile_rows - 1) / a.tile_rows;
      sc += c[j];
      st += nt[j];
    }
    int ic = sc, it = st;  // inclusive scans of the lane totals
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int uc = __shfl_up(ic, off, 64), ut = __shfl_up(it, off, 64);
      if (lane >= off) {
        ic += uc;
        it += ut;
      }
    }
    int rc = ic - sc, rt = it - st;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e < E) {
        base[e] = rc;
        tstart[e] = rt;
        a.offsets[e] = rc;
        a.counts[e] = c[j];
      }
      rc += c[j];
      rt += nt[j];
    }
    if (lane == 63) {
      a.offsets[E] = ic;
      *a.num_tiles = it;
    }
  }
  __syncthreads();
  // one descriptor per tile_rows rows of every non-empty group
  for (int e = tid; e < E; e += NT) {
    const int c = cnt[e];
    if (c > 0) {
      const int slot = a.slot_table[e];
      int ti = tstart[e];
      for (int r0 = 0; r0 < c; r0 += a.tile_rows) a.tiles[ti++] = make_int4(e, slot, base[e] + r0, min(a.tile_rows, c - r0));
    }
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int chunk = 0; chunk < R; chunk += NT) {
    for (int i = tid; i < NW * 256; i += NT) (&wc[0][0])[i] = 0;
    __syncthreads();
    const int i = chunk + tid;
    const bool valid = i < R;
    const int e = valid ? a.topk_idx[i] : 0;
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
      a.perm[pos] = i;
      a.inv[i] = pos;
    }
    __syncthreads();
    for (int x = tid; x < E; x += NT) {
      int s = 0;
      for (int w = 0; w < NW; ++w) s += wc[w][x];
      base[x] += s;
    }
    __syncthreads();
  }
}

}  // namespace moe
