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

// The same regroup in one pass for R <= NT rows (one row per thread), with
// fewer barriers: the ballot ranks give every wave's count per expert at
// once, so no LDS histogram is needed.  The caller has zeroed the per-wave
// counts, regroup_wave_counts(lds), and passed a barrier since.  Same outputs,
// bit for bit, as regroup_block.
template <int NT>
__device__ __forceinline__ int* regroup_wave_counts(char* lds) {
  return reinterpret_cast<int*>(lds);  // [NT / 64][256]
}
template <int NT>
__device__ void regroup_block_onepass(const RegroupArgs& a, char* lds) {
  constexpr int NW = NT / 64;
  static_assert(NT >= 256, "one thread per expert in the scan");
  int (*wc)[256] = reinterpret_cast<int (*)[256]>(regroup_wave_counts<NT>(lds));
  int* wtot = reinterpret_cast<int*>(lds + NW * 256 * 4);  // [2][4]: the scan's wave totals
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = a.R, E = a.E, tr = a.tile_rows;
  // this row's expert, its rank among the wave's rows of that expert, and
  // (by the first of them) the wave's count of that expert
  const bool valid = tid < R;
  const int e = valid ? a.topk_idx[tid] : 0;
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(peers & lt_mask);
  if (valid && rank == 0) wc[wave][e] = __popcll(peers);
  __syncthreads();
  // thread x < 256: expert x's rows and row tiles, exclusive scans of both
  // over the experts (lane scans, then the totals of the waves before)
  int c = 0, nt = 0, ic = 0, it = 0;
  if (tid < 256) {
    if (tid < E) {
#pragma unroll
      for (int w = 0; w < NW; ++w) c += wc[w][tid];
      nt = (c + tr - 1) / tr;
    }
    ic = c;
    it = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int uc = __shfl_up(ic, off, 64), ut = __shfl_up(it, off, 64);
      if (lane >= off) {
        ic += uc;
        it += ut;
      }
    }
    if (lane == 63) {
      wtot[wave] = ic;
      wtot[4 + wave] = it;
    }
  }
  __syncthreads();
  if (tid < 256) {
    int bc = 0, bt = 0;
    for (int w = 0; w < wave; ++w) {
      bc += wtot[w];
      bt += wtot[4 + w];
    }
    const int base = bc + ic - c;
    if (tid < E) {
      a.offsets[tid] = base;
      a.counts[tid] = c;
      // the waves' first positions in the group, in place of their counts
      int run = base;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int v = wc[w][tid];
        wc[w][tid] = run;
        run += v;
      }
      if (c > 0) {
        const int slot = a.slot_table[tid];
        int ti = bt + it - nt;
        for (int r0 = 0; r0 < c; r0 += tr) a.tiles[ti++] = make_int4(tid, slot, base + r0, min(tr, c - r0));
      }
    }
    if (tid == 255) {
      a.offsets[E] = bc + ic;
      *a.num_tiles = bt + it;
    }
  }
  __syncthreads();
  if (valid) {
    const int pos = wc[wave][e] + rank;
    a.perm[pos] = tid;
    a.inv[tid] = pos;
  }
}

}  // namespace moe
