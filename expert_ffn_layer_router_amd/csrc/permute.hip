// Regroup routed rows by expert id.
//
// Strata page, section 4.2: after routing, tokens are reordered by expert id
// so that each expert's tokens are contiguous and its weights are loaded once
// for all of them; section 3.2 runs the group GEMM over these groups.
//
// One workgroup: per-wave expert counts, an exclusive scan, then a stable
// counting-sort scatter.  Rows keep ascending assignment order a = t*k + j
// inside each expert's group: inside a wave a lane's rank among same-expert
// lanes comes from ballots over the bits of the id, and across waves from the
// per-wave counts in LDS.  Also emits the GEMM row-tile list: one descriptor
// (expert, slot, first grouped row, rows) for every tile_rows rows of every
// non-empty group, in expert order.
#include "device_common.h"
#include "plan.h"
#include "regroup.h"

namespace moe {

__global__ __launch_bounds__(kPermuteThreads) void permute_kernel(RegroupArgs a) {
  // R <= kPermuteThreads: the one-pass form
  __shared__ __attribute__((aligned(16))) char lds[regroup_lds_bytes<kPermuteThreads>()];
  for (int x = threadIdx.x; x < (kPermuteThreads / 64) * 256; x += kPermuteThreads)
    regroup_wave_counts<kPermuteThreads>(lds)[x] = 0;
  __syncthreads();
  regroup_block_onepass<kPermuteThreads>(a, lds);
}

// Many rows: the same regroup over chunks of kPermuteThreads assignments, one
// block each.  regroup_scatter_kernel: chunk b places its rows at offsets[e] +
// (rows of e in chunks before b) + (rank inside the chunk), so rows stay in
// ascending assignment order inside each group; block 0 also writes counts,
// offsets and the tile list.  The counts per expert come from the block's own
// count of all ids (up to kSelfCountChunks chunks), or beyond that from
// regroup_hist_kernel (chunk b's expert histogram to hist[b][e]), run first.
__global__ __launch_bounds__(kPermuteThreads) void regroup_hist_kernel(const int32_t* __restrict__ topk_idx, int R,
                                                                       int E, int32_t* __restrict__ hist) {
  __shared__ int cnt[256];
  for (int e = threadIdx.x; e < E; e += kPermuteThreads) cnt[e] = 0;
  __syncthreads();
  const int i = blockIdx.x * kPermuteThreads + threadIdx.x;
  if (i < R) atomicAdd(&cnt[topk_idx[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermuteThreads) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// hist null: every block counts the expert ids itself (all rows, and the rows
// of the chunks before its own) instead of reading a histogram kernel's
// output -- one kernel less, at the price of each block reading all R ids:
// worth it up to kSelfCountChunks chunks (4 chunks: regroup 11.1 -> 9.7 us;
// 24 chunks of 64 experts: 13 -> 23 us).
constexpr int kSelfCountChunks = 8;
__global__ __launch_bounds__(kPermuteThreads) void regroup_scatter_kernel(RegroupArgs a, const int32_t* __restrict__ hist,
                                                                          int nblocks) {
  constexpr int NW = kPermuteThreads / 64;
  __shared__ int tot[256], base[256], tstart[256];
  __shared__ int wc[NW][256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = a.R, E = a.E, b = blockIdx.x;
  if (!hist) {
    for (int e = tid; e < 256; e += kPermuteThreads) tot[e] = base[e] = 0;
    __syncthreads();
    // four chunks per pass, their ids loaded first; per wave, the first lane
    // of each run of equal ids (ballots over the id's bits) adds the run's size
    for (int c0 = 0; c0 < nblocks; c0 += 4) {
      int ids[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = (c0 + u) * kPermuteThreads + tid;
        ids[u] = i < R ? a.topk_idx[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = ids[u];
        uint64_t peers = __ballot(e >= 0);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
          const bool v = (e >> bit) & 1;
          const uint64_t m = __ballot(v);
          peers &= v ? m : ~m;
        }
        const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        if (e >= 0 && __popcll(peers & lt_mask) == 0) {
          const int n = __popcll(peers);
          atomicAdd(&tot[e], n);
          if (c0 + u < b) atomicAdd(&base[e], n);  // rows of e in earlier chunks
        }
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < E && hist; e += kPermuteThreads) {
    int t = 0, pre = 0;
    for (int q0 = 0; q0 < nblocks; q0 += 8) {  // eight loads in flight at a time
      int h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) h[u] = q0 + u < nblocks ? hist[(size_t)(q0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (q0 + u < b) pre += h[u];
        t += h[u];
      }
    }
    tot[e] = t;
    base[e] = pre;  // rows of e in earlier chunks; the group offset is added below
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scans over experts of the totals and of the tile counts (E <= 256)
    int c[4], nt[4], sc = 0, st = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      c[j] = e < E ? tot[e] : 0;
      nt[j] = (c[j] + a.tile_rows - 1) / a.tile_rows;
      sc += c[j];
      st += nt[j];
    }
    int ic = sc, it = st;
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
        base[e] += rc;
        tstart[e] = rt;
        if (b == 0) {
          a.offsets[e] = rc;
          a.counts[e] = c[j];
        }
      }
      rc += c[j];
      rt += nt[j];
    }
    if (b == 0 && lane == 63) {
      a.offsets[E] = ic;
      *a.num_tiles = it;
    }
  }
  for (int i = tid; i < NW * 256; i += kPermuteThreads) (&wc[0][0])[i] = 0;
  __syncthreads();
  if (b == 0) {  // one descriptor per tile_rows rows of every non-empty group
    for (int e = tid; e < E; e += kPermuteThreads) {
      const int c = tot[e];
      if (c > 0) {
        const int slot = a.slot_table[e];
        const int off = base[e];  // chunk 0: no earlier rows, so this is the group offset
        int ti = tstart[e];
        for (int r0 = 0; r0 < c; r0 += a.tile_rows) a.tiles[ti++] = make_int4(e, slot, off + r0, min(a.tile_rows, c - r0));
      }
    }
  }
  // rank of each row among the chunk's rows of its expert: within a wave from
  // ballots over the bits of the id, across waves from per-wave counts
  const int i = b * kPermuteThreads + tid;
  const bool valid = i < R;
  const int e = valid ? a.topk_idx[i] : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool v = (e >> bit) & 1;
    const uint64_t m = __ballot(v);
    peers &= v ? m : ~m;
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
  const RegroupArgs a = regroup_args(c, p, slot_table, ws);
  const int nb = (p.R + kPermuteThreads - 1) / kPermuteThreads;
  if (nb <= 1) {
    permute_kernel<<<1, kPermuteThreads, 0, s>>>(a);
    return;
  }
  int32_t* hist = nullptr;
  if (nb > kSelfCountChunks) {
    hist = reinterpret_cast<int32_t*>(ws + p.rhist);
    regroup_hist_kernel<<<nb, kPermuteThreads, 0, s>>>(a.topk_idx, p.R, c.num_experts, hist);
  }
  regroup_scatter_kernel<<<nb, kPermuteThreads, 0, s>>>(a, hist, nb);
}

}  // namespace moe
