// Few-token router as a device function: logits = x W_r^T + b summed in
// fp64, the top-k of every token with its renormalised gate weights, and the
// regroup of the routed rows.  Used by the stand-alone router kernel and by
// the decode kernel that runs the router beside the gate/up GEMM.
//
// Strata page, section 1.1: each token picks its top-2 (or top-1) experts.
// Co-inference page, section 5.1: the router stays at full precision.  The
// products bf16 x fp32 are exact in fp64 and are summed in fp64, so the
// selection matches an fp64 evaluation of the logits; exact ties (equal
// logits) go to the lower expert id, because every expert's logit runs
// through the same sequence of operations.
#pragma once

#include "device_common.h"
#include "plan.h"
#include "regroup.h"

namespace moe {

// Top-k of one token, run by one wave: add the bias to the (split-summed)
// logits, then k rounds of a wave-wide arg-max over the experts not yet
// chosen (largest logit, ties to the lower id), then
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).  Token t's row of topk_idx /
// topk_w has kt = k + ns columns: the k routed experts, then the ns shared
// experts E .. E+ns-1 with weight 1.
// kCoherent: read the logits with device-scope coherent loads (they were
// written by other blocks of the same kernel); otherwise plain loads, summing
// nsplit k-split partials.
template <bool kCoherent>
__device__ void topk_token(const double* __restrict__ logits, int nsplit, const float* __restrict__ bias, int T,
                           int E, int k, int ns, int t, int lane, int32_t* __restrict__ topk_idx,
                           float* __restrict__ topk_w) {
  const int kt = k + ns;
  constexpr int kPer = 4;  // experts per lane: E <= 256
  double l[kPer];
  bool live[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + 64 * j;
    live[j] = e < E;
    double v = 0.0;
    if (live[j]) {
      // the splits in order, then the bias; eight loads in flight at a time
      // (a missing split adds +0.0, which changes no sum)
      const double bv = bias ? (double)bias[e] : 0.0;
      auto ld = [&](int s) {
        const double* q = &logits[((size_t)s * T + t) * E + e];
        return kCoherent ? load_coherent(q) : *q;
      };
      for (int s0 = 0; s0 < nsplit; s0 += 8) {
        double p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) p[u] = s0 + u < nsplit ? ld(s0 + u) : 0.0;
#pragma unroll
        for (int u = 0; u < 8; ++u) v += p[u];
      }
      if (bias) v += bv;
    }
    l[j] = v;
  }
  // (loops over the k <= 8 rounds are unrolled with guards, so that these
  // arrays stay in registers: indexed at run time they would live in
  // scratch memory, which every wave of the kernel would then reserve)
  double best[8];
  int bid[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    best[r] = 0.0;
    bid[r] = 0;
    if (r >= k) continue;
    // this lane's best: largest value, lowest id (ids ascend with j)
    double v = 0.0;
    int id = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (live[j] && (id == 0x7fffffff || l[j] > v)) {
        v = l[j];
        id = lane + 64 * j;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(v, off, 64);
      const int oid = __shfl_xor(id, off, 64);
      const bool take = (oid != 0x7fffffff) && (id == 0x7fffffff || ov > v || (ov == v && oid < id));
      if (take) {
        v = ov;
        id = oid;
      }
    }
    best[r] = v;
    bid[r] = id;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (lane + 64 * j == id) live[j] = false;
  }
  // lane j < k takes choice j: exp(l_j - l_0) in parallel, then the sum in
  // order j = 0 .. k-1 (every lane forms the same sum)
  double bj = best[0];
  int ij = bid[0];
#pragma unroll
  for (int r = 1; r < 8; ++r)
    if (lane == r) {
      bj = best[r];
      ij = bid[r];
    }
  const double ex = lane < k ? exp(bj - best[0]) : 0.0;
  double den = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const double ej = __shfl(ex, j, 64);
    if (j < k) den += ej;
  }
  if (lane < k) {
    topk_idx[(size_t)t * kt + lane] = ij;
    topk_w[(size_t)t * kt + lane] = (float)(ex / den);
  }
  if (lane == 0) {
    for (int j = 0; j < ns; ++j) {
      topk_idx[(size_t)t * kt + k + j] = E + j;
      topk_w[(size_t)t * kt + k + j] = 1.0f;
    }
  }
}

struct RouterSmallArgs {
  const uint16_t* hidden;  // [T][d] bf16
  const float* wr;         // [E][d]
  const float* bias;       // [E] or null
  double* logits;          // [nsplit][T][E] partial logits
  int T, d, E, k, ns;      // E, k: routed experts; ns shared ones (columns k .. k+ns-1)
  int nsplit;              // k-splits of d (blocks per expert and token group)
  int32_t* topk_idx;       // [T][k + ns]
  float* topk_w;           // [T][k + ns]
  uint32_t* flags;         // cleared by the finishing block
  uint32_t* ticket;        // completion ticket (a control word, zero between calls)
  // Dense gate/up tiles: per expert (routed and shared) a control word that
  // the finish sets to kMaskKnown | (bit t: token t routed to the expert), with
  // coherent stores, for the gate/up blocks running beside the router; the
  // down GEMM clears them.  Null otherwise.
  uint32_t* tmask;
  RegroupArgs ra;
};
constexpr uint32_t kMaskKnown = 0x80000000u;

// LDS the body needs for a finish that stages up to MAX_TE logits of at most
// MAX_T tokens: per-wave partials and the ticket flag, then the logits, bias,
// slots and chosen ids, then the regroup's working space.
template <int MAX_TE, int MAX_T>
constexpr int router_small_lds_bytes() {
  return 4 * kRouterTokTile * 8 + 16 + (MAX_TE + 1) * 8 + 256 * 8 + 256 * 4 + MAX_T * 8 * 4 + regroup_lds_bytes<256>();
}

// One block of the few-token router: expert e, tokens t0 .. t0+15 (fewer at
// the end), k-split z of a.nsplit, one of `nblocks` blocks.  Its 4 waves take
// a quarter of the split's k range each, lane l accumulating k = 8l .. 8l+7 of
// every 512 for all tokens of the group, the loads of TG tokens in flight at
// a time; a butterfly over the lanes and a fixed-order sum over the 4 waves
// finish each partial logit.  The last block to finish (an atomic ticket)
// then runs the top-k of every token and the regroup, and clears the ticket
// for the next call.  smem: router_small_lds_bytes<MAX_TE, MAX_T>() bytes,
// 16-byte aligned.
template <int MAX_TE, int MAX_T, int TG>
__device__ void router_small_body(const RouterSmallArgs& a, int e, int t0, int z, int nblocks, char* smem) {
  static_assert(kRouterTokTile % TG == 0, "token groups of the load loop");
  double (*part)[kRouterTokTile] = reinterpret_cast<double (*)[kRouterTokTile]>(smem);
  int* is_last = reinterpret_cast<int*>(smem + 4 * kRouterTokTile * 8);
  double* lg = reinterpret_cast<double*>(smem + 4 * kRouterTokTile * 8 + 16);
  double* sbias = lg + MAX_TE + 1;
  int32_t* sslot = reinterpret_cast<int32_t*>(sbias + 256);
  int32_t* sid = sslot + 256;
  char* rg_lds = reinterpret_cast<char*>(sid + MAX_T * 8);  // the regroup's working space
  const int T = a.T, d = a.d, E = a.E, k = a.k, ns = a.ns;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nt = min(kRouterTokTile, T - t0);
  double acc[kRouterTokTile];
#pragma unroll
  for (int t = 0; t < kRouterTokTile; ++t) acc[t] = 0.0;
  const int nsplit = a.nsplit;           // block z covers k in [z d / nsplit, (z + 1) d / nsplit)
  const int kq = d / (4 * nsplit);       // per wave, a multiple of 32
  const int kbeg = z * (d / nsplit) + wave * kq, kend = kbeg + kq;
  const float* wrow = a.wr + (size_t)e * d;
  for (int kk = kbeg + lane * 8; kk < kend; kk += 512) {
    const float4 w0 = *reinterpret_cast<const float4*>(wrow + kk);
    const float4 w1 = *reinterpret_cast<const float4*>(wrow + kk + 4);
    const double wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int h = 0; h < kRouterTokTile; h += TG) {
      u32x4 xv[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t)  // rows past T re-read the group's first row
        xv[t] = *reinterpret_cast<const u32x4*>(a.hidden + (size_t)(t0 + (h + t < nt ? h + t : 0)) * d + kk);
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const uint32_t xs[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[h + t] = fma((double)__uint_as_float(xs[i] << 16), wv[2 * i], acc[h + t]);
          acc[h + t] = fma((double)__uint_as_float(xs[i] & 0xFFFF0000u), wv[2 * i + 1], acc[h + t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouterTokTile; ++t) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[t] += __shfl_xor(acc[t], off, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < kRouterTokTile; ++t) part[wave][t] = acc[t];
  }
  __syncthreads();
  if (wave == 0 && lane < nt) {
    const double v = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
    store_coherent(&a.logits[((size_t)z * T + t0 + lane) * E + e], v);
  }
  // the last block to finish does the top-k of every token and the regroup
  if (!last_block_ticket(a.ticket, (uint32_t)nblocks, is_last)) return;
  if (threadIdx.x == 0) *a.flags = 0u;
  const RegroupArgs& ra = a.ra;
  if (T * E <= MAX_TE && T <= MAX_T) {
    // slot table and the biased fp64 logits into LDS (lg[t * E + e]).  The
    // coherent loads see the latency of the memory side of the L2, so they
    // are issued without conditions, four per thread in flight at a time
    // (indices past the end re-read the last logit and land in a spare LDS
    // slot), together with the bias and slot loads.
    const int TE = T * E;
    for (int i0 = 0; i0 < TE; i0 += 4 * 256) {
      float bv = 0.0f;
      int sl = 0;
      if (i0 == 0 && (int)threadIdx.x < ra.E) {  // slots of routed and shared experts, bias of routed ones
        bv = (a.bias && (int)threadIdx.x < E) ? a.bias[threadIdx.x] : 0.0f;
        sl = ra.slot_table[threadIdx.x];
      }
      // logit = split 0 + split 1 + ... in order; up to kRouterSmallMaxSplit
      // splits are loaded (missing ones re-read split 0 and add zero)
      double v[4], w[4][kRouterSmallMaxSplit - 1];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = min(i0 + (int)threadIdx.x + 256 * u, TE - 1);
        v[u] = load_coherent(&a.logits[i]);
#pragma unroll
        for (int sp = 1; sp < kRouterSmallMaxSplit; ++sp)
          w[u][sp - 1] = load_coherent(&a.logits[(size_t)(sp < nsplit ? sp : 0) * TE + i]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int sp = 1; sp < kRouterSmallMaxSplit; ++sp) v[u] += sp < nsplit ? w[u][sp - 1] : 0.0;
      if (i0 == 0 && (int)threadIdx.x < ra.E) {
        sbias[threadIdx.x] = bv;
        sslot[threadIdx.x] = sl;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + (int)threadIdx.x + 256 * u;
        lg[i < TE ? i : MAX_TE] = v[u] + sbias[i < TE ? i % E : 0];
      }
    }
    __syncthreads();
    // Top-k of every token at once: a segment of S lanes per token (S a power
    // of two, S * T <= 256), lane j of the segment holding experts j, j + S,
    // ...  Each of the k rounds takes every lane's best live expert (largest
    // fp64 logit, lowest id), reduces the segment with a butterfly, and
    // retires the winner; w_j = exp(l_j - l_0) / sum exp(l_i - l_0).
    int S = 64;
    while (S > 1 && S * T > 256) S >>= 1;
    const int seg = threadIdx.x / S, j = threadIdx.x % S;
    const int t = seg;
    if (t < T) {
      const double* lt = lg + (size_t)t * E;
      uint64_t dead = 0;  // bit m: expert j + S m chosen (E / S <= 64)
      double val[8];
      int cid[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        val[r] = 0.0;
        cid[r] = 0;
        if (r < k) {
          double best = 0.0;
          int bid = 0x7fffffff;
          for (int e2 = j, m = 0; e2 < E; e2 += S, ++m) {
            const double v = lt[e2];
            if (!((dead >> m) & 1) && (bid == 0x7fffffff || v > best)) {
              best = v;
              bid = e2;
            }
          }
          for (int off = S >> 1; off >= 1; off >>= 1) {
            const double ov = __shfl_xor(best, off, 64);
            const int oid = __shfl_xor(bid, off, 64);
            if (oid != 0x7fffffff && (bid == 0x7fffffff || ov > best || (ov == best && oid < bid))) {
              best = ov;
              bid = oid;
            }
          }
          val[r] = best;
          cid[r] = bid;
          if (bid % S == j) dead |= 1ull << (bid / S);
        }
      }
      if (j == 0) {
        float ex[8], den = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          ex[r] = r < k ? expf((float)(val[r] - val[0])) : 0.0f;
          den += ex[r];
        }
        const int kt = k + ns;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r < k) {
            a.topk_idx[(size_t)t * kt + r] = cid[r];
            a.topk_w[(size_t)t * kt + r] = ex[r] / den;
            sid[t * kt + r] = cid[r];
          } else if (r < kt) {  // shared experts
            a.topk_idx[(size_t)t * kt + r] = E + r - k;
            a.topk_w[(size_t)t * kt + r] = 1.0f;
            sid[t * kt + r] = E + r - k;
          }
        }
      }
    }
    __syncthreads();
    if (a.tmask && T <= 31) {
      for (int x = threadIdx.x; x < ra.E; x += 256) {
        uint32_t m = 0;
        for (int i = 0; i < T * (k + ns); ++i) m |= (sid[i] == x ? 1u : 0u) << (i / (k + ns));
        __hip_atomic_store(&a.tmask[x], m | kMaskKnown, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    RegroupArgs la = ra;
    la.topk_idx = sid;
    la.slot_table = sslot;
    regroup_block<256>(la, rg_lds);
    if (threadIdx.x == 0) reset_ticket(a.ticket);
    return;
  }
  for (int t = wave; t < T; t += 4)
    topk_token<true>(a.logits, nsplit, a.bias, T, E, k, ns, t, lane, a.topk_idx, a.topk_w);
  __syncthreads();
  regroup_block<256>(ra, rg_lds);
  if (threadIdx.x == 0) reset_ticket(a.ticket);
}

}  // namespace moe
