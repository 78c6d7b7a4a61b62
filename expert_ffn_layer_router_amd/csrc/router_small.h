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

constexpr int kNoExpert = 0x7fffffff;

// A lane's partner value in a DPP exchange inside its row of 16 lanes (CTRL:
// a quad permutation or a row mirror, each an involution).
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Max (NaN ignored) and min over an aligned segment of 2^LGS <= 16 lanes:
// lane ^ 1, lane ^ 2, then the half-row and row mirrors; after the LGS steps
// every lane of the segment holds the result.
template <int LGS>
__device__ __forceinline__ double segment_max(double v) {
  if constexpr (LGS >= 1) v = fmax(v, dpp_f64<0xB1>(v));
  if constexpr (LGS >= 2) v = fmax(v, dpp_f64<0x4E>(v));
  if constexpr (LGS >= 3) v = fmax(v, dpp_f64<0x141>(v));
  if constexpr (LGS >= 4) v = fmax(v, dpp_f64<0x140>(v));
  return v;
}
template <int LGS>
__device__ __forceinline__ int segment_min(int v) {
  if constexpr (LGS >= 1) v = min(v, dpp_i32<0xB1>(v));
  if constexpr (LGS >= 2) v = min(v, dpp_i32<0x4E>(v));
  if constexpr (LGS >= 3) v = min(v, dpp_i32<0x141>(v));
  if constexpr (LGS >= 4) v = min(v, dpp_i32<0x140>(v));
  return v;
}

// Order of the segment top-k: a beats b if its logit is larger, or equal
// with a lower id; a NaN logit (no expert, or one already chosen) beats
// nothing and loses to everything else.
__device__ __forceinline__ bool beats(double a, int ia, double b, int ib) {
  return !__builtin_isnan(a) && (__builtin_isnan(b) || a > b || (a == b && ia < ib));
}
__device__ __forceinline__ void order_pair(double& a, int& ia, double& b, int& ib) {
  const bool sw = beats(b, ib, a, ia);
  const double x = a;
  const int ix = ia;
  a = sw ? b : a;
  ia = sw ? ib : ia;
  b = sw ? x : b;
  ib = sw ? ix : ib;
}

// The k <= 8 rounds of the top-k of one token over a segment of 2^LGS lanes,
// lane j holding experts j + 2^LGS m (m < 4): h[m], hid[m] its logits and ids
// (NaN and kNoExpert where it has none).  Every lane of the segment ends with
// the chosen logits and ids in round order.  The lane sorts its four (logit,
// id) pairs once, then each round reduces the heads of the segment's lanes
// (the largest logit, then the lowest id holding it) and the winning lane pops
// its head.
template <int LGS, int K8 = 8>
__device__ __forceinline__ void topk_rounds_heads(double (&h)[4], int (&hid)[4], int k, double (&val)[K8],
                                                  int (&cid)[K8]) {
  order_pair(h[0], hid[0], h[1], hid[1]);
  order_pair(h[2], hid[2], h[3], hid[3]);
  order_pair(h[0], hid[0], h[2], hid[2]);
  order_pair(h[1], hid[1], h[3], hid[3]);
  order_pair(h[1], hid[1], h[2], hid[2]);
#pragma unroll
  for (int r = 0; r < K8; ++r) {
    val[r] = 0.0;
    cid[r] = 0;
    if (r < k) {
      const double smx = segment_max<LGS>(h[0]);
      const int win = segment_min<LGS>(h[0] == smx ? hid[0] : kNoExpert);
      val[r] = smx;
      cid[r] = win;
      const bool pop = hid[0] == win;
      h[0] = pop ? h[1] : h[0];
      hid[0] = pop ? hid[1] : hid[0];
      h[1] = pop ? h[2] : h[1];
      hid[1] = pop ? hid[2] : hid[1];
      h[2] = pop ? h[3] : h[2];
      hid[2] = pop ? hid[3] : hid[2];
      h[3] = pop ? __builtin_nan("") : h[3];
      hid[3] = pop ? kNoExpert : hid[3];
    }
  }
}

// The same with the token's E <= 4 * 2^LGS logits in LDS (lt).
template <int LGS, int K8 = 8>
__device__ __forceinline__ void topk_rounds_sorted(const double* lt, int E, int k, int j, double (&val)[K8],
                                                   int (&cid)[K8]) {
  double h[4];
  int hid[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e2 = j + (m << LGS);
    const double x = lt[min(e2, E - 1)];
    h[m] = e2 < E ? x : __builtin_nan("");
    hid[m] = e2 < E ? e2 : kNoExpert;
  }
  topk_rounds_heads<LGS>(h, hid, k, val, cid);
}

// The same for more than four experts per lane: each round scans the lane's
// logits in LDS (four loads in flight), reduces the segment, and retires the
// winner by writing NaN over its logit (the LDS accesses of one wave take
// effect in order, so the next round's reads see it).
template <int LGS, int K8 = 8>
__device__ __forceinline__ void topk_rounds_scan(double* lt, int E, int k, int j, double (&val)[K8],
                                                 int (&cid)[K8]) {
#pragma unroll
  for (int r = 0; r < K8; ++r) {
    val[r] = 0.0;
    cid[r] = 0;
    if (r < k) {
      double mx = __builtin_nan("");
      int id = kNoExpert;
      for (int m0 = 0; j + (m0 << LGS) < E; m0 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e2 = j + ((m0 + u) << LGS);
          const double x = lt[min(e2, E - 1)];
          const double v = e2 < E ? x : __builtin_nan("");
          const bool take = beats(v, e2, mx, id);
          mx = take ? v : mx;
          id = take ? e2 : id;
        }
      }
      const double smx = segment_max<LGS>(mx);
      const int win = segment_min<LGS>(mx == smx ? id : kNoExpert);
      val[r] = smx;
      cid[r] = win;
      if ((win & ((1 << LGS) - 1)) == j) lt[win] = __builtin_nan("");
    }
  }
}

template <int LGS>
__device__ __forceinline__ void topk_rounds(double* lt, int E, int k, int j, double (&val)[8], int (&cid)[8]) {
  if (E <= (4 << LGS))
    topk_rounds_sorted<LGS>(lt, E, k, j, val, cid);
  else
    topk_rounds_scan<LGS>(lt, E, k, j, val, cid);
}

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
// a time; a reduce-scatter over the lanes and a fixed-order sum over the 4
// waves finish each partial logit.  The last block to finish (an atomic ticket)
// then runs the top-k of every token and the regroup, and clears the ticket
// for the next call.  smem: router_small_lds_bytes<MAX_TE, MAX_T>() bytes,
// 16-byte aligned.  kWaveFinish = false leaves out the finish for T * E >
// MAX_TE or T > MAX_T (one wave per token reading the logits from memory): its
// caller's plan never runs such shapes, and that code would need scratch
// memory beside a GEMM's register budget.
template <int MAX_TE, int MAX_T, int TG, bool kWaveFinish = true>
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
  // Reduce-scatter over the lanes: at the exchanges with lane ^ 32, ^ 16, ^ 8
  // and ^ 4 each lane keeps half of its tokens and adds its partner's half, so
  // that a lane ends with one token, 8 b5 + 4 b4 + 2 b3 + b2 (b_i: bit i of
  // the lane), summed over 16 lanes; lane ^ 2 and ^ 1 finish the sum.  Every
  // logit of a token takes the same sequence of additions.
  static_assert(kRouterTokTile == 16, "four halving exchanges");
  double r8[8], r4[4], r2[2], r1;
  {
    const bool hi = lane & 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) r8[i] = (hi ? acc[8 + i] : acc[i]) + __shfl_xor(hi ? acc[i] : acc[8 + i], 32, 64);
  }
  {
    const bool hi = lane & 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) r4[i] = (hi ? r8[4 + i] : r8[i]) + __shfl_xor(hi ? r8[i] : r8[4 + i], 16, 64);
  }
  {
    const bool hi = lane & 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) r2[i] = (hi ? r4[2 + i] : r4[i]) + __shfl_xor(hi ? r4[i] : r4[2 + i], 8, 64);
  }
  {
    const bool hi = lane & 4;
    r1 = (hi ? r2[1] : r2[0]) + __shfl_xor(hi ? r2[0] : r2[1], 4, 64);
  }
  r1 += __shfl_xor(r1, 2, 64);
  r1 += __shfl_xor(r1, 1, 64);
  if ((lane & 3) == 0)
    part[wave][((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1)] = r1;
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
    // Top-k of every token at once: a segment of S = 2^lgS lanes per token
    // (S <= 16, S * T <= 256), lane j of the segment holding experts j,
    // j + S, ...; k rounds each take the largest live logit of the segment (a
    // max reduction with DPP exchanges inside the lane's row of 16), then the
    // lowest id holding it (a min reduction), and retire that expert
    // (topk_rounds).  NaN marks "no expert" (fmax ignores it, and it equals
    // nothing; the logits of finite inputs are finite).  This code runs on one
    // block while the rest of the GPU waits, so it is written for a short
    // dependent chain per round rather than for throughput.
    // w_j = exp(l_j - l_0) / sum exp(l_i - l_0).
    int lgS = 4;
    while (lgS > 0 && (T << lgS) > 256) --lgS;
    const int S = 1 << lgS;
    const int t = threadIdx.x >> lgS, j = threadIdx.x & (S - 1);
    if (t < T) {  // segments are aligned, so a segment is wholly inside or outside
      double* lt = lg + (size_t)t * E;
      double val[8];
      int cid[8];
      switch (lgS) {
        case 4: topk_rounds<4>(lt, E, k, j, val, cid); break;
        case 3: topk_rounds<3>(lt, E, k, j, val, cid); break;
        case 2: topk_rounds<2>(lt, E, k, j, val, cid); break;
        case 1: topk_rounds<1>(lt, E, k, j, val, cid); break;
        default: topk_rounds<0>(lt, E, k, j, val, cid); break;
      }
      if (j == 0) {
        // (the hardware exp2 of an fp32 argument <= 0 and one reciprocal:
        // errors near 1e-7, far inside what fp32 weights carry anyway)
        float ex[8], den = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          ex[r] = r < k ? __expf((float)(val[r] - val[0])) : 0.0f;
          den += ex[r];
        }
        const float inv = 1.0f / den;
        const int kt = k + ns;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r < kt) {
            const bool routed = r < k;
            const int e2 = routed ? cid[r] : E + r - k;  // then the shared experts
            a.topk_idx[(size_t)t * kt + r] = e2;
            a.topk_w[(size_t)t * kt + r] = routed ? ex[r] * inv : 1.0f;
            sid[t * kt + r] = e2;
          }
        }
      }
    }
    // few rows: the one-pass regroup, whose per-wave counts start at zero
    const bool onepass = ra.R <= 256;
    if (onepass)
      for (int x = threadIdx.x; x < 4 * 256; x += 256) regroup_wave_counts<256>(rg_lds)[x] = 0;
    __syncthreads();
    if (a.tmask && T <= 31) {
      for (int x = threadIdx.x; x < ra.E; x += 256) {
        uint32_t m = 0;
        for (int tt = 0, i = 0; tt < T; ++tt)
          for (int r = 0; r < k + ns; ++r, ++i) m |= (sid[i] == x ? 1u : 0u) << tt;
        __hip_atomic_store(&a.tmask[x], m | kMaskKnown, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    RegroupArgs la = ra;
    la.topk_idx = sid;
    la.slot_table = sslot;
    if (onepass)
      regroup_block_onepass<256>(la, rg_lds);
    else
      regroup_block<256>(la, rg_lds);
    if (threadIdx.x == 0) reset_ticket(a.ticket);
    return;
  }
  if constexpr (kWaveFinish) {
    for (int t = wave; t < T; t += 4)
      topk_token<true>(a.logits, nsplit, a.bias, T, E, k, ns, t, lane, a.topk_idx, a.topk_w);
    __syncthreads();
    regroup_block<256>(ra, rg_lds);
  }
  if (threadIdx.x == 0) reset_ticket(a.ticket);
}

}  // namespace moe
