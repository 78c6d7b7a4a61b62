// Router: logits = x W_r^T + b, top-k selection, renormalised gate weights.
//
// Strata page, section 1.1: each token picks its top-2 (or top-1) experts.
// Co-inference page, section 5.1: the router stays at full precision.  The
// products bf16 x fp32 are exact in fp64 and are summed in fp64, so the
// selection matches an fp64 evaluation of the logits; exact ties (equal
// logits) go to the lower expert id, because every expert's logit runs
// through the same sequence of operations.
#include "device_common.h"
#include "plan.h"
#include "regroup.h"

namespace moe {

constexpr int kFusedLogitsLds = 4096;  // logits (T x E) the fused router's last block stages in LDS

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
      if (kCoherent) {
        v = load_coherent(&logits[(size_t)t * E + e]);
        for (int s = 1; s < nsplit; ++s) v += load_coherent(&logits[((size_t)s * T + t) * E + e]);
      } else {
        v = logits[(size_t)t * E + e];
        for (int s = 1; s < nsplit; ++s) v += logits[((size_t)s * T + t) * E + e];
      }
      if (bias) v += (double)bias[e];
    }
    l[j] = v;
  }
  double best[8];
  int bid[8];
  for (int r = 0; r < k; ++r) {
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
  if (lane == 0) {
    double ex[8], den = 0.0;
    for (int j = 0; j < k; ++j) {
      ex[j] = exp(best[j] - best[0]);
      den += ex[j];
    }
    for (int j = 0; j < k; ++j) {
      topk_idx[(size_t)t * kt + j] = bid[j];
      topk_w[(size_t)t * kt + j] = (float)(ex[j] / den);
    }
    for (int j = 0; j < ns; ++j) {
      topk_idx[(size_t)t * kt + k + j] = E + j;
      topk_w[(size_t)t * kt + k + j] = 1.0f;
    }
  }
}

// Few tokens (T <= kStreamMaxTokens): one block per (expert, group of
// kRouterTokTile tokens); its 4 waves take a quarter of d each, lane l
// accumulating k = 8l .. 8l+7 of every 512 for all tokens of the group; a
// butterfly over the lanes and a fixed-order sum over the 4 waves (through
// LDS) finish each logit.  The last block to finish (an atomic ticket in the
// workspace's control words) then runs the top-k of every token and the
// regroup, and clears the ticket for the next call.  E and k count the routed
// experts; the ns shared experts (groups E .. E+ns-1 of the regroup, ra.E =
// E + ns) take the last ns columns of every token.
__global__ __launch_bounds__(256) void router_small_kernel(const uint16_t* __restrict__ hidden,
                                                           const float* __restrict__ wr,
                                                           const float* __restrict__ bias,
                                                           double* __restrict__ logits, int T, int d, int E,
                                                           int k, int ns, int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w,
                                                           uint32_t* __restrict__ flags,
                                                           uint32_t* __restrict__ ticket, RegroupArgs ra) {
  __shared__ double part[4][kRouterTokTile];
  __shared__ int is_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kRouterTokTile;
  const int nt = min(kRouterTokTile, T - t0);
  double acc[kRouterTokTile];
#pragma unroll
  for (int t = 0; t < kRouterTokTile; ++t) acc[t] = 0.0;
  const int nsplit = gridDim.z;          // k-splits: block z covers k in [z d / nsplit, (z + 1) d / nsplit)
  const int kq = d / (4 * nsplit);       // per wave, a multiple of 32
  const int kbeg = blockIdx.z * (d / nsplit) + wave * kq, kend = kbeg + kq;
  const float* wrow = wr + (size_t)e * d;
  for (int kk = kbeg + lane * 8; kk < kend; kk += 512) {
    const float4 w0 = *reinterpret_cast<const float4*>(wrow + kk);
    const float4 w1 = *reinterpret_cast<const float4*>(wrow + kk + 4);
    const double wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    u32x4 xv[kRouterTokTile];
#pragma unroll
    for (int t = 0; t < kRouterTokTile; ++t)  // rows past T re-read the group's first row
      xv[t] = *reinterpret_cast<const u32x4*>(hidden + (size_t)(t0 + (t < nt ? t : 0)) * d + kk);
#pragma unroll
    for (int t = 0; t < kRouterTokTile; ++t) {
      const uint32_t xs[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[t] = fma((double)__uint_as_float(xs[i] << 16), wv[2 * i], acc[t]);
        acc[t] = fma((double)__uint_as_float(xs[i] & 0xFFFF0000u), wv[2 * i + 1], acc[t]);
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
    store_coherent(&logits[((size_t)blockIdx.z * T + t0 + lane) * E + e], v);
  }
  // the last block to finish does the top-k of every token and the regroup
  if (!last_block_ticket(ticket, gridDim.x * gridDim.y * gridDim.z, &is_last)) return;
  if (threadIdx.x == 0) *flags = 0u;
  if (T * E <= kFusedLogitsLds && T <= 256) {
    // slot table and the biased fp64 logits into LDS (lg[t * E + e]).  The
    // coherent loads see the latency of the memory side of the L2, so they
    // are issued without conditions, four per thread in flight at a time
    // (indices past the end re-read the last logit and land in a spare LDS
    // slot), together with the bias and slot loads.
    __shared__ double lg[kFusedLogitsLds + 1];
    __shared__ double sbias[256];
    __shared__ int32_t sslot[256];
    __shared__ int32_t sid[256 * 8];
    const int TE = T * E;
    for (int i0 = 0; i0 < TE; i0 += 4 * 256) {
      float bv = 0.0f;
      int sl = 0;
      if (i0 == 0 && threadIdx.x < ra.E) {  // slots of routed and shared experts, bias of routed ones
        bv = (bias && threadIdx.x < E) ? bias[threadIdx.x] : 0.0f;
        sl = ra.slot_table[threadIdx.x];
      }
      // logit = split 0 + split 1 + ... in order; up to kRouterSmallMaxSplit
      // splits are loaded (missing ones re-read split 0 and add zero)
      double v[4], w[4][kRouterSmallMaxSplit - 1];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = min(i0 + (int)threadIdx.x + 256 * u, TE - 1);
        v[u] = load_coherent(&logits[i]);
#pragma unroll
        for (int sp = 1; sp < kRouterSmallMaxSplit; ++sp)
          w[u][sp - 1] = load_coherent(&logits[(size_t)(sp < nsplit ? sp : 0) * TE + i]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int sp = 1; sp < kRouterSmallMaxSplit; ++sp) v[u] += sp < nsplit ? w[u][sp - 1] : 0.0;
      if (i0 == 0 && threadIdx.x < ra.E) {
        sbias[threadIdx.x] = bv;
        sslot[threadIdx.x] = sl;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + (int)threadIdx.x + 256 * u;
        lg[i < TE ? i : kFusedLogitsLds] = v[u] + sbias[i < TE ? i % E : 0];
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
          for (int e = j, m = 0; e < E; e += S, ++m) {
            const double v = lt[e];
            if (!((dead >> m) & 1) && (bid == 0x7fffffff || v > best)) {
              best = v;
              bid = e;
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
            topk_idx[(size_t)t * kt + r] = cid[r];
            topk_w[(size_t)t * kt + r] = ex[r] / den;
            sid[t * kt + r] = cid[r];
          } else if (r < kt) {  // shared experts
            topk_idx[(size_t)t * kt + r] = E + r - k;
            topk_w[(size_t)t * kt + r] = 1.0f;
            sid[t * kt + r] = E + r - k;
          }
        }
      }
    }
    __syncthreads();
    RegroupArgs la = ra;
    la.topk_idx = sid;
    la.slot_table = sslot;
    regroup_block<256>(la);
    if (threadIdx.x == 0) reset_ticket(ticket);
    return;
  }
  for (int t = wave; t < T; t += 4) topk_token<true>(logits, nsplit, bias, T, E, k, ns, t, lane, topk_idx, topk_w);
  __syncthreads();
  regroup_block<256>(ra);
  if (threadIdx.x == 0) reset_ticket(ticket);
}

// Many tokens: the logits as an fp64 GEMM on the matrix cores
// (v_mfma_f64_16x16x4_f64).  The products bf16 x fp32 are exact in fp64 and
// every logit is summed by the same sequence of fp64 operations (k in steps
// of 4 inside the matrix core, then the k-splits in order), so exact ties
// still go to the lower expert id.  A block computes 64 tokens x TN experts
// over one k-split; each wave 16 tokens x TN experts.  Chunks of 32 k are
// loaded into registers one chunk ahead, widened to fp64 and stored k-major
// in LDS, where each MFMA operand is one conflict-free ds_read_b64 (lane l:
// A = x[t0 + l % 16][k + l / 16], B = W[e0 + l % 16][k + l / 16]; D element
// r of lane l is (token l / 16 + 4 r, expert l % 16)).  Output:
// logits[split][t][e], summed in split order by router_topk_kernel.
template <int TN>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const uint16_t* __restrict__ hidden,
                                                                 const float* __restrict__ wr,
                                                                 double* __restrict__ logits, int T, int d, int E,
                                                                 int kchunk) {
  constexpr int TM = kRouterMfmaTokens, KC = kRouterMfmaK, NB = TN / 16;
  __shared__ double xs[KC][TM];
  __shared__ double wsh[KC][TN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TN, split = blockIdx.z;
  const int kbeg = split * kchunk, kend = kbeg + kchunk;
  // staging: thread -> x row t0 + tid % 64, k 8 (tid / 64) .. +8 of the chunk;
  // W row e0 + tid % TN (the first 4 TN threads: 8 k each)
  const int xr = tid % TM, xk = 8 * (tid / TM);
  const bool xok = t0 + xr < T;
  const uint16_t* xsrc = hidden + (size_t)(xok ? t0 + xr : 0) * d + xk;
  const int wrow = tid % TN, wk = 8 * (tid / TN);
  const bool wact = tid < 4 * TN, wok = wact && e0 + wrow < E;
  const float* wsrc = wr + (size_t)(wok ? e0 + wrow : 0) * d + (wact ? wk : 0);
  u32x4 xv;
  float4 w0, w1;
  auto fetch = [&](int kc) {
    xv = *reinterpret_cast<const u32x4*>(xsrc + kc);
    if (wact) {
      w0 = *reinterpret_cast<const float4*>(wsrc + kc);
      w1 = *reinterpret_cast<const float4*>(wsrc + kc + 4);
    }
  };
  auto stage = [&]() {
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[xk + 2 * i][xr] = xok ? (double)__uint_as_float(xw[i] << 16) : 0.0;
      xs[xk + 2 * i + 1][xr] = xok ? (double)__uint_as_float(xw[i] & 0xFFFF0000u) : 0.0;
    }
    if (wact) {
      const float wf[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) wsh[wk + i][wrow] = wok ? (double)wf[i] : 0.0;
    }
  };
  f64x4 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f64x4{0.0, 0.0, 0.0, 0.0};
  fetch(kbeg);
  for (int kc = kbeg; kc < kend; kc += KC) {
    __syncthreads();  // the previous chunk's operands are read
    stage();
    __syncthreads();
    if (kc + KC < kend) fetch(kc + KC);  // next chunk's loads in flight during the products
#pragma unroll
    for (int k4 = 0; k4 < KC; k4 += 4) {
      const double av = xs[k4 + lane / 16][16 * wave + lane % 16];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const double bv = wsh[k4 + lane / 16][16 * n + lane % 16];
        acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[n], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * wave + lane / 16 + 4 * r, e = e0 + 16 * n + lane % 16;
      if (t < T && e < E) logits[((size_t)split * T + t) * E + e] = acc[n][r];
    }
}

__global__ __launch_bounds__(256) void router_topk_kernel(const double* __restrict__ logits, int nsplit,
                                                          const float* __restrict__ bias,
                                                          const uint16_t* __restrict__ hidden, int d, int T,
                                                          int E, int k, int ns, int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w, float* __restrict__ xsum,
                                                          uint16_t* __restrict__ xperm, uint32_t* __restrict__ flags) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *flags = 0u;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  topk_token<false>(logits, nsplit, bias, T, E, k, ns, t, lane, topk_idx, topk_w);
  // row sum of x (for the gate/up GEMM's zero-point term) and x in fragment
  // k-order (the gate/up GEMM's A operand then needs no permutes)
  double sx = 0.0;
  for (int kk = lane * 8; kk < d; kk += 512) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(hidden + (size_t)t * d + kk);
    *reinterpret_cast<u32x4*>(xperm + (size_t)t * d + kk) = permute_a(xv);
    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sx += (double)__uint_as_float(xs[i] << 16) + (double)__uint_as_float(xs[i] & 0xFFFF0000u);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sx += __shfl_xor(sx, off, 64);
  if (lane == 0) xsum[t] = (float)sx;
}

void launch_router(const moe_config& c, const Plan& p, const uint16_t* hidden, const float* router_w,
                   const float* router_bias, const int32_t* slot_table, char* ws, hipStream_t s) {
  // c counts shared experts among the experts and the columns of each token;
  // the router itself sees the routed ones only
  const int ns = c.num_shared, E = c.num_experts - ns, k = c.top_k - ns;
  double* logits = reinterpret_cast<double*>(ws + p.logits);
  int32_t* topk_idx = reinterpret_cast<int32_t*>(ws + p.topk_idx);
  float* topk_w = reinterpret_cast<float*>(ws + p.topk_w);
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws + p.flags);
  if (p.fused_small) {
    dim3 grid(E, (p.T + kRouterTokTile - 1) / kRouterTokTile, p.small_split);
    router_small_kernel<<<grid, 256, 0, s>>>(hidden, router_w, router_bias, logits, p.T, c.d_model, E, k, ns,
                                             topk_idx, topk_w, flags, reinterpret_cast<uint32_t*>(ws + p.ctrl),
                                             regroup_args(c, p, slot_table, ws));
    return;
  }
  const int tn = router_tile_experts(E);
  dim3 grid((p.T + kRouterMfmaTokens - 1) / kRouterMfmaTokens, (E + tn - 1) / tn, p.router_split);
  const int kchunk = c.d_model / p.router_split;
  if (tn == 64)
    router_logits_mfma_kernel<64><<<grid, 256, 0, s>>>(hidden, router_w, logits, p.T, c.d_model, E, kchunk);
  else if (tn == 32)
    router_logits_mfma_kernel<32><<<grid, 256, 0, s>>>(hidden, router_w, logits, p.T, c.d_model, E, kchunk);
  else
    router_logits_mfma_kernel<16><<<grid, 256, 0, s>>>(hidden, router_w, logits, p.T, c.d_model, E, kchunk);
  router_topk_kernel<<<(p.T + 3) / 4, 256, 0, s>>>(logits, p.router_split, router_bias, hidden, c.d_model, p.T,
                                                   E, k, ns, topk_idx, topk_w,
                                                   reinterpret_cast<float*>(ws + p.xsum),
                                                   reinterpret_cast<uint16_t*>(ws + p.xperm), flags);
}

}  // namespace moe
