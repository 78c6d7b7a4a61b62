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
#include "router_small.h"

namespace moe {

// Few tokens (T <= kStreamMaxTokens): one block per (expert, group of
// kRouterTokTile tokens, k-split); the last block to finish runs the top-k of
// every token and the regroup (router_small_body).  Logits of up to
// kSmallLogitsLds (T x E) are staged in LDS for the finish.
constexpr int kSmallLogitsLds = 4096;
__global__ __launch_bounds__(256) void router_small_kernel(RouterSmallArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[router_small_lds_bytes<kSmallLogitsLds, 256>()];
  router_small_body<kSmallLogitsLds, 256, kRouterTokTile>(a, blockIdx.x, blockIdx.y * kRouterTokTile, blockIdx.z,
                                                          gridDim.x * gridDim.y * gridDim.z, smem);
}

// Many tokens: the logits as an fp64 GEMM on the matrix cores
// (v_mfma_f64_16x16x4_f64).  The products bf16 x fp32 are exact in fp64 and
// every logit is summed by the same sequence of fp64 operations (k in steps
// of 4 inside the matrix core, then the k-splits in order), so exact ties
// still go to the lower expert id.  A block computes 64 tokens x TN experts
// over one k-split; each wave 16 tokens x TN experts.  Chunks of 32 k are
// loaded into registers one chunk ahead, widened to fp64 and stored k-major
// in one of two LDS buffers (the products of one chunk run while the next is
// stored into the other, one barrier per chunk), where each MFMA operand is
// one conflict-free ds_read_b64 (lane l: A = x[t0 + l % 16][k + l / 16],
// B = W[e0 + l % 16][k + l / 16]; D element r of lane l is (token l / 16 +
// 4 r, expert l % 16)).  Output: logits[split][t][e], summed in split order
// by router_topk_kernel.  The blocks of the first expert tile also write
// their part of x in fragment k-order (xperm, the prefill gate/up GEMM's A
// operand) and per token the fp64 sum of their k range (xsum_part[split][t],
// for the GEMM's zero-point term), so x is read from HBM once.
template <int TN>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const uint16_t* __restrict__ hidden,
                                                                 const float* __restrict__ wr,
                                                                 double* __restrict__ logits, int T, int d, int E,
                                                                 int kchunk, uint16_t* __restrict__ xperm,
                                                                 double* __restrict__ xsum_part) {
  constexpr int TM = kRouterMfmaTokens, KC = kRouterMfmaK, NB = TN / 16;
  __shared__ double xs[2][KC][TM];
  __shared__ double wsh[2][KC][TN];
  __shared__ double srow[4][TM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TN, split = blockIdx.z;
  const int kbeg = split * kchunk, kend = kbeg + kchunk;
  const bool xcopy = blockIdx.y == 0;  // this block writes its part of xperm and xsum_part
  // staging: thread -> x row t0 + tid % 64, k 8 (tid / 64) .. +8 of the chunk;
  // W row e0 + tid % TN (the first 4 TN threads: 8 k each)
  const int xr = tid % TM, xk = 8 * (tid / TM);
  const bool xok = t0 + xr < T;
  const uint16_t* xsrc = hidden + (size_t)(xok ? t0 + xr : 0) * d + xk;
  uint16_t* xdst = xperm + (size_t)(xok ? t0 + xr : 0) * d + xk;
  const int wrow = tid % TN, wk = 8 * (tid / TN);
  const bool wact = tid < 4 * TN, wok = wact && e0 + wrow < E;
  const float* wsrc = wr + (size_t)(wok ? e0 + wrow : 0) * d + (wact ? wk : 0);
  u32x4 xv;
  float4 w0, w1;
  double sx = 0.0;  // this thread's x values, summed
  auto fetch = [&](int kc) {
    xv = *reinterpret_cast<const u32x4*>(xsrc + kc);
    if (wact) {
      w0 = *reinterpret_cast<const float4*>(wsrc + kc);
      w1 = *reinterpret_cast<const float4*>(wsrc + kc + 4);
    }
  };
  auto stage = [&](int buf, int kc) {
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double lo = (double)__uint_as_float(xw[i] << 16), hi = (double)__uint_as_float(xw[i] & 0xFFFF0000u);
      xs[buf][xk + 2 * i][xr] = xok ? lo : 0.0;
      xs[buf][xk + 2 * i + 1][xr] = xok ? hi : 0.0;
      sx += lo + hi;
    }
    if (xcopy && xok) *reinterpret_cast<u32x4*>(xdst + kc) = permute_a(xv);
    if (wact) {
      const float wf[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) wsh[buf][wk + i][wrow] = wok ? (double)wf[i] : 0.0;
    }
  };
  f64x4 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f64x4{0.0, 0.0, 0.0, 0.0};
  fetch(kbeg);
  stage(0, kbeg);
  __syncthreads();
  for (int kc = kbeg, buf = 0; kc < kend; kc += KC, buf ^= 1) {
    const bool more = kc + KC < kend;
    if (more) fetch(kc + KC);  // next chunk's loads in flight during the products
#pragma unroll
    for (int k4 = 0; k4 < KC; k4 += 4) {
      const double av = xs[buf][k4 + lane / 16][16 * wave + lane % 16];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const double bv = wsh[buf][k4 + lane / 16][16 * n + lane % 16];
        acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[n], 0, 0, 0);
      }
    }
    // the other buffer was last read before the previous barrier
    if (more) stage(buf ^ 1, kc + KC);
    __syncthreads();
  }
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * wave + lane / 16 + 4 * r, e = e0 + 16 * n + lane % 16;
      if (t < T && e < E) logits[((size_t)split * T + t) * E + e] = acc[n][r];
    }
  if (xcopy) {  // the four threads of each row, in a fixed order
    srow[tid / TM][xr] = sx;
    __syncthreads();
    if (tid < TM && t0 + tid < T)
      xsum_part[(size_t)split * T + t0 + tid] = ((srow[0][tid] + srow[1][tid]) + srow[2][tid]) + srow[3][tid];
  }
}

// One wave per token: the top-k (topk_token) and the row sum of x for the
// gate/up GEMM's zero-point term (the logits kernel's per-split sums, added
// in split order).  Grouped int4 weights (xgsum not null): also the sums of
// x over each group of 128 k, [T][d / 128].
__global__ __launch_bounds__(256) void router_topk_kernel(const double* __restrict__ logits, int nsplit,
                                                          const float* __restrict__ bias, int T, int E, int k,
                                                          int ns, int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          const double* __restrict__ xsum_part,
                                                          float* __restrict__ xsum, uint32_t* __restrict__ flags,
                                                          const uint16_t* __restrict__ hidden, int d,
                                                          float* __restrict__ xgsum) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *flags = 0u;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  // the row sum's parts, loaded first (lane l: splits l, l + 64, ...) so that
  // their latency overlaps the top-k; summed lane by lane, then across the
  // lanes by a butterfly (a fixed order: the sum is rounded to fp32 anyway)
  double sx = 0.0;
  for (int s = lane; s < nsplit; s += 64) sx += xsum_part[(size_t)s * T + t];
  topk_token<false>(logits, nsplit, bias, T, E, k, ns, t, lane, topk_idx, topk_w);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sx += __shfl_xor(sx, off, 64);
  if (lane == 0) xsum[t] = (float)sx;
  if (xgsum) {
    // lane l: k = 8 l .. 8 l + 7 of every 512, so 16 lanes cover a group
    for (int kk = 0; kk < d; kk += 512) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(hidden + (size_t)t * d + kk + 8 * lane);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      float g = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) g += __uint_as_float(xw[i] << 16) + __uint_as_float(xw[i] & 0xFFFF0000u);
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) g += __shfl_xor(g, off, 64);
      if ((lane & 15) == 0) xgsum[(size_t)t * (d / 128) + (kk + 8 * lane) / 128] = g;
    }
  }
}

// The same for at most 64 routed experts with 16 lanes per token (four
// tokens per wave): lane j holds experts j, j + 16, j + 32, j + 48, each
// logit the same sum (splits in order, then the bias), chosen by the rounds
// of topk_rounds_heads (one max and one min reduction per round, DPP
// exchanges inside the segment) instead of k rounds of a 64-lane butterfly.
// The weights, the row sum and the group sums take the same operations as in
// router_topk_kernel (the row sum's parts in another fixed order).
__global__ __launch_bounds__(256) void router_topk_seg_kernel(const double* __restrict__ logits, int nsplit,
                                                              const float* __restrict__ bias, int T, int E, int k,
                                                              int ns, int32_t* __restrict__ topk_idx,
                                                              float* __restrict__ topk_w,
                                                              const double* __restrict__ xsum_part,
                                                              float* __restrict__ xsum, uint32_t* __restrict__ flags,
                                                              const uint16_t* __restrict__ hidden, int d,
                                                              float* __restrict__ xgsum) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *flags = 0u;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (t >= T) return;  // whole segments: the exchanges below stay inside one
  const int j = threadIdx.x & 15;
  // the row sum's parts first (lane j: splits j, j + 16, ...)
  double sx = 0.0;
  for (int s = j; s < nsplit; s += 16) sx += xsum_part[(size_t)s * T + t];
  double h[4];
  int hid[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = j + 16 * m;
    const bool ok = e < E;
    const int ee = ok ? e : 0;
    double v = 0.0;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {  // eight loads in flight (a missing split adds +0.0)
      double q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) q[u] = s0 + u < nsplit ? logits[((size_t)(s0 + u) * T + t) * E + ee] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) v += q[u];
    }
    if (bias) v += (double)bias[ee];
    h[m] = ok ? v : __builtin_nan("");
    hid[m] = ok ? e : kNoExpert;
  }
  double val[8];
  int cid[8];
  topk_rounds_heads<4>(h, hid, k, val, cid);
  // lane j < k takes choice j: exp(l_j - l_0), then the sum in order j = 0 .. k-1
  double bj = val[0];
  int ij = cid[0];
#pragma unroll
  for (int r = 1; r < 8; ++r)
    if (j == r) {
      bj = val[r];
      ij = cid[r];
    }
  const double ex = j < k ? exp(bj - val[0]) : 0.0;
  double den = 0.0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const double er = __shfl(ex, r, 16);
    if (r < k) den += er;
  }
  const int kt = k + ns;
  if (j < k) {
    topk_idx[(size_t)t * kt + j] = ij;
    topk_w[(size_t)t * kt + j] = (float)(ex / den);
  }
  if (j == 0) {
    for (int q = 0; q < ns; ++q) {
      topk_idx[(size_t)t * kt + k + q] = E + q;
      topk_w[(size_t)t * kt + k + q] = 1.0f;
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) sx += __shfl_xor(sx, off, 16);
  if (j == 0) xsum[t] = (float)sx;
  if (xgsum) {
    // one group of 128 k at a time: lane j sums k = 8 j .. 8 j + 7 of it, then
    // a butterfly over the segment
    for (int g = 0; g < d / 128; ++g) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(hidden + (size_t)t * d + 128 * g + 8 * j);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      float gs = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) gs += __uint_as_float(xw[i] << 16) + __uint_as_float(xw[i] & 0xFFFF0000u);
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) gs += __shfl_xor(gs, off, 16);
      if (j == 0) xgsum[(size_t)t * (d / 128) + g] = gs;
    }
  }
}

RouterSmallArgs router_small_args(const moe_config& c, const Plan& p, const uint16_t* hidden,
                                  const float* router_w, const float* router_bias, const int32_t* slot_table,
                                  char* ws) {
  // c counts shared experts among the experts and the columns of each token;
  // the router itself sees the routed ones only
  RouterSmallArgs a{};
  a.ns = c.num_shared;
  a.E = c.num_experts - a.ns;
  a.k = c.top_k - a.ns;
  a.hidden = hidden;
  a.wr = router_w;
  a.bias = router_bias;
  a.logits = reinterpret_cast<double*>(ws + p.logits);
  a.T = p.T;
  a.d = c.d_model;
  a.nsplit = p.small_split;
  a.topk_idx = reinterpret_cast<int32_t*>(ws + p.topk_idx);
  a.topk_w = reinterpret_cast<float*>(ws + p.topk_w);
  a.flags = reinterpret_cast<uint32_t*>(ws + p.flags);
  a.ticket = reinterpret_cast<uint32_t*>(ws + p.ctrl);
  a.tmask = p.dense ? reinterpret_cast<uint32_t*>(ws + p.ctrl + p.tmask) : nullptr;
  a.ra = regroup_args(c, p, slot_table, ws);
  return a;
}

void launch_router(const moe_config& c, const Plan& p, const uint16_t* hidden, const float* router_w,
                   const float* router_bias, const int32_t* slot_table, char* ws, hipStream_t s) {
  const int ns = c.num_shared, E = c.num_experts - ns, k = c.top_k - ns;
  double* logits = reinterpret_cast<double*>(ws + p.logits);
  int32_t* topk_idx = reinterpret_cast<int32_t*>(ws + p.topk_idx);
  float* topk_w = reinterpret_cast<float*>(ws + p.topk_w);
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws + p.flags);
  if (p.fused_small) {
    dim3 grid(E, (p.T + kRouterTokTile - 1) / kRouterTokTile, p.small_split);
    router_small_kernel<<<grid, 256, 0, s>>>(router_small_args(c, p, hidden, router_w, router_bias, slot_table, ws));
    return;
  }
  const int tn = router_tile_experts(E);
  dim3 grid((p.T + kRouterMfmaTokens - 1) / kRouterMfmaTokens, (E + tn - 1) / tn, p.router_split);
  const int kchunk = c.d_model / p.router_split;
  uint16_t* xperm = reinterpret_cast<uint16_t*>(ws + p.xperm);
  double* xsum_part = reinterpret_cast<double*>(ws + p.xsum_part);
  if (tn == 64)
    router_logits_mfma_kernel<64><<<grid, 256, 0, s>>>(hidden, router_w, logits, p.T, c.d_model, E, kchunk, xperm,
                                                       xsum_part);
  else if (tn == 32)
    router_logits_mfma_kernel<32><<<grid, 256, 0, s>>>(hidden, router_w, logits, p.T, c.d_model, E, kchunk, xperm,
                                                       xsum_part);
  else
    router_logits_mfma_kernel<16><<<grid, 256, 0, s>>>(hidden, router_w, logits, p.T, c.d_model, E, kchunk, xperm,
                                                       xsum_part);
  float* xgsum = c.group_size && c.weight_bits == 4 ? reinterpret_cast<float*>(ws + p.xgsum) : nullptr;
  if (E <= 64)
    router_topk_seg_kernel<<<(p.T + 15) / 16, 256, 0, s>>>(logits, p.router_split, router_bias, p.T, E, k, ns,
                                                           topk_idx, topk_w, xsum_part,
                                                           reinterpret_cast<float*>(ws + p.xsum), flags, hidden,
                                                           c.d_model, xgsum);
  else
    router_topk_kernel<<<(p.T + 3) / 4, 256, 0, s>>>(logits, p.router_split, router_bias, p.T, E, k, ns, topk_idx,
                                                     topk_w, xsum_part, reinterpret_cast<float*>(ws + p.xsum), flags,
                                                     hidden, c.d_model, xgsum);
}

}  // namespace moe
