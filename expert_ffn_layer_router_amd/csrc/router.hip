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

namespace moe {

// Partial logits over one k-range: part[split][t][e] (fp64).
// Block: 16 tokens x 64 experts; thread (ty, tx) owns token ty and experts
// tx, tx+16, tx+32, tx+48.
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ hidden,
                                                            const float* __restrict__ wr,
                                                            double* __restrict__ part, int T, int d,
                                                            int E, int kchunk) {
  __shared__ float xs[kRouterTokTile][kRouterKChunk + 1];
  __shared__ float ws[kRouterExpTile][kRouterKChunk + 1];
  const int t0 = blockIdx.x * kRouterTokTile;
  const int e0 = blockIdx.y * kRouterExpTile;
  const int split = blockIdx.z;
  const int kbeg = split * kchunk;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int kc = kbeg; kc < kbeg + kchunk; kc += kRouterKChunk) {
    for (int i = tid; i < kRouterTokTile * kRouterKChunk; i += 256) {
      const int r = i / kRouterKChunk, c = i % kRouterKChunk;
      const int t = t0 + r;
      xs[r][c] = (t < T) ? bf16_to_f32(hidden[(size_t)t * d + kc + c]) : 0.0f;
    }
    for (int i = tid; i < kRouterExpTile * kRouterKChunk; i += 256) {
      const int r = i / kRouterKChunk, c = i % kRouterKChunk;
      const int e = e0 + r;
      ws[r][c] = (e < E) ? wr[(size_t)e * d + kc + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kRouterKChunk; ++c) {
      const double xv = xs[ty][c];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fma(xv, (double)ws[tx + 16 * j][c], acc[j]);
    }
    __syncthreads();
  }
  const int t = t0 + ty;
  if (t < T) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx + 16 * j;
      if (e < E) part[((size_t)split * T + t) * E + e] = acc[j];
    }
  }
}

// One thread per token: sum the partial logits in split order, add the bias,
// keep the k largest (strictly larger replaces, so the earlier, lower id wins
// a tie), then w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
// Also clears the device error flags of this forward.
__global__ __launch_bounds__(256) void router_topk_kernel(const double* __restrict__ part, int nsplit,
                                                          const float* __restrict__ bias, int T, int E,
                                                          int k, int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          uint32_t* __restrict__ flags) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *flags = 0u;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  double best[8];
  int bid[8];
  int n = 0;
  for (int e = 0; e < E; ++e) {
    double l = part[(size_t)t * E + e];
    for (int s = 1; s < nsplit; ++s) l += part[((size_t)s * T + t) * E + e];
    if (bias) l += (double)bias[e];
    if (n < k) {
      int i = n++;
      while (i > 0 && best[i - 1] < l) {
        best[i] = best[i - 1];
        bid[i] = bid[i - 1];
        --i;
      }
      best[i] = l;
      bid[i] = e;
    } else if (l > best[k - 1]) {
      int i = k - 1;
      while (i > 0 && best[i - 1] < l) {
        best[i] = best[i - 1];
        bid[i] = bid[i - 1];
        --i;
      }
      best[i] = l;
      bid[i] = e;
    }
  }
  double den = 0.0;
  double ex[8];
  for (int j = 0; j < k; ++j) {
    ex[j] = exp(best[j] - best[0]);
    den += ex[j];
  }
  for (int j = 0; j < k; ++j) {
    topk_idx[(size_t)t * k + j] = bid[j];
    topk_w[(size_t)t * k + j] = (float)(ex[j] / den);
  }
}

void launch_router(const moe_config& c, const Plan& p, const uint16_t* hidden, const float* router_w,
                   const float* router_bias, char* ws, hipStream_t s) {
  double* part = reinterpret_cast<double*>(ws + p.logit_part);
  dim3 grid((p.T + kRouterTokTile - 1) / kRouterTokTile, (c.num_experts + kRouterExpTile - 1) / kRouterExpTile,
            p.router_split);
  router_logits_kernel<<<grid, 256, 0, s>>>(hidden, router_w, part, p.T, c.d_model, c.num_experts,
                                            c.d_model / p.router_split);
  router_topk_kernel<<<(p.T + 255) / 256, 256, 0, s>>>(
      part, p.router_split, router_bias, p.T, c.num_experts, c.top_k,
      reinterpret_cast<int32_t*>(ws + p.topk_idx), reinterpret_cast<float*>(ws + p.topk_w),
      reinterpret_cast<uint32_t*>(ws + p.flags));
}

}  // namespace moe
