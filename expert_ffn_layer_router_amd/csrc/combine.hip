// Weighted scatter-back of the expert outputs: combine_kernel for the
// many-token path (bf16 rows), combine_partials_kernel for the few-token path
// above 8 tokens (the down GEMM's fp32 split partials); up to 8 tokens the
// down GEMM's last blocks run the same sums themselves.
//
// Strata page, section 4.2: the regrouped rows go back to their tokens after
// the group GEMM.  Written as a gather: out[t] = sum_j w[t,j] * y[inv[t*k+j]]
// in fp32, in a fixed order (j = 0..k-1), so the result is deterministic and
// needs no atomics.  y rows are bf16 (the down GEMM rounds them once: half the
// bytes to write and to gather); bf16 output, round to nearest even.
#include "device_common.h"
#include "plan.h"

namespace moe {

// one thread: 8 columns of one token
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y, int d,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ topk_w, int T, int k,
                                                      uint16_t* __restrict__ out) {
  const int per_row = d / 8;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)T * per_row) return;
  const int t = (int)(idx / per_row);
  const int c = (int)(idx % per_row) * 8;
  // all k row indices and weights first, then all k row loads in flight at
  // once, then the sums in order j = 0..k-1 (k <= 8 is uniform: no divergence)
  int pos[8];
  float wt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      pos[j] = inv[(size_t)t * k + j];
      wt[j] = topk_w[(size_t)t * k + j];
    }
  }
  u32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k) v[j] = *reinterpret_cast<const u32x4*>(y + (size_t)pos[j] * d + c);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      const uint32_t vw[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wt[j], __uint_as_float(vw[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wt[j], __uint_as_float(vw[i] & 0xFFFF0000u), acc[2 * i + 1]);
      }
    }
  }
  u32x4 o;
  o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
  *reinterpret_cast<u32x4*>(out + (size_t)t * d + c) = o;
}

// Few tokens, the down kernel's fp32 partials ypart[split][p][d]: per output
// the rows j = 0..k-1 in order, each the sum of its splits in split order,
// weighted -- the same operations, in the same order, as the combine the down
// kernel runs in its last blocks.  One thread: 4 columns of one token.  All k
// row indices and weights are loaded first, then each split's k loads are
// issued together (k <= 8 is uniform: no divergence), so the dependent round
// trips are 1 + nsplit instead of k (1 + nsplit).
__global__ __launch_bounds__(256) void combine_partials_kernel(const float* __restrict__ ypart, int R, int d,
                                                               int nsplit, const int32_t* __restrict__ inv,
                                                               const float* __restrict__ topk_w, int T, int k,
                                                               uint16_t* __restrict__ out) {
  const int per_row = d / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * per_row) return;
  const int t = idx / per_row, c = (idx % per_row) * 4;
  int pos[8];
  float wt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      pos[j] = inv[t * k + j];
      wt[j] = topk_w[t * k + j];
    }
  }
  float4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k) v[j] = *reinterpret_cast<const float4*>(ypart + (size_t)pos[j] * d + c);
  for (int sp = 1; sp < nsplit; ++sp) {
    float4 u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) u[j] = *reinterpret_cast<const float4*>(ypart + ((size_t)sp * R + pos[j]) * d + c);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        v[j].x += u[j].x;
        v[j].y += u[j].y;
        v[j].z += u[j].z;
        v[j].w += u[j].w;
      }
    }
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      acc.x = fmaf(wt[j], v[j].x, acc.x);
      acc.y = fmaf(wt[j], v[j].y, acc.y);
      acc.z = fmaf(wt[j], v[j].z, acc.z);
      acc.w = fmaf(wt[j], v[j].w, acc.w);
    }
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
  o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
  *reinterpret_cast<uint2*>(out + (size_t)t * d + c) = o;
}

void launch_combine_partials(const moe_config& c, const Plan& p, uint16_t* out, char* ws, hipStream_t s) {
  const int n = p.T * (c.d_model / 4);
  combine_partials_kernel<<<(n + 255) / 256, 256, 0, s>>>(
      reinterpret_cast<const float*>(ws + p.y), p.R, c.d_model, p.down_split,
      reinterpret_cast<const int32_t*>(ws + p.inv), reinterpret_cast<const float*>(ws + p.topk_w), p.T, c.top_k,
      out);
}

void launch_combine(const moe_config& c, const Plan& p, uint16_t* out, char* ws, hipStream_t s) {
  const size_t n = (size_t)p.T * (c.d_model / 8);
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<const uint16_t*>(ws + p.y), c.d_model, reinterpret_cast<const int32_t*>(ws + p.inv),
      reinterpret_cast<const float*>(ws + p.topk_w), p.T, c.top_k, out);
}

}  // namespace moe
