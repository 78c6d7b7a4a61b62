// Weighted scatter-back of the expert outputs.
//
// Strata page, section 4.2: the regrouped rows go back to their tokens after
// the group GEMM.  Written as a gather: out[t] = sum_j w[t,j] * y[inv[t*k+j]],
// with y summed over the down projection's k-splits first, all in fp32 and
// in a fixed order (splits, then j = 0..k-1), so the result is deterministic
// and needs no atomics.  bf16 output, round to nearest even.
#include "device_common.h"
#include "plan.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ypart, int nsplit, int R,
                                                      int d, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ topk_w, int T, int k,
                                                      uint16_t* __restrict__ out) {
  const int per_row = d / 4;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)T * per_row) return;
  const int t = (int)(idx / per_row);
  const int c = (int)(idx % per_row) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int p = inv[(size_t)t * k + j];
    const float w = topk_w[(size_t)t * k + j];
    float4 v = *reinterpret_cast<const float4*>(ypart + (size_t)p * d + c);
    for (int s = 1; s < nsplit; ++s) {
      const float4 u = *reinterpret_cast<const float4*>(ypart + ((size_t)s * R + p) * d + c);
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
  o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
  *reinterpret_cast<uint2*>(out + (size_t)t * d + c) = o;
}

void launch_combine(const moe_config& c, const Plan& p, uint16_t* out, char* ws, hipStream_t s) {
  const size_t n = (size_t)p.T * (c.d_model / 4);
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<const float*>(ws + p.y), p.down_split, p.R, c.d_model,
      reinterpret_cast<const int32_t*>(ws + p.inv), reinterpret_cast<const float*>(ws + p.topk_w), p.T,
      c.top_k, out);
}

}  // namespace moe
