// Measurement helper: a read-only HBM stream, the yardstick a benchmark puts
// next to the layer's weight-streaming rate.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_measure.h"

namespace moe {
moe_status api_fail(moe_status st, const char* fmt, ...);
}

namespace {

// Each wave reads whole 4 KB runs (four 1 KB loads in flight, one per 64
// lanes of 16 bytes), the runs handed out to the waves round-robin; the last
// partial run is read vector by vector by the grid's threads.
__global__ __launch_bounds__(256) void hbm_read_kernel(const moe::u32x4* __restrict__ p, size_t n, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const size_t wave = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6), waves = (size_t)gridDim.x * 4;
  const size_t runs = n / 256;  // 256 vectors of 16 bytes per run
  moe::u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t r = wave; r < runs; r += waves) {
    const moe::u32x4* q = p + r * 256 + lane;
    const moe::u32x4 a = __builtin_nontemporal_load(q);
    const moe::u32x4 b = __builtin_nontemporal_load(q + 64);
    const moe::u32x4 c = __builtin_nontemporal_load(q + 128);
    const moe::u32x4 d = __builtin_nontemporal_load(q + 192);
    acc ^= a ^ b ^ c ^ d;
  }
  for (size_t i = runs * 256 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    acc ^= __builtin_nontemporal_load(p + i);
  uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v ^= __shfl_xor(v, off, 64);
  if (lane == 0) atomicXor(sink, v);
}

}  // namespace

extern "C" __attribute__((visibility("default"))) moe_status moe_hbm_read_probe(const void* src, size_t bytes,
                                                                                 uint32_t* sink, int32_t blocks,
                                                                                 moe_stream stream) {
  if (!src || !sink) return moe::api_fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(src) % 16 || bytes % 16)
    return moe::api_fail(MOE_ERR_INVALID_ARG, "src must be 16-byte aligned and bytes a multiple of 16");
  if (reinterpret_cast<uintptr_t>(sink) % 4) return moe::api_fail(MOE_ERR_INVALID_ARG, "sink must be 4-byte aligned");
  if (blocks < 1 || blocks > 65536) return moe::api_fail(MOE_ERR_INVALID_ARG, "blocks=%d outside [1, 65536]", blocks);
  if (bytes == 0) return MOE_OK;
  hbm_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const moe::u32x4*>(src),
                                                                         bytes / 16, sink);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return moe::api_fail(MOE_ERR_HIP, "launch: %s", hipGetErrorString(err));
  return MOE_OK;
}
