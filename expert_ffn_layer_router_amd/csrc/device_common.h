// Device helpers shared by the gfx950 kernels: bf16 conversions, MFMA operand
// types and the int4 -> bf16 operand conversion used on the weight load path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float fp16_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Fragment k-order.  An MFMA lane holds 8 consecutive-k operands of one row
// (A) or one column (B).  A byte of int4 codes holds k = 2m and 2m+1, so the
// cheap mask-and-or conversion below produces the 8 codes of a 32-bit word in
// the order k = 0,4,1,5,2,6,3,7.  The contraction over k does not care about
// the order as long as A uses the same one, so every A fragment is put in that
// order too (permute_a for natural-order rows; the gate/up kernel stores h
// already in this order, see h_phys_col).

// Four 32-bit words of 8 natural-order bf16 -> the 0,4,1,5,2,6,3,7 order.
__device__ __forceinline__ u32x4 permute_a(u32x4 a) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(a.z, a.x, 0x05040100u);  // (k0, k4)
  r.y = __builtin_amdgcn_perm(a.z, a.x, 0x07060302u);  // (k1, k5)
  r.z = __builtin_amdgcn_perm(a.w, a.y, 0x05040100u);  // (k2, k6)
  r.w = __builtin_amdgcn_perm(a.w, a.y, 0x07060302u);  // (k3, k7)
  return r;
}

// Physical position, inside its group of 8, of logical column i of h.
__device__ __forceinline__ int h_phys_col(int n) {
  return (n & ~7) | ((n & 3) << 1) | ((n >> 2) & 1);
}

// int4 dequantisation on the load path.  OR-ing a code q (0..15) into the
// mantissa of bf16 128.0 (0x4300) gives exactly 128 + q, so one 32-bit word
// of 8 codes becomes four bf16 pairs with a shift and an and-or each.  The
// MFMA then accumulates sum_k a_k (128 + q_k); the per-row scale s and
// zero-point z are applied once per output in the epilogue:
//     sum_k a_k (q_k - z) s = s * (acc - (128 + z) * sum_k a_k).
constexpr float kCodeBias = 128.0f;

// Each output is one v_and_or_b32.  That encoding takes no literal constants,
// so with literal masks the compiler splits it into an and and an or; the two
// constants are therefore materialised opaquely (an SGPR and a VGPR, hoisted
// out of loops) and the and-or itself stays compiler-generated, so that the
// compiler still sees the writes the matrix cores read.
__device__ __forceinline__ u32x4 codes_to_bf16(uint32_t w) {
  uint32_t mask, bias;
  asm("s_mov_b32 %0, 0x000f000f" : "=s"(mask));
  asm("v_mov_b32 %0, 0x43004300" : "=v"(bias));
  u32x4 r;
  r.x = (w & mask) | bias;          // (q0, q4)
  r.y = ((w >> 4) & mask) | bias;   // (q1, q5)
  r.z = ((w >> 8) & mask) | bias;   // (q2, q6)
  r.w = ((w >> 12) & mask) | bias;  // (q3, q7)
  return r;
}

// The same with the mask and bias given (zero for both gives zeros).
__device__ __forceinline__ u32x4 codes_to_bf16_masked(uint32_t w, uint32_t mask, uint32_t bias) {
  u32x4 r;
  r.x = (w & mask) | bias;
  r.y = ((w >> 4) & mask) | bias;
  r.z = ((w >> 8) & mask) | bias;
  r.w = ((w >> 12) & mask) | bias;
  return r;
}

// 8-bit codes on the load path: bytes k0..k3 in w0 and k4..k7 in w1 -> the
// bf16 pairs (k0, k4), (k1, k5), (k2, k6), (k3, k7), the fragment k-order
// above.  A code 0..255 has at most 8 significant bits, so it converts to
// fp32 exactly (v_cvt_f32_ubyteN) and its bf16 pattern is the top half of the
// fp32 one (one v_perm_b32 per pair); the MFMA accumulates sum_k a_k q_k and
// the epilogue applies s * (acc - z * sum_k a_k).
__device__ __forceinline__ float code_byte_f32(uint32_t w, int i) { return (float)((w >> (8 * i)) & 0xFFu); }
__device__ __forceinline__ uint32_t pack_exact_bf16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ u32x4 bytes_to_bf16(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r.x = pack_exact_bf16(code_byte_f32(w0, 0), code_byte_f32(w1, 0));
  r.y = pack_exact_bf16(code_byte_f32(w0, 1), code_byte_f32(w1, 1));
  r.z = pack_exact_bf16(code_byte_f32(w0, 2), code_byte_f32(w1, 2));
  r.w = pack_exact_bf16(code_byte_f32(w0, 3), code_byte_f32(w1, 3));
  return r;
}

// 8-bit codes to bf16(q f + m), in the fragment order of bytes_to_bf16 (the
// conversion rounds to nearest even).  With f = 1 and m = -z (integer z)
// this is q - z, exact: |q - z| <= 255 has at most 8 significant bits; f = 0,
// m = 0 gives zeros.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ u32x4 dequant_int8_bf16(uint32_t w0, uint32_t w1, float s, float m) {
  u32x4 r;
  r.x = pack_bf16_rne(fmaf(code_byte_f32(w0, 0), s, m), fmaf(code_byte_f32(w1, 0), s, m));
  r.y = pack_bf16_rne(fmaf(code_byte_f32(w0, 1), s, m), fmaf(code_byte_f32(w1, 1), s, m));
  r.z = pack_bf16_rne(fmaf(code_byte_f32(w0, 2), s, m), fmaf(code_byte_f32(w1, 2), s, m));
  r.w = pack_bf16_rne(fmaf(code_byte_f32(w0, 3), s, m), fmaf(code_byte_f32(w1, 3), s, m));
  return r;
}

// Offset the widened codes carry: 128 for int4 (128 + q), none for 8-bit.
template <int BITS>
constexpr float code_bias() { return BITS == 4 ? kCodeBias : 0.0f; }

// bf16 1.0 in every slot: a B operand whose product gives row sums of A.
__device__ __forceinline__ u32x4 ones_bf16() {
  u32x4 r;
  r.x = r.y = r.z = r.w = 0x3F803F80u;
  return r;
}

// D += A(16x32) * B(32x16), bf16 in, fp32 accumulate.  Lane l holds A row
// l%16 and B column l%16 for the k-slice of lane group l/16; D row
// 4*(l/16) + i, column l%16 sits in element i.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (about 1 ulp
// each, far below the bf16 rounding h gets next).  Saturates correctly:
// e^-g -> inf gives g * 0, e^-g -> 0 gives g.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

// Hand-over between blocks of one kernel without flushing caches.  The L2 of
// each XCD is not coherent with the others for ordinary accesses, and a
// device-scope fence writes back and invalidates the whole L2.  Data that
// the last block of a kernel reads from the other blocks is instead written
// and read with device-scope relaxed atomics (coherent single accesses), the
// writer waits for its stores to complete before taking its completion
// ticket, and the ticket is a device-scope atomic counter.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), (uint64_t)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_coherent(const double* p) {
  return __longlong_as_double(
      (long long)__hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<double*>(p)), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT));
}
// Waits until this thread's memory operations have completed (no cache flush).
__device__ __forceinline__ void wait_all_memory() {
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Takes a completion ticket; true for the last of `total` blocks.  Every thread
// of the block must call it (it contains barriers); the caller has stored its
// hand-over data with store_coherent.
__device__ __forceinline__ bool last_block_ticket(uint32_t* ticket, uint32_t total, int* lds_flag) {
  wait_all_memory();
  __syncthreads();
  if (threadIdx.x == 0)
    *lds_flag = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1;
  __syncthreads();
  const bool last = *lds_flag != 0;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return last;
}
__device__ __forceinline__ void reset_ticket(uint32_t* ticket) {
  __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe
