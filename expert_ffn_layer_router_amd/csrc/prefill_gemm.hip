// Prefill family of the grouped expert GEMMs: many rows per expert, so the
// layer is bound by the matrix cores.
//
// Strata page, section 3.2: the tokens routed to one expert are concatenated
// and the experts' products run as one group GEMM (the chunked prefill of
// section 4.3 brings 2048-token chunks); section 3.1: per-expert int4 weights
// with their own scale and zero-point, dequantised on the load path.
//
// A block computes a 128-row tile of one expert's group against 256 weight
// rows (gate/up: 128 output columns of gate and of up; down: 256 output
// columns) on v_mfma_f32_32x32x16_bf16.  Its 4 waves are 2 x 2, each owning
// 64 rows x 128 weight rows (8 accumulators of 32 x 32).  The k range is
// walked in stages of 64: per stage the activation tile (128 rows x 128 B)
// and the int4 weight tile (256 rows x 32 B) are copied from global memory
// straight into LDS (global_load_lds_dwordx4), double-buffered and
// XOR-swizzled for conflict-free fragment reads.  Both A operands (x, copied
// by the router's top-k kernel, and h) are stored in the fragment k-order of
// the codes, so fragments go to the matrix cores as read.  Each lane widens one 32-bit
// word of codes into a bf16 B fragment (codes_to_bf16); scale and zero-point
// are applied in the epilogue with precomputed row sums of A (token row sums
// from the router, h row sums from the gate/up epilogue), which keeps the
// matrix cores free of the extra row-sum product the decode kernels use.
#include "device_common.h"
#include "plan.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = kPrefillTileRows;   // 128 rows per block
constexpr int kBK = 64;                 // k per stage
constexpr int kARow = kBK * 2;          // 128 bytes of an activation row per stage
constexpr int kWRow = kBK / 2;          // 32 bytes of a weight row per stage
constexpr int kABytes = kBM * kARow;    // 16 KB
#ifndef MOE_PF_GU_STAGES
#define MOE_PF_GU_STAGES 2
#endif
#ifndef MOE_PF_GU_BLOCKS
#define MOE_PF_GU_BLOCKS 2
#endif
#ifndef MOE_PF_DN_STAGES
#define MOE_PF_DN_STAGES 2
#endif
#ifndef MOE_PF_DN_BLOCKS
#define MOE_PF_DN_BLOCKS 2
#endif
// stage buffers (copies in flight + 1) and blocks per compute unit aimed for
constexpr int kPrefillGateUpStages = MOE_PF_GU_STAGES, kPrefillGateUpBlocks = MOE_PF_GU_BLOCKS;
constexpr int kPrefillDownStages = MOE_PF_DN_STAGES, kPrefillDownBlocks = MOE_PF_DN_BLOCKS;

__device__ __forceinline__ void load_lds16(const void* g, char* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds_base, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// swizzled chunk positions: activation rows hold 8 chunks of 16 B, weight rows 2
__device__ __forceinline__ int apos(int row, int c) { return c ^ ((row >> 1) & 7); }
__device__ __forceinline__ int wpos(int row, int c) { return c ^ ((row >> 3) & 1); }

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

}  // namespace

struct PrefillArgs {
  const uint16_t* act;        // gate/up: hidden [T][d]; down: h [R][dff]
  const int32_t* perm;        // gate/up: grouped position -> assignment
  const int4* tiles;
  const int32_t* num_tiles;
  const float* xsum;          // gate/up: [T] row sums of hidden
  float* hsum_part;           // gate/up writes, down reads: [R][dff / 128]
  int num_slots, d, dff, topk;
  const uint8_t* w0;          // gate (or down) codes
  const uint8_t* w1;          // up codes
  const uint16_t *s0, *z0, *s1, *z1;
  uint16_t* h;                // gate/up output [R][dff], fragment k-order
  float* y;                   // down output [R][d]
  uint32_t* flags;
};

// NJ: 32-column MFMA blocks per wave; a block holds 2 x NJ x 32 weight rows.
// GATEUP (NJ = 4): h = silu(x Wg^T) * (x Wu^T) for 128 rows x 128 columns,
// plus the rows' partial sums of h over those columns.  !GATEUP: y = h Wd^T
// for 128 rows x 64 NJ columns.  kNBuf LDS stage buffers (kNBuf - 1 stages in
// flight); OCC blocks per compute unit (2 keeps the accumulators in VGPRs
// and lets two blocks hide each other's barriers and LDS latency).
template <bool GATEUP, int NJ, int kNBuf, int OCC>
__global__ __launch_bounds__(256, OCC) void prefill_gemm_kernel(PrefillArgs a) {
  constexpr int kWRows = 64 * NJ;             // weight rows per block
  constexpr int kWBytes = kWRows * kWRow;
  constexpr int kStage = kABytes + kWBytes;
  constexpr int kWI = NJ / 2;                 // weight-load instructions per wave per stage
  static_assert(!GATEUP || NJ == 4, "gate/up blocks pair 2 gate and 2 up column blocks per wave");
  // One LDS object for the stage ring and the row sums: with several, the
  // compiler's alias information makes every LDS read wait for all
  // direct-to-LDS copies in flight (next stages included); the explicit
  // vmcnt waits below order the reads instead.
  __shared__ __attribute__((aligned(1024))) char smem[kNBuf * kStage + 3 * kBM * 4];
  float* rowsum = reinterpret_cast<float*>(smem + kNBuf * kStage);       // [kBM]
  float (*hpart)[kBM] = reinterpret_cast<float (*)[kBM]>(rowsum + kBM);  // [2][kBM]
  const int ntiles = *a.num_tiles;
  const int tile = blockIdx.y;
  if (tile >= ntiles) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int4 td = a.tiles[tile];  // (expert, slot, first grouped row, rows)
  const int slot = td.y, pbase = td.z, rows = td.w;
  const int ncols = GATEUP ? a.dff : a.d;
  const int K = GATEUP ? a.d : a.dff;
  const int n0 = blockIdx.x * (GATEUP ? kWRows / 2 : kWRows);  // first output column
  if (slot < 0 || slot >= a.num_slots) {
    if (tid == 0) atomicOr(a.flags, MOE_FLAG_BAD_SLOT);
    if (!GATEUP) {
      for (int i = tid; i < rows * kWRows; i += 256)
        a.y[(size_t)(pbase + i / kWRows) * a.d + n0 + i % kWRows] = 0.0f;
    }
    return;
  }
  const size_t wrow_bytes = (size_t)K / 2;

  // activation rows this lane copies: 16 instructions of 8 rows per stage, 4 per wave
  const uint8_t* asrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (wave * 4 + j) * 8 + lane / 8;
    const int rr = r < rows ? r : 0;
    const uint16_t* rowp = GATEUP ? a.act + (size_t)(a.perm[pbase + rr] / a.topk) * a.d
                                  : a.act + (size_t)(pbase + rr) * a.dff;
    asrc[j] = reinterpret_cast<const uint8_t*>(rowp) + 16 * apos(r, lane % 8);
  }
  // weight rows: 2 NJ instructions of 32 rows per stage, NJ / 2 per wave
  const uint8_t* wsrc[kWI];
#pragma unroll
  for (int j = 0; j < kWI; ++j) {
    const int r = (wave * kWI + j) * 32 + lane / 2;
    const uint8_t* base = a.w0;
    int n = n0 + r;
    if (GATEUP) {
      base = r < kWRows / 2 ? a.w0 : a.w1;
      n = n0 + (r % (kWRows / 2));
    }
    wsrc[j] = base + ((size_t)slot * ncols + n) * wrow_bytes + 16 * wpos(r, lane % 2);
  }
  // row sums of A for the zero-point term
  if (tid < kBM) {
    float v = 0.0f;
    if (tid < rows) {
      if (GATEUP) {
        v = a.xsum[a.perm[pbase + tid] / a.topk];
      } else {
        const int nparts = a.dff / 128;
        const float* hp = a.hsum_part + (size_t)(pbase + tid) * nparts;
        for (int i = 0; i < nparts; ++i) v += hp[i];
      }
    }
    rowsum[tid] = v;
  }

  auto issue = [&](int st) {
    char* buf = smem + (st % kNBuf) * kStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) load_lds16(asrc[j] + (size_t)st * kARow, buf + (wave * 4 + j) * 1024);
#pragma unroll
    for (int j = 0; j < kWI; ++j)
      load_lds16(wsrc[j] + (size_t)st * kWRow, buf + kABytes + (wave * kWI + j) * 1024);
  };

  f32x16 acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  // this wave's weight rows: gate/up -> gate 64wn + 32j (j < 2) and up 128 + 64wn + 32(j-2);
  // down -> 32 NJ wn + 32j
  int wr[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    wr[j] = GATEUP ? (j < 2 ? 64 * wn + 32 * j : kWRows / 2 + 64 * wn + 32 * (j - 2)) : 32 * NJ * wn + 32 * j;

  const int nst = K / kBK;
#pragma unroll
  for (int st = 0; st < kNBuf - 1; ++st)
    if (st < nst) issue(st);
  for (int st = 0; st < nst; ++st) {
    if (st + kNBuf - 1 < nst) issue(st + kNBuf - 1);
    // wait until stage st has landed: the stages issued after it may stay in flight
    const int later = min(kNBuf - 1, nst - 1 - st);
    if (kNBuf > 3 && later >= 3)
      wait_vmem<(kNBuf > 3 ? 3 : 0) * (4 + kWI)>();
    else if (kNBuf > 2 && later >= 2)
      wait_vmem<(kNBuf > 2 ? 2 : 0) * (4 + kWI)>();
    else if (later >= 1)
      wait_vmem<4 + kWI>();
    else
      wait_vmem<0>();
    lds_barrier();
    const char* buf = smem + (st % kNBuf) * kStage;
    u32x4 bq[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = wr[j] + l32;
      bq[j] = *reinterpret_cast<const u32x4*>(buf + kABytes + r * kWRow + 16 * wpos(r, hh));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 av[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + l32;
        const u32x4 raw = *reinterpret_cast<const u32x4*>(buf + r * kARow + 16 * apos(r, 4 * hh + s));
        av[i] = raw;  // x and h are stored in fragment order already
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4 b = codes_to_bf16(bq[j][s]);
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][j] = mfma32(av[i], b, acc[i][j]);
      }
    }
    lds_barrier();
  }

  // epilogue; accumulator element e of lane l is row 8(e/4) + 4(l/32) + e%4, column l%32
  if (GATEUP) {
    float psum[2][16];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int n = n0 + 64 * wn + 32 * jj + l32;
      const size_t sidx = (size_t)slot * ncols + n;
      const float sg = fp16_to_f32(a.s0[sidx]), cg = kCodeBias + fp16_to_f32(a.z0[sidx]);
      const float su = fp16_to_f32(a.s1[sidx]), cu = kCodeBias + fp16_to_f32(a.z1[sidx]);
      const int hcol = h_phys_col(n);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 64 * wm + 32 * i + 8 * (e / 4) + 4 * hh + (e % 4);
          const float xs = rowsum[row];
          const float g = sg * (acc[i][jj][e] - cg * xs);
          const float u = su * (acc[i][jj + 2][e] - cu * xs);
          const uint16_t hb = f32_to_bf16(silu(g) * u);
          const float hv = bf16_to_f32(hb);
          psum[i][e] = (jj == 0 ? 0.0f : psum[i][e]) + hv;
          if (row < rows) a.h[(size_t)(pbase + row) * a.dff + hcol] = hb;
        }
      }
    }
    // sum each row's partials over the 32 lanes holding its columns, then over the 2 waves
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = psum[i][e];
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, 32);
        psum[i][e] = v;
      }
    if (l32 == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) hpart[wn][64 * wm + 32 * i + 8 * (e / 4) + 4 * hh + (e % 4)] = psum[i][e];
    }
    __syncthreads();
    if (tid < rows && tid < kBM)
      a.hsum_part[(size_t)(pbase + tid) * (a.dff / 128) + blockIdx.x] = hpart[0][tid] + hpart[1][tid];
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + 32 * NJ * wn + 32 * j + l32;
      const size_t sidx = (size_t)slot * ncols + n;
      const float sd = fp16_to_f32(a.s0[sidx]), cd = kCodeBias + fp16_to_f32(a.z0[sidx]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 64 * wm + 32 * i + 8 * (e / 4) + 4 * hh + (e % 4);
          if (row < rows) a.y[(size_t)(pbase + row) * a.d + n] = sd * (acc[i][j][e] - cd * rowsum[row]);
        }
      }
    }
  }
}

void launch_gateup_prefill(const moe_config& c, const Plan& p, const uint16_t* hidden, const moe_weights& w,
                           char* ws, hipStream_t s) {
  PrefillArgs a{};
  (void)hidden;  // read through the router's copy of x in fragment k-order
  a.act = reinterpret_cast<const uint16_t*>(ws + p.xperm);
  a.perm = reinterpret_cast<const int32_t*>(ws + p.perm);
  a.tiles = reinterpret_cast<const int4*>(ws + p.tiles);
  a.num_tiles = reinterpret_cast<const int32_t*>(ws + p.num_tiles);
  a.xsum = reinterpret_cast<const float*>(ws + p.xsum);
  a.hsum_part = reinterpret_cast<float*>(ws + p.hsum_part);
  a.num_slots = c.num_slots;
  a.d = c.d_model;
  a.dff = c.d_ff;
  a.topk = c.top_k;
  a.w0 = w.w_gate;
  a.w1 = w.w_up;
  a.s0 = w.s_gate;
  a.z0 = w.z_gate;
  a.s1 = w.s_up;
  a.z1 = w.z_up;
  a.h = reinterpret_cast<uint16_t*>(ws + p.h);
  a.flags = reinterpret_cast<uint32_t*>(ws + p.flags);
  dim3 grid(c.d_ff / 128, p.max_tiles);
  prefill_gemm_kernel<true, 4, kPrefillGateUpStages, kPrefillGateUpBlocks><<<grid, 256, 0, s>>>(a);
}

void launch_down_prefill(const moe_config& c, const Plan& p, const moe_weights& w, char* ws, hipStream_t s) {
  PrefillArgs a{};
  a.act = reinterpret_cast<const uint16_t*>(ws + p.h);
  a.tiles = reinterpret_cast<const int4*>(ws + p.tiles);
  a.num_tiles = reinterpret_cast<const int32_t*>(ws + p.num_tiles);
  a.hsum_part = reinterpret_cast<float*>(ws + p.hsum_part);
  a.num_slots = c.num_slots;
  a.d = c.d_model;
  a.dff = c.d_ff;
  a.topk = c.top_k;
  a.w0 = w.w_down;
  a.s0 = w.s_down;
  a.z0 = w.z_down;
  a.y = reinterpret_cast<float*>(ws + p.y);
  a.flags = reinterpret_cast<uint32_t*>(ws + p.flags);
  if (c.d_model % 256 == 0) {
    prefill_gemm_kernel<false, 4, kPrefillDownStages, kPrefillDownBlocks><<<dim3(c.d_model / 256, p.max_tiles), 256, 0, s>>>(a);
  } else {
    prefill_gemm_kernel<false, 2, 2, 2><<<dim3(c.d_model / 128, p.max_tiles), 256, 0, s>>>(a);
  }
}

}  // namespace moe
