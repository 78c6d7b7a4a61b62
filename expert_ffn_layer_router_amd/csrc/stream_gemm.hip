// Decode family of the grouped expert GEMMs: few rows per expert, so the
// layer is bound by streaming its int4 weights from HBM.
//
// Strata page, section 3.2: the tokens of one expert are concatenated and all
// active experts run as one group GEMM; section 3.1: per-expert int4 weights
// with their own scale and zero-point, dequantised on the load path.
//
// A block owns one row tile of one expert (up to 16 rows of its group) and
// 64 x NCW output columns; each of its 4 waves computes 16 x NCW of them.  The
// k range is walked in stages of kStageK: per stage the block copies 128 bytes
// of every weight row it needs (gate and up rows, or down rows) and 512 bytes
// of every activation row straight from HBM into LDS (global_load_lds_dwordx4,
// full 128-byte lines, several rows per instruction) into one of two
// buffers, so the next stage is in flight while one is multiplied; activation
// rows past the tile's end are not copied.  Wider blocks (NCW = 2) halve the
// activation bytes staged per weight byte.  The 16-byte
// chunks are XOR-swizzled in LDS so that the MFMA fragment reads are free of
// bank conflicts.  Codes are widened to bf16 in registers (codes_to_bf16) and
// the scale / zero-point are applied in the epilogue; the row sums of A the
// zero-point term needs come from one extra MFMA against a B of ones.
//
// With few tokens the weighted scatter-back (combine) is fused into the down
// kernel: the last block to finish a 64-column slice (an atomic ticket per
// slice in the workspace's control words) sums that slice of every token's
// expert rows, in the same fixed order as the stand-alone combine kernel.
#include "device_common.h"
#include "plan.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kStageK = 256;                  // k per stage
constexpr int kWRowBytes = kStageK / 2;       // int4 bytes of one weight row per stage
constexpr int kARowBytes = kStageK * 2;       // bf16 bytes of one activation row per stage
constexpr int kRowsPerWInst = 1024 / kWRowBytes;  // weight rows per 1 KB load instruction (8)
constexpr int kRowsPerAInst = 1024 / kARowBytes;  // activation rows per instruction (2)

// 16 bytes from global memory to LDS: lane l of the wave writes lds_base + 16 l.
__device__ __forceinline__ void load_lds16(const void* g, char* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds_base, 16, 0, 0);
}

// Wait until at most `n` vector-memory operations of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] and [15:14], expcnt[6:4] and lgkmcnt[11:8] left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also orders global
// memory, which makes the compiler wait for every outstanding global load --
// including the next stage's copies, defeating the double buffering.  The LDS
// copies of a stage are waited for explicitly (wait_vmem) before this.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS reads written as inline assembly.  The compiler treats a plain LDS read
// as depending on every direct-to-LDS copy still in flight (it cannot tell
// the two stage buffers apart) and waits for all of them, next stage included,
// which would serialise the copy pipeline.  These reads are ordered by the
// explicit waits and barriers instead: lds_wait() waits for the wave's LDS
// reads, and lds_ready(v) makes each value depend on that wait, so no use of
// v is scheduled before it.
__device__ __forceinline__ u32x4 lds_read16(const char* p) {
  u32x4 v;
  const uint32_t addr = (uint32_t)(uintptr_t)(const lds_void*)p;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_ready(u32x4& v) { asm volatile("" : "+v"(v)); }

// Swizzled 16-byte chunk positions inside a stage buffer.
__device__ __forceinline__ int wchunk_pos(int row, int c) { return c ^ ((row >> 1) & 7); }  // c < 8
__device__ __forceinline__ int achunk_pos(int row, int q) { return q ^ (row & 15); }         // q < 32

// wait_vmem with a run-time count n in [BASE, BASE + EXTRA]
template <int BASE, int EXTRA>
__device__ __forceinline__ void wait_vmem_rt(int n) {
  if constexpr (EXTRA > 0) {
    if (n > BASE) {
      wait_vmem_rt<BASE + 1, EXTRA - 1>(n);
      return;
    }
  }
  wait_vmem<BASE>();
}

}  // namespace

struct FusedCombine {
  uint32_t* tickets;         // [d / columns per block] per column slice, zero between calls; null: none
  const int32_t* inv;        // [R]
  const float* topk_w;       // [R]
  uint16_t* out;             // [T][d]
  int T, k;
};

struct StreamArgs {
  const uint16_t* act;       // gate/up: hidden [T][d]; down: h [R][dff]
  const int32_t* perm;       // gate/up: grouped position -> assignment
  const int4* tiles;
  const int32_t* num_tiles;
  int num_slots, d, dff, topk, R, kchunk;
  const uint8_t* w0;         // gate (or down) codes
  const uint8_t* w1;         // up codes (gate/up only)
  const uint16_t *s0, *z0, *s1, *z1;
  uint16_t* h;               // gate/up output
  float* ypart;              // down output [split][R][d]
  uint32_t* flags;
  FusedCombine fc;
};

// GATEUP: h rows of one tile, silu(x Wg^T) * (x Wu^T) in bf16, columns of
// every group of 8 in the fragment k-order (h_phys_col).
// !GATEUP: ypart[split][p] = h[p] Wd^T over the k range of `split`, fp32,
// written with coherent stores; with a FusedCombine, the last block of each
// column slice also writes that slice of out[].
template <bool GATEUP, int NCW>
__global__ __launch_bounds__(256) void stream_gemm_kernel(StreamArgs a) {
  constexpr int COLS = 64 * NCW;                        // output columns per block
  constexpr int NWR = (GATEUP ? 2 : 1) * COLS;          // weight rows per stage
  constexpr int WBYTES = NWR * kWRowBytes, ABYTES = kStreamTileRows * kARowBytes;
  constexpr int SBYTES = WBYTES + ABYTES;
  constexpr int WI = NWR / kRowsPerWInst / 4;           // weight-load instructions per wave per stage
  constexpr int AI = kStreamTileRows / kRowsPerAInst / 4;  // activation-load instructions per wave per stage
  static_assert(WI * kRowsPerWInst * 4 == NWR && AI * kRowsPerAInst * 4 == kStreamTileRows, "even split over waves");
  __shared__ __attribute__((aligned(1024))) char smem[2 * SBYTES];
  __shared__ int is_last;

  const int ntiles = *a.num_tiles;
  const int tile = blockIdx.y;
  if (tile >= ntiles) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * COLS;
  const int4 td = a.tiles[tile];  // (expert, slot, first grouped row, rows <= 16)
  const int slot = td.y, pbase = td.z, rows = td.w;
  const int ncols_total = GATEUP ? a.dff : a.d;   // output columns of this GEMM
  const int K = GATEUP ? a.d : a.kchunk;          // k range of this block
  const int kbeg = GATEUP ? 0 : blockIdx.z * a.kchunk;
  const size_t row_bytes = (size_t)(GATEUP ? a.d : a.dff) / 2;
  const bool bad = slot < 0 || slot >= a.num_slots;
  float* yrow = GATEUP ? nullptr : a.ypart + ((size_t)blockIdx.z * a.R + pbase) * a.d;

  if (bad) {
    if (threadIdx.x == 0) atomicOr(a.flags, MOE_FLAG_BAD_SLOT);
    if (GATEUP) return;
#pragma unroll
    for (int cb = 0; cb < NCW; ++cb) {
      const int n = n0 + wave * 16 * NCW + cb * 16 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (grp * 4 + i < rows) store_coherent(&yrow[(size_t)(grp * 4 + i) * a.d + n], 0.0f);
    }
  } else {
    // activation row sources (gate/up: tokens through perm -- dependent loads first)
    int arow[AI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
      const int m = (wave * AI + j) * kRowsPerAInst + lane / 32;
      const int mm = m < rows ? m : 0;
      arow[j] = GATEUP ? a.perm[pbase + mm] : pbase + mm;
    }
    const uint8_t* wsrc[WI];
#pragma unroll
    for (int j = 0; j < WI; ++j) {
      const int r = (wave * WI + j) * kRowsPerWInst + lane / 8;  // block weight row
      const uint8_t* base = (!GATEUP || r < COLS) ? a.w0 : a.w1;
      const int n = n0 + (r % COLS);
      wsrc[j] = base + ((size_t)slot * ncols_total + n) * row_bytes + kbeg / 2 + 16 * wchunk_pos(r, lane % 8);
    }
    const int nst = (K + kStageK - 1) / kStageK;
    const bool half_last = (K % kStageK) != 0;
    auto issue_w = [&](int st) {
      char* buf = smem + (st & 1) * SBYTES;
      const bool half = half_last && st == nst - 1;
#pragma unroll
      for (int j = 0; j < WI; ++j) {
        const int r = (wave * WI + j) * kRowsPerWInst + lane / 8;
        if (!half || wchunk_pos(r, lane % 8) < 4)  // global chunk < 4: k inside the half stage
          load_lds16(wsrc[j] + (size_t)st * kWRowBytes, buf + (wave * WI + j) * 1024);
      }
    };
    issue_w(0);
    const uint8_t* asrc[AI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
      const int m = (wave * AI + j) * kRowsPerAInst + lane / 32;
      const uint16_t* rowp = GATEUP ? a.act + (size_t)(arow[j] / a.topk) * a.d
                                    : a.act + (size_t)arow[j] * a.dff + kbeg;
      asrc[j] = reinterpret_cast<const uint8_t*>(rowp) + 16 * achunk_pos(m, lane % 32);
    }
    // Activation rows past the tile's end are not copied (their LDS rows hold
    // stale data, which only reaches output rows that are never stored).  An
    // instruction whose rows all lie past the end is not issued at all: na of
    // this wave's AI instructions are, the same number every stage.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int na = min(AI, max(0, (rows - wave_u * AI * kRowsPerAInst + kRowsPerAInst - 1) / kRowsPerAInst));
    auto issue_a = [&](int st) {
      char* buf = smem + (st & 1) * SBYTES;
      const bool half = half_last && st == nst - 1;
#pragma unroll
      for (int j = 0; j < AI; ++j) {
        if (j < na) {
          const int m = (wave * AI + j) * kRowsPerAInst + lane / 32;
          if (m < rows && (!half || achunk_pos(m, lane % 32) < 16))
            load_lds16(asrc[j] + (size_t)st * kARowBytes, buf + WBYTES + (wave * AI + j) * 1024);
        }
      }
    };
    issue_a(0);

    f32x4 acc0[NCW], acc1[NCW], accs = {0, 0, 0, 0};
#pragma unroll
    for (int cb = 0; cb < NCW; ++cb) acc0[cb] = acc1[cb] = f32x4{0, 0, 0, 0};
    const u32x4 ones = ones_bf16();

    for (int st = 0; st < nst; ++st) {
      if (st + 1 < nst) {
        issue_w(st + 1);
        issue_a(st + 1);
      }
      // wait for this stage's copies; the next stage's (WI + na instructions,
      // unless it is a half stage, which counts as none: wait longer, never
      // shorter) stay in flight
      if (st + 1 < nst && !(half_last && st + 1 == nst - 1))
        wait_vmem_rt<WI, AI>(WI + na);
      else
        wait_vmem<0>();
      lds_barrier();
      const char* buf = smem + (st & 1) * SBYTES;
      const int nss = (half_last && st == nst - 1) ? 1 : 2;
      for (int ss = 0; ss < nss; ++ss) {
        const int c = 4 * ss + grp;
        u32x4 b0[NCW], b1[NCW], av[4];
#pragma unroll
        for (int cb = 0; cb < NCW; ++cb) {
          const int r0 = wave * 16 * NCW + cb * 16 + lr;
          b0[cb] = lds_read16(buf + r0 * kWRowBytes + 16 * wchunk_pos(r0, c));
          if (GATEUP) {
            const int r1 = COLS + r0;
            b1[cb] = lds_read16(buf + r1 * kWRowBytes + 16 * wchunk_pos(r1, c));
          }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) av[s] = lds_read16(buf + WBYTES + lr * kARowBytes + 16 * achunk_pos(lr, 16 * ss + 4 * grp + s));
        lds_wait();
#pragma unroll
        for (int cb = 0; cb < NCW; ++cb) {
          lds_ready(b0[cb]);
          if (GATEUP) lds_ready(b1[cb]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) lds_ready(av[s]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 x = GATEUP ? permute_a(av[s]) : av[s];  // h is stored in fragment order already
#pragma unroll
          for (int cb = 0; cb < NCW; ++cb) {
            acc0[cb] = mfma16(x, codes_to_bf16(b0[cb][s]), acc0[cb]);
            if (GATEUP) acc1[cb] = mfma16(x, codes_to_bf16(b1[cb][s]), acc1[cb]);
          }
          accs = mfma16(x, ones, accs);
        }
      }
      lds_barrier();
    }

#pragma unroll
    for (int cb = 0; cb < NCW; ++cb) {
      const int n = n0 + wave * 16 * NCW + cb * 16 + lr;
      const size_t sidx = (size_t)slot * ncols_total + n;
      const float sc0 = fp16_to_f32(a.s0[sidx]), cc0 = kCodeBias + fp16_to_f32(a.z0[sidx]);
      float sc1 = 0.0f, cc1 = 0.0f;
      if (GATEUP) {
        sc1 = fp16_to_f32(a.s1[sidx]);
        cc1 = kCodeBias + fp16_to_f32(a.z1[sidx]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = grp * 4 + i;
        if (row < rows) {
          const float sx = accs[i];
          const float v0 = sc0 * (acc0[cb][i] - cc0 * sx);
          if (GATEUP) {
            const float v1 = sc1 * (acc1[cb][i] - cc1 * sx);
            a.h[(size_t)(pbase + row) * a.dff + h_phys_col(n)] = f32_to_bf16(silu(v0) * v1);
          } else {
            store_coherent(&yrow[(size_t)row * a.d + n], v0);
          }
        }
      }
    }
  }

  if (GATEUP || a.fc.tickets == nullptr) return;
  // fused combine: the last block of this column slice gathers it for every token
  if (!last_block_ticket(&a.fc.tickets[blockIdx.x], (uint32_t)(ntiles * gridDim.z), &is_last)) return;
  const int nsplit = gridDim.z;
  __shared__ int rp[kStreamMaxTokens * 8];
  __shared__ float rw[kStreamMaxTokens * 8];
  for (int i = threadIdx.x; i < a.fc.T * a.fc.k; i += 256) {
    rp[i] = a.fc.inv[i];
    rw[i] = a.fc.topk_w[i];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.fc.T * COLS; i += 256) {
    const int t = i / COLS, col = n0 + i % COLS;
    float acc = 0.0f;
    for (int j = 0; j < a.fc.k; ++j) {
      const int p = rp[t * a.fc.k + j];
      float v = load_coherent(&a.ypart[(size_t)p * a.d + col]);
      for (int s = 1; s < nsplit; ++s) v += load_coherent(&a.ypart[((size_t)s * a.R + p) * a.d + col]);
      acc = fmaf(rw[t * a.fc.k + j], v, acc);
    }
    a.fc.out[(size_t)t * a.d + col] = f32_to_bf16(acc);
  }
  if (threadIdx.x == 0) reset_ticket(&a.fc.tickets[blockIdx.x]);
}

namespace {
template <bool GATEUP, int NCW>
void launch_stream(const moe_config& c, const Plan& p, const StreamArgs& args, hipStream_t s) {
  const int ncols = GATEUP ? c.d_ff : c.d_model;
  dim3 grid(ncols / (64 * NCW), p.max_tiles, GATEUP ? 1 : p.down_split);
  stream_gemm_kernel<GATEUP, NCW><<<grid, 256, 0, s>>>(args);
}
}  // namespace

void launch_gateup_stream(const moe_config& c, const Plan& p, const uint16_t* hidden, const moe_weights& w,
                          char* ws, hipStream_t s) {
  StreamArgs a{};
  a.act = hidden;
  a.perm = reinterpret_cast<const int32_t*>(ws + p.perm);
  a.tiles = reinterpret_cast<const int4*>(ws + p.tiles);
  a.num_tiles = reinterpret_cast<const int32_t*>(ws + p.num_tiles);
  a.num_slots = c.num_slots;
  a.d = c.d_model;
  a.dff = c.d_ff;
  a.topk = c.top_k;
  a.R = p.R;
  a.w0 = w.w_gate;
  a.w1 = w.w_up;
  a.s0 = w.s_gate;
  a.z0 = w.z_gate;
  a.s1 = w.s_up;
  a.z1 = w.z_up;
  a.h = reinterpret_cast<uint16_t*>(ws + p.h);
  a.flags = reinterpret_cast<uint32_t*>(ws + p.flags);
  if (p.gateup_ncw == 2)
    launch_stream<true, 2>(c, p, a, s);
  else
    launch_stream<true, 1>(c, p, a, s);
}

void launch_down_stream(const moe_config& c, const Plan& p, const moe_weights& w, uint16_t* out, char* ws,
                        hipStream_t s) {
  StreamArgs a{};
  a.act = reinterpret_cast<const uint16_t*>(ws + p.h);
  a.tiles = reinterpret_cast<const int4*>(ws + p.tiles);
  a.num_tiles = reinterpret_cast<const int32_t*>(ws + p.num_tiles);
  a.num_slots = c.num_slots;
  a.d = c.d_model;
  a.dff = c.d_ff;
  a.topk = c.top_k;
  a.R = p.R;
  a.kchunk = c.d_ff / p.down_split;
  a.w0 = w.w_down;
  a.s0 = w.s_down;
  a.z0 = w.z_down;
  a.ypart = reinterpret_cast<float*>(ws + p.y);
  a.flags = reinterpret_cast<uint32_t*>(ws + p.flags);
  if (p.fused_small) {
    a.fc.tickets = reinterpret_cast<uint32_t*>(ws + p.ctrl) + 1;
    a.fc.inv = reinterpret_cast<const int32_t*>(ws + p.inv);
    a.fc.topk_w = reinterpret_cast<const float*>(ws + p.topk_w);
    a.fc.out = out;
    a.fc.T = p.T;
    a.fc.k = c.top_k;
  }
  if (p.down_ncw == 2)
    launch_stream<false, 2>(c, p, a, s);
  else
    launch_stream<false, 1>(c, p, a, s);
}

}  // namespace moe
