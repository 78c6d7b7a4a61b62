// Prefill family of the grouped expert GEMMs: many rows per expert, so the
// layer is bound by the matrix cores.
//
// Strata page, section 3.2: the tokens routed to one expert are concatenated
// and the experts' products run as one group GEMM (the chunked prefill of
// section 4.3 brings 2048-token chunks); section 3.1: per-expert int4 weights
// with their own scale and zero-point, dequantised on the load path.
//
// A block computes a 128-row tile of one expert's group against 64 NJ weight
// rows on v_mfma_f32_32x32x16_bf16.  Gate/up: 8 waves side by side along 512
// weight rows (256 output columns of gate and of up), one block per compute
// unit; down: 4 waves along 256 weight rows (256 output columns), two blocks
// per compute unit.  Each wave owns 128 rows x 64 weight rows (8 accumulators
// of 32 x 32), so every widened weight fragment feeds 4 products and is
// widened by one wave only.  The k range is walked in stages (128 k for the
// int4 gate/up blocks, 64 k otherwise): per stage the activation tile (128
// rows) and the weight-code tile are copied from global memory straight into
// LDS (global_load_lds_dwordx4) through a 2-stage ring, with a chunk swizzle
// that keeps the fragment reads free of bank conflicts.  Both A operands (x,
// copied by the router's top-k kernel, and h) are stored in the fragment
// k-order of the codes, so fragments go to the matrix cores as read.  Each
// lane widens one 32-bit word of codes into a bf16 B fragment
// (codes_to_bf16); scale and zero-point are applied in the epilogue with
// precomputed row sums of A (token row sums from the router, h row sums from
// the gate/up epilogue), which keeps the matrix cores free of the extra
// row-sum product the decode kernels use.
#include <type_traits>

#include "device_common.h"
#include "plan.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = kPrefillTileRows;   // 128 rows per block
constexpr int kQGroup = 128;            // k per (s, z) group of the grouped formats
#ifndef MOE_PF_GU_STAGES
#define MOE_PF_GU_STAGES 2
#endif
#ifndef MOE_PF_GU_BLOCKS
#define MOE_PF_GU_BLOCKS 1
#endif
// k per stage of the int4 gate/up blocks (8-bit: 64, so that two stages fit the LDS)
#ifndef MOE_PF_GU_BK4
#define MOE_PF_GU_BK4 128
#endif
// per-row gate/up formats: stages handed over inside the last k-step
#ifndef MOE_PF_GU_HANDOVER
#define MOE_PF_GU_HANDOVER 1
#endif
// ... with each k-step's B fragments widened one step ahead
#ifndef MOE_PF_GU_WIDEN_AHEAD
#define MOE_PF_GU_WIDEN_AHEAD 1
#endif
#ifndef MOE_PF_DN_BK4
#define MOE_PF_DN_BK4 64   // k per stage of the int4 down blocks
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
#ifndef MOE_PF_GU_NJ
#define MOE_PF_GU_NJ 8
#endif
#ifndef MOE_PF_GU_NW
#define MOE_PF_GU_NW 8
#endif
#ifndef MOE_PF_GU_WN
#define MOE_PF_GU_WN MOE_PF_GU_NW
#endif
#ifndef MOE_PF_DN_NW
#define MOE_PF_DN_NW 4
#endif
#ifndef MOE_PF_DN_NJ
#define MOE_PF_DN_NJ 4
#endif
#ifndef MOE_PF_DN_WN
#define MOE_PF_DN_WN MOE_PF_DN_NW
#endif
// gate/up blocks: 64 NJ weight rows (32 NJ output columns) on NW waves, 1 x NW;
// down blocks: 256 weight rows on NW waves, 1 x NW
constexpr int kPrefillGateUpNJ = MOE_PF_GU_NJ, kPrefillGateUpWaves = MOE_PF_GU_NW;
constexpr int kPrefillDownWaves = MOE_PF_DN_NW;

__device__ __forceinline__ void load_lds16(const void* g, char* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds_base, 16, 0, 0);
}
// 4 bytes: lane l of the wave writes lds_base + 4 l.
__device__ __forceinline__ void load_lds4(const void* g, char* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds_base, 4, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Swizzled position of 16-byte chunk c of a row of NC chunks in a stage
// buffer (activation rows: 8 or 16 chunks; weight rows: 2, 4 or 8).  A
// fragment read (ds_read_b128) serves 16 lanes -- 16 consecutive rows -- per
// LDS cycle, 256 bytes across the 64 banks: 256 / (16 NC) rows share one
// 256-byte line, so the chunk is XORed with the row's index among the rows
// that fall on the same bank groups, (row / (16 / NC)) mod NC, and the 16
// rows hit 16 different 16-byte bank groups.
template <int NC>
__device__ __forceinline__ int spos(int row, int c) {
  static_assert(NC == 2 || NC == 4 || NC == 8 || NC == 16, "rows of 2 to 16 chunks");
  constexpr int kShift = NC == 2 ? 3 : NC == 4 ? 2 : NC == 8 ? 1 : 0;  // log2(16 / NC)
  return c ^ ((row >> kShift) & (NC - 1));
}

// Sum over the lane's row of 16 lanes: partners by lane ^ 1, lane ^ 2, then
// the half-row and row mirrors (DPP); every lane of the row ends with the same
// sum.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_partner<0xB1>(v);
  v += dpp_partner<0x4E>(v);
  v += dpp_partner<0x141>(v);
  v += dpp_partner<0x140>(v);
  return v;
}

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
  float* hsum_part;           // gate/up writes, down reads: [R][hparts] sums of h per 128 columns
  int hparts;                 // dff / 128
  // grouped formats: per row and 128-k group, the sum of A over the group
  // (gate/up: [T][d / 128] of hidden, by token; down: hsum_part)
  const float* gsum;
  int gsum_stride;
  int num_slots, d, dff, topk;
  const uint8_t* w0;          // gate (or down) codes
  const uint8_t* w1;          // up codes
  const uint16_t *s0, *z0, *s1, *z1;
  uint16_t* h;                // gate/up output [R][dff], fragment k-order
  uint16_t* y;                // down output [R][d], bf16
  uint32_t* flags;
};

// A block holds 128 rows and 64 NJ weight rows.  GATEUP: h = silu(x Wg^T) *
// (x Wu^T) for 128 rows x 32 NJ columns, plus the rows' partial sums of h
// over those columns.  !GATEUP: y = h Wd^T for 128 rows x 64 NJ columns.  The
// NW waves are (NW / WN) x WN over (rows x weight rows): a wave owns MI row
// blocks of 32 and NJW weight-row blocks of 32 (gate/up: half gate, half up,
// for the same columns), so every widened weight fragment feeds MI matrix-core
// products and every staged activation byte feeds 64 NJ weight rows.  kNBuf
// LDS stage buffers (kNBuf - 1 stages in flight); OCC blocks per compute unit.
//
// BITS: int4 or 8-bit codes (a stage holds 32 or 64 bytes of every weight
// row).  Per-row formats widen the codes exactly and apply (s, z) in the
// epilogue.  GROUPED (one (s, z) per output row and 128-k group): every
// stage also copies the (s, z) of its group for the block's weight rows into
// LDS, and each accumulator is kept in units of its column's current group
// scale: at a group boundary it is multiplied by s_old / s_new (one fp32
// rounding per group); the epilogue multiplies by the last scale.  A zero
// scale zeroes its group's terms and keeps the previous scale.  The
// zero-point z:
//  - int4: the codes are widened as for the per-row formats (128 + q, exact),
//    the stage also copies, for the block's rows, the sum S of A over the
//    group (precomputed), and the group's offset term -(128 + z) S enters
//    through one more matrix-core product per accumulator: S split into
//    three bf16 parts (about 24 significant bits) against -(128 + z) (exact
//    in bf16).  Cheaper in vector instructions than widening to q - z;
//  - 8-bit: the codes are widened to q - z (exact in bf16: at most 8
//    significant bits).  (The offset product measured slower here.)
template <bool GATEUP, int NJ, int kNBuf, int OCC, int WN, int NW, int BITS, bool GROUPED, int kBK>
__global__ __launch_bounds__(64 * NW, OCC) void prefill_gemm_kernel(PrefillArgs a) {
  static_assert(BITS == 4 || BITS == 8, "int4 or 8-bit codes");
  static_assert(kBK == 64 || kBK == 128, "stages of 64 or 128 k");
  constexpr int kThreads = 64 * NW;
  constexpr int kARow = kBK * 2;              // bytes of an activation row per stage
  constexpr int kACh = kARow / 16;            // its 16-byte chunks
  constexpr int kABytes = kBM * kARow;
  constexpr int kNS = kBK / 16;               // matrix-core k-steps per stage
  constexpr int kWRows = 64 * NJ;             // weight rows per block
  constexpr int kWRow = kBK * BITS / 8;       // bytes of a weight row per stage
  constexpr int kCPR = kWRow / 16;            // 16-byte chunks per weight row
  constexpr int kWBytes = kWRows * kWRow;
  // grouped: (s, z) of the stage's group, 2 kWRows fp16 entries, in 256-byte
  // copies (4 bytes per lane), kPI per wave
  constexpr int kPI = GROUPED ? (4 * kWRows + 256 * NW - 1) / (256 * NW) : 0;
  constexpr int kPBytes = kPI * 256 * NW;
  // grouped: the group sums S of the block's rows, one 256-byte copy (4 bytes
  // per lane) per wave, row (64 wave + lane) mod 128
  constexpr bool kOffsetMfma = GROUPED && BITS == 4;  // int4 grouped: the offset term as a product
  constexpr int kGI = kOffsetMfma ? 1 : 0;
  constexpr int kGBytes = kGI * 256 * NW;
  constexpr int kStage = kABytes + kWBytes + kPBytes + kGBytes;
  constexpr int kAI = (kABytes / 1024) / NW;  // activation-load instructions (1 KB) per wave per stage
  constexpr int kWI = (kWBytes / 1024) / NW;  // weight-load instructions per wave per stage
  constexpr float kBias = code_bias<BITS>();
  static_assert(!GROUPED || 2 * kWRows * 2 <= kPBytes, "the (s, z) of a stage fit");
  constexpr int WM = NW / WN;                 // waves along the rows
  constexpr int MI = (kBM / 32) / WM;         // row blocks of 32 per wave
  constexpr int NJW = (kWRows / 32) / WN;     // weight-row blocks of 32 per wave
  static_assert(kAI * NW * 1024 == kABytes && kWI * NW * 1024 == kWBytes, "even copy split");
  static_assert(WM * WN == NW && MI * WM * 32 == kBM && NJW * WN * 32 == kWRows, "wave grid");
  static_assert(!GATEUP || NJW % 2 == 0, "gate/up waves pair gate and up column blocks");
  // One LDS object for the stage ring and the row sums: with several, the
  // compiler's alias information makes every LDS read wait for all
  // direct-to-LDS copies in flight (next stages included); the explicit
  // vmcnt waits below order the reads instead.
  __shared__ __attribute__((aligned(1024))) char smem[kNBuf * kStage + kBM * 4];
  float* rowsum = reinterpret_cast<float*>(smem + kNBuf * kStage);  // [kBM]
  const int ntiles = *a.num_tiles;
  const int tile = blockIdx.y;
  if (tile >= ntiles) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hh = lane >> 5;
  const int4 td = a.tiles[tile];  // (expert, slot, first grouped row, rows)
  const int slot = td.y, pbase = td.z, rows = td.w;
  const int ncols = GATEUP ? a.dff : a.d;
  const int K = GATEUP ? a.d : a.dff;
  const int n0 = blockIdx.x * (GATEUP ? kWRows / 2 : kWRows);  // first output column
  if (slot < 0 || slot >= a.num_slots) {
    if (tid == 0) atomicOr(a.flags, MOE_FLAG_BAD_SLOT);
    if (!GATEUP) {
      for (int i = tid; i < rows * kWRows; i += kThreads)
        a.y[(size_t)(pbase + i / kWRows) * a.d + n0 + i % kWRows] = 0;
    }
    return;
  }
  const size_t wrow_bytes = (size_t)K * BITS / 8;

  // activation rows this lane copies: instructions of 1024 / kARow rows per stage, kAI per wave
  const uint8_t* asrc[kAI];
#pragma unroll
  for (int j = 0; j < kAI; ++j) {
    const int r = (wave * kAI + j) * (64 / kACh) + lane / kACh;
    const int rr = r < rows ? r : 0;
    const uint16_t* rowp = GATEUP ? a.act + (size_t)(a.perm[pbase + rr] / a.topk) * a.d
                                  : a.act + (size_t)(pbase + rr) * a.dff;
    asrc[j] = reinterpret_cast<const uint8_t*>(rowp) + 16 * spos<kACh>(r, lane % kACh);
  }
  // weight rows: instructions of 64 / kCPR rows per stage, kWI per wave
  const uint8_t* wsrc[kWI];
#pragma unroll
  for (int j = 0; j < kWI; ++j) {
    const int r = (wave * kWI + j) * (64 / kCPR) + lane / kCPR;
    const uint8_t* base = a.w0;
    int n = n0 + r;
    if (GATEUP) {
      base = r < kWRows / 2 ? a.w0 : a.w1;
      n = n0 + (r % (kWRows / 2));
    }
    wsrc[j] = base + ((size_t)slot * ncols + n) * wrow_bytes + 16 * spos<kCPR>(r, lane % kCPR);
  }
  // grouped: the (s, z) of the stage's group, entries e = 0 .. 2 kWRows - 1
  // in LDS (e < kWRows: s of block weight row e, then z), 2 entries per lane;
  // copies past the last entry load duplicates into the spare end of the area
  const int ngroups = K / kQGroup;
  const uint8_t* psrc[kPI > 0 ? kPI : 1] = {};
  if constexpr (GROUPED) {
#pragma unroll
    for (int q = 0; q < kPI; ++q) {
      const int e = ((q * NW + wave) * 128 + 2 * lane) % (2 * kWRows);
      const int r = e % kWRows;
      const bool zp = e >= kWRows;
      const uint16_t* arr = (!GATEUP || r < kWRows / 2) ? (zp ? a.z0 : a.s0) : (zp ? a.z1 : a.s1);
      const int n = n0 + (GATEUP ? r % (kWRows / 2) : r);
      psrc[q] = reinterpret_cast<const uint8_t*>(arr + (size_t)slot * ngroups * ncols + n);
    }
  }
  // grouped: this lane's row of the group sums
  const float* gsrc = nullptr;
  if constexpr (kOffsetMfma) {
    const int r = (64 * wave + lane) % kBM;
    const int rr = r < rows ? r : 0;
    const int grow = GATEUP ? a.perm[pbase + rr] / a.topk : pbase + rr;
    gsrc = a.gsum + (size_t)grow * a.gsum_stride;
  }
  auto issue = [&](int st) {
    char* buf = smem + (st % kNBuf) * kStage;
#pragma unroll
    for (int j = 0; j < kAI; ++j) load_lds16(asrc[j] + (size_t)st * kARow, buf + (wave * kAI + j) * 1024);
#pragma unroll
    for (int j = 0; j < kWI; ++j)
      load_lds16(wsrc[j] + (size_t)st * kWRow, buf + kABytes + (wave * kWI + j) * 1024);
    if constexpr (GROUPED) {
#pragma unroll
      for (int q = 0; q < kPI; ++q)
        load_lds4(psrc[q] + (size_t)(st * kBK / kQGroup) * ncols * 2, buf + kABytes + kWBytes + (q * NW + wave) * 256);
      if constexpr (kOffsetMfma) load_lds4(gsrc + st * kBK / kQGroup, buf + kABytes + kWBytes + kPBytes + wave * 256);
    }
  };

  f32x16 acc[MI][NJW];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJW; ++j) acc[i][j] = f32x16{};
  // this wave's weight rows: gate/up -> gate 16 NJW wn + 32j (j < NJW/2) and
  // up kWRows/2 + 16 NJW wn + 32(j - NJW/2); down -> 32 NJW wn + 32j
  constexpr int HJ = NJW / 2;
  int wr[NJW];
#pragma unroll
  for (int j = 0; j < NJW; ++j)
    wr[j] = GATEUP ? (j < HJ ? 32 * HJ * wn + 32 * j : kWRows / 2 + 32 * HJ * wn + 32 * (j - HJ)) : 32 * NJW * wn + 32 * j;

  // grouped formats: per weight-row block of this wave, the scale its sums
  // are kept in; int4: the current group's code mask and bias (zero for a
  // zero scale); 8-bit: its code factor (1, or 0 for a zero scale) and
  // offset (-z times it)
  float cur_s[NJW], gf[NJW], gm[NJW];
  uint32_t gmask[NJW], gbias[NJW];
#pragma unroll
  for (int j = 0; j < NJW; ++j) cur_s[j] = gf[j] = 1.0f, gm[j] = 0.0f, gmask[j] = gbias[j] = 0u;

  // row blocks of 32 of this wave that hold rows of the tile (the rest are
  // skipped: a tile's last rows may be missing)
  const int live_mi = __builtin_amdgcn_readfirstlane(min(MI, max(0, (rows - 32 * MI * wm + 31) / 32)));
  const int nst = K / kBK;
#pragma unroll
  for (int st = 0; st < kNBuf - 1; ++st)
    if (st < nst) issue(st);
  // Row sums of A for the zero-point term, loaded while the first stages are
  // in flight.  Gate/up: one token sum per row.  Down: the gate/up epilogue's
  // partial sums of h per 128 columns, hparts per row; the kThreads / kBM
  // threads of a row take contiguous runs of them with all loads of a batch
  // of 32 issued together (one round trip for up to 32 per thread; 16-byte
  // loads when the runs are whole 16-byte groups), then add the runs in a
  // fixed order.
  if constexpr (GATEUP) {
    if (tid < kBM) rowsum[tid] = tid < rows ? a.xsum[a.perm[pbase + tid] / a.topk] : 0.0f;
  } else {
    constexpr int kPer = kThreads / kBM;  // threads per row: 2 or 4, adjacent lanes
    static_assert(kPer * kBM == kThreads && (kPer == 1 || kPer == 2 || kPer == 4), "threads per row");
    const int r = tid / kPer, part = tid % kPer;
    const int run = (a.hparts + kPer - 1) / kPer;
    const int i0 = min(a.hparts, part * run), i1 = min(a.hparts, i0 + run);
    const float* hp = a.hsum_part + (size_t)(pbase + (r < rows ? r : 0)) * a.hparts;
    float v = 0.0f;
    if (a.hparts % (4 * kPer) == 0) {
      // rows of whole 16-byte groups and runs of them: 16-byte loads
      for (int i = i0; i < i1; i += 32) {
        float4 t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          t[u] = i + 4 * u < i1 ? *reinterpret_cast<const float4*>(hp + i + 4 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < 8; ++u) v += ((t[u].x + t[u].y) + t[u].z) + t[u].w;
      }
    } else {
      for (int i = i0; i < i1; i += 32) {
        float t[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) t[u] = i + u < i1 ? hp[i + u] : 0.0f;
#pragma unroll
        for (int u = 0; u < 32; ++u) v += t[u];
      }
    }
    if (kPer >= 2) v += __shfl_xor(v, 1, 64);
    if (kPer >= 4) v += __shfl_xor(v, 2, 64);
    if (part == 0) rowsum[r] = r < rows ? v : 0.0f;
  }
  // Per-row formats: the scales and zero-points of this wave's output
  // columns (gate/up: gate and up of HJ column blocks; down: NJW blocks),
  // loaded before the main loop so that the epilogue does not wait for them.
  constexpr int kEpi = GATEUP ? HJ : NJW;
  uint16_t es0[kEpi], ez0[kEpi], es1[kEpi], ez1[kEpi];
#pragma unroll
  for (int t = 0; t < kEpi; ++t) {
    es0[t] = ez0[t] = es1[t] = ez1[t] = 0;
    if constexpr (!GROUPED) {
      const size_t sidx = (size_t)slot * ncols + n0 + (GATEUP ? 32 * HJ * wn : 32 * NJW * wn) + 32 * t + l32;
      es0[t] = a.s0[sidx];
      ez0[t] = a.z0[sidx];
      if constexpr (GATEUP) {
        es1[t] = a.s1[sidx];
        ez1[t] = a.z1[sidx];
      }
    }
  }
  // The main loop for ML live row blocks of 32 (a tile's last rows may be
  // missing; their products are skipped), instantiated for each ML so that
  // the loop carries no branches.
  auto main_loop = [&](auto ml_tag) {
    constexpr int ML = decltype(ml_tag)::value;
    for (int st = 0; st < nst; ++st) {
      // wait until stage st has landed (the later stages issued so far -- at
      // most kNBuf - 2 -- may stay in flight), then a barrier: every wave is
      // past stage st - 1, so its buffer can be refilled with stage st + kNBuf - 1
      const int later = min(kNBuf - 2, nst - 1 - st);
      if (kNBuf > 3 && later >= 2)
        wait_vmem<(kNBuf > 3 ? 2 : 0) * (kAI + kWI + kPI + kGI)>();
      else if (kNBuf > 2 && later >= 1)
        wait_vmem<(kNBuf > 2 ? 1 : 0) * (kAI + kWI + kPI + kGI)>();
      else
        wait_vmem<0>();
      lds_barrier();
      if (st + kNBuf - 1 < nst) issue(st + kNBuf - 1);
      const char* buf = smem + (st % kNBuf) * kStage;
      // this lane's codes of the stage (k from kBK / 2 hh on): step s uses word s
      // (int4) or words 2s, 2s + 1 (8-bit); its A chunk is kNS hh + s
      u32x4 bq[NJW][kCPR / 2];
#pragma unroll
      for (int j = 0; j < NJW; ++j) {
        const int r = wr[j] + l32;
#pragma unroll
        for (int c = 0; c < kCPR / 2; ++c)
          bq[j][c] = *reinterpret_cast<const u32x4*>(buf + kABytes + r * kWRow +
                                                     16 * spos<kCPR>(r, (kCPR / 2) * hh + c));
      }
      if constexpr (GROUPED) {
        if ((st * kBK) % kQGroup == 0 && !kOffsetMfma) {  // 8-bit: first stage of a group
          const uint16_t* pz = reinterpret_cast<const uint16_t*>(buf + kABytes + kWBytes);
#pragma unroll
          for (int j = 0; j < NJW; ++j) {
            const int r = wr[j] + l32;
            const float sj = fp16_to_f32(pz[r]), zj = fp16_to_f32(pz[kWRows + r]);
            const bool live = sj != 0.0f;
            const float rho = live ? cur_s[j] / sj : 1.0f;
            cur_s[j] = live ? sj : cur_s[j];
            gf[j] = live ? 1.0f : 0.0f;
            gm[j] = -zj * gf[j];
#pragma unroll
            for (int i = 0; i < MI; ++i)
              if (i < ML) acc[i][j] *= rho;
          }
        }
        if ((st * kBK) % kQGroup == 0 && kOffsetMfma) {
          // int4: first stage of a group: its (s, z); rescale the sums, then
          // add the group's offset term -(128 + z) S as one product per
          // accumulator (A: S in three bf16 parts at k 0..2 of the lanes of
          // k-group 0; B: -(128 + z) at the same k; the rest zero)
          const uint16_t* pz = reinterpret_cast<const uint16_t*>(buf + kABytes + kWBytes);
          const float* gs = reinterpret_cast<const float*>(buf + kABytes + kWBytes + kPBytes);
          u32x4 sa[MI];
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            const float sv = gs[32 * MI * wm + 32 * i + l32];
            const uint16_t h0 = f32_to_bf16(sv);
            const float r1 = sv - bf16_to_f32(h0);
            const uint16_t h1 = f32_to_bf16(r1);
            const uint16_t h2 = f32_to_bf16(r1 - bf16_to_f32(h1));
            sa[i] = hh == 0 ? u32x4{(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2, 0u, 0u}
                            : u32x4{0u, 0u, 0u, 0u};
          }
#pragma unroll
          for (int j = 0; j < NJW; ++j) {
            const int r = wr[j] + l32;
            const float sj = fp16_to_f32(pz[r]), zj = fp16_to_f32(pz[kWRows + r]);
            const bool live = sj != 0.0f;
            const float rho = live ? cur_s[j] / sj : 1.0f;
            cur_s[j] = live ? sj : cur_s[j];
            gmask[j] = live ? 0x000F000Fu : 0u;
            gbias[j] = live ? 0x43004300u : 0u;
            const uint32_t nc = live ? (uint32_t)f32_to_bf16(-(kBias + zj)) : 0u;  // exact: an integer below 2^8
            const u32x4 sb = hh == 0 ? u32x4{nc | (nc << 16), nc, 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < MI; ++i)
              if (i < ML) acc[i][j] = mfma32(sa[i], sb, acc[i][j] * rho);
          }
        }
      }
      auto widen = [&](int j, int s) {
        const uint32_t w0 = bq[j][(BITS / 4) * s / 4][((BITS / 4) * s) % 4];
        if constexpr (BITS == 4) {
          if constexpr (GROUPED)
            return codes_to_bf16_masked(w0, gmask[j], gbias[j]);  // bias + q, or 0 for a zero scale
          else
            return codes_to_bf16(w0);
        } else {
          const uint32_t w1 = bq[j][(2 * s + 1) / 4][(2 * s + 1) % 4];
          if constexpr (GROUPED)
            return dequant_int8_bf16(w0, w1, gf[j], gm[j]);  // q - z, or 0 for a zero scale
          else
            return bytes_to_bf16(w0, w1);
        }
      };
      // A fragments (fragment order already) of step s; the next step's are read
      // before this step's products, so the LDS latency hides behind them
      auto read_a = [&](int s, u32x4(&av)[MI]) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int r = 32 * MI * wm + 32 * i + l32;
          if (i < ML) av[i] = *reinterpret_cast<const u32x4*>(buf + r * kARow + 16 * spos<kACh>(r, kNS * hh + s));
        }
      };
      u32x4 av0[MI], av1[MI];
      read_a(0, av0);
#pragma unroll
      for (int s = 0; s < kNS; ++s) {
        u32x4(&cur)[MI] = (s & 1) ? av1 : av0;
        u32x4(&nxt)[MI] = (s & 1) ? av0 : av1;
        if (s + 1 < kNS) read_a(s + 1, nxt);
#pragma unroll
        for (int j = 0; j < NJW; ++j) {
          const u32x4 b = widen(j, s);
#pragma unroll
          for (int i = 0; i < MI; ++i)
            if (i < ML) acc[i][j] = mfma32(cur[i], b, acc[i][j]);
        }
      }
    }
  };
  // Per-row gate/up formats with a 2-stage ring hand the stages over in the
  // middle of a stage's last k-step instead of at its start.  By then a wave
  // holds that step's fragments in registers (its A fragments were read during
  // the step before, its codes at the stage's start), so it waits for the next
  // stage, passes the barrier -- after which no wave reads the current buffer
  // again -- issues the copies of the stage after next into that buffer, reads
  // the next stage's codes and first A fragments, and only then runs the last
  // step's products: the LDS latency after the barrier hides behind them.
  auto main_loop_handover = [&](auto ml_tag) {
    constexpr int ML = decltype(ml_tag)::value;
    auto read_b = [&](const char* buf, u32x4(&bq)[NJW][kCPR / 2]) {
#pragma unroll
      for (int j = 0; j < NJW; ++j) {
        const int r = wr[j] + l32;
#pragma unroll
        for (int c = 0; c < kCPR / 2; ++c)
          bq[j][c] = *reinterpret_cast<const u32x4*>(buf + kABytes + r * kWRow +
                                                     16 * spos<kCPR>(r, (kCPR / 2) * hh + c));
      }
    };
    auto read_a = [&](const char* buf, int s, u32x4(&av)[MI]) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = 32 * MI * wm + 32 * i + l32;
        if (i < ML) av[i] = *reinterpret_cast<const u32x4*>(buf + r * kARow + 16 * spos<kACh>(r, kNS * hh + s));
      }
    };
    auto widen = [&](const u32x4(&bq)[NJW][kCPR / 2], int j, int s) {
      const uint32_t w0 = bq[j][(BITS / 4) * s / 4][((BITS / 4) * s) % 4];
      if constexpr (BITS == 4) {
        return codes_to_bf16(w0);
      } else {
        const uint32_t w1 = bq[j][(2 * s + 1) / 4][(2 * s + 1) % 4];
        return bytes_to_bf16(w0, w1);
      }
    };
    static_assert(kNS % 2 == 0, "the last step's A fragments are in av1, the next stage's first in av0");
    u32x4 bq[NJW][kCPR / 2], av0[MI], av1[MI], bc[NJW];
    wait_vmem<0>();
    lds_barrier();
    if (1 < nst) issue(1);
    read_b(smem, bq);
    read_a(smem, 0, av0);
#if MOE_PF_GU_WIDEN_AHEAD
#pragma unroll
    for (int j = 0; j < NJW; ++j) bc[j] = widen(bq, j, 0);
#endif
    for (int st = 0; st < nst; ++st) {
      const char* buf = smem + (st % 2) * kStage;
#pragma unroll
      for (int s = 0; s + 1 < kNS; ++s) {
        u32x4(&cur)[MI] = (s & 1) ? av1 : av0;
        u32x4(&nxt)[MI] = (s & 1) ? av0 : av1;
        read_a(buf, s + 1, nxt);
#if MOE_PF_GU_WIDEN_AHEAD
        // the next step's B fragments are widened, and its A fragments read,
        // before this step's products: no product waits for a widening
        // instruction or a read issued just before it
        u32x4 bn[NJW];
#pragma unroll
        for (int j = 0; j < NJW; ++j) bn[j] = widen(bq, j, s + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NJW; ++j)
#pragma unroll
          for (int i = 0; i < MI; ++i)
            if (i < ML) acc[i][j] = mfma32(cur[i], bc[j], acc[i][j]);
#pragma unroll
        for (int j = 0; j < NJW; ++j) bc[j] = bn[j];
#else
#pragma unroll
        for (int j = 0; j < NJW; ++j) {
          const u32x4 b = widen(bq, j, s);
#pragma unroll
          for (int i = 0; i < MI; ++i)
            if (i < ML) acc[i][j] = mfma32(cur[i], b, acc[i][j]);
        }
#endif
      }
      u32x4 bl[NJW];
#pragma unroll
      for (int j = 0; j < NJW; ++j) bl[j] = MOE_PF_GU_WIDEN_AHEAD ? bc[j] : widen(bq, j, kNS - 1);
      // Unconditional, so that no control-flow merge makes the compiler wait
      // for these reads before the products below: after the last stage the
      // reads take the other buffer's stale contents (unused) and the barrier
      // is one more that every wave takes.
      __builtin_amdgcn_sched_barrier(0);  // the earlier steps' products stay before the barrier
      wait_vmem<0>();  // stage st + 1 (this wave's copies of it)
      lds_barrier();   // ... and every wave's; no wave reads buffer st % 2 again
      const char* nb = smem + ((st + 1) % 2) * kStage;
      read_b(nb, bq);
      read_a(nb, 0, av0);
      __builtin_amdgcn_sched_barrier(0);  // all of these reads go out before the products
#pragma unroll
      for (int j = 0; j < NJW; ++j)
#pragma unroll
        for (int i = 0; i < MI; ++i)
          if (i < ML) acc[i][j] = mfma32(av1[i], bl[j], acc[i][j]);
#if MOE_PF_GU_WIDEN_AHEAD
#pragma unroll
      for (int j = 0; j < NJW; ++j) bc[j] = widen(bq, j, 0);
#endif
      // the copies of the stage after next, into the buffer just retired
      // (issued after the products, so that the reads and products above
      // stay in one block)
      if (st + 2 < nst) issue(st + 2);
    }
  };
  // exactly one instance runs on every path: each takes part in every barrier
  // (live_mi = 0 -- no row of this wave in the tile -- runs the 1-block one)
  auto run = [&](auto ml_tag) {
    if constexpr (GATEUP && !GROUPED && kNBuf == 2 && MOE_PF_GU_HANDOVER)
      main_loop_handover(ml_tag);
    else
      main_loop(ml_tag);
  };
  if (live_mi >= MI)
    run(std::integral_constant<int, MI>{});
  else if (live_mi == 3)
    run(std::integral_constant<int, 3>{});
  else if (live_mi == 2)
    run(std::integral_constant<int, 2>{});
  else
    run(std::integral_constant<int, 1>{});

  // epilogue; accumulator element e of lane l is row 8(e/4) + 4(l/32) + e%4, column l%32.
  // Results go through LDS (the stage ring is free once every wave is past
  // its last stage), so that global memory sees whole-row 16-byte stores.
  // The barriers here wait for LDS only: a store has read its data out of LDS
  // once issued, and nothing here reads global memory the stores write.
  lds_barrier();
  if constexpr (GATEUP) {
    constexpr int kCols = kWRows / 2;  // output columns of the block
    static_assert(kBM * kCols * 2 <= kNBuf * kStage, "h tile fits the stage ring");
    uint16_t* htile = reinterpret_cast<uint16_t*>(smem);  // [kBM][kCols], columns in h_phys_col order
#pragma unroll
    for (int jj = 0; jj < HJ; ++jj) {
      const int nl = 32 * HJ * wn + 32 * jj + l32;  // column inside the block (n0 is a multiple of 8)
      // grouped formats: the weights were dequantised in full already
      const float sg = GROUPED ? cur_s[jj] : fp16_to_f32(es0[jj]);
      const float cg = GROUPED ? 0.0f : kBias + fp16_to_f32(ez0[jj]);
      const float su = GROUPED ? cur_s[jj + HJ] : fp16_to_f32(es1[jj]);
      const float cu = GROUPED ? 0.0f : kBias + fp16_to_f32(ez1[jj]);
      const int hcol = h_phys_col(nl);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 32 * MI * wm + 32 * i + 8 * (e / 4) + 4 * hh + (e % 4);
          const float xs = rowsum[row];
          const float g = sg * (acc[i][jj][e] - cg * xs);
          const float u = su * (acc[i][jj + HJ][e] - cu * xs);
          htile[row * kCols + hcol] = f32_to_bf16(silu(g) * u);
        }
      }
    }
    lds_barrier();
    // Copy-out in whole-row 16-byte chunks; thread c takes chunk c % kChunks of
    // row c / kChunks, so the 16 chunks of a 128-column group (a group of the
    // grouped formats) are the 16 lanes of one DPP row: each thread adds its
    // chunk's 8 bf16 values of h and the row of lanes sums them, giving the
    // down GEMM the per-row sums of h per 128 columns for its zero-point term.
    // Every row of the tile takes part (uniform trip count for the
    // exchanges); only the tile's rows are stored.
    constexpr int kChunks = kCols / 8;  // 16-byte chunks per row
    constexpr int kGroups = kCols / kQGroup;
    static_assert(kGroups * kQGroup == kCols && kThreads % kChunks == 0 && kQGroup / 8 == 16,
                  "a group of 128 columns is one row of 16 lanes");
    for (int c = tid; c < kBM * kChunks; c += kThreads) {
      const int r = c / kChunks, q = c % kChunks;
      const u32x4 v = *reinterpret_cast<const u32x4*>(htile + r * kCols + 8 * q);
      if (r < rows) *reinterpret_cast<u32x4*>(a.h + (size_t)(pbase + r) * a.dff + n0 + 8 * q) = v;
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
      float cs = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) cs += __uint_as_float(vw[i] << 16) + __uint_as_float(vw[i] & 0xFFFF0000u);
      cs = row16_sum(cs);
      if (r < rows && q % 16 == 0) a.hsum_part[(size_t)(pbase + r) * a.hparts + blockIdx.x * kGroups + q / 16] = cs;
    }
  } else if constexpr (WM == 1) {
    // one pass per 32-row block: every wave holds all rows of the block
    static_assert(32 * kWRows * 4 <= kNBuf * kStage, "y tile fits the stage ring");
    float* ytile = reinterpret_cast<float*>(smem);  // [32][kWRows]
    float sd[NJW], cd[NJW];
#pragma unroll
    for (int j = 0; j < NJW; ++j) {
      sd[j] = GROUPED ? cur_s[j] : fp16_to_f32(es0[j]);
      cd[j] = GROUPED ? 0.0f : kBias + fp16_to_f32(ez0[j]);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (32 * i >= rows) break;
#pragma unroll
      for (int j = 0; j < NJW; ++j) {
        const int nl = 32 * NJW * wn + 32 * j + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int rl = 8 * (e / 4) + 4 * hh + (e % 4);
          ytile[rl * kWRows + nl] = sd[j] * (acc[i][j][e] - cd[j] * rowsum[32 * i + rl]);
        }
      }
      lds_barrier();
      constexpr int kChunks = kWRows / 8;  // 8 columns -> one 16-byte bf16 store
      const int nr = min(32, rows - 32 * i);
      for (int c = tid; c < nr * kChunks; c += kThreads) {
        const int r = c / kChunks, q = c % kChunks;
        const float4 v0 = *reinterpret_cast<const float4*>(ytile + r * kWRows + 8 * q);
        const float4 v1 = *reinterpret_cast<const float4*>(ytile + r * kWRows + 8 * q + 4);
        u32x4 o;
        o.x = (uint32_t)f32_to_bf16(v0.x) | ((uint32_t)f32_to_bf16(v0.y) << 16);
        o.y = (uint32_t)f32_to_bf16(v0.z) | ((uint32_t)f32_to_bf16(v0.w) << 16);
        o.z = (uint32_t)f32_to_bf16(v1.x) | ((uint32_t)f32_to_bf16(v1.y) << 16);
        o.w = (uint32_t)f32_to_bf16(v1.z) | ((uint32_t)f32_to_bf16(v1.w) << 16);
        *reinterpret_cast<u32x4*>(a.y + (size_t)(pbase + 32 * i + r) * a.d + n0 + 8 * q) = o;
      }
      lds_barrier();
    }
  } else {
#pragma unroll
    for (int j = 0; j < NJW; ++j) {
      const int n = n0 + 32 * NJW * wn + 32 * j + l32;
      const float sd = GROUPED ? cur_s[j] : fp16_to_f32(es0[j]);
      const float cd = GROUPED ? 0.0f : kBias + fp16_to_f32(ez0[j]);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 32 * MI * wm + 32 * i + 8 * (e / 4) + 4 * hh + (e % 4);
          if (row < rows) a.y[(size_t)(pbase + row) * a.d + n] = f32_to_bf16(sd * (acc[i][j][e] - cd * rowsum[row]));
        }
      }
    }
  }
}

namespace {
// gate/up blocks are 32 NJ output columns wide: the wide block when d_ff allows it
bool gateup_wide(const moe_config& c) { return c.d_ff % (32 * kPrefillGateUpNJ) == 0; }
int gateup_blocks(const moe_config& c) { return c.d_ff / (gateup_wide(c) ? 32 * kPrefillGateUpNJ : 128); }
// Calls f(bits, grouped) with the weight format as compile-time constants.
template <class F>
void with_format(const moe_config& c, F&& f) {
  using std::integral_constant;
  if (c.weight_bits == 8) {
    if (c.group_size) f(integral_constant<int, 8>{}, integral_constant<bool, true>{});
    else f(integral_constant<int, 8>{}, integral_constant<bool, false>{});
  } else {
    if (c.group_size) f(integral_constant<int, 4>{}, integral_constant<bool, true>{});
    else f(integral_constant<int, 4>{}, integral_constant<bool, false>{});
  }
}
}  // namespace

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
  a.gsum = reinterpret_cast<const float*>(ws + p.xgsum);
  a.gsum_stride = c.d_model / 128;
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
  a.hparts = c.d_ff / 128;
  dim3 grid(gateup_blocks(c), p.max_tiles);
  with_format(c, [&](auto bits, auto grouped) {
    constexpr int B = decltype(bits)::value;
    constexpr bool G = decltype(grouped)::value;
    if (gateup_wide(c))
      prefill_gemm_kernel<true, kPrefillGateUpNJ, kPrefillGateUpStages, kPrefillGateUpBlocks, MOE_PF_GU_WN,
                          kPrefillGateUpWaves, B, G, B == 4 ? MOE_PF_GU_BK4 : 64>
          <<<grid, 64 * kPrefillGateUpWaves, 0, s>>>(a);
    else
      prefill_gemm_kernel<true, 4, 2, 2, 4, 4, B, G, 64><<<grid, 256, 0, s>>>(a);
  });
}

void launch_down_prefill(const moe_config& c, const Plan& p, const moe_weights& w, char* ws, hipStream_t s) {
  PrefillArgs a{};
  a.act = reinterpret_cast<const uint16_t*>(ws + p.h);
  a.tiles = reinterpret_cast<const int4*>(ws + p.tiles);
  a.num_tiles = reinterpret_cast<const int32_t*>(ws + p.num_tiles);
  a.hsum_part = reinterpret_cast<float*>(ws + p.hsum_part);
  a.hparts = c.d_ff / 128;
  a.gsum = a.hsum_part;
  a.gsum_stride = a.hparts;
  a.num_slots = c.num_slots;
  a.d = c.d_model;
  a.dff = c.d_ff;
  a.topk = c.top_k;
  a.w0 = w.w_down;
  a.s0 = w.s_down;
  a.z0 = w.z_down;
  a.y = reinterpret_cast<uint16_t*>(ws + p.y);
  a.flags = reinterpret_cast<uint32_t*>(ws + p.flags);
  with_format(c, [&](auto bits, auto grouped) {
    constexpr int B = decltype(bits)::value;
    constexpr bool G = decltype(grouped)::value;
    if (c.d_model % (64 * MOE_PF_DN_NJ) == 0) {
      prefill_gemm_kernel<false, MOE_PF_DN_NJ, kPrefillDownStages, kPrefillDownBlocks, MOE_PF_DN_WN,
                          kPrefillDownWaves, B, G, (B == 4 ? MOE_PF_DN_BK4 : 64)>
          <<<dim3(c.d_model / (64 * MOE_PF_DN_NJ), p.max_tiles), 64 * kPrefillDownWaves, 0, s>>>(a);
    } else {
      prefill_gemm_kernel<false, 2, 2, 2, 2, 4, B, G, 64><<<dim3(c.d_model / 128, p.max_tiles), 256, 0, s>>>(a);
    }
  });
}

}  // namespace moe
