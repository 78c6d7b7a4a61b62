// Decode family of the grouped expert GEMMs: few rows per expert, so the
// layer is bound by streaming its int4 weights from HBM.
//
// Strata page, section 3.2: the tokens of one expert are concatenated and all
// active experts run as one group GEMM; section 3.1: per-expert int4 weights
// with their own scale and zero-point, dequantised on the load path.
//
// A block owns one row tile of one expert (up to 16 rows of its group) and
// 64 x NCW output columns, and walks its k range in stages of kStageK.  Per
// stage it copies 128 bytes of every weight row it needs (gate and up rows,
// or down rows) straight from HBM into LDS (global_load_lds_dwordx4, full
// 128-byte lines, 8 rows per instruction) into a ring of NBUF buffers, so
// the next stages are in flight while one is multiplied.  The 16-byte chunks
// are XOR-swizzled in LDS so that the MFMA fragment reads spread over the
// banks.
//
// The four waves split each stage's k range into KW parts and the block's
// columns into 4 / KW parts (wave w takes k part kp = w % KW and column part
// cp = w / KW).  Each wave loads its activation fragments straight from L2
// into registers, one stage ahead: per MFMA k-step 16 contiguous bytes of
// one row per lane.  The LDS thus holds weights only (2 x 16 KB for gate/up,
// 2 x 8 KB for down at NCW = 1), so more blocks -- and more weight bytes in
// flight -- fit on a CU than if the activations were staged there too; with
// KW = 4 no two waves load the same activation bytes.
//
// Codes are widened to bf16 in registers (codes_to_bf16); the row sums of A
// that the zero-point term needs come from one extra MFMA against a B of
// ones.  At the end every wave turns its k part into s (acc - (128 + z) sum a),
// which is linear in the k parts, and the parts are added in a fixed order
// through LDS by the wave that owns each column tile, which also stores it.
//
// With very few tokens the weighted scatter-back (combine) is fused into the
// down kernel: the last block to finish a 64-column slice (an atomic ticket
// per slice in the workspace's control words) sums that slice of every
// token's expert rows, in the same fixed order as the stand-alone kernel that
// otherwise sums the partials after it (combine.hip).
#include "device_common.h"
#include "plan.h"
#include "router_small.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWRowBytes = 128;              // bytes of one weight row per stage (256 int4 or 128 8-bit codes)
constexpr int kRowsPerWInst = 1024 / kWRowBytes;  // weight rows per 1 KB load instruction (8)
constexpr int kQGroup = 128;                 // k per (s, z) group of the grouped formats
constexpr int kPBytes = 1024;                // grouped formats: (s, z) bytes staged per stage

// 16 bytes from global memory to LDS: lane l of the wave writes lds_base + 16 l.
// NT: with the non-temporal hint, for lines read once per launch: they are
// marked for early eviction, so streaming them leaves the caches to the
// activations and to the next kernels' inputs.
template <bool NT>
__device__ __forceinline__ void load_lds16(const void* g, char* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds_base, 16, 0, NT ? 2 /* nt */ : 0);
}
// 4 bytes: lane l of the wave writes lds_base + 4 l.
__device__ __forceinline__ void load_lds4(const void* g, char* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds_base, 4, 0, 0);
}
// The same with the sc1 cache bit: coherent with stores of other blocks made
// with device-scope atomics (it reads past this XCD's L2).
__device__ __forceinline__ void load_lds4_coherent(const void* g, char* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds_base, 4, 0, 16 /* sc1 */);
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
// including the next stages' copies, defeating the ring.  The LDS copies of a
// stage are waited for explicitly (wait_vmem) before this.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS reads written as inline assembly.  The compiler treats a plain LDS read
// as depending on every direct-to-LDS copy still in flight (it cannot tell
// the ring's buffers apart) and waits for all of them, later stages included,
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
__device__ __forceinline__ u32x2 lds_read8(const char* p) {
  u32x2 v;
  const uint32_t addr = (uint32_t)(uintptr_t)(const lds_void*)p;
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ uint32_t lds_read_u16(const char* p) {
  uint32_t v;
  const uint32_t addr = (uint32_t)(uintptr_t)(const lds_void*)p;
  asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ uint32_t lds_read_b32(const char* p) {
  uint32_t v;
  const uint32_t addr = (uint32_t)(uintptr_t)(const lds_void*)p;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_ready(uint32_t& v) { asm volatile("" : "+v"(v)); }

// Swizzled position of 16-byte chunk c (< 8) of weight row `row` in a stage buffer.
__device__ __forceinline__ int wchunk_pos(int row, int c) { return c ^ ((row >> 1) & 7); }

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
  int max_tiles;             // grid rows of tiles (dense tiles: every expert)
  const uint8_t* w0;         // gate (or down) codes
  const uint8_t* w1;         // up codes (gate/up only)
  const uint16_t *s0, *z0, *s1, *z1;
  uint16_t* h;               // gate/up output
  float* ypart;              // down output [split][R][d]
  uint32_t* flags;
  FusedCombine fc;
  // Dense tiles (few tokens, experts that are nearly all routed to): gate/up
  // tile e is expert e with all T tokens in token order, h rows e*T .. e*T+T-1,
  // so it needs no routing (and raises no bad-slot flag: only experts with
  // routed rows may, in the down GEMM); the down GEMM runs the routed tiles
  // and reads the row of grouped position p at e*T + (token of p).
  int dense, T;
  const int32_t* slot_table;  // [E] dense gate/up tiles: the slot of expert e
  int num_experts;            // E (routed and shared)
  uint32_t* tmask;            // [E] dense plans: the router's token masks (control words)
};

// The down kernel's partial outputs: read by its own last blocks (fused
// combine: coherent stores, the readers are other blocks of this kernel) or
// by the next kernel (plain stores: the kernel boundary orders them).
__device__ __forceinline__ void store_y(const StreamArgs& a, float* p, float v) {
  if (a.fc.tickets)
    store_coherent(p, v);
  else
    *p = v;
}

// Fused combine: the last block to finish a column slice (an atomic ticket
// per slice) gathers that slice of out[] for every token: per token the k
// routed rows in order j = 0..k-1, each the fixed-order sum of its k-splits.
template <int COLS>
__device__ void fused_combine_tail(const StreamArgs& a, int bx, int ntiles, int nsplit) {
  __shared__ int is_last;
  if (!last_block_ticket(&a.fc.tickets[bx], (uint32_t)(ntiles * nsplit), &is_last)) return;
  const int n0 = bx * COLS;
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
  if (threadIdx.x == 0) reset_ticket(&a.fc.tickets[bx]);
}

// GATEUP: h rows of one tile, silu(x Wg^T) * (x Wu^T) in bf16, columns of
// every group of 8 in the fragment k-order (h_phys_col).
// !GATEUP: ypart[split][p] = h[p] Wd^T over the k range of `split`, fp32,
// written with coherent stores; with a FusedCombine, the last block of each
// column slice also writes that slice of out[].
#ifndef MOE_STREAM_WPE
#define MOE_STREAM_WPE 4
#endif
// RG row groups of 16 per tile (tiles of up to 16 RG rows of one expert): a
// widened weight fragment then feeds RG matrix-core products, so an expert's
// weights are streamed once for up to 16 RG of its rows.
//
// BITS: int4 codes (two per byte, widened with codes_to_bf16) or 8-bit codes
// (bytes_to_bf16); a stage is 128 bytes of every weight row either way (256
// or 128 k).  GROUPED: one (s, z) per output row and group of 128 k, in
// [K/128][N] arrays.  A wave's k part of a stage then lies in one group, so
// the wave multiplies it into accumulators of its own, turns them into
// s (acc - (bias + z) sum_k a) with that group's (s, z) and adds that to its
// running sums; the (s, z) of a stage's groups are copied into LDS beside
// its weights (one more 1 KB copy per stage).  Per-row formats apply (s, z)
// once, in the epilogue.
// The stage ring, and for dense gate/up tiles two words per wave after it
// that receive the router's token mask.
template <bool GATEUP, int NCW, int NBUF, int BITS, bool GROUPED, bool DENSE = false>
constexpr int stream_smem_bytes() {
  return NBUF * ((GATEUP ? 2 : 1) * 64 * NCW * kWRowBytes + (GROUPED ? kPBytes : 0)) + (DENSE ? 4 * 8 : 0);
}

// One block: column slice bx, row tile by, k-split bz of nz; smem holds
// stream_smem_bytes<...>() bytes, 1 KB aligned.  DENSE: a gate/up block of
// dense tiles (tile by is expert by with all T tokens).
template <bool GATEUP, int NCW, int NBUF, int KW, bool NT, int RG, int BITS, bool GROUPED, bool DENSE = false>
__device__ __forceinline__ void stream_gemm_body(const StreamArgs& a, int bx, int by, int bz, int nz, char* smem) {
  static_assert(NBUF == 2 || NBUF == 3, "stage ring of 2 or 3 buffers");
  static_assert(KW == 2 || KW == 4, "k split over 2 or 4 waves");
  static_assert(RG == 1 || RG == 2, "tiles of 16 or 32 rows");
  static_assert(BITS == 4 || BITS == 8, "int4 or 8-bit codes");
  static_assert(!GROUPED || NCW == 1, "grouped formats run 64-column blocks");
  constexpr int SK = kWRowBytes * 8 / BITS;             // k per stage
  constexpr int COLS = 64 * NCW;                        // output columns per block
  constexpr int NWR = (GATEUP ? 2 : 1) * COLS;          // weight rows per stage
  constexpr int WBYTES = NWR * kWRowBytes;              // weights of one stage
  constexpr int PBYTES = GROUPED ? kPBytes : 0;         // (s, z) of one stage
  constexpr int SBYTES = WBYTES + PBYTES;               // one stage buffer
  constexpr int WI = NWR / kRowsPerWInst / 4;           // weight-load instructions per wave per stage
  constexpr int CW = 4 / KW;                            // column parts
  constexpr int CT = COLS / 16 / CW;                    // 16-column tiles per wave and weight matrix
  constexpr int NB = (GATEUP ? 2 : 1) * CT;             // B fragments per wave per stage
  constexpr int KR = SK / KW;                           // k per wave per stage
  constexpr int KS = KR / 32;                           // MFMA k-steps per wave per stage (16 B of A each)
  constexpr int WPS = BITS / 4;                         // 32-bit code words per lane and k-step
  constexpr int LB = KS * WPS * 4;                      // code bytes per lane and weight row per stage
  constexpr float kBias = code_bias<BITS>();
  static_assert(KS >= 1 && (LB == 8 || LB == 16), "lane slices of 8 or 16 code bytes");
  static_assert(!GROUPED || (kQGroup % KR == 0 && SK <= 2 * kQGroup), "a wave's k part lies in one group");
  static_assert(!GROUPED || 4 * 2 * COLS * 2 == kPBytes, "4 arrays x 2 groups x 64 columns of fp16 per stage");
  static_assert(WI * kRowsPerWInst * 4 == NWR, "even split over waves");
  static_assert(NBUF * SBYTES == stream_smem_bytes<GATEUP, NCW, NBUF, BITS, GROUPED>(), "stage ring size");
  char* const mask_slots = smem + NBUF * SBYTES + 8 * (threadIdx.x >> 6);  // dense tiles: this wave's polls

  constexpr bool dense_tile = GATEUP && DENSE;
  static_assert(!dense_tile || RG == 1, "dense tiles hold at most 16 tokens");
  const int ntiles = dense_tile ? a.max_tiles : *a.num_tiles;
  const int tile = by;
  if (tile >= ntiles) return;
  // dense plans: the down GEMM's first block returns the router's token
  // masks to zero for the next call (every gate/up block has finished)
  if (!GATEUP && a.dense && bx == 0 && tile == 0 && bz == 0)
    for (int x = threadIdx.x; x < a.num_experts; x += 256) reset_ticket(&a.tmask[x]);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, grp = lane >> 4;
  const int kp = wave % KW, cp = wave / KW;
  const int n0 = bx * COLS;
  // (expert, slot, first grouped row, rows <= 16 RG); dense gate/up: expert `tile`, all tokens
  const int4 td = dense_tile ? make_int4(tile, a.slot_table[tile], tile * a.T, a.T) : a.tiles[tile];
  const int slot = td.y, pbase = td.z, rows = td.w;
  const int ncols_total = GATEUP ? a.dff : a.d;
  const int K = GATEUP ? a.d : a.kchunk;
  const int kbeg = GATEUP ? 0 : bz * a.kchunk;
  const size_t row_bytes = (size_t)(GATEUP ? a.d : a.dff) * BITS / 8;
  const bool bad = slot < 0 || slot >= a.num_slots;
  float* yrow = GATEUP ? nullptr : a.ypart + ((size_t)bz * a.R + pbase) * a.d;

  if (bad) {
    if (threadIdx.x == 0 && !dense_tile) atomicOr(a.flags, MOE_FLAG_BAD_SLOT);
    if (GATEUP) return;
    for (int i = threadIdx.x; i < rows * COLS; i += 256) store_y(a, &yrow[(size_t)(i / COLS) * a.d + n0 + i % COLS], 0.0f);
  } else {
    // this lane's activation rows (row lr + 16 g of the tile) and k offset in
    // every stage: KR kp + (KR / 4) grp, KS x 8 values
    const int ka = KR * kp + (KR / 4) * grp;
    const uint16_t* asrc[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int mm = lr + 16 * g < rows ? lr + 16 * g : 0;
      const int tok = dense_tile ? mm : a.perm[pbase + mm] / a.topk;  // the token of tile row mm
      const int hrow = a.dense ? td.x * a.T + tok : pbase + mm;       // down: its row of h
      asrc[g] = GATEUP ? a.act + (size_t)tok * a.d + ka : a.act + (size_t)hrow * a.dff + kbeg + ka;
    }
    const uint8_t* wsrc[WI];
#pragma unroll
    for (int j = 0; j < WI; ++j) {
      const int r = (wave * WI + j) * kRowsPerWInst + lane / 8;  // block weight row
      const uint8_t* base = (!GATEUP || r < COLS) ? a.w0 : a.w1;
      const int n = n0 + (r % COLS);
      wsrc[j] = base + ((size_t)slot * ncols_total + n) * row_bytes + (size_t)kbeg * BITS / 8 +
                16 * wchunk_pos(r, lane % 8);
    }
    // grouped: wave w copies 256 bytes of every stage's (s, z) -- array w
    // (gate/up: s_gate, z_gate, s_up, z_up; down: s, z, s, z), the block's 64
    // columns of the stage's groups 0 and 1 (lane / 32), 2 columns per lane;
    // in LDS: [array][group of the stage][column]
    const int ngroups = (GATEUP ? a.d : a.dff) / kQGroup;
    const uint8_t* psrc = nullptr;
    if constexpr (GROUPED) {
      const bool up = GATEUP && wave >= 2;
      const uint16_t* arr = (wave & 1) ? (up ? a.z1 : a.z0) : (up ? a.s1 : a.s0);
      psrc = reinterpret_cast<const uint8_t*>(arr + (size_t)slot * ngroups * ncols_total + n0 + 2 * (lane % 32));
    }
    const int nst = (K + SK - 1) / SK;
    const bool half_last = (K % SK) != 0;  // the last stage has only its lower half of k
    const bool idle_half = KR * kp >= SK / 2;  // this wave has no k in a half stage
    // The copies are issued without per-lane conditions, so that the
    // compiler's own wait for the activation registers is exact: a half
    // stage copies its upper 4 chunks from the lower ones (into LDS nobody
    // reads), and lanes of rows past the tile's end load row 0 (their
    // registers only reach output rows that are never stored).  A stage's
    // second group past the matrix's last re-reads the last (unused).
    auto issue_w = [&](int st) {
      char* buf = smem + (st % NBUF) * SBYTES;
      const bool half = half_last && st == nst - 1;
#pragma unroll
      for (int j = 0; j < WI; ++j) {
        const int r = (wave * WI + j) * kRowsPerWInst + lane / 8;
        const int back = (half && wchunk_pos(r, lane % 8) >= 4) ? 64 : 0;
        load_lds16<NT>(wsrc[j] + (size_t)st * kWRowBytes - back, buf + (wave * WI + j) * 1024);
      }
      if constexpr (GROUPED) {
        const int gi = min((kbeg + st * SK) / kQGroup + lane / 32, ngroups - 1);
        load_lds4(psrc + (size_t)gi * ncols_total * 2, buf + WBYTES + wave * 256);
      }
    };
    auto load_a = [&](int st, u32x4 (&av)[RG][KS]) {
      const int sa = (half_last && st == nst - 1 && idle_half) ? 0 : st;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const u32x4* src = reinterpret_cast<const u32x4*>(asrc[g] + (size_t)sa * SK);
#pragma unroll
        for (int j = 0; j < KS; ++j) av[g][j] = src[j];
      }
    };

    f32x4 acc[RG][NB], accs[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      accs[g] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < NB; ++t) acc[g][t] = f32x4{0, 0, 0, 0};
    }
    const u32x4 ones = ones_bf16();
    // this lane's bytes of every weight row: LB bytes at (KR BITS / 8) kp + LB grp
    const int boff = (KR * BITS / 8) * kp + LB * grp;
    const int pgrp = GROUPED ? (KR * kp) / kQGroup : 0;  // group of this wave's k part inside a stage
    auto compute = [&](int st, const u32x4 (&acur)[RG][KS]) {
      if (half_last && st == nst - 1 && idle_half) return;
      const char* buf = smem + (st % NBUF) * SBYTES;
      uint32_t bw[NB][LB / 4];
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const int r = (t >= CT ? COLS : 0) + 16 * (CT * cp + t % CT) + lr;
        const char* p = buf + r * kWRowBytes + 16 * wchunk_pos(r, boff / 16) + boff % 16;
        if constexpr (LB == 16) {
          const u32x4 v = lds_read16(p);
          bw[t][0] = v.x; bw[t][1] = v.y; bw[t][2] = v.z; bw[t][3] = v.w;
        } else {
          const u32x2 v = lds_read8(p);
          bw[t][0] = v.x; bw[t][1] = v.y;
        }
      }
      uint32_t ps[GROUPED ? NB : 1], pz[GROUPED ? NB : 1];
      if constexpr (GROUPED) {
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const int q = (t >= CT ? 2 : 0);  // s of gate (or down) / up; z follows
          const int nl = 16 * (CT * cp + t % CT) + lr;
          ps[t] = lds_read_u16(buf + WBYTES + ((q * 2 + pgrp) * 64 + nl) * 2);
          pz[t] = lds_read_u16(buf + WBYTES + (((q + 1) * 2 + pgrp) * 64 + nl) * 2);
        }
      }
      lds_wait();
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int j = 0; j < LB / 4; ++j) lds_ready(bw[t][j]);
      if constexpr (GROUPED) {
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          lds_ready(ps[t]);
          lds_ready(pz[t]);
        }
      }
      u32x4 x[RG][KS];
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int j = 0; j < KS; ++j) x[g][j] = GATEUP ? permute_a(acur[g][j]) : acur[g][j];  // h is in fragment order
      auto widen = [&](int t, int j) {
        if constexpr (BITS == 4)
          return codes_to_bf16(bw[t][j]);
        else
          return bytes_to_bf16(bw[t][2 * j], bw[t][2 * j + 1]);
      };
      if constexpr (!GROUPED) {
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
          for (int j = 0; j < KS; ++j) accs[g] = mfma16(x[g][j], ones, accs[g]);
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
          for (int j = 0; j < KS; ++j) {
            const u32x4 b = widen(t, j);
#pragma unroll
            for (int g = 0; g < RG; ++g) acc[g][t] = mfma16(x[g][j], b, acc[g][t]);
          }
      } else {
        // this stage's products and row sums, then s (acc - (bias + z) sum a)
        f32x4 sacc[RG][NB], ssum[RG];
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          ssum[g] = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < KS; ++j) ssum[g] = mfma16(x[g][j], ones, ssum[g]);
#pragma unroll
          for (int t = 0; t < NB; ++t) sacc[g][t] = f32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
          for (int j = 0; j < KS; ++j) {
            const u32x4 b = widen(t, j);
#pragma unroll
            for (int g = 0; g < RG; ++g) sacc[g][t] = mfma16(x[g][j], b, sacc[g][t]);
          }
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const float sg = fp16_to_f32((uint16_t)ps[t]), cg = kBias + fp16_to_f32((uint16_t)pz[t]);
#pragma unroll
          for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[g][t][i] += sg * (sacc[g][t][i] - cg * ssum[g][i]);
        }
      }
    };

    // Issue order: A(0), W(0) .. W(NBUF - 2); then at stage s, A(s + 1) and
    // W(s + NBUF - 1) (each W with its (s, z) copy for the grouped formats).
    // At stage s the copies younger than W(s) are at least A(s + 1) and
    // W(s + 1) (NBUF = 2), or W(s + 1), A(s + 1) and W(s + 2) (NBUF = 3), so
    // waiting until that many are pending completes W(s).  The last NBUF - 1
    // stages issue no weight copies and wait for all.
    constexpr int kPending = (NBUF - 1) * (WI + (GROUPED ? 1 : 0)) + RG * KS;
    // The activation fragments of stage st + 1 are loaded one stage ahead.
    // Dense tiles use two register sets in turn (a loop unrolled twice): there,
    // copying a prefetched set into a working one at the top of each stage
    // made the compiler wait for every load in flight, the poll and the next
    // stage's weight copies included.
    u32x4 aset0[RG][KS], aset1[RG][KS];
    // Dense tiles: until the router publishes the expert's token mask, tile
    // row r is token r for every r; once a wave sees the mask it loads only
    // the routed tokens' rows (the other lanes repeat the first routed row, so
    // their loads coalesce), which cuts the activation traffic.  Row r stays
    // token r, so a routed token's products are whole whenever the switch
    // happens; the other rows' h is never read.  Stage st's poll is a coherent
    // direct-to-LDS load by lane 0 into this wave's slot st % 2, issued after
    // the stage's copies; the copy wait of stage st lets it stay in flight and
    // that of stage st + 1 completes it, so no register ever waits on it.  The
    // poll before the loop (slot 1) gives the first stage a value.  Every
    // stage polls, so that every stage leaves the same number of loads in
    // flight (a branch around the poll made the compiler wait for all of them).
    uint32_t known = 0;
    auto poll = [&](int st) {
      if constexpr (dense_tile)
        if (lane == 0) load_lds4_coherent(a.tmask + td.x, mask_slots + 4 * (st & 1));
    };
    // Reads wave 0's poll of the given slot (after a barrier that wave 0
    // passed once its poll had landed, so every wave reads the same value) and
    // switches to the routed rows once the mask is known.
    char* const wave0_slots = smem + NBUF * SBYTES;
    auto take_mask = [&](int slot) {
      uint32_t polled = lds_read_b32(wave0_slots + 4 * slot);
      lds_wait();
      lds_ready(polled);
      if (!(known & kMaskKnown) && (polled & kMaskKnown)) {  // block-uniform
        known = polled;
        const uint32_t m = known & 0xFFFFu;
        const int row = ((m >> lr) & 1u) ? lr : (m ? __builtin_ctz(m) : 0);
        asrc[0] = a.act + (size_t)row * a.d + KR * kp + (KR / 4) * grp;
      }
    };
    load_a(0, aset0);
    issue_w(0);
    if (NBUF == 3 && nst > 1) issue_w(1);
    poll(-1);
    // stage st of the main loop: its fragments are in `use`, stage st + 1's go
    // to `fill`.  (A block of an expert left without rows runs to the end:
    // leaving the loop early cost the main loop registers.)
    auto main_stage = [&](int st, const u32x4 (&use)[RG][KS], u32x4 (&fill)[RG][KS]) {
      load_a(st + 1, fill);
      issue_w(st + NBUF - 1);
      poll(st);
      wait_vmem<kPending + (dense_tile ? 1 : 0)>();
      lds_barrier();
      if constexpr (dense_tile) take_mask((st + 1) & 1);  // the previous poll
      compute(st, use);
      lds_barrier();
    };
    const int nmain = max(0, nst - (NBUF - 1));
    if constexpr (dense_tile) {
      int st = 0;
      for (; st + 1 < nmain; st += 2) {
        main_stage(st, aset0, aset1);
        main_stage(st + 1, aset1, aset0);
      }
      if (st < nmain) {
        main_stage(st, aset0, aset1);
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
          for (int j = 0; j < KS; ++j) aset0[g][j] = aset1[g][j];
      }
    } else {
      // (one set copied into the other per stage: the compiler waits for the
      // copied loads without holding back the weight copies here, and this
      // form measured slightly faster than the unrolled one)
      for (int st = 0; st < nmain; ++st) {
        u32x4 acur[RG][KS];
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
          for (int j = 0; j < KS; ++j) acur[g][j] = aset0[g][j];
        main_stage(st, acur, aset0);
      }
    }
    // per-row formats: scale and code offset (bias + z) of this wave's
    // columns, loaded while the last stages land (grouped: already applied)
    const size_t sbase = (size_t)slot * ncols_total + n0;
    float sc[NB], cc[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int nl = 16 * (CT * cp + t % CT) + lr;  // column inside the block
      const bool up = GATEUP && t >= CT;
      sc[t] = GROUPED ? 1.0f : fp16_to_f32((up ? a.s1 : a.s0)[sbase + nl]);
      cc[t] = GROUPED ? 0.0f : kBias + fp16_to_f32((up ? a.z1 : a.z0)[sbase + nl]);
    }
    for (int st = nmain; st < nst; ++st) {
      // the last stages: no weight copies left to keep in flight
      u32x4 acur[RG][KS];
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int j = 0; j < KS; ++j) acur[g][j] = aset0[g][j];
      if (st + 1 < nst) load_a(st + 1, aset0);
      wait_vmem<0>();
      lds_barrier();
      compute(st, acur);
      lds_barrier();
    }

    // Every wave turns its k part into s (acc - (bias + z) sum_k a) -- linear
    // in the k parts -- and hands it over through LDS (the ring is free, one
    // row group at a time); the KW waves of a column part then add the k
    // parts in fixed order, each for the column tiles it owns (local tile tl
    // with tl % KW == kp).
    float* part = reinterpret_cast<float*>(smem);  // [wave][tile][4][64]
    static_assert(4 * NB * 4 * 64 * 4 <= NBUF * SBYTES, "the k-part hand-over fits the stage ring");
    uint16_t* hrow = GATEUP ? a.h + (size_t)pbase * a.dff + n0 : nullptr;
    float* ybase = GATEUP ? nullptr : yrow + n0;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      if (16 * g >= rows) break;  // block-uniform
      if (g > 0) __syncthreads();  // the previous group's hand-over is read
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          part[((wave * NB + t) * 4 + i) * 64 + lane] = sc[t] * (acc[g][t][i] - cc[t] * accs[g][i]);
      __syncthreads();
      for (int tl = kp; tl < CT; tl += KW) {
        const int nl = 16 * (CT * cp + tl) + lr;
        float v0[4] = {0, 0, 0, 0}, v1[4] = {0, 0, 0, 0};
        for (int q = 0; q < KW; ++q) {
          const int wq = cp * KW + q;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v0[i] += part[((wq * NB + tl) * 4 + i) * 64 + lane];
            if (GATEUP) v1[i] += part[((wq * NB + CT + tl) * 4 + i) * 64 + lane];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * g + grp * 4 + i;
          if (row < rows) {
            if (GATEUP)
              hrow[(uint32_t)(row * a.dff + h_phys_col(nl))] = f32_to_bf16(silu(v0[i]) * v1[i]);
            else
              store_y(a, &ybase[(uint32_t)(row * a.d + nl)], v0[i]);
          }
        }
      }
    }
  }

  if (GATEUP || a.fc.tickets == nullptr) return;
  fused_combine_tail<COLS>(a, bx, ntiles, nz);
}

#ifndef MOE_STREAM_WPE_DN1
#define MOE_STREAM_WPE_DN1 7  // 16-row down tiles: 7 blocks per CU (72 VGPRs)
#endif
#ifndef MOE_STREAM_WPE_DN2
#define MOE_STREAM_WPE_DN2 3
#endif
template <bool GATEUP, int NCW, int NBUF, int KW, bool NT, int RG, int BITS, bool GROUPED>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(GROUPED ? (RG == 1 ? 3 : 2)
                                           : (GATEUP ? (RG == 1 ? MOE_STREAM_WPE : 3)
                                                     : (RG == 1 ? MOE_STREAM_WPE_DN1 : MOE_STREAM_WPE_DN2)))))
void stream_gemm_kernel(StreamArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[stream_smem_bytes<GATEUP, NCW, NBUF, BITS, GROUPED>()];
  stream_gemm_body<GATEUP, NCW, NBUF, KW, NT, RG, BITS, GROUPED>(a, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.z,
                                                                  smem);
}

// The router beside the gate/up GEMM of dense tiles (few tokens, nearly every
// expert routed to): with dense tiles the gate/up GEMM does not depend on the
// routing, so both run in one launch and the router's latency hides behind
// the weight stream.  Blocks 0 .. nrouter-1 are the router's (expert
// b % E, k-split b / E, all T <= 16 tokens); the rest are gate/up blocks in the
// order of the stand-alone kernel's grid (column slice fastest).  Neither
// waits for the other; the down GEMM, the next launch, reads the routing.
constexpr int kDenseRouterLogits = 1024;  // T x E logits the router's finish stages in LDS
template <int NCW, int NBUF, int KW, bool NT, int BITS, bool GROUPED>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(GROUPED ? 3 : (NCW == 2 ? 2 : MOE_STREAM_WPE))))
void stream_gemm_router_kernel(StreamArgs a, RouterSmallArgs r, int nrouter) {
  constexpr int kGemm = stream_smem_bytes<true, NCW, NBUF, BITS, GROUPED, true>();
  constexpr int kRouter = router_small_lds_bytes<kDenseRouterLogits, kRouterTokTile>();
  __shared__ __attribute__((aligned(1024))) char smem[kGemm > kRouter ? kGemm : kRouter];
  const int b = blockIdx.x;
  if (b < nrouter) {
    router_small_body<kDenseRouterLogits, kRouterTokTile, 8, false>(r, b % r.E, 0, b / r.E, nrouter, smem);
    return;
  }
  const int g = b - nrouter, ncb = a.dff / (64 * NCW);
  stream_gemm_body<true, NCW, NBUF, KW, NT, 1, BITS, GROUPED, true>(a, g % ncb, g / ncb, 0, 1, smem);
}

namespace {
#ifndef MOE_STREAM_NBUF
#define MOE_STREAM_NBUF 2
#endif
#ifndef MOE_STREAM_KW_GU
#define MOE_STREAM_KW_GU 4
#endif
#ifndef MOE_STREAM_KW_DN
#define MOE_STREAM_KW_DN 4
#endif
#ifndef MOE_DENSE_NCW
#define MOE_DENSE_NCW 1
#endif
// Weights are streamed with the nt hint: most lines are read once per launch,
// and early eviction keeps the activations and the router's inputs (read
// again by the next layer step) in the caches.  Measured to help every
// decode shape, multi-tile experts included.
template <bool GATEUP, int NCW, int BITS, bool GROUPED>
void launch_stream(const moe_config& c, const Plan& p, const StreamArgs& args, hipStream_t s) {
  const int ncols = GATEUP ? c.d_ff : c.d_model;
  dim3 grid(ncols / (64 * NCW), p.max_tiles, GATEUP ? 1 : p.down_split);
  constexpr int KW = GATEUP ? MOE_STREAM_KW_GU : MOE_STREAM_KW_DN;
  if (p.tile_rows == 2 * kStreamTileRows)
    stream_gemm_kernel<GATEUP, NCW, MOE_STREAM_NBUF, KW, true, 2, BITS, GROUPED><<<grid, 256, 0, s>>>(args);
  else
    stream_gemm_kernel<GATEUP, NCW, MOE_STREAM_NBUF, KW, true, 1, BITS, GROUPED><<<grid, 256, 0, s>>>(args);
}

// The weight format picks the kernel; the grouped formats run 64-column blocks.
template <bool GATEUP>
void launch_stream_format(const moe_config& c, const Plan& p, const StreamArgs& a, int ncw, hipStream_t s) {
  const bool grouped = c.group_size != 0;
  if (c.weight_bits == 8) {
    if (grouped)
      launch_stream<GATEUP, 1, 8, true>(c, p, a, s);
    else if (ncw == 2)
      launch_stream<GATEUP, 2, 8, false>(c, p, a, s);
    else
      launch_stream<GATEUP, 1, 8, false>(c, p, a, s);
  } else {
    if (grouped)
      launch_stream<GATEUP, 1, 4, true>(c, p, a, s);
    else if (ncw == 2)
      launch_stream<GATEUP, 2, 4, false>(c, p, a, s);
    else
      launch_stream<GATEUP, 1, 4, false>(c, p, a, s);
  }
}
}  // namespace

// Fields of the arguments both GEMMs share.
void stream_common_args(const moe_config& c, const Plan& p, const int32_t* slot_table, char* ws, StreamArgs* a) {
  a->tiles = reinterpret_cast<const int4*>(ws + p.tiles);
  a->num_tiles = reinterpret_cast<const int32_t*>(ws + p.num_tiles);
  a->num_slots = c.num_slots;
  a->d = c.d_model;
  a->dff = c.d_ff;
  a->topk = c.top_k;
  a->R = p.R;  // rows of the down output
  a->max_tiles = p.max_tiles;
  a->flags = reinterpret_cast<uint32_t*>(ws + p.flags);
  a->dense = p.dense ? 1 : 0;
  a->T = p.T;
  a->slot_table = slot_table;
  a->perm = reinterpret_cast<const int32_t*>(ws + p.perm);
  a->num_experts = c.num_experts;
  a->tmask = reinterpret_cast<uint32_t*>(ws + p.ctrl + p.tmask);
}

StreamArgs gateup_stream_args(const moe_config& c, const Plan& p, const uint16_t* hidden, const int32_t* slot_table,
                              const moe_weights& w, char* ws) {
  StreamArgs a{};
  stream_common_args(c, p, slot_table, ws, &a);
  a.act = hidden;
  a.perm = reinterpret_cast<const int32_t*>(ws + p.perm);
  a.w0 = w.w_gate;
  a.w1 = w.w_up;
  a.s0 = w.s_gate;
  a.z0 = w.z_gate;
  a.s1 = w.s_up;
  a.z1 = w.z_up;
  a.h = reinterpret_cast<uint16_t*>(ws + p.h);
  return a;
}

void launch_gateup_stream(const moe_config& c, const Plan& p, const uint16_t* hidden, const int32_t* slot_table,
                          const moe_weights& w, char* ws, hipStream_t s) {
  launch_stream_format<true>(c, p, gateup_stream_args(c, p, hidden, slot_table, w, ws), p.gateup_ncw, s);
}

void launch_gateup_router_stream(const moe_config& c, const Plan& p, const uint16_t* hidden, const float* router_w,
                                 const float* router_bias, const int32_t* slot_table, const moe_weights& w,
                                 char* ws, hipStream_t s) {
  StreamArgs a = gateup_stream_args(c, p, hidden, slot_table, w, ws);
  a.max_tiles = c.num_experts;  // one dense tile per expert
  const RouterSmallArgs r = router_small_args(c, p, hidden, router_w, router_bias, slot_table, ws);
  const int nrouter = r.E * p.small_split;  // T <= 16: one token group
  constexpr int KW = MOE_STREAM_KW_GU;
  constexpr int NCW = MOE_DENSE_NCW;  // per-row formats: blocks of 64 NCW columns
  // the plan runs dense tiles for per-row int4 weights only
  const dim3 grid(nrouter + c.num_experts * (c.d_ff / (64 * NCW)));
  stream_gemm_router_kernel<NCW, MOE_STREAM_NBUF, KW, true, 4, false><<<grid, 256, 0, s>>>(a, r, nrouter);
}

void launch_down_stream(const moe_config& c, const Plan& p, const int32_t* slot_table, const moe_weights& w,
                        uint16_t* out, char* ws, hipStream_t s) {
  StreamArgs a{};
  stream_common_args(c, p, slot_table, ws, &a);
  a.act = reinterpret_cast<const uint16_t*>(ws + p.h);
  a.kchunk = c.d_ff / p.down_split;
  a.w0 = w.w_down;
  a.s0 = w.s_down;
  a.z0 = w.z_down;
  a.ypart = reinterpret_cast<float*>(ws + p.y);
  if (p.fused_combine) {
    a.fc.tickets = reinterpret_cast<uint32_t*>(ws + p.ctrl) + 1;
    a.fc.inv = reinterpret_cast<const int32_t*>(ws + p.inv);
    a.fc.topk_w = reinterpret_cast<const float*>(ws + p.topk_w);
    a.fc.out = out;
    a.fc.T = p.T;
    a.fc.k = c.top_k;
  }
  launch_stream_format<false>(c, p, a, p.down_ncw, s);
}

}  // namespace moe
