// Grouped expert GEMMs over int4 weights with the dequantisation fused into
// the weight load.
//
// Strata page, section 3.2: the expert FFN (a two-layer MLP) is the most
// expensive part of the layer; the tokens routed to one expert are
// concatenated and the active experts' products run as one group GEMM
// instead of many small ones.  Section 3.1: weights are per-expert int4 with
// their own scale and zero-point, dequantised on the load path rather than by
// a kernel of their own.  Here the int4 codes stay packed in HBM, each lane
// widens one 32-bit word of codes into an MFMA B fragment in registers, and
// the scale and zero-point are applied per output in the epilogue (see
// codes_to_bf16).
//
// Work unit: one wave = one row tile of one expert (up to kTileRows rows of
// its group, as 16-row MFMA blocks) x 16*NB output columns, streaming the
// whole k range of its weight rows once.  Row sums of A, needed by the
// zero-point correction, come from one extra MFMA against a B of ones.
// Weights are read through slot = slot_table[e] (the cache slot of the
// Co-inference page, section 2.2); an out-of-range slot raises
// MOE_FLAG_BAD_SLOT and the expert contributes zero.
#include "device_common.h"
#include "plan.h"

namespace moe {

constexpr int kMaxMB = kTileRows / 16;

// h[p] = silu(x Wg^T) * (x Wu^T) for the rows p of one tile, stored as bf16
// with the columns of every group of 8 in the fragment k-order (h_phys_col).
template <int NB>
__global__ __launch_bounds__(256) void gateup_swiglu_kernel(
    const uint16_t* __restrict__ hidden, int d, int dff, int topk, const int32_t* __restrict__ perm,
    const int4* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int num_slots,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, const uint16_t* __restrict__ sg,
    const uint16_t* __restrict__ zg, const uint16_t* __restrict__ su, const uint16_t* __restrict__ zu,
    uint16_t* __restrict__ h, uint32_t* __restrict__ flags) {
  const int tile = blockIdx.y;
  if (tile >= *num_tiles) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, grp = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * (16 * NB);
  const int4 td = tiles[tile];  // (expert, slot, first grouped row, rows)
  const int slot = td.y, pbase = td.z, rows = td.w;
  if (slot < 0 || slot >= num_slots) {
    if (threadIdx.x == 0) atomicOr(flags, MOE_FLAG_BAD_SLOT);
    return;
  }
  const int nmb = (rows + 15) >> 4;

  const uint16_t* arow[kMaxMB];
  bool aval[kMaxMB];
#pragma unroll
  for (int mb = 0; mb < kMaxMB; ++mb) {
    const int rr = mb * 16 + lr;
    aval[mb] = rr < rows;
    const int tok = aval[mb] ? perm[pbase + rr] / topk : 0;
    arow[mb] = hidden + (size_t)tok * d + grp * 32;
  }
  const size_t half_d = (size_t)d / 2;
  const uint8_t* bg[NB];
  const uint8_t* bu[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const size_t row = (size_t)slot * dff + n0 + nb * 16 + lr;
    bg[nb] = wg + row * half_d + grp * 16;
    bu[nb] = wu + row * half_d + grp * 16;
  }

  f32x4 accg[kMaxMB][NB], accu[kMaxMB][NB], accs[kMaxMB];
#pragma unroll
  for (int mb = 0; mb < kMaxMB; ++mb) {
    accs[mb] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) accg[mb][nb] = accu[mb][nb] = f32x4{0, 0, 0, 0};
  }
  const u32x4 ones = ones_bf16();
  const u32x4 zero4 = u32x4{0, 0, 0, 0};

  for (int kb = 0; kb < d; kb += kGemmKStep) {
    u32x4 qg[NB], qu[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      qg[nb] = *reinterpret_cast<const u32x4*>(bg[nb] + kb / 2);
      qu[nb] = *reinterpret_cast<const u32x4*>(bu[nb] + kb / 2);
    }
    u32x4 a[kMaxMB][4];
#pragma unroll
    for (int mb = 0; mb < kMaxMB; ++mb) {
      if (mb < nmb) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          a[mb][s] = aval[mb] ? *reinterpret_cast<const u32x4*>(arow[mb] + kb + s * 8) : zero4;
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 ap[kMaxMB];
#pragma unroll
      for (int mb = 0; mb < kMaxMB; ++mb)
        if (mb < nmb) ap[mb] = permute_a(a[mb][s]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 b_g = codes_to_bf16(qg[nb][s]);
        const u32x4 b_u = codes_to_bf16(qu[nb][s]);
#pragma unroll
        for (int mb = 0; mb < kMaxMB; ++mb) {
          if (mb < nmb) {
            accg[mb][nb] = mfma16(ap[mb], b_g, accg[mb][nb]);
            accu[mb][nb] = mfma16(ap[mb], b_u, accu[mb][nb]);
          }
        }
      }
#pragma unroll
      for (int mb = 0; mb < kMaxMB; ++mb)
        if (mb < nmb) accs[mb] = mfma16(ap[mb], ones, accs[mb]);
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n0 + nb * 16 + lr;
    const size_t sidx = (size_t)slot * dff + n;
    const float s_g = fp16_to_f32(sg[sidx]), c_g = kCodeBias + fp16_to_f32(zg[sidx]);
    const float s_u = fp16_to_f32(su[sidx]), c_u = kCodeBias + fp16_to_f32(zu[sidx]);
    const int hcol = h_phys_col(n);
#pragma unroll
    for (int mb = 0; mb < kMaxMB; ++mb) {
      if (mb < nmb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mb * 16 + grp * 4 + i;
          if (row < rows) {
            const float sx = accs[mb][i];
            const float g = s_g * (accg[mb][nb][i] - c_g * sx);
            const float u = s_u * (accu[mb][nb][i] - c_u * sx);
            h[(size_t)(pbase + row) * dff + hcol] = f32_to_bf16(silu(g) * u);
          }
        }
      }
    }
  }
}

// ypart[split][p] = h[p] Wd^T over the k-range of `split` (fp32).
template <int NB>
__global__ __launch_bounds__(256) void down_kernel(
    const uint16_t* __restrict__ h, int d, int dff, int kchunk, int R, const int4* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int num_slots, const uint8_t* __restrict__ wd,
    const uint16_t* __restrict__ sd, const uint16_t* __restrict__ zd, float* __restrict__ ypart,
    uint32_t* __restrict__ flags) {
  const int tile = blockIdx.y;
  if (tile >= *num_tiles) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, grp = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * (16 * NB);
  const int split = blockIdx.z;
  const int kbeg = split * kchunk;
  const int4 td = tiles[tile];  // (expert, slot, first grouped row, rows)
  const int slot = td.y, pbase = td.z, rows = td.w;
  const int nmb = (rows + 15) >> 4;
  float* yrow = ypart + ((size_t)split * R + pbase) * d;

  if (slot < 0 || slot >= num_slots) {
    if (threadIdx.x == 0) atomicOr(flags, MOE_FLAG_BAD_SLOT);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      for (int row = grp * 4; row < rows; row += 16)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (row + i < rows) yrow[(size_t)(row + i) * d + n0 + nb * 16 + lr] = 0.0f;
    return;
  }

  const uint16_t* arow[kMaxMB];
  bool aval[kMaxMB];
#pragma unroll
  for (int mb = 0; mb < kMaxMB; ++mb) {
    const int rr = mb * 16 + lr;
    aval[mb] = rr < rows;
    arow[mb] = h + (size_t)(pbase + (aval[mb] ? rr : 0)) * dff + kbeg + grp * 32;
  }
  const size_t half_k = (size_t)dff / 2;
  const uint8_t* bd[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    bd[nb] = wd + ((size_t)slot * d + n0 + nb * 16 + lr) * half_k + kbeg / 2 + grp * 16;

  f32x4 acc[kMaxMB][NB], accs[kMaxMB];
#pragma unroll
  for (int mb = 0; mb < kMaxMB; ++mb) {
    accs[mb] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0, 0, 0, 0};
  }
  const u32x4 ones = ones_bf16();
  const u32x4 zero4 = u32x4{0, 0, 0, 0};

  for (int kb = 0; kb < kchunk; kb += kGemmKStep) {
    u32x4 q[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) q[nb] = *reinterpret_cast<const u32x4*>(bd[nb] + kb / 2);
    u32x4 a[kMaxMB][4];
#pragma unroll
    for (int mb = 0; mb < kMaxMB; ++mb) {
      if (mb < nmb) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          a[mb][s] = aval[mb] ? *reinterpret_cast<const u32x4*>(arow[mb] + kb + s * 8) : zero4;
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 b = codes_to_bf16(q[nb][s]);
#pragma unroll
        for (int mb = 0; mb < kMaxMB; ++mb)
          if (mb < nmb) acc[mb][nb] = mfma16(a[mb][s], b, acc[mb][nb]);
      }
#pragma unroll
      for (int mb = 0; mb < kMaxMB; ++mb)
        if (mb < nmb) accs[mb] = mfma16(a[mb][s], ones, accs[mb]);
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n0 + nb * 16 + lr;
    const size_t sidx = (size_t)slot * d + n;
    const float s_d = fp16_to_f32(sd[sidx]), c_d = kCodeBias + fp16_to_f32(zd[sidx]);
#pragma unroll
    for (int mb = 0; mb < kMaxMB; ++mb) {
      if (mb < nmb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mb * 16 + grp * 4 + i;
          if (row < rows) yrow[(size_t)row * d + n] = s_d * (acc[mb][nb][i] - c_d * accs[mb][i]);
        }
      }
    }
  }
}

namespace {
constexpr int kNB = 2;  // generic family: 4 waves x kNB x 16 = kGemmColsPerBlock columns per block
}  // namespace

void launch_gateup(const moe_config& c, const Plan& p, const uint16_t* hidden, const moe_weights& w, char* ws,
                   hipStream_t s) {
  if (p.family == GemmFamily::kStream) return launch_gateup_stream(c, p, hidden, w, ws, s);
  dim3 grid(c.d_ff / kGemmColsPerBlock, p.max_tiles, 1);
  gateup_swiglu_kernel<kNB><<<grid, 256, 0, s>>>(
      hidden, c.d_model, c.d_ff, c.top_k, reinterpret_cast<const int32_t*>(ws + p.perm),
      reinterpret_cast<const int4*>(ws + p.tiles), reinterpret_cast<const int32_t*>(ws + p.num_tiles),
      c.num_slots, w.w_gate, w.w_up,
      w.s_gate, w.z_gate, w.s_up, w.z_up, reinterpret_cast<uint16_t*>(ws + p.h),
      reinterpret_cast<uint32_t*>(ws + p.flags));
}

void launch_down(const moe_config& c, const Plan& p, const moe_weights& w, uint16_t* out, char* ws,
                 hipStream_t s) {
  if (p.family == GemmFamily::kStream) return launch_down_stream(c, p, w, out, ws, s);
  dim3 grid(c.d_model / kGemmColsPerBlock, p.max_tiles, p.down_split);
  down_kernel<kNB><<<grid, 256, 0, s>>>(
      reinterpret_cast<const uint16_t*>(ws + p.h), c.d_model, c.d_ff, c.d_ff / p.down_split, p.R,
      reinterpret_cast<const int4*>(ws + p.tiles), reinterpret_cast<const int32_t*>(ws + p.num_tiles),
      c.num_slots, w.w_down, w.s_down,
      w.z_down, reinterpret_cast<float*>(ws + p.y), reinterpret_cast<uint32_t*>(ws + p.flags));
}

}  // namespace moe
