// Expert FFN kernels (gfx950): activation quantization, grouped gate/up and
// down GEMMs on fp8 MFMA with per-K-block scale promotion, SiLU(gate)*up
// with 1x128 requantization, the bf16 shared expert and the fixed-order
// combine.
//
// Sources: routed experts are fp8 e4m3 with block scales and are stored as a
// [gate_proj, up_proj, down_proj] triple (MoE-Infinity PR #140, fp8 store and
// expert-node commits); activations are quantized to e4m3 per 128 columns
// (mstar PR #388, FlashInfer crossover note); the layer runs union -> GEMM ->
// SiLU -> GEMM and sums in a fixed order, writing pad rows as zeros
// (openinfer PR #610, description and "Gates").
//
// One procedure per output element, shared by every kernel here:
//   routed GEMM  K-blocks split into fixed contiguous segments (kSegGU for
//                gate/up, kSegDN for down); per segment acc = 0 and, for
//                K-blocks kb ascending, acc = fma(s_act[kb] * s_w[kb], P_kb,
//                acc) with P_kb one 16x16x128 fp8 MFMA from a zero
//                accumulator; the element is ((seg0 + seg1) + seg2) + ...;
//   shared GEMM  fixed K segments (kSegSG for gate/up, kSegSD for down),
//                each a bf16 16x16x32 MFMA chain from zero, summed in order;
//   combine      acc = fma(w_j, D[slot(r, j)], acc) for j ascending, then
//                + S[r] when the shared expert is present, then bf16 RNE.
// Which tile, wave or kernel computes an element never changes its bits
// (the MFMA result does not depend on the row or column an element occupies).
#include <algorithm>

#include "moe_chains.h"

namespace moe {

// Eight consecutive values of a row as fp32 (bf16: one 16-byte load; fp32:
// two).
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8_f32<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8_f32<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// max over the 16 lanes of a DPP row (every lane of the row gets it)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v))));
  return v;
}

// rows [0, R) of a [R, C] matrix; rows with mask 0 are skipped (never read).
// One wave per (row, group of kQGroup 128-column blocks).  The 16 lanes of a
// DPP row hold one block, 8 values each, so a wave covers 4 blocks per
// step: one 16-byte load (bf16) and one 8-byte store of codes per lane, the
// block maximum from 4 DPP steps.  Each block is quantized as on its own
// (the same rule as quant_pair: s = fl32(amax / 448), codes of v / s, all
// codes 0 for a zero block).
constexpr int kQGroup = 8;
constexpr int kQSteps = kQGroup / 4;

template <typename T>
__global__ __launch_bounds__(256) void k_quant_rows(const T* in, const uint8_t* mask, int R, int C, uint8_t* codes,
                                                    float* scales) {
  const int lane = threadIdx.x & 63, part = lane & 15, sub = lane >> 4;
  const int nb = C / kBlk;
  const int ng = (nb + kQGroup - 1) / kQGroup;
  const long item = (long)blockIdx.x * 4 + wave_id();
  const int r = (int)(item / ng);
  const int b0 = (int)(item % ng) * kQGroup;
  if (r >= R || !row_real(mask, r)) return;
  const T* p = in + (size_t)r * C + part * 8;
  float v[kQSteps][8];
#pragma unroll
  for (int i = 0; i < kQSteps; ++i) {
    const int b = min(b0 + 4 * i + sub, nb - 1);   // past the row's end: reload its last block, not stored
    load8_f32<T>(p + b * kBlk, v[i]);
  }
#pragma unroll
  for (int i = 0; i < kQSteps; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[i][k]));
    const float amax = row16_max(m);
    const float s = quant_scale(amax);
    uint32_t lo = 0, hi = 0;
    if (amax != 0.0f) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo |= quant_code(v[i][k], s) << (8 * k);
        hi |= quant_code(v[i][4 + k], s) << (8 * k);
      }
    }
    const int b = b0 + 4 * i + sub;
    if (b < nb) {
      *reinterpret_cast<uint2*>(codes + (size_t)r * C + b * kBlk + part * 8) = make_uint2(lo, hi);
      if (part == 0) scales[(size_t)r * nb + b] = s;
    }
  }
}

// ---------------------------------------------------------------- plan
// Checks a caller-supplied routing and derives the column-tile schedule.
// A malformed routing -- n_union out of range, offsets not starting at 0 or
// not ascending, union ids not ascending in [0, E), more slots than M*K, an
// expert's rows not strictly ascending, a row outside [0, M) or a pad row --
// schedules no routed work and sets sched[SCHED_BAD] = 1.  (Strictly
// ascending real rows are what the split kernels assume: each of an expert's
// slots is found from its row, so a repeated row would leave a slot unwritten.)
constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void k_plan(FfnArgs a) {
  __shared__ int s_bad, s_nu, s_mt;
  const int tid = threadIdx.x;
  if (tid == 0) {
    int nu = *a.n_union;
    const int max_u = min(a.E, a.M * a.K);
    bool bad = nu < 0 || nu > max_u;
    int mt = 0, prev_e = -1;
    if (!bad) {
      if (a.offs[0] != 0) bad = true;
      for (int u = 0; u < nu && !bad; ++u) {
        const int e = a.union_ids[u];
        const int lo = a.offs[u], hi = a.offs[u + 1];
        if (e <= prev_e || e >= a.E || hi < lo || hi > a.M * a.K) { bad = true; break; }
        prev_e = e;
        a.mtile_offs[u] = mt;
        mt += (hi - lo + kMTile - 1) / kMTile;
      }
    }
    s_bad = bad ? 1 : 0;
    s_nu = bad ? 0 : nu;
    s_mt = mt;
  }
  __syncthreads();
  // rows of every slot: in range, real, strictly ascending inside an expert
  // (the expert of slot s found by a binary search over the checked offsets)
  int bad = s_bad;
  const int nu = s_nu;
  if (!bad && nu > 0) {
    const int slots = a.offs[nu];
    for (int s = tid; s < slots; s += kPlanThreads) {
      const int r = a.rows[s];
      if (r < 0 || r >= a.M || !row_real(a.mask, r)) { bad = 1; break; }
      int lo = 0, hi = nu - 1;              // largest u with offs[u] <= s
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.offs[mid] <= s) lo = mid; else hi = mid - 1;
      }
      if (s > a.offs[lo] && a.rows[s - 1] >= r) { bad = 1; break; }
    }
  }
  bad = __syncthreads_or(bad);
  if (tid != 0) return;
  if (bad) {
    a.sched[SCHED_NUNION] = 0;
    a.sched[SCHED_MTILES] = 0;
    a.sched[SCHED_SLOTS] = 0;
    a.sched[SCHED_BAD] = 1;
    a.mtile_offs[0] = 0;
    return;
  }
  a.mtile_offs[nu] = s_mt;
  a.sched[SCHED_NUNION] = nu;
  a.sched[SCHED_MTILES] = s_mt;
  a.sched[SCHED_SLOTS] = a.offs[nu];
  a.sched[SCHED_BAD] = 0;
}

// ---------------------------------------------------------------- work items
// One wave per work item.  The grid covers the largest item count the call
// can produce (the union is only known on the device); waves past the real
// count exit at once, and the hardware dispatcher balances the rest.
__device__ __forceinline__ int wave_item() { return blockIdx.x * 4 + wave_id(); }

// Gate/up tiles: the 16 MFMA A rows are the 16 rows n0..n0+15 of one packed
// weight group, gate rows or up rows (items alternate: gate, then up of the
// same columns), so each load instruction of the wave reads 1 KB of
// contiguous memory; lane (kq, c) holds columns n = n0 + 4 kq + i of row c.

// ---------------------------------------------------------------- gate/up (split small steps)
// M <= kSmallRows: each item is one K segment of the gate (or the up) rows of
// one 16-column tile of one union expert for one row half (one wave); it
// writes fp32 partials, reduced in segment order by k_post_gateup.  The MFMA
// columns are the half's rows (column c is row 16 h + c; rows not routed to
// the item's expert are computed and dropped); the x
// codes (a few KB per row, L2-resident) stream through the chain's ring with
// the weights.
// Shared expert h_s = bf16(silu(g) u) of row r, columns n, n + 1, from the
// gate/up segment partials summed in order (2 columns per thread).
__device__ __forceinline__ void form_hs(const FfnArgs& a, long idx) {
  const int r = (int)(idx / a.Is), n = (int)(idx % a.Is);
  if (r >= a.M || !row_real(a.mask, r)) return;
  const size_t st = (size_t)a.M * 2 * a.Is;
  const float* pg = a.part_sh + ((size_t)r * 2 + 0) * a.Is + n;
  const float* pu = a.part_sh + ((size_t)r * 2 + 1) * a.Is + n;
  float2 g = *reinterpret_cast<const float2*>(pg);
  float2 u = *reinterpret_cast<const float2*>(pu);
  for (int s = 1; s < kSegSG; ++s) {
    const float2 gs = *reinterpret_cast<const float2*>(pg + s * st);
    const float2 us = *reinterpret_cast<const float2*>(pu + s * st);
    g.x = g.x + gs.x; g.y = g.y + gs.y;
    u.x = u.x + us.x; u.y = u.y + us.y;
  }
  const uint32_t h = (uint32_t)f32_to_bf16(silu_mul(g.x, u.x)) | ((uint32_t)f32_to_bf16(silu_mul(g.y, u.y)) << 16);
  *reinterpret_cast<uint32_t*>(a.hsh + (size_t)r * a.Is + n) = h;
}

// Blocks [0, hs_blocks) form the shared expert's h_s (its gate/up partials
// are complete by now; first in the grid so they do not extend the tail);
// the rest run routed items, one wave each.
// Slot of (row, expert union index u) in the expert's row list (ascending), or -1.
__device__ __forceinline__ int slot_of_row(const FfnArgs& a, int u, int row) {
  const int lo = a.offs[u], hi = a.offs[u + 1];
  int slot = -1;
  for (int s = lo; s < hi; ++s)
    if (a.rows[s] == row) slot = s;
  return slot;
}

// NB = row halves of the step (1: rows 0..15; 2: rows 0..31, both halves in
// one item, sharing each weight fragment).
template <int NB>
__global__ __launch_bounds__(256) void k_gateup_split(FfnArgs a, int hs_blocks) {
  if ((int)blockIdx.x < hs_blocks) {
    form_hs(a, ((long)blockIdx.x * blockDim.x + threadIdx.x) * 2);
    return;
  }
  const int nkb = a.H / kBlk;
  const int ntI = a.I / 8;                 // (16-column tile, gate | up) pairs per expert
  const int n_items = a.sched[SCHED_NUNION] * ntI * kSegGU;
  const int t = ((int)blockIdx.x - hs_blocks) * 4 + wave_id();
  if (t >= n_items) return;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, kq = lane >> 4;
  const int seg = t % kSegGU;
  const int item = t / kSegGU;
  const int u = item / ntI, rem = item % ntI;
  const int gu = rem & 1, n0 = (rem >> 1) * 16;
  const int e = a.union_ids[u];
  const uint8_t* wp = tile_row(gu ? a.wu : a.wg, (size_t)e * a.I + n0 + c, nkb, kq);
  const float* swp = (gu ? a.su : a.sg) + ((size_t)e * (a.I / kBlk) + n0 / kBlk) * nkb;
  const int kb0 = seg_begin(nkb, seg, kSegGU), kb1 = seg_begin(nkb, seg + 1, kSegGU);
  const size_t out = ((size_t)seg * a.M * a.K) * 2;
  const bool col0 = c < a.M && row_real(a.mask, c);
  const int xr0 = col0 ? c : 0;
  if (NB == 1) {
    const v4f p = fp8_chain(wp, swp, a.xq + (size_t)xr0 * a.H + kq * 32, a.xs + (size_t)xr0 * nkb, col0, kb0, kb1);
    if (!col0) return;
    const int slot = slot_of_row(a, u, c);
    if (slot >= 0) store_f4(a.part_gu + (out + (size_t)slot * 2 + gu) * a.I + n0 + 4 * kq, p);
  } else {
    const int r1 = kColRows + c;
    const bool col1 = r1 < a.M && row_real(a.mask, r1);
    const int xr1 = col1 ? r1 : 0;
    v4f p0, p1;
    fp8_chain2(wp, swp, a.xq + (size_t)xr0 * a.H + kq * 32, a.xq + (size_t)xr1 * a.H + kq * 32,
               a.xs + (size_t)xr0 * nkb, a.xs + (size_t)xr1 * nkb, col0, col1, kb0, kb1, p0, p1);
    if (col0) {
      const int slot = slot_of_row(a, u, c);
      if (slot >= 0) store_f4(a.part_gu + (out + (size_t)slot * 2 + gu) * a.I + n0 + 4 * kq, p0);
    }
    if (col1) {
      const int slot = slot_of_row(a, u, r1);
      if (slot >= 0) store_f4(a.part_gu + (out + (size_t)slot * 2 + gu) * a.I + n0 + 4 * kq, p1);
    }
  }
}

// ---------------------------------------------------------------- requantization
// Split steps: routed h per (slot, 128-column block) for the slots in use,
// from the gate/up segment partials summed in order, h = silu(G) U.
// Shared expert down, one K segment of one 16-column tile of H: fp32
// partials for every real row (t < (H / 16) * kSegSD); NB row halves as in
// k_gateup_split.
template <int NB>
__device__ __forceinline__ void shared_down_item(const FfnArgs& a, int t, int lane) {
  const int c = lane & 15, kq = lane >> 4;
  const int seg = t % kSegSD, nt = t / kSegSD;
  const uint8_t* wp = tile_row(a.wsd, (size_t)nt * 16 + c, a.Is * 2 / kBlk, kq);
  const int nst = a.Is / 32;
  const int s0 = seg_begin(nst, seg, kSegSD), s1 = seg_begin(nst, seg + 1, kSegSD);
  const bool v0 = c < a.M && row_real(a.mask, c);
  const uint16_t* bp0 = a.hsh + (size_t)(v0 ? c : 0) * a.Is + kq * 8;
  float* out = a.part_s + (size_t)seg * a.M * a.H + nt * 16 + kq * 4;
  if (NB == 1) {
    const v4f p = bf16_chain(wp, bp0, v0, s0, s1);
    if (v0) store_f4(out + (size_t)c * a.H, p);
  } else {
    const int r1 = kColRows + c;
    const bool v1 = r1 < a.M && row_real(a.mask, r1);
    const uint16_t* bp1 = a.hsh + (size_t)(v1 ? r1 : 0) * a.Is + kq * 8;
    v4f p0, p1;
    bf16_chain2(wp, bp0, bp1, v0, v1, s0, s1, p0, p1);
    if (v0) store_f4(out + (size_t)c * a.H, p0);
    if (v1) store_f4(out + (size_t)r1 * a.H, p1);
  }
}

// Routed h requantization, one wave per (slot, 128-column block).
__global__ __launch_bounds__(256) void k_post_gateup(FfnArgs a) {
  const int lane = threadIdx.x & 63;
  const long item = (long)blockIdx.x * 4 + wave_id();
  const int nbI = a.I / kBlk;
  const int slot = (int)(item / nbI);
  const int b = (int)(item % nbI);
  if (slot >= a.sched[SCHED_SLOTS]) return;
  const int n = b * kBlk + 2 * lane;
  const size_t st = (size_t)a.M * a.K * 2 * a.I;            // segment stride
  const float* pg = a.part_gu + ((size_t)slot * 2 + 0) * a.I + n;
  const float* pu = a.part_gu + ((size_t)slot * 2 + 1) * a.I + n;
  float2 g = *reinterpret_cast<const float2*>(pg);
  float2 u = *reinterpret_cast<const float2*>(pu);
  for (int s = 1; s < kSegGU; ++s) {
    const float2 gs = *reinterpret_cast<const float2*>(pg + s * st);
    const float2 us = *reinterpret_cast<const float2*>(pu + s * st);
    g.x = g.x + gs.x; g.y = g.y + gs.y;
    u.x = u.x + us.x; u.y = u.y + us.y;
  }
  const float h0 = silu_mul(g.x, u.x);
  const float h1 = silu_mul(g.y, u.y);
  quant_pair(h0, h1, a.hq + (size_t)slot * a.I + b * kBlk, a.hs + (size_t)slot * nbI + b, lane);
}

// ---------------------------------------------------------------- down (split small steps)
// Per-segment items: routed D[slot, n] partials for 16 columns of H and one
// half (16 slots) of one union expert's slots (at most kSmallRows in all).
constexpr int kCols = 16;

// NB row halves as in k_gateup_split: an item covers the expert's slots
// 0..15 (and 16..31 when NB = 2).
template <int NB>
__global__ __launch_bounds__(256, 2) void k_down(FfnArgs a, int sd_blocks) {
  const int lane = threadIdx.x & 63;
  if ((int)blockIdx.x < sd_blocks) {
    const int t = (int)blockIdx.x * 4 + wave_id();
    if (t < (a.H / 16) * kSegSD) shared_down_item<NB>(a, t, lane);
    return;
  }
  const int c = lane & 15, kq = lane >> 4;
  const int ntH = a.H / kCols;
  const int total = a.sched[SCHED_MTILES] * ntH * kSegDN;
  const int t = ((int)blockIdx.x - sd_blocks) * 4 + wave_id();
  if (t >= total) return;
  const int seg = t % kSegDN, it = t / kSegDN;
  const Tile tl = routed_tile(a, it / ntH);
  const int nt = it % ntH;
  const int nkb = a.I / kBlk;
  const uint8_t* wp = tile_row(a.wd, (size_t)tl.e * a.H + nt * kCols + c, nkb, kq);
  const float* swp = a.sd + ((size_t)tl.e * (a.H / kBlk) + (nt * kCols) / kBlk) * nkb;
  const int kb0 = seg_begin(nkb, seg, kSegDN), kb1 = seg_begin(nkb, seg + 1, kSegDN);
  float* out = a.part_d + (size_t)seg * a.M * a.K * a.H + nt * kCols + kq * 4;
  const int slot0 = c < tl.mcnt ? tl.s0 + c : -1;
  const uint8_t* bp0 = a.hq + (size_t)(slot0 < 0 ? 0 : slot0) * a.I + kq * 32;
  const float* shp0 = a.hs + (size_t)(slot0 < 0 ? 0 : slot0) * nkb;
  if (NB == 1) {
    const v4f p = fp8_chain(wp, swp, bp0, shp0, slot0 >= 0, kb0, kb1);
    if (slot0 >= 0) store_f4(out + (size_t)slot0 * a.H, p);
  } else {
    const int i1 = kColRows + c;
    const int slot1 = i1 < tl.mcnt ? tl.s0 + i1 : -1;
    const uint8_t* bp1 = a.hq + (size_t)(slot1 < 0 ? 0 : slot1) * a.I + kq * 32;
    const float* shp1 = a.hs + (size_t)(slot1 < 0 ? 0 : slot1) * nkb;
    v4f p0, p1;
    fp8_chain2(wp, swp, bp0, bp1, shp0, shp1, slot0 >= 0, slot1 >= 0, kb0, kb1, p0, p1);
    if (slot0 >= 0) store_f4(out + (size_t)slot0 * a.H, p0);
    if (slot1 >= 0) store_f4(out + (size_t)slot1 * a.H, p1);
  }
}

// ---------------------------------------------------------------- combine
// y[r, n] = bf16( chain_j fma(w_j, D[slot_of[r, j], n]) (+ S[r, n]) ); pads 0.
// Split steps first sum the down partials of each slot (and of S) in order.
__device__ __forceinline__ v4f load_f4(const float* p) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  v4f r = {v.x, v.y, v.z, v.w};
  return r;
}

// Slots are taken in groups of kCombGroup whose loads are all issued before
// the first use, so a row costs one memory round trip per group instead of
// one per slot; the fma chain still runs in j order and skips invalid slots.
constexpr int kCombGroup = 8;

__device__ __forceinline__ v4f slot_down(const FfnArgs& a, int s, int n) {
  if (!a.split) return load_f4(a.D + (size_t)s * a.H + n);
  const size_t st = (size_t)a.M * a.K * a.H;
  v4f d = load_f4(a.part_d + (size_t)s * a.H + n);
#pragma unroll
  for (int g = 1; g < kSegDN; ++g) d = add4(d, load_f4(a.part_d + g * st + (size_t)s * a.H + n));
  return d;
}

// The fp32 value of y[r, n .. n + 3] before its bf16 rounding (real row r).
__device__ __forceinline__ v4f combine_at(const FfnArgs& a, int r, int n, int with_shared) {
  const int slots = a.sched[SCHED_SLOTS];
  v4f sv = {0.f, 0.f, 0.f, 0.f};
  if (with_shared) {
    if (a.split) {
      const size_t st = (size_t)a.M * a.H;
      sv = load_f4(a.part_s + (size_t)r * a.H + n);
#pragma unroll
      for (int g = 1; g < kSegSD; ++g) sv = add4(sv, load_f4(a.part_s + g * st + (size_t)r * a.H + n));
    } else {
      sv = load_f4(a.S + (size_t)r * a.H + n);
    }
  }
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const int32_t* slp = a.slot_of + (size_t)r * a.K;
  const float* wp = a.w + (size_t)r * a.K;
  for (int j0 = 0; j0 < a.K; j0 += kCombGroup) {
    int sl[kCombGroup];
    float wj[kCombGroup];
    bool ok[kCombGroup];
#pragma unroll
    for (int i = 0; i < kCombGroup; ++i) {
      const int j = min(j0 + i, a.K - 1);
      sl[i] = slp[j];
      wj[i] = wp[j];
    }
    v4f d[kCombGroup];
#pragma unroll
    for (int i = 0; i < kCombGroup; ++i) {
      ok[i] = j0 + i < a.K && sl[i] >= 0 && sl[i] < slots;
      d[i] = slot_down(a, ok[i] ? sl[i] : 0, n);
    }
#pragma unroll
    for (int i = 0; i < kCombGroup; ++i) {
      if (ok[i]) {
        acc[0] = __builtin_fmaf(wj[i], d[i][0], acc[0]);
        acc[1] = __builtin_fmaf(wj[i], d[i][1], acc[1]);
        acc[2] = __builtin_fmaf(wj[i], d[i][2], acc[2]);
        acc[3] = __builtin_fmaf(wj[i], d[i][3], acc[3]);
      }
    }
  }
  if (with_shared) acc = add4(acc, sv);
  return acc;
}

__global__ __launch_bounds__(256) void k_combine(FfnArgs a, int with_shared) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int q = a.H / 4;
  const int r = (int)(idx / q);
  if (r >= a.M) return;
  const int n = (int)(idx % q) * 4;
  uint16_t* yp = a.y + (size_t)r * a.H + n;
  if (!row_real(a.mask, r)) {
    *reinterpret_cast<uint2*>(yp) = make_uint2(0u, 0u);
    return;
  }
  store_bf16x4(yp, combine_at(a, r, n, with_shared));
}

// ---------------------------------------------------------------- residual add + RMSNorm
// The epilogue that feeds the next layer (mstar PR #388: each all-reduce
// fused with the next add + RMSNorm; fused and unfused emit the same bits).
// One workgroup of norm_threads(H) threads per row, one procedure whether y
// comes from memory or from the combine in the same pass:
//   r_new = bf16(fl32(residual) + fl32(y))                 (y: the bf16 layer output)
//   ss    = sum of r_new^2: each thread fma-accumulates its 4-column groups
//           (g = tid, tid + norm_threads(H), ...) in order, then an xor
//           butterfly inside each wave (lane 0's result), then the waves'
//           sums in ascending wave order
//   inv   = 1 / sqrt(ss / H + eps)                         (IEEE division and square root)
//   out   = bf16((r_new * inv) * gamma)
// Pad rows: r_new = out = +0.0 (and y = +0.0); their inputs are never read.
constexpr int kNormThreads = 1024;                 // most threads per row workgroup
constexpr int kNormWaves = kNormThreads / 64;

__device__ __forceinline__ uint2 pack_bf16x4(const float (&v)[4]) {
  return make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                    (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
}

__device__ __forceinline__ void unpack_bf16x4(uint2 b, float (&v)[4]) {
  v[0] = __uint_as_float(b.x << 16);
  v[1] = __uint_as_float(b.x & 0xFFFF0000u);
  v[2] = __uint_as_float(b.y << 16);
  v[3] = __uint_as_float(b.y & 0xFFFF0000u);
}

// yfn(n) returns the bf16 bits of y[r, n .. n + 3] (as a uint2).  Rows of up
// to kNormRegGroups * kNormThreads 4-column groups keep r_new in registers
// and take all their y values before the first store (so the loads of a
// thread's groups overlap); longer rows stream group by group and re-read
// their own r_new.  Both give the same bits.
constexpr int kNormRegGroups = 2;

// Threads of the row workgroup for rows of H columns: enough for
// kNormRegGroups 4-column groups each (whole waves), at most kNormThreads, so
// every thread of a row of up to 8192 columns takes the same number of
// groups.  A function of H alone: both kernels reduce in the same order.
__host__ __device__ __forceinline__ int norm_threads(int H) {
  const int ng = H / 4;
  const int t = ((ng + kNormRegGroups - 1) / kNormRegGroups + 63) / 64 * 64;
  return t < 64 ? 64 : (t > kNormThreads ? kNormThreads : t);
}

__device__ __forceinline__ void add_group(const NormArgs& nm, size_t row, int n, uint2 yb, uint2& b, float& ss) {
  float y[4], res[4], s[4], f[4];
  unpack_bf16x4(yb, y);
  unpack_bf16x4(*reinterpret_cast<const uint2*>(nm.res + row + n), res);
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = res[i] + y[i];
  b = pack_bf16x4(s);
  *reinterpret_cast<uint2*>(nm.res_out + row + n) = b;
  unpack_bf16x4(b, f);
#pragma unroll
  for (int i = 0; i < 4; ++i) ss = __builtin_fmaf(f[i], f[i], ss);
}

__device__ __forceinline__ void norm_group(const NormArgs& nm, size_t row, int n, uint2 b, float inv) {
  float f[4], gm[4], o[4];
  unpack_bf16x4(b, f);
  unpack_bf16x4(*reinterpret_cast<const uint2*>(nm.gamma + n), gm);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (f[i] * inv) * gm[i];
  *reinterpret_cast<uint2*>(nm.out + row + n) = pack_bf16x4(o);
}

template <typename YFn>
__device__ __forceinline__ void add_rmsnorm_row(const NormArgs& nm, int r, int H, YFn yfn) {
  __shared__ float red[kNormWaves];
  const int tid = threadIdx.x, lane = tid & 63, nt = blockDim.x;   // nt = norm_threads(H)
  const size_t row = (size_t)r * H;
  const int ng = H / 4;
  const bool in_regs = ng <= kNormRegGroups * nt;
  float ss = 0.0f;
  uint2 keep[kNormRegGroups];
  if (in_regs) {
    uint2 yb[kNormRegGroups];
#pragma unroll
    for (int k = 0; k < kNormRegGroups; ++k) {
      const int g = tid + k * nt;
      yb[k] = g < ng ? yfn(4 * g) : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kNormRegGroups; ++k) {
      const int g = tid + k * nt;
      if (g < ng) add_group(nm, row, 4 * g, yb[k], keep[k], ss);
    }
  } else {
    for (int g = tid; g < ng; g += nt) {
      uint2 b;
      add_group(nm, row, 4 * g, yfn(4 * g), b, ss);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  ss = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(ss)));   // lane 0's order for the whole wave
  if (lane == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = red[0];
  for (int w = 1; w < nt / 64; ++w) tot += red[w];
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(tot, (float)H) + nm.eps));
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kNormRegGroups; ++k) {
      const int g = tid + k * nt;
      if (g < ng) norm_group(nm, row, 4 * g, keep[k], inv);
    }
  } else {
    for (int g = tid; g < ng; g += nt)
      norm_group(nm, row, 4 * g, *reinterpret_cast<const uint2*>(nm.res_out + row + 4 * g), inv);   // own writes
  }
}

__device__ __forceinline__ void zero_row(uint16_t* p, int H) {
  if (p == nullptr) return;
  for (int g = threadIdx.x; g < H / 4; g += blockDim.x) *reinterpret_cast<uint2*>(p + 4 * g) = make_uint2(0u, 0u);
}

// Standalone: y read from memory.
__global__ __launch_bounds__(kNormThreads) void k_add_rmsnorm(const uint16_t* y, const uint8_t* mask, int H,
                                                              NormArgs nm) {
  const int r = blockIdx.x;
  if (!row_real(mask, r)) {
    zero_row(nm.res_out + (size_t)r * H, H);
    zero_row(nm.out + (size_t)r * H, H);
    return;
  }
  add_rmsnorm_row(nm, r, H, [&](int n) { return *reinterpret_cast<const uint2*>(y + (size_t)r * H + n); });
}

// Fused: y computed by the combine in the same pass (and stored when a.y is set).
__global__ __launch_bounds__(kNormThreads) void k_combine_norm(FfnArgs a, NormArgs nm, int with_shared) {
  const int r = blockIdx.x;
  if (!row_real(a.mask, r)) {
    zero_row(a.y ? a.y + (size_t)r * a.H : nullptr, a.H);
    zero_row(nm.res_out + (size_t)r * a.H, a.H);
    zero_row(nm.out + (size_t)r * a.H, a.H);
    return;
  }
  add_rmsnorm_row(nm, r, a.H, [&](int n) {
    const v4f acc = combine_at(a, r, n, with_shared);
    const float v[4] = {acc[0], acc[1], acc[2], acc[3]};
    const uint2 b = pack_bf16x4(v);
    if (a.y) *reinterpret_cast<uint2*>(a.y + (size_t)r * a.H + n) = b;
    return b;
  });
}

hipError_t launch_add_rmsnorm(const uint16_t* y, const uint8_t* mask, int M, int H, const NormArgs& nm,
                              hipStream_t s) {
  MOE_LAUNCH(KID_ADD_NORM, k_add_rmsnorm, dim3((unsigned)M), dim3(norm_threads(H)), 0, s, y, mask, H, nm);
  return hipSuccess;
}

// ---------------------------------------------------------------- tensor-parallel partials
// y[r, n..n+3] = bf16 of the float32 sum of parts[r, s, n..n+3] over s
// ascending (one thread per row and 4 columns); pad rows +0.0.
__global__ __launch_bounds__(256) void k_sum_partials(const uint16_t* parts, const uint8_t* mask, int M, int H,
                                                      int nsrc, uint16_t* y) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int q = H / 4;
  const int r = (int)(idx / q);
  if (r >= M) return;
  const int n = (int)(idx % q) * 4;
  uint16_t* yp = y + (size_t)r * H + n;
  if (!row_real(mask, r)) {
    *reinterpret_cast<uint2*>(yp) = make_uint2(0u, 0u);
    return;
  }
  const uint16_t* p = parts + (size_t)r * nsrc * H + n;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsrc; s0 += 8) {
    uint2 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const uint2*>(p + (size_t)min(s0 + i, nsrc - 1) * H);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (s0 + i >= nsrc) break;
      float f[4];
      unpack_bf16x4(v[i], f);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = acc[k] + f[k];
    }
  }
  *reinterpret_cast<uint2*>(yp) = pack_bf16x4(acc);
}

hipError_t launch_sum_partials(const uint16_t* parts, const uint8_t* mask, int M, int H, int nsrc, uint16_t* y,
                               hipStream_t s) {
  const long threads = (long)M * (H / 4);
  MOE_LAUNCH(KID_SUM_PARTIALS, k_sum_partials, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, parts, mask,
             M, H, nsrc, y);
  return hipSuccess;
}

// ---------------------------------------------------------------- weight packing
// Row-major [rows, row_bytes] -> packed tiles (see tile_row).  One thread per
// 16-byte chunk of the destination: tile t = (row group, stage), half h and
// lane (r, q) of the fragment it holds.  fp8 fragments hold K bytes
// [32 q, 32 q + 32) of a stage (first 16 in half 0); bf16 fragments hold the
// two 32-deep steps of a stage (step h, elements [8 q, 8 q + 8)).
__global__ __launch_bounds__(256) void k_pack(const uint8_t* src, uint8_t* dst, long chunks, int nst, int is_bf16) {
  const long ci = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (ci >= chunks) return;
  const long tile = ci >> 7;
  const int within = (int)(ci & 127);
  const int h = within >> 6, lane = within & 63;
  const int r = lane & 15, q = lane >> 4;
  const long g = tile / nst;
  const int st = (int)(tile % nst);
  const long row = g * 16 + r;
  const int b = is_bf16 ? st * kBlk + 64 * h + 16 * q : st * kBlk + 32 * q + 16 * h;
  *reinterpret_cast<uint4*>(dst + ci * 16) = *reinterpret_cast<const uint4*>(src + row * ((long)nst * kBlk) + b);
}

// ---------------------------------------------------------------- launchers

hipError_t launch_pack(const void* src, void* dst, long rows, int row_bytes, int is_bf16, hipStream_t s) {
  const long chunks = rows * (row_bytes / 16);
  MOE_LAUNCH(KID_PACK, k_pack, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, (const uint8_t*)src,
             (uint8_t*)dst, chunks, row_bytes / kBlk, is_bf16);
  return hipSuccess;
}

hipError_t launch_plan(const FfnArgs& a, hipStream_t s) {
  MOE_LAUNCH(KID_PLAN, k_plan, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipSuccess;
}

hipError_t launch_prep(const FfnArgs& a, hipStream_t s) {
  const long waves = (long)a.M * ((a.H / kBlk + kQGroup - 1) / kQGroup);
  MOE_LAUNCH(KID_QUANT_X, k_quant_rows<uint16_t>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a.x, a.mask,
             a.M, a.H, a.xq, a.xs);
  return hipSuccess;
}

hipError_t launch_quant_generic(const void* in, int is_bf16, int R, int C, uint8_t* codes, float* scales,
                                hipStream_t s) {
  const long waves = (long)R * ((C / kBlk + kQGroup - 1) / kQGroup);
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (is_bf16) {
    MOE_LAUNCH(KID_QUANT, k_quant_rows<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)in, nullptr, R, C, codes,
               scales);
  } else {
    MOE_LAUNCH(KID_QUANT, k_quant_rows<float>, grid, dim3(256), 0, s, (const float*)in, nullptr, R, C, codes,
               scales);
  }
  return hipSuccess;
}

bool use_split(int M, int H, int I) { return M <= split_rows(I) && H > 0; }

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s, const NormArgs* nm) {
  const int with_shared = a.Is > 0 ? 1 : 0;
  const long max_union = std::min<long>(a.E, (long)a.M * a.K);
  if (a.split) {
    // one slot tile per union expert; the shared expert's gate/up ran in the front launch
    // gate/up also forms the shared h_s; the down launch also runs the shared down
    const int nh = row_halves(a.M);
    const long items = max_union * (a.I / 8) * kSegGU;
    const int gu_blocks = (int)((items + 3) / 4);
    const int hs_blocks = with_shared ? (int)(((long)a.M * a.Is / 2 + 255) / 256) : 0;
    const dim3 gu_grid((unsigned)(hs_blocks + gu_blocks));
    if (nh == 1) {
      MOE_LAUNCH(KID_GATEUP, k_gateup_split<1>, gu_grid, dim3(256), 0, s, a, hs_blocks);
    } else {
      MOE_LAUNCH(KID_GATEUP, k_gateup_split<2>, gu_grid, dim3(256), 0, s, a, hs_blocks);
    }
    const long post_waves = (long)a.M * a.K * (a.I / kBlk);
    const int post_blocks = (int)((post_waves + 3) / 4);
    MOE_LAUNCH(KID_POST_GATEUP, k_post_gateup, dim3((unsigned)post_blocks), dim3(256), 0, s, a);
    const int sd_blocks = with_shared ? ((a.H / 16) * kSegSD + 3) / 4 : 0;
    const long dn_items = max_union * (a.H / kCols) * kSegDN;
    const dim3 dn_grid((unsigned)(sd_blocks + (dn_items + 3) / 4));
    if (nh == 1) {
      MOE_LAUNCH(KID_DOWN, k_down<1>, dn_grid, dim3(256), 0, s, a, sd_blocks);
    } else {
      MOE_LAUNCH(KID_DOWN, k_down<2>, dn_grid, dim3(256), 0, s, a, sd_blocks);
    }
  } else {
    // slot tiles: at most ceil(M*K / kMTile) + (union size), one partial tile per expert
    const long mtiles_max = ((long)a.M * a.K + kMTile - 1) / kMTile + max_union;
    const hipError_t e = launch_tiled(a, mtiles_max, s);
    if (e != hipSuccess) return e;
  }
  if (nm != nullptr && a.split) {
    // Few rows: one row workgroup per row would run the combine on a handful
    // of CUs, so the element-wise combine runs first and the row epilogue
    // after it (the same bits as the single pass).  Without a caller y the
    // combine writes into S, which small steps leave unused (they keep the
    // shared expert's down partials apart).
    FfnArgs b = a;
    if (b.y == nullptr) b.y = reinterpret_cast<uint16_t*>(a.S);
    const long threads = (long)a.M * (a.H / 4);
    MOE_LAUNCH(KID_COMBINE, k_combine, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, b, with_shared);
    return launch_add_rmsnorm(b.y, a.mask, a.M, a.H, *nm, s);
  }
  if (nm != nullptr) {
    MOE_LAUNCH(KID_COMBINE_NORM, k_combine_norm, dim3((unsigned)a.M), dim3(norm_threads(a.H)), 0, s, a, *nm,
               with_shared);
    return hipSuccess;
  }
  const long threads = (long)a.M * (a.H / 4);
  MOE_LAUNCH(KID_COMBINE, k_combine, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a, with_shared);
  return hipSuccess;
}

}  // namespace moe
