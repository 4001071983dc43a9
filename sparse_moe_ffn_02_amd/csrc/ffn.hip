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
//   routed GEMM  out[s, n] = chain over K-blocks kb ascending of
//                acc = fma(s_act[s, kb] * s_w[n/128, kb], P_kb, acc), acc0 = 0,
//                P_kb = one 16x16x128 fp8 MFMA with a zero accumulator;
//   shared GEMM  one bf16 16x16x32 MFMA chain over K ascending from zero;
//   combine      acc = fma(w_j, D[slot(r, j)], acc) for j ascending, then
//                + S[r] when the shared expert is present, then bf16 RNE.
// Which tile, wave or kernel computes an element never changes its bits.
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {


__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  v8i r = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  return r;
}

__device__ __forceinline__ v4i load16(const uint16_t* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  v4i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  return r;
}

__device__ __forceinline__ bool row_real(const uint8_t* mask, int r) { return mask == nullptr || mask[r] != 0; }

__device__ __forceinline__ void store_bf16x4(uint16_t* p, const v4f& v) {
  const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

// ---------------------------------------------------------------- quantization
// One wave per (row, 128-column block): amax, s = fl32(amax/448) (1 for a
// zero block), code = e4m3_rne_sat(fl32(v/s)); zero blocks give zero codes.
template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void quant_block(const T* in, uint8_t* codes, float* scale, int lane) {
  const float v0 = load_as_f32<T>(in + 2 * lane);
  const float v1 = load_as_f32<T>(in + 2 * lane + 1);
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const float s = quant_scale(amax);
  uint32_t c0 = 0, c1 = 0;
  if (amax != 0.0f) {
    c0 = quant_code(v0, s);
    c1 = quant_code(v1, s);
  }
  *reinterpret_cast<uint16_t*>(codes + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) *scale = s;
}

// rows [0, R) of a [R, C] matrix; rows with mask 0 are skipped (never read).
template <typename T>
__global__ __launch_bounds__(256) void k_quant_rows(const T* in, const uint8_t* mask, int R, int C, uint8_t* codes,
                                                    float* scales) {
  const int lane = threadIdx.x & 63;
  const int nb = C / kBlk;
  const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int r = (int)(item / nb);
  const int b = (int)(item % nb);
  if (r >= R || !row_real(mask, r)) return;
  quant_block<T>(in + (size_t)r * C + b * kBlk, codes + (size_t)r * C + b * kBlk, scales + (size_t)r * nb + b, lane);
}

// First kernel of every call: quantize x (real rows).
__global__ __launch_bounds__(256) void k_prep(const uint16_t* x, const uint8_t* mask, int M, int H, uint8_t* xq,
                                              float* xs) {
  const int lane = threadIdx.x & 63;
  const int nb = H / kBlk;
  const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int r = (int)(item / nb);
  const int b = (int)(item % nb);
  if (r >= M || !row_real(mask, r)) return;
  quant_block<uint16_t>(x + (size_t)r * H + b * kBlk, xq + (size_t)r * H + b * kBlk, xs + (size_t)r * nb + b, lane);
}

// After gate/up: requantize routed h per (slot, block) for the slots in use.
__global__ __launch_bounds__(256) void k_post_gateup(FfnArgs a) {
  const int lane = threadIdx.x & 63;
  const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nbI = a.I / kBlk;
  const int slot = (int)(item / nbI);
  const int b = (int)(item % nbI);
  if (slot >= a.sched[SCHED_SLOTS]) return;
  quant_block<float>(a.hbuf + (size_t)slot * a.I + b * kBlk, a.hq + (size_t)slot * a.I + b * kBlk,
                     a.hs + (size_t)slot * nbI + b, lane);
}

// ---------------------------------------------------------------- plan
// Checks a caller-supplied routing and derives the column-tile schedule.
// A malformed routing (n_union out of range, offsets not starting at 0 or
// not ascending, union ids not ascending in [0, E), more slots than M*K)
// schedules no routed work and sets sched[SCHED_BAD] = 1.
__global__ __launch_bounds__(64) void k_plan(FfnArgs a) {
  if (threadIdx.x != 0) return;
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
  if (bad) {
    a.sched[SCHED_NUNION] = 0;
    a.sched[SCHED_MTILES] = 0;
    a.sched[SCHED_SLOTS] = 0;
    a.sched[SCHED_BAD] = 1;
    a.mtile_offs[0] = 0;
    return;
  }
  a.mtile_offs[nu] = mt;
  a.sched[SCHED_NUNION] = nu;
  a.sched[SCHED_MTILES] = mt;
  a.sched[SCHED_SLOTS] = a.offs[nu];
  a.sched[SCHED_BAD] = 0;
}

// ---------------------------------------------------------------- work items
struct Tile {
  int e;       // expert id
  int s0;      // first slot of the column tile
  int mcnt;    // slots in the tile (<= 16)
};

__device__ __forceinline__ Tile routed_tile(const FfnArgs& a, int mtg) {
  const int nu = a.sched[SCHED_NUNION];
  int lo = 0, hi = nu - 1;          // largest u with mtile_offs[u] <= mtg
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.mtile_offs[mid] <= mtg) lo = mid; else hi = mid - 1;
  }
  Tile t;
  t.e = a.union_ids[lo];
  t.s0 = a.offs[lo] + (mtg - a.mtile_offs[lo]) * kMTile;
  t.mcnt = min(kMTile, a.offs[lo + 1] - t.s0);
  return t;
}

// One wave per work item.  The grid covers the largest item count the call
// can produce (the union is only known on the device); waves past the real
// count exit at once, and the hardware dispatcher balances the rest.
__device__ __forceinline__ int wave_item() { return blockIdx.x * 4 + (threadIdx.x >> 6); }

constexpr int kRing = 4;      // fp8 K-blocks in flight per wave
constexpr int kRingBf = 8;    // bf16 K-steps (32 deep) in flight per wave

// Routed gate+up for 8 columns of I and one tile of <= 16 slots.  The 16
// rows of the MFMA A operand are gate rows n0..n0+7 (rows 0-7) and up rows
// n0..n0+7 (rows 8-15), so lane l (l < 32) holds G and lane l + 32 holds U of
// the same (slot, n).  Writes h = silu(G) * U (fp32) for the tile's slots.
__device__ void routed_gateup(const FfnArgs& a, const Tile& t, int nt, int lane) {
  const int c = lane & 15, kq = lane >> 4;
  const int n0 = nt * 8;
  const int nkb = a.H / kBlk;
  int row = -1;
  if (c < t.mcnt) {
    row = a.rows[t.s0 + c];
    if (row < 0 || row >= a.M) row = -1;
  }
  const uint8_t* bp = a.xq + (size_t)(row < 0 ? 0 : row) * a.H + kq * 32;
  const float* sxp = a.xs + (size_t)(row < 0 ? 0 : row) * nkb;
  const uint8_t* wp = (c < 8 ? a.wg : a.wu) + ((size_t)t.e * a.I + n0 + (c & 7)) * a.H + kq * 32;
  const float* swp = (kq < 2 ? a.sg : a.su) + ((size_t)t.e * (a.I / kBlk) + n0 / kBlk) * nkb;
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  v8i wb[kRing], xb[kRing];
  float sxb[kRing], swb[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    if (i < nkb) {
      wb[i] = load32(wp + i * kBlk);
      xb[i] = row >= 0 ? load32(bp + i * kBlk) : zero8;
      sxb[i] = row >= 0 ? sxp[i] : 0.0f;
      swb[i] = swp[i];
    }
  }
  for (int kb0 = 0; kb0 < nkb; kb0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int kb = kb0 + i;
      if (kb >= nkb) break;
      const v4f p = mfma_fp8_k128(wb[i], xb[i]);
      scale_acc(acc, p, sxb[i], swb[i]);
      const int nk = kb + kRing;
      if (nk < nkb) {
        wb[i] = load32(wp + nk * kBlk);
        if (row >= 0) {
          xb[i] = load32(bp + nk * kBlk);
          sxb[i] = sxp[nk];
        }
        swb[i] = swp[nk];
      }
    }
  }
  float u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = __shfl_xor(acc[i], 32, 64);
  if (kq < 2 && row >= 0) {
    float4 h;
    h.x = silu_mul(acc[0], u[0]);
    h.y = silu_mul(acc[1], u[1]);
    h.z = silu_mul(acc[2], u[2]);
    h.w = silu_mul(acc[3], u[3]);
    *reinterpret_cast<float4*>(a.hbuf + (size_t)(t.s0 + c) * a.I + n0 + kq * 4) = h;
  }
}

// Shared gate+up for 8 columns of I_s and 16 rows, arranged as above (gate
// rows 0-7, up rows 8-15); writes h_s = bf16(silu(g) * u).
__device__ void shared_gateup(const FfnArgs& a, int mt, int nt, int lane) {
  const int c = lane & 15, kq = lane >> 4;
  const int n0 = nt * 8;
  const int row = mt * kMTile + c;
  const bool valid = row < a.M && row_real(a.mask, row);
  const uint16_t* wp = (c < 8 ? a.wsg : a.wsu) + (size_t)(n0 + (c & 7)) * a.H + kq * 8;
  const uint16_t* bp = a.x + (size_t)(valid ? row : 0) * a.H + kq * 8;
  const v4i zero4 = {0, 0, 0, 0};
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const int ns = a.H / 32;
  v4i wb[kRingBf], xb[kRingBf];
#pragma unroll
  for (int i = 0; i < kRingBf; ++i) {
    if (i < ns) {
      wb[i] = load16(wp + i * 32);
      xb[i] = valid ? load16(bp + i * 32) : zero4;
    }
  }
  for (int s0 = 0; s0 < ns; s0 += kRingBf) {
#pragma unroll
    for (int i = 0; i < kRingBf; ++i) {
      const int st = s0 + i;
      if (st >= ns) break;
      acc = mfma_bf16_k32(wb[i], xb[i], acc);
      const int nx = st + kRingBf;
      if (nx < ns) {
        wb[i] = load16(wp + nx * 32);
        if (valid) xb[i] = load16(bp + nx * 32);
      }
    }
  }
  float u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = __shfl_xor(acc[i], 32, 64);
  if (kq < 2 && valid) {
    const v4f h = {silu_mul(acc[0], u[0]), silu_mul(acc[1], u[1]), silu_mul(acc[2], u[2]), silu_mul(acc[3], u[3])};
    store_bf16x4(a.hsh + (size_t)row * a.Is + n0 + kq * 4, h);
  }
}

// Shared items first (the longest), then routed items.
__global__ __launch_bounds__(256, 2) void k_gateup(FfnArgs a) {
  const int lane = threadIdx.x & 63;
  const int ntI = a.I / 8;
  const int ntS = a.Is / 8;
  const int n_sh = (a.Is > 0) ? ((a.M + kMTile - 1) / kMTile) * ntS : 0;
  const int total = n_sh + a.sched[SCHED_MTILES] * ntI;
  const int t = wave_item();
  if (t >= total) return;
  if (t < n_sh) {
    shared_gateup(a, t / ntS, t % ntS, lane);
  } else {
    const int tt = t - n_sh;
    routed_gateup(a, routed_tile(a, tt / ntI), tt % ntI, lane);
  }
}

// ---------------------------------------------------------------- down
// D[slot, n] for 16 columns of H and one tile of <= 16 slots.
__device__ __forceinline__ v4f routed_down_chain(const FfnArgs& a, int e, int slot, int n0, int lane) {
  const int c = lane & 15, kq = lane >> 4;
  const int nkb = a.I / kBlk;
  const uint8_t* wp = a.wd + ((size_t)e * a.H + n0 + c) * a.I + kq * 32;
  const uint8_t* bp = a.hq + (size_t)(slot < 0 ? 0 : slot) * a.I + kq * 32;
  const float* shp = a.hs + (size_t)(slot < 0 ? 0 : slot) * nkb;
  const float* swp = a.sd + ((size_t)e * (a.H / kBlk) + n0 / kBlk) * nkb;
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  v8i wb[kRing], hb[kRing];
  float shb[kRing], swb[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    if (i < nkb) {
      wb[i] = load32(wp + i * kBlk);
      hb[i] = slot >= 0 ? load32(bp + i * kBlk) : zero8;
      shb[i] = slot >= 0 ? shp[i] : 0.0f;
      swb[i] = swp[i];
    }
  }
  for (int kb0 = 0; kb0 < nkb; kb0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int kb = kb0 + i;
      if (kb >= nkb) break;
      const v4f p = mfma_fp8_k128(wb[i], hb[i]);
      scale_acc(acc, p, shb[i], swb[i]);
      const int nk = kb + kRing;
      if (nk < nkb) {
        wb[i] = load32(wp + nk * kBlk);
        if (slot >= 0) {
          hb[i] = load32(bp + nk * kBlk);
          shb[i] = shp[nk];
        }
        swb[i] = swp[nk];
      }
    }
  }
  return acc;
}

__device__ __forceinline__ v4f shared_down_chain(const FfnArgs& a, int row_or_neg, int n0, int lane) {
  const int c = lane & 15, kq = lane >> 4;
  const uint16_t* wp = a.wsd + (size_t)(n0 + c) * a.Is + kq * 8;
  const uint16_t* bp = a.hsh + (size_t)(row_or_neg < 0 ? 0 : row_or_neg) * a.Is + kq * 8;
  const v4i zero4 = {0, 0, 0, 0};
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const int ns = a.Is / 32;
  v4i wb[kRingBf], hb[kRingBf];
#pragma unroll
  for (int i = 0; i < kRingBf; ++i) {
    if (i < ns) {
      wb[i] = load16(wp + i * 32);
      hb[i] = row_or_neg >= 0 ? load16(bp + i * 32) : zero4;
    }
  }
  for (int st0 = 0; st0 < ns; st0 += kRingBf) {
#pragma unroll
    for (int i = 0; i < kRingBf; ++i) {
      const int st = st0 + i;
      if (st >= ns) break;
      acc = mfma_bf16_k32(wb[i], hb[i], acc);
      const int nx = st + kRingBf;
      if (nx < ns) {
        wb[i] = load16(wp + nx * 32);
        if (row_or_neg >= 0) hb[i] = load16(bp + nx * 32);
      }
    }
  }
  return acc;
}

// Shared-down items first, then routed down items.
__global__ __launch_bounds__(256, 2) void k_down(FfnArgs a) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, kq = lane >> 4;
  const int ntH = a.H / 16;
  const int n_sh = (a.Is > 0) ? ((a.M + kMTile - 1) / kMTile) * ntH : 0;
  const int total = n_sh + a.sched[SCHED_MTILES] * ntH;
  const int t = wave_item();
  if (t < total) {
    if (t < n_sh) {
      const int mt = t / ntH, nt = t % ntH;
      const int row = mt * kMTile + c;
      const bool valid = row < a.M && row_real(a.mask, row);
      const v4f r = shared_down_chain(a, valid ? row : -1, nt * 16, lane);
      if (valid)
        *reinterpret_cast<float4*>(a.S + (size_t)row * a.H + nt * 16 + kq * 4) = make_float4(r[0], r[1], r[2], r[3]);
    } else {
      const int tt = t - n_sh;
      const Tile tl = routed_tile(a, tt / ntH);
      const int nt = tt % ntH;
      const int slot = c < tl.mcnt ? tl.s0 + c : -1;
      const v4f r = routed_down_chain(a, tl.e, slot, nt * 16, lane);
      if (slot >= 0)
        *reinterpret_cast<float4*>(a.D + (size_t)slot * a.H + nt * 16 + kq * 4) = make_float4(r[0], r[1], r[2], r[3]);
    }
  }
}

// y[r, n] = bf16( chain_j fma(w_j, D[slot_of[r, j], n]) (+ S[r, n]) ); pads 0.
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
  const int slots = a.sched[SCHED_SLOTS];
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.K; ++j) {
    const int s = a.slot_of[(size_t)r * a.K + j];
    if (s < 0 || s >= slots) continue;
    const float wj = a.w[(size_t)r * a.K + j];
    const float4 d = *reinterpret_cast<const float4*>(a.D + (size_t)s * a.H + n);
    acc[0] = __builtin_fmaf(wj, d.x, acc[0]);
    acc[1] = __builtin_fmaf(wj, d.y, acc[1]);
    acc[2] = __builtin_fmaf(wj, d.z, acc[2]);
    acc[3] = __builtin_fmaf(wj, d.w, acc[3]);
  }
  if (with_shared) {
    const float4 sv = *reinterpret_cast<const float4*>(a.S + (size_t)r * a.H + n);
    acc[0] = acc[0] + sv.x;
    acc[1] = acc[1] + sv.y;
    acc[2] = acc[2] + sv.z;
    acc[3] = acc[3] + sv.w;
  }
  store_bf16x4(yp, acc);
}

// ---------------------------------------------------------------- launchers

hipError_t launch_plan(const FfnArgs& a, hipStream_t s) {
  MOE_LAUNCH(KID_PLAN, k_plan, dim3(1), dim3(64), 0, s, a);
  return hipSuccess;
}

hipError_t launch_prep(const FfnArgs& a, hipStream_t s) {
  const long waves = (long)a.M * (a.H / kBlk);
  MOE_LAUNCH(KID_QUANT_X, k_prep, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a.x, a.mask, a.M, a.H, a.xq,
             a.xs);
  return hipSuccess;
}

hipError_t launch_quant_generic(const void* in, int is_bf16, int R, int C, uint8_t* codes, float* scales,
                                hipStream_t s) {
  const long waves = (long)R * (C / kBlk);
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

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  const int with_shared = a.Is > 0 ? 1 : 0;
  // column tiles of <= 16 slots: at most ceil(M*K/16) + (union size) of them
  const long mtiles_max = ((long)a.M * a.K + kMTile - 1) / kMTile + std::min<long>(a.E, (long)a.M * a.K);
  const long sh_tiles = with_shared ? (a.M + kMTile - 1) / kMTile : 0;
  const long gu_items = sh_tiles * (a.Is / 8) + mtiles_max * (a.I / 8);
  MOE_LAUNCH(KID_GATEUP, k_gateup, dim3((unsigned)((gu_items + 3) / 4)), dim3(256), 0, s, a);
  const long post_waves = (long)a.M * a.K * (a.I / kBlk);
  MOE_LAUNCH(KID_POST_GATEUP, k_post_gateup, dim3((unsigned)((post_waves + 3) / 4)), dim3(256), 0, s, a);
  const long dn_items = (sh_tiles + mtiles_max) * (a.H / 16);
  MOE_LAUNCH(KID_DOWN, k_down, dim3((unsigned)((dn_items + 3) / 4)), dim3(256), 0, s, a);
  const long threads = (long)a.M * (a.H / 4);
  MOE_LAUNCH(KID_COMBINE, k_combine, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a, with_shared);
  return hipSuccess;
}

}  // namespace moe
