// Device building blocks shared by the routing and expert kernels: vector
// loads, stores, the 1x128 quantization of a 128-value block held by one
// wave, the fp8 / bf16 MFMA chains of the small-step kernels (one K segment
// each) and the slot-tile lookup.
#pragma once

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

__device__ __forceinline__ void store_f4(float* p, const v4f& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ v4f add4(const v4f& a, const v4f& b) {
  v4f r = {a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
  return r;
}

// first K-block (or K-step) of segment s when n blocks are split into S
__device__ __forceinline__ int seg_begin(int n, int s, int S) { return (n * s) / S; }

// ---------------------------------------------------------------- packed weights
// Weights are stored in 2048-byte tiles of 16 rows x 128 bytes of K (fp8: one
// K-block; bf16: two 32-deep K steps), the tiles of a 16-row group
// consecutive along K.  In a tile, the 16 bytes that lane (row r, quarter q)
// loads first sit at (r + 16 q) * 16 and the next 16 at 1024 + (r + 16 q) * 16,
// so each of a wave's two loads reads 1 KB of contiguous memory.
constexpr int kTile = 2048;

__device__ __forceinline__ int tile_lane(int r, int q) { return (r + 16 * q) * 16; }

// Lane address of row `row` (of a [rows, K] matrix with `nst` tiles per row
// group) at K stage 0; stage s is + s * kTile.
__device__ __forceinline__ const uint8_t* tile_row(const void* base, size_t row, int nst, int q) {
  return reinterpret_cast<const uint8_t*>(base) + (size_t)(row >> 4) * nst * kTile + tile_lane((int)(row & 15), q);
}

__device__ __forceinline__ v8i load_frag(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 1024);
  v8i r = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  return r;
}

// ---------------------------------------------------------------- quantization
// One wave per (row, 128-column block): amax, s = fl32(amax/448) (1 for a
// zero block), code = e4m3_rne_sat(fl32(v/s)); zero blocks give zero codes.
__device__ __forceinline__ void quant_pair(float v0, float v1, uint8_t* codes, float* scale, int lane) {
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

// ---------------------------------------------------------------- GEMM chains
constexpr int kRing = 4;      // fp8 K-blocks in flight per wave
constexpr int kRingBf = 8;    // bf16 K-steps (32 deep) in flight per wave

__device__ __forceinline__ v8i mask8(const v8i& v, int keep) {
  v8i r = {v[0] & keep, v[1] & keep, v[2] & keep, v[3] & keep, v[4] & keep, v[5] & keep, v[6] & keep, v[7] & keep};
  return r;
}

__device__ __forceinline__ v4i mask4(const v4i& v, int keep) {
  v4i r = {v[0] & keep, v[1] & keep, v[2] & keep, v[3] & keep};
  return r;
}

// fp8 chain over K-blocks [kb0, kb1) for one 16x16 tile.  A (packed weight
// tiles; wp = the lane's tile_row address at K-block 0) and B (row-major)
// stream from global memory through a ring.  Lanes with bvalid == false
// contribute a zero B column and a zero activation scale (bp must point at a
// readable row for every lane; the zeros come from a value mask at use).
// The main loop runs whole ring turns whose refills all lie inside the
// range, so its loads are unconditional and no branch separates a load from
// its wait; the last turns refill only what remains.
__device__ __forceinline__ v4f fp8_chain(const uint8_t* wp, const float* swp, const uint8_t* bp, const float* sxp,
                                         bool bvalid, int kb0, int kb1) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  if (kb0 >= kb1) return acc;
  const int last = kb1 - 1;
  const int keep = bvalid ? -1 : 0;
  v8i wb[kRing], xb[kRing];
  float swb[kRing], sxb[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    const int kb = min(kb0 + i, last);
    wb[i] = load_frag(wp + (size_t)kb * kTile);
    swb[i] = swp[kb];
    xb[i] = load32(bp + kb * kBlk);
    sxb[i] = sxp[kb];
  }
  auto step = [&](int i) {
    const v4f p = mfma_fp8_k128(wb[i], mask8(xb[i], keep));
    scale_acc(acc, p, bvalid ? sxb[i] : 0.0f, swb[i]);
  };
  auto refill = [&](int i, int nk) {
    wb[i] = load_frag(wp + (size_t)nk * kTile);
    swb[i] = swp[nk];
    xb[i] = load32(bp + nk * kBlk);
    sxb[i] = sxp[nk];
  };
  int k0 = kb0;
  for (; k0 + 2 * kRing <= kb1; k0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      step(i);
      refill(i, k0 + i + kRing);
    }
  }
  for (; k0 < kb1; k0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      if (k0 + i < kb1) step(i);
      if (k0 + i + kRing < kb1) refill(i, k0 + i + kRing);
    }
  }
  return acc;
}

// The same chain for two B tiles (two row halves) sharing each A fragment:
// acc0 over B rows bp0 (valid v0), acc1 over bp1 (v1).  Each accumulator
// takes exactly the steps fp8_chain gives it, so the values are the same.
__device__ __forceinline__ void fp8_chain2(const uint8_t* wp, const float* swp, const uint8_t* bp0,
                                           const uint8_t* bp1, const float* sxp0, const float* sxp1, bool v0,
                                           bool v1, int kb0, int kb1, v4f& acc0, v4f& acc1) {
  acc0 = v4f{0.f, 0.f, 0.f, 0.f};
  acc1 = acc0;
  if (kb0 >= kb1) return;
  const int last = kb1 - 1;
  const int keep0 = v0 ? -1 : 0, keep1 = v1 ? -1 : 0;
  v8i wb[kRing], xa[kRing], xc[kRing];
  float swb[kRing], sa[kRing], sc[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    const int kb = min(kb0 + i, last);
    wb[i] = load_frag(wp + (size_t)kb * kTile);
    swb[i] = swp[kb];
    xa[i] = load32(bp0 + kb * kBlk);
    sa[i] = sxp0[kb];
    xc[i] = load32(bp1 + kb * kBlk);
    sc[i] = sxp1[kb];
  }
  auto step = [&](int i) {
    const v4f p0 = mfma_fp8_k128(wb[i], mask8(xa[i], keep0));
    scale_acc(acc0, p0, v0 ? sa[i] : 0.0f, swb[i]);
    const v4f p1 = mfma_fp8_k128(wb[i], mask8(xc[i], keep1));
    scale_acc(acc1, p1, v1 ? sc[i] : 0.0f, swb[i]);
  };
  auto refill = [&](int i, int nk) {
    wb[i] = load_frag(wp + (size_t)nk * kTile);
    swb[i] = swp[nk];
    xa[i] = load32(bp0 + nk * kBlk);
    sa[i] = sxp0[nk];
    xc[i] = load32(bp1 + nk * kBlk);
    sc[i] = sxp1[nk];
  };
  int k0 = kb0;
  for (; k0 + 2 * kRing <= kb1; k0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      step(i);
      refill(i, k0 + i + kRing);
    }
  }
  for (; k0 < kb1; k0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      if (k0 + i < kb1) step(i);
      if (k0 + i + kRing < kb1) refill(i, k0 + i + kRing);
    }
  }
}

// bf16 chain over K-steps [s0, s1) (32 deep each) for one 16x16 tile; loads
// as in fp8_chain.  wp = the lane's packed tile_row address at stage 0 (step
// st is in stage st / 2, half st % 2); bp = the lane's row-major B row.
__device__ __forceinline__ v4i load_step(const uint8_t* wp, int st) {
  const uint4 v = *reinterpret_cast<const uint4*>(wp + (size_t)(st >> 1) * kTile + (st & 1) * 1024);
  v4i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  return r;
}

__device__ __forceinline__ v4f bf16_chain(const uint8_t* wp, const uint16_t* bp, bool bvalid, int s0, int s1) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  if (s0 >= s1) return acc;
  const int last = s1 - 1;
  const int keep = bvalid ? -1 : 0;
  v4i wb[kRingBf], xb[kRingBf];
#pragma unroll
  for (int i = 0; i < kRingBf; ++i) {
    const int st = min(s0 + i, last);
    wb[i] = load_step(wp, st);
    xb[i] = load16(bp + st * 32);
  }
  int k0 = s0;
  for (; k0 + 2 * kRingBf <= s1; k0 += kRingBf) {
#pragma unroll
    for (int i = 0; i < kRingBf; ++i) {
      acc = mfma_bf16_k32(wb[i], mask4(xb[i], keep), acc);
      wb[i] = load_step(wp, k0 + i + kRingBf);
      xb[i] = load16(bp + (k0 + i + kRingBf) * 32);
    }
  }
  for (; k0 < s1; k0 += kRingBf) {
#pragma unroll
    for (int i = 0; i < kRingBf; ++i) {
      if (k0 + i < s1) acc = mfma_bf16_k32(wb[i], mask4(xb[i], keep), acc);
      const int nx = k0 + i + kRingBf;
      if (nx < s1) {
        wb[i] = load_step(wp, nx);
        xb[i] = load16(bp + nx * 32);
      }
    }
  }
  return settle_bf16(acc);
}

// bf16_chain for two B tiles (two row halves) sharing each A fragment; each
// accumulator takes exactly the steps bf16_chain gives it.
__device__ __forceinline__ void bf16_chain2(const uint8_t* wp, const uint16_t* bp0, const uint16_t* bp1, bool v0,
                                            bool v1, int s0, int s1, v4f& acc0, v4f& acc1) {
  acc0 = v4f{0.f, 0.f, 0.f, 0.f};
  acc1 = acc0;
  if (s0 >= s1) return;
  const int last = s1 - 1;
  const int keep0 = v0 ? -1 : 0, keep1 = v1 ? -1 : 0;
  v4i wb[kRingBf], xa[kRingBf], xc[kRingBf];
#pragma unroll
  for (int i = 0; i < kRingBf; ++i) {
    const int st = min(s0 + i, last);
    wb[i] = load_step(wp, st);
    xa[i] = load16(bp0 + st * 32);
    xc[i] = load16(bp1 + st * 32);
  }
  int k0 = s0;
  for (; k0 + 2 * kRingBf <= s1; k0 += kRingBf) {
#pragma unroll
    for (int i = 0; i < kRingBf; ++i) {
      acc0 = mfma_bf16_k32(wb[i], mask4(xa[i], keep0), acc0);
      acc1 = mfma_bf16_k32(wb[i], mask4(xc[i], keep1), acc1);
      wb[i] = load_step(wp, k0 + i + kRingBf);
      xa[i] = load16(bp0 + (k0 + i + kRingBf) * 32);
      xc[i] = load16(bp1 + (k0 + i + kRingBf) * 32);
    }
  }
  for (; k0 < s1; k0 += kRingBf) {
#pragma unroll
    for (int i = 0; i < kRingBf; ++i) {
      if (k0 + i < s1) {
        acc0 = mfma_bf16_k32(wb[i], mask4(xa[i], keep0), acc0);
        acc1 = mfma_bf16_k32(wb[i], mask4(xc[i], keep1), acc1);
      }
      const int nx = k0 + i + kRingBf;
      if (nx < s1) {
        wb[i] = load_step(wp, nx);
        xa[i] = load16(bp0 + nx * 32);
        xc[i] = load16(bp1 + nx * 32);
      }
    }
  }
  acc0 = settle_bf16(acc0);
  acc1 = settle_bf16(acc1);
}

// ---------------------------------------------------------------- slot tiles
// A tile of <= kMTile consecutive slots of one union expert.  Tiles are
// numbered expert by expert (mtile_offs[u] = first tile of union expert u).
struct Tile {
  int e;       // expert id
  int s0;      // first slot of the tile
  int mcnt;    // slots in the tile (<= kMTile)
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

}  // namespace moe
