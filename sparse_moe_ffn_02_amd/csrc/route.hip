// Router, top-k selection, expert union and row compaction (gfx950).
//
// noaux-tc routing as the pages state it (mstar PR #388: NoAuxTcRouter with
// its router kernel; MoE-Infinity PR #140: the per-expert router bias): a
// score per expert, a correction bias added for selection only, top-k.
// The union of the step's experts is formed in ascending expert id with
// rows ascending inside each expert, the same order whichever slots carry
// the rows (openinfer PR #610, "Gates": same union order under both row
// mappings).
//
// Logits are float64: bf16 x bf16 products are exact in float64, so the
// selection agrees with a float64 evaluation except on near-exact ties.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- logits
// Every logit l[r, e] is computed by one fixed procedure, whatever row tile
// or expert group it falls in: lane j of a wave accumulates (float64 FMA, in
// ascending order) the products for h = 512 i + 8 j + t (i ascending, then
// t = 0..7), and the 64 lane partials are summed by an xor butterfly.
template <int EPW>
__global__ __launch_bounds__(256) void k_router_logits(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * 8;
  const int e0 = (blockIdx.y * 4 + wave) * EPW;
  if (e0 >= a.E) return;
  bool rv[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) rv[r] = (r0 + r < a.M) && (a.mask == nullptr || a.mask[r0 + r] != 0);
  double acc[8][EPW];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int e = 0; e < EPW; ++e) acc[r][e] = 0.0;

  for (int h0 = lane * 8; h0 < a.H; h0 += 512) {
    uint4 wv[EPW];
#pragma unroll
    for (int e = 0; e < EPW; ++e)
      wv[e] = (e0 + e < a.E) ? *reinterpret_cast<const uint4*>(a.wr + (size_t)(e0 + e) * a.H + h0)
                             : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (!rv[r]) continue;
      const uint4 xv = *reinterpret_cast<const uint4*>(a.x + (size_t)(r0 + r) * a.H + h0);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const double xd = (double)bf16_to_f32((uint16_t)(xw[t >> 1] >> ((t & 1) * 16)));
#pragma unroll
        for (int e = 0; e < EPW; ++e) {
          const uint32_t ww[4] = {wv[e].x, wv[e].y, wv[e].z, wv[e].w};
          const double wd = (double)bf16_to_f32((uint16_t)(ww[t >> 1] >> ((t & 1) * 16)));
          acc[r][e] = __builtin_fma(xd, wd, acc[r][e]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (!rv[r]) continue;
#pragma unroll
    for (int e = 0; e < EPW; ++e) {
      const double s = wave_sum_f64(acc[r][e]);
      if (lane == 0 && e0 + e < a.E) a.logits[(size_t)(r0 + r) * a.E + e0 + e] = s;
    }
  }
}

// ---------------------------------------------------------------- select
// One wave per row.  c = sigmoid(l) + bias; the k largest c win, exact ties
// to the lower expert id.  Output ids ascending; w = scale * sig / sum(sig)
// with the sum taken in ascending id order (float64, stored as float32).
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 256;

__global__ __launch_bounds__(256) void k_route_select(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.M) return;
  const int nwords = (a.E + 31) / 32;
  const bool real = (a.mask == nullptr || a.mask[row] != 0);
  if (!real) {
    if (lane < a.K) {
      a.ids[(size_t)row * a.K + lane] = -1;
      a.w[(size_t)row * a.K + lane] = 0.0f;
    }
    if (lane < nwords) a.rowbits[(size_t)row * nwords + lane] = 0u;
    return;
  }
  double c[4], sg[4];
  bool ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    ok[q] = e < a.E;
    c[q] = -INFINITY;
    sg[q] = 0.0;
    if (ok[q]) {
      const double l = a.logits[(size_t)row * a.E + e];
      sg[q] = 1.0 / (1.0 + exp(-l));
      const double cc = sg[q] + (double)a.bias[e];
      c[q] = (cc == cc) ? cc : -INFINITY;
    }
  }
  int sel[kMaxTopK];
  double ssel[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    sel[j] = 0x7fffffff;
    ssel[j] = 0.0;
    if (j >= a.K) continue;
    double bc = -INFINITY, bs = 0.0;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (ok[q] && (c[q] > bc || (c[q] == bc && e < be))) { bc = c[q]; be = e; bs = sg[q]; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double oc = __shfl_xor(bc, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      const double os = __shfl_xor(bs, o, 64);
      if (oc > bc || (oc == bc && oe < be)) { bc = oc; be = oe; bs = os; }
    }
    sel[j] = be;
    ssel[j] = bs;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q == be) ok[q] = false;
  }
  // ascending id order (k <= 16, wave-uniform insertion sort)
#pragma unroll
  for (int i = 1; i < kMaxTopK; ++i) {
#pragma unroll
    for (int j = i; j > 0; --j) {
      if (sel[j] < sel[j - 1]) {
        const int te = sel[j]; sel[j] = sel[j - 1]; sel[j - 1] = te;
        const double ts = ssel[j]; ssel[j] = ssel[j - 1]; ssel[j - 1] = ts;
      }
    }
  }
  double tot = 0.0;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < a.K) tot += ssel[j];
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= a.K) continue;
    if (lane == j) {
      a.ids[(size_t)row * a.K + j] = sel[j];
      a.w[(size_t)row * a.K + j] = (float)((double)a.scale * (ssel[j] / tot));
    }
    if ((sel[j] >> 5) == lane) word |= 1u << (sel[j] & 31);
  }
  if (lane < nwords) a.rowbits[(size_t)row * nwords + lane] = word;
}

// ---------------------------------------------------------------- union
// One workgroup.  Counts per expert, the ascending union with its slot
// offsets and column-tile offsets, then each expert's rows in ascending row
// order (ballot + prefix popcount), and slot_of[r, j] for every (row, pick).
__global__ __launch_bounds__(1024) void k_union(RouteArgs a) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const int nwords = (a.E + 31) / 32;
  for (int e = tid; e < a.E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int r = tid; r < a.M; r += blockDim.x) {
    const bool real = (a.mask == nullptr || a.mask[r] != 0);
    for (int j = 0; j < a.K; ++j) {
      if (real) {
        const int e = a.ids[(size_t)r * a.K + j];
        if (e >= 0 && e < a.E) atomicAdd(&cnt[e], 1);
      } else {
        a.slot_of[(size_t)r * a.K + j] = -1;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int nu = 0, acc = 0, mt = 0;
    for (int e = 0; e < a.E; ++e) {
      const int n = cnt[e];
      base[e] = acc;
      if (n) {
        a.union_ids[nu] = e;
        a.offs[nu] = acc;
        a.mtile_offs[nu] = mt;
        ++nu;
        acc += n;
        mt += (n + kMTile - 1) / kMTile;
      }
    }
    a.offs[nu] = acc;
    a.mtile_offs[nu] = mt;
    *a.n_union = nu;
    a.sched[SCHED_NUNION] = nu;
    a.sched[SCHED_MTILES] = mt;
    a.sched[SCHED_SLOTS] = acc;
    a.sched[SCHED_BAD] = 0;
  }
  __syncthreads();
  for (int e = wave; e < a.E; e += nwaves) {
    if (cnt[e] == 0) continue;
    int b = base[e];
    const int wi = e >> 5;
    const uint32_t bit = 1u << (e & 31);
    for (int r0 = 0; r0 < a.M; r0 += 64) {
      const int r = r0 + lane;
      bool hit = false;
      uint32_t word = 0;
      if (r < a.M) {
        word = a.rowbits[(size_t)r * nwords + wi];
        hit = (word & bit) != 0;
      }
      const uint64_t m = __ballot(hit);
      if (hit) {
        const int p = b + __popcll(m & ((1ull << lane) - 1ull));
        a.rows[p] = r;
        int j = __popc(word & (bit - 1u));
        for (int w2 = 0; w2 < wi; ++w2) j += __popc(a.rowbits[(size_t)r * nwords + w2]);
        a.slot_of[(size_t)r * a.K + j] = p;
      }
      b += __popcll(m);
    }
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const dim3 blk(256);
  if (a.M <= kDecodeMaxRows) {
    MOE_LAUNCH(KID_ROUTER_LOGITS, k_router_logits<1>, dim3((a.M + 7) / 8, (a.E + 3) / 4), blk, 0, s, a);
  } else {
    MOE_LAUNCH(KID_ROUTER_LOGITS, k_router_logits<4>, dim3((a.M + 7) / 8, (a.E + 15) / 16), blk, 0, s, a);
  }
  MOE_LAUNCH(KID_ROUTE_SELECT, k_route_select, dim3((a.M + 3) / 4), blk, 0, s, a);
  MOE_LAUNCH(KID_UNION, k_union, dim3(1), dim3(1024), 0, s, a);
  return hipSuccess;
}

}  // namespace moe
