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
#include <string.h>

#include <algorithm>

#include "moe_chains.h"

namespace moe {

// ---------------------------------------------------------------- logits
// bf16 element t (0..7) of 8 packed in a uint4
__device__ __forceinline__ uint16_t u16_of(const uint4& v, int t) {
  const uint32_t w = t < 2 ? v.x : t < 4 ? v.y : t < 6 ? v.z : v.w;
  return (uint16_t)(w >> ((t & 1) * 16));
}

// Every logit l[r, e] is computed by one fixed procedure, whatever row tile
// or expert group it falls in: lane j of a wave accumulates (float64 FMA, in
// ascending order) the products for h = 512 i + 8 j + t (i ascending, then
// t = 0..7), and the 64 lane partials are summed by an xor butterfly.
// A block computes 8 rows by 4 * EPW experts.  Workgroups are dealt to the 8
// XCDs round-robin, so block b runs on XCD b % 8; the blocks of one row group
// (all its expert groups) are given indices of one residue and consecutive
// quotients, so they run together on one XCD and its L2 serves their reads
// of the rows after the first.
template <int EPW>
__global__ __launch_bounds__(256) void k_router_logits(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int neg = (a.E + 4 * EPW - 1) / (4 * EPW);       // expert groups
  const int j = blockIdx.x / 8;
  const int r0 = (8 * (j / neg) + (int)(blockIdx.x % 8)) * 8;
  const int e0 = ((j % neg) * 4 + wave) * EPW;
  if (r0 >= a.M || e0 >= a.E) return;
  bool rv[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) rv[r] = (r0 + r < a.M) && (a.mask == nullptr || a.mask[r0 + r] != 0);
  double acc[8][EPW];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int e = 0; e < EPW; ++e) acc[r][e] = 0.0;

  // rows past M or masked read row r0 (in range) and are never stored
  const uint16_t* xrow[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) xrow[r] = a.x + (size_t)(rv[r] ? r0 + r : r0) * a.H;
  for (int h0 = lane * 8; h0 < a.H; h0 += 512) {
    uint4 wv[EPW], xv[8];
#pragma unroll
    for (int e = 0; e < EPW; ++e)
      wv[e] = (e0 + e < a.E) ? *reinterpret_cast<const uint4*>(a.wr + (size_t)(e0 + e) * a.H + h0)
                             : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 8; ++r) xv[r] = *reinterpret_cast<const uint4*>(xrow[r] + h0);
    // element t of the chunk: each weight converted once for the 8 rows, each
    // x value once for the EPW experts; every accumulator still takes its
    // products in ascending t
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      double wd[EPW];
#pragma unroll
      for (int e = 0; e < EPW; ++e) wd[e] = (double)bf16_to_f32(u16_of(wv[e], t));
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const double xd = (double)bf16_to_f32(u16_of(xv[r], t));
#pragma unroll
        for (int e = 0; e < EPW; ++e) acc[r][e] = __builtin_fma(xd, wd[e], acc[r][e]);
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
// Pad rows get ids -1, weights 0, slot_of -1 and an empty expert bitmask.
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 256;

// k rounds of a wave-wide argmax of (score, -id) over candidates held four per
// lane (id = lane + 64 q): the k largest scores, ties to the lower id.  The
// winners are marked in picked[] and cleared from ok[].  Scores are never NaN
// (route_score maps NaN to -inf); -inf candidates still rank by id.
__device__ __forceinline__ void topk_rounds(const double (&c)[4], bool (&ok)[4], bool (&picked)[4], int k, int lane) {
  for (int j = 0; j < k; ++j) {
    double m = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (ok[q]) m = fmax(m, c[q]);
    m = wave_max_f64(m);
    int best = -1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t b = __ballot(ok[q] && c[q] == m);
      if (best < 0 && b != 0ull) best = 64 * q + __ffsll((long long)b) - 1;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q == best) { ok[q] = false; picked[q] = true; }
  }
}

__device__ void select_row(const RouteArgs& a, int row, int lane, uint32_t* lds_bits) {
  const int nwords = (a.E + 31) / 32;
  const bool real = (a.mask == nullptr || a.mask[row] != 0);
  if (!real) {
    if (lane < a.K) {
      a.ids[(size_t)row * a.K + lane] = -1;
      a.w[(size_t)row * a.K + lane] = 0.0f;
      a.slot_of[(size_t)row * a.K + lane] = -1;
    }
    if (lane < nwords) {
      a.rowbits[(size_t)row * nwords + lane] = 0u;
      if (lds_bits) lds_bits[lane] = 0u;
    }
    return;
  }
  double c[4], sg[4];
  bool ok[4], picked[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    ok[q] = e < a.E;
    picked[q] = false;
    c[q] = -INFINITY;
    sg[q] = 0.0;
    if (ok[q]) {
      const double l = a.logits[(size_t)row * a.E + e];
      route_score(l, a.bias[e], sg[q], c[q]);
    }
  }
  topk_rounds(c, ok, picked, a.K, lane);
  // Ascending id order: id = lane + 64 q, so positions follow q, then lane.
  // Each pick is pushed to lane `position` (ds_permute); lane 63 is never a
  // position (k <= 16) and takes the pushes of lanes without a pick.
  int my_e = -1;
  double my_s = 0.0;
  int base = 0;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t m = __ballot(picked[q]);
    const int pos = base + __popcll(m & below);
    const int dst = picked[q] ? pos : 63;
    const int tag = picked[q] ? (lane + 64 * q + 1) : 0;
    const uint64_t sb = (uint64_t)__double_as_longlong(sg[q]);
    const int rt = __builtin_amdgcn_ds_permute(dst * 4, tag);
    const int rlo = __builtin_amdgcn_ds_permute(dst * 4, (int)(uint32_t)sb);
    const int rhi = __builtin_amdgcn_ds_permute(dst * 4, (int)(uint32_t)(sb >> 32));
    if (rt != 0 && lane < a.K) {
      my_e = rt - 1;
      my_s = __longlong_as_double((long long)(((uint64_t)(uint32_t)rhi << 32) | (uint32_t)rlo));
    }
    if (lane < 8) {
      const uint32_t word = (uint32_t)(lane == 2 * q ? m : (lane == 2 * q + 1 ? (m >> 32) : 0ull));
      if (lane == 2 * q || lane == 2 * q + 1) {
        if (lane < nwords) {
          a.rowbits[(size_t)row * nwords + lane] = word;
          if (lds_bits) lds_bits[lane] = word;
        }
      }
    }
    base += __popcll(m);
  }
  double tot = 0.0;
  for (int j = 0; j < a.K; ++j) tot += __shfl(my_s, j, 64);     // ascending id order
  if (lane < a.K) {
    a.ids[(size_t)row * a.K + lane] = my_e;
    a.w[(size_t)row * a.K + lane] = (float)((double)a.scale * (my_s / tot));
  }
}

__global__ __launch_bounds__(256) void k_route_select(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave_id();
  if (row >= a.M) return;
  select_row(a, row, lane, nullptr);
}

// ---------------------------------------------------------------- union
// Larger steps: the rows are cut into kUChunks chunks.  (1) per chunk and
// expert, the number of rows that picked the expert; (2) one workgroup turns
// the counts into each chunk's first slot per expert, the ascending union
// with its slot and tile offsets; (3) per chunk and expert, the chunk's rows
// that picked the expert are written in ascending row order from that first
// slot, with slot_of[r, j] (j = the pick's position among the row's ascending
// ids).  The result is the same as one ordered pass over all rows.
__device__ __forceinline__ int chunk_rows(int M) { return (M + kUChunks - 1) / kUChunks; }

__global__ __launch_bounds__(kMaxExperts) void k_union_count(RouteArgs a) {
  const int c = blockIdx.x, e = threadIdx.x;
  if (e >= a.E) return;
  const int nwords = (a.E + 31) / 32;
  const int cr = chunk_rows(a.M);
  const int r0 = c * cr, r1 = min(a.M, r0 + cr);
  const uint32_t bit = 1u << (e & 31);
  int n = 0;
  for (int r = r0; r < r1; ++r) n += (a.rowbits[(size_t)r * nwords + (e >> 5)] & bit) ? 1 : 0;
  a.ucount[(size_t)c * a.E + e] = n;
}

// Inclusive scan over a workgroup of kMaxExperts threads (4 waves).
__device__ __forceinline__ uint32_t block_incl_scan256(uint32_t v, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const uint32_t x = wave_incl_scan(v, lane);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += tmp[w];
  __syncthreads();
  return x + before;
}

__global__ __launch_bounds__(kMaxExperts) void k_union_scan(RouteArgs a) {
  __shared__ uint32_t tmp[4];
  __shared__ uint32_t tot[2];
  const int e = threadIdx.x;
  const bool ok = e < a.E;
  // per-expert exclusive prefix over the chunks (kept in registers)
  int pre[kUChunks];
  int n = 0;
#pragma unroll
  for (int c = 0; c < kUChunks; ++c) {
    pre[c] = n;
    n += ok ? a.ucount[(size_t)c * a.E + e] : 0;
  }
  // across experts: first slot (32-bit scan) and union index | first tile (packed scan)
  const uint32_t nt = (uint32_t)((n + kMTile - 1) / kMTile);
  const uint32_t v1 = (uint32_t)n;
  const uint32_t v2 = (n > 0 ? 1u : 0u) | (nt << 16);
  const uint32_t i1 = block_incl_scan256(v1, tmp);
  const uint32_t i2 = block_incl_scan256(v2, tmp);
  const int off = (int)(i1 - v1);
  const int uidx = (int)((i2 - v2) & 0xFFFFu), mto = (int)((i2 - v2) >> 16);
  if (ok && n > 0) {
    a.union_ids[uidx] = e;
    a.offs[uidx] = off;
    a.mtile_offs[uidx] = mto;
  }
  if (ok) {
#pragma unroll
    for (int c = 0; c < kUChunks; ++c) a.ucount[(size_t)c * a.E + e] = off + pre[c];
  }
  if (e == kMaxExperts - 1) {
    tot[0] = i1;
    tot[1] = i2;
  }
  __syncthreads();
  if (e == 0) {
    const int nu = (int)(tot[1] & 0xFFFFu), total_mt = (int)(tot[1] >> 16), total = (int)tot[0];
    a.offs[nu] = total;
    a.mtile_offs[nu] = total_mt;
    *a.n_union = nu;
    a.sched[SCHED_NUNION] = nu;
    a.sched[SCHED_MTILES] = total_mt;
    a.sched[SCHED_SLOTS] = total;
    a.sched[SCHED_BAD] = 0;
  }
}

// Rows are taken 8 at a time: their expert bitmasks are loaded together, so
// a chunk costs one memory round trip per 8 rows instead of one per row.
constexpr int kScatterRows = 8;
constexpr int kMaskWords = kMaxExperts / 32;

__global__ __launch_bounds__(kMaxExperts) void k_union_scatter(RouteArgs a) {
  const int c = blockIdx.x, e = threadIdx.x;
  if (e >= a.E) return;
  const int nwords = (a.E + 31) / 32;
  const int cr = chunk_rows(a.M);
  const int r0 = c * cr, r1 = min(a.M, r0 + cr);
  const int wi = e >> 5;
  const uint32_t bit = 1u << (e & 31);
  int slot = a.ucount[(size_t)c * a.E + e];
  for (int rb0 = r0; rb0 < r1; rb0 += kScatterRows) {
    uint32_t m[kScatterRows][kMaskWords];
#pragma unroll
    for (int i = 0; i < kScatterRows; ++i) {
      const uint32_t* rb = a.rowbits + (size_t)min(rb0 + i, r1 - 1) * nwords;   // rows past r1: a valid row, unused
#pragma unroll
      for (int w2 = 0; w2 < kMaskWords; ++w2) m[i][w2] = rb[min(w2, nwords - 1)];
    }
#pragma unroll
    for (int i = 0; i < kScatterRows; ++i) {
      const int r = rb0 + i;
      if (r >= r1) break;
      // the row's word holding e, and the count of the row's experts in lower words
      uint32_t word = 0;
      int below = 0;
#pragma unroll
      for (int w2 = 0; w2 < kMaskWords; ++w2) {
        const uint32_t mw = w2 < nwords ? m[i][w2] : 0u;
        if (w2 < wi) below += __popc(mw);
        word = w2 == wi ? mw : word;
      }
      if (!(word & bit)) continue;
      const int j = below + __popc(word & (bit - 1u));
      a.rows[slot] = r;
      a.slot_of[(size_t)r * a.K + j] = slot;
      ++slot;
    }
  }
}

// ---------------------------------------------------------------- small steps
// For M <= 32 rows.  Logits: one workgroup per expert with one wave per row,
// the row's chunks streamed through a ring (same per-lane procedure as
// above); the kernel also stores sigmoid(l) and the biased score c.  Then one
// workgroup selects every row's top-k by rank and builds the union and the
// row lists in LDS.  The kernel boundary orders the two phases.
constexpr int kSmallRing = 4;

__device__ __forceinline__ double dot_chunk(const uint4& xv, const uint4& wv, double acc) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const double xd = (double)bf16_to_f32((uint16_t)(xw[t >> 1] >> ((t & 1) * 16)));
    const double wd = (double)bf16_to_f32((uint16_t)(ww[t >> 1] >> ((t & 1) * 16)));
    acc = __builtin_fma(xd, wd, acc);
  }
  return acc;
}

// logit l of (row r, expert e) for the calling wave (every lane gets it)
__device__ __forceinline__ double logit_dot(const RouteArgs& a, int r, int e, int lane) {
  const uint16_t* wrow = a.wr + (size_t)e * a.H + 8 * lane;
  const uint16_t* xrow = a.x + (size_t)r * a.H + 8 * lane;
  const int nch = (a.H + 511) / 512;
  uint4 wv[kSmallRing], xv[kSmallRing];
#pragma unroll
  for (int i = 0; i < kSmallRing; ++i) {
    const bool in = i < nch && 512 * i + 8 * lane < a.H;
    wv[i] = in ? *reinterpret_cast<const uint4*>(wrow + 512 * i) : make_uint4(0, 0, 0, 0);
    xv[i] = in ? *reinterpret_cast<const uint4*>(xrow + 512 * i) : make_uint4(0, 0, 0, 0);
  }
  double acc = 0.0;
  for (int i0 = 0; i0 < nch; i0 += kSmallRing) {
#pragma unroll
    for (int ii = 0; ii < kSmallRing; ++ii) {
      const int i = i0 + ii;
      if (i >= nch) break;
      if (512 * i + 8 * lane < a.H) acc = dot_chunk(xv[ii], wv[ii], acc);
      const int ni = i + kSmallRing;
      if (ni < nch && 512 * ni + 8 * lane < a.H) {
        wv[ii] = *reinterpret_cast<const uint4*>(wrow + 512 * ni);
        xv[ii] = *reinterpret_cast<const uint4*>(xrow + 512 * ni);
      }
    }
  }
  return wave_sum_f64(acc);
}

// logit of (row r, expert e) for the calling wave; stores the biased score c
// in logits and sigmoid(l) in sig (the form the small-step selection reads)
__device__ __forceinline__ void logit_row(const RouteArgs& a, int r, int e, int lane) {
  const double l = logit_dot(a, r, e, lane);
  if (lane == 0) {
    double sig, c;
    route_score(l, a.bias[e], sig, c);
    a.logits[(size_t)r * a.E + e] = c;
    a.sig[(size_t)r * a.E + e] = sig;
  }
}

// Logits of steps up to kGroupedLogitRows rows: one 8-wave block per
// (expert b % E, group of 8 rows b / E), one logit per wave, so a step of a
// few dozen rows still spreads over thousands of waves; the router row is
// re-read by each row group from L2.  Its time grows with the rows (≈ 20 µs
// at 64 rows, 83 µs at 256 for 256 experts, hidden 6144) while
// k_router_logits stays near 43 µs up to 256 rows: they meet near 128.  kRaw: store the raw logit l, as
// k_router_logits does, for k_route_select; else the score c and sigmoid(l)
// for k_select_union_small.
constexpr int kGroupedLogitRows = 128;

template <bool kRaw>
__global__ __launch_bounds__(512) void k_logits_grouped(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x % a.E;
  const int r = (blockIdx.x / a.E) * 8 + wave_id();
  if (r >= a.M || (a.mask != nullptr && a.mask[r] == 0)) return;
  if (kRaw) {
    const double l = logit_dot(a, r, e, lane);
    if (lane == 0) a.logits[(size_t)r * a.E + e] = l;
  } else {
    logit_row(a, r, e, lane);
  }
}

// The front of a split small step (M <= kSmallRows), one launch of
// kFrontWaves-wave workgroups:
//   blocks [0, E nlg)         logits of expert b % E, wave w: row 8 (b / E) + w
//                             (nlg = ceil(M / 8) row groups: one round for any M)
//   blocks [E nlg, E nlg + nq) x quantization, one (row, 128-block) per wave
//   blocks [E + nq, ...)      shared expert gate/up, one K segment of the
//                             gate or up rows of one 16-column tile per wave
//                             (fp32 partials)
// The shared expert needs no routing, so its weights stream while the router
// runs.
// Shared expert gate/up, one K segment of the gate (or the up) rows of one
// 16-column tile (item t of the segments [seg0, seg0 + nseg); items
// alternate gate and up of the same columns, and the 16 rows of one packed
// group make each load read 1 KB of contiguous memory): fp32 partials of g
// or u for every real row.  NB row halves: rows 0..15 (and 16..31 when
// NB = 2, sharing each weight fragment).
template <int NB>
__device__ __forceinline__ void shared_gu_item(const FfnArgs& f, int t, int seg0, int nseg, int lane) {
  const int c = lane & 15, kq = lane >> 4;
  const int seg = seg0 + t % nseg, it = t / nseg;
  const int gu = it & 1, n0 = (it >> 1) * 16;
  const uint8_t* wp = tile_row(gu ? f.wsu : f.wsg, (size_t)n0 + c, f.H * 2 / kBlk, kq);
  const int nst = f.H / 32;
  const int s0 = seg_begin(nst, seg, kSegSG), s1 = seg_begin(nst, seg + 1, kSegSG);
  float* out = f.part_sh + ((size_t)seg * f.M * 2 + gu) * f.Is + n0 + 4 * kq;
  const bool v0 = c < f.M && row_real(f.mask, c);
  const uint16_t* bp0 = f.x + (size_t)(v0 ? c : 0) * f.H + kq * 8;
  if (NB == 1) {
    const v4f p = bf16_chain(wp, bp0, v0, s0, s1);
    if (v0) store_f4(out + (size_t)c * 2 * f.Is, p);
  } else {
    const int r1 = kColRows + c;
    const bool v1 = r1 < f.M && row_real(f.mask, r1);
    const uint16_t* bp1 = f.x + (size_t)(v1 ? r1 : 0) * f.H + kq * 8;
    v4f p0, p1;
    bf16_chain2(wp, bp0, bp1, v0, v1, s0, s1, p0, p1);
    if (v0) store_f4(out + (size_t)c * 2 * f.Is, p0);
    if (v1) store_f4(out + (size_t)r1 * 2 * f.Is, p1);
  }
}

// Split steps, first launch: blocks [0, E nlg) logits (one block per expert
// and group of kFrontWaves rows, one row per wave); then the x quantization;
// then the shared expert's gate/up for the first half of its K segments (the
// second half runs beside the top-k in k_select_union_small).  Workgroups
// stay at 8 waves so that the logit blocks leave room on their CUs for the
// streaming shared-expert blocks.
constexpr int kFrontWaves = 8;

template <int NB>
__global__ __launch_bounds__(64 * kFrontWaves) void k_front(RouteArgs r, FfnArgs f, int nq) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int nlg = (r.M + kFrontWaves - 1) / kFrontWaves;
  const int nl = r.E * nlg;
  const int b = blockIdx.x;
  if (b < nl) {
    const int row = (b / r.E) * kFrontWaves + wave;
    if (row < r.M && (r.mask == nullptr || r.mask[row] != 0)) logit_row(r, row, b % r.E, lane);
    return;
  }
  if (b < nl + nq) {
    const int item = (b - nl) * kFrontWaves + wave;
    const int nb = f.H / kBlk;
    const int row = item / nb, blk = item % nb;
    if (row >= f.M || !row_real(f.mask, row)) return;
    const uint16_t* p = f.x + (size_t)row * f.H + blk * kBlk + 2 * lane;
    quant_pair(bf16_to_f32(p[0]), bf16_to_f32(p[1]), f.xq + (size_t)row * f.H + blk * kBlk, f.xs + (size_t)row * nb + blk,
               lane);
    return;
  }
  const int t = (b - nl - nq) * kFrontWaves + wave;
  if (f.Is == 0 || t >= (f.Is / 8) * (kSegSG / 2)) return;
  shared_gu_item<NB>(f, t, 0, kSegSG / 2, lane);
}

// Block 0 (SW waves; wave w serves rows w, w + SW, ...): top-k of every row,
// then the union and the row lists in LDS.  With do_sh, blocks >= 1 run the
// shared expert's gate/up for the second half of its K segments.  Steps of
// up to 8 rows use 8-wave workgroups, larger ones 16 (fewer rounds of rows).
template <int NB, int SW>
__global__ __launch_bounds__(64 * SW) void k_select_union_small(RouteArgs a, FfnArgs f, int do_sh) {
  __shared__ double ssig[kDecodeMaxRows][kMaxTopK];
  __shared__ int sid[kDecodeMaxRows][kMaxTopK];
  __shared__ uint32_t sbits[kDecodeMaxRows][8];
  __shared__ int soff[kMaxExperts];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  if (blockIdx.x > 0) {
    if (!do_sh) return;
    const int t = (blockIdx.x - 1) * SW + wave;
    if (t >= (f.Is / 8) * (kSegSG - kSegSG / 2)) return;
    shared_gu_item<NB>(f, t, kSegSG / 2, kSegSG - kSegSG / 2, lane);
    return;
  }
  const int nwords = (a.E + 31) / 32;
  // Phase A (row r): top-k, ids in ascending order, row bitmaps.
  for (int r = wave; r < a.M; r += SW) {
    const bool real = a.mask == nullptr || a.mask[r] != 0;
    if (real) {
      double c[4], sg[4];
      bool ok[4], picked[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        ok[q] = e < a.E;
        picked[q] = false;
        c[q] = -INFINITY;
        sg[q] = 0.0;
        if (ok[q]) {
          c[q] = a.logits[(size_t)r * a.E + e];
          sg[q] = a.sig[(size_t)r * a.E + e];
        }
      }
      topk_rounds(c, ok, picked, a.K, lane);
      // ascending id order: id = lane + 64 q, so positions follow q, then lane
      int base = 0;
      const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint64_t m = __ballot(picked[q]);
        if (picked[q]) {
          const int pos = base + __popcll(m & below);
          ssig[r][pos] = sg[q];
          sid[r][pos] = lane + 64 * q;
          a.ids[(size_t)r * a.K + pos] = lane + 64 * q;
        }
        if (lane == 2 * q || lane == 2 * q + 1) {
          const uint32_t word = (uint32_t)(lane == 2 * q ? m : (m >> 32));
          if (lane < nwords) {
            sbits[r][lane] = word;
            a.rowbits[(size_t)r * nwords + lane] = word;
          }
        }
        base += __popcll(m);
      }
    } else {
      if (lane < a.K) {
        a.ids[(size_t)r * a.K + lane] = -1;
        a.w[(size_t)r * a.K + lane] = 0.0f;
        a.slot_of[(size_t)r * a.K + lane] = -1;
      }
      if (lane < nwords) {
        sbits[r][lane] = 0u;
        a.rowbits[(size_t)r * nwords + lane] = 0u;
      }
    }
  }
  __syncthreads();
  // Phase B (last wave; lane l owns experts 4 l .. 4 l + 3): per-expert row
  // counts, then one exclusive scan of a packed word gives each expert's
  // first slot (bits 0-12), union index (bits 13-21) and first tile (22-31).
  if (wave == SW - 1) {
    uint32_t cnt[4], pk[4], run = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      cnt[i] = 0;
      if (e < a.E) {
#pragma unroll
        for (int q = 0; q < kDecodeMaxRows; ++q)
          if (q < a.M) cnt[i] += (sbits[q][e >> 5] >> (e & 31)) & 1u;
      }
      pk[i] = run;
      run += cnt[i] | ((cnt[i] > 0 ? 1u : 0u) << 13) | (((cnt[i] + kMTile - 1) / kMTile) << 22);
    }
    const uint32_t incl = wave_incl_scan(run, lane);
    const uint32_t base = incl - run;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (cnt[i] == 0) continue;
      const int e = 4 * lane + i;
      const uint32_t v = base + pk[i];
      const int off = (int)(v & 0x1FFFu), uidx = (int)((v >> 13) & 0x1FFu);
      a.union_ids[uidx] = e;
      a.offs[uidx] = off;
      a.mtile_offs[uidx] = (int)(v >> 22);
      soff[e] = off;
    }
    if (lane == 63) {
      const int nu = (int)((incl >> 13) & 0x1FFu), total = (int)(incl & 0x1FFFu), total_mt = (int)(incl >> 22);
      a.offs[nu] = total;
      a.mtile_offs[nu] = total_mt;
      *a.n_union = nu;
      a.sched[SCHED_NUNION] = nu;
      a.sched[SCHED_MTILES] = total_mt;
      a.sched[SCHED_SLOTS] = total;
      a.sched[SCHED_BAD] = 0;
    }
  }
  __syncthreads();
  // Phase C (row r, lane j = pick j): combine weight and slot.  An expert's
  // slots list its rows ascending, so row r's slot is the expert's first slot
  // plus the number of earlier rows that picked it.
  for (int r = wave; r < a.M; r += SW) {
    const bool real = a.mask == nullptr || a.mask[r] != 0;
    if (!real || lane >= a.K) continue;
    double tot = 0.0;
    for (int j = 0; j < a.K; ++j) tot += ssig[r][j];     // ascending id order
    a.w[(size_t)r * a.K + lane] = (float)((double)a.scale * (ssig[r][lane] / tot));
    const int e = sid[r][lane];
    int before = 0;
#pragma unroll
    for (int q = 0; q < kDecodeMaxRows; ++q)
      if (q < r) before += (sbits[q][e >> 5] >> (e & 31)) & 1u;
    const int slot = soff[e] + before;
    a.slot_of[(size_t)r * a.K + lane] = slot;
    a.rows[slot] = r;
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const dim3 blk(256);
  // One selection workgroup up to kSmallRows rows; above, the per-row
  // selection over many workgroups and the union kernels (faster from 25
  // rows on: 221 against 229 us for a 32-row layer step)
  if (a.M <= kSmallRows) {
    FfnArgs none;
    memset(&none, 0, sizeof(none));
    MOE_LAUNCH(KID_ROUTER_LOGITS, k_logits_grouped<false>, dim3((unsigned)(a.E * ((a.M + 7) / 8))), dim3(512), 0, s, a);
    if (a.M <= 8) {
      MOE_LAUNCH(KID_ROUTE_SMALL, (k_select_union_small<1, 8>), dim3(1), dim3(64 * 8), 0, s, a, none, 0);
    } else {
      MOE_LAUNCH(KID_ROUTE_SMALL, (k_select_union_small<1, 16>), dim3(1), dim3(64 * 16), 0, s, a, none, 0);
    }
    return hipSuccess;
  }
  if (a.M <= kGroupedLogitRows) {
    MOE_LAUNCH(KID_ROUTER_LOGITS, k_logits_grouped<true>, dim3((unsigned)(a.E * ((a.M + 7) / 8))), dim3(512), 0, s, a);
  } else {
    const long groups8 = ((a.M + 7) / 8 + 7) / 8 * 8;     // row groups, padded to a multiple of 8
    constexpr int kEpw = 8;                                 // experts per wave (32 per workgroup)
    MOE_LAUNCH(KID_ROUTER_LOGITS, k_router_logits<kEpw>, dim3((unsigned)(groups8 * ((a.E + 4 * kEpw - 1) / (4 * kEpw)))),
               blk, 0, s, a);
  }
  MOE_LAUNCH(KID_ROUTE_SELECT, k_route_select, dim3((a.M + 3) / 4), blk, 0, s, a);
  MOE_LAUNCH(KID_UNION, k_union_count, dim3(kUChunks), dim3(kMaxExperts), 0, s, a);
  MOE_LAUNCH(KID_UNION, k_union_scan, dim3(1), dim3(kMaxExperts), 0, s, a);
  MOE_LAUNCH(KID_UNION, k_union_scatter, dim3(kUChunks), dim3(kMaxExperts), 0, s, a);
  return hipSuccess;
}

hipError_t launch_front_split(const RouteArgs& r, const FfnArgs& f, hipStream_t s) {
  const int nq = (f.M * (f.H / kBlk) + kFrontWaves - 1) / kFrontWaves;
  const int nlg = (f.M + kFrontWaves - 1) / kFrontWaves;
  const int items1 = f.Is > 0 ? (f.Is / 8) * (kSegSG / 2) : 0;
  const int items2 = f.Is > 0 ? (f.Is / 8) * (kSegSG - kSegSG / 2) : 0;
  const dim3 fg((unsigned)(r.E * nlg + nq + (items1 + kFrontWaves - 1) / kFrontWaves));
  const dim3 sg8((unsigned)(1 + (items2 + 7) / 8)), sg16((unsigned)(1 + (items2 + 15) / 16));
  const int do_sh = f.Is > 0 ? 1 : 0;
  if (f.M <= 8) {
    MOE_LAUNCH(KID_FRONT, k_front<1>, fg, dim3(64 * kFrontWaves), 0, s, r, f, nq);
    MOE_LAUNCH(KID_ROUTE_SMALL, (k_select_union_small<1, 8>), sg8, dim3(64 * 8), 0, s, r, f, do_sh);
  } else if (row_halves(f.M) == 1) {
    MOE_LAUNCH(KID_FRONT, k_front<1>, fg, dim3(64 * kFrontWaves), 0, s, r, f, nq);
    MOE_LAUNCH(KID_ROUTE_SMALL, (k_select_union_small<1, 16>), sg16, dim3(64 * 16), 0, s, r, f, do_sh);
  } else {
    MOE_LAUNCH(KID_FRONT, k_front<2>, fg, dim3(64 * kFrontWaves), 0, s, r, f, nq);
    MOE_LAUNCH(KID_ROUTE_SMALL, (k_select_union_small<2, 16>), sg16, dim3(64 * 16), 0, s, r, f, do_sh);
  }
  return hipSuccess;
}

}  // namespace moe
