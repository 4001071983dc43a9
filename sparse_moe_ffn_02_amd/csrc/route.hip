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

// A pad row: ids -1, weights 0, slot_of -1, an empty expert bitmask.
__device__ void select_pad(const RouteArgs& a, int row, int lane, uint32_t* lds_bits) {
  const int nwords = (a.E + 31) / 32;
  if (lane < a.K) {
    a.ids[(size_t)row * a.K + lane] = -1;
    a.w[(size_t)row * a.K + lane] = 0.0f;
    a.slot_of[(size_t)row * a.K + lane] = -1;
  }
  if (lane < nwords) {
    a.rowbits[(size_t)row * nwords + lane] = 0u;
    if (lds_bits) lds_bits[lane] = 0u;
  }
}

// The selection of a real row from its scores: c (biased score) and sg
// (sigmoid of the logit) of expert lane + 64 q, ok[q] = expert q may be
// picked.  The k largest c among the ok experts win (ties to the lower id);
// ids ascending, weights scale * sg / sum(sg) summed in ascending id order.
__device__ void select_scored(const RouteArgs& a, int row, int lane, const double (&c)[4], const double (&sg)[4],
                              bool (&ok)[4], uint32_t* lds_bits) {
  const int nwords = (a.E + 31) / 32;
  bool picked[4] = {false, false, false, false};
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

__device__ void select_row(const RouteArgs& a, int row, int lane, uint32_t* lds_bits) {
  if (!(a.mask == nullptr || a.mask[row] != 0)) {
    select_pad(a, row, lane, lds_bits);
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
      route_score(l, a.bias[e], sg[q], c[q]);
    }
  }
  select_scored(a, row, lane, c, sg, ok, lds_bits);
}

__global__ __launch_bounds__(256) void k_route_select(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave_id();
  if (row >= a.M) return;
  select_row(a, row, lane, nullptr);
}

// ---------------------------------------------------------------- certified selection
// Steps above kCertMinRows rows (mstar PR #388 router notes: only the top-k decision and the
// picked experts' sigmoids leave the router).  The float64 logit is needed
// only where it can change the decision, so the selection is certified:
//
// 1. bf16 MFMA (fp32 accumulation) gives an estimate L of every logit and
//    S = sum |x_h| |w_h| (the same MFMA on the operands' magnitudes).  bf16
//    products are exact in fp32; any order of fp32 additions with faithful
//    rounding (error at most 2u per addition, twice round-to-nearest's)
//    leaves |L - sum x_h w_h| <= gamma S with gamma = 2 n u / (1 - 2 n u),
//    u = 2^-24, n <= H + 1 additions (the K halves are added at the end).
//    The certified path runs for H <= kCertMaxH = 8192, where
//    gamma <= 2^-10 (1 + 2^-9); the computed S is at least S / (1 + gamma).
//    So Delta = S (2^-10 (1 + 2^-8) + 2^-30) + 2^-100 covers the estimate,
//    the float64 procedure's own rounding (2^-30 S) and products below
//    fp32's normal range (2^-100).
// 2. c is non-decreasing in l, so each expert's score lies between the
//    float32 scores of L - Delta and L + Delta (float32 sigmoid, within
//    2^-22 of the float64 one), widened by 2^-19.  T = the k-th largest lower
//    end; an expert whose upper end is below T has k experts strictly above
//    it and cannot be picked.  The others are the candidates (at least k).
// 3. The candidates' logits are computed by the fixed float64 procedure of
//    k_router_logits (same bits), and the selection runs on them alone.
//    A row with a non-finite L or S takes every expert as a candidate.
// The ids and weights are therefore those of a float64 logit for every
// expert; only the number of float64 dot products changes.
//
// Two kernels: k_route_est writes L and S for 64-row x 64-expert tiles, the
// two halves of K in separate workgroups (K half 0 into the logit
// workspace, half 1 into the sigmoid workspace, each as float L [M, E] then
// float S [M, E]); k_route_cert adds the halves, certifies and selects one
// row per wave.
constexpr int kEstRows = 64;
constexpr int kEstExperts = 64;
constexpr int kEstK = 128;          // K per staged chunk
constexpr int kCertGroup = 4;       // candidate logits per pass over the row
constexpr int kCertMaxH = 8192;
// Up to this many rows every logit in float64 is as fast (measured at hidden
// 6144, 256 experts: 70 against 90 us at 256 rows, level at 384 and 512,
// 114 against 95 at 768, 136 against 97 at 1024 for the whole routing).
constexpr int kCertMinRows = 512;

__device__ __forceinline__ double cert_delta(float S) {
  return (double)S * (0x1p-10 * (1.0 + 0x1p-8) + 0x1p-30) + 0x1p-100;
}

// LDS slot of 16-byte column c (0..15) of tile row r: columns are rotated
// by the row so that the 16 rows an MFMA operand read touches, at one
// column, fall in 16 different bank groups.
__device__ __forceinline__ int est_slot(int r, int c) { return r * 16 + (c ^ (r & 15)); }

// Workgroup (row tile, expert tile): 4 waves, wave w owns rows 16 w .. 16 w + 15
// of the tile against all 64 experts (4 MFMA column blocks, L and S each).
// Operand chunks of 128 K are staged through LDS (two buffers); global loads
// run three chunks ahead in registers, so several chunks' round trips
// overlap.

// one chunk's operand pieces of a thread: 4 of x, then 4 of the router weight
struct EstStage {
  v4i p[8];
};

// Loads past the last chunk re-read the last chunk (never staged): every
// load is issued unconditionally, so the compiler's wait counts can leave the
// newer chunks in flight while an older one is staged.
__device__ __forceinline__ void est_load(EstStage& r, const uint16_t* const (&xs)[4], const uint16_t* const (&ws)[4],
                                         int ch, int nch) {
  const int c = min(ch, nch - 1);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r.p[j] = *reinterpret_cast<const v4i*>(xs[j] + c * kEstK);
    r.p[4 + j] = *reinterpret_cast<const v4i*>(ws[j] + c * kEstK);
  }
}

__device__ __forceinline__ void est_stage(const EstStage& r, v4i* sx, v4i* sw, const int (&slot)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sx[slot[j]] = r.p[j];
    sw[slot[j]] = r.p[4 + j];
  }
}

__device__ __forceinline__ void est_chunk(const v4i* sx, const v4i* sw, int ar, int kc, int lane, v4f (&accL)[4],
                                          v4f (&accS)[4]) {
  const v4i mag = {0x7FFF7FFF, 0x7FFF7FFF, 0x7FFF7FFF, 0x7FFF7FFF};
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const v4i xa = sx[est_slot(ar, 4 * st + kc)];
    const v4i xm = xa & mag;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const v4i wb = sw[est_slot(16 * b + (lane & 15), 4 * st + kc)];
      accL[b] = mfma_bf16_k32(xa, wb, accL[b]);
      accS[b] = mfma_bf16_k32(xm, wb & mag, accS[b]);
    }
  }
}

__global__ __launch_bounds__(256) void k_route_est(RouteArgs a) {
  __shared__ v4i sx[2][kEstRows * 16];
  __shared__ v4i sw[2][kEstExperts * 16];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  // jobs j = (K half, row tile); the expert tiles of one job take workgroup
  // indices of one residue mod 8, so they run on one XCD and share its L2
  // for the x rows (workgroup b runs on XCD b % 8)
  const int nte = (a.E + kEstExperts - 1) / kEstExperts;
  const int nrt = (a.M + kEstRows - 1) / kEstRows;
  const int rest = blockIdx.x >> 3;
  const int job = 8 * (rest / nte) + (int)(blockIdx.x & 7);
  if (job >= 2 * nrt) return;
  const int half = job / nrt;                                // K half
  if (half == 1 && a.H / kEstK < 2) return;
  const int r0 = (job - half * nrt) * kEstRows;
  const int e0 = (rest % nte) * kEstExperts;
  const int nall = a.H / kEstK;
  const int cb = half == 0 ? 0 : (nall + 1) / 2;            // first chunk of this half
  const int nch = (nall >= 2 ? (half == 0 ? (nall + 1) / 2 : nall / 2) : nall);
  // staging: thread t moves 16-byte pieces i = t + 256 j (j < 4) of each
  // operand: tile row i / 16, column i % 16 (rows past M read row M - 1 and
  // experts past E read expert E - 1; their results are never stored)
  const uint16_t* xsrc[4];
  const uint16_t* wsrc[4];
  int slot[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = threadIdx.x + 256 * j;
    const int r = i >> 4, c = i & 15;
    xsrc[j] = a.x + (size_t)min(r0 + r, a.M - 1) * a.H + cb * kEstK + 8 * c;
    wsrc[j] = a.wr + (size_t)min(e0 + r, a.E - 1) * a.H + cb * kEstK + 8 * c;
    slot[j] = est_slot(r, c);
  }
  // chunk c travels in stage c % 3 (three named register sets, so that no
  // set is ever indexed at run time)
  EstStage q0, q1, q2;
  est_load(q0, xsrc, wsrc, 0, nch);
  est_load(q1, xsrc, wsrc, 1, nch);
  est_load(q2, xsrc, wsrc, 2, nch);
  est_stage(q0, sx[0], sw[0], slot);
  est_load(q0, xsrc, wsrc, 3, nch);
  __syncthreads();
  v4f accL[4], accS[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    accL[b] = v4f{0.f, 0.f, 0.f, 0.f};
    accS[b] = accL[b];
  }
  const int ar = 16 * wave + (lane & 15);      // A row of this lane in the tile
  const int kc = lane >> 4;                    // 8-element K column within a 32-step
  // chunk ch: multiply the staged buffer, stage chunk ch + 1 (held in NXT),
  // refill NXT with chunk ch + 4.  In the main loop every step runs whole,
  // with no branch around its loads (so the compiler's wait counts leave two
  // chunks in flight); staging past the last chunk writes the buffer nobody
  // reads any more.  The last nch % 3 chunks take guarded steps.
#define MOE_EST_STEP(ch, NXT)                                                  \
  est_chunk(sx[(ch) & 1], sw[(ch) & 1], ar, kc, lane, accL, accS);             \
  est_stage(NXT, sx[((ch) + 1) & 1], sw[((ch) + 1) & 1], slot);                \
  est_load(NXT, xsrc, wsrc, (ch) + 4, nch);                                    \
  __syncthreads();
  const int nmain = nch - nch % 3;
  for (int c0 = 0; c0 < nmain; c0 += 3) {
    MOE_EST_STEP(c0, q1)
    MOE_EST_STEP(c0 + 1, q2)
    MOE_EST_STEP(c0 + 2, q0)
  }
  if (nmain < nch) {
    MOE_EST_STEP(nmain, q1)
  }
  if (nmain + 1 < nch) {
    MOE_EST_STEP(nmain + 1, q2)
  }
#undef MOE_EST_STEP
  float* estL = reinterpret_cast<float*>(half == 0 ? a.logits : a.sig);
  float* estS = estL + (size_t)a.M * a.E;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const v4f l = settle_bf16(accL[b]);
    const v4f sm = settle_bf16(accS[b]);
    const int e = e0 + 16 * b + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 16 * wave + 4 * (lane >> 4) + i;
      if (r < a.M && e < a.E) {
        estL[(size_t)r * a.E + e] = l[i];
        estS[(size_t)r * a.E + e] = sm[i];
      }
    }
  }
}

// id of the p-th set bit over the four 64-bit masks (q-major), or -1
__device__ __forceinline__ int nth_candidate(const uint64_t (&m)[4], int p) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = __popcll(m[q]);
    if (p < c) {
      uint64_t b = m[q];
      for (int i = 0; i < p; ++i) b &= b - 1ull;
      return 64 * q + __ffsll((long long)b) - 1;
    }
    p -= c;
  }
  return -1;
}

// The k-th largest of v over the ok entries (expert lane + 64 q), counted
// with multiplicity: k rounds of a wave maximum, each removing one holder.
__device__ __forceinline__ float kth_largest(const float (&v)[4], const bool (&ok)[4], int k, int lane) {
  bool left[4] = {ok[0], ok[1], ok[2], ok[3]};
  float m = -INFINITY;
  for (int j = 0; j < k; ++j) {
    float mm = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (left[q]) mm = fmaxf(mm, v[q]);
    m = wave_max(mm);
    bool done = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t b = __ballot(left[q] && v[q] == m);
      if (!done && b != 0ull) {
        if (lane == __ffsll((long long)b) - 1) left[q] = false;
        done = true;
      }
    }
  }
  return m;
}

// One wave per row: the score intervals from L and S, the threshold, the
// candidates' float64 logits, then the selection over the candidates.  The
// row x is parked in LDS (each lane keeps the 16-byte pieces it reads back,
// so no wave sync is needed); the candidates' weight chunks are loaded three
// chunks ahead, every load unconditional (clamped addresses) so that the
// compiler's wait counts keep the next chunks in flight.
__device__ __forceinline__ void cert_wload(uint4 (&w)[kCertGroup], const uint16_t* const (&wrow)[kCertGroup], int i,
                                           int lane, int H) {
  const int h = min(512 * i + 8 * lane, H - 8);
#pragma unroll
  for (int j = 0; j < kCertGroup; ++j) w[j] = *reinterpret_cast<const uint4*>(wrow[j] + h);
}

__device__ __forceinline__ void cert_chunk(double (&acc)[kCertGroup], const uint4 (&w)[kCertGroup], const uint4* sxr,
                                           int i, int lane, int H, int ng) {
  if (512 * i + 8 * lane >= H) return;
  const uint4 xv = sxr[64 * i + lane];
  double xd[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) xd[t] = (double)bf16_to_f32(u16_of(xv, t));
#pragma unroll
  for (int j = 0; j < kCertGroup; ++j) {
    if (j >= ng) break;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[j] = __builtin_fma(xd[t], (double)bf16_to_f32(u16_of(w[j], t)), acc[j]);
  }
}

__global__ __launch_bounds__(256, 3) void k_route_cert(RouteArgs a) {
  extern __shared__ uint4 cert_x[];          // [4 waves][H / 8]
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int row = blockIdx.x * 4 + wave;
  if (row >= a.M) return;
  if (!(a.mask == nullptr || a.mask[row] != 0)) {
    select_pad(a, row, lane, nullptr);
    return;
  }
  const int nch = (a.H + 511) / 512;
  uint4* sxr = cert_x + (size_t)wave * (a.H / 8);
  {
    // all chunks of the row in one round trip (addresses clamped into the row)
    constexpr int kMaxCh = kCertMaxH / 512;
    const uint16_t* xrow = a.x + (size_t)row * a.H;
    uint4 xv[kMaxCh];
#pragma unroll
    for (int i = 0; i < kMaxCh; ++i)
      xv[i] = *reinterpret_cast<const uint4*>(xrow + min(512 * i + 8 * lane, a.H - 8));
#pragma unroll
    for (int i = 0; i < kMaxCh; ++i)
      if (512 * i + 8 * lane < a.H) sxr[64 * i + lane] = xv[i];
  }
  const float* estL = reinterpret_cast<const float*>(a.logits) + (size_t)row * a.E;
  const float* estS = estL + (size_t)a.M * a.E;
  const bool halves = a.H / kEstK >= 2;
  const float* estL1 = reinterpret_cast<const float*>(a.sig) + (size_t)row * a.E;
  const float* estS1 = estL1 + (size_t)a.M * a.E;
  // score bounds in float32: v = L -+ Delta rounded outward, sigmoid in
  // float32 (within 2^-22 of the float64 sigmoid), the bias added, and the
  // result widened by 2^-19 and rounded outward
  float lo[4], hi[4];
  bool ok[4];
  bool bad = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    ok[q] = e < a.E;
    lo[q] = -INFINITY;
    hi[q] = -INFINITY;
    if (ok[q]) {
      const float L = halves ? estL[e] + estL1[e] : estL[e];
      const float S = halves ? estS[e] + estS1[e] : estS[e];
      if (!(isfinite(L) && isfinite(S))) bad = true;
      const double d = cert_delta(S);
      const float vlo = __double2float_rd((double)L - d), vhi = __double2float_ru((double)L + d);
      const float slo = 1.0f / (1.0f + expf(-vlo)), shi = 1.0f / (1.0f + expf(-vhi));
      lo[q] = __double2float_rd((double)slo + (double)a.bias[e] - 0x1p-19);
      hi[q] = __double2float_ru((double)shi + (double)a.bias[e] + 0x1p-19);
    }
  }
  bad = __ballot(bad) != 0ull;
  const float T = kth_largest(lo, ok, a.K, lane);      // the k-th largest lower end
  uint64_t cm[4];
  int n = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    cm[q] = __ballot(ok[q] && (bad || hi[q] >= T));
    n += __popcll(cm[q]);
  }
  // float64 logits of the candidates, kCertGroup per pass over the row, by
  // the fixed procedure of k_router_logits
  double c[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, sg[4] = {0.0, 0.0, 0.0, 0.0};
  for (int g0 = 0; g0 < n; g0 += kCertGroup) {
    const int ng = min(kCertGroup, n - g0);
    int eg[kCertGroup];
    const uint16_t* wrow[kCertGroup];
#pragma unroll
    for (int j = 0; j < kCertGroup; ++j) {
      eg[j] = j < ng ? nth_candidate(cm, g0 + j) : -1;
      wrow[j] = a.wr + (size_t)(eg[j] >= 0 ? eg[j] : 0) * a.H;
    }
    double acc[kCertGroup];
#pragma unroll
    for (int j = 0; j < kCertGroup; ++j) acc[j] = 0.0;
    // three chunks in flight: chunk i travels in stage i % 3
    uint4 w0[kCertGroup], w1[kCertGroup], w2[kCertGroup];
    cert_wload(w0, wrow, 0, lane, a.H);
    cert_wload(w1, wrow, min(1, nch - 1), lane, a.H);
    cert_wload(w2, wrow, min(2, nch - 1), lane, a.H);
    for (int i = 0; i < nch; i += 3) {
      cert_chunk(acc, w0, sxr, i, lane, a.H, ng);
      cert_wload(w0, wrow, min(i + 3, nch - 1), lane, a.H);
      if (i + 1 < nch) cert_chunk(acc, w1, sxr, i + 1, lane, a.H, ng);
      cert_wload(w1, wrow, min(i + 4, nch - 1), lane, a.H);
      if (i + 2 < nch) cert_chunk(acc, w2, sxr, i + 2, lane, a.H, ng);
      cert_wload(w2, wrow, min(i + 5, nch - 1), lane, a.H);
    }
#pragma unroll
    for (int j = 0; j < kCertGroup; ++j) {
      if (j >= ng) break;
      const double l = wave_sum_f64(acc[j]);
      double sgj, cj;
      route_score(l, a.bias[eg[j]], sgj, cj);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (eg[j] == lane + 64 * q) {
          c[q] = cj;
          sg[q] = sgj;
        }
    }
  }
  bool cand[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) cand[q] = ((cm[q] >> lane) & 1ull) != 0ull;
  select_scored(a, row, lane, c, sg, cand, nullptr);
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
constexpr int kSmallRing = 6;   // chunks in flight: two round trips for a hidden-6144 row (4: 105.4, 6: 104.6 us span-8)

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
    MOE_LAUNCH(KID_ROUTE_SELECT, k_route_select, dim3((a.M + 3) / 4), blk, 0, s, a);
  } else if (a.H > kCertMaxH || a.M <= kCertMinRows) {
    const long groups8 = ((a.M + 7) / 8 + 7) / 8 * 8;     // row groups, padded to a multiple of 8
    constexpr int kEpw = 8;                                 // experts per wave (32 per workgroup)
    MOE_LAUNCH(KID_ROUTER_LOGITS, k_router_logits<kEpw>, dim3((unsigned)(groups8 * ((a.E + 4 * kEpw - 1) / (4 * kEpw)))),
               blk, 0, s, a);
    MOE_LAUNCH(KID_ROUTE_SELECT, k_route_select, dim3((a.M + 3) / 4), blk, 0, s, a);
  } else {
    const int nte = (a.E + kEstExperts - 1) / kEstExperts;
    const int jobs8 = (2 * ((a.M + kEstRows - 1) / kEstRows) + 7) / 8;     // (K half, row tile) jobs / 8
    MOE_LAUNCH(KID_ROUTER_LOGITS, k_route_est, dim3((unsigned)(8 * jobs8 * nte)), blk, 0, s, a);
    MOE_LAUNCH(KID_ROUTE_SELECT, k_route_cert, dim3((unsigned)((a.M + 3) / 4)), blk, (size_t)4 * a.H * 2, s, a);
  }
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
