// Tiled grouped GEMMs for steps that do not take the split small-step path.
//
// A workgroup of eight waves computes one tile of kTM = 128 slots (routed
// experts) or rows (shared expert) by the tile's output columns:
//   gate/up: 128 h columns, i.e. 128 gate rows and 128 up rows of the weights;
//   down:    256 columns of H (shared expert) or 512 (routed experts).
// Each wave owns 32 weight rows (two 16-row MFMA tiles; for gate/up the gate
// and the up rows of the same 16 h columns; 64 rows in the routed down tiles,
// see the wide tiles below), streams them from global memory
// straight into MFMA operand registers two K stages ahead, and applies them to
// all 128 slots (eight 16-column MFMA tiles).  The tile's activation rows,
// which all eight waves read, are staged through four LDS buffers with one
// barrier per two K stages (tile_gemm, wide_gemm).
// With at least 8 slot (or row) tiles, all column tiles of one tile are
// numbered to run on one XCD, one after another, so the tile's activation
// rows are read from HBM once and from that XCD's L2 by the other column
// tiles (xcd_tile, range_tile below).
//
// Every output element follows the same procedure as in the small-step
// kernels: one fp8 16x16x128 MFMA per 128-deep K-block scaled into a fp32
// chain (or bf16 16x16x32 MFMAs accumulating in the chain), one chain per K
// segment, segments added in order.  So a row's bits do not depend on the
// tile, the tile shape or the other rows of the step.  The gate/up epilogue
// forms h = silu(G) U and requantizes each 1x128 block of h (the block is the
// tile's column range); the shared-expert epilogue rounds h to bf16.
#include "moe_chains.h"

namespace moe {

constexpr int kTM = kMTile;                // slots (rows) per tile
constexpr int kStageBytes = 128;           // bytes of one row per K stage
constexpr int kLdsRow = kStageBytes + 16;  // padded LDS row: the 16 lanes of a fragment read hit distinct banks
constexpr int kWaves = 8;
constexpr int kTileThreads = 64 * kWaves;
constexpr int kNA = 2;                     // 16-row weight tiles per wave
constexpr int kNB = kTM / 16;              // 16-column slot tiles per wave
// Activation staging: each 16-byte load instruction of a wave covers 8 whole
// 128-byte rows (8 threads per row); thread t loads part t % 8 of rows
// t / 8 + kBRowStep * i.
constexpr int kBVec = kStageBytes * kTM / kTileThreads / 16;   // 16-byte loads per thread per stage
constexpr int kBRowStep = kTileThreads / 8;                    // rows between a thread's loads

// Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8), each XCD with its own L2.  A range of workgroups starting at a
// multiple of 8 maps its index r to (row tile, column tile) so that all column
// tiles of one row tile share r % 8, i.e. one XCD, and follow each other on
// it: r = 8 (q ncols + n) + x is row tile 8 q + x, column tile n.  The row
// tile's activations are then read from HBM once and from that L2 by the
// other column tiles.  Ranges are sized for a multiple of 8 row tiles; indices
// past the real row tiles return row tile >= nrows.
constexpr int kXcds = 8;

__host__ __device__ inline int xcd_rows(int nrows) { return (nrows + kXcds - 1) / kXcds * kXcds; }

__device__ __forceinline__ void xcd_tile(int r, int ncols, int& row, int& col) {
  const int x = r % kXcds, rest = r / kXcds;
  col = rest % ncols;
  row = (rest / ncols) * kXcds + x;
}

// The XCD grouping pays when every XCD gets row tiles of its own.  With
// fewer than kXcdMinRows row tiles it would crowd the column tiles of the
// few row tiles onto as many XCDs (a step of one row tile would run on one
// XCD of eight), so the range is then dealt out in plain order: index r is
// row tile r / ncols, column tile r % ncols, and the workgroups of one row
// tile spread over all XCDs.  The range keeps its size (xcd_rows(nrows) *
// ncols, a multiple of 8); indices past the real tiles return row >= nrows.
constexpr int kXcdMinRows = 8;

__device__ __forceinline__ void range_tile(int r, int nrows, int ncols, int& row, int& col) {
  if (nrows >= kXcdMinRows) {
    xcd_tile(r, ncols, row, col);
  } else {
    row = r / ncols;
    col = r % ncols;
  }
}

struct TileIn {
  const uint8_t* a[kNA]; // per lane: packed-tile address (tile_row) of each of the wave's A tiles, stage 0
  const float* sw[kNA];  // fp8: weight scales of each A tile, indexed by K-block
  const uint8_t* b[kBVec];  // per thread: 16-byte part tid % 8 of activation row tid / 8 + kBRowStep i (always valid)
  const float* bs;       // fp8: activation scales of row tid (threads < kTM), indexed by K-block (always valid)
  bool bok[kBVec];       // the thread's activation rows are real (else they contribute zeros)
  bool bsok;             // the thread's scale row is real (else zero)
  int nstage;            // K stages of 128 bytes
  int nseg;              // K segments (fp8: over K-blocks; bf16: over 32-deep K steps)
};

constexpr int kLdsStages = 4;              // LDS activation stage buffers

struct TileLds {
  uint8_t b[kLdsStages][kTM * kLdsRow];
  float s[kLdsStages][kTM];
};

// An LDS float pointer the compiler cannot see through.  Reads at constant
// offsets from it become one base register with immediate offsets; from a
// base it can see through, the compiler materializes one address register per
// (stage buffer, slot tile) and spills them.
typedef __attribute__((address_space(3))) const float lds_cf;

__device__ __forceinline__ lds_cf* opaque_lds(const void* p) {
  lds_cf* r = (lds_cf*)p;
  asm volatile("" : "+v"(r));
  return r;
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Weight fragments of one stage, with the fp8 weight scales of that K-block.
struct AStage {
  v8i v[kNA];
  float s[kNA];
};

template <bool kFp8>
__device__ __forceinline__ void load_a(AStage& dst, const TileIn& in, int st) {
#pragma unroll
  for (int t = 0; t < kNA; ++t) {
    if (kFp8) dst.s[t] = in.sw[t][st];
    dst.v[t] = load_frag(in.a[t] + (size_t)st * kTile);
  }
}

struct BStage {
  uint4 v[kBVec];
  float s;
};

// Loads are unconditional (rows out of range read a valid row) so that no
// branch separates a load from its wait and the compiler's in-order load
// counting stays exact; rows out of range are zeroed when the registers are
// written to LDS after the stage's compute, so the loaded values are not
// touched early.
template <bool kFp8>
__device__ __forceinline__ void load_b(BStage& r, const TileIn& in, int st) {
#pragma unroll
  for (int i = 0; i < kBVec; ++i) r.v[i] = ld16(in.b[i] + (size_t)st * kStageBytes);
  if (kFp8) r.s = in.bs[st];
}

template <bool kFp8>
__device__ __forceinline__ void store_b(TileLds& L, int buf, const BStage& r, const TileIn& in) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kBVec; ++i) {
    uint8_t* d = &L.b[buf][(tid / 8 + kBRowStep * i) * kLdsRow + (tid % 8) * 16];
    const uint32_t keep = in.bok[i] ? 0xFFFFFFFFu : 0u;  // value select (a select of lvalues would force memory)
    const uint4 v = r.v[i];
    *reinterpret_cast<uint4*>(d) = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
  }
  if (kFp8 && tid < kTM) {
    const float sv = r.s;
    L.s[buf][tid] = in.bsok ? sv : 0.0f;
  }
}

// All four results of a group of MFMAs wait out the MFMA latency together
// before any vector-ALU read (see settle_fp8).
__device__ __forceinline__ void settle4(v4f& p0, v4f& p1, v4f& p2, v4f& p3) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(p0), "+v"(p1), "+v"(p2), "+v"(p3));
}

__device__ __forceinline__ v4f mfma_fp8_raw(const v8i& a, const v8i& b) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

struct SegState {
  int seg, end, nunits, nseg;
};

using Acc = v4f[kNA][kNB];

// Close every K segment that ends at or before `done` units: tot = acc for
// the first segment, tot = tot + acc after it.  Further segments ending at the
// same point are empty and add zeros (tot + 0, once: repeats change nothing).
// The loops over the arrays stay free of data-dependent trip counts so that
// acc and tot stay in registers.
template <bool kFp8>
__device__ __forceinline__ void close_segments(SegState& g, int done, Acc& acc, Acc& tot) {
  if (g.seg >= g.nseg || g.end > done) return;
  const bool first = g.seg == 0;
#pragma unroll
  for (int t = 0; t < kNA; ++t)
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const v4f v = kFp8 ? acc[t][b] : settle_bf16(acc[t][b]);
      tot[t][b] = first ? v : add4(tot[t][b], v);
      acc[t][b] = v4f{0.f, 0.f, 0.f, 0.f};
    }
  ++g.seg;
  g.end = seg_begin(g.nunits, g.seg + 1, g.nseg);
  bool empty = false;
  while (g.seg < g.nseg && g.end <= done) {
    ++g.seg;
    g.end = seg_begin(g.nunits, g.seg + 1, g.nseg);
    empty = true;
  }
  if (empty) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kNA; ++t)
#pragma unroll
      for (int b = 0; b < kNB; ++b) tot[t][b] = add4(tot[t][b], z);
  }
}

// MFMA B fragments (and activation scales) of slot tiles b and b + 1 from an
// LDS activation stage: lane (q, c) takes 32 bytes of row 16 b + c at 32 q;
// ls points at the stage's scale of row c.
__device__ __forceinline__ void lds_frag_pair(const uint8_t* lb, lds_cf* ls, int b, int c, int q, v8i (&x)[2],
                                              float (&s)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint8_t* src = lb + (16 * (b + j) + c) * kLdsRow + q * 32;
    const uint4 lo = ld16(src), hi = ld16(src + 16);
    x[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    s[j] = ls[16 * (b + j)];
  }
}

// One K stage on LDS buffer `buf` with A fragments `a`.  Only slot tiles
// 0 .. NL - 1 are computed; the caller picks NL >= the tile's slot tiles
// holding rows (the rest hold zeros and are never stored).
template <bool kFp8, int NL>
__device__ __forceinline__ void tile_stage(const TileLds& L, int buf, const AStage& as, int st, Acc& acc, Acc& tot,
                                           SegState& g) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const v8i(&a)[kNA] = as.v;
  if (kFp8) {
    const float sw0 = as.s[0], sw1 = as.s[1];
    // The fragments of the next pair of slot tiles are read from LDS while
    // the MFMAs of this pair run, so the LDS latency is not waited out once
    // per pair.
    v8i xb[2], xn[2];
    float sx[2], sxn[2];
    lds_cf* ls = opaque_lds(&L.s[0][c]) + buf * kTM;
    lds_frag_pair(L.b[buf], ls, 0, c, q, xb, sx);
#pragma unroll
    for (int b = 0; b < NL; b += 2) {
      if (b + 2 < NL) lds_frag_pair(L.b[buf], ls, b + 2, c, q, xn, sxn);
      v4f p0 = mfma_fp8_raw(a[0], xb[0]), p1 = mfma_fp8_raw(a[1], xb[0]);
      v4f p2 = mfma_fp8_raw(a[0], xb[1]), p3 = mfma_fp8_raw(a[1], xb[1]);
      settle4(p0, p1, p2, p3);
      scale_acc(acc[0][b], p0, sx[0], sw0);
      scale_acc(acc[1][b], p1, sx[0], sw1);
      scale_acc(acc[0][b + 1], p2, sx[1], sw0);
      scale_acc(acc[1][b + 1], p3, sx[1], sw1);
      asm volatile("" : "+v"(acc[0][b]), "+v"(acc[1][b]), "+v"(acc[0][b + 1]), "+v"(acc[1][b + 1]));
      if (b + 2 < NL) {
        xb[0] = xn[0];
        xb[1] = xn[1];
        sx[0] = sxn[0];
        sx[1] = sxn[1];
      }
      __builtin_amdgcn_sched_barrier(0);     // one pair in flight, the next pair's fragments loading
    }
    close_segments<true>(g, st + 1, acc, tot);
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // the next slot tile's fragment is read while this tile's MFMAs run
      uint4 xv = ld16(&L.b[buf][c * kLdsRow + j * 64 + q * 16]);
#pragma unroll
      for (int b = 0; b < NL; ++b) {
        uint4 xnv = xv;
        if (b + 1 < NL) xnv = ld16(&L.b[buf][(16 * (b + 1) + c) * kLdsRow + j * 64 + q * 16]);
        const v4i xb = {(int)xv.x, (int)xv.y, (int)xv.z, (int)xv.w};
#pragma unroll
        for (int t = 0; t < kNA; ++t) {
          const v4i ah = {a[t][4 * j], a[t][4 * j + 1], a[t][4 * j + 2], a[t][4 * j + 3]};
          acc[t][b] = mfma_bf16_k32(ah, xb, acc[t][b]);
        }
        xv = xnv;
        __builtin_amdgcn_sched_barrier(0);
      }
      close_segments<false>(g, 2 * st + j + 1, acc, tot);
    }
  }
}

// The K loop of one tile: tot[t][b] = the element values of A tile t by slot
// tile b (lane layout of the 16x16 MFMA output).  Weight fragments and their
// block scales are loaded two stages ahead into registers.  The activation
// rows go through four LDS stage buffers: stages s, s + 1 (s even) read
// buffers s % 4, (s + 1) % 4 and write stages s + 2, s + 3 into the other
// two, each stage loading the rows it writes at its start (its compute
// covers their latency), then one barrier closes the pair.  With a double
// buffer every stage needs a barrier, and the two waves of a SIMD run in
// lockstep: the faster one idles at every barrier.
template <bool kFp8, int NL = kNB>
__device__ __forceinline__ void tile_gemm(const TileIn& in, TileLds& L, Acc& tot) {
  static_assert(NL % 2 == 0 && NL >= 2 && NL <= kNB, "slot tiles in pairs");
  // keeps the first loads below the caller's branch between instantiations
  // (hoisted above it they stretch live ranges across all of them)
  asm volatile("" ::: "memory");
  Acc acc;
#pragma unroll
  for (int t = 0; t < kNA; ++t)
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      acc[t][b] = v4f{0.f, 0.f, 0.f, 0.f};
      tot[t][b] = acc[t][b];
    }
  SegState g;
  g.seg = 0;
  g.nseg = in.nseg;
  g.nunits = kFp8 ? in.nstage : 2 * in.nstage;
  g.end = seg_begin(g.nunits, 1, g.nseg);
  close_segments<kFp8>(g, 0, acc, tot);
  const int n = in.nstage;
  AStage ar0, ar1;                 // weight ring (two stages)
  BStage br0, br1;
  // Refills past the last stage reload stage n - 1 (in range, unused): every
  // step issues the same loads, with no branch around them.
  const int last = n - 1;
  load_a<kFp8>(ar0, in, 0);
  load_a<kFp8>(ar1, in, min(1, last));
  load_b<kFp8>(br0, in, 0);
  load_b<kFp8>(br1, in, min(1, last));
  store_b<kFp8>(L, 0, br0, in);
  store_b<kFp8>(L, 1, br1, in);
  __syncthreads();
  // Stage st0 + D on buffer D (st0 a multiple of 4): load the activations of
  // stage st + 2, compute, refill the weight register set AR two stages
  // ahead, write stage st + 2 to buffer (D + 2) % 4; a barrier after odd D.
  // Unrolled by four (compile-time buffer indices), the remaining steps
  // guarded after the loop.
#define MOE_TILE_STEP(D, AR, SYNC)                             \
  {                                                            \
    const int st = st0 + (D);                                  \
    load_b<kFp8>(br0, in, min(st + 2, last));                  \
    tile_stage<kFp8, NL>(L, (D), AR, st, acc, tot, g);         \
    load_a<kFp8>(AR, in, min(st + 2, last));                   \
    store_b<kFp8>(L, ((D) + 2) & 3, br0, in);                  \
    if (SYNC) __syncthreads();                                 \
  }
  int st0 = 0;
  for (; st0 + 4 <= n; st0 += 4) {
    MOE_TILE_STEP(0, ar0, false)
    MOE_TILE_STEP(1, ar1, true)
    MOE_TILE_STEP(2, ar0, false)
    MOE_TILE_STEP(3, ar1, true)
  }
  if (st0 < n) MOE_TILE_STEP(0, ar0, false)
  if (st0 + 1 < n) MOE_TILE_STEP(1, ar1, true)
  if (st0 + 2 < n) MOE_TILE_STEP(2, ar0, false)
#undef MOE_TILE_STEP
}

// ---------------------------------------------------------------- fp8 wide tiles
// The routed down tiles (one K segment) give each wave a wider register tile:
// 4 weight tiles (64 weight rows) by the 8 slot tiles, so every activation
// fragment read from LDS feeds 4 MFMAs instead of 2, the LDS bytes and
// barriers per MFMA halve, and each wave keeps twice the weight bytes in
// flight.  Its 128 accumulators leave no room for a second (segment) set, so
// the form serves the one-segment down GEMM; gate/up (two segments) keeps the
// tile above.
constexpr int kWA = 4;                                                // 16-row weight tiles per wave
constexpr int kWBV = kTM * kStageBytes / kTileThreads / 16;           // 16-byte activation loads per thread per K-block
constexpr int kWBRow = kTileThreads / 8;                              // rows between a thread's loads
constexpr int kWBuf = kTM * kLdsRow;                                  // one activation stage in LDS
constexpr int kWLdsB = kLdsStages * kWBuf;                           // stage buffers
constexpr int kWLds = kWLdsB + kLdsStages * kTM * (int)sizeof(float); // + the activation scales

struct WideIn {
  const uint8_t* a;       // per lane: packed-tile address of weight tile 0 at K-block 0
  long astep;             // bytes from one weight tile (16 rows) to the next
  const float* sw;        // weight scales of the wave's 64 rows (one 128-row block), indexed by K-block
  // Activation rows and scales as one uniform base plus 32-bit per-thread
  // offsets (fewer registers than 64-bit pointers; the offsets stay below
  // 2^32 for every supported row count).
  const uint8_t* bbase;
  uint32_t boff[kWBV];    // per thread: byte offset of its activation row part at K-block 0 (a valid row)
  bool bok[kWBV];         // those rows are real (else they contribute zeros)
  const float* sbase;
  uint32_t soff;          // scale row of thread tid < kTM, in floats (a valid row)
  bool bsok;
  int nkb;                // K-blocks
};

struct WStage {
  v8i v[kWA];
  float s;
};

struct WB {
  uint4 v[kWBV];
  float s;
};

using WAcc = v4f[kWA][kNB];

__device__ __forceinline__ void wide_load_a(WStage& d, const WideIn& in, int kb) {
  d.s = in.sw[kb];
#pragma unroll
  for (int t = 0; t < kWA; ++t) d.v[t] = load_frag(in.a + t * in.astep + (long)kb * kTile);
}

__device__ __forceinline__ void wide_load_b(WB& r, const WideIn& in, int kb) {
#pragma unroll
  for (int i = 0; i < kWBV; ++i) r.v[i] = ld16(in.bbase + (in.boff[i] + (uint32_t)kb * kStageBytes));
  r.s = in.sbase[in.soff + (uint32_t)kb];
}

// Write a thread's activation registers (and scale) to stage buffer `buf`;
// rows out of range become zero codes and a zero scale.
__device__ __forceinline__ void wide_store_b(uint8_t* smem, int buf, const WB& r, const WideIn& in) {
  const int tid = threadIdx.x;
  uint8_t* base = smem + buf * kWBuf;
#pragma unroll
  for (int i = 0; i < kWBV; ++i) {
    const uint32_t keep = in.bok[i] ? 0xFFFFFFFFu : 0u;
    const uint4 v = r.v[i];
    *reinterpret_cast<uint4*>(base + (tid / 8 + kWBRow * i) * kLdsRow + (tid % 8) * 16) =
        make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
  }
  if (tid < kTM) {
    const float sv = r.s;
    reinterpret_cast<float*>(smem + kWLdsB)[buf * kTM + tid] = in.bsok ? sv : 0.0f;
  }
}

// One K-block on stage buffer `buf`: 4 MFMAs for each of slot tiles
// 0 .. NL - 1 (32 for a full tile), each partial scaled into its chain as in
// every other kernel.  The caller picks NL >= the tile's slot tiles holding
// real rows (the rest hold zero codes and are never stored).
template <int NL>
__device__ __forceinline__ void wide_stage(const uint8_t* smem, int buf, const WStage& as, WAcc& acc) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const uint8_t* lb = smem + buf * kWBuf;
  lds_cf* ls = opaque_lds(smem + kWLdsB + c * sizeof(float)) + buf * kTM;
  const float sw = as.s;
  // the next slot tile's fragment is read from LDS while this tile's MFMAs run
  auto frag = [&](int b, v8i& x, float& sx) {
    const uint8_t* src = lb + (16 * b + c) * kLdsRow + q * 32;
    const uint4 lo = ld16(src), hi = ld16(src + 16);
    x = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    sx = ls[16 * b];
  };
  v8i xb, xn;
  float sx, sxn;
  frag(0, xb, sx);
#pragma unroll
  for (int b = 0; b < NL; ++b) {
    if (b + 1 < NL) frag(b + 1, xn, sxn);
    v4f p0 = mfma_fp8_raw(as.v[0], xb), p1 = mfma_fp8_raw(as.v[1], xb);
    v4f p2 = mfma_fp8_raw(as.v[2], xb), p3 = mfma_fp8_raw(as.v[3], xb);
    settle4(p0, p1, p2, p3);
    scale_acc(acc[0][b], p0, sx, sw);
    scale_acc(acc[1][b], p1, sx, sw);
    scale_acc(acc[2][b], p2, sx, sw);
    scale_acc(acc[3][b], p3, sx, sw);
    // pin the chain updates here: left free, the compiler sinks them below
    // later MFMAs and keeps every partial of the K-block live at once
    asm volatile("" : "+v"(acc[0][b]), "+v"(acc[1][b]), "+v"(acc[2][b]), "+v"(acc[3][b]));
    if (b + 1 < NL) {
      xb = xn;
      sx = sxn;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The K loop of one wide tile: acc = the element chains over all K-blocks.
// Weight fragments are loaded two K-blocks ahead into registers.  Four LDS
// stage buffers: K-blocks s, s + 1 (s even) read buffers s % 4, (s + 1) % 4
// and write K-blocks s + 2, s + 3 into the other two, then one barrier; a
// thread's activation rows for the K-block it writes are loaded into
// registers at the start of the step, so the compute covers their latency.  Loads past the last K-block reload it (valid, unused),
// so every step issues the same loads with no branch around them.
template <int NL>
__device__ __forceinline__ void wide_gemm(const WideIn& in, uint8_t* smem, WAcc& acc) {
  const int n = in.nkb, last = n - 1;
  // keeps the K loop's first loads below the caller's branch between
  // instantiations: hoisted above it (they are the same loads in each), they
  // stretch live ranges across every instantiation and the kernel spills
  asm volatile("" ::: "memory");
#pragma unroll
  for (int t = 0; t < kWA; ++t)
#pragma unroll
    for (int b = 0; b < kNB; ++b) acc[t][b] = v4f{0.f, 0.f, 0.f, 0.f};
  WStage ar0, ar1;
  WB br;
  wide_load_a(ar0, in, 0);
  wide_load_a(ar1, in, min(1, last));
  wide_load_b(br, in, 0);
  wide_store_b(smem, 0, br, in);
  wide_load_b(br, in, min(1, last));
  wide_store_b(smem, 1, br, in);
  __syncthreads();
  // K-block s0 + D on buffer D (s0 a multiple of 4): load the activation rows
  // of K-block st + 2, compute, refill AR, write st + 2 to buffer (D + 2) % 4
#define MOE_WIDE_STEP(D, AR, SYNC)                      \
  {                                                     \
    const int st = s0 + (D);                            \
    wide_load_b(br, in, min(st + 2, last));             \
    wide_stage<NL>(smem, (D), AR, acc);                 \
    wide_load_a(AR, in, min(st + 2, last));             \
    wide_store_b(smem, ((D) + 2) & 3, br, in);          \
    if (SYNC) __syncthreads();                          \
  }
  // groups of four steps (the ring indices are compile-time), then the rest
  int s0 = 0;
  for (; s0 + 4 <= n; s0 += 4) {
    MOE_WIDE_STEP(0, ar0, false)
    MOE_WIDE_STEP(1, ar1, true)
    MOE_WIDE_STEP(2, ar0, false)
    MOE_WIDE_STEP(3, ar1, true)
  }
  if (s0 < n) MOE_WIDE_STEP(0, ar0, false)
  if (s0 + 1 < n) MOE_WIDE_STEP(1, ar1, true)
  if (s0 + 2 < n) MOE_WIDE_STEP(2, ar0, false)
#undef MOE_WIDE_STEP
}

// ---------------------------------------------------------------- gate/up
// One shared-expert gate/up tile (row tile mt, 128-column tile nt) over its
// first NL 16-row groups: h_s = silu(G) U, rounded to bf16, for the real
// rows.  Wave w holds the gate (A tile 0) and up (A tile 1) rows of h
// columns n0 + 16 w .. + 15.
template <int NL>
__device__ __forceinline__ void shared_gateup_tile(const FfnArgs& a, TileLds& L, int mt, int nt) {
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int n0 = nt * kBlk + 16 * w;                 // wave's first h column
  TileIn in;
  in.a[0] = tile_row(a.wsg, (size_t)n0 + c, a.H * 2 / kBlk, q);
  in.a[1] = tile_row(a.wsu, (size_t)n0 + c, a.H * 2 / kBlk, q);
  in.sw[0] = in.sw[1] = nullptr;
#pragma unroll
  for (int i = 0; i < kBVec; ++i) {
    const int brow = mt * kTM + tid / 8 + kBRowStep * i;
    in.bok[i] = brow < a.M && row_real(a.mask, brow);
    in.b[i] = reinterpret_cast<const uint8_t*>(a.x + (size_t)(in.bok[i] ? brow : 0) * a.H) + (tid % 8) * 16;
  }
  in.bs = nullptr;
  in.bsok = false;
  in.nstage = a.H * 2 / kStageBytes;
  in.nseg = kSegSG;
  Acc tot;
  tile_gemm<false, NL>(in, L, tot);
#pragma unroll
  for (int b = 0; b < NL; ++b) {
    const int row = mt * kTM + 16 * b + c;
    if (row >= a.M || !row_real(a.mask, row)) continue;
    const v4f h = {silu_mul(tot[0][b][0], tot[1][b][0]), silu_mul(tot[0][b][1], tot[1][b][1]),
                   silu_mul(tot[0][b][2], tot[1][b][2]), silu_mul(tot[0][b][3], tot[1][b][3])};
    store_bf16x4(a.hsh + (size_t)row * a.Is + n0 + 4 * q, h);
  }
}

// Blocks [0, n_sh): shared-expert tiles (row tile, 128-column tile); then
// routed tiles (slot tile of one expert, 128-column tile).  Wave w holds the
// gate (A tile 0) and up (A tile 1) rows of h columns n0 + 16 w .. + 15.
__global__ __launch_bounds__(kTileThreads) void k_gateup_tiled(FfnArgs a) {
  __shared__ TileLds L;
  __shared__ float samax[kWaves][kTM];
  const int ntI = a.I / kBlk, ntS = a.Is / kBlk;
  const int nrow_sh = a.Is > 0 ? (a.M + kTM - 1) / kTM : 0;
  const int n_sh = xcd_rows(nrow_sh) * ntS;          // a multiple of 8
  const int mtiles = a.sched[SCHED_MTILES];
  const int bid = blockIdx.x;
  if (bid >= n_sh + xcd_rows(mtiles) * ntI) return;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, q = lane >> 4, c = lane & 15;
  Acc tot;
  if (bid < n_sh) {
    int mt, nt;
    range_tile(bid, nrow_sh, ntS, mt, nt);
    if (mt >= nrow_sh) return;
    // the row tile's 16-row groups holding rows, rounded up to 2, 4 or 8
    const int live = (min(kTM, a.M - mt * kTM) + 15) / 16;
    if (live <= 2)
      shared_gateup_tile<2>(a, L, mt, nt);
    else if (live <= 4)
      shared_gateup_tile<4>(a, L, mt, nt);
    else
      shared_gateup_tile<kNB>(a, L, mt, nt);
    return;
  }
  int it, nt;
  range_tile(bid - n_sh, mtiles, ntI, it, nt);
  if (it >= mtiles) return;
  const Tile tl = routed_tile(a, it);
  const int n0 = nt * kBlk + 16 * w;
  const int nkb = a.H / kBlk;
  TileIn in;
  in.a[0] = tile_row(a.wg, (size_t)tl.e * a.I + n0 + c, nkb, q);
  in.a[1] = tile_row(a.wu, (size_t)tl.e * a.I + n0 + c, nkb, q);
  in.sw[0] = a.sg + ((size_t)tl.e * ntI + nt) * nkb;
  in.sw[1] = a.su + ((size_t)tl.e * ntI + nt) * nkb;
  {
#pragma unroll
    for (int v = 0; v < kBVec; ++v) {
      const int i = tid / 8 + kBRowStep * v;
      const int row = i < tl.mcnt ? a.rows[tl.s0 + i] : -1;
      in.bok[v] = row >= 0 && row < a.M;
      in.b[v] = a.xq + (size_t)(in.bok[v] ? row : 0) * a.H + (tid % 8) * 16;
    }
    const int rs = (tid < kTM && tid < tl.mcnt) ? a.rows[tl.s0 + tid] : -1;
    in.bsok = rs >= 0 && rs < a.M;
    in.bs = a.xs + (size_t)(in.bsok ? rs : 0) * nkb;
  }
  in.nstage = nkb;
  in.nseg = kSegGU;
  // the slot tiles holding real rows, rounded up to 2, 4 or 8
  const int live = (tl.mcnt + 15) / 16;
  if (live <= 2)
    tile_gemm<true, 2>(in, L, tot);
  else if (live <= 4)
    tile_gemm<true, 4>(in, L, tot);
  else
    tile_gemm<true, kNB>(in, L, tot);
  // h = silu(G) U in place of G; 1x128 requantization over the tile's 128
  // columns; slot tiles past the last one holding rows are skipped
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    if (b >= live) break;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tot[0][b][i] = silu_mul(tot[0][b][i], tot[1][b][i]);
      m = fmaxf(m, fabsf(tot[0][b][i]));
    }
    // max over the four lanes of the same column (xor 16, xor 32)
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(m, fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1])));
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(m, fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1])));
    if (q == 0) samax[w][16 * b + c] = m;
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    if (b >= live) break;
    const int i = 16 * b + c;
    if (i >= tl.mcnt) continue;
    const int slot = tl.s0 + i;
    float amax = samax[0][i];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) amax = fmaxf(amax, samax[v][i]);
    const float s = quant_scale(amax);
    uint32_t word = 0;
    if (amax != 0.0f)
#pragma unroll
      for (int k = 0; k < 4; ++k) word |= quant_code(tot[0][b][k], s) << (8 * k);
    *reinterpret_cast<uint32_t*>(a.hq + (size_t)slot * a.I + n0 + 4 * q) = word;
    if (w == 0 && q == 0) a.hs[(size_t)slot * ntI + nt] = s;
  }
}

// ---------------------------------------------------------------- down
// Blocks [0, n_sh): shared-expert tiles (row tile, 256-column tile of H;
// wave w holds output columns n0 + 32 w .. + 31, A tiles 0 and 1); then
// routed wide tiles (slot tile of one expert, 512-column tile).
constexpr int kDnCols = 32 * kWaves;

// Routed tiles: 512 columns of H (wave w: columns n0 + 64 w .. + 63, weight
// tiles 0-3), one K segment over the whole I.
static_assert(kSegDN == 1, "the routed down tiles run one K segment per wave");
constexpr int kDnColsW = 16 * kWA * kWaves;
constexpr int kDnLds = kWLds > (int)sizeof(TileLds) ? kWLds : (int)sizeof(TileLds);

// One shared-expert down tile (row tile mt, kDnCols-column tile nt) over its
// first NL 16-row groups: S = h_s Wsd^T in fp32 for the real rows.  Wave w
// holds output columns n0 + 32 w .. + 31 (A tiles 0 and 1); waves past H
// compute on in-range rows and store nothing.
template <int NL>
__device__ __forceinline__ void shared_down_tile(const FfnArgs& a, TileLds& L, int mt, int nt) {
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int n0 = nt * kDnCols + 32 * w;
  TileIn in;
  const int nr = n0 < a.H ? n0 : a.H - 32;
#pragma unroll
  for (int t = 0; t < kNA; ++t) {
    in.a[t] = tile_row(a.wsd, (size_t)nr + 16 * t + c, a.Is * 2 / kBlk, q);
    in.sw[t] = nullptr;
  }
#pragma unroll
  for (int i = 0; i < kBVec; ++i) {
    const int brow = mt * kTM + tid / 8 + kBRowStep * i;
    in.bok[i] = brow < a.M && row_real(a.mask, brow);
    in.b[i] = reinterpret_cast<const uint8_t*>(a.hsh + (size_t)(in.bok[i] ? brow : 0) * a.Is) + (tid % 8) * 16;
  }
  in.bs = nullptr;
  in.bsok = false;
  in.nstage = a.Is * 2 / kStageBytes;
  in.nseg = kSegSD;
  Acc tot;
  tile_gemm<false, NL>(in, L, tot);
  if (n0 >= a.H) return;
#pragma unroll
  for (int b = 0; b < NL; ++b) {
    const int row = mt * kTM + 16 * b + c;
    if (row >= a.M || !row_real(a.mask, row)) continue;
#pragma unroll
    for (int t = 0; t < kNA; ++t) store_f4(a.S + (size_t)row * a.H + n0 + 16 * t + 4 * q, tot[t][b]);
  }
}

// One routed wide tile over its first NL slot tiles: the K loop, then the
// real slots' D rows (waves past H store nothing).
template <int NL>
__device__ __forceinline__ void down_wide_tile(const FfnArgs& a, const WideIn& in, uint8_t* smem, const Tile& tl,
                                               int n0) {
  WAcc acc;
  wide_gemm<NL>(in, smem, acc);
  if (n0 >= a.H) return;
  const int c = threadIdx.x & 15, q = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int b = 0; b < NL; ++b) {
    const int i = 16 * b + c;
    if (i >= tl.mcnt) continue;
#pragma unroll
    for (int t = 0; t < kWA; ++t) store_f4(a.D + (size_t)(tl.s0 + i) * a.H + n0 + 16 * t + 4 * q, acc[t][b]);
  }
}

__global__ __launch_bounds__(kTileThreads) void k_down_tiled(FfnArgs a) {
  __shared__ __align__(16) uint8_t smem[kDnLds];
  TileLds& L = *reinterpret_cast<TileLds*>(smem);
  const int ntH = (a.H + kDnCols - 1) / kDnCols;
  const int ntW = (a.H + kDnColsW - 1) / kDnColsW;
  const int nrow_sh = a.Is > 0 ? (a.M + kTM - 1) / kTM : 0;
  const int n_sh = xcd_rows(nrow_sh) * ntH;          // a multiple of 8
  const int mtiles = a.sched[SCHED_MTILES];
  const int bid = blockIdx.x;
  if (bid >= n_sh + xcd_rows(mtiles) * ntW) return;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, q = lane >> 4, c = lane & 15;
  Acc tot;
  if (bid < n_sh) {
    int mt, nt;
    range_tile(bid, nrow_sh, ntH, mt, nt);
    if (mt >= nrow_sh) return;
    // the row tile's 16-row groups holding rows, rounded up to 2, 4 or 8
    const int live = (min(kTM, a.M - mt * kTM) + 15) / 16;
    if (live <= 2)
      shared_down_tile<2>(a, L, mt, nt);
    else if (live <= 4)
      shared_down_tile<4>(a, L, mt, nt);
    else
      shared_down_tile<kNB>(a, L, mt, nt);
    return;
  }
  int it, nt;
  range_tile(bid - n_sh, mtiles, ntW, it, nt);
  if (it >= mtiles) return;
  const Tile tl = routed_tile(a, it);
  const int n0 = nt * kDnColsW + 16 * kWA * w;
  const int nkb = a.I / kBlk;
  // waves past H compute on in-range rows and store nothing
  const int nr = n0 < a.H ? n0 : a.H - 16 * kWA;
  WideIn in;
  in.a = tile_row(a.wd, (size_t)tl.e * a.H + nr + c, nkb, q);
  in.astep = (long)nkb * kTile;
  in.sw = a.sd + ((size_t)tl.e * (a.H / kBlk) + nr / kBlk) * nkb;
#pragma unroll
  for (int v = 0; v < kWBV; ++v) {
    const int i = tid / 8 + kWBRow * v;
    in.bok[v] = i < tl.mcnt;
    in.boff[v] = (uint32_t)((size_t)(tl.s0 + (in.bok[v] ? i : 0)) * a.I + (tid % 8) * 16);
  }
  in.bbase = a.hq;
  in.bsok = tid < kTM && tid < tl.mcnt;
  in.sbase = a.hs;
  in.soff = (uint32_t)((size_t)(tl.s0 + (in.bsok ? tid : 0)) * nkb);
  in.nkb = nkb;
  // the slot tiles holding real rows, rounded up to 1, 2, 4 or 8
  const int live = (tl.mcnt + 15) / 16;
  if (live <= 1)
    down_wide_tile<1>(a, in, smem, tl, n0);
  else if (live <= 2)
    down_wide_tile<2>(a, in, smem, tl, n0);
  else if (live <= 4)
    down_wide_tile<4>(a, in, smem, tl, n0);
  else
    down_wide_tile<kNB>(a, in, smem, tl, n0);
}

hipError_t launch_tiled(const FfnArgs& a, long mtiles_max, hipStream_t s) {
  const long sh_tiles = a.Is > 0 ? xcd_rows((a.M + kTM - 1) / kTM) : 0;
  const long mt8 = xcd_rows((int)mtiles_max);
  const long gu = sh_tiles * (a.Is / kBlk) + mt8 * (a.I / kBlk);
  MOE_LAUNCH(KID_GATEUP, k_gateup_tiled, dim3((unsigned)gu), dim3(kTileThreads), 0, s, a);
  const long ntH = (a.H + kDnCols - 1) / kDnCols;
  const long ntW = (a.H + kDnColsW - 1) / kDnColsW;
  const long dn = sh_tiles * ntH + mt8 * ntW;
  MOE_LAUNCH(KID_DOWN, k_down_tiled, dim3((unsigned)dn), dim3(kTileThreads), 0, s, a);
  return hipSuccess;
}

}  // namespace moe
