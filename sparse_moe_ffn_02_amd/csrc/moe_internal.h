// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMTile = 128;          // slots (or rows) per tile of the tiled grouped GEMMs
constexpr int kDecodeMaxRows = 32;  // LDS capacity (rows) of the small-step selection kernel
constexpr int kSmallRows = 24;      // most rows of a split small step (experts of inter <= kNarrowInter)
constexpr int kSmallRowsWide = 16;  // most rows of a split small step for wider experts
constexpr int kNarrowInter = 512;
// Rows up to which the split small-step kernels beat the tiled ones (measured
// crossover): wide experts (inter 2048) reach the tiled kernels' speed from
// 17 rows, narrow ones (a TP8 shard's inter 256) keep the split path to 24.
inline int split_rows(int inter) { return inter <= kNarrowInter ? kSmallRows : kSmallRowsWide; }
// The split kernels' work items take the step's rows (or an expert's slots)
// as the 16 MFMA columns, in row halves of kColRows: rows 16 h .. 16 h + 15.
constexpr int kColRows = 16;
__host__ __device__ inline int row_halves(int m) { return (m + kColRows - 1) / kColRows; }
constexpr int kUChunks = 128;       // row chunks of the larger-step union (4096 rows: 36 us for the three kernels, 48 with 64 chunks)
// Every GEMM element is the fixed-order sum of its K-segment chains:
// routed gate/up over kSegGU segments of K = H, shared gate/up over kSegSG,
// routed down over kSegDN and shared down over kSegSD segments of K = I.  Small steps run each segment as its own work
// item and reduce the fp32 partials later; larger steps run them in-wave.
constexpr int kSegGU = 2;
constexpr int kSegDN = 1;
constexpr int kSegSD = 4;           // shared expert down
constexpr int kSegSG = 16;          // shared expert gate/up (bf16 steps stream half the bytes per load)

// sched[] words written by the union / plan kernels and read by the FFN kernels
enum { SCHED_NUNION = 0, SCHED_MTILES = 1, SCHED_SLOTS = 2, SCHED_BAD = 3, SCHED_WORDS = 8 };

struct RouteArgs {
  const uint16_t* x;       // bf16 [M, H]
  const uint8_t* mask;     // [M] or null
  const uint16_t* wr;      // bf16 [E, H]
  const float* bias;       // [E]
  int M, H, E, K;
  float scale;
  double* logits;          // ws [M, E] logits (large steps) or biased scores c (small steps)
  double* sig;             // ws [M, E] sigmoid of the logits (small steps)
  uint32_t* rowbits;       // ws [M, ceil(E/32)]
  int32_t* ids;            // [M, K]
  float* w;                // [M, K]
  int32_t* n_union;        // [1]
  int32_t* union_ids;      // [E]
  int32_t* offs;           // [E + 1]
  int32_t* rows;           // [M * K]
  int32_t* slot_of;        // [M, K]
  int32_t* sched;          // ws [SCHED_WORDS]
  int32_t* mtile_offs;     // ws [E + 1]
  int32_t* ucount;         // ws [kUChunks, E] per row-chunk counts, then first slots (larger steps)
};

struct FfnArgs {
  int M, H, E, K, I, Is;
  const uint16_t* x;       // bf16 [M, H]
  const uint8_t* mask;     // [M] or null
  // routing
  const int32_t* ids;      // [M, K]
  const float* w;          // [M, K]
  const int32_t* n_union;
  const int32_t* union_ids;
  const int32_t* offs;
  const int32_t* rows;
  const int32_t* slot_of;
  // routed expert weights
  const uint8_t *wg, *wu, *wd;
  const float *sg, *su, *sd;
  // shared expert (null when Is == 0)
  const uint16_t *wsg, *wsu, *wsd;
  // workspace
  int32_t* sched;
  int32_t* mtile_offs;
  uint8_t* xq; float* xs;  // [M, H], [M, H/128]
  uint8_t* hq; float* hs;  // [M*K, I], [M*K, I/128]
  uint16_t* hsh;           // [M, Is] bf16 shared h
  float* S;                // [M, H]
  float* D;                // [M*K, H]
  // split small-step path (M <= kSmallRows): per-segment fp32 partials
  int split;
  float* part_gu;          // [kSegGU][M*K][2][I]  routed gate / up
  float* part_sh;          // [kSegSG][M][2][Is]   shared gate / up
  float* part_d;           // [kSegDN][M*K][H]     routed down
  float* part_s;           // [kSegSD][M][H]       shared down
  uint16_t* y;             // bf16 [M, H]
};

// Residual add + RMSNorm epilogue (bf16 [M, H] rows; gamma bf16 [H]).
struct NormArgs {
  const uint16_t* res;     // residual in
  const uint16_t* gamma;
  float eps;
  uint16_t* res_out;       // r_new (may equal res)
  uint16_t* out;           // normalized rows
};

// Kernel ids reported by the timing hook (moe_trace_set).
enum KernelId {
  KID_ROUTER_LOGITS = 0, KID_ROUTE_SELECT, KID_UNION, KID_QUANT_X, KID_PLAN, KID_GATEUP, KID_POST_GATEUP,
  KID_DOWN, KID_COMBINE, KID_QUANT, KID_ROUTE_SMALL, KID_FRONT, KID_PACK, KID_COMBINE_NORM, KID_ADD_NORM,
  KID_SUM_PARTIALS, KID_PREFETCH, KID_COUNT
};

void trace_before(hipStream_t s);
void trace_after(int kid, hipStream_t s);

// Launch, capture the launch status, record the timing events when tracing,
// and return the status from the enclosing launcher on failure.
#define MOE_LAUNCH(kid, kernel, grid, block, shmem, stream, ...)                 \
  do {                                                                           \
    ::moe::trace_before(stream);                                                 \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);         \
    const hipError_t moe_launch_err_ = hipGetLastError();                        \
    ::moe::trace_after(kid, stream);                                             \
    if (moe_launch_err_ != hipSuccess) return moe_launch_err_;                   \
  } while (0)

hipError_t launch_route(const RouteArgs& a, hipStream_t s);
// split small steps: logits + x quantization + shared gate/up, then select/union + shared h_s
hipError_t launch_front_split(const RouteArgs& r, const FfnArgs& f, hipStream_t s);
hipError_t launch_plan(const FfnArgs& a, hipStream_t s);
hipError_t launch_prep(const FfnArgs& a, hipStream_t s);   // quantize x
// nm != nullptr: the combine also runs the residual add + RMSNorm epilogue
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s, const NormArgs* nm = nullptr);
hipError_t launch_add_rmsnorm(const uint16_t* y, const uint8_t* mask, int M, int H, const NormArgs& nm,
                              hipStream_t s);
// steps that do not take the split path: tiled gate/up (+ SiLU, requant) and down
hipError_t launch_tiled(const FfnArgs& a, long mtiles_max, hipStream_t s);
bool use_split(int M, int H, int I);   // M <= split_rows(I)
hipError_t launch_pack(const void* src, void* dst, long rows, int row_bytes, int is_bf16, hipStream_t s);
hipError_t launch_sum_partials(const uint16_t* parts, const uint8_t* mask, int M, int H, int nsrc, uint16_t* y,
                               hipStream_t s);
// Route-ahead prefetch: read the packed matrices mats[0..nmat) (each [E] x
// mat_bytes) of the experts union_ids[0 .. *n_union) in union order, at most
// max_chunks chunks of prefetch_chunk_bytes(); checksum (optional) += the
// 32-bit word sum of every byte read.
long prefetch_chunk_bytes();
hipError_t launch_prefetch(const int32_t* n_union, const int32_t* union_ids, int E, const uint8_t* const* mats,
                           int nmat, long mat_bytes, long max_chunks, int workgroups, uint32_t* checksum,
                           hipStream_t s);
hipError_t launch_quant_generic(const void* in, int is_bf16, int R, int C, uint8_t* codes, float* scales,
                                hipStream_t s);

}  // namespace moe
