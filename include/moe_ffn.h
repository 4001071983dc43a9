/*
 * moe_ffn.h -- C ABI of the routed fp8 mixture-of-experts FFN layer on one
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the routed MoE block of a GLM-5.2-style model: a noaux-tc
 * router (a score per expert plus an e_score_correction_bias used for
 * selection only, top-k; mstar PR #388 "Speed up GLM-5.2 with fp8 kernels and
 * one-graph MTP", router notes; MoE-Infinity PR #140, "[256] router bias"),
 * the step's expert union and GEMM / SiLU / GEMM phases with fixed-order
 * reductions and zero-filled pad rows (openinfer PR #610 "TP8 span row
 * mapping", description and "Gates"), routed experts stored as an fp8 e4m3
 * [gate_proj, up_proj, down_proj] triple with block scales (MoE-Infinity
 * PR #140, fp8 store and expert-node commits), activations quantized to e4m3
 * per 128 columns (mstar PR #388, FlashInfer crossover note), and a bf16
 * shared expert added to every row.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer is a DEVICE pointer unless its comment says "host".  The
 *   caller allocates and owns all memory; the library never allocates, frees
 *   or keeps a pointer after a call returns.
 * - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *   No call synchronizes the host, so calls are safe inside stream capture.
 *   Calls that share a workspace or outputs on different streams race.
 * - Matrices are row-major and dense, except expert and shared-expert
 *   weights, which are passed in the packed tile layout written by
 *   moe_pack_weights (same size).  Device pointers must be 16-byte aligned.
 *   bf16 values are passed as uint16_t bit patterns; e4m3 values as uint8_t
 *   codes (OCP FP8 e4m3fn: bias 7, max 448, no infinities).
 * - `row_mask` (device, uint8 [M]) marks real rows with 1 and pad rows with
 *   0; NULL means every row is real.  Kernels read it at run time, so one
 *   captured graph serves every mask.  A pad row's input is never read; its
 *   outputs are written as +0.0 (ids -1, weights 0).
 * - Return value: MOE_OK or an error status.  All arguments are checked on
 *   the host before anything is enqueued; a call that returns an error other
 *   than MOE_ELAUNCH enqueued nothing.  M == 0 returns MOE_OK and enqueues
 *   nothing.
 *
 * Numerics (the same procedure for every row, whatever its slot, the other
 * rows of the step or the number of rows, so a row's bits never depend on
 * its neighbours):
 * - logits in float64 (exact bf16 products), score c = sigmoid(l) + bias,
 *   top-k of c with exact ties to the lower id, ids listed ascending,
 *   w = routed_scale * sigmoid(l_j) / sum of the selected sigmoids;
 * - activation quantization per row and 128-column block:
 *   s = fl32(amax / 448) (1 for an all-zero block), code = round-to-nearest-
 *   even saturating e4m3 of fl32(v / s);
 * - GEMMs accumulate in fp32: per 128-deep K-block one fp8 MFMA partial,
 *   then acc = fma(s_act * s_w, partial, acc) in ascending K-block order;
 * - h = silu(gate) * up in fp32, requantized per 1x128 block as above;
 * - y = bf16(fma chain over the row's experts in ascending id, + shared).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_EINVAL 1       /* null required pointer, bad dims, misaligned pointer, M < 0 */
#define MOE_EUNSUPPORTED 2 /* n_experts > MOE_MAX_EXPERTS, top_k > MOE_MAX_TOPK or > n_experts, M > MOE_MAX_ROWS,
                              inter > MOE_MAX_INTER */
#define MOE_EWORKSPACE 3   /* ws_bytes smaller than moe_workspace_bytes() for this M */
#define MOE_ELAUNCH 4      /* a kernel launch failed (hipGetLastError after each launch) */

#define MOE_MAX_ROWS 16384
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 16
#define MOE_MAX_INTER 8192 /* keeps every byte offset into the [M*top_k, inter] activation codes below 2^31 */

/* Layer dimensions (host struct).  hidden, inter and shared_inter must be
 * multiples of 128; shared_inter may be 0 (no shared expert). */
typedef struct {
  int32_t hidden;       /* H */
  int32_t n_experts;    /* E, 1..256 */
  int32_t top_k;        /* k, 1..min(16, E) */
  int32_t inter;        /* I, routed expert intermediate size */
  int32_t shared_inter; /* I_s, shared expert intermediate size, 0 = none */
  float routed_scale;   /* factor applied to the renormalized top-k weights (2.5 for GLM-5.2) */
} moe_dims;

/* Router parameters (device). */
typedef struct {
  const uint16_t* w;  /* bf16 [E, H] */
  const float* bias;  /* fp32 [E], e_score_correction_bias, used for selection only */
} moe_router_w;

/* Layout tags of the weight structs below.  The expert kernels read
 * weights only in the packed tile layout that moe_pack_weights writes; a
 * caller states which layout its pointers hold, so that checkpoint-layout
 * (row-major) weights are refused instead of being read as tiles (the pages
 * require that an fp8 checkpoint missing its scales is refused rather than
 * loaded as unscaled weights: mstar PR #388, fp8 checkpoint commit).  A
 * zero-initialized struct carries MOE_WEIGHTS_ROW_MAJOR. */
#define MOE_WEIGHTS_ROW_MAJOR 0u          /* checkpoint layout: refused with MOE_EUNSUPPORTED */
#define MOE_WEIGHTS_PACKED 0x4B43504Du    /* every matrix rearranged by moe_pack_weights */

/* Routed experts (device): e4m3 codes of the output-major matrices below
 * (K contiguous in the checkpoint), each packed by moe_pack_weights
 * (is_bf16 = 0), and one fp32 scale per 128x128 block (scales stay
 * row-major).  The [gate_proj, up_proj, down_proj] triple is consumed by
 * position (MoE-Infinity PR #140, expert-node commit).  All six pointers are
 * required: an fp8 expert without its scales is refused (MOE_EINVAL).
 * layout must be MOE_WEIGHTS_PACKED (MOE_WEIGHTS_ROW_MAJOR: MOE_EUNSUPPORTED;
 * any other value: MOE_EINVAL). */
typedef struct {
  const uint8_t* w_gate; /* [E, I, H], packed */
  const uint8_t* w_up;   /* [E, I, H], packed */
  const uint8_t* w_down; /* [E, H, I], packed */
  const float* s_gate;   /* [E, I/128, H/128] */
  const float* s_up;     /* [E, I/128, H/128] */
  const float* s_down;   /* [E, H/128, I/128] */
  uint32_t layout;       /* MOE_WEIGHTS_PACKED */
} moe_expert_w;

/* Shared expert (device): bf16, output-major, each matrix packed by
 * moe_pack_weights (is_bf16 = 1); layout as in moe_expert_w. */
typedef struct {
  const uint16_t* w_gate; /* [I_s, H], packed */
  const uint16_t* w_up;   /* [I_s, H], packed */
  const uint16_t* w_down; /* [H, I_s], packed */
  uint32_t layout;        /* MOE_WEIGHTS_PACKED */
} moe_shared_w;

/* Routing of one step (device buffers, written by moe_route / moe_layer and
 * read by moe_ffn_fp8).  Slots number the (row, pick) pairs expert by expert
 * in union order; inside an expert its rows are ascending. */
typedef struct {
  int32_t* topk_ids;  /* [M, k] expert ids, ascending per row; -1 for pads */
  float* topk_w;      /* [M, k] weights in the same order; 0 for pads */
  int32_t* n_union;   /* [1] number of experts picked by any real row */
  int32_t* union_ids; /* [E] first n_union entries: the union, ascending */
  int32_t* offs;      /* [E + 1] slot offsets: expert union_ids[u] owns slots [offs[u], offs[u+1]) */
  int32_t* rows;      /* [M * k] row of each slot */
  int32_t* slot_of;   /* [M, k] slot of (row, pick); -1 for pads */
} moe_routing;

/* Optional copies of the quantized activations (device; NULL fields or a
 * NULL struct = not written).  Slot order as in moe_routing. */
typedef struct {
  uint8_t* x_codes; /* [M, H] e4m3 codes of x (real rows) */
  float* x_scales;  /* [M, H/128] */
  uint8_t* h_codes; /* [M * k, I] e4m3 codes of silu(gate)*up per slot */
  float* h_scales;  /* [M * k, I/128] */
} moe_taps;

/* Device workspace bytes needed by moe_route / moe_ffn_fp8 / moe_layer for
 * any M <= max_rows.  Returns 0 for invalid dims or max_rows outside
 * [0, MOE_MAX_ROWS]. */
size_t moe_workspace_bytes(const moe_dims* dims, int32_t max_rows);

/* Router and union (mstar PR #388 router notes; openinfer PR #610 "Gates"):
 * logits, sigmoid + bias top-k, weights, the ascending expert union and the
 * per-expert row lists.  x: bf16 [M, H].  Writes every field of *out. */
int moe_route(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
              const moe_router_w* router, moe_routing* out, void* ws, size_t ws_bytes, void* stream);

/* Routed experts only (openinfer PR #610 "What": union / GEMM / SiLU / GEMM
 * phases): quantize x, gate/up GEMMs, SiLU*up with 1x128 requantization,
 * down GEMM, fixed-order weighted combine.  `in` may come from moe_route or
 * from any producer of the same layout; a malformed routing (n_union or
 * offsets out of range, union not ascending, an expert's rows not strictly
 * ascending, a row outside [0, M) or a pad row in a row list) contributes
 * nothing: y is then the zero-routing output (+0.0 for every row).
 * y: bf16 [M, H], routed part only (no shared expert); pad rows +0.0. */
int moe_ffn_fp8(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
                const moe_routing* in, const moe_expert_w* experts, uint16_t* y, moe_taps* taps, void* ws,
                size_t ws_bytes, void* stream);

/* The whole layer (openinfer PR #610, "What": one layer of a step runs the
 * expert union, the gate/up GEMMs, SiLU and the down GEMM over the step's
 * rows, then combines in a fixed order; mstar PR #388, decode table note:
 * one layer's routed and shared experts timed per call): moe_route, then the
 * routed experts and the bf16 shared expert (shared may be NULL only when
 * dims->shared_inter == 0).  y: bf16 [M, H]; the routing is written to
 * *out. */
int moe_layer(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
              const moe_router_w* router, const moe_expert_w* experts, const moe_shared_w* shared, uint16_t* y,
              moe_routing* out, moe_taps* taps, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: moe_layer
 * without a workspace argument.  The call runs in a static device array of
 * MOE_STATIC_WS_BYTES inside the library, one per GPU (the GPU current on the
 * calling thread), held until the process ends; the call allocates nothing.
 * Steps whose moe_workspace_bytes(dims, M) exceeds MOE_STATIC_WS_BYTES are
 * refused with MOE_EWORKSPACE before anything is enqueued (at GLM-5.2's
 * hidden 6144, 256 experts top-8, inter 2048: every step of up to 265
 * rows).  Every call on
 * a GPU shares that GPU's array, so calls that overlap on one GPU (on any
 * streams) race; the array needs no clearing (each call writes every word it
 * reads).  Other arguments and statuses as moe_layer. */
#define MOE_STATIC_WS_BYTES (64u << 20)
int moe_layer_static(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
                     const moe_router_w* router, const moe_expert_w* experts, const moe_shared_w* shared,
                     uint16_t* y, moe_routing* out, moe_taps* taps, void* stream);

/* Residual add + RMSNorm, the epilogue that feeds the next layer (mstar PR
 * #388: the "kernel switches" note fuses each all-reduce with the next add +
 * RMSNorm; its "Tests" list checks that the fused wiring emits what the
 * unfused ops do).  Per real row r, over its H columns:
 *   residual_out = bf16(fl32(residual) + fl32(y))
 *   out          = bf16(residual_out * (1 / sqrt(mean(residual_out^2) + eps)) * gamma)
 * with a fixed float32 reduction order, so the same y gives the same bits
 * from either call below.  Pad rows (row_mask 0): residual_out = out = +0.0,
 * their y and residual never read.  y, residual, residual_out, out: bf16
 * [M, H] (device); gamma: bf16 [H]; eps >= 0 (else MOE_EINVAL).
 * residual_out may be residual itself (in place); no other overlap.
 * H must be a multiple of 128. */
int moe_add_rmsnorm(int32_t M, int32_t H, const uint16_t* y, const uint8_t* row_mask, const uint16_t* residual,
                    const uint16_t* gamma, float eps, uint16_t* residual_out, uint16_t* out, void* stream);

/* moe_layer with the combine running the residual add + RMSNorm above in the
 * same pass (one launch instead of two, y never re-read), except for the
 * small steps (at most 16 rows, or 24 when dims->inter <= 512), where the
 * element-wise combine and the row epilogue run
 * as two launches (more workgroups; the same bits).  y (the layer output,
 * bf16 [M, H]) is also stored unless y is NULL; residual_out and out as in
 * moe_add_rmsnorm with H = dims->hidden. */
int moe_layer_add_rmsnorm(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
                          const moe_router_w* router, const moe_expert_w* experts, const moe_shared_w* shared,
                          const uint16_t* residual, const uint16_t* gamma, float eps, uint16_t* y,
                          uint16_t* residual_out, uint16_t* out, moe_routing* routing, moe_taps* taps, void* ws,
                          size_t ws_bytes, void* stream);

/* Fixed-order sum of tensor-parallel partial outputs (openinfer PR #610,
 * description and "How": under TP8 each rank produces a partial layer
 * output for every row into one region laid out [row][src][hidden], shared by
 * the Dp8 and span row mappings, and the partials are summed in a fixed
 * order; "Gates": the same rows through both mappings give the same bits).
 * Per real row r and column n:
 *   y[r, n] = bf16( (((0 + fl32(parts[r, 0, n])) + fl32(parts[r, 1, n])) + ...) )
 * float32 additions in ascending source order, one RNE rounding; pad rows
 * (row_mask 0) get +0.0 and their partials are never read.
 * parts: bf16 [M, nsrc, H] (device); y: bf16 [M, H] (device, must not overlap
 * parts); 1 <= nsrc <= 64; H a multiple of 4. */
int moe_sum_partials(int32_t M, int32_t H, int32_t nsrc, const uint16_t* parts, const uint8_t* row_mask, uint16_t* y,
                     void* stream);

/* Route-ahead prefetch (MoE-Infinity PR #140, route-ahead expert prefetch
 * commit: the per-token union of the routed experts of a coming block is
 * fetched ahead of use while other work runs).  With every expert resident in
 * HBM, what is fetched ahead is the experts' packed weight bytes, read once so
 * that they pass into the memory-side Infinity Cache for a later layer call.
 * Reads, for u = 0 .. *n_union - 1 in order, the matrices of expert
 * union_ids[u] selected by parts (MOE_PREFETCH_GATE_UP: w_gate then w_up;
 * MOE_PREFETCH_DOWN: w_down; gate/up first when both), each in address
 * order, stopping after max_bytes rounded down to whole 16 KiB chunks
 * (max_bytes 0: nothing is launched).  n_union and union_ids are device
 * buffers in moe_routing's layout (e.g. the fields of a moe_route result):
 * n_union is read on the device and clamped to [0, E]; entries outside
 * [0, E) are skipped.  Scales are not read.  checksum (device, optional):
 * the wrapping 32-bit sum of every little-endian 32-bit word read is added
 * to *checksum (the caller clears it first); NULL: nothing is written.
 * workgroups: grid size, 0 = 256 (one per compute unit); fewer leave more of
 * the chip to kernels running beside it on other streams.  The call has no
 * effect on any result of the library.  Errors: MOE_EINVAL for bad dims,
 * weights (as moe_layer), null or misaligned n_union / union_ids, parts 0 or
 * with unknown bits, negative max_bytes or workgroups; MOE_EUNSUPPORTED for
 * workgroups above MOE_PREFETCH_MAX_WORKGROUPS. */
#define MOE_PREFETCH_GATE_UP 1u
#define MOE_PREFETCH_DOWN 2u
#define MOE_PREFETCH_MAX_WORKGROUPS 4096
int moe_prefetch_experts(const moe_dims* dims, const int32_t* n_union, const int32_t* union_ids,
                         const moe_expert_w* experts, uint32_t parts, int64_t max_bytes, int32_t workgroups,
                         uint32_t* checksum, void* stream);

/* The 1x128 activation quantization step on its own (mstar PR #388,
 * FlashInfer crossover note): rows x cols values (fp32 if is_bf16 == 0, else
 * bf16 bits) -> e4m3 codes [rows, cols] and fp32 scales [rows, cols/128].
 * cols must be a multiple of 128. */
int moe_quant_fp8(const void* in, int32_t is_bf16, int32_t rows, int32_t cols, uint8_t* codes, float* scales,
                  void* stream);

/* Weight packing (once, when weights are loaded).  The expert kernels read
 * weights in 2048-byte tiles of 16 rows x 128 bytes of K, the tiles of a
 * 16-row group consecutive along K and the groups consecutive, so that each
 * load instruction of a wave reads 1 KB of contiguous memory and a wave
 * streaming K reads whole tiles in address order.  Inside a tile, the 32
 * bytes an MFMA lane (row r = 0..15, quarter q = 0..3) needs for one fp8
 * 16x16x128 step (K bytes [32 q, 32 q + 32)) or one pair of bf16 16x16x32
 * steps (elements [8 q, 8 q + 8) of each step) are split in two 16-byte
 * halves at (r + 16 q) * 16 and 1024 + (r + 16 q) * 16.
 * src: row-major [rows, row_bytes] (e4m3 codes, or bf16 with is_bf16 != 0);
 * dst: same size, must not overlap src.  rows must be a multiple of 16 and
 * row_bytes of 128 (an expert stack [E, N, K] is rows = E * N). */
int moe_pack_weights(const void* src, void* dst, int64_t rows, int32_t row_bytes, int32_t is_bf16, void* stream);

/* Kernel timing hook for measurement (host).  The pages time one layer's
 * experts per call with every call's weights read from HBM (mstar PR #388,
 * decode table note); this hook times each kernel of a call.  While a table
 * is set, every kernel the library enqueues is bracketed by
 * hipEventRecord(pairs[i].start) and hipEventRecord(pairs[i].stop) on the
 * launch stream, kernel_ids[i] receives the kernel's id and *count is
 * incremented, until *count reaches capacity.  The events (hipEvent_t) and
 * the three arrays are the caller's and must outlive the traced calls.
 * pairs == NULL switches tracing off.  The table belongs to the calling host
 * thread: only calls made from that thread are traced, and the hook is for
 * measurement only (it is the one piece of state the library keeps between
 * calls).  Returns MOE_EINVAL for capacity < 0 or a NULL ids or count with a
 * non-NULL table. */
typedef struct {
  void* start; /* hipEvent_t */
  void* stop;  /* hipEvent_t */
} moe_event_pair;
int moe_trace_set(moe_event_pair* pairs, int32_t capacity, int32_t* kernel_ids, int32_t* count);

/* Name of a kernel id reported by moe_trace_set (static string; "?" if unknown). */
const char* moe_kernel_name(int32_t kernel_id);

/* Human-readable name of a status code (static string). */
const char* moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
