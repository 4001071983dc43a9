// C ABI of the MoE FFN library: argument checks, workspace layout and the
// launch sequence of each entry point.  Nothing here allocates, frees or
// synchronizes; every check happens before the first launch.
#include <math.h>
#include <algorithm>
#include <mutex>
#include <string.h>

#include "moe_ffn.h"
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t sched, mtile, ucount, logits, sig, rowbits, xq, xs, hq, hs, hsh, S, D, part_gu, part_sh, part_d, part_s, total;
  bool split;
};

Layout make_layout(const moe_dims& d, int M) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t m = (size_t)M, H = d.hidden, E = d.n_experts, K = d.top_k, I = d.inter, Is = d.shared_inter;
  L.sched = take(SCHED_WORDS * sizeof(int32_t));
  L.mtile = take((E + 1) * sizeof(int32_t));
  L.ucount = take(kUChunks * E * sizeof(int32_t));
  L.logits = take(m * E * sizeof(double));
  L.sig = take(m * E * sizeof(double));
  L.rowbits = take(m * ((E + 31) / 32) * sizeof(uint32_t));
  L.xq = take(m * H);
  L.xs = take(m * (H / 128) * sizeof(float));
  L.hq = take(m * K * I);
  L.hs = take(m * K * (I / 128) * sizeof(float));
  L.hsh = take(m * Is * sizeof(uint16_t));
  L.S = take(m * H * sizeof(float));
  L.D = take(m * K * H * sizeof(float));
  L.split = use_split(M, d.hidden, d.inter);
  const size_t sp = L.split ? 1 : 0;
  L.part_gu = take(sp * kSegGU * m * K * 2 * I * sizeof(float));
  L.part_sh = take(sp * kSegSG * m * 2 * Is * sizeof(float));
  L.part_d = take(sp * kSegDN * m * K * H * sizeof(float));
  L.part_s = take(sp * kSegSD * m * H * sizeof(float));
  L.total = off;
  return L;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_dims(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->hidden <= 0 || d->hidden % 128 || d->inter <= 0 || d->inter % 128) return MOE_EINVAL;
  if (d->shared_inter < 0 || d->shared_inter % 128) return MOE_EINVAL;
  if (d->n_experts <= 0 || d->top_k <= 0) return MOE_EINVAL;
  if (!isfinite(d->routed_scale)) return MOE_EINVAL;
  if (d->n_experts > MOE_MAX_EXPERTS || d->top_k > MOE_MAX_TOPK || d->top_k > d->n_experts) return MOE_EUNSUPPORTED;
  if (d->inter > MOE_MAX_INTER) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int check_rows(int32_t M) {
  if (M < 0) return MOE_EINVAL;
  if (M > MOE_MAX_ROWS) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// required device pointer with the given alignment
inline bool ok_ptr(const void* p, size_t a) { return p != nullptr && aligned(p, a); }
// optional device pointer
inline bool ok_opt(const void* p, size_t a) { return p == nullptr || aligned(p, a); }

int check_routing(const moe_routing* r) {
  if (!r) return MOE_EINVAL;
  if (!ok_ptr(r->topk_ids, 4) || !ok_ptr(r->topk_w, 4) || !ok_ptr(r->n_union, 4) || !ok_ptr(r->union_ids, 4) ||
      !ok_ptr(r->offs, 4) || !ok_ptr(r->rows, 4) || !ok_ptr(r->slot_of, 4))
    return MOE_EINVAL;
  return MOE_OK;
}

// The kernels read weights only as packed tiles; a struct that does not say
// so is refused before anything is enqueued.
int check_layout(uint32_t layout) {
  if (layout == MOE_WEIGHTS_PACKED) return MOE_OK;
  return layout == MOE_WEIGHTS_ROW_MAJOR ? MOE_EUNSUPPORTED : MOE_EINVAL;
}

int check_experts(const moe_expert_w* w) {
  if (!w) return MOE_EINVAL;
  if (!ok_ptr(w->w_gate, 16) || !ok_ptr(w->w_up, 16) || !ok_ptr(w->w_down, 16)) return MOE_EINVAL;
  if (!ok_ptr(w->s_gate, 4) || !ok_ptr(w->s_up, 4) || !ok_ptr(w->s_down, 4)) return MOE_EINVAL;
  return check_layout(w->layout);
}

int check_shared(const moe_shared_w* w) {
  if (!w || !ok_ptr(w->w_gate, 16) || !ok_ptr(w->w_up, 16) || !ok_ptr(w->w_down, 16)) return MOE_EINVAL;
  return check_layout(w->layout);
}

int check_taps(const moe_taps* t) {
  if (!t) return MOE_OK;
  if (!ok_opt(t->x_codes, 16) || !ok_opt(t->x_scales, 4) || !ok_opt(t->h_codes, 16) || !ok_opt(t->h_scales, 4))
    return MOE_EINVAL;
  return MOE_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

RouteArgs route_args(const moe_dims& d, int M, const uint16_t* x, const uint8_t* mask, const moe_router_w& rw,
                     const moe_routing& out, char* ws, const Layout& L) {
  RouteArgs a;
  a.x = x;
  a.mask = mask;
  a.wr = rw.w;
  a.bias = rw.bias;
  a.M = M;
  a.H = d.hidden;
  a.E = d.n_experts;
  a.K = d.top_k;
  a.scale = d.routed_scale;
  a.logits = reinterpret_cast<double*>(ws + L.logits);
  a.sig = reinterpret_cast<double*>(ws + L.sig);
  a.rowbits = reinterpret_cast<uint32_t*>(ws + L.rowbits);
  a.ids = out.topk_ids;
  a.w = out.topk_w;
  a.n_union = out.n_union;
  a.union_ids = out.union_ids;
  a.offs = out.offs;
  a.rows = out.rows;
  a.slot_of = out.slot_of;
  a.sched = reinterpret_cast<int32_t*>(ws + L.sched);
  a.mtile_offs = reinterpret_cast<int32_t*>(ws + L.mtile);
  a.ucount = reinterpret_cast<int32_t*>(ws + L.ucount);
  return a;
}

FfnArgs ffn_args(const moe_dims& d, int M, const uint16_t* x, const uint8_t* mask, const moe_routing& rt,
                 const moe_expert_w& ew, const moe_shared_w* sw, uint16_t* y, const moe_taps* taps, char* ws,
                 const Layout& L) {
  FfnArgs a;
  memset(&a, 0, sizeof(a));
  a.M = M;
  a.H = d.hidden;
  a.E = d.n_experts;
  a.K = d.top_k;
  a.I = d.inter;
  a.Is = sw ? d.shared_inter : 0;
  a.x = x;
  a.mask = mask;
  a.ids = rt.topk_ids;
  a.w = rt.topk_w;
  a.n_union = rt.n_union;
  a.union_ids = rt.union_ids;
  a.offs = rt.offs;
  a.rows = rt.rows;
  a.slot_of = rt.slot_of;
  a.wg = ew.w_gate;
  a.wu = ew.w_up;
  a.wd = ew.w_down;
  a.sg = ew.s_gate;
  a.su = ew.s_up;
  a.sd = ew.s_down;
  if (sw) {
    a.wsg = sw->w_gate;
    a.wsu = sw->w_up;
    a.wsd = sw->w_down;
  }
  a.sched = reinterpret_cast<int32_t*>(ws + L.sched);
  a.mtile_offs = reinterpret_cast<int32_t*>(ws + L.mtile);
  a.xq = (taps && taps->x_codes) ? taps->x_codes : reinterpret_cast<uint8_t*>(ws + L.xq);
  a.xs = (taps && taps->x_scales) ? taps->x_scales : reinterpret_cast<float*>(ws + L.xs);
  a.hq = (taps && taps->h_codes) ? taps->h_codes : reinterpret_cast<uint8_t*>(ws + L.hq);
  a.hs = (taps && taps->h_scales) ? taps->h_scales : reinterpret_cast<float*>(ws + L.hs);
  a.hsh = reinterpret_cast<uint16_t*>(ws + L.hsh);
  a.S = reinterpret_cast<float*>(ws + L.S);
  a.D = reinterpret_cast<float*>(ws + L.D);
  a.split = L.split ? 1 : 0;
  a.part_gu = reinterpret_cast<float*>(ws + L.part_gu);
  a.part_sh = reinterpret_cast<float*>(ws + L.part_sh);
  a.part_d = reinterpret_cast<float*>(ws + L.part_d);
  a.part_s = reinterpret_cast<float*>(ws + L.part_s);
  a.y = y;
  return a;
}

// The timing hook's table, per host thread: calls from other threads are
// never traced.
struct Tracer {
  moe_event_pair* pairs = nullptr;
  int32_t cap = 0;
  int32_t* ids = nullptr;
  int32_t* count = nullptr;
};
thread_local Tracer g_trace;

const char* const kKernelNames[KID_COUNT] = {
    "router_logits", "route_select", "union", "quant_x", "plan", "gateup", "post_gateup",
    "down", "combine", "quant", "select_union", "front", "pack", "combine_norm", "add_rmsnorm",
    "sum_partials", "prefetch",
};

}  // namespace

namespace moe {

void trace_before(hipStream_t s) {
  if (g_trace.pairs && *g_trace.count < g_trace.cap)
    (void)hipEventRecord(static_cast<hipEvent_t>(g_trace.pairs[*g_trace.count].start), s);
}

void trace_after(int kid, hipStream_t s) {
  if (g_trace.pairs && *g_trace.count < g_trace.cap) {
    (void)hipEventRecord(static_cast<hipEvent_t>(g_trace.pairs[*g_trace.count].stop), s);
    g_trace.ids[*g_trace.count] = kid;
    ++*g_trace.count;
  }
}

}  // namespace moe

extern "C" {

int moe_trace_set(moe_event_pair* pairs, int32_t capacity, int32_t* kernel_ids, int32_t* count) {
  if (pairs == nullptr) {
    g_trace = Tracer();
    return MOE_OK;
  }
  if (capacity < 0 || kernel_ids == nullptr || count == nullptr) return MOE_EINVAL;
  g_trace.pairs = pairs;
  g_trace.cap = capacity;
  g_trace.ids = kernel_ids;
  g_trace.count = count;
  return MOE_OK;
}

const char* moe_kernel_name(int32_t kernel_id) {
  return (kernel_id >= 0 && kernel_id < KID_COUNT) ? kKernelNames[kernel_id] : "?";
}


size_t moe_workspace_bytes(const moe_dims* dims, int32_t max_rows) {
  if (check_dims(dims) != MOE_OK || check_rows(max_rows) != MOE_OK) return 0;
  // small steps keep per-segment partials, so the largest layout for M <=
  // max_rows is either at max_rows or at the largest split row count
  size_t need = make_layout(*dims, max_rows).total;
  const int cap = split_rows(dims->inter);
  const int split_m = max_rows < cap ? max_rows : cap;
  need = std::max(need, make_layout(*dims, split_m).total);
  return need;
}

int moe_route(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
              const moe_router_w* router, moe_routing* out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_rows(M)) != MOE_OK) return st;
  if (!router || !ok_ptr(router->w, 16) || !ok_ptr(router->bias, 4)) return MOE_EINVAL;
  if (!ok_ptr(x, 16) || (st = check_routing(out)) != MOE_OK) return st != MOE_OK ? st : MOE_EINVAL;
  if (!ok_ptr(ws, 16)) return MOE_EINVAL;
  if (M == 0) return MOE_OK;
  const Layout L = make_layout(*dims, M);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  char* w = static_cast<char*>(ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const RouteArgs a = route_args(*dims, M, x, row_mask, *router, *out, w, L);
  return to_status(launch_route(a, s));
}

int moe_ffn_fp8(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
                const moe_routing* in, const moe_expert_w* experts, uint16_t* y, moe_taps* taps, void* ws,
                size_t ws_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_rows(M)) != MOE_OK) return st;
  if ((st = check_routing(in)) != MOE_OK) return st;
  if ((st = check_experts(experts)) != MOE_OK) return st;
  if ((st = check_taps(taps)) != MOE_OK) return st;
  if (!ok_ptr(x, 16) || !ok_ptr(y, 16) || !ok_ptr(ws, 16)) return MOE_EINVAL;
  if (M == 0) return MOE_OK;
  const Layout L = make_layout(*dims, M);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  const FfnArgs a = ffn_args(*dims, M, x, row_mask, *in, *experts, nullptr, y, taps, static_cast<char*>(ws), L);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = to_status(launch_prep(a, s))) != MOE_OK) return st;
  if ((st = to_status(launch_plan(a, s))) != MOE_OK) return st;
  return to_status(launch_ffn(a, s));
}

}  // extern "C"

namespace {

// Pointers and eps of the residual add + RMSNorm epilogue: MOE_OK or MOE_EINVAL.
int check_norm(const uint16_t* residual, const uint16_t* gamma, float eps, const uint16_t* residual_out,
               const uint16_t* out) {
  if (!ok_ptr(residual, 16) || !ok_ptr(gamma, 16) || !ok_ptr(residual_out, 16) || !ok_ptr(out, 16))
    return MOE_EINVAL;
  if (!isfinite(eps) || eps < 0.0f) return MOE_EINVAL;
  return MOE_OK;
}

// moe_layer, with the combine optionally running the add + RMSNorm epilogue
// (nm != nullptr; y may then be null).
int static_scratch(void** out);

// ws == nullptr with use_static: the call runs in this GPU's static scratch
// array (resolved only after every other check has passed).
int layer_impl(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
               const moe_router_w* router, const moe_expert_w* experts, const moe_shared_w* shared, uint16_t* y,
               const NormArgs* nm, moe_routing* out, moe_taps* taps, void* ws, size_t ws_bytes, void* stream,
               bool use_static = false) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_rows(M)) != MOE_OK) return st;
  if (!router || !ok_ptr(router->w, 16) || !ok_ptr(router->bias, 4)) return MOE_EINVAL;
  if ((st = check_routing(out)) != MOE_OK) return st;
  if ((st = check_experts(experts)) != MOE_OK) return st;
  if ((st = check_taps(taps)) != MOE_OK) return st;
  if (dims->shared_inter > 0) {
    if ((st = check_shared(shared)) != MOE_OK) return st;
  } else {
    shared = nullptr;
  }
  if (!ok_ptr(x, 16) || (!use_static && !ok_ptr(ws, 16))) return MOE_EINVAL;
  if (nm ? !ok_opt(y, 16) : !ok_ptr(y, 16)) return MOE_EINVAL;
  if (M == 0) return MOE_OK;
  const Layout L = make_layout(*dims, M);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (use_static && (st = static_scratch(&ws)) != MOE_OK) return st;
  char* w = static_cast<char*>(ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const RouteArgs ra = route_args(*dims, M, x, row_mask, *router, *out, w, L);
  const FfnArgs a = ffn_args(*dims, M, x, row_mask, *out, *experts, shared, y, taps, w, L);
  if (a.split) {
    // one front launch computes the logits, quantizes x and streams the
    // shared expert's gate/up while the router runs
    if ((st = to_status(launch_front_split(ra, a, s))) != MOE_OK) return st;
  } else {
    if ((st = to_status(launch_prep(a, s))) != MOE_OK) return st;
    if ((st = to_status(launch_route(ra, s))) != MOE_OK) return st;
  }
  return to_status(launch_ffn(a, s, nm));
}

// ---------------------------------------------------------------- static scratch
// The workspace of moe_layer_static: one array of MOE_STATIC_WS_BYTES per GPU,
// part of the library's device code, so it exists on every GPU the library
// runs on until the process ends and no call ever allocates.  Host code must
// not use the symbol itself (on the host it is only a stand-in for the device
// address): the device address is looked up once per device, with that device
// current, and kept.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_WS_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch array (MOE_ELAUNCH if the HIP
// runtime cannot report the device or the symbol).
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ELAUNCH;
  if (dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ELAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
              const moe_router_w* router, const moe_expert_w* experts, const moe_shared_w* shared, uint16_t* y,
              moe_routing* out, moe_taps* taps, void* ws, size_t ws_bytes, void* stream) {
  return layer_impl(dims, M, x, row_mask, router, experts, shared, y, nullptr, out, taps, ws, ws_bytes, stream);
}

int moe_layer_static(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
                     const moe_router_w* router, const moe_expert_w* experts, const moe_shared_w* shared,
                     uint16_t* y, moe_routing* out, moe_taps* taps, void* stream) {
  return layer_impl(dims, M, x, row_mask, router, experts, shared, y, nullptr, out, taps, nullptr,
                    MOE_STATIC_WS_BYTES, stream, true);
}

int moe_layer_add_rmsnorm(const moe_dims* dims, int32_t M, const uint16_t* x, const uint8_t* row_mask,
                          const moe_router_w* router, const moe_expert_w* experts, const moe_shared_w* shared,
                          const uint16_t* residual, const uint16_t* gamma, float eps, uint16_t* y,
                          uint16_t* residual_out, uint16_t* out, moe_routing* routing, moe_taps* taps, void* ws,
                          size_t ws_bytes, void* stream) {
  const int st = check_norm(residual, gamma, eps, residual_out, out);
  if (st != MOE_OK) return st;
  NormArgs nm;
  nm.res = residual;
  nm.gamma = gamma;
  nm.eps = eps;
  nm.res_out = residual_out;
  nm.out = out;
  return layer_impl(dims, M, x, row_mask, router, experts, shared, y, &nm, routing, taps, ws, ws_bytes, stream);
}

int moe_add_rmsnorm(int32_t M, int32_t H, const uint16_t* y, const uint8_t* row_mask, const uint16_t* residual,
                    const uint16_t* gamma, float eps, uint16_t* residual_out, uint16_t* out, void* stream) {
  if (H <= 0 || H % 128) return MOE_EINVAL;
  int st = check_rows(M);
  if (st != MOE_OK) return st;
  if (!ok_ptr(y, 16)) return MOE_EINVAL;
  if ((st = check_norm(residual, gamma, eps, residual_out, out)) != MOE_OK) return st;
  if (M == 0) return MOE_OK;
  NormArgs nm;
  nm.res = residual;
  nm.gamma = gamma;
  nm.eps = eps;
  nm.res_out = residual_out;
  nm.out = out;
  return to_status(launch_add_rmsnorm(y, row_mask, M, H, nm, static_cast<hipStream_t>(stream)));
}

int moe_sum_partials(int32_t M, int32_t H, int32_t nsrc, const uint16_t* parts, const uint8_t* row_mask, uint16_t* y,
                     void* stream) {
  if (H <= 0 || H % 4 || nsrc < 1) return MOE_EINVAL;
  if (nsrc > 64) return MOE_EUNSUPPORTED;
  int st = check_rows(M);
  if (st != MOE_OK) return st;
  if (!ok_ptr(parts, 8) || !ok_ptr(y, 8)) return MOE_EINVAL;
  const uintptr_t a = (uintptr_t)parts, b = (uintptr_t)y;
  const uintptr_t na = (uintptr_t)M * nsrc * H * 2, nb = (uintptr_t)M * H * 2;
  if (M > 0 && a < b + nb && b < a + na) return MOE_EINVAL;     // overlapping buffers
  if (M == 0) return MOE_OK;
  return to_status(launch_sum_partials(parts, row_mask, M, H, nsrc, y, static_cast<hipStream_t>(stream)));
}

int moe_prefetch_experts(const moe_dims* dims, const int32_t* n_union, const int32_t* union_ids,
                         const moe_expert_w* experts, uint32_t parts, int64_t max_bytes, int32_t workgroups,
                         uint32_t* checksum, void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_experts(experts)) != MOE_OK) return st;
  if (!ok_ptr(n_union, 4) || !ok_ptr(union_ids, 4) || !ok_opt(checksum, 4)) return MOE_EINVAL;
  if (parts == 0 || (parts & ~(MOE_PREFETCH_GATE_UP | MOE_PREFETCH_DOWN)) != 0) return MOE_EINVAL;
  if (max_bytes < 0 || workgroups < 0) return MOE_EINVAL;
  if (workgroups > MOE_PREFETCH_MAX_WORKGROUPS) return MOE_EUNSUPPORTED;
  const uint8_t* mats[3];
  int nmat = 0;
  if (parts & MOE_PREFETCH_GATE_UP) {
    mats[nmat++] = experts->w_gate;
    mats[nmat++] = experts->w_up;
  }
  if (parts & MOE_PREFETCH_DOWN) mats[nmat++] = experts->w_down;
  const long mat_bytes = (long)dims->inter * dims->hidden;
  const long max_chunks = (long)(max_bytes / prefetch_chunk_bytes());
  if (max_chunks == 0) return MOE_OK;
  return to_status(launch_prefetch(n_union, union_ids, dims->n_experts, mats, nmat, mat_bytes, max_chunks,
                                   workgroups ? workgroups : 256, checksum, static_cast<hipStream_t>(stream)));
}

int moe_quant_fp8(const void* in, int32_t is_bf16, int32_t rows, int32_t cols, uint8_t* codes, float* scales,
                  void* stream) {
  if (rows < 0 || cols <= 0 || cols % 128) return MOE_EINVAL;
  if (rows > MOE_MAX_ROWS * MOE_MAX_TOPK) return MOE_EUNSUPPORTED;
  if (!ok_ptr(in, 16) || !ok_ptr(codes, 16) || !ok_ptr(scales, 4)) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  return to_status(
      launch_quant_generic(in, is_bf16 ? 1 : 0, rows, cols, codes, scales, static_cast<hipStream_t>(stream)));
}

int moe_pack_weights(const void* src, void* dst, int64_t rows, int32_t row_bytes, int32_t is_bf16, void* stream) {
  if (rows < 0 || rows % 16 || row_bytes <= 0 || row_bytes % 128) return MOE_EINVAL;
  if (!ok_ptr(src, 16) || !ok_ptr(dst, 16)) return MOE_EINVAL;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst, n = (uintptr_t)rows * (uintptr_t)row_bytes;
  if (n && a < b + n && b < a + n) return MOE_EINVAL;     // overlapping buffers
  if (rows == 0) return MOE_OK;
  return to_status(launch_pack(src, dst, (long)rows, row_bytes, is_bf16 ? 1 : 0, static_cast<hipStream_t>(stream)));
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported size";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
