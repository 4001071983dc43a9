// Route-ahead expert prefetch (MoE-Infinity PR #140, route-ahead expert
// prefetch commit: the union of the routed experts a coming block will use is
// fetched ahead of the block, while other work runs).  Here the experts are
// already resident in HBM; what can be fetched ahead is their packed weight
// bytes into the memory-side Infinity Cache, which every HBM read passes
// through.  The kernel reads the listed experts' matrices and keeps nothing
// but an optional 32-bit word sum of what it read.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kPfThreads = 256;
constexpr int kPfUnroll = 4;
// bytes one work-group reads per iteration; every matrix holds I*H bytes with
// I and H multiples of 128, so a whole number of these chunks
constexpr long kPfChunk = (long)kPfThreads * kPfUnroll * 16;

__device__ inline uint32_t word_sum(const uint4& v) { return v.x + v.y + v.z + v.w; }

// Chunk c of the fetch order: union entry u = c / (nmat * cpm) in ascending
// position, its matrices in the order m0, m1, m2 (those passed), each read in
// address order.  Entries outside [0, E) are skipped; n_union is clamped to
// [0, E].  The grid strides over the first `chunks` chunks.
__global__ __launch_bounds__(kPfThreads) void k_prefetch(const int32_t* n_union, const int32_t* union_ids, int E,
                                                         const uint8_t* m0, const uint8_t* m1, const uint8_t* m2,
                                                         int nmat, long mat_bytes, long max_chunks,
                                                         uint32_t* checksum) {
  const int nu = min(max(*n_union, 0), E);
  const long cpm = mat_bytes / kPfChunk;
  const long chunks = min((long)nu * nmat * cpm, max_chunks);
  uint32_t acc = 0;
  for (long c = blockIdx.x; c < chunks; c += gridDim.x) {
    const long j = c / cpm;
    const long within = c - j * cpm;
    const int u = (int)(j / nmat);
    const int m = (int)(j - (long)u * nmat);
    const int e = union_ids[u];
    if (e < 0 || e >= E) continue;
    const uint8_t* base = m == 0 ? m0 : (m == 1 ? m1 : m2);
    const uint4* p = reinterpret_cast<const uint4*>(base + (size_t)e * mat_bytes + within * kPfChunk) + threadIdx.x;
    uint4 v[kPfUnroll];
#pragma unroll
    for (int i = 0; i < kPfUnroll; ++i) v[i] = p[i * kPfThreads];
#pragma unroll
    for (int i = 0; i < kPfUnroll; ++i) acc += word_sum(v[i]);
  }
  if (checksum == nullptr) return;
  // wave sum, then one device-scope add per wave (vector atomic)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) atomicAdd(checksum, acc);
}

}  // namespace

long prefetch_chunk_bytes() { return kPfChunk; }

hipError_t launch_prefetch(const int32_t* n_union, const int32_t* union_ids, int E, const uint8_t* const* mats,
                           int nmat, long mat_bytes, long max_chunks, int workgroups, uint32_t* checksum,
                           hipStream_t s) {
  MOE_LAUNCH(KID_PREFETCH, k_prefetch, dim3((unsigned)workgroups), dim3(kPfThreads), 0, s, n_union, union_ids, E,
             mats[0], nmat > 1 ? mats[1] : mats[0], nmat > 2 ? mats[2] : mats[0], nmat, mat_bytes, max_chunks,
             checksum);
  return hipSuccess;
}

}  // namespace moe
