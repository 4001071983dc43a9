// Device-side helpers shared by every kernel of the MoE FFN library (gfx950).
//
// Everything that decides a bit of a result lives here once, so that the
// decode and prefill kernels compute each output element by the same
// procedure: the e4m3 encoder, the bf16 rounding, the SiLU product, the
// per-K-block scale step and the MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kBlk = 128;       // quantization block (1x128 activations, 128x128 weights)
constexpr int kWave = 64;

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: values derived from it (work items, K ranges) then stay in scalar
// registers and the branches on them are scalar, which keeps the compiler's
// wait counting across those branches exact.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// ---------------------------------------------------------------- MFMA
// The matrix core does not interlock a vector-ALU, LDS or memory read of an
// MFMA result: such a reader has to issue a fixed number of wait states after
// the MFMA (12 for the fp8 16x16x128 form, 8 for bf16 16x16x32 on gfx950).
// The compiler pads this inside a basic block, but it was seen to leave a
// reader on a branch path 8 instructions behind the MFMA, which then read
// stale accumulator values.  So every result passes through an explicit wait
// tied to it (the asm both reads and "writes" the registers, so no reader can
// move above it), with margin over the required count.
__device__ __forceinline__ v4f settle_fp8(v4f p) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(p));       // 16 wait states
  return p;
}
__device__ __forceinline__ v4f settle_bf16(v4f p) {
  asm volatile("s_nop 7\n\ts_nop 3" : "+v"(p));       // 12 wait states
  return p;
}

// fp8 e4m3 x e4m3 -> fp32, 16x16 output, K = 128, zero initial accumulator.
// Operand layout (both operands): lane l holds 32 consecutive K values of
// row/column (l % 16), starting at K = 32 * (l / 16).
// Output layout: lane l holds C[4 * (l / 16) + i][l % 16], i = 0..3.
// The result is settled and may be read at once.
__device__ __forceinline__ v4f mfma_fp8_k128(const v8i& a, const v8i& b) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return settle_fp8(__builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0));
}

// bf16 x bf16 -> fp32, 16x16 output, K = 32, accumulating into c.
// Operand layout: lane l holds 8 consecutive K values of row/column (l % 16)
// starting at K = 8 * (l / 16).  Output layout as above.  The result may feed
// the next call's c directly; pass it through settle_bf16 before any other read.
__device__ __forceinline__ v4f mfma_bf16_k32(const v4i& a, const v4i& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                 c, 0, 0, 0);
}

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> OCP e4m3 (bias 7, max 448) code, round to nearest even; magnitudes
// at or above 448, infinities and NaN saturate to 448 with the sign kept.
// gfx950's v_cvt_pk_fp8_f32 rounds to nearest even into OCP e4m3 and agrees
// with the format's integer rounding (grid 2^-9 below 2^-6, 4 significant
// bits above, ties to even) for every fp32 of magnitude below 464, both
// signs, zeros and subnormals included (an exhaustive device check); the
// saturated magnitudes take the explicit code.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sat = ((b >> 24) & 0x80u) | 0x7eu;
  const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xffu;
  return (b & 0x7fffffffu) >= 0x43e00000u ? sat : hw;
}

// Per-block quantization scale: s = fl32(amax / 448), s = 1 for a zero block.
__device__ __forceinline__ float quant_scale(float amax) {
  return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
}

// Code of one value under scale s (zero blocks give code 0 via v = 0).
__device__ __forceinline__ uint32_t quant_code(float v, float s) {
  return f32_to_e4m3(__fdiv_rn(v, s));
}

// Router score of a float64 logit: sigmoid s = 1 / (1 + exp(-l)) and the
// selection score c = s + bias (a NaN score becomes -inf, so the selection
// stays defined).
__device__ __forceinline__ void route_score(double l, float bias, double& sig, double& c) {
  sig = 1.0 / (1.0 + exp(-l));
  const double cc = sig + (double)bias;
  c = (cc == cc) ? cc : -INFINITY;
}

// h = silu(g) * u in fp32, silu(g) = g / (1 + exp(-g)).
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float s = __fdiv_rn(g, 1.0f + expf(-g));
  return s * u;
}

// One K-block step of a block-scaled accumulation:
// acc = fma(s_a * s_w, partial, acc) for the 4 outputs of a lane.
__device__ __forceinline__ void scale_acc(v4f& acc, const v4f& p, float sa, float sw) {
  const float ss = sa * sw;
  acc[0] = __builtin_fmaf(ss, p[0], acc[0]);
  acc[1] = __builtin_fmaf(ss, p[1], acc[1]);
  acc[2] = __builtin_fmaf(ss, p[2], acc[2]);
  acc[3] = __builtin_fmaf(ss, p[3], acc[3]);
}

// ---------------------------------------------------------------- cross-lane, VALU only
// DPP lane patterns (within rows of 16 lanes) and the gfx950 row swaps move
// data between lanes without the LDS round trip of ds_bpermute.
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;       // lane i <-> 15 - i within 16
constexpr int kDppRowShr1 = 0x111;      // row_shr:n = 0x110 + n

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, true);
}

// max of a value over the wave.  The mirrors pair whole quads / halves after
// the quad steps, so every lane ends with the row maximum; each row swap puts
// the partner row's value in one of its two outputs (the lane's own value in
// the other), so taking the max over both covers either ordering.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v))));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(v, fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1])));
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(v, fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1])));
  return v;
}

__device__ __forceinline__ double u2_to_f64(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return u2_to_f64(dpp_u32<kCtrl>((uint32_t)b), dpp_u32<kCtrl>((uint32_t)(b >> 32)));
}

__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dpp_f64<kDppXor1>(v));
  v = fmax(v, dpp_f64<kDppXor2>(v));
  v = fmax(v, dpp_f64<kDppHalfMirror>(v));
  v = fmax(v, dpp_f64<kDppMirror>(v));
  {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    v = fmax(v, fmax(u2_to_f64(lo[0], hi[0]), u2_to_f64(lo[1], hi[1])));
  }
  {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    v = fmax(v, fmax(u2_to_f64(lo[0], hi[0]), u2_to_f64(lo[1], hi[1])));
  }
  return v;
}

// Inclusive prefix sum over the wave (unsigned, wrapping): Hillis-Steele
// shifts within each row of 16, then the totals of the rows below.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
  v += dpp_u32<kDppRowShr1>(v);           // row_shr with zero fill at the row start
  v += dpp_u32<kDppRowShr1 + 1>(v);
  v += dpp_u32<kDppRowShr1 + 3>(v);
  v += dpp_u32<kDppRowShr1 + 7>(v);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moe
