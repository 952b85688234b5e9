// Device helpers shared by the MSA kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand layout used throughout (v_mfma_f32_16x16x32_bf16):
//   A (16 x 32, M x K): lane l holds A[l % 16][8 * (l / 16) + j], j = 0..7
//   B (32 x 16, K x N): lane l holds B[8 * (l / 16) + j][l % 16], j = 0..7
//   C (16 x 16)       : lane l holds C[4 * (l / 16) + i][l % 16], i = 0..3
// The K index is a dummy summation index, so any bijection between (lane
// group, j) and the contracted dimension works as long as A and B agree;
// the kernels use that freedom to read memory in wide contiguous pieces.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;  // tokens per block == tokens per page
constexpr int kDim = 128;    // head dim
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Number of set bits of the 64-bit wave mask in lanes below this one.
__device__ __forceinline__ int mask_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

template <typename T>
__device__ __forceinline__ T uniform(T x) {
  return __builtin_amdgcn_readfirstlane(x);
}

// 16-byte and 8-byte global loads of raw bits.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Two floats -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Four e4m3fn bytes (one dword) -> four bf16 (two dwords), exact widening.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Eight e4m3fn bytes -> eight bf16 (one MFMA operand).
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 w) {
  u32x2 a = fp8x4_to_bf16x4(w.x), b = fp8x4_to_bf16x4(w.y);
  return u32x4{a.x, a.y, b.x, b.y};
}

// Low (sel = 0) or high (sel = 1) 16-bit halves of x and y packed as
// (x_half | y_half << 16).
__device__ __forceinline__ uint32_t pick_halves(uint32_t x, uint32_t y, int odd) {
  return __builtin_amdgcn_perm(y, x, odd ? 0x07060302u : 0x05040100u);
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (the four row groups of
// an MFMA C tile that share a column), with the gfx950 VALU lane swaps:
// v_permlane16_swap(x, x) leaves {x[l], x[l ^ 16]} in its two results (in
// either order, measured on every lane) and v_permlane32_swap likewise
// {x[l], x[l ^ 32]}, so one max or add of the pair is a butterfly step --
// a few cycles, where a cross-row shuffle would go through the LDS crossbar.
__device__ __forceinline__ float xor16_max(float x) {
  const u32x2 s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s.x), __uint_as_float(s.y));
}
__device__ __forceinline__ float xor32_max(float x) {
  const u32x2 s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s.x), __uint_as_float(s.y));
}
__device__ __forceinline__ float colgroup_max(float x) { return xor32_max(xor16_max(x)); }
__device__ __forceinline__ float colgroup_sum(float x) {
  const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a.x) + __uint_as_float(a.y);
  const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b.x) + __uint_as_float(b.y);
}

// Order-preserving map float -> uint32 (larger float, larger key); -0 and +0
// map to the same key so that equal scores tie exactly.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Records `bit` (kErrPage, kErrLength) in the device error word (rare paths
// only; null: not reported).
__device__ __forceinline__ void report_error(uint32_t* err, uint32_t bit) {
  if (err) __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 2^x with the hardware instruction (v_exp_f32): exact at 0, 0 at -inf,
// ~1 ulp elsewhere; results below the normal range flush to 0, which only
// affects probabilities under 2^-126.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace msa
