// Global -> LDS DMA and LDS transpose reads (gfx950), shared by the kernels
// that stage tiles in LDS.
#pragma once

#include "msa_common.h"

namespace msa {

typedef __attribute__((address_space(3))) char lds_char;

// Global -> LDS copy of 16 bytes per lane: lane L's bytes land at lds_dst +
// 16 L (lds_dst is wave-uniform).  Written as inline asm (M0 = LDS address,
// one wait state, the DMA; no register outputs) rather than the builtin,
// because the compiler treats a builtin DMA as a pending LDS write and waits
// for every one of them before any later LDS read, which would drain the
// tile ring on every block.  The callers order each stage's reads after its
// DMA themselves: an explicit vmcnt wait for this wave's own DMA, then a
// workgroup barrier for everyone else's.
// M0 is reserved to the compiler, which warns about the clobber; nothing in
// these kernels keeps a value in M0 across a DMA (every M0 write in the
// generated code is the one above its DMA).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* src, char* lds_dst) {
  const uint32_t lds_addr = uniform((uint32_t)(uintptr_t)(lds_char*)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate that waits until at most n of this wave's vector-memory
// operations are outstanding (lgkm and exp counters not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// 8-byte transposing LDS reads of 16-bit and of 8-bit elements
__device__ __forceinline__ u32x2 lds_tr_b16(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_char*)p);
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x2 lds_tr_b8(const char* p) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds_char*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Column swizzle of FP8 tiles (128-byte rows of e4m3): 16-byte column c of
// row pos is stored at c ^ fp8_vswz(pos), built from bits 1, 4 and 2 of pos,
// which keeps the rows of a transposing 8-bit read (ds_read_b64_tr_b8) in
// distinct bank groups.
__device__ __forceinline__ int fp8_vswz(int pos) {
  return ((pos >> 1) & 1) | (((pos >> 4) & 1) << 1) | (((pos >> 2) & 1) << 2);
}

}  // namespace msa
