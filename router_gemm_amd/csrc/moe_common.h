// moe_common.h -- device helpers shared by the gfx950 kernels of the MoE layer:
// number formats, MFMA wrappers, wave reductions, launch-side structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "moe_kernels.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kWave = 64;
constexpr float kFp8Max = 448.0f;  // largest finite OCP E4M3FN value

// ---------------------------------------------------------------- formats

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// binary32 -> bf16, round to nearest even (NaN stays NaN): gfx950's
// conversion instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two binary32 values -> two bf16 codes (a in the low 16 bits), one packed
// conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Two binary32 values -> two E4M3FN codes in the low 16 bits.  The hardware
// conversion rounds to nearest even; values are clamped to +-448 first so that
// out-of-range magnitudes saturate instead of becoming NaN.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -kFp8Max), kFp8Max);
  b = __builtin_fminf(__builtin_fmaxf(b, -kFp8Max), kFp8Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four binary32 values -> four E4M3FN codes packed little-endian.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  return f32x2_to_e4m3(a, b) | (f32x2_to_e4m3(c, d) << 16);
}

// Four values of a 1x128 group -> four E4M3FN codes: code = RNE(v / s) with
// an IEEE binary32 division (not a multiply by a reciprocal, whose last bit
// can move a quotient across an e4m3 rounding boundary), saturating.
__device__ __forceinline__ uint32_t quant4_e4m3(float a, float b, float c, float d, float s) {
  return f32x4_to_e4m3(__fdiv_rn(a, s), __fdiv_rn(b, s), __fdiv_rn(c, s), __fdiv_rn(d, s));
}

// Scale of a 1x128 group: amax / 448 with an IEEE binary32 division; 1 for an
// all-zero group.
__device__ __forceinline__ float group_scale(float amax) {
  return amax == 0.0f ? 1.0f : __fdiv_rn(amax, kFp8Max);
}

// silu(z) * u for the SwiGLU epilogue, with the hardware exp and reciprocal
// (h is not compared bit for bit; its rounding error is ~1e-7 relative).
__device__ __forceinline__ float swiglu(float z, float u) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)) * u;
}

// ---------------------------------------------------------------- MFMA

// D(16x16, f32) += A(16x32 bf16) * B(32x16 bf16).  Lane l supplies row (A) /
// column (B) l%16 and 8 consecutive k; lane l receives D[4*(l/16)+r][l%16].
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, f32) = A(16x128 e4m3) * B(128x16 e4m3) + C, unscaled (OCP E4M3 for
// both operands).  Lane l supplies row/column l%16 and 32 codes of k.
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// (16x16, f32) = A(16x128 E2M1, per-lane E8M0 scale sa) * B(128x16 e4m3),
// returned unscaled by the B side (its scale byte is 127, i.e. 1).  Lane l of A
// supplies row l%16 and inputs 32(l/16)..+31 (16 bytes, the stored packing);
// of B, column l%16 and inputs 16(l/16)..+15 (blo) and 64+16(l/16)..+15 (bhi).
__device__ __forceinline__ f32x4 mfma_mx(const i32x4 &a, const i32x4 &blo, const i32x4 &bhi, int sa) {
  const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const i32x8 b8 = {blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 0, 0, sa, 0, 127);
}

// ---------------------------------------------------------------- waves

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x / kWave); }

__device__ __forceinline__ float wave_xor_max(float v, int width) {
  for (int o = 1; o < width; o <<= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---------------------------------------------------------------- memory

__device__ __forceinline__ i32x4 load16(const void *p) { return *reinterpret_cast<const i32x4 *>(p); }
__device__ __forceinline__ void store16(void *p, const i32x4 &v) { *reinterpret_cast<i32x4 *>(p) = v; }

// ---------------------------------------------------------------- LDS staging

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// Copy 16 bytes per lane from global memory to LDS at base + 16 * lane.
__device__ __forceinline__ void dma16(const void *g, uint8_t *lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void *)g, (lds_void *)lds_base, 16, 0, 0);
}
// As dma16, with the non-temporal cache policy (the "nt" bit, aux = 2): for
// data read exactly once per line, so that streaming it does not evict lines
// that are still being reused (scale words, token rows).
__device__ __forceinline__ void dma16_stream(const void *g, uint8_t *lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void *)g, (lds_void *)lds_base, 16, 0, 2);
}
// Copy 4 bytes per lane to LDS at base + 4 * lane.
__device__ __forceinline__ void dma4(const void *g, uint8_t *lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void *)g, (lds_void *)lds_base, 4, 0, 0);
}

// The same copies through a buffer resource: base address and size in four
// SGPRs, a per-lane 32-bit byte offset (voff) and a wave-uniform one (soff),
// so that a copy inside a loop needs one VGPR and no 64-bit address.  Word 3
// is the gfx9 descriptor with a 32-bit data format (a zero format reads 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_base, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void bdma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_base, 4, (int)voff, (int)soff, 0, 0);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0], [15:14]).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt vmcnt(N) lgkmcnt(0).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// s_waitcnt lgkmcnt(0) only (LDS and scalar-memory operations complete).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// Workgroup barrier without a memory fence (the direct-to-LDS copies are
// waited for explicitly with vmcnt); the empty asm keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS rows of 128 bytes with the 16-byte column XOR-swizzled by row % 8, so
// that MFMA operand reads of 8 consecutive rows hit distinct banks.
__device__ __forceinline__ int swz_f(int row) { return row & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ swz_f(row)) << 4); }

// Row offset e of an expert group: G.off[e], or, for a group given without an
// offsets array (one expert holding every row), 0 / nrows.
__device__ __forceinline__ int group_off(const FfnGroup &G, int e) {
  return G.off ? G.off[e] : (e == 0 ? 0 : G.nrows);
}

// A value the compiler may keep in a scalar register (uniform across the wave).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }


}  // namespace moe
