// fmt.hpp -- device-side decoders and small helpers shared by the MSA kernels
// (gfx950 / CDNA4).
//
// NVFP4 [ainewsbites page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on
// NVIDIA and AMD GPUs", section "A model built for efficient inference": the
// KV cache is NVFP4; upstreambeat page, section "What changed": it is
// dequantised inside the kernels]. An element is a 4-bit E2M1 code times the
// OCP E4M3 scale of its 16-element group. The product of a 2-significant-bit
// E2M1 value and a 4-significant-bit E4M3 scale has at most 6 significant
// bits and lies in [2^-10, 2688], so it is exact in fp16: the kernels decode
// codes and scales to fp16 with the gfx950 hardware converters (scale operand
// 1.0, i.e. no extra exponent shift) and multiply them with v_pk_mul_f16.
// FP8 E4M3 indexer keys decode exactly to bf16 with the hardware converter.
//
// The packed-result conversion builtins are always consumed as whole 32-bit
// registers (bit_cast of the 2-element vector); taking single elements out of
// their results mis-compiles on this toolchain.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef _Float16 f16;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kBlock = 128;
constexpr int kHeadDim = 128;
constexpr int kIdxDim = 64;
constexpr int kWave = 64;

// ---------------------------------------------------------------- NVFP4

// Two E2M1 codes held in byte SEL of `w` (even element in the low nibble)
// -> packed fp16 pair (low half = even element).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((int)w, 1.0f, SEL));
}

// Eight E2M1 codes (one dword, element i in nibble i) -> 8 fp16 as 4 dwords.
__device__ __forceinline__ u32x4 fp4x8_f16x8(uint32_t w) {
  u32x4 r;
  r.x = fp4x2_f16x2<0>(w);
  r.y = fp4x2_f16x2<1>(w);
  r.z = fp4x2_f16x2<2>(w);
  r.w = fp4x2_f16x2<3>(w);
  return r;
}

// Two E4M3 bytes held in 16-bit word HI of `w` -> packed fp16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI));
}

// Two E4M3 bytes held in 16-bit word HI of `w` -> packed bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// Packed fp16 multiply (v_pk_mul_f16): exact for E2M1 x E4M3 products.
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, uint32_t b) {
  f16x2 r = __builtin_bit_cast(f16x2, a) * __builtin_bit_cast(f16x2, b);
  return __builtin_bit_cast(uint32_t, r);
}

// Broadcast the low / high fp16 of a packed pair into both halves. Written
// as a vector shuffle, so that a packed fp16 operation consuming it takes
// the half through its operand-select bits instead of a separate permute.
__device__ __forceinline__ uint32_t bcast_lo16(uint32_t x) {
  const f16x2 v = __builtin_bit_cast(f16x2, x);
  return __builtin_bit_cast(uint32_t, (f16x2)__builtin_shufflevector(v, v, 0, 0));
}
__device__ __forceinline__ uint32_t bcast_hi16(uint32_t x) {
  const f16x2 v = __builtin_bit_cast(f16x2, x);
  return __builtin_bit_cast(uint32_t, (f16x2)__builtin_shufflevector(v, v, 1, 1));
}

// Eight NVFP4 elements of one scale group: codes (dword) times the scale
// given as a broadcast fp16 pair -> 8 fp16 (exact).
__device__ __forceinline__ u32x4 nvfp4x8_f16(uint32_t codes, uint32_t scale2) {
  u32x4 v = fp4x8_f16x8(codes);
  v.x = mul_f16x2(v.x, scale2);
  v.y = mul_f16x2(v.y, scale2);
  v.z = mul_f16x2(v.z, scale2);
  v.w = mul_f16x2(v.w, scale2);
  return v;
}

// Eight NVFP4 elements with one scale each: codes (dword, element i in nibble
// i) times scales (8 fp16 as 4 packed dwords, element i in half i).
__device__ __forceinline__ u32x4 nvfp4x8_f16_each(uint32_t codes, u32x4 scales) {
  u32x4 v = fp4x8_f16x8(codes);
  v.x = mul_f16x2(v.x, scales.x);
  v.y = mul_f16x2(v.y, scales.y);
  v.z = mul_f16x2(v.z, scales.z);
  v.w = mul_f16x2(v.w, scales.w);
  return v;
}

// Eight E4M3 bytes (two dwords) -> 8 bf16 (exact).
__device__ __forceinline__ u32x4 fp8x8_bf16(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r.x = fp8x2_bf16x2<false>(lo);
  r.y = fp8x2_bf16x2<true>(lo);
  r.z = fp8x2_bf16x2<false>(hi);
  r.w = fp8x2_bf16x2<true>(hi);
  return r;
}

// Eight E4M3 bytes (two dwords) -> 8 fp16 (exact).
__device__ __forceinline__ u32x4 fp8x8_f16(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r.x = fp8x2_f16x2<false>(lo);
  r.y = fp8x2_f16x2<true>(lo);
  r.z = fp8x2_f16x2<false>(hi);
  r.w = fp8x2_f16x2<true>(hi);
  return r;
}

// ---------------------------------------------------------------- buffers

// Raw buffer resource over [base, base + bytes): loads beyond `bytes` return
// zero without touching memory. Word 3 is the gfx9-family raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache policy bits of buffer loads (gfx94x/gfx950): nontemporal.
constexpr int kAuxNT = 2;

template <int AUX>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX));
}
template <int AUX>
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, AUX));
}
template <int AUX>
__device__ __forceinline__ float buf_load4f(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, AUX));
}

// ---------------------------------------------------------------- floats

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float a, float b) {
  f16x2 r;
  r[0] = (f16)a;
  r[1] = (f16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Two fp32 -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
}

// Order-preserving map of a float to uint32 (-0 treated as +0):
// a < b  <=>  ord(a) < ord(b) for non-NaN values.
__device__ __forceinline__ uint32_t float_ord(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-scope ordering of LDS traffic between the lanes of one wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Clamped context length and query position helpers (device contract of
// msa.h: lengths above max_blocks*128 are clamped).
__device__ __forceinline__ int clamp_ctx(int L, int max_blocks) {
  int cap = max_blocks * kBlock;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

}  // namespace msa
