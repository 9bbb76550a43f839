// insert.hip -- KV-insert: quantise the new tokens' K, V and indexer keys and
// write them into the paged caches (gfx950).
//
// [ainewsbites page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on NVIDIA
// and AMD GPUs": section "A model built for efficient inference", the model
// is trained for an NVFP4 KV cache; section "Kernel and serving
// optimizations", the KV-insert runs fused with the kernels that produce K
// and V.] The quantiser follows the NVFP4 storage the decode kernels read: a
// 4-bit E2M1 code per element and one E4M3 scale per 16-element group, the
// scale chosen so that the group's largest magnitude maps to E2M1's largest
// value 6; FP8 indexer keys carry one fp32 scale per token that maps the
// largest magnitude to E4M3's largest value 448.
//
// Work split: one workgroup per (sequence, KV head, chunk of 64 new tokens)
// for K and V, and one per (sequence, chunk) for the indexer keys (one wave
// per token, lane = dim; NVFP4 indexer keys use the K/V quantiser per group
// of 16 lanes). Every rounding decision is taken on IEEE double values, so
// it is exact for bf16 inputs with a unit tensor scale (a quotient of a bf16
// value by an E4M3 value never lies within double rounding of a midpoint
// unless it is one). In the dim-major V page one byte holds two consecutive tokens;
// each touched byte has one owning thread (the new token in its even slot,
// or the first new token when it starts in an odd slot), which merges the
// new nibbles with the kept one, so workgroups never write the same byte.
#include "fmt.hpp"
#include "msa_internal.hpp"

namespace msa {

namespace {

constexpr int kInsChunk = 64;  // new tokens per workgroup

// |a| -> E4M3 magnitude code: the nearest E4M3 value, ties to the even code,
// saturating at 448 (code 0x7E); 0 for a <= 0.
__device__ __forceinline__ uint32_t e4m3_mag_code(double a) {
  if (!(a > 0.0)) return 0u;
  if (a >= 448.0) return 0x7Eu;
  if (a < 0.015625) return (uint32_t)rint(a * 512.0);  // subnormals, step 2^-9 (8 -> 2^-6)
  int e;
  const double f = frexp(a, &e);  // a = f * 2^e, f in [0.5, 1)
  int E = e - 1;
  double m = rint((2.0 * f - 1.0) * 8.0);
  if (m >= 8.0) {  // rounded up to the next power of two
    m = 0.0;
    E += 1;
  }
  return (uint32_t)(((E + 7) << 3) | (int)m);  // a < 448 keeps this <= 0x7E
}

__device__ __forceinline__ double e4m3_mag_value(uint32_t c) {
  const int e = (int)((c >> 3) & 15u), m = (int)(c & 7u);
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

// |a| -> E2M1 magnitude code 0..7 (0, .5, 1, 1.5, 2, 3, 4, 6): the count of
// midpoints between consecutive values that a lies above, a midpoint itself
// going to the even code; saturates at 6.
__device__ __forceinline__ uint32_t e2m1_mag_code(double a) {
  constexpr double kVal[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 7; i++) {
    const double mid = 0.5 * (kVal[i] + kVal[i + 1]);
    c += (a > mid || (a == mid && ((i + 1) & 1) == 0)) ? 1u : 0u;
  }
  return c;
}

// One 16-element NVFP4 group from 16 bf16 values: y = x / ts, scale code =
// E4M3(max|y| / 6), codes E2M1(y / scale) (+0 when the scale is 0).
__device__ __forceinline__ void quant_group(const uint16_t* src, double ts, uint32_t& scode, uint32_t (&code)[16]) {
  const u32x4 w0 = reinterpret_cast<const u32x4*>(src)[0], w1 = reinterpret_cast<const u32x4*>(src)[1];
  double y[16];
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const uint32_t w = i < 8 ? w0[i >> 1] : w1[(i - 8) >> 1];
    const float x = bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xFFFFu));
    y[i] = (double)x / ts;
    amax = fmax(amax, fabs(y[i]));
  }
  scode = e4m3_mag_code(amax / 6.0);
  const double s = e4m3_mag_value(scode);
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const uint32_t mag = s > 0.0 ? e2m1_mag_code(fabs(y[i] / s)) : 0u;
    code[i] = mag | ((y[i] < 0.0 && mag != 0u) ? 8u : 0u);
  }
}

// Page and slot of new token t of sequence b, or page -1 when it is skipped.
__device__ __forceinline__ void token_slot(const InsertArgs& a, int b, int t, int& page, int& slot) {
  const int64_t pos = (int64_t)a.ctx_lens[b] - a.Tq + t;
  page = -1;
  slot = 0;
  if (pos < 0 || pos >= (int64_t)a.maxb * kBlock) return;
  const int pg = a.block_table[(size_t)b * a.maxb + (int)(pos / kBlock)];
  if (pg < 0 || pg >= a.num_pages) return;
  page = pg;
  slot = (int)(pos % kBlock);
}

__global__ __launch_bounds__(256) void insert_kernel(InsertArgs a) {
  __shared__ uint8_t vcode[kInsChunk + 1][kHeadDim];  // V codes of the chunk (+ the next token)
  __shared__ int32_t tpage[kInsChunk + 1], tslot[kInsChunk + 1];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / (a.Hkv + 1), j = blockIdx.x % (a.Hkv + 1);
  const int t0 = blockIdx.y * kInsChunk;
  const int nt = min(kInsChunk, a.Tq - t0);
  if (nt <= 0) return;

  if (j == a.Hkv) {
    // ---- indexer keys: one wave per token, lane = dim
    const int lane = lane_id(), wave = tid >> 6;
    for (int tl = wave; tl < nt; tl += 4) {
      int page, slot;
      token_slot(a, b, t0 + tl, page, slot);
      if (page < 0) continue;  // uniform over the wave
      const uint16_t bits = a.new_idx_k[((size_t)b * a.Tq + t0 + tl) * kIdxDim + lane];
      const size_t row = (size_t)page * kBlock + slot;
      if (a.idx_format == 0) {  // bf16
        reinterpret_cast<uint16_t*>(a.idx_k)[row * kIdxDim + lane] = bits;
        continue;
      }
      const float x = bf16_bits_to_f32(bits);
      if (a.idx_format == 1) {  // FP8, one fp32 scale per token
        float amax = fabsf(x);
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, shfl_xor(amax, m));
        const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
        const uint32_t mag = e4m3_mag_code(fabs((double)x / (double)s));
        a.idx_k[row * kIdxDim + lane] = (uint8_t)(mag | ((x < 0.0f && mag != 0u) ? 0x80u : 0u));
        if (lane == 0) static_cast<float*>(a.idx_k_scale)[row] = s;
        continue;
      }
      // NVFP4: the 16 lanes of a group share one E4M3 scale
      const double y = (double)x / a.idx_ts;
      double amax = fabs(y);
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) amax = fmax(amax, shfl_xor(amax, m));
      const uint32_t scode = e4m3_mag_code(amax / 6.0);
      const double s = e4m3_mag_value(scode);
      const uint32_t mag = s > 0.0 ? e2m1_mag_code(fabs(y / s)) : 0u;
      const uint32_t code = mag | ((y < 0.0 && mag != 0u) ? 8u : 0u);
      const uint32_t hi = (uint32_t)shfl_xor((int)code, 1);  // the odd dim's code
      if ((lane & 1) == 0) a.idx_k[row * (kIdxDim / 2) + lane / 2] = (uint8_t)(code | (hi << 4));
      if ((lane & 15) == 0) static_cast<uint8_t*>(a.idx_k_scale)[row * 4 + lane / 16] = (uint8_t)scode;
    }
    return;
  }

  // ---- K and V of KV head g
  const int g = j;
  const int ntv = min(kInsChunk + 1, a.Tq - t0);  // V codes also of the token after the chunk
  if (tid < ntv) {
    int page, slot;
    token_slot(a, b, t0 + tid, page, slot);
    tpage[tid] = page;
    tslot[tid] = slot;
  }
  __syncthreads();
  const size_t src0 = (size_t)b * a.Tq * a.Hkv;
  if (!a.nvfp4) {
    // bf16 cache: K token-major [slot][128], V dim-major [d][slot]
    for (int e = tid; e < nt * kHeadDim; e += 256) {
      const int tl = e / kHeadDim, d = e % kHeadDim;
      const int page = tpage[tl], slot = tslot[tl];
      if (page < 0) continue;
      const size_t src = ((src0 + (size_t)(t0 + tl) * a.Hkv + g) * kHeadDim) + d;
      const size_t pg = (size_t)page * a.Hkv + g;
      reinterpret_cast<uint16_t*>(a.k_data)[(pg * kBlock + slot) * kHeadDim + d] = a.new_k[src];
      reinterpret_cast<uint16_t*>(a.v_data)[(pg * kHeadDim + d) * kBlock + slot] = a.new_v[src];
    }
    return;
  }
  for (int pr = tid; pr < ntv * 8; pr += 256) {
    const int tl = pr >> 3, c = pr & 7;
    const size_t src = ((src0 + (size_t)(t0 + tl) * a.Hkv + g) * kHeadDim) + 16 * c;
    const int page = tpage[tl], slot = tslot[tl];
    const size_t pg = (size_t)(page < 0 ? 0 : page) * a.Hkv + g;
    uint32_t scode, code[16];
    if (tl < nt && page >= 0) {
      quant_group(a.new_k + src, a.k_ts, scode, code);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        lo |= code[i] << (4 * i);
        hi |= code[8 + i] << (4 * i);
      }
      *reinterpret_cast<uint2*>(a.k_data + pg * 8192 + slot * 64 + 8 * c) = make_uint2(lo, hi);
      a.k_scale[pg * 1024 + slot * 8 + c] = (uint8_t)scode;
    }
    quant_group(a.new_v + src, a.v_ts, scode, code);
#pragma unroll
    for (int i = 0; i < 16; i++) vcode[tl][16 * c + i] = (uint8_t)code[i];
    if (tl < nt && page >= 0) a.v_scale[pg * 1024 + c * 128 + slot] = (uint8_t)scode;
  }
  __syncthreads();
  // V codes: one owning thread per touched byte (dim d, slots 2i and 2i+1)
  for (int e = tid; e < nt * kHeadDim; e += 256) {
    const int tl = e / kHeadDim, d = e % kHeadDim;
    const int page = tpage[tl], slot = tslot[tl], t = t0 + tl;
    if (page < 0 || ((slot & 1) && t != 0)) continue;
    uint8_t* byte = a.v_data + ((size_t)page * a.Hkv + g) * 8192 + d * 64 + slot / 2;
    uint32_t v;
    if (slot & 1) {
      v = (*byte & 0x0Fu) | ((uint32_t)vcode[tl][d] << 4);
    } else {
      const uint32_t hi = t + 1 < a.Tq ? (uint32_t)vcode[tl + 1][d] : (uint32_t)(*byte >> 4);
      v = (uint32_t)vcode[tl][d] | (hi << 4);
    }
    *byte = (uint8_t)v;
  }
}

}  // namespace

hipError_t launch_insert(const InsertArgs& a, hipStream_t s) {
  if (a.B < 1 || a.Tq < 1 || a.Hkv < 1) return hipErrorInvalidValue;
  const int64_t chunks = ((int64_t)a.Tq + kInsChunk - 1) / kInsChunk;
  const int64_t gx = (int64_t)a.B * (a.Hkv + 1);
  if (chunks > 65535 || gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  insert_kernel<<<dim3((uint32_t)gx, (uint32_t)chunks), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace msa
