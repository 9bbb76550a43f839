// attn.hip -- exact attention over the selected blocks, NVFP4 (or bf16)
// paged K/V dequantised inside the kernel (gfx950).
//
// [ainewsbites page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on NVIDIA
// and AMD GPUs", section "A model built for efficient inference": main
// attention runs exactly over the top 16 blocks only, at most 2,048 keys per
// query; the KV cache is NVFP4. upstreambeat page "vLLM turns MiniMax's
// day-zero promise into GPU-specific serving code", section "What changed":
// NVFP4 is dequantised inside the sparse-attention kernels.]
//
// Work split. One workgroup per (sequence, query token, KV head) with W
// wavefronts; wave w takes the selected blocks w, w+W, ... and keeps an online
// softmax state (running max m, sum l, output O) for the G <= 16 query heads
// that share the KV head. The W states are merged in LDS by a fixed-order
// tree (log-sum-exp combine), so the result is bitwise reproducible.
//
// Per block (128 keys) and wave:
//   S^T = K Q^T    16x16x32 MFMA, A = K rows (keys), B = Q^T (heads): 8 key
//                  tiles x 4 steps over head_dim.
//   softmax        every lane holds one head (l%16) and 32 of the block's
//                  keys; max/sum across the 4 lanes of a head by xor-shuffles.
//   O^T += V^T P^T 16x16x32 MFMA, A = V^T rows (dims), B = P^T (keys x heads):
//                  8 dim tiles x 4 steps over the 128 keys.
// The lane layouts of v_mfma_f32_16x16x32_{f16,bf16} (checked on gfx950):
// lane l supplies A[row l%16][k = 8*(l/16) + e], B[k = 8*(l/16) + e][col l%16]
// and receives D[row 4*(l/16) + r][col l%16], r = 0..3.
// The keys of S^T tile tau, row rho are chosen as
//   kappa(tau, rho) = 32*(rho/4) + 8*(tau/2) + 4*(tau%2) + rho%4,
// which makes the S^T output of tiles 2s, 2s+1 exactly the P^T operand of PV
// step s, and makes the keys of PV step s for lane group q the contiguous
// run 32q + 8s .. 32q + 8s + 7 -- contiguous in the dim-major V page, so each
// lane fetches its V codes with one 16-byte load per dim tile.
//
// Numerics. NVFP4 codes and scales decode to fp16 exactly (product of an
// E2M1 and an E4M3 value), Q is converted bf16 -> fp16 (exact in range; rows
// with |q| >= 2^15 are pre-scaled by a power of two that the score scale
// undoes), P is rounded to fp16, every product accumulates in fp32, and the
// softmax runs in fp32 with exp2. The per-tensor K scale multiplies the score
// scale, the V scale multiplies the output.
#include "fmt.hpp"
#include "msa_internal.hpp"

namespace msa {

namespace {

constexpr int kSlotFloats = 16 * kHeadDim + 32;  // O[16][128], m[16], l[16]

__device__ __forceinline__ int kappa(int tau, int rho) {
  return 32 * (rho >> 2) + 8 * (tau >> 1) + 4 * (tau & 1) + (rho & 3);
}

template <bool NVFP4>
struct MfmaT;
template <>
struct MfmaT<true> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) { return f32x2_to_f16x2(x, y); }
};
template <>
struct MfmaT<false> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) { return f32x2_to_bf16x2(x, y); }
};

struct SoftmaxState {
  float m;       // running max (log2 domain), per head
  float l;       // this lane's share of the running sum
  f32x4 o[8];    // O^T tile delta: dims 16*delta + 4*(lane/16) + r, head lane%16
};

__device__ __forceinline__ float lse_weight(float m, float M) {
  return (m == -INFINITY) ? 0.0f : fast_exp2(m - M);
}

template <bool NVFP4, int W>
__global__ __launch_bounds__(64 * W) void sparse_attn_kernel(AttnArgs a) {
  typedef MfmaT<NVFP4> MT;
  typedef typename MT::vec vec;
  // per-wave fp16 V-scale staging during the scan; merge slots afterwards
  constexpr int kStageBytes = W * 1024 * 2;
  constexpr int kMergeBytes = (W / 2) * kSlotFloats * 4;
  constexpr int kLdsBytes = kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ int32_t blist[16], plist[16];
  __shared__ int32_t nlist;

  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int item = blockIdx.x;
  const int g = item % a.Hkv;
  const int bt = item / a.Hkv;
  const int t = bt % a.Tq, b = bt / a.Tq;
  const int Lc = clamp_ctx(a.ctx_lens[b], a.maxb);
  const int p = Lc - a.Tq + t;  // last visible key
  const int h = lane & 15;      // head within the group (MFMA column)
  const int q4 = lane >> 4;     // lane group 0..3

  // ---- selected blocks that exist: compacted, order kept
  if (wave == 0) {
    bool ok = false;
    int blk = -1, page = -1;
    if (lane < a.top_k && p >= 0) {
      blk = a.sel[(size_t)bt * a.top_k + lane];
      if (blk >= 0 && blk < a.maxb && blk * kBlock <= p) {
        page = a.block_table[(size_t)b * a.maxb + blk];
        ok = page >= 0 && page < a.num_pages;
      }
    }
    const uint64_t bal = __ballot(ok);
    if (ok) {
      const int pos = __popcll(bal & ((1ull << lane) - 1ull));
      blist[pos] = blk;
      plist[pos] = page;
    }
    if (lane == 0) nlist = __popcll(bal);
  }

  // ---- Q^T operand: head h, dims 32*q4 + 8s + e
  vec qb[4];
  float cscale;
  {
    const bool ok = h < a.grp;
    const uint16_t* qrow = a.q + ((size_t)bt * a.Hq + g * a.grp + h) * kHeadDim + 32 * q4;
    u32x4 raw[4];
#pragma unroll
    for (int s = 0; s < 4; s++) raw[s] = ok ? reinterpret_cast<const u32x4*>(qrow)[s] : u32x4{0, 0, 0, 0};
    if constexpr (NVFP4) {
      float amax = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; s++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint32_t w = raw[s][e];
          amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w & 0xFFFFu)), fabsf(bf16_bits_to_f32(w >> 16))));
        }
      amax = fmaxf(amax, shfl_xor(amax, 16));
      amax = fmaxf(amax, shfl_xor(amax, 32));
      // power-of-two pre-scale keeping the row inside fp16's range
      int sh = 0;
      if (amax >= 32768.0f) sh = ((int)((__float_as_uint(amax) >> 23) & 255) - 127) - 14;
      const float down = __uint_as_float((uint32_t)(127 - sh) << 23);
      cscale = a.score_scale * __uint_as_float((uint32_t)(127 + sh) << 23);
#pragma unroll
      for (int s = 0; s < 4; s++) {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint32_t w = raw[s][e];
          v[e] = f32x2_to_f16x2(bf16_bits_to_f32(w & 0xFFFFu) * down, bf16_bits_to_f32(w >> 16) * down);
        }
        qb[s] = __builtin_bit_cast(vec, v);
      }
    } else {
      cscale = a.score_scale;
#pragma unroll
      for (int s = 0; s < 4; s++) qb[s] = __builtin_bit_cast(vec, raw[s]);
    }
  }
  __syncthreads();
  const int n = nlist;

  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int d = 0; d < 8; d++) st.o[d] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // fp16 V scales of the current block: [8 groups][128 keys]
  f16* vs_stage = reinterpret_cast<f16*>(lds) + wave * 1024;

  for (int i = wave; i < n; i += W) {
    const int blk = blist[i];
    const size_t pg = (size_t)plist[i] * a.Hkv + g;
    const int rho = lane & 15;

    // ---- issue the block's loads
    u32x4 kd[8];
    uint32_t ksc[8];
    u32x4 vd[8];
    u32x4 vsraw;
    if constexpr (NVFP4) {
      const uint8_t* kb = a.k_data + pg * (kBlock * 64);
      const uint8_t* ks = a.k_scale + pg * (kBlock * 8);
#pragma unroll
      for (int tau = 0; tau < 8; tau++) {
        const int key = kappa(tau, rho);
        kd[tau] = *reinterpret_cast<const u32x4*>(kb + key * 64 + 16 * q4);
        ksc[tau] = *reinterpret_cast<const uint16_t*>(ks + key * 8 + 2 * q4);
      }
      const uint8_t* vb = a.v_data + pg * (kHeadDim * 64);
#pragma unroll
      for (int dt = 0; dt < 8; dt++) vd[dt] = *reinterpret_cast<const u32x4*>(vb + (16 * dt + rho) * 64 + 16 * q4);
      vsraw = *reinterpret_cast<const u32x4*>(a.v_scale + pg * 1024 + 16 * lane);
    }

    // ---- S^T = K Q^T for the 8 key tiles
    f32x4 sacc[8];
    if constexpr (NVFP4) {
#pragma unroll
      for (int tau = 0; tau < 8; tau++) {
        const uint32_t sc2 = fp8x2_f16x2<false>(ksc[tau]);  // groups 2*q4, 2*q4+1
        const uint32_t slo = bcast_lo16(sc2), shi = bcast_hi16(sc2);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; s++) {
          const u32x4 kv = nvfp4x8_f16(kd[tau][s], s < 2 ? slo : shi);
          acc = MT::mma(__builtin_bit_cast(vec, kv), qb[s], acc);
        }
        sacc[tau] = acc;
      }
    } else {
      const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k_data) + pg * (kBlock * kHeadDim);
#pragma unroll
      for (int tau = 0; tau < 8; tau++) {
        const u32x4* kr = reinterpret_cast<const u32x4*>(kb + kappa(tau, rho) * kHeadDim + 32 * q4);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; s++) acc = MT::mma(__builtin_bit_cast(vec, kr[s]), qb[s], acc);
        sacc[tau] = acc;
      }
    }

    // ---- V scales to fp16 in LDS (wave-private)
    if constexpr (NVFP4) {
      u32x4 lo, hi;
      lo = fp8x8_f16(vsraw.x, vsraw.y);
      hi = fp8x8_f16(vsraw.z, vsraw.w);
      u32x4* dst = reinterpret_cast<u32x4*>(vs_stage + 16 * lane);
      dst[0] = lo;
      dst[1] = hi;
      wave_lds_sync();
    }

    // ---- online softmax over the block (log2 domain)
    float bmax = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 8; tau++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int pos = blk * kBlock + kappa(tau, 4 * q4 + r);
        const float v = (pos <= p) ? sacc[tau][r] * cscale : -INFINITY;
        sacc[tau][r] = v;
        bmax = fmaxf(bmax, v);
      }
    bmax = fmaxf(bmax, shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, shfl_xor(bmax, 32));
    const float mnew = fmaxf(st.m, bmax);
    const float alpha = lse_weight(st.m, mnew);
    float psum = 0.0f;
    vec pb[4];
#pragma unroll
    for (int s = 0; s < 4; s++) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        pv[e] = fast_exp2(sacc[2 * s + (e >> 2)][e & 3] - mnew);
        psum += pv[e];
      }
      u32x4 pk;
      pk.x = MT::pack(pv[0], pv[1]);
      pk.y = MT::pack(pv[2], pv[3]);
      pk.z = MT::pack(pv[4], pv[5]);
      pk.w = MT::pack(pv[6], pv[7]);
      pb[s] = __builtin_bit_cast(vec, pk);
    }
    st.l = st.l * alpha + psum;
    st.m = mnew;
#pragma unroll
    for (int d = 0; d < 8; d++) st.o[d] *= alpha;

    // ---- O^T += V^T P^T
    if constexpr (NVFP4) {
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
          const u32x4 sc = *reinterpret_cast<const u32x4*>(vs_stage + dt * 128 + 32 * q4 + 8 * s);
          const u32x4 vv = nvfp4x8_f16_each(vd[dt][s], sc);
          st.o[dt] = MT::mma(__builtin_bit_cast(vec, vv), pb[s], st.o[dt]);
        }
      }
      wave_lds_sync();  // the stage is overwritten by the next block
    } else {
      const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.v_data) + pg * (kHeadDim * kBlock);
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const u32x4* vr = reinterpret_cast<const u32x4*>(vb + (16 * dt + rho) * kBlock + 32 * q4);
#pragma unroll
        for (int s = 0; s < 4; s++) st.o[dt] = MT::mma(__builtin_bit_cast(vec, vr[s]), pb[s], st.o[dt]);
      }
    }
  }

  // ---- full row sum of this wave (the 4 lanes of a head)
  st.l += shfl_xor(st.l, 16);
  st.l += shfl_xor(st.l, 32);

  // ---- merge the W wave states: fixed tree, LDS slots
  float* slots = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int step = W / 2; step >= 1; step >>= 1) {
    __syncthreads();
    if (wave >= step && wave < 2 * step) {
      float* sl = slots + (wave - step) * kSlotFloats;
#pragma unroll
      for (int d = 0; d < 8; d++) *reinterpret_cast<f32x4*>(sl + h * kHeadDim + 16 * d + 4 * q4) = st.o[d];
      if (q4 == 0) {
        sl[16 * kHeadDim + h] = st.m;
        sl[16 * kHeadDim + 16 + h] = st.l;
      }
    }
    __syncthreads();
    if (wave < step) {
      const float* sl = slots + wave * kSlotFloats;
      const float m2 = sl[16 * kHeadDim + h], l2 = sl[16 * kHeadDim + 16 + h];
      const float M = fmaxf(st.m, m2);
      const float a1 = lse_weight(st.m, M), a2 = lse_weight(m2, M);
#pragma unroll
      for (int d = 0; d < 8; d++) {
        const f32x4 o2 = *reinterpret_cast<const f32x4*>(sl + h * kHeadDim + 16 * d + 4 * q4);
        st.o[d] = st.o[d] * a1 + o2 * a2;
      }
      st.l = st.l * a1 + l2 * a2;
      st.m = M;
    }
  }

  // ---- write bf16 output (and lse) for the real heads
  if (wave == 0 && h < a.grp) {
    const size_t row = (size_t)bt * a.Hq + g * a.grp + h;
    const bool empty = !(st.l > 0.0f);
    const float inv = empty ? 0.0f : a.v_scale_mul / st.l;
    uint16_t* orow = a.out + row * kHeadDim;
#pragma unroll
    for (int d = 0; d < 8; d++) {
      const f32x4 o = st.o[d];
      uint2 pk;
      pk.x = f32x2_to_bf16x2(o[0] * inv, o[1] * inv);
      pk.y = f32x2_to_bf16x2(o[2] * inv, o[3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * d + 4 * q4) = pk;
    }
    if (a.lse && q4 == 0) a.lse[row] = empty ? -INFINITY : (st.m + __log2f(st.l)) * 0.69314718055994530942f;
  }
}

template <bool NVFP4>
hipError_t launch_w(const AttnArgs& a, int waves, hipStream_t s) {
  const dim3 grid(a.B * a.Tq * a.Hkv);
  switch (waves) {
    case 1: sparse_attn_kernel<NVFP4, 1><<<grid, 64, 0, s>>>(a); break;
    case 2: sparse_attn_kernel<NVFP4, 2><<<grid, 128, 0, s>>>(a); break;
    case 4: sparse_attn_kernel<NVFP4, 4><<<grid, 256, 0, s>>>(a); break;
    case 8: sparse_attn_kernel<NVFP4, 8><<<grid, 512, 0, s>>>(a); break;
    case 16: sparse_attn_kernel<NVFP4, 16><<<grid, 1024, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, bool nvfp4, int waves, hipStream_t s) {
  return nvfp4 ? launch_w<true>(a, waves, s) : launch_w<false>(a, waves, s);
}

}  // namespace msa
