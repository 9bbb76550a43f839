// attn_impl.hpp -- device code of the MSA sparse attention (gfx950); the
// design is described at the top of attn.hip. The pieces (query operand,
// block streaming with the online softmax, the merge of wave states, the
// output) are used by the attention kernel (attn_body) and by the
// single-launch decode layer (layer.hip), which splits an item's blocks
// over several workgroups.
#pragma once
#include "fmt.hpp"
#include "msa_internal.hpp"
#include "topk.hpp"

namespace msa {

namespace {


constexpr int kSlotFloats = 16 * kHeadDim + 32;  // O[16][128], m[16], l[16]

__device__ __forceinline__ int kappa(int tau, int rho) {
  return 32 * (rho >> 2) + 8 * (tau >> 1) + 4 * (tau & 1) + (rho & 3);
}
// kappa(tau, rho) = krow(rho) + ktau(tau)
__host__ __device__ constexpr int ktau(int tau) { return 8 * (tau >> 1) + 4 * (tau & 1); }

template <bool NVFP4>
struct MfmaT;
template <>
struct MfmaT<true> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) { return f32x2_to_f16x2(x, y); }
  // acc + both halves of a packed pair (v_dot2_f32_f16 against ones)
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), f16x2{(f16)1.0f, (f16)1.0f}, acc, false);
  }
};
template <>
struct MfmaT<false> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) { return f32x2_to_bf16x2(x, y); }
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    return acc + bf16_bits_to_f32(p & 0xFFFFu) + bf16_bits_to_f32(p >> 16);
  }
};

struct SoftmaxState {
  float m;       // running max (log2 domain), per head
  float l;       // this lane's share of the running sum
  f32x4 o[8];    // O^T tile delta: dims 16*delta + 4*(lane/16) + r, head lane%16
};

__device__ __forceinline__ float lse_weight(float m, float M) {
  return (m == -INFINITY) ? 0.0f : fast_exp2(m - M);
}

// ---------------------------------------------------------------- NVFP4 I/O

// Buffer resources of one block of one KV head (K codes, K scales, V codes,
// V scales); empty ranges when `none`.
struct KvRsrc {
  __amdgpu_buffer_rsrc_t kd, ks, vd, vs;
};
__device__ __forceinline__ KvRsrc nvfp4_rsrc(const AttnArgs& a, int page, int g, bool none) {
  const size_t pg = (size_t)(none ? 0 : page) * a.Hkv + g;
  const uint32_t n8k = none ? 0u : 8192u, n1k = none ? 0u : 1024u;
  KvRsrc r;
  r.kd = make_rsrc(a.k_data + pg * 8192, n8k);
  r.ks = make_rsrc(a.k_scale + pg * 1024, n1k);
  r.vd = make_rsrc(a.v_data + pg * 8192, n8k);
  r.vs = make_rsrc(a.v_scale + pg * 1024, n1k);
  return r;
}

// This lane's share of a block: K codes of key kappa(tau, l%16), dims
// 32*(l/16) .. +31 (16 bytes), and 16 bytes of the [128][8] K scale array
// (the scales a lane uses lie 32 bytes apart: the wave loads the whole array
// with one instruction and exchanges it through LDS, where eight 2-byte loads
// per block cost more vector memory issue); V codes of dim 16*dt + l%16,
// tokens 32*(l/16) .. +31, and 16 bytes of the [8][128] V scale array.
struct KRegs {
  u32x4 kd[8];
  u32x4 ks;
};
struct VRegs {
  u32x4 vd[8];
  u32x4 vs;
};
struct LaneOff {
  uint32_t k, ks, v, vs;
};

__device__ __forceinline__ void load_k(const KvRsrc& r, const LaneOff& o, KRegs& K) {
#pragma unroll
  for (int tau = 0; tau < 8; tau++) {
    K.kd[tau] = buf_load16<kAuxNT>(r.kd, o.k, (uint32_t)(64 * ktau(tau)));
  }
  K.ks = buf_load16<kAuxNT>(r.ks, o.ks, 0);
}
__device__ __forceinline__ void load_v(const KvRsrc& r, const LaneOff& o, VRegs& V) {
#pragma unroll
  for (int dt = 0; dt < 8; dt++) V.vd[dt] = buf_load16<kAuxNT>(r.vd, o.v, (uint32_t)(1024 * dt));
  V.vs = buf_load16<kAuxNT>(r.vs, o.vs, 0);
}

// ---------------------------------------------------------------- pieces

// Raw Q^T operand of this lane: head g*grp + lane%16 of row bt, dims
// 32*(lane/16) + 8s + e; zero for lanes past the group's heads. The group's
// rows are one buffer range and those lanes read past its end (zeros), so
// the loads take no branch: a branch around them made the compiler wait for
// them at its join, before the selection's first reads were issued.
__device__ __forceinline__ void load_q(const AttnArgs& a, int bt, int g, int lane, u32x4 (&qraw)[4]) {
  const int h = lane & 15, q4 = lane >> 4;
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(a.q + ((size_t)bt * a.Hq + (size_t)g * a.grp) * kHeadDim, (uint32_t)(a.grp * kHeadDim * 2));
  const uint32_t off = (uint32_t)(h * kHeadDim * 2 + 64 * q4);
#pragma unroll
  for (int s = 0; s < 4; s++) qraw[s] = buf_load16<0>(r, off + 16 * s, 0);
}

// Q^T operand in the matrix-core format and the score scale (log2 domain,
// >= 0) that the softmax applies to the raw dot products.
template <bool NVFP4>
__device__ __forceinline__ void convert_q(const AttnArgs& a, const u32x4 (&qraw)[4], typename MfmaT<NVFP4>::vec (&qb)[4],
                                          float& cscale) {
  typedef typename MfmaT<NVFP4>::vec vec;
  if constexpr (NVFP4) {
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; s++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const uint32_t w = qraw[s][e];
        amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w & 0xFFFFu)), fabsf(bf16_bits_to_f32(w >> 16))));
      }
    amax = fmaxf(amax, shfl_xor(amax, 16));
    amax = fmaxf(amax, shfl_xor(amax, 32));
    // power-of-two pre-scale keeping the row inside fp16's range
    int sh = 0;
    if (amax >= 32768.0f) sh = ((int)((__float_as_uint(amax) >> 23) & 255) - 127) - 14;
    // the sign of the score scale (a negative K tensor scale) moves into Q,
    // so that the softmax can take the max of the raw dot products
    const float sgn = a.score_scale < 0.0f ? -1.0f : 1.0f;
    const float down = sgn * __uint_as_float((uint32_t)(127 - sh) << 23);
    cscale = fabsf(a.score_scale) * __uint_as_float((uint32_t)(127 + sh) << 23);
#pragma unroll
    for (int s = 0; s < 4; s++) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const uint32_t w = qraw[s][e];
        v[e] = f32x2_to_f16x2(bf16_bits_to_f32(w & 0xFFFFu) * down, bf16_bits_to_f32(w >> 16) * down);
      }
      qb[s] = __builtin_bit_cast(vec, v);
    }
  } else {
    // bf16 Q is used as is; a negative score scale (negative K tensor scale)
    // flips Q's sign bits so that the softmax sees a scale >= 0
    const uint32_t flip = a.score_scale < 0.0f ? 0x80008000u : 0u;
    cscale = fabsf(a.score_scale);
#pragma unroll
    for (int s = 0; s < 4; s++) qb[s] = __builtin_bit_cast(vec, qraw[s] ^ flip);
  }
}

__device__ __forceinline__ void init_state(SoftmaxState& st) {
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int d = 0; d < 8; d++) st.o[d] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// This wave's online softmax and P.V over blocks wave, wave + W, ... < n of
// the lists blist (logical block) / plist (page) in LDS; at most MAXB blocks
// per wave. p: the query's last visible key. Ends with st.l summed over the
// four lanes of each head. lds: at least W * 4 KB (K- and V-scale stages).
template <bool NVFP4, int W, int MAXB>
__device__ __forceinline__ void stream_blocks(const AttnArgs& a, int g, int p, const int32_t* blist,
                                              const int32_t* plist, int n,
                                              const typename MfmaT<NVFP4>::vec (&qb)[4], float cscale,
                                              uint8_t* lds, int wave, int lane, SoftmaxState& st) {
  typedef MfmaT<NVFP4> MT;
  typedef typename MT::vec vec;
  const int q4 = lane >> 4;

  // raw scores of one block (S^T tiles) -> online softmax update and the P^T
  // operand. cscale >= 0, so the max of the scaled scores is cscale times the
  // max of the raw ones.
  auto softmax_update = [&](f32x4 (&sacc)[8], float rmax, bool masked, vec (&pb)[4]) {
    rmax = fmaxf(rmax, shfl_xor(rmax, 16));
    rmax = fmaxf(rmax, shfl_xor(rmax, 32));
    const float bmax = rmax == -INFINITY ? -INFINITY : rmax * cscale;
    const float mnew = fmaxf(st.m, bmax);
    float psum = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float x = sacc[2 * s + (e >> 2)][e & 3];
        float v = fast_exp2(fmaf(x, cscale, -mnew));
        if (masked) v = x == -INFINITY ? 0.0f : v;
        pv[e] = v;
      }
      u32x4 pk;
      pk.x = MT::pack(pv[0], pv[1]);
      pk.y = MT::pack(pv[2], pv[3]);
      pk.z = MT::pack(pv[4], pv[5]);
      pk.w = MT::pack(pv[6], pv[7]);
      pb[s] = __builtin_bit_cast(vec, pk);
      // the row sum takes the same rounded P that multiplies V
#pragma unroll
      for (int e = 0; e < 4; e++) psum = MT::sum2(pk[e], psum);
    }
    // rescale the running state only if some head's max grew
    if (__ballot(mnew != st.m) != 0) {
      const float alpha = lse_weight(st.m, mnew);
      st.l *= alpha;
#pragma unroll
      for (int d = 0; d < 8; d++) st.o[d] *= alpha;
    }
    st.l += psum;
    st.m = mnew;
  };
  // The block holding keys past p (the context's last block) takes the masked
  // path; the two paths are whole branches so that full blocks do not pay for
  // the mask.
  auto softmax_block = [&](f32x4 (&sacc)[8], int blk, bool partial, vec (&pb)[4]) {
    if (partial) {
      float rmax = -INFINITY;
#pragma unroll
      for (int tau = 0; tau < 8; tau++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const bool vis = blk * kBlock + kappa(tau, 4 * q4 + r) <= p;
          sacc[tau][r] = vis ? sacc[tau][r] : -INFINITY;
          rmax = fmaxf(rmax, sacc[tau][r]);
        }
      softmax_update(sacc, rmax, true, pb);
    } else {
      float rmax = -INFINITY;
#pragma unroll
      for (int tau = 0; tau < 8; tau++)
#pragma unroll
        for (int r = 0; r < 4; r++) rmax = fmaxf(rmax, sacc[tau][r]);
      softmax_update(sacc, rmax, false, pb);
    }
  };

  if constexpr (NVFP4) {
    // fp16 V scales of the current block: [8 groups][128 keys] per wave; fp16
    // K scales: [128 keys][8 groups] per wave
    f16* vs_stage = reinterpret_cast<f16*>(lds) + wave * 1024;
    f16* ks_stage = reinterpret_cast<f16*>(lds) + (W + wave) * 1024;
    const int rho = lane & 15;
    LaneOff off;
    off.k = (uint32_t)((32 * (rho >> 2) + (rho & 3)) * 64 + 16 * q4);
    off.ks = (uint32_t)(16 * lane);
    off.v = (uint32_t)(rho * 64 + 16 * q4);
    off.vs = (uint32_t)(16 * lane);
    KRegs K;
    VRegs V;
    {
      const bool none = wave >= n;
      const int pg = none ? 0 : __builtin_amdgcn_readfirstlane(plist[wave]);
      const KvRsrc r0 = nvfp4_rsrc(a, pg, g, none);
      load_k(r0, off, K);
      load_v(r0, off, V);
    }
    // Fully unrolled over the wave's at most MAXB blocks: straight-line code
    // keeps the compiler's load counters exact across blocks (a loop header
    // merges the first and later iterations' load orders and makes every
    // block wait for all outstanding loads). Iterations past the wave's last
    // block run on empty resources and skip the softmax and P.V.
#pragma unroll
    for (int it = 0; it < MAXB; it++) {
      const int i = wave + it * W;
      const bool valid = i < n;
      const int blk = valid ? __builtin_amdgcn_readfirstlane(blist[i]) : 0;
      const bool none = i + W >= n;
      const int pgn = none ? 0 : __builtin_amdgcn_readfirstlane(plist[i + W]);
      const KvRsrc rn = nvfp4_rsrc(a, pgn, g, none);

      // ---- K scales to fp16 in LDS (wave-private; the previous block's
      // reads of the stage are done: LDS operations of a wave stay in order)
      {
        u32x4* dst = reinterpret_cast<u32x4*>(ks_stage + 16 * lane);
        dst[0] = fp8x8_f16(K.ks.x, K.ks.y);
        dst[1] = fp8x8_f16(K.ks.z, K.ks.w);
        wave_lds_sync();
      }

      // ---- S^T = K Q^T, then the next block's K
      f32x4 sacc[8];
#pragma unroll
      for (int tau = 0; tau < 8; tau++) {
        // groups 2*q4, 2*q4+1 of key kappa(tau, rho)
        const uint32_t sc2 = *reinterpret_cast<const uint32_t*>(ks_stage + 8 * kappa(tau, rho) + 2 * q4);
        const uint32_t slo = bcast_lo16(sc2), shi = bcast_hi16(sc2);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; s++) {
          const u32x4 kv = nvfp4x8_f16(K.kd[tau][s], s < 2 ? slo : shi);
          acc = MT::mma(__builtin_bit_cast(vec, kv), qb[s], acc);
        }
        sacc[tau] = acc;
      }
      if (it + 1 < MAXB) load_k(rn, off, K);

      if (valid) {
        // ---- V scales to fp16 in LDS (wave-private)
        {
          const u32x4 lo = fp8x8_f16(V.vs.x, V.vs.y), hi = fp8x8_f16(V.vs.z, V.vs.w);
          u32x4* dst = reinterpret_cast<u32x4*>(vs_stage + 16 * lane);
          dst[0] = lo;
          dst[1] = hi;
          wave_lds_sync();
        }

        // ---- online softmax
        vec pb[4];
        softmax_block(sacc, blk, blk * kBlock + kBlock - 1 > p, pb);

        // ---- O^T += V^T P^T; the scales of dim tile dt+1 are read while
        // tile dt is decoded and multiplied
        u32x4 sc[4], scn[4];
#pragma unroll
        for (int s = 0; s < 4; s++) sc[s] = *reinterpret_cast<const u32x4*>(vs_stage + 32 * q4 + 8 * s);
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
          if (dt + 1 < 8) {
#pragma unroll
            for (int s = 0; s < 4; s++)
              scn[s] = *reinterpret_cast<const u32x4*>(vs_stage + (dt + 1) * 128 + 32 * q4 + 8 * s);
          }
#pragma unroll
          for (int s = 0; s < 4; s++) {
            const u32x4 vv = nvfp4x8_f16_each(V.vd[dt][s], sc[s]);
            st.o[dt] = MT::mma(__builtin_bit_cast(vec, vv), pb[s], st.o[dt]);
          }
#pragma unroll
          for (int s = 0; s < 4; s++) sc[s] = scn[s];
        }
        wave_lds_sync();  // the stage is overwritten by the next block
      }
      if (it + 1 < MAXB) load_v(rn, off, V);
    }
  } else {
    for (int i = wave; i < n; i += W) {
      const int blk = __builtin_amdgcn_readfirstlane(blist[i]);
      const size_t pg = (size_t)__builtin_amdgcn_readfirstlane(plist[i]) * a.Hkv + g;
      const int rho = lane & 15;
      const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k_data) + pg * (kBlock * kHeadDim);
      f32x4 sacc[8];
#pragma unroll
      for (int tau = 0; tau < 8; tau++) {
        const u32x4* kr = reinterpret_cast<const u32x4*>(kb + kappa(tau, rho) * kHeadDim + 32 * q4);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; s++) acc = MT::mma(__builtin_bit_cast(vec, kr[s]), qb[s], acc);
        sacc[tau] = acc;
      }
      vec pb[4];
      softmax_block(sacc, blk, blk * kBlock + kBlock - 1 > p, pb);
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
}

// acc := log-sum-exp merge of acc and the state (m2, l2, o2), in that order.
// merge_state on ND of the 8 dim tiles (the max and sum as for all of them)
template <int ND>
__device__ __forceinline__ void merge_tiles(float& m, float& l, f32x4 (&o)[ND], float m2, float l2,
                                            const f32x4 (&o2)[ND]) {
  const float M = fmaxf(m, m2);
  const float a1 = lse_weight(m, M), a2 = lse_weight(m2, M);
#pragma unroll
  for (int d = 0; d < ND; d++) o[d] = o[d] * a1 + o2[d] * a2;
  l = l * a1 + l2 * a2;
  m = M;
}
__device__ __forceinline__ void merge_state(SoftmaxState& acc, float m2, float l2, const f32x4 (&o2)[8]) {
  merge_tiles<8>(acc.m, acc.l, acc.o, m2, l2, o2);
}

// Fixed-order tree merge of the W wave states through LDS slots (at least
// W/2 * kSlotFloats floats at lds); wave 0 ends with the workgroup's state.
// Every thread of the workgroup calls it.
template <int W>
__device__ __forceinline__ void merge_waves(SoftmaxState& st, uint8_t* lds, int wave, int lane) {
  const int h = lane & 15, q4 = lane >> 4;
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
      f32x4 o2[8];
#pragma unroll
      for (int d = 0; d < 8; d++) o2[d] = *reinterpret_cast<const f32x4*>(sl + h * kHeadDim + 16 * d + 4 * q4);
      merge_state(st, sl[16 * kHeadDim + h], sl[16 * kHeadDim + 16 + h], o2);
    }
  }
}

// bf16 output rows (and lse) of KV head g of row bt from wave 0's state
// (called by wave 0 only).
// write_out of dim tiles d0 .. d0 + ND - 1 (held in o[0 .. ND)) of a state
// with max m and sum l; the lse too when with_lse
template <int ND>
__device__ __forceinline__ void write_tiles(const AttnArgs& a, int bt, int g, float m, float l,
                                            const f32x4 (&o)[ND], int d0, bool with_lse, int lane) {
  const int h = lane & 15, q4 = lane >> 4;
  if (h >= a.grp) return;
  const size_t row = (size_t)bt * a.Hq + g * a.grp + h;
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : a.v_scale_mul / l;
  uint16_t* orow = a.out + row * kHeadDim;
#pragma unroll
  for (int d = 0; d < ND; d++) {
    uint2 pk;
    pk.x = f32x2_to_bf16x2(o[d][0] * inv, o[d][1] * inv);
    pk.y = f32x2_to_bf16x2(o[d][2] * inv, o[d][3] * inv);
    *reinterpret_cast<uint2*>(orow + 16 * (d0 + d) + 4 * q4) = pk;
  }
  if (with_lse && a.lse && q4 == 0) a.lse[row] = empty ? -INFINITY : (m + __log2f(l)) * 0.69314718055994530942f;
}
__device__ __forceinline__ void write_out(const AttnArgs& a, int bt, int g, const SoftmaxState& st, int lane) {
  write_tiles<8>(a, bt, g, st.m, st.l, st.o, 0, true, lane);
}

// NaN output rows and lse of KV head g of row bt: the item's inputs never
// arrived (a bounded wait gave up). Threads tid < NT share the writes.
__device__ __forceinline__ void write_invalid(const AttnArgs& a, int bt, int g, int tid, int NT) {
  uint16_t* orow = a.out + ((size_t)bt * a.Hq + (size_t)g * a.grp) * kHeadDim;
  for (int i = tid; i < a.grp * kHeadDim; i += NT) orow[i] = 0x7FC0;
  if (a.lse && tid < a.grp) a.lse[(size_t)bt * a.Hq + g * a.grp + tid] = __builtin_nanf("");
}

// ---------------------------------------------------------------- kernel

// The attention of workgroup wg (item wg / splits, share wg % splits) with
// W waves; lds: the dynamic LDS region (attn_lds_bytes); tid: threadIdx.x.
// With a.pooled the workgroup first selects its query token's blocks from
// the pooled scores; otherwise it reads them from a.sel. Every thread of the
// workgroup calls it.
template <bool NVFP4, int W>
__device__ __forceinline__ void attn_body(const AttnArgs& a, int wg, uint8_t* lds, int tid) {
  typedef MfmaT<NVFP4> MT;
  typedef typename MT::vec vec;
  constexpr int NT = 64 * W;
  __shared__ TopkLds tk;
  __shared__ int32_t sel_lds[kTopkMax], blist[kTopkMax], plist[kTopkMax];
  __shared__ int32_t nlist, last_lds;

  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps block loops scalar
  const int item = wg / a.splits;   // (sequence, token, KV head)
  const int split = wg % a.splits;  // this workgroup's share of the item's blocks
  const int g = item % a.Hkv;
  const int bt = item / a.Hkv;
  const int b = bt / a.Tq;
  const int Lc = clamp_ctx(a.ctx_lens[b], a.maxb);
  const int p = Lc - a.Tq + bt % a.Tq;  // last visible key
  const int h = lane & 15;      // head within the group (MFMA column)
  const int q4 = lane >> 4;     // lane group 0..3

  // ---- Q^T operand (issued before the selection; it does not depend on it)
  u32x4 qraw[4];
  load_q(a, bt, g, lane, qraw);

  // ---- selected blocks (fused: from the pooled scores; the block-table
  // entries of all visible blocks are fetched in the same pass into an LDS
  // page table, so the winners' pages need no second dependent load)
  int nsel;
  int32_t* pages = reinterpret_cast<int32_t*>(lds);  // [nvis], fused path only
  const int32_t* bt_row = a.block_table + (size_t)b * a.maxb;
  if (a.pooled) {
    const int nvis = p < 0 ? 0 : p / kBlock + 1;
    const float* src = a.pooled + (size_t)bt * a.maxb;
    nsel = block_topk<NT>([&](int i) { return src[i]; }, [&](int i) { return bt_row[i]; }, pages, nvis,
                          a.top_k, a.keep_last != 0, sel_lds, tk);
    if (g == 0 && a.sel)
      for (int k = tid; k < a.top_k; k += NT) a.sel[(size_t)bt * a.top_k + k] = k < nsel ? sel_lds[k] : -1;
  } else {
    if (tid < a.top_k) sel_lds[tid] = a.sel[(size_t)bt * a.top_k + tid];
    nsel = a.top_k;
    __syncthreads();
  }
  // blocks that exist, compacted, order kept; a split item keeps its share
  // (split s of S: positions [s*per, (s+1)*per), per = ceil(count / S))
  if (wave == 0) {
    bool ok = false;
    int blk = -1, page = -1;
    if (lane < nsel && p >= 0) {
      blk = sel_lds[lane];
      if (blk >= 0 && blk < a.maxb && blk * kBlock <= p) {
        page = a.pooled ? pages[blk] : bt_row[blk];
        ok = page >= 0 && page < a.num_pages;
      }
    }
    const uint64_t bal = __ballot(ok);
    const int cnt = __popcll(bal);
    const int per = (cnt + a.splits - 1) / a.splits, first = split * per;
    const int pos = __popcll(bal & ((1ull << lane) - 1ull)) - first;
    if (ok && pos >= 0 && pos < per) {
      blist[pos] = blk;
      plist[pos] = page;
    }
    if (lane == 0) nlist = max(0, min(per, cnt - first));
  }

  vec qb[4];
  float cscale;
  convert_q<NVFP4>(a, qraw, qb, cscale);
  __syncthreads();
  const int n = __builtin_amdgcn_readfirstlane(nlist);

  SoftmaxState st;
  init_state(st);
  stream_blocks<NVFP4, W, kTopkMax / W>(a, g, p, blist, plist, n, qb, cscale, lds, wave, lane, st);
  merge_waves<W>(st, lds, wave, lane);

  if (a.splits > 1) {
    // ---- split item: publish this workgroup's state; the last of the
    // item's workgroups to arrive combines all of them in split order. The
    // arrival word holds (epoch << 32) | count; a word from an older launch
    // (another epoch) counts as zero, so the workspace needs no clearing.
    float* mine = a.partials + ((size_t)item * a.splits + split) * (16 * kPartRow);
    if (wave == 0) {
#pragma unroll
      for (int d = 0; d < 8; d++) *reinterpret_cast<f32x4*>(mine + h * kPartRow + 16 * d + 4 * q4) = st.o[d];
      if (q4 == 0) {
        mine[h * kPartRow + 128] = st.m;
        mine[h * kPartRow + 129] = st.l;
      }
    }
    __threadfence();  // release: the state is visible device-wide before the arrival
    __syncthreads();
    if (tid == 0) {
      unsigned long long* word = a.arrivals + item;
      const unsigned long long fresh = (unsigned long long)a.epoch << 32;
      unsigned long long seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), mine_cnt;
      for (;;) {  // ends within `splits` rounds: every failure is another workgroup's success
        const unsigned long long want = ((seen >> 32) == a.epoch ? seen : fresh) + 1ull;
        const unsigned long long prev = atomicCAS(word, seen, want);
        if (prev == seen) {
          mine_cnt = want & 0xFFFFFFFFull;
          break;
        }
        seen = prev;
      }
      last_lds = (int)mine_cnt == a.splits;
    }
    __syncthreads();
    if (!last_lds) return;
    __threadfence();  // acquire: the other workgroups' states
    if (wave == 0) {
      const float* all = a.partials + (size_t)item * a.splits * (16 * kPartRow);
      float M = -INFINITY;
      for (int sp = 0; sp < a.splits; sp++) M = fmaxf(M, all[sp * (16 * kPartRow) + h * kPartRow + 128]);
      float l = 0.0f;
      f32x4 o[8];
#pragma unroll
      for (int d = 0; d < 8; d++) o[d] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int sp = 0; sp < a.splits; sp++) {
        const float* row = all + sp * (16 * kPartRow) + h * kPartRow;
        const float w = lse_weight(row[128], M);
        l += w * row[129];
#pragma unroll
        for (int d = 0; d < 8; d++) o[d] += w * *reinterpret_cast<const f32x4*>(row + 16 * d + 4 * q4);
      }
      st.m = M;
      st.l = l;
#pragma unroll
      for (int d = 0; d < 8; d++) st.o[d] = o[d];
    }
  }

  // ---- write bf16 output (and lse) for the real heads
  if (wave == 0) write_out(a, bt, g, st, lane);
}

// Dynamic LDS: the pooled scores of one token (fused selection), the
// per-wave K- and V-scale stages, and the merge slots reuse one region.
inline size_t attn_lds_bytes(const AttnArgs& a, int W) {
  size_t sel = a.pooled ? (size_t)a.maxb * sizeof(int32_t) : 0;  // page table
  size_t stage = (size_t)W * 1024 * 4;
  size_t merge = (size_t)(W / 2) * kSlotFloats * 4;
  size_t m = sel > stage ? sel : stage;
  return m > merge ? m : merge;
}

}  // namespace

}  // namespace msa
