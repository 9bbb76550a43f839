// indexer.hip -- MSA indexer scan + per-block max pool (gfx950).
//
// [ainewsbites page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on NVIDIA
// and AMD GPUs", section "A model built for efficient inference": a
// lightweight indexer scores every key of the context and the scores are
// pooled into one score per 128-token block.] The score of key j for query
// token t of sequence b is
//     s = sum_h w[t,h] * max(0, <qi[t,h,:], k_j>),   k_j = e4m3(code) * s_tok
// and the pooled block score is the max over the block's keys j <= p_t.
//
// Design. The scan reads every indexer key once, so it is HBM bound (68 bytes
// per token for FP8 keys). One wavefront owns `ppw` consecutive blocks of one
// sequence and streams them through the block table, prefetching the next
// block while it computes the current one. The dot products of all T_q*H_i
// query rows with 32 keys at a time are one 32x32x16 bf16 MFMA chain
// (v_mfma_f32_32x32x16_bf16, 4 steps over the 64 dims): rows are query
// vectors (t*HP + h, padded to 32), columns are keys, so every lane ends up
// holding one key's dots for 16 query rows and the head sum, ReLU and weight
// happen in registers. FP8 codes are widened to bf16 exactly by the hardware
// converter; the per-token scale multiplies the dot before the ReLU.
//
// Operand layout of v_mfma_f32_32x32x16_bf16 (checked on gfx950): lane l
// supplies A[row l%32][k = 8*(l/32) + e] and B[k = 8*(l/32) + e][col l%32],
// e = 0..7, and receives D[row 8*(r/4) + 4*(l/32) + r%4][col l%32] in
// register r = 0..15. The k order inside a step is free as long as A and B
// agree: lane half c = l/32 takes the contiguous dims 32c..32c+31 of its key
// and uses dims 32c + 8s + e in step s.
#include "fmt.hpp"
#include "msa_internal.hpp"

namespace msa {

namespace {

template <bool FP8>
struct KeyTile;

template <>
struct KeyTile<true> {  // 32 FP8 codes + the key's fp32 scale, per tile
  u32x4 v[4][2];
  float s[4];
};
template <>
struct KeyTile<false> {  // 32 bf16 values per tile
  u32x4 v[4][4];
};

template <bool FP8>
__device__ __forceinline__ void load_block(const IndexerArgs& a, int page, int lane, KeyTile<FP8>& kt) {
  const int j = lane & 31, c = lane >> 5;
  if constexpr (FP8) {
    const uint8_t* base = a.idx_k + (size_t)page * (kBlock * kIdxDim);
#pragma unroll
    for (int tile = 0; tile < 4; tile++) {
      const u32x4* p = reinterpret_cast<const u32x4*>(base + (tile * 32 + j) * kIdxDim + 32 * c);
      kt.v[tile][0] = p[0];
      kt.v[tile][1] = p[1];
      kt.s[tile] = a.idx_k_scale[(size_t)page * kBlock + tile * 32 + j];
    }
  } else {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(a.idx_k) + (size_t)page * (kBlock * kIdxDim);
#pragma unroll
    for (int tile = 0; tile < 4; tile++) {
      const u32x4* p = reinterpret_cast<const u32x4*>(base + (tile * 32 + j) * kIdxDim + 32 * c);
#pragma unroll
      for (int s = 0; s < 4; s++) kt.v[tile][s] = p[s];
    }
  }
}

// HP: padded heads per query token in the row layout (row = t*HP + h);
// TQ: query tokens (compile-time) -- TQ*HP <= 32.
template <bool FP8, int HP, int TQ>
__global__ __launch_bounds__(256) void indexer_pool_kernel(IndexerArgs a) {
  static_assert(TQ * HP <= 32, "query rows exceed one 32-row MFMA tile");
  // register groups r/4 that can hold a real token
  constexpr int NG = (HP == 8) ? TQ : (TQ + 1) / 2;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int c = lane >> 5;
  const int j = lane & 31;
  const int Lc = clamp_ctx(a.ctx_lens[b], a.maxb);
  const int nblk = (Lc + kBlock - 1) / kBlock;
  const int cover = a.scores ? a.maxb : nblk;  // scores are written for every block
  const int blk0 = (blockIdx.x * 4 + wave) * a.ppw;
  if (blk0 >= cover) return;
  const int blk1 = min(blk0 + a.ppw, cover);

  // A operand: query row i = j (t = i / HP, h = i % HP), dims 32c + 8s + e.
  bf16x8 qa[4];
  {
    const int t = j / HP, h = j % HP;
    const bool ok = (t < a.Tq) && (h < a.Hi);
    const uint16_t* qrow = a.idx_q + ((size_t)(b * a.Tq + t) * a.Hi + h) * kIdxDim + 32 * c;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      u32x4 v = ok ? reinterpret_cast<const u32x4*>(qrow)[s] : u32x4{0, 0, 0, 0};
      qa[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // head weight of output register r: row 8*(r/4) + 4c + r%4
  float wr[4 * NG];
  int tg[NG];
#pragma unroll
  for (int g = 0; g < NG; g++) {
    tg[g] = (HP == 8) ? g : 2 * g + c;
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      const int row = 8 * g + 4 * c + rr;
      const int t = row / HP, h = row % HP;
      wr[4 * g + rr] = (t < a.Tq && h < a.Hi) ? a.idx_w[(size_t)(b * a.Tq + t) * a.Hi + h] : 0.0f;
    }
  }
  int pt[NG];
#pragma unroll
  for (int g = 0; g < NG; g++) pt[g] = Lc - a.Tq + tg[g];
  // lanes that write token tg[g]: with HP == 8 the two halves hold the same total
  const bool writer = (HP == 8) ? (c == 0) : true;

  auto page_of = [&](int blk) -> int {
    if (blk >= nblk) return -1;
    int pg = a.block_table[(size_t)b * a.maxb + blk];
    return (pg >= 0 && pg < a.num_pages) ? pg : -1;
  };

  KeyTile<FP8> cur, nxt;
  int page_cur = page_of(blk0);
  if (page_cur >= 0) load_block<FP8>(a, page_cur, lane, cur);

  for (int blk = blk0; blk < blk1; blk++) {
    const int page_nxt = (blk + 1 < blk1) ? page_of(blk + 1) : -1;
    if (page_nxt >= 0) load_block<FP8>(a, page_nxt, lane, nxt);

    float mx[NG];
#pragma unroll
    for (int g = 0; g < NG; g++) mx[g] = -INFINITY;

#pragma unroll
    for (int tile = 0; tile < 4; tile++) {
      const int pos = blk * kBlock + tile * 32 + j;
      float tot[NG];
      if (page_cur >= 0) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < 4; s++) {
          bf16x8 kb;
          if constexpr (FP8) {
            const u32x4 h = cur.v[tile][s >> 1];
            kb = __builtin_bit_cast(bf16x8, (s & 1) ? fp8x8_bf16(h.z, h.w) : fp8x8_bf16(h.x, h.y));
          } else {
            kb = __builtin_bit_cast(bf16x8, cur.v[tile][s]);
          }
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kb, acc, 0, 0, 0);
        }
        float ks = 1.0f;
        if constexpr (FP8) ks = cur.s[tile];
#pragma unroll
        for (int g = 0; g < NG; g++) {
          float part = 0.0f;
#pragma unroll
          for (int rr = 0; rr < 4; rr++) part = fmaf(wr[4 * g + rr], fmaxf(acc[4 * g + rr] * ks, 0.0f), part);
          if constexpr (HP == 8) part += shfl_xor(part, 32);
          tot[g] = part;
        }
      } else {
#pragma unroll
        for (int g = 0; g < NG; g++) tot[g] = -INFINITY;
      }
#pragma unroll
      for (int g = 0; g < NG; g++) {
        const float sc = (pos <= pt[g]) ? tot[g] : -INFINITY;
        if (a.scores && writer && tg[g] < a.Tq)
          a.scores[((size_t)(b * a.Tq + tg[g])) * a.maxb * kBlock + pos] = sc;
        mx[g] = fmaxf(mx[g], sc);
      }
    }
    if (a.pooled) {
#pragma unroll
      for (int g = 0; g < NG; g++) {
        float m = mx[g];
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) m = fmaxf(m, shfl_xor(m, off));
        if (j == 0 && writer && tg[g] < a.Tq) a.pooled[((size_t)(b * a.Tq + tg[g])) * a.maxb + blk] = m;
      }
    }
    cur = nxt;
    page_cur = page_nxt;
  }
}

template <bool FP8, int HP>
hipError_t launch_hp(const IndexerArgs& a, dim3 grid, hipStream_t s) {
  switch (a.Tq) {
#define MSA_TQ_CASE(T)                                                       \
  case T:                                                                    \
    if constexpr (T * HP <= 32) {                                            \
      indexer_pool_kernel<FP8, HP, T><<<grid, 256, 0, s>>>(a);               \
      return hipGetLastError();                                              \
    }                                                                        \
    break;
    MSA_TQ_CASE(1)
    MSA_TQ_CASE(2)
    MSA_TQ_CASE(3)
    MSA_TQ_CASE(4)
    MSA_TQ_CASE(5)
    MSA_TQ_CASE(6)
    MSA_TQ_CASE(7)
    MSA_TQ_CASE(8)
#undef MSA_TQ_CASE
    default:
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, bool fp8, int hp, hipStream_t s) {
  const int waves_per_seq = (a.maxb + a.ppw - 1) / a.ppw;
  dim3 grid((waves_per_seq + 3) / 4, a.B);
  if (fp8) return hp == 8 ? launch_hp<true, 8>(a, grid, s) : launch_hp<true, 4>(a, grid, s);
  return hp == 8 ? launch_hp<false, 8>(a, grid, s) : launch_hp<false, 4>(a, grid, s);
}

}  // namespace msa
