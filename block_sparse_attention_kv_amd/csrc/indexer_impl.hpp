// indexer_impl.hpp -- device code of the MSA indexer scan + per-block max
// pool (gfx950); the design is described at the top of indexer.hip. Used by
// the indexer kernel and by the single-launch decode layer.
#pragma once
#include "fmt.hpp"
#include "indexer_args.hpp"

namespace msa {

namespace {


// Key loads stream through the caches once: nontemporal unless built with
// MSA_IDX_NT=0.
#ifndef MSA_IDX_NT
#define MSA_IDX_NT 1
#endif
constexpr int kIdxAux = MSA_IDX_NT ? kAuxNT : 0;

// Key formats (the template parameter KF of the kernel).
constexpr int kKfBf16 = 0, kKfFp8 = 1, kKfNvfp4 = 2;

// Bytes per token of the key codes.
constexpr uint32_t key_row_bytes(int kf) { return kf == kKfBf16 ? 128u : kf == kKfFp8 ? 64u : 32u; }

// This lane's share of one tile (16 keys x 64 dims): key 16k + l%16,
// dims 16*(l/16) .. 16*(l/16) + 15. NVFP4 keys' scales come per block
// (load_kscales).
template <int KF>
struct KTile;
template <>
struct KTile<kKfFp8> {
  u32x4 v;   // 16 E4M3 codes
  float s;   // the key's fp32 scale
};
template <>
struct KTile<kKfBf16> {
  u32x4 v[2];  // 16 bf16 values
};
template <>
struct KTile<kKfNvfp4> {
  u32x2 c;     // 16 E2M1 codes
};

// Lane offset (bytes) of this lane's share of tile 0 inside a page; tile k
// adds 16*k keys.
template <int KF>
__device__ __forceinline__ uint32_t ktile_lane_off(int lane) {
  return (uint32_t)(lane & 15) * key_row_bytes(KF) + (key_row_bytes(KF) / 4) * (uint32_t)(lane >> 4);
}

// Buffer resources of one page's keys and scales (uniform). An absent page
// gets an empty range, so its loads return zeros without a memory access.
template <int KF>
struct PageRsrc {
  __amdgpu_buffer_rsrc_t keys, scales;
};
template <int KF>
__device__ __forceinline__ PageRsrc<KF> page_rsrc(const IndexerArgs& a, int page, bool absent) {
  constexpr uint32_t kPageBytes = kBlock * key_row_bytes(KF);
  constexpr uint32_t kScaleBytes = kBlock * 4u;  // fp32 per token, or 4 E4M3 per token
  const int pg = absent ? 0 : page;
  PageRsrc<KF> r;
  r.keys = make_rsrc(a.idx_k + (size_t)pg * kPageBytes, absent ? 0u : kPageBytes);
  if constexpr (KF != kKfBf16)
    r.scales = make_rsrc(static_cast<const uint8_t*>(a.idx_k_scale) + (size_t)pg * kScaleBytes,
                         absent ? 0u : kScaleBytes);
  return r;
}

template <int KF>
__device__ __forceinline__ void load_ktile(const PageRsrc<KF>& r, int k, int lane, uint32_t loff, KTile<KF>& t) {
  constexpr uint32_t kTileBytes = 16 * key_row_bytes(KF);
  // the tile offset goes to the scalar offset: one offset register per lane
  const uint32_t soff = kTileBytes * k, voff = loff;
  if constexpr (KF == kKfFp8) {
    t.v = buf_load16<kIdxAux>(r.keys, voff, soff);
    t.s = buf_load4f<kIdxAux>(r.scales, (uint32_t)(4 * (lane & 15)), (uint32_t)(64 * k));
  } else if constexpr (KF == kKfNvfp4) {
    t.c = buf_load8<kIdxAux>(r.keys, voff, soff);
  } else {
    t.v[0] = buf_load16<kIdxAux>(r.keys, voff, soff);
    t.v[1] = buf_load16<kIdxAux>(r.keys, voff + 16, soff);
  }
}

// NVFP4 keys: the four E4M3 group scales of every key of a block (512
// bytes); lane l holds keys 2l and 2l+1. A lane uses one scale byte of a
// different key in every tile, so the wave loads the block's scales with one
// instruction and exchanges them through LDS (score_block): eight 1-byte
// loads per block cost more vector memory issue than the exchange (128K with
// NVFP4 keys: 61.8-62.0 against 62.2-62.9 us). FP8 keys keep one 4-byte
// load per tile, which ran faster than the exchange (128K: 72.1-72.5 against
// 73.2-73.4 us).
template <int KF>
__device__ __forceinline__ u32x2 load_kscales(const PageRsrc<KF>& r, int lane) {
  if constexpr (KF != kKfNvfp4) return u32x2{0u, 0u};
  else return buf_load8<kIdxAux>(r.scales, (uint32_t)(8 * lane), 0u);
}
constexpr uint32_t kScaleStageBytes = kBlock * 4;  // per wave

// Dynamic LDS of the scan: the prefix sums (B + 1 ints), then four waves'
// scale stages.
__host__ __device__ constexpr size_t indexer_stage_offset(int B) { return (((size_t)B + 1) * 4 + 15) & ~(size_t)15; }
__host__ __device__ constexpr size_t indexer_lds_bytes(int B) { return indexer_stage_offset(B) + 4 * kScaleStageBytes; }

// DPP lane moves (gfx9 encodings): quad_perm and row_ror.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}

// Max over each 16-lane row; every lane of the row receives it.
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x124>(v));   // row_ror:4
  v = fmaxf(v, dpp_f<0x128>(v));   // row_ror:8
  return v;
}

// Compile-time shape: HP heads per token (4 or 8), TQ query tokens.
template <int HP, int TQ>
struct Shape {
  static constexpr int HQ = HP / 4;               // row tiles per token tile
  static constexpr int NTT = (TQ + 3) / 4;        // token tiles
  static constexpr int RT = HQ * NTT;             // row tiles
};

// MFMA operand type of the key format: fp16 for NVFP4 keys, else bf16.
template <int KF>
struct KeyVec {
  typedef bf16x8 type;
};
template <>
struct KeyVec<kKfNvfp4> {
  typedef f16x8 type;
};

// Per-sequence state of a wave: A operands, weights, positions.
template <int KF, int HP, int TQ>
struct SeqState {
  typedef Shape<HP, TQ> S;
  typename KeyVec<KF>::type qa[S::RT][2];
  float wr[S::NTT][HP];   // weight of (token 4*tau + g, head h)
  int pt[S::NTT];         // position of token 4*tau + g
  float kq;               // factor undoing the fp16 pre-scale of the queries (NVFP4 keys)
};

template <int KF, int HP, int TQ>
__device__ __forceinline__ void load_seq(const IndexerArgs& a, int b, int Lc, int lane, SeqState<KF, HP, TQ>& st) {
  typedef Shape<HP, TQ> S;
  const int g = lane >> 4, rr = lane & 15;
  u32x4 raw[S::RT][2];
#pragma unroll
  for (int rho = 0; rho < S::RT; rho++) {
    const int t = 4 * (rho / S::HQ) + (rr >> 2), h = 4 * (rho % S::HQ) + (rr & 3);
    const bool ok = (t < a.Tq) && (h < a.Hi);
    // step s uses dims 16g + 8s + e for every key format
    const u32x4* q = reinterpret_cast<const u32x4*>(a.idx_q + ((size_t)(b * a.Tq + t) * a.Hi + h) * kIdxDim + 16 * g);
#pragma unroll
    for (int s = 0; s < 2; s++) raw[rho][s] = ok ? q[s] : u32x4{0, 0, 0, 0};
  }
  st.kq = 1.0f;
  if constexpr (KF == kKfNvfp4) {
    // one power of two for the sequence's queries: the largest magnitude
    // lands in [2^14, 2^15), far inside fp16's range
    float amax = 0.0f;
#pragma unroll
    for (int rho = 0; rho < S::RT; rho++)
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint32_t w = raw[rho][s][e];
          amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w & 0xFFFFu)), fabsf(bf16_bits_to_f32(w >> 16))));
        }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, shfl_xor(amax, m));
    // (clamped so that both factors stay normal floats)
    const int ex = amax > 0.0f ? min(112, max(-112, (int)((__float_as_uint(amax) >> 23) & 255) - 127 - 14)) : 0;
    const float down = __uint_as_float((uint32_t)(127 - ex) << 23);
    st.kq = __uint_as_float((uint32_t)(127 + ex) << 23);
#pragma unroll
    for (int rho = 0; rho < S::RT; rho++)
#pragma unroll
      for (int s = 0; s < 2; s++) {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint32_t w = raw[rho][s][e];
          v[e] = f32x2_to_f16x2(bf16_bits_to_f32(w & 0xFFFFu) * down, bf16_bits_to_f32(w >> 16) * down);
        }
        st.qa[rho][s] = __builtin_bit_cast(f16x8, v);
      }
  } else {
#pragma unroll
    for (int rho = 0; rho < S::RT; rho++)
#pragma unroll
      for (int s = 0; s < 2; s++) st.qa[rho][s] = __builtin_bit_cast(bf16x8, raw[rho][s]);
  }
#pragma unroll
  for (int tau = 0; tau < S::NTT; tau++) {
    const int t = 4 * tau + g;
#pragma unroll
    for (int h = 0; h < HP; h++)
      st.wr[tau][h] = (t < a.Tq && h < a.Hi) ? a.idx_w[(size_t)(b * a.Tq + t) * a.Hi + h] : 0.0f;
    st.pt[tau] = Lc - a.Tq + t;
  }
}

// Scores of one block held in the ring T (8 tiles of 16 keys) and, for NVFP4
// keys, its scales ks_blk; refills both with the next block when PREFETCH.
// stage: this wave's kScaleStageBytes of LDS. mx[tau]: this lane's max over its keys for
// token 4*tau + g.
template <int KF, int HP, int TQ, bool PREFETCH, bool SCORES>
__device__ __forceinline__ void score_block(const IndexerArgs& a, KTile<KF> (&T)[8], u32x2& ks_blk, uint8_t* stage,
                                            const SeqState<KF, HP, TQ>& st, int b, int lane, uint32_t loff, int blk,
                                            bool absent, const PageRsrc<KF>& rn, float (&mx)[Shape<HP, TQ>::NTT]) {
  typedef Shape<HP, TQ> S;
  const int g = lane >> 4;
#pragma unroll
  for (int tau = 0; tau < S::NTT; tau++) mx[tau] = -INFINITY;
  // NVFP4: the block's scales to LDS (the previous block's reads of the
  // stage are done: LDS operations of a wave stay in order), then the next
  // block's
  if constexpr (KF == kKfNvfp4) {
    *reinterpret_cast<u32x2*>(stage + 8 * lane) = ks_blk;
    wave_lds_sync();
    if constexpr (PREFETCH) ks_blk = load_kscales<KF>(rn, lane);
  }
#pragma unroll
  for (int k = 0; k < 8; k++) {
    typedef typename KeyVec<KF>::type vec;
    vec kb[2];
    float ks = 1.0f;
    if constexpr (KF == kKfFp8) {
      kb[0] = __builtin_bit_cast(vec, fp8x8_bf16(T[k].v.x, T[k].v.y));
      kb[1] = __builtin_bit_cast(vec, fp8x8_bf16(T[k].v.z, T[k].v.w));
      ks = T[k].s;
    } else if constexpr (KF == kKfNvfp4) {
      const uint32_t sraw = stage[4 * (16 * k + (lane & 15)) + g];  // the group's E4M3 scale
      const uint32_t s2 = bcast_lo16(fp8x2_f16x2<false>(sraw));
      kb[0] = __builtin_bit_cast(vec, nvfp4x8_f16(T[k].c.x, s2));
      kb[1] = __builtin_bit_cast(vec, nvfp4x8_f16(T[k].c.y, s2));
      ks = a.idx_ts * st.kq;
    } else {
      kb[0] = __builtin_bit_cast(vec, T[k].v[0]);
      kb[1] = __builtin_bit_cast(vec, T[k].v[1]);
    }
    if constexpr (PREFETCH) load_ktile<KF>(rn, k, lane, loff, T[k]);
    f32x4 acc[S::RT];
#pragma unroll
    for (int rho = 0; rho < S::RT; rho++) {
      if constexpr (KF == kKfNvfp4) {
        acc[rho] = __builtin_amdgcn_mfma_f32_16x16x32_f16(st.qa[rho][0], kb[0], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        acc[rho] = __builtin_amdgcn_mfma_f32_16x16x32_f16(st.qa[rho][1], kb[1], acc[rho], 0, 0, 0);
      } else {
        acc[rho] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.qa[rho][0], kb[0], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        acc[rho] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.qa[rho][1], kb[1], acc[rho], 0, 0, 0);
      }
    }
    const float bound = ks >= 0.0f ? INFINITY : -INFINITY;
    const int pos = blk * kBlock + 16 * k + (lane & 15);
#pragma unroll
    for (int tau = 0; tau < S::NTT; tau++) {
      float part = 0.0f;
#pragma unroll
      for (int h = 0; h < HP; h++)
        part = fmaf(st.wr[tau][h], __builtin_amdgcn_fmed3f(acc[tau * S::HQ + h / 4][h % 4], 0.0f, bound), part);
      const float sc = (!absent && pos <= st.pt[tau]) ? part * ks : -INFINITY;
      if constexpr (SCORES) {
        const int t = 4 * tau + g;
        if (t < a.Tq) a.scores[((size_t)(b * a.Tq + t)) * a.maxb * kBlock + pos] = sc;
      }
      mx[tau] = fmaxf(mx[tau], sc);
    }
    // keep the tiles in order: one tile's temporaries live at a time
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Work blocks of sequence b: every block up to the context's last one, or
// every column of the block table when all scores are written.
template <bool SCORES>
__device__ __forceinline__ int work_blocks(const IndexerArgs& a, int b) {
  if constexpr (SCORES) return a.maxb;
  const int Lc = clamp_ctx(a.ctx_lens[b], a.maxb);
  return (Lc + kBlock - 1) / kBlock;
}

// Waves per SIMD each instantiation is compiled for (its register budget:
// 4 -> 128 VGPRs, 3 -> 168, 2 -> 256). bf16 keys need twice the ring.
constexpr int indexer_occupancy(int kf, int hp, int tq) {
  return kf == kKfBf16 ? 2 : (hp == 4 && tq > 4) ? 3 : 4;
}

// The indexer scan of workgroup wg of nwg (persistent: every workgroup of the
// grid calls it once). SCORES: write every key's score instead of the pooled
// block maxima. NRING tile rings per wave (blocks in flight); prefix: the
// dynamic LDS, indexer_lds_bytes(B) bytes. Wave w of the workgroup scans the global work blocks
// [W * total / (4 nwg), (W + 1) * total / (4 nwg)), W = 4 wg + w, where the
// work blocks of the batch are numbered sequence after sequence.
// COHERENT: for readers in the same grid, every pooled score is stored as
// one 64-bit word (tag << 32) | (fp32 bits) in a.pooled viewed as uint64
// [B][Tq][maxb], with a device-scope relaxed atomic store (written through
// to the device's coherence point); a reader that finds the call's tag in a
// word holds that call's score.
template <int KF, int HP, int TQ, bool SCORES, int NRING, bool COHERENT = false>
__device__ __forceinline__ void indexer_body(const IndexerArgs& a, int32_t* prefix, int wg, int nwg,
                                             uint32_t tag = 0) {
  typedef Shape<HP, TQ> S;
  static_assert(S::RT <= 2, "at most 32 query rows");
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps loop control scalar
  const uint32_t loff = ktile_lane_off<KF>(lane);
  // this wave's scale stage, after the prefix sums
  uint8_t* stage = reinterpret_cast<uint8_t*>(prefix) + indexer_stage_offset(a.B) + wave * kScaleStageBytes;

  // ---- prefix sum of work blocks over the batch (each thread: a run of
  // consecutive sequences)
  {
    const int per = (a.B + 255) / 256;
    int tot = 0;
    for (int i = 0; i < per; i++) {
      const int bb = tid * per + i;
      if (bb < a.B) tot += work_blocks<SCORES>(a, bb);
    }
    int incl = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int run = incl - tot;
    for (int w = 0; w < wave; w++) run += wsum[w];
    for (int i = 0; i < per; i++) {
      const int bb = tid * per + i;
      if (bb < a.B) {
        prefix[bb] = run;
        run += work_blocks<SCORES>(a, bb);
      }
    }
    if (tid == 0) prefix[a.B] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  // values read from LDS land in vector registers: make the uniform ones
  // scalar again so that loop control and addresses stay in SGPRs
  const int64_t total = __builtin_amdgcn_readfirstlane(prefix[a.B]);
  const int64_t NW = (int64_t)nwg * 4;
  const int64_t W = (int64_t)wg * 4 + wave;
  int64_t gcur = W * total / NW;
  const int64_t gend = (W + 1) * total / NW;

  while (gcur < gend) {
    // sequence of block gcur: prefix[b] <= gcur < prefix[b + 1]
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(prefix[mid]) <= gcur) lo = mid;
      else hi = mid;
    }
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int seq_first = __builtin_amdgcn_readfirstlane(prefix[b]);
    const int seq_next = __builtin_amdgcn_readfirstlane(prefix[b + 1]);
    const int64_t seg_end = min(gend, (int64_t)seq_next);
    const int blk_first = (int)(gcur - seq_first);
    const int Lc = clamp_ctx(a.ctx_lens[b], a.maxb);
    const int nblk = (Lc + kBlock - 1) / kBlock;
    SeqState<KF, HP, TQ> st;
    load_seq<KF, HP, TQ>(a, b, Lc, lane, st);

    for (int w0 = blk_first; w0 < blk_first + (int)(seg_end - gcur); w0 += 64) {
      const int nb = min(64, blk_first + (int)(seg_end - gcur) - w0);
      // page of block w0 + lane (-1: absent or past the context)
      int mypage = -1;
      if (lane < nb && w0 + lane < nblk) {
        const int pg = a.block_table[(size_t)b * a.maxb + w0 + lane];
        if (pg >= 0 && pg < a.num_pages) mypage = pg;
      }
      // NRING rings: block i sits in ring i % NRING (codes T, scales KS)
      KTile<KF> T[NRING][8];
      u32x2 KS[NRING];
      if constexpr (NRING == 1) {
        const int pg = __builtin_amdgcn_readfirstlane(mypage);
        const PageRsrc<KF> r0 = page_rsrc<KF>(a, pg, pg < 0);
        KS[0] = load_kscales<KF>(r0, lane);
#pragma unroll
        for (int k = 0; k < 8; k++) load_ktile<KF>(r0, k, lane, loff, T[0][k]);
      } else {
#pragma unroll
        for (int r = 0; r < NRING; r++) {
          const int pg = r < nb ? __builtin_amdgcn_readlane(mypage, r) : -1;
          const PageRsrc<KF> r0 = page_rsrc<KF>(a, pg, pg < 0);
          KS[r] = load_kscales<KF>(r0, lane);
#pragma unroll
          for (int k = 0; k < 8; k++) load_ktile<KF>(r0, k, lane, loff, T[r][k]);
        }
      }
      // P[tau][g2]: lane i holds the max of block w0 + i for token 4*tau + g2
      float P[S::NTT][4];
#pragma unroll
      for (int tau = 0; tau < S::NTT; tau++)
#pragma unroll
        for (int g2 = 0; g2 < 4; g2++) P[tau][g2] = -INFINITY;
      float mx[S::NTT];
      auto keep_max = [&](int i) {
        if constexpr (!SCORES) {
#pragma unroll
          for (int tau = 0; tau < S::NTT; tau++) {
            const float m = row_max(mx[tau]);
#pragma unroll
            for (int g2 = 0; g2 < 4; g2++) {
              const float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), 16 * g2));
              P[tau][g2] = (lane == i) ? v : P[tau][g2];
            }
          }
        }
      };
      // straight-line steady state: each iteration scores NRING blocks and
      // refills every ring with the block NRING further on (an empty range
      // past the window); the last NRING or fewer blocks are peeled
      int i = 0;
      if constexpr (NRING == 1) {
        for (; i + 1 < nb; i++) {
          const bool absent = __builtin_amdgcn_readlane(mypage, i) < 0;
          const int pgn = __builtin_amdgcn_readlane(mypage, i + 1);
          const PageRsrc<KF> rn = page_rsrc<KF>(a, pgn, pgn < 0);
          score_block<KF, HP, TQ, true, SCORES>(a, T[0], KS[0], stage, st, b, lane, loff, w0 + i, absent, rn, mx);
          keep_max(i);
        }
        const bool absent = __builtin_amdgcn_readlane(mypage, i) < 0;
        score_block<KF, HP, TQ, false, SCORES>(a, T[0], KS[0], stage, st, b, lane, loff, w0 + i, absent,
                                               PageRsrc<KF>{}, mx);
        keep_max(i);
      } else {
      for (; i + NRING < nb; i += NRING) {
#pragma unroll
        for (int r = 0; r < NRING; r++) {
          const bool absent = __builtin_amdgcn_readlane(mypage, i + r) < 0;
          const int pgn = i + r + NRING < nb ? __builtin_amdgcn_readlane(mypage, i + r + NRING) : -1;
          const PageRsrc<KF> rn = page_rsrc<KF>(a, pgn, pgn < 0);
          score_block<KF, HP, TQ, true, SCORES>(a, T[r], KS[r], stage, st, b, lane, loff, w0 + i + r, absent, rn,
                                                mx);
          keep_max(i + r);
        }
      }
#pragma unroll
      for (int r = 0; r < NRING; r++) {
        if (i + r < nb) {
          const bool absent = __builtin_amdgcn_readlane(mypage, i + r) < 0;
          score_block<KF, HP, TQ, false, SCORES>(a, T[r], KS[r], stage, st, b, lane, loff, w0 + i + r, absent,
                                                 PageRsrc<KF>{}, mx);
          keep_max(i + r);
        }
      }
      }
      if constexpr (!SCORES) {
        if (lane < nb) {
#pragma unroll
          for (int tau = 0; tau < S::NTT; tau++)
#pragma unroll
            for (int g2 = 0; g2 < 4; g2++) {
              const int t = 4 * tau + g2;
              if (t < a.Tq) {
                const size_t at = ((size_t)(b * a.Tq + t)) * a.maxb + w0 + lane;
                if constexpr (COHERENT)
                  __hip_atomic_store(reinterpret_cast<uint64_t*>(a.pooled) + at,
                                     ((uint64_t)tag << 32) | __float_as_uint(P[tau][g2]), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
                else
                  a.pooled[at] = P[tau][g2];
              }
            }
        }
      }
    }
    gcur = seg_end;
  }
}

}  // namespace

}  // namespace msa
