// topk.hpp -- workgroup-wide top-k block selection with the keep-last rule
// (gfx950).
//
// [ainewsbites page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on NVIDIA
// and AMD GPUs", section "A model built for efficient inference": attention
// runs only over the top 16 blocks and the most recent block is always kept.]
// Blocks are ranked by (pooled score desc, block index asc); with keep-last
// the block holding the query position ranks first.
//
// Every block i becomes a unique, nonzero 64-bit key: the order-preserving
// image of its fp32 score in the high word and ~i in the low word, so the top
// k blocks are the k largest keys. A wave finds the k largest of the keys it
// holds (at most five per lane) with an MSB-first search for the threshold:
// bit by bit, keep the bit if at least k keys lie at or above the candidate,
// counting with one 64-bit compare and a ballot population count per key
// slot, and stop as soon as exactly k keys do. No atomics and no barriers are
// involved, so near-equal scores cost no more than distinct ones. Each wave
// reduces its share of the blocks to at most k winners in chunks of 256;
// one wave then reduces the winners of all waves the same way and sorts the
// final k by block index. The result does not depend on thread timing.
#pragma once
#include <climits>

#include "fmt.hpp"

namespace msa {

constexpr int kTopkCap = 16;  // k <= 16

// per wave: winners of its share; then the merged list
struct TopkLds {
  uint64_t win[16][kTopkCap];  // [wave][slot]
  int32_t nwin[16];
  int32_t stale[16];           // [wave]: tagged scores still absent at the poll limit
  uint64_t fin[kTopkCap];
};

// Scores published by other workgroups of the same grid as 64-bit words
// (tag << 32) | (fp32 bits): a word holds a valid score once its high half
// equals `tag`. src[i] is block i's word; a missing word is read again,
// `limit` polls at most.
struct TaggedScores {
  const uint64_t* src;
  uint32_t tag;
  int limit;
};

__device__ __forceinline__ uint64_t block_key(float v, int i, bool forced) {
  const uint32_t o = forced ? 0xFFFFFFFFu : float_ord(v);
  return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

// Number of keys >= c over the NK key slots of the wave (uniform).
template <int NK>
__device__ __forceinline__ int count_ge(const uint64_t (&k)[NK], uint64_t c) {
  int n = 0;
#pragma unroll
  for (int j = 0; j < NK; j++) n += __popcll(__ballot(k[j] >= c));
  return n;
}

// Max (MAX) or min of v over the 64 lanes, returned uniform. DPP moves keep
// the reduction in registers: shifts by 1, 2, 4 and 8 lanes within each row
// of 16 (a lane with no source lane takes the identity) leave the row's
// extremum in its lane 15; row_bcast:15 folds row 0 into row 1 and row 2
// into row 3, row_bcast:31 folds lane 31 into rows 2 and 3, so lane 63 holds
// the result. (A shuffle-based butterfly costs an LDS-crossbar round trip
// per step.)
template <bool MAX>
__device__ __forceinline__ uint32_t wave_extremum_u32(uint32_t v) {
  constexpr int id = MAX ? 0 : -1;
  auto op = [](uint32_t x, int y) { return MAX ? max(x, (uint32_t)y) : min(x, (uint32_t)y); };
  v = op(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = op(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = op(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = op(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = op(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15 -> rows 1, 3
  v = op(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31 -> rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_extremum_u32<true>(v); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_extremum_u32<false>(v); }

// Threshold T with exactly K keys >= T, where K <= have, the number of
// nonzero keys (keys are unique). Returns T (uniform). With K = have every
// nonzero key is a winner and T = 1 without a search.
//
// The search starts below the bits that all nonzero, non-forced keys share
// (the common prefix of their largest and smallest high words): a candidate
// with any higher bit changed would exceed every such key, leaving at most
// the one forced key above it, fewer than K >= 2. With K = 1, or with no
// such key, the search covers all 64 bits.
template <int NK>
__device__ __forceinline__ uint64_t kth_threshold(const uint64_t (&k)[NK], int K, int have) {
  if (K >= have) return 1ull;
  uint32_t hmax = 0u, hmin = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < NK; j++) {
    const uint32_t hi = (uint32_t)(k[j] >> 32);
    const bool use = k[j] != 0ull && hi != 0xFFFFFFFFu;
    hmax = use ? max(hmax, hi) : hmax;
    hmin = use ? min(hmin, hi) : hmin;
  }
  hmax = wave_max_u32(hmax);
  hmin = wave_min_u32(hmin);
  uint64_t T = 0;
  int top = 63;
  if (K >= 2 && hmin <= hmax) {
    const uint32_t d = hmax ^ hmin;
    if (d != 0u) {
      const int b = 31 - __builtin_clz(d);
      T = (uint64_t)(b == 31 ? 0u : (hmax >> (b + 1)) << (b + 1)) << 32;
      top = 32 + b;
    } else {
      T = (uint64_t)hmax << 32;
      top = 31;
    }
  }
  for (int bit = top; bit >= 0; bit--) {
    const uint64_t cand = T | (1ull << bit);
    const int c = count_ge<NK>(k, cand);
    if (c >= K) {
      T = cand;
      if (c == K) break;
    }
  }
  return T;
}

// Number of lanes among 0..15 whose v is below this lane's v, read from the
// lanes' registers (no LDS round trips). All 64 lanes call it; a lane
// outside the ranked set passes INT_MAX, which no value counts.
__device__ __forceinline__ int rank_among16(int v) {
  int r = 0;
#pragma unroll
  for (int q = 0; q < kTopkCap; q++) r += __builtin_amdgcn_readlane(v, q) < v ? 1 : 0;
  return r;
}

// Writes the keys >= T of the NK slots (exactly `cnt` of them) to dst[0..cnt)
// in slot-major, lane-minor order.
template <int NK>
__device__ __forceinline__ void compact_ge(const uint64_t (&k)[NK], uint64_t T, uint64_t* dst) {
  const int lane = lane_id();
  int base = 0;
#pragma unroll
  for (int j = 0; j < NK; j++) {
    const uint64_t m = __ballot(k[j] >= T);
    if (k[j] >= T) dst[base + __popcll(m & ((1ull << lane) - 1ull))] = k[j];
    base += __popcll(m);
  }
}

// The top_k of the n scores score(0..n-1), as ascending block indices in
// out[0..cnt) (LDS), cnt = min(top_k, n); with keep_last the block n-1 is
// ranked first. score(i) may read global memory or LDS: each wave issues the
// reads of a whole chunk (4 per lane) together and prefetches the next chunk.
// When `pages` is not null, pages[i] = page(i) is stored for every i < n as a
// side load of the same pass. All NT threads (a multiple of 64, at most 1024)
// call it; it ends with a barrier, after which out[] and pages[] are visible
// to all of them.
//
// TAGGED: the scores come from tw (score is unused) and are read with
// device-scope atomic loads; a chunk's missing words are polled again (a
// short sleep between polls) until present or until tw.limit polls. Then
// s.stale[w] = 1 for every wave w that gave up (the selection is then
// meaningless), else 0 (also when n <= top_k: no score is read).
template <int NT, bool TAGGED = false, typename ScoreFn, typename PageFn>
__device__ int block_topk(ScoreFn score, PageFn page, int32_t* pages, int n, int top_k, bool keep_last,
                          int32_t* out, TopkLds& s, TaggedScores tw = TaggedScores{nullptr, 0u, 0}) {
  static_assert(NT % 64 == 0 && NT <= 1024, "workgroup size");
  constexpr int NW = NT / 64;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (n <= top_k) {
    for (int k = threadIdx.x; k < n; k += NT) {
      out[k] = k;
      if (pages) pages[k] = page(k);
    }
    if (lane == 0) s.stale[wave] = 0;
    __syncthreads();
    return n < 0 ? 0 : n;
  }
  // ---- this wave's share: blocks [lo, hi), in chunks of 256 (4 per lane)
  const int per = (n + NW - 1) / NW;
  const int lo = min(n, wave * per), hi = min(n, lo + per);
  // TAGGED: the raw words of a chunk are requested first (wv) and turned into
  // scores (v) only when the chunk is searched, after the next chunk's
  // requests are out
  float v[4];
  uint64_t wv[4];
  int pg[4];
  bool stale = false;
  const uint64_t absent_ok = (uint64_t)tw.tag << 32;  // score 0 with the expected tag
  auto fetch = [&](int base, float (&vv)[4], uint64_t (&ww)[4], int (&pp)[4]) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int i = base + 64 * j + lane;
      if constexpr (TAGGED)
        ww[j] = i < hi ? __hip_atomic_load(tw.src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : absent_ok;
      else
        vv[j] = i < hi ? score(i) : 0.0f;
      if (pages) pp[j] = i < hi ? page(i) : -1;
    }
  };
  auto settle = [&](int base) {
    if constexpr (TAGGED) {
      for (int polls = 0;;) {
        bool miss = false;
#pragma unroll
        for (int j = 0; j < 4; j++) miss |= (uint32_t)(wv[j] >> 32) != tw.tag;
        if (__ballot(miss) == 0ull) break;
        if (++polls >= tw.limit) {
          stale = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int i = base + 64 * j + lane;
          if ((uint32_t)(wv[j] >> 32) != tw.tag)
            wv[j] = __hip_atomic_load(tw.src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; j++) v[j] = __uint_as_float((uint32_t)wv[j]);
    }
  };
  if (lo < hi) fetch(lo, v, wv, pg);
  uint64_t carry = 0;  // lanes 0..nc-1: current winners
  int nc = 0;
  for (int base = lo; base < hi; base += 256) {
    float vn[4];
    uint64_t wn[4];
    int pn[4];
    if (base + 256 < hi) fetch(base + 256, vn, wn, pn);
    settle(base);
    uint64_t k[5];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int i = base + 64 * j + lane;
      k[j] = i < hi ? block_key(v[j], i, keep_last && i == n - 1) : 0ull;
      if (pages && i < hi) pages[i] = pg[j];
    }
    k[4] = carry;
    const int have = nc + min(256, hi - base);
    const int K = min(top_k, have);
    if (base == lo) {  // first chunk: no winners carried yet
      const uint64_t (&k4)[4] = reinterpret_cast<const uint64_t (&)[4]>(k);
      compact_ge<4>(k4, kth_threshold<4>(k4, K, have), s.win[wave]);
    } else {
      compact_ge<5>(k, kth_threshold<5>(k, K, have), s.win[wave]);
    }
    wave_lds_sync();
    nc = K;
    carry = lane < nc ? s.win[wave][lane] : 0ull;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if constexpr (TAGGED) wv[j] = wn[j];
      else v[j] = vn[j];
      pg[j] = pn[j];
    }
  }
  if (lane == 0) {
    s.nwin[wave] = nc;
    s.stale[wave] = stale ? 1 : 0;
  }
  __syncthreads();
  // ---- wave 0: top_k of all waves' winners (at most 16 x 16), then sort
  if (wave == 0) {
    constexpr int NJ = (NW * kTopkCap + 63) / 64;  // key slots per lane
    uint64_t k[NJ];
    int have = 0;
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int slot = 64 * j + lane;  // wave slot/16, entry slot%16
      const int w = slot / kTopkCap, e = slot % kTopkCap;
      k[j] = (w < NW && e < s.nwin[w]) ? s.win[w][e] : 0ull;
    }
#pragma unroll
    for (int w = 0; w < NW; w++) have += s.nwin[w];
    const int K = min(top_k, have);
    const uint64_t T = kth_threshold<NJ>(k, K, have);
    compact_ge<NJ>(k, T, s.fin);
    wave_lds_sync();
    const int mine = lane < K ? (int)(0xFFFFFFFFu - (uint32_t)s.fin[lane]) : INT_MAX;
    const int rank = rank_among16(mine);
    if (lane < K) out[rank] = mine;
    if (lane == 0) s.nwin[0] = K;
  }
  __syncthreads();
  return s.nwin[0];
}

}  // namespace msa
