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
#include "fmt.hpp"

namespace msa {

constexpr int kTopkCap = 16;  // k <= 16

// per wave: winners of its share; then the merged list
struct TopkLds {
  uint64_t win[16][kTopkCap];  // [wave][slot]
  int32_t nwin[16];
  uint64_t fin[kTopkCap];
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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = max(v, (uint32_t)shfl_xor((int)v, m));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = min(v, (uint32_t)shfl_xor((int)v, m));
  return v;
}

// Threshold T with exactly K keys >= T, K <= number of nonzero keys (keys
// are unique). Returns T (uniform).
//
// The search starts below the bits that all nonzero, non-forced keys share
// (the common prefix of their largest and smallest high words): a candidate
// with any higher bit changed would exceed every such key, leaving at most
// the one forced key above it, fewer than K >= 2. With K = 1, or with no
// such key, the search covers all 64 bits.
template <int NK>
__device__ __forceinline__ uint64_t kth_threshold(const uint64_t (&k)[NK], int K) {
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
template <int NT, typename ScoreFn, typename PageFn>
__device__ int block_topk(ScoreFn score, PageFn page, int32_t* pages, int n, int top_k, bool keep_last,
                          int32_t* out, TopkLds& s) {
  static_assert(NT % 64 == 0 && NT <= 1024, "workgroup size");
  constexpr int NW = NT / 64;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (n <= top_k) {
    for (int k = threadIdx.x; k < n; k += NT) {
      out[k] = k;
      if (pages) pages[k] = page(k);
    }
    __syncthreads();
    return n < 0 ? 0 : n;
  }
  // ---- this wave's share: blocks [lo, hi), in chunks of 256 (4 per lane)
  const int per = (n + NW - 1) / NW;
  const int lo = min(n, wave * per), hi = min(n, lo + per);
  float v[4];
  int pg[4];
  auto fetch = [&](int base, float (&vv)[4], int (&pp)[4]) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int i = base + 64 * j + lane;
      vv[j] = i < hi ? score(i) : 0.0f;
      if (pages) pp[j] = i < hi ? page(i) : -1;
    }
  };
  if (lo < hi) fetch(lo, v, pg);
  uint64_t carry = 0;  // lanes 0..nc-1: current winners
  int nc = 0;
  for (int base = lo; base < hi; base += 256) {
    float vn[4];
    int pn[4];
    if (base + 256 < hi) fetch(base + 256, vn, pn);
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
      compact_ge<4>(k4, kth_threshold<4>(k4, K), s.win[wave]);
    } else {
      compact_ge<5>(k, kth_threshold<5>(k, K), s.win[wave]);
    }
    wave_lds_sync();
    nc = K;
    carry = lane < nc ? s.win[wave][lane] : 0ull;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[j] = vn[j];
      pg[j] = pn[j];
    }
  }
  if (lane == 0) s.nwin[wave] = nc;
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
    const uint64_t T = kth_threshold<NJ>(k, K);
    compact_ge<NJ>(k, T, s.fin);
    wave_lds_sync();
    if (lane < K) {
      const int mine = (int)(0xFFFFFFFFu - (uint32_t)s.fin[lane]);
      int rank = 0;
      for (int q = 0; q < K; q++) rank += (int)(0xFFFFFFFFu - (uint32_t)s.fin[q]) < mine;
      out[rank] = mine;
    }
    if (lane == 0) s.nwin[0] = K;
  }
  __syncthreads();
  return s.nwin[0];
}

}  // namespace msa
