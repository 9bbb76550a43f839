// select.hip -- top-k block selection with the keep-last rule (gfx950).
//
// [ainewsbites page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on NVIDIA
// and AMD GPUs", section "A model built for efficient inference": attention
// runs only over the top 16 blocks and the most recent block is always kept.]
// Blocks are ranked by (pooled score desc, block index asc); with keep-last
// the block holding the query position ranks first.
//
// One 256-thread workgroup per (sequence, query token). Each block i becomes
// a unique 64-bit key (order-preserving image of its fp32 score << 32 |
// ~i), so "top k" is "every key >= the k-th largest key". The k-th largest
// key is found by an MSB-first radix select over 8-bit digits with an LDS
// histogram, starting at the first bit where the keys differ (an AND/OR
// reduction finds it), which avoids a pass where every key lands in one bin.
// The k selected indices are then compacted and sorted (k <= 16) by rank.
// The result is deterministic and independent of thread timing.
#include "fmt.hpp"
#include "msa_internal.hpp"

namespace msa {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = shfl_xor(lo, m);
  hi = shfl_xor(hi, m);
  return ((uint64_t)hi << 32) | lo;
}

// KPT: keys per thread (max_blocks <= KPT * 256).
template <int KPT>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  __shared__ float pooled_lds[KPT * kThreads];
  __shared__ uint32_t hist[256];
  __shared__ uint64_t red_and[4], red_or[4];
  __shared__ uint32_t bcast[3];
  __shared__ int32_t picked[32];
  __shared__ uint32_t npicked;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int bt = blockIdx.x;
  const int b = bt / a.Tq, t = bt % a.Tq;
  const int Lc = clamp_ctx(a.ctx_lens[b], a.maxb);
  const int p = Lc - a.Tq + t;
  const int n = p < 0 ? 0 : p / kBlock + 1;  // blocks visible to this token
  int32_t* sel = a.sel + (size_t)bt * a.top_k;

  // ---- pooled scores of this token: from the indexer, or pooled here from
  // the token scores (max over the visible keys of each block).
  if (a.scores_in) {
    const float* sc = a.scores_in + (size_t)bt * a.maxb * kBlock;
    for (int i = wave; i < a.maxb; i += 4) {
      float m = -INFINITY;
      if (i < n) {
        const int j0 = i * kBlock + 2 * lane;
        const float2 v = *reinterpret_cast<const float2*>(sc + j0);
        if (j0 <= p) m = v.x;
        if (j0 + 1 <= p) m = fmaxf(m, v.y);
        for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, shfl_xor(m, off));
      }
      if (lane == 0) {
        if (i < KPT * kThreads) pooled_lds[i] = m;
        if (a.pooled_out) a.pooled_out[(size_t)bt * a.maxb + i] = m;
      }
    }
    __syncthreads();
  }

  if (n <= a.top_k) {  // every visible block is selected
    for (int k = tid; k < a.top_k; k += kThreads) sel[k] = k < n ? k : -1;
    if (tid == 0 && a.nsel) a.nsel[bt] = n;
    return;
  }

  // ---- keys
  uint64_t key[KPT];
  bool ok[KPT];
#pragma unroll
  for (int m = 0; m < KPT; m++) {
    const int i = tid + m * kThreads;
    ok[m] = i < n;
    float v = 0.0f;
    if (ok[m]) v = a.scores_in ? pooled_lds[i] : a.pooled_in[(size_t)bt * a.maxb + i];
    uint32_t o = float_ord(v);
    if (a.keep_last && i == n - 1) o = 0xFFFFFFFFu;
    key[m] = ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
  }

  // ---- first differing bit of the keys
  uint64_t kand = ~0ull, kor = 0ull;
#pragma unroll
  for (int m = 0; m < KPT; m++)
    if (ok[m]) { kand &= key[m]; kor |= key[m]; }
  for (int off = 1; off < 64; off <<= 1) {
    kand &= shfl_xor_u64(kand, off);
    kor |= shfl_xor_u64(kor, off);
  }
  if (lane == 0) { red_and[wave] = kand; red_or[wave] = kor; }
  __syncthreads();
  kand = red_and[0] & red_and[1] & red_and[2] & red_and[3];
  kor = red_or[0] | red_or[1] | red_or[2] | red_or[3];
  const uint64_t diff = kand ^ kor;          // nonzero: indices differ
  const int top_bit = 63 - __clzll(diff);
  int shift = (top_bit / 8) * 8;
  uint64_t mask = (shift + 8 >= 64) ? 0ull : (~0ull << (shift + 8));
  uint64_t prefix = kand & mask;
  uint32_t krem = (uint32_t)a.top_k;

  // ---- radix select of the top_k-th largest key
  for (;;) {
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < KPT; m++)
      if (ok[m] && (key[m] & mask) == prefix) atomicAdd(&hist[(uint32_t)(key[m] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane owns digits 4*lane .. 4*lane+3; suffix sums from the top digit down
      uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      uint32_t loc = h0 + h1 + h2 + h3;
      uint32_t incl = loc;  // sum over lanes >= lane
      for (int off = 1; off < 64; off <<= 1) {
        uint32_t o = __shfl_down(incl, off, kWave);
        if (lane + off < 64) incl += o;
      }
      uint32_t above = incl - loc;  // digits above this lane's four
      const uint32_t hs[4] = {h0, h1, h2, h3};
#pragma unroll
      for (int q = 3; q >= 0; q--) {
        if (above < krem && above + hs[q] >= krem) {
          bcast[0] = 4 * lane + q;
          bcast[1] = above;
          bcast[2] = hs[q];
        }
        above += hs[q];
      }
    }
    __syncthreads();
    const uint32_t d = bcast[0], above = bcast[1], eq = bcast[2];
    prefix |= (uint64_t)d << shift;
    mask |= 255ull << shift;
    krem -= above;
    if (eq == krem || shift == 0) break;
    shift -= 8;
    __syncthreads();  // hist is cleared again at the top of the loop
  }
  // every key >= prefix (low bits zero) is selected: exactly top_k keys
  if (tid == 0) npicked = 0;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < KPT; m++)
    if (ok[m] && key[m] >= prefix) {
      uint32_t slot = atomicAdd(&npicked, 1u);
      if (slot < 32) picked[slot] = tid + m * kThreads;
    }
  __syncthreads();
  if (wave == 0) {
    const int cnt = min((int)npicked, a.top_k);
    if (lane < cnt) {
      const int mine = picked[lane];
      int rank = 0;
      for (int q = 0; q < cnt; q++) rank += picked[q] < mine;
      sel[rank] = mine;
    } else if (lane < a.top_k) {
      sel[lane] = -1;
    }
    if (lane == 0 && a.nsel) a.nsel[bt] = cnt;
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const dim3 grid(a.B * a.Tq);
  const int need = (a.maxb + kThreads - 1) / kThreads;
  if (need <= 1) select_kernel<1><<<grid, kThreads, 0, s>>>(a);
  else if (need <= 2) select_kernel<2><<<grid, kThreads, 0, s>>>(a);
  else if (need <= 4) select_kernel<4><<<grid, kThreads, 0, s>>>(a);
  else if (need <= 8) select_kernel<8><<<grid, kThreads, 0, s>>>(a);
  else if (need <= 16) select_kernel<16><<<grid, kThreads, 0, s>>>(a);
  else if (need <= 32) select_kernel<32><<<grid, kThreads, 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
