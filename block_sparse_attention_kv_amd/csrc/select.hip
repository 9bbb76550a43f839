// select.hip -- pooling of per-key scores and top-k block selection with the
// keep-last rule, for the unfused entry point msa_pool_select_blocks (gfx950).
//
// [ainewsbites page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on NVIDIA
// and AMD GPUs", section "A model built for efficient inference": the scores
// are pooled into one score per block; attention runs only over the top 16
// blocks and the most recent block is always kept.] One 256-thread workgroup
// per (sequence, query token): the visible blocks' scores are max-pooled into
// LDS (or copied there when already pooled), then the workgroup-wide radix
// select of topk.hpp picks the blocks. The fused decode layer runs the same
// selection inside the attention kernel.
#include "fmt.hpp"
#include "msa_internal.hpp"
#include "topk.hpp"

namespace msa {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  extern __shared__ float vals[];  // [maxb]
  __shared__ TopkLds s;
  __shared__ int32_t out[kTopkMax];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int bt = blockIdx.x;
  const int b = bt / a.Tq, t = bt % a.Tq;
  const int Lc = clamp_ctx(a.ctx_lens[b], a.maxb);
  const int p = Lc - a.Tq + t;
  const int n = p < 0 ? 0 : p / kBlock + 1;  // blocks visible to this token

  auto no_page = [](int) { return -1; };
  int cnt;
  if (a.scores_in) {
    // max over the visible keys of each block (2 keys per lane per block)
    const float* sc = a.scores_in + (size_t)bt * a.maxb * kBlock;
    for (int i = wave; i < a.maxb; i += kThreads / 64) {
      float m = -INFINITY;
      if (i < n) {
        const int j0 = i * kBlock + 2 * lane;
        const float2 v = *reinterpret_cast<const float2*>(sc + j0);
        if (j0 <= p) m = v.x;
        if (j0 + 1 <= p) m = fmaxf(m, v.y);
        for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, shfl_xor(m, off));
      }
      if (lane == 0) {
        vals[i] = m;
        if (a.pooled_out) a.pooled_out[(size_t)bt * a.maxb + i] = m;
      }
    }
    __syncthreads();
    cnt = block_topk<kThreads>([&](int i) { return vals[i]; }, no_page, nullptr, n, a.top_k, a.keep_last != 0,
                               out, s);
  } else {
    const float* src = a.pooled_in + (size_t)bt * a.maxb;
    cnt = block_topk<kThreads>([&](int i) { return src[i]; }, no_page, nullptr, n, a.top_k, a.keep_last != 0,
                               out, s);
  }
  int32_t* sel = a.sel + (size_t)bt * a.top_k;
  for (int k = tid; k < a.top_k; k += kThreads) sel[k] = k < cnt ? out[k] : -1;
  if (tid == 0 && a.nsel) a.nsel[bt] = cnt;
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.maxb < 1 || a.maxb > kSelectMaxBlocks || a.top_k < 1 || a.top_k > kTopkMax)
    return hipErrorInvalidValue;
  const size_t lds = (size_t)a.maxb * sizeof(float);
  select_kernel<<<dim3(a.B * a.Tq), kThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace msa
