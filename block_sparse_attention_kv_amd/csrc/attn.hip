// attn.hip -- exact attention over the selected blocks, NVFP4 (or bf16)
// paged K/V dequantised inside the kernel (gfx950).
//
// [ainewsbites page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on NVIDIA
// and AMD GPUs", section "A model built for efficient inference": main
// attention runs exactly over the top 16 blocks only, at most 2,048 keys per
// query, the most recent block always among them; the KV cache is NVFP4.
// upstreambeat page "vLLM turns MiniMax's day-zero promise into
// GPU-specific serving code", section "What changed": NVFP4 is dequantised
// inside the sparse-attention kernels.]
//
// Work split. One workgroup per (sequence, query token, KV head) with W
// wavefronts; for small bf16 batches S = 4 workgroups per item each take a
// quarter of the selected blocks (one per wave), publish their softmax
// states to the workspace, and the last to arrive merges them in a fixed
// order. In the fused decode layer the workgroup first picks its query
// token's blocks from the pooled scores (topk.hpp); the selection is cheap
// next to the K/V traffic, so the KV heads of one token each repeat it rather
// than wait for one another. Wave w then takes the selected blocks w, w+W, ...
// and keeps an online softmax state (running max m, sum l, output O) for the
// G <= 16 query heads of the KV head. The W states are merged in LDS by a
// fixed-order tree (log-sum-exp combine), so the result is bitwise
// reproducible.
//
// Streaming (NVFP4). A wave keeps the next block's loads in flight while it
// computes the current one: the K of its next block is requested as soon as
// S of the current block is formed, and the V as soon as the P.V product is
// done, into the same registers. Loads go through per-block buffer resources;
// when there is no next block the resources are empty (the loads return
// zeros without touching memory), so the loop is straight-line code and the
// compiler's load counters stay exact.
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
#include "attn_impl.hpp"

namespace msa {

namespace {

template <bool NVFP4, int W>
__global__ __launch_bounds__(64 * W, (W <= 4 ? 2 : 1)) void sparse_attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // select / V-scale stages / merge
  attn_body<NVFP4, W>(a, blockIdx.x, lds, (int)threadIdx.x);
}

template <bool NVFP4>
hipError_t launch_w(const AttnArgs& a, int waves, hipStream_t s, const KTimer* tm) {
  const dim3 grid(a.B * a.Tq * a.Hkv * a.splits);
  const size_t lds = attn_lds_bytes(a, waves);
  switch (waves) {
    case 4: return launch_kernel(sparse_attn_kernel<NVFP4, 4>, grid, dim3(256), lds, s, a, tm);
    case 8: return launch_kernel(sparse_attn_kernel<NVFP4, 8>, grid, dim3(512), lds, s, a, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, bool nvfp4, int waves, hipStream_t s, const KTimer* tm) {
  if (a.top_k < 1 || a.top_k > kTopkMax || a.maxb < 1 || a.maxb > kSelectMaxBlocks) return hipErrorInvalidValue;
  if (a.splits < 1 || a.splits > kTopkMax || (a.splits > 1 && (!a.partials || !a.arrivals)))
    return hipErrorInvalidValue;
  if (a.splits > 1) waves = 4;  // a split share is at most 4 blocks: one per wave
  return nvfp4 ? launch_w<true>(a, waves, s, tm) : launch_w<false>(a, waves, s, tm);
}

}  // namespace msa
