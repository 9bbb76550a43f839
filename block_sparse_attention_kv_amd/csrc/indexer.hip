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
// Work split. The scan reads every indexer key once, so it is HBM bound (68
// bytes per token for FP8 keys). The grid is persistent (as many workgroups
// as fit on the chip at once). Every workgroup first turns the context
// lengths into a prefix sum of blocks per sequence (in LDS); the blocks of the
// whole batch, laid end to end, are then cut into one contiguous range per
// wavefront, so ragged batches are balanced and every wave streams several
// blocks. A wave walks its range one sequence segment at a time: it loads
// that sequence's queries, weights and the page numbers of up to 64 blocks
// (one per lane), then streams the blocks through a ring of eight 16-key
// tiles held in registers; each tile buffer is refilled with the same tile of
// the next block as soon as it has been consumed, so about one block (8.5 KB)
// per wave is always in flight, and the loop body is straight-line so the
// load counters stay exact.
//
// Matrix cores. The dot products of all T_q*H_i query rows with 16 keys are
// v_mfma_f32_16x16x32_bf16 chains (2 steps over the 64 dims per row tile of
// 16 query rows). Operand layout (checked on gfx950): lane l supplies
// A[row l%16][k = 8*(l/16) + e], B[k = 8*(l/16) + e][col l%16], e = 0..7, and
// receives D[row 4*(l/16) + r][col l%16], r = 0..3. Columns are keys, so the
// four lanes l%16 + 16g (g = 0..3) of a key together hold its whole 64-byte
// FP8 row: lane group g loads dims 16g..16g+15 with one 16-byte load, and one
// load instruction covers 16 consecutive keys = 1 KB of contiguous memory. In
// step s lane group g uses dims 16g + 8s + e (A and B agree on this order).
// FP8 codes widen exactly to bf16 with the hardware converter.
//
// Rows. Query row (t, h) sits in row tile rho = (HP/4)*(t/4) + h/4 at row
// 4*(t%4) + h%4 (HP = heads padded to 4 or 8). Lane group g thus receives
// all heads of token 4*tau + g for every token tile tau, so the head sum, the
// ReLU and the weights need no cross-lane traffic. The per-token key scale
// is applied after the head sum:
//     sum_h w_h max(0, ks*d_h) = ks * sum_h w_h med3(d_h, 0, ks >= 0 ? inf : -inf)
// for either sign of ks. The block max over the 16 keys of a lane group is a
// 4-step DPP reduction inside one 16-lane row.
//
// NVFP4 keys (36 bytes per token) [ainewsbites page, section "Getting
// started and RL support": an NVFP4 indexer KV dtype]: lane group g loads
// the 8 code bytes of dims 16g..16g+15 and their E4M3 scale, and decodes
// them to fp16 exactly (E2M1 x E4M3, as in the attention kernel); the query
// rows of a sequence are scaled into fp16 range by one power of two 2^-e
// (exact), and 2^e times the per-tensor scale is applied after the head sum
// like the FP8 per-token scale (the ReLU commutes with a positive factor).
#include "indexer_impl.hpp"
#include "msa_internal.hpp"

namespace msa {

namespace {

template <int KF, int HP, int TQ, bool SCORES>
__global__ __launch_bounds__(256, indexer_occupancy(KF, HP, TQ)) void indexer_pool_kernel(IndexerArgs a) {
  extern __shared__ __attribute__((aligned(16))) int32_t prefix[];  // indexer_lds_bytes(B): prefix sums, scale stages
  indexer_body<KF, HP, TQ, SCORES, 1>(a, prefix, blockIdx.x, gridDim.x);
}

// Persistent grid: the workgroups resident at once (register and LDS
// limits), capped by the blocks the batch can have (4 waves per workgroup).
int persistent_grid(const IndexerArgs& a, int occupancy, size_t lds) {
  int64_t per_cu = occupancy;  // 4 waves per workgroup: one per SIMD
  const int64_t lds_cap = (int64_t)(160 * 1024) / (int64_t)(lds + 16);
  if (per_cu > lds_cap) per_cu = lds_cap;
  if (per_cu > a.wgs_per_cu) per_cu = a.wgs_per_cu;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = per_cu * a.cus;
  const int64_t need = ((int64_t)a.B * a.maxb + 3) / 4;
  if (grid > need) grid = need;
  return (int)(grid < 1 ? 1 : grid);
}

template <int KF, int HP, bool SCORES>
hipError_t launch_hp(const IndexerArgs& a, hipStream_t s, const KTimer* tm) {
  const size_t lds = indexer_lds_bytes(a.B);
  switch (a.Tq) {
#define MSA_TQ_CASE(T)                                                                                 \
  case T:                                                                                              \
    if constexpr (Shape<HP, T>::RT <= 2) {                                                             \
      const int grid = persistent_grid(a, indexer_occupancy(KF, HP, T), lds);                          \
      return launch_kernel(indexer_pool_kernel<KF, HP, T, SCORES>, dim3(grid), dim3(256), lds, s, a, tm); \
    }                                                                                                  \
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

template <int KF>
hipError_t launch_kf(const IndexerArgs& a, int hp, hipStream_t s, const KTimer* tm) {
  if (a.scores) return hp == 8 ? launch_hp<KF, 8, true>(a, s, tm) : launch_hp<KF, 4, true>(a, s, tm);
  return hp == 8 ? launch_hp<KF, 8, false>(a, s, tm) : launch_hp<KF, 4, false>(a, s, tm);
}

hipError_t launch_indexer(const IndexerArgs& a, int key_format, int hp, hipStream_t s, const KTimer* tm) {
  if ((a.scores != nullptr) == (a.pooled != nullptr)) return hipErrorInvalidValue;
  if (a.B < 1 || a.B > kIndexerMaxSeqs || a.cus < 1 || a.wgs_per_cu < 1) return hipErrorInvalidValue;
  switch (key_format) {
    case kKfBf16: return launch_kf<kKfBf16>(a, hp, s, tm);
    case kKfFp8: return launch_kf<kKfFp8>(a, hp, s, tm);
    case kKfNvfp4: return launch_kf<kKfNvfp4>(a, hp, s, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
