// indexer_args.hpp -- argument block of the indexer + pool kernel (its own
// header, so that the kernel's sources are exactly indexer.hip, fmt.hpp and
// this file).
#pragma once
#include <stdint.h>

namespace msa {

// Indexer + per-block max pool over the paged indexer-key cache.
struct IndexerArgs {
  const int32_t* block_table;  // [B][maxb]
  const int32_t* ctx_lens;     // [B]
  const uint8_t* idx_k;        // FP8 u8[P][128][64], NVFP4 u8[P][128][32] or bf16 [P][128][64]
  const void* idx_k_scale;     // FP8 f32[P][128], NVFP4 u8[P][128][4], bf16 none
  float idx_ts;                // NVFP4 per-tensor scale
  const uint16_t* idx_q;       // bf16 [B][Tq][Hi][64]
  const float* idx_w;          // [B][Tq][Hi]
  float* pooled;               // [B][Tq][maxb] or nullptr
  float* scores;               // [B][Tq][maxb*128] or nullptr
  int B, Tq, Hi, maxb, num_pages;
  int cus;                     // compute units of the device
  int wgs_per_cu;              // cap on resident workgroups per CU (tuning)
};

// The indexer keeps a prefix sum of blocks per sequence in LDS.
constexpr int kIndexerMaxSeqs = 8192;

}  // namespace msa
