// msa_internal.hpp -- kernel argument blocks and launchers shared between the
// kernel translation units and the C-ABI layer (msa_api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// Indexer + per-block max pool over the paged indexer-key cache.
struct IndexerArgs {
  const int32_t* block_table;  // [B][maxb]
  const int32_t* ctx_lens;     // [B]
  const uint8_t* idx_k;        // FP8 u8[P][128][64] or bf16 [P][128][64]
  const float* idx_k_scale;    // [P][128] (FP8 only)
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

// Pool (optional) + top-k block selection per (sequence, query token).
struct SelectArgs {
  const int32_t* ctx_lens;
  const float* pooled_in;  // [B][Tq][maxb] (already pooled) or nullptr
  const float* scores_in;  // [B][Tq][maxb*128] (pooled here) or nullptr
  float* pooled_out;       // [B][Tq][maxb] or nullptr (with scores_in)
  int32_t* sel;            // [B][Tq][top_k]
  int32_t* nsel;           // [B][Tq] or nullptr
  int B, Tq, maxb, top_k, keep_last;
};

// Sparse attention over the selected blocks with the in-WG LSE combine.
struct AttnArgs {
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* sel;       // [B][Tq][top_k]
  const uint16_t* q;        // bf16 [B][Tq][Hq][128]
  const uint8_t* k_data;
  const uint8_t* k_scale;
  const uint8_t* v_data;
  const uint8_t* v_scale;
  uint16_t* out;            // bf16 [B][Tq][Hq][128]
  float* lse;               // [B][Tq][Hq] or nullptr
  float score_scale;        // softmax_scale * log2(e) * k_tensor_scale
  float v_scale_mul;        // v_tensor_scale
  int B, Tq, Hq, Hkv, grp, maxb, num_pages, top_k;
};

hipError_t launch_indexer(const IndexerArgs& a, bool fp8, int hp, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, bool nvfp4, int waves, hipStream_t s);
hipError_t launch_debug_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t n_groups,
                              float* out, hipStream_t s);
hipError_t launch_debug_fp8(const uint8_t* codes, int64_t n, float* out, hipStream_t s);

}  // namespace msa
