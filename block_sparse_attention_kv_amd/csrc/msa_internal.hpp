// msa_internal.hpp -- kernel argument blocks and launchers shared between the
// kernel translation units and the C-ABI layer (msa_api.hip).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "indexer_args.hpp"

namespace msa {

// Selection: at most 16 blocks per query token; the pooled scores of one
// token (at most 8192 blocks) are held in LDS.
constexpr int kTopkMax = 16;
// Split attention: per head, O[128], m, l and two pad floats (16-byte rows).
constexpr int kPartRow = 132;
constexpr int kAttnSplits = 4;         // workgroups per item for small batches
constexpr int kAttnSplitMaxItems = 64; // items up to which the work is split
constexpr int kSelectMaxBlocks = 8192;

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

// Sparse attention over the selected blocks with the in-workgroup LSE
// combine. With `pooled` set, every workgroup first selects its query
// token's blocks from the pooled scores (fused decode layer) and the
// workgroups of KV head 0 write the selection to `sel` if it is not null;
// otherwise the selection is read from `sel`.
struct AttnArgs {
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const float* pooled;      // [B][Tq][maxb] or nullptr
  int32_t* sel;             // [B][Tq][top_k]: input, or output when pooled
  const uint16_t* q;        // bf16 [B][Tq][Hq][128]
  const uint8_t* k_data;
  const uint8_t* k_scale;
  const uint8_t* v_data;
  const uint8_t* v_scale;
  uint16_t* out;            // bf16 [B][Tq][Hq][128]
  float* lse;               // [B][Tq][Hq] or nullptr
  float* partials;          // [items][splits][16][kPartRow] softmax states (splits > 1)
  unsigned long long* arrivals;  // [items]: (epoch << 32) | workgroups arrived (splits > 1)
  uint32_t epoch;           // distinct per call: older arrival words count as zero; the
                            // single launch's tag of the pooled scores
  int spin_limit;           // single launch: polls of a pooled score before an item gives up
  int splits;               // workgroups per (sequence, token, KV head) item
  float score_scale;        // softmax_scale * log2(e) * k_tensor_scale
  float v_scale_mul;        // v_tensor_scale
  int B, Tq, Hq, Hkv, grp, maxb, num_pages, top_k, keep_last;
};

// KV-insert of the new tokens into the paged caches (writes through the
// cache pointers).
struct InsertArgs {
  const int32_t* block_table;  // [B][maxb]
  const int32_t* ctx_lens;     // [B]
  uint8_t* k_data;             // NVFP4 u8[P][G][128][64] or bf16 [P][G][128][128]
  uint8_t* k_scale;            // u8[P][G][128][8] (NVFP4)
  uint8_t* v_data;             // NVFP4 u8[P][G][128 d][64] or bf16 [P][G][128 d][128]
  uint8_t* v_scale;            // u8[P][G][8][128] (NVFP4)
  uint8_t* idx_k;              // FP8 u8[P][128][64], NVFP4 u8[P][128][32] or bf16 [P][128][64]
  void* idx_k_scale;           // FP8 f32[P][128], NVFP4 u8[P][128][4]
  const uint16_t* new_k;       // bf16 [B][Tq][G][128]
  const uint16_t* new_v;       // bf16 [B][Tq][G][128]
  const uint16_t* new_idx_k;   // bf16 [B][Tq][64]
  double k_ts, v_ts, idx_ts;   // tensor scales (NVFP4)
  int B, Tq, Hkv, maxb, num_pages;
  int nvfp4, idx_format;       // idx_format: msa_idx_dtype_t
};

// Kernel timing hook: when either event is set, the kernel is dispatched with
// hipExtLaunchKernel, which records the kernel's own start and end into them
// (no extra packets in the queue between kernels).
struct KTimer {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Launch of a kernel taking one argument block by value.
template <typename Args>
hipError_t launch_kernel(void (*kern)(Args), dim3 grid, dim3 block, size_t lds, hipStream_t s, const Args& a,
                         const KTimer* t) {
  if (t && (t->start || t->stop)) {
    Args copy = a;
    void* args[] = {&copy};
    const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, args, lds, s,
                                            t->start, t->stop, 0);
    return e != hipSuccess ? e : hipGetLastError();
  }
  kern<<<grid, block, lds, s>>>(a);
  return hipGetLastError();
}

// key_format: msa_idx_dtype_t (0 bf16, 1 FP8, 2 NVFP4)
hipError_t launch_indexer(const IndexerArgs& a, int key_format, int hp, hipStream_t s, const KTimer* t = nullptr);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_insert(const InsertArgs& a, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, bool nvfp4, int waves, hipStream_t s, const KTimer* t = nullptr);
// The decode layer as one launch (layer.hip); NVFP4 K/V, FP8 or NVFP4
// indexer keys, q_len <= 4. ia.pooled / aa.pooled: the workspace's tagged
// pooled scores, 8 bytes per entry; aa.splits: workgroups per attention
// item (1, 2 or 4); epoch: distinct per call, never 0.
constexpr int kLayerMaxIdxWgs = 4096;
// Candidate record of one selector of the single launch (a range of at most
// 1,024 blocks of one query token): a header word (count of candidates,
// kRecordStale when the selection gave up) and three words per candidate
// (ranking key, logical block, page); every word tagged with the call's
// epoch. Padded to kRecordWords words.
constexpr int kRecordWords = 56;
// Tagged softmax state of one split of a split item: 34 rows of 64 words, row
// j < 32 holding O element j of every lane of the publishing wave, rows 32
// and 33 m and l of the 16 heads.
constexpr int kStateWords = 34 * 64;
constexpr uint32_t kRecordStale = 0x80000000u;
struct LayerScratch {
  uint64_t* records;            // [B * Tq][selectors][kRecordWords] (split shape)
  uint64_t* partials;           // [items][splits - 1][kStateWords] tagged softmax states (splits > 1)
  unsigned long long* gave_up;  // (epoch << 32) | workgroups of that call that gave up a wait
};
// Selectors per query token in the split shape for a block table of
// max_blocks columns.
int layer_selectors(int max_blocks);
// fused: one workgroup per item selects and attends (aa.splits must be 1);
// otherwise selectors plus aa.splits attention workgroups per item.
hipError_t launch_layer_single(const IndexerArgs& ia, const AttnArgs& aa, const LayerScratch& ws, uint32_t epoch,
                               bool fused, int key_format, int hp, hipStream_t s, const KTimer* t = nullptr);
// Poll limit of the single-launch layer's waits for later launches (0: the
// default of about a second).
void set_layer_spin_limit(int polls);
hipError_t launch_debug_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t n_groups,
                              float* out, hipStream_t s);
hipError_t launch_debug_fp8(const uint8_t* codes, int64_t n, float* out, hipStream_t s);

}  // namespace msa
