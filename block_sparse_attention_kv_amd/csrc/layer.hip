// layer.hip -- the decode step of one layer in a single launch (gfx950):
// indexer + block max-pool, then selection and sparse attention per
// (sequence, query token, KV head), ordered by tags on the pooled scores
// instead of a kernel boundary.
//
// [upstreambeat page "vLLM turns MiniMax's day-zero promise into
// GPU-specific serving code", section "What changed": on MI355X the decode
// path runs as one launch (the "mono" kernel) to save launch overhead.]
//
// Grid. Workgroups 0 .. n_idx-1 run the persistent indexer scan
// (indexer_impl.hpp) over the batch's (sequence, block) work exactly as the
// indexer kernel does, with two workgroups per compute unit (the register
// budget of the attention) and two blocks of keys in flight per wave. Every
// pooled score is published as one 64-bit word, the call's epoch in the high
// half and the fp32 score in the low half. Workgroups n_idx + i take
// attention item i (attn_impl.hpp, 4 waves): they read the pooled scores of
// their query token right away and read again any word that does not carry
// the epoch yet, then run the selection and the attention. No flag, counter
// or fence is involved, a word left by an older call holds another epoch (the
// workspace is never cleared), and an item needs no knowledge of which
// indexer workgroups cover its sequence. The attention workgroups come after
// every indexer workgroup in dispatch order and the indexer workgroups wait
// on nothing, so the waits end; as indexer workgroups retire, attention
// workgroups take their slots. A wait is also bounded (about a second; a
// debug export can lower the bound): an item that gives up writes NaN
// outputs and lse and a selection of -1.
//
// Coherence. The compute units of different XCDs have separate L2 caches, so
// a device-scope release / acquire fence writes back / invalidates the L2;
// one per workgroup costs several microseconds at the end of the scan. Here
// only device-scope relaxed atomics cross workgroups: 64-bit atomic stores
// of the tagged scores (written through to the coherence point) and 64-bit
// atomic loads; a word is valid by itself, so no ordering between words is
// needed. No plain load or store touches the pooled scores in this kernel.
//
// The pooled scores and the selection equal the two-kernel path's bit for
// bit, and so does the output wherever that path's attention also runs 4
// waves per item (batches with at least two items per compute unit).
// Supported: NVFP4 K/V, FP8 or NVFP4 indexer keys, q_len <= 4.
#include <atomic>

#include "indexer_impl.hpp"
#include "attn_impl.hpp"

namespace msa {

namespace {

constexpr int kLayerWaves = 4;
constexpr int kLayerWgsPerCu = 2;
constexpr int kSpinLimit = 1 << 20;  // polls of one chunk of pooled scores (a memory round trip each)

// Poll limit of the next launches (0: kSpinLimit); set by a debug export.
std::atomic<int> g_spin_limit{0};

struct LayerArgs {
  IndexerArgs ia;
  AttnArgs aa;  // aa.epoch: the tag of the pooled scores; aa.spin_limit: polls of one score
  int idx_wgs;  // workgroups running the indexer
};

template <int KF, int HP, int TQ>
__global__ __launch_bounds__(64 * kLayerWaves, kLayerWgsPerCu) void decode_layer_single_kernel(LayerArgs L) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  if ((int)blockIdx.x < L.idx_wgs) {
    indexer_body<KF, HP, TQ, false, 2, true>(L.ia, reinterpret_cast<int32_t*>(lds), blockIdx.x, L.idx_wgs,
                                             L.aa.epoch);
    return;
  }
  // Until its selection is made an item runs at the highest wave priority:
  // reading the pooled scores and the selection are a chain of dependent
  // steps with little issue work, on the critical path of every item, while
  // the waves it shares a compute unit with stream keys. attn_body drops the
  // priority once the blocks are known (to 1 for the later half of the
  // items, which is dispatched last and ends the kernel: its waves share
  // compute units with older attention waves of the first half, which win
  // issue arbitration by age; to 0 for the rest).
  __builtin_amdgcn_s_setprio(3);
  attn_body<true, kLayerWaves, true>(L.aa, blockIdx.x - L.idx_wgs, lds, (int)threadIdx.x);
}

template <int KF, int HP>
hipError_t launch_single_hp(const LayerArgs& L, int items, hipStream_t s, const KTimer* tm) {
  void (*kern)(LayerArgs) = nullptr;
  switch (L.ia.Tq) {
    case 1: kern = decode_layer_single_kernel<KF, HP, 1>; break;
    case 2: kern = decode_layer_single_kernel<KF, HP, 2>; break;
    case 3: kern = decode_layer_single_kernel<KF, HP, 3>; break;
    case 4: kern = decode_layer_single_kernel<KF, HP, 4>; break;
    default: return hipErrorInvalidValue;
  }
  const size_t idx_lds = ((size_t)L.ia.B + 1) * sizeof(int32_t);
  const size_t att_lds = attn_lds_bytes(L.aa, kLayerWaves);
  const size_t lds = idx_lds > att_lds ? idx_lds : att_lds;
  return launch_kernel(kern, dim3(L.idx_wgs + items), dim3(64 * kLayerWaves), lds, s, L, tm);
}

}  // namespace

void set_layer_spin_limit(int polls) { g_spin_limit.store(polls, std::memory_order_relaxed); }

hipError_t launch_layer_single(const IndexerArgs& ia, const AttnArgs& aa, uint32_t epoch, int key_format, int hp,
                               hipStream_t s, const KTimer* tm) {
  if (!ia.pooled || ia.scores || aa.pooled != ia.pooled || aa.splits != 1) return hipErrorInvalidValue;
  if (ia.B < 1 || ia.B > kIndexerMaxSeqs || ia.cus < 1) return hipErrorInvalidValue;
  if (aa.top_k < 1 || aa.top_k > kTopkMax || aa.maxb < 1 || aa.maxb > kSelectMaxBlocks) return hipErrorInvalidValue;
  if (aa.B != ia.B || aa.Tq != ia.Tq || aa.maxb != ia.maxb || aa.ctx_lens != ia.ctx_lens) return hipErrorInvalidValue;
  const int64_t items = (int64_t)aa.B * aa.Tq * aa.Hkv;
  int64_t n_idx = (int64_t)kLayerWgsPerCu * ia.cus;
  const int64_t need = ((int64_t)ia.B * ia.maxb + 3) / 4;  // at least one block per wave
  if (n_idx > need) n_idx = need;
  if (items < 1 || n_idx + items > INT32_MAX || n_idx > kLayerMaxIdxWgs) return hipErrorInvalidValue;
  const int limit = g_spin_limit.load(std::memory_order_relaxed);
  LayerArgs L{ia, aa, (int)n_idx};
  L.aa.epoch = epoch;
  L.aa.spin_limit = limit > 0 ? limit : kSpinLimit;
  switch (key_format) {
    case kKfFp8:
      return hp == 8 ? launch_single_hp<kKfFp8, 8>(L, (int)items, s, tm) : launch_single_hp<kKfFp8, 4>(L, (int)items, s, tm);
    case kKfNvfp4:
      return hp == 8 ? launch_single_hp<kKfNvfp4, 8>(L, (int)items, s, tm)
                     : launch_single_hp<kKfNvfp4, 4>(L, (int)items, s, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
