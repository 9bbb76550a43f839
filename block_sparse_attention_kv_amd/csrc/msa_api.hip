// msa_api.hip -- the C ABI of libmsa (include/msa.h): host-side validation,
// workspace carving, launch-shape choice and launches on the caller's stream.
// No device memory is allocated here and nothing synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <mutex>

#include "../../include/msa.h"
#include "msa_internal.hpp"

using namespace msa;

// Scratch of msa_decode_layer_single_static: one array per GPU (the code
// object's copy on each device), held until the process ends. Host code never
// uses this name as an address: the device address comes from
// hipGetSymbolAddress, once per device (static_scratch below).
static __device__ __align__(256) uint8_t scratch[MSA_STATIC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

msa_status_t fail(msa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

msa_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Shape checks shared by every entry point.
msa_status_t check_params(const msa_params_t* p) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "params is NULL");
  if (p->num_seqs < 1 || p->q_len < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->idx_heads < 1 ||
      p->max_blocks_per_seq < 1 || p->num_pages < 1 || p->top_k < 1)
    return fail(MSA_ERR_INVALID_ARG, "sizes must be positive (B=%d Tq=%d Hq=%d Hkv=%d Hi=%d maxb=%d pages=%d top_k=%d)",
                p->num_seqs, p->q_len, p->num_q_heads, p->num_kv_heads, p->idx_heads, p->max_blocks_per_seq,
                p->num_pages, p->top_k);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(MSA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", p->num_q_heads,
                p->num_kv_heads);
  if (p->keep_last != 0 && p->keep_last != 1) return fail(MSA_ERR_INVALID_ARG, "keep_last must be 0 or 1");
  if (p->head_dim != MSA_HEAD_DIM) return fail(MSA_ERR_UNSUPPORTED, "head_dim %d (only 128)", p->head_dim);
  if (p->idx_dim != MSA_IDX_DIM) return fail(MSA_ERR_UNSUPPORTED, "idx_dim %d (only 64)", p->idx_dim);
  if (p->block_size != MSA_BLOCK_SIZE) return fail(MSA_ERR_UNSUPPORTED, "block_size %d (only 128)", p->block_size);
  if (p->top_k > MSA_MAX_TOP_K) return fail(MSA_ERR_UNSUPPORTED, "top_k %d > %d", p->top_k, MSA_MAX_TOP_K);
  if (p->num_q_heads / p->num_kv_heads > MSA_MAX_GROUP)
    return fail(MSA_ERR_UNSUPPORTED, "query heads per KV head %d > %d", p->num_q_heads / p->num_kv_heads,
                MSA_MAX_GROUP);
  if (!((p->q_len <= 4 && p->idx_heads <= 8) || (p->q_len <= 8 && p->idx_heads <= 4)))
    return fail(MSA_ERR_UNSUPPORTED, "q_len %d with idx_heads %d (need q_len<=4 & idx_heads<=8 or q_len<=8 & idx_heads<=4)",
                p->q_len, p->idx_heads);
  if (p->max_blocks_per_seq > MSA_MAX_BLOCKS)
    return fail(MSA_ERR_UNSUPPORTED, "max_blocks_per_seq %d > %d", p->max_blocks_per_seq, MSA_MAX_BLOCKS);
  if (p->num_seqs > MSA_MAX_SEQS) return fail(MSA_ERR_UNSUPPORTED, "num_seqs %d > %d", p->num_seqs, MSA_MAX_SEQS);
  if ((int64_t)p->num_seqs * p->q_len * p->num_kv_heads > 0x7FFFFFFF)
    return fail(MSA_ERR_UNSUPPORTED, "too many (sequence, token, head) items");
  if (p->kv_dtype != MSA_KV_BF16 && p->kv_dtype != MSA_KV_NVFP4)
    return fail(MSA_ERR_UNSUPPORTED, "kv_dtype %d", p->kv_dtype);
  if (p->idx_dtype != MSA_IDX_BF16 && p->idx_dtype != MSA_IDX_FP8_E4M3 && p->idx_dtype != MSA_IDX_NVFP4)
    return fail(MSA_ERR_UNSUPPORTED, "idx_dtype %d", p->idx_dtype);
  if (!(p->softmax_scale == p->softmax_scale)) return fail(MSA_ERR_INVALID_ARG, "softmax_scale is NaN");
  return MSA_OK;
}

msa_status_t check_cache_kv(const msa_params_t* p, const msa_cache_t* c) {
  if (!c) return fail(MSA_ERR_INVALID_ARG, "cache is NULL");
  if (!c->k_data || !c->v_data) return fail(MSA_ERR_INVALID_ARG, "k_data / v_data is NULL");
  if (p->kv_dtype == MSA_KV_NVFP4) {
    if (!c->k_scale || !c->v_scale) return fail(MSA_ERR_INVALID_ARG, "NVFP4 cache needs k_scale and v_scale");
    if (!(isfinite(c->k_tensor_scale) && isfinite(c->v_tensor_scale)))
      return fail(MSA_ERR_INVALID_ARG, "tensor scales must be finite");
  } else if (c->k_scale || c->v_scale) {
    return fail(MSA_ERR_INVALID_ARG, "bf16 cache takes no k_scale / v_scale");
  }
  if (!c->block_table || !c->ctx_lens) return fail(MSA_ERR_INVALID_ARG, "block_table / ctx_lens is NULL");
  return MSA_OK;
}

msa_status_t check_cache_idx(const msa_params_t* p, const msa_cache_t* c) {
  if (!c) return fail(MSA_ERR_INVALID_ARG, "cache is NULL");
  if (!c->idx_k) return fail(MSA_ERR_INVALID_ARG, "idx_k is NULL");
  if (p->idx_dtype == MSA_IDX_FP8_E4M3 && !c->idx_k_scale)
    return fail(MSA_ERR_INVALID_ARG, "FP8 indexer keys need idx_k_scale");
  if (p->idx_dtype == MSA_IDX_NVFP4) {
    if (!c->idx_k_scale) return fail(MSA_ERR_INVALID_ARG, "NVFP4 indexer keys need idx_k_scale");
    if (!isfinite(c->idx_k_tensor_scale))
      return fail(MSA_ERR_INVALID_ARG, "idx_k_tensor_scale must be finite");
  }
  if (p->idx_dtype == MSA_IDX_BF16 && c->idx_k_scale)
    return fail(MSA_ERR_INVALID_ARG, "bf16 indexer keys take no idx_k_scale");
  if (!c->block_table || !c->ctx_lens) return fail(MSA_ERR_INVALID_ARG, "block_table / ctx_lens is NULL");
  return MSA_OK;
}

// Workspace: the pooled block scores of the two-kernel layer (fp32); the
// single-launch layer's tagged 64-bit words (pooled scores in a region of
// their own, so that no fp32 pair the other layer left can pass for a tagged
// word; the selection records; the split items' softmax states; the give-up
// word); and, for small bf16 batches whose two-kernel attention items are
// split over several workgroups, the per-split softmax states and one
// arrival word per item.
struct Layout {
  size_t pooled_off, tagged_off, records_off, lpart_off, gave_up_off, part_off, arrive_off, total;
  int splits;
};
// Most workgroups per item the single launch uses: its split-state region is
// sized for this, whatever the device.
constexpr int kLayerMaxSplits = 4;
// Only the bf16 path splits: its block loop has no prefetch, so a wave pays
// the full load latency per block and one block per wave halves the chain.
// The NVFP4 path prefetches the next block, and there the repeated fused
// selection and the publish/combine of the states cost more than one fewer
// block per wave saves (measured on the 32K and 512K workloads).
int attn_splits(const msa_params_t* p) {
  const int64_t items = (int64_t)p->num_seqs * p->q_len * p->num_kv_heads;
  return (p->kv_dtype == MSA_KV_BF16 && items <= kAttnSplitMaxItems) ? kAttnSplits : 1;
}
Layout layout(const msa_params_t* p) {
  Layout L;
  const size_t bt = (size_t)p->num_seqs * p->q_len;
  const size_t items = bt * p->num_kv_heads;
  L.splits = attn_splits(p);
  L.pooled_off = 0;
  L.tagged_off = align256(bt * p->max_blocks_per_seq * sizeof(float));
  L.records_off = L.tagged_off + align256(bt * p->max_blocks_per_seq * sizeof(uint64_t));
  L.lpart_off = L.records_off + align256(bt * layer_selectors(p->max_blocks_per_seq) * kRecordWords * sizeof(uint64_t));
  L.gave_up_off = L.lpart_off + align256(items * (kLayerMaxSplits - 1) * kStateWords * sizeof(uint64_t));
  L.part_off = L.gave_up_off + 256;
  const size_t part = L.splits > 1 ? items * L.splits * 16 * kPartRow * sizeof(float) : 0;
  L.arrive_off = L.part_off + align256(part);
  L.total = L.arrive_off + (L.splits > 1 ? align256(items * sizeof(unsigned long long)) : 0);
  return L;
}

// Whether `s` is being captured into a HIP graph. The single launch and the
// split attention tag their data with a per-call epoch that the host draws
// at the call; a captured call would replay one epoch and take the previous
// replay's words for its own. (A failed query counts as capturing.)
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return cs != hipStreamCaptureStatusNone;
}

// A distinct epoch per attention launch (arrival words of older launches
// then read as zero); the start is drawn from the clock so that workspaces
// reused across processes do not meet the same sequence.
uint32_t next_epoch() {
  static std::atomic<uint32_t> ctr{0};
  static const uint32_t base = (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u;
  for (;;) {  // never 0: zero-filled memory then holds no call's tag
    const uint32_t e = base + ctr.fetch_add(1, std::memory_order_relaxed) + 1u;
    if (e != 0u) return e;
  }
}

// Splits the two-kernel attention of small bf16 batches when the workspace
// has room and the stream is not being captured.
void set_splits(AttnArgs& a, const msa_params_t* p, void* workspace, size_t ws_bytes, hipStream_t s) {
  const Layout L = layout(p);
  a.splits = 1;
  a.partials = nullptr;
  a.arrivals = nullptr;
  a.epoch = 0;
  if (L.splits > 1 && workspace && ws_bytes >= L.total && (reinterpret_cast<uintptr_t>(workspace) & 255) == 0 &&
      !capturing(s)) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.splits = L.splits;
    a.partials = reinterpret_cast<float*>(ws + L.part_off);
    a.arrivals = reinterpret_cast<unsigned long long*>(ws + L.arrive_off);
    a.epoch = next_epoch();
  }
}

// The epoch of the latest single-launch call on each of the last few
// workspaces (for msa_decode_layer_gave_up).
struct EpochSlot {
  const void* ws;
  uint32_t epoch;
};
std::mutex g_epoch_mu;
EpochSlot g_epochs[64];
int g_epoch_next = 0;

void remember_epoch(const void* ws, uint32_t e) {
  std::lock_guard<std::mutex> lk(g_epoch_mu);
  for (EpochSlot& sl : g_epochs)
    if (sl.ws == ws) {
      sl.epoch = e;
      return;
    }
  g_epochs[g_epoch_next] = EpochSlot{ws, e};
  g_epoch_next = (g_epoch_next + 1) % 64;
}

bool recalled_epoch(const void* ws, uint32_t* e) {
  std::lock_guard<std::mutex> lk(g_epoch_mu);
  for (const EpochSlot& sl : g_epochs)
    if (sl.ws == ws && ws) {
      *e = sl.epoch;
      return true;
    }
  return false;
}

// Shape of the single launch. With at least one (sequence, token, KV head)
// item per compute unit, one workgroup per item selects and attends (fused).
// With fewer items a lone item per compute unit streaming four blocks per
// wave (and, over thousands of blocks, a selection by one workgroup) leaves
// the chip idle: each item split over 4 workgroups of one block per wave,
// with selectors over 1,024-block ranges per token where a context spans
// more than one range (32K-token contexts, 16 items: 20.3 against 23.9 us
// per step fused). A debug export can force the shape: 1 = fused, 2 or 4 =
// split with that many workgroups per item.
std::atomic<int> g_layer_splits{0};
int device_cus();
int layer_splits(const msa_params_t* p) {
  const int forced = g_layer_splits.load(std::memory_order_relaxed);
  if (forced > 0) return forced;
  const int64_t items = (int64_t)p->num_seqs * p->q_len * p->num_kv_heads;
  return items >= (int64_t)device_cus() ? 1 : 4;
}

// Compute units of the current device (the persistent indexer grid is sized
// from it).
#ifndef MSA_INDEXER_WGS_PER_CU
#define MSA_INDEXER_WGS_PER_CU 4
#endif
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Waves per attention workgroup: 4 (two workgroups per compute unit) when
// the batch has at least two (sequence, token, KV head) items per compute
// unit, else 8 so that the selected blocks of the few items are spread over
// more waves.
#ifndef MSA_ATTN_WAVES
#define MSA_ATTN_WAVES 0
#endif
int attn_waves(const msa_params_t* p) {
  if (MSA_ATTN_WAVES > 0) return MSA_ATTN_WAVES;
  const int64_t items = (int64_t)p->num_seqs * p->q_len * p->num_kv_heads;
  return items >= 2 * (int64_t)device_cus() ? 4 : 8;
}

IndexerArgs indexer_args(const msa_params_t* p, const msa_cache_t* c, const void* idx_q, const float* idx_w) {
  IndexerArgs a;
  a.block_table = c->block_table;
  a.ctx_lens = c->ctx_lens;
  a.idx_k = static_cast<const uint8_t*>(c->idx_k);
  a.idx_k_scale = c->idx_k_scale;
  a.idx_ts = c->idx_k_tensor_scale;
  a.idx_q = static_cast<const uint16_t*>(idx_q);
  a.idx_w = idx_w;
  a.pooled = nullptr;
  a.scores = nullptr;
  a.B = p->num_seqs;
  a.Tq = p->q_len;
  a.Hi = p->idx_heads;
  a.maxb = p->max_blocks_per_seq;
  a.num_pages = p->num_pages;
  a.cus = device_cus();
  a.wgs_per_cu = MSA_INDEXER_WGS_PER_CU;
  return a;
}

float softmax_scale(const msa_params_t* p) {
  return p->softmax_scale > 0.0f ? p->softmax_scale : 1.0f / sqrtf((float)p->head_dim);
}

AttnArgs attn_args(const msa_params_t* p, const msa_cache_t* c, const void* q, const float* pooled, int32_t* sel,
                   void* out, float* lse) {
  AttnArgs a;
  a.block_table = c->block_table;
  a.ctx_lens = c->ctx_lens;
  a.pooled = pooled;
  a.sel = sel;
  a.q = static_cast<const uint16_t*>(q);
  a.k_data = static_cast<const uint8_t*>(c->k_data);
  a.k_scale = static_cast<const uint8_t*>(c->k_scale);
  a.v_data = static_cast<const uint8_t*>(c->v_data);
  a.v_scale = static_cast<const uint8_t*>(c->v_scale);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  const bool fp4 = p->kv_dtype == MSA_KV_NVFP4;
  a.score_scale = softmax_scale(p) * 1.4426950408889634f * (fp4 ? c->k_tensor_scale : 1.0f);
  a.v_scale_mul = fp4 ? c->v_tensor_scale : 1.0f;
  a.partials = nullptr;
  a.arrivals = nullptr;
  a.epoch = 0;
  a.spin_limit = 0;
  a.splits = 1;
  a.B = p->num_seqs;
  a.Tq = p->q_len;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.grp = p->num_q_heads / p->num_kv_heads;
  a.maxb = p->max_blocks_per_seq;
  a.num_pages = p->num_pages;
  a.top_k = p->top_k;
  a.keep_last = p->keep_last;
  return a;
}

// Start/stop events of stage i from the caller's array (2 per stage).
KTimer stage_timer(void* const* ev, int i) {
  KTimer t;
  if (ev) {
    t.start = static_cast<hipEvent_t>(ev[2 * i]);
    t.stop = static_cast<hipEvent_t>(ev[2 * i + 1]);
  }
  return t;
}

// Host-visible checks of the single-launch entries.
msa_status_t check_single(const msa_params_t* p, const msa_cache_t* c, const void* q, const void* idx_q,
                          const float* idx_w, void* out) {
  msa_status_t st = check_params(p);
  if (st != MSA_OK) return st;
  if (p->kv_dtype != MSA_KV_NVFP4 || (p->idx_dtype != MSA_IDX_FP8_E4M3 && p->idx_dtype != MSA_IDX_NVFP4) ||
      p->q_len > 4)
    return fail(MSA_ERR_UNSUPPORTED, "single-launch layer: NVFP4 K/V, FP8 or NVFP4 indexer keys, q_len <= 4");
  if ((st = check_cache_kv(p, c)) != MSA_OK) return st;
  if ((st = check_cache_idx(p, c)) != MSA_OK) return st;
  if (!q || !idx_q || !idx_w || !out) return fail(MSA_ERR_INVALID_ARG, "q / idx_q / idx_w / out is NULL");
  return MSA_OK;
}

// Device scratch of one single-launch call: the tagged pooled scores, the
// selection records, the split items' states, the give-up word.
struct SingleScratch {
  uint8_t *tagged, *records, *partials, *gave_up;
};

// The single launch on scratch `sc`; `owner` identifies the scratch for
// msa_decode_layer_gave_up.
msa_status_t run_single(const msa_params_t* p, const msa_cache_t* c, const void* q, const void* idx_q,
                        const float* idx_w, void* out, float* lse, int32_t* sel_out, const SingleScratch& sc,
                        const void* owner, hipStream_t s, void* const* ev) {
  if (capturing(s))
    return fail(MSA_ERR_UNSUPPORTED, "single-launch layer: the stream is being captured into a graph (its data "
                                     "carry a per-call tag drawn on the host, which a replay would repeat)");
  float* pooled = reinterpret_cast<float*>(sc.tagged);  // tagged 64-bit words
  IndexerArgs ia = indexer_args(p, c, idx_q, idx_w);
  ia.pooled = pooled;
  AttnArgs aa = attn_args(p, c, q, pooled, sel_out, out, lse);
  aa.splits = layer_splits(p);
  if (aa.splits > kLayerMaxSplits) return fail(MSA_ERR_UNSUPPORTED, "%d workgroups per item", aa.splits);
  LayerScratch ls;
  ls.records = reinterpret_cast<uint64_t*>(sc.records);
  ls.partials = reinterpret_cast<uint64_t*>(sc.partials);
  ls.gave_up = reinterpret_cast<unsigned long long*>(sc.gave_up);
  const uint32_t epoch = next_epoch();
  remember_epoch(owner, epoch);
  const KTimer tm = stage_timer(ev, 0);
  hipError_t e = launch_layer_single(ia, aa, ls, epoch, aa.splits == 1, p->idx_dtype, p->idx_heads <= 4 ? 4 : 8, s,
                                     &tm);
  return e == hipSuccess ? MSA_OK : hip_fail(e, "single-launch layer");
}

// Offsets in the static scratch: the single launch's regions only, the
// split states only for the shape that uses them.
struct StaticLayout {
  size_t tagged_off, records_off, lpart_off, gave_up_off, total;
};
StaticLayout static_layout(const msa_params_t* p, int splits) {
  StaticLayout L;
  const size_t bt = (size_t)p->num_seqs * p->q_len;
  const size_t items = bt * p->num_kv_heads;
  L.tagged_off = 0;
  L.records_off = align256(bt * p->max_blocks_per_seq * sizeof(uint64_t));
  L.lpart_off = L.records_off + align256(bt * layer_selectors(p->max_blocks_per_seq) * kRecordWords * sizeof(uint64_t));
  L.gave_up_off = L.lpart_off + (splits > 1 ? align256(items * (splits - 1) * kStateWords * sizeof(uint64_t)) : 0);
  L.total = L.gave_up_off + 256;
  return L;
}

// Device address of the static scratch on the current device, looked up
// once per device with that device current.
std::mutex g_scratch_mu;
uint8_t* g_scratch[64];
msa_status_t static_scratch(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MSA_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch[dev];
  return MSA_OK;
}

}  // namespace

namespace msa {
// Streaming read of `bytes` (a multiple of 16) of device memory (debug.hip).
hipError_t launch_debug_read(const void* buf, int64_t bytes, uint32_t* out, int cus, hipStream_t s);
}  // namespace msa

extern "C" {

size_t msa_workspace_size(const msa_params_t* p) {
  if (check_params(p) != MSA_OK) return 0;
  return layout(p).total;
}

msa_status_t msa_indexer_scores(const msa_params_t* p, const msa_cache_t* c, const void* idx_q, const float* idx_w,
                                float* scores, void* stream) {
  g_err[0] = 0;
  msa_status_t st = check_params(p);
  if (st != MSA_OK) return st;
  if ((st = check_cache_idx(p, c)) != MSA_OK) return st;
  if (!idx_q || !idx_w || !scores) return fail(MSA_ERR_INVALID_ARG, "idx_q / idx_w / scores is NULL");
  IndexerArgs a = indexer_args(p, c, idx_q, idx_w);
  a.scores = scores;
  hipError_t e = launch_indexer(a, p->idx_dtype, p->idx_heads <= 4 ? 4 : 8,
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "indexer launch");
}

msa_status_t msa_pool_select_blocks(const msa_params_t* p, const int32_t* ctx_lens, const float* scores,
                                    float* pooled, int32_t* sel, int32_t* nsel, void* stream) {
  g_err[0] = 0;
  msa_status_t st = check_params(p);
  if (st != MSA_OK) return st;
  if (!ctx_lens || !scores || !sel) return fail(MSA_ERR_INVALID_ARG, "ctx_lens / scores / sel is NULL");
  SelectArgs a;
  a.ctx_lens = ctx_lens;
  a.pooled_in = nullptr;
  a.scores_in = scores;
  a.pooled_out = pooled;
  a.sel = sel;
  a.nsel = nsel;
  a.B = p->num_seqs;
  a.Tq = p->q_len;
  a.maxb = p->max_blocks_per_seq;
  a.top_k = p->top_k;
  a.keep_last = p->keep_last;
  hipError_t e = launch_select(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "select launch");
}

msa_status_t msa_sparse_attn_decode(const msa_params_t* p, const msa_cache_t* c, const void* q, const int32_t* sel,
                                    void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  msa_status_t st = check_params(p);
  if (st != MSA_OK) return st;
  if ((st = check_cache_kv(p, c)) != MSA_OK) return st;
  if (!q || !sel || !out) return fail(MSA_ERR_INVALID_ARG, "q / sel / out is NULL");
  AttnArgs a = attn_args(p, c, q, nullptr, const_cast<int32_t*>(sel), out, lse);
  set_splits(a, p, workspace, ws_bytes, static_cast<hipStream_t>(stream));
  hipError_t e = launch_attn(a, p->kv_dtype == MSA_KV_NVFP4, attn_waves(p), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "attention launch");
}

msa_status_t msa_decode_layer_traced(const msa_params_t* p, const msa_cache_t* c, const void* q, const void* idx_q,
                                     const float* idx_w, void* out, float* lse, int32_t* sel_out, void* workspace,
                                     size_t ws_bytes, void* stream, void* const* ev) {
  g_err[0] = 0;
  msa_status_t st = check_params(p);
  if (st != MSA_OK) return st;
  if ((st = check_cache_kv(p, c)) != MSA_OK) return st;
  if ((st = check_cache_idx(p, c)) != MSA_OK) return st;
  if (!q || !idx_q || !idx_w || !out) return fail(MSA_ERR_INVALID_ARG, "q / idx_q / idx_w / out is NULL");
  const Layout L = layout(p);
  if (!workspace) return fail(MSA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
  if (ws_bytes < L.total) return fail(MSA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(MSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* pooled = reinterpret_cast<float*>(ws + L.pooled_off);

  IndexerArgs ia = indexer_args(p, c, idx_q, idx_w);
  ia.pooled = pooled;
  const KTimer t0 = stage_timer(ev, 0), t1 = stage_timer(ev, 1);
  hipError_t e = launch_indexer(ia, p->idx_dtype, p->idx_heads <= 4 ? 4 : 8, s, &t0);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");

  // selection (from the pooled scores) fused into the attention kernel
  AttnArgs aa = attn_args(p, c, q, pooled, sel_out, out, lse);
  set_splits(aa, p, workspace, ws_bytes, s);
  e = launch_attn(aa, p->kv_dtype == MSA_KV_NVFP4, attn_waves(p), s, &t1);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return MSA_OK;
}

msa_status_t msa_decode_layer(const msa_params_t* p, const msa_cache_t* c, const void* q, const void* idx_q,
                              const float* idx_w, void* out, float* lse, int32_t* sel_out, void* workspace,
                              size_t ws_bytes, void* stream) {
  return msa_decode_layer_traced(p, c, q, idx_q, idx_w, out, lse, sel_out, workspace, ws_bytes, stream, nullptr);
}

msa_status_t msa_decode_layer_single_traced(const msa_params_t* p, const msa_cache_t* c, const void* q,
                                            const void* idx_q, const float* idx_w, void* out, float* lse,
                                            int32_t* sel_out, void* workspace, size_t ws_bytes, void* stream,
                                            void* const* ev) {
  g_err[0] = 0;
  msa_status_t st = check_single(p, c, q, idx_q, idx_w, out);
  if (st != MSA_OK) return st;
  const Layout L = layout(p);
  if (!workspace) return fail(MSA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
  if (ws_bytes < L.total) return fail(MSA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(MSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  SingleScratch sc;
  sc.tagged = ws + L.tagged_off;
  sc.records = ws + L.records_off;
  sc.partials = ws + L.lpart_off;
  sc.gave_up = ws + L.gave_up_off;
  return run_single(p, c, q, idx_q, idx_w, out, lse, sel_out, sc, workspace, static_cast<hipStream_t>(stream), ev);
}

msa_status_t msa_decode_layer_single_static(const msa_params_t* p, const msa_cache_t* c, const void* q,
                                            const void* idx_q, const float* idx_w, void* out, float* lse,
                                            int32_t* sel_out, void* stream) {
  g_err[0] = 0;
  msa_status_t st = check_single(p, c, q, idx_q, idx_w, out);
  if (st != MSA_OK) return st;
  const StaticLayout L = static_layout(p, layer_splits(p));
  if (L.total > (size_t)MSA_STATIC_SCRATCH_BYTES)
    return fail(MSA_ERR_UNSUPPORTED, "static scratch: %zu bytes needed, the array holds %u (use "
                                     "msa_decode_layer_single with a workspace)", L.total, MSA_STATIC_SCRATCH_BYTES);
  uint8_t* base = nullptr;
  if ((st = static_scratch(&base)) != MSA_OK) return st;
  SingleScratch sc;
  sc.tagged = base + L.tagged_off;
  sc.records = base + L.records_off;
  sc.partials = base + L.lpart_off;
  sc.gave_up = base + L.gave_up_off;
  return run_single(p, c, q, idx_q, idx_w, out, lse, sel_out, sc, base, static_cast<hipStream_t>(stream), nullptr);
}

msa_status_t msa_decode_layer_gave_up(const msa_params_t* p, const void* workspace, size_t ws_bytes, void* stream,
                                      int64_t* count) {
  g_err[0] = 0;
  msa_status_t st = check_params(p);
  if (st != MSA_OK) return st;
  if (!count) return fail(MSA_ERR_INVALID_ARG, "count is NULL");
  const Layout L = layout(p);
  if (!workspace) return fail(MSA_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < L.total) return fail(MSA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  *count = 0;
  uint32_t epoch = 0;
  if (!recalled_epoch(workspace, &epoch)) return MSA_OK;  // no single-launch call on it from this process
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long word = 0;
  hipError_t e = hipMemcpyAsync(&word, static_cast<const uint8_t*>(workspace) + L.gave_up_off, sizeof(word),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the give-up word");
  if ((uint32_t)(word >> 32) == epoch) *count = (int64_t)(word & 0xFFFFFFFFull);
  return MSA_OK;
}

msa_status_t msa_decode_layer_single(const msa_params_t* p, const msa_cache_t* c, const void* q, const void* idx_q,
                                     const float* idx_w, void* out, float* lse, int32_t* sel_out, void* workspace,
                                     size_t ws_bytes, void* stream) {
  return msa_decode_layer_single_traced(p, c, q, idx_q, idx_w, out, lse, sel_out, workspace, ws_bytes, stream,
                                        nullptr);
}

msa_status_t msa_kv_insert(const msa_params_t* p, const msa_cache_t* c, const void* new_k, const void* new_v,
                           const void* new_idx_k, void* stream) {
  g_err[0] = 0;
  if (!p) return fail(MSA_ERR_INVALID_ARG, "params is NULL");
  if (p->num_seqs < 1 || p->q_len < 1 || p->num_kv_heads < 1 || p->max_blocks_per_seq < 1 || p->num_pages < 1)
    return fail(MSA_ERR_INVALID_ARG, "sizes must be positive (B=%d Tq=%d Hkv=%d maxb=%d pages=%d)", p->num_seqs,
                p->q_len, p->num_kv_heads, p->max_blocks_per_seq, p->num_pages);
  if (p->head_dim != MSA_HEAD_DIM) return fail(MSA_ERR_UNSUPPORTED, "head_dim %d (only 128)", p->head_dim);
  if (p->idx_dim != MSA_IDX_DIM) return fail(MSA_ERR_UNSUPPORTED, "idx_dim %d (only 64)", p->idx_dim);
  if (p->block_size != MSA_BLOCK_SIZE) return fail(MSA_ERR_UNSUPPORTED, "block_size %d (only 128)", p->block_size);
  if (p->max_blocks_per_seq > MSA_MAX_BLOCKS)
    return fail(MSA_ERR_UNSUPPORTED, "max_blocks_per_seq %d > %d", p->max_blocks_per_seq, MSA_MAX_BLOCKS);
  if (p->kv_dtype != MSA_KV_BF16 && p->kv_dtype != MSA_KV_NVFP4)
    return fail(MSA_ERR_UNSUPPORTED, "kv_dtype %d", p->kv_dtype);
  if (p->idx_dtype != MSA_IDX_BF16 && p->idx_dtype != MSA_IDX_FP8_E4M3 && p->idx_dtype != MSA_IDX_NVFP4)
    return fail(MSA_ERR_UNSUPPORTED, "idx_dtype %d", p->idx_dtype);
  if ((int64_t)p->q_len > (int64_t)65535 * 64) return fail(MSA_ERR_UNSUPPORTED, "q_len %d too large", p->q_len);
  if ((int64_t)p->num_seqs * (p->num_kv_heads + 1) > 0x7FFFFFFF)
    return fail(MSA_ERR_UNSUPPORTED, "too many (sequence, head) items");
  msa_status_t st;
  if ((st = check_cache_kv(p, c)) != MSA_OK) return st;
  if ((st = check_cache_idx(p, c)) != MSA_OK) return st;
  if (p->kv_dtype == MSA_KV_NVFP4 && (c->k_tensor_scale == 0.0f || c->v_tensor_scale == 0.0f))
    return fail(MSA_ERR_INVALID_ARG, "tensor scales must be nonzero");
  if (p->idx_dtype == MSA_IDX_NVFP4 && c->idx_k_tensor_scale == 0.0f)
    return fail(MSA_ERR_INVALID_ARG, "idx_k_tensor_scale must be nonzero");
  if (!new_k || !new_v || !new_idx_k) return fail(MSA_ERR_INVALID_ARG, "new_k / new_v / new_idx_k is NULL");
  InsertArgs a;
  a.block_table = c->block_table;
  a.ctx_lens = c->ctx_lens;
  a.k_data = static_cast<uint8_t*>(const_cast<void*>(c->k_data));
  a.k_scale = static_cast<uint8_t*>(const_cast<void*>(c->k_scale));
  a.v_data = static_cast<uint8_t*>(const_cast<void*>(c->v_data));
  a.v_scale = static_cast<uint8_t*>(const_cast<void*>(c->v_scale));
  a.idx_k = static_cast<uint8_t*>(const_cast<void*>(c->idx_k));
  a.idx_k_scale = const_cast<void*>(c->idx_k_scale);
  a.new_k = static_cast<const uint16_t*>(new_k);
  a.new_v = static_cast<const uint16_t*>(new_v);
  a.new_idx_k = static_cast<const uint16_t*>(new_idx_k);
  a.k_ts = (double)c->k_tensor_scale;
  a.v_ts = (double)c->v_tensor_scale;
  a.idx_ts = (double)c->idx_k_tensor_scale;
  a.B = p->num_seqs;
  a.Tq = p->q_len;
  a.Hkv = p->num_kv_heads;
  a.maxb = p->max_blocks_per_seq;
  a.num_pages = p->num_pages;
  a.nvfp4 = p->kv_dtype == MSA_KV_NVFP4;
  a.idx_format = p->idx_dtype;
  hipError_t e = launch_insert(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "insert launch");
}

msa_status_t msa_debug_layer_spin_limit(int32_t polls) {
  g_err[0] = 0;
  if (polls < 0) return fail(MSA_ERR_INVALID_ARG, "polls must be >= 0");
  set_layer_spin_limit(polls);
  return MSA_OK;
}

msa_status_t msa_debug_layer_splits(int32_t splits) {
  g_err[0] = 0;
  if (splits != 0 && splits != 1 && splits != 2 && splits != 4)
    return fail(MSA_ERR_INVALID_ARG, "splits must be 0 (automatic), 1, 2 or 4");
  g_layer_splits.store(splits, std::memory_order_relaxed);
  return MSA_OK;
}

msa_status_t msa_debug_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t n_groups, float* out,
                                     void* stream) {
  g_err[0] = 0;
  if (n_groups < 0) return fail(MSA_ERR_INVALID_ARG, "n_groups < 0");
  if (n_groups > 0 && (!codes || !scales || !out)) return fail(MSA_ERR_INVALID_ARG, "NULL buffer");
  if (n_groups > (int64_t)0xFFFFFFFF * 256) return fail(MSA_ERR_UNSUPPORTED, "n_groups too large");
  hipError_t e = launch_debug_nvfp4(codes, scales, n_groups, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "debug launch");
}

msa_status_t msa_debug_dequant_fp8(const uint8_t* codes, int64_t n, float* out, void* stream) {
  g_err[0] = 0;
  if (n < 0) return fail(MSA_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && (!codes || !out)) return fail(MSA_ERR_INVALID_ARG, "NULL buffer");
  if (n > (int64_t)0xFFFFFFFF * 2048) return fail(MSA_ERR_UNSUPPORTED, "n too large");
  hipError_t e = launch_debug_fp8(codes, n, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "debug launch");
}

msa_status_t msa_debug_read_bandwidth(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
  g_err[0] = 0;
  if (bytes < 0 || bytes % 16 != 0) return fail(MSA_ERR_INVALID_ARG, "bytes must be a non-negative multiple of 16");
  if (bytes > 0 && (!buf || !out)) return fail(MSA_ERR_INVALID_ARG, "NULL buffer");
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0) return fail(MSA_ERR_INVALID_ARG, "buf must be 16-byte aligned");
  hipError_t e = launch_debug_read(buf, bytes, out, device_cus(), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "debug launch");
}

const char* msa_status_string(msa_status_t s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error(void) { return g_err; }

const char* msa_version(void) { return "libmsa 0.1 (gfx950)"; }

}  // extern "C"
