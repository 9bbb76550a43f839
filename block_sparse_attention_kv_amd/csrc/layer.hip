// layer.hip -- the decode step of one layer in a single launch (gfx950):
// indexer + block max-pool, then selection and sparse attention per
// (sequence, query token, KV head), ordered by completion flags of the
// indexer waves instead of a kernel boundary.
//
// [upstreambeat page "vLLM turns MiniMax's day-zero promise into
// GPU-specific serving code", section "What changed": on MI355X the decode
// path runs as one launch (the "mono" kernel) to save launch overhead.]
//
// Grid. Workgroups 0 .. n_idx-1 run the persistent indexer scan
// (indexer_impl.hpp) over the batch's (sequence, block) work exactly as the
// indexer kernel does, with two workgroups per compute unit (the register
// budget of the attention) and two blocks of keys in flight per wave. When
// all four waves of such a workgroup are done, it stores the call's epoch
// into its own flag word. Workgroups n_idx + i take attention item i
// (attn_impl.hpp, 4 waves): from the context lengths they find which indexer
// workgroups cover the item's sequence, wait until those flags hold the
// epoch, and run the selection and the attention. The attention workgroups
// come after every indexer workgroup in dispatch order and the indexer
// workgroups wait on nothing, so the waits end; as indexer workgroups retire,
// attention workgroups take their slots. One flag per workgroup, written by
// one thread: no contended atomics, and no clearing (a flag of an older call
// holds another epoch). A wait is also bounded (about a second; a debug
// export can lower the bound): a workgroup that gives up writes NaN outputs
// and lse and a selection of -1.
//
// Coherence. The compute units of different XCDs have separate L2 caches, so
// a device-scope release / acquire fence writes back / invalidates the L2;
// one per workgroup costs several microseconds at the end of the scan. Here
// only device-scope relaxed atomics cross workgroups instead: the pooled
// scores are stored with them (written through to the coherence point), each
// wave waits for the acknowledgement of its stores (s_waitcnt) before the
// workgroup's flag store, and the attention reads the flags and the pooled
// scores with device-scope atomic loads, issued only after the flags were
// seen. No plain load or store touches the pooled scores in this kernel.
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
constexpr int kSpinLimit = 1 << 22;  // polls of one flag (~100 ns each)

// Poll limit of the next launches (0: kSpinLimit); set by a debug export.
std::atomic<int> g_spin_limit{0};

struct LayerArgs {
  IndexerArgs ia;
  AttnArgs aa;
  uint32_t* wg_done;    // [idx_wgs]: epoch once the workgroup's ranges are pooled
  uint32_t epoch;
  int idx_wgs;          // workgroups running the indexer
  int spin_limit;       // polls of one flag before an item gives up
};

// Indexer wave covering global work block g (the inverse of the split
// [W * T / NW, (W + 1) * T / NW)): the largest W with W * T / NW <= g.
__device__ __forceinline__ int64_t covering_wave(int64_t g, int64_t T, int64_t NW) {
  return ((g + 1) * NW + T - 1) / T - 1;
}

template <int KF, int HP, int TQ>
__global__ __launch_bounds__(64 * kLayerWaves, kLayerWgsPerCu) void decode_layer_single_kernel(LayerArgs L) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int64_t red[2][kLayerWaves];
  __shared__ int gave_up;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  if ((int)blockIdx.x < L.idx_wgs) {
    indexer_body<KF, HP, TQ, false, 2, true>(L.ia, reinterpret_cast<int32_t*>(lds), blockIdx.x, L.idx_wgs);
    // release: every wave waits until its device-scope pooled stores are
    // acknowledged, then one flag store (see the note on coherence above)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(L.wg_done + blockIdx.x, L.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const AttnArgs& aa = L.aa;
  const int item = blockIdx.x - L.idx_wgs;
  const int b = item / aa.Hkv / aa.Tq;
  // Until its selection is made an item runs at the highest wave priority:
  // the flag wait and the selection are a chain of dependent steps with
  // little issue work, on the critical path of every item, while the waves
  // it shares a compute unit with stream keys. attn_body drops the priority
  // once the blocks are known (to 1 for the later half of the items, which
  // is dispatched last and ends the kernel: its waves share compute units
  // with older attention waves of the first half, which win issue
  // arbitration by age; to 0 for the rest).
  __builtin_amdgcn_s_setprio(3);

  // work blocks before sequence b and in total (the indexer's numbering)
  int64_t before = 0, total = 0;
  for (int s = tid; s < aa.B; s += 64 * kLayerWaves) {
    const int n = (clamp_ctx(aa.ctx_lens[s], aa.maxb) + kBlock - 1) / kBlock;
    total += n;
    before += s < b ? n : 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    before += __shfl_xor(before, off, kWave);
    total += __shfl_xor(total, off, kWave);
  }
  if (lane == 0) {
    red[0][wave] = before;
    red[1][wave] = total;
  }
  if (tid == 0) gave_up = 0;
  __syncthreads();
  before = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  total = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const int nb = (clamp_ctx(aa.ctx_lens[b], aa.maxb) + kBlock - 1) / kBlock;
  if (nb > 0) {
    const int64_t NW = (int64_t)L.idx_wgs * 4;
    const int64_t wg_lo = covering_wave(before, total, NW) / 4;
    const int64_t wg_hi = covering_wave(before + nb - 1, total, NW) / 4;
    for (int64_t w = wg_lo + tid; w <= wg_hi; w += 64 * kLayerWaves) {
      int n = 0;
      while (__hip_atomic_load(L.wg_done + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != L.epoch &&
             ++n < L.spin_limit)
        __builtin_amdgcn_s_sleep(2);
      if (n >= L.spin_limit) gave_up = 1;
    }
  }
  __syncthreads();
  if (gave_up) {  // mark this item's results invalid: NaN output and lse, no selection
    const int bt = item / aa.Hkv, g = item % aa.Hkv;
    uint16_t* orow = aa.out + ((size_t)bt * aa.Hq + (size_t)g * aa.grp) * kHeadDim;
    for (int i = tid; i < aa.grp * kHeadDim; i += 64 * kLayerWaves) orow[i] = 0x7FC0;
    if (aa.lse && tid < aa.grp) aa.lse[(size_t)bt * aa.Hq + g * aa.grp + tid] = __builtin_nanf("");
    if (g == 0 && aa.sel && tid < aa.top_k) aa.sel[(size_t)bt * aa.top_k + tid] = -1;
    return;
  }
  attn_body<true, kLayerWaves, true>(aa, item, lds, tid);
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

hipError_t launch_layer_single(const IndexerArgs& ia, const AttnArgs& aa, uint32_t* wg_done, uint32_t epoch,
                               int key_format, int hp, hipStream_t s, const KTimer* tm) {
  if (!ia.pooled || ia.scores || aa.pooled != ia.pooled || aa.splits != 1 || !wg_done) return hipErrorInvalidValue;
  if (ia.B < 1 || ia.B > kIndexerMaxSeqs || ia.cus < 1) return hipErrorInvalidValue;
  if (aa.top_k < 1 || aa.top_k > kTopkMax || aa.maxb < 1 || aa.maxb > kSelectMaxBlocks) return hipErrorInvalidValue;
  if (aa.B != ia.B || aa.Tq != ia.Tq || aa.maxb != ia.maxb || aa.ctx_lens != ia.ctx_lens) return hipErrorInvalidValue;
  const int64_t items = (int64_t)aa.B * aa.Tq * aa.Hkv;
  int64_t n_idx = (int64_t)kLayerWgsPerCu * ia.cus;
  const int64_t need = ((int64_t)ia.B * ia.maxb + 3) / 4;  // at least one block per wave
  if (n_idx > need) n_idx = need;
  if (items < 1 || n_idx + items > INT32_MAX || n_idx > kLayerMaxIdxWgs) return hipErrorInvalidValue;
  const int limit = g_spin_limit.load(std::memory_order_relaxed);
  LayerArgs L{ia, aa, wg_done, epoch, (int)n_idx, limit > 0 ? limit : kSpinLimit};
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
