// layer.hip -- the decode step of one layer in a single launch (gfx950):
// indexer + block max-pool, top-k selection, then sparse attention per
// (sequence, query token, KV head), ordered by tags on the data the
// workgroups exchange instead of kernel boundaries.
//
// [upstreambeat page "vLLM turns MiniMax's day-zero promise into
// GPU-specific serving code", section "What changed": on MI355X the decode
// path runs as one launch (the "mono" kernel) to save launch overhead.]
//
// The grid starts with n_idx indexer workgroups: the persistent scan of
// indexer_impl.hpp over the batch's (sequence, block) work, two workgroups
// per compute unit, two blocks of keys in flight per wave. Every pooled score
// is published as one 64-bit word: the call's epoch in the high half, the
// fp32 score in the low half. The rest of the grid has one of two shapes.
//
// Fused (batches with at least one (sequence, token, KV head) item per
// compute unit): one workgroup per item reads its token's tagged pooled
// scores (reading again any word that does not carry the epoch yet), selects
// the top-k blocks itself (topk.hpp) and attends, four blocks per wave. The
// KV heads of a token repeat the cheap selection rather than wait for one
// another.
//
// Split (fewer items, where one item per workgroup would leave most of the
// chip idle and a lone wave streams a block in several microseconds): per
// query token, NSUB selector workgroups followed by H_kv * S attention
// workgroups.
//   selector j     takes blocks [1024 j, 1024 (j+1)) of the token's visible
//                  blocks and publishes its top-k of them as a tagged
//                  candidate record: a header word (count, give-up flag) and,
//                  per candidate, its ranking key (the order-preserving image
//                  of its pooled score), its logical block and its page.
//   attention      (KV head g, split s < S) reads the token's NSUB records
//                  (one round trip once they are there), takes the top-k of
//                  all candidates -- the top-k of the whole context, since
//                  every winner is among its range's top-k -- and attends to
//                  positions [s*per, (s+1)*per) of the selected blocks (per =
//                  ceil(count / S)), one block per wave. Splits s < S-1
//                  publish their merged softmax state (m, l, O of every head
//                  of the group) as tagged words; the last split's waves read
//                  them in parallel, and each of its waves merges two of the
//                  eight dim tiles of splits 0, 1, ..., S-1 in that order, so
//                  the result does not depend on timing.
// Contexts of at most 1,024 blocks get no selectors: every attention
// workgroup then selects from the token's tagged pooled scores itself, as in
// the fused shape, and the selector's hand-over is saved.
// Every wait is on a workgroup earlier in dispatch order, and the indexer
// workgroups wait on nothing: with each XCD dispatching its workgroups in
// order, the earliest unfinished workgroup of the grid can always run to its
// end, so every wait ends. A wait is also bounded (about a second; a debug
// export can lower the bound): a workgroup that gives up marks its results
// invalid (NaN outputs and lse, selection -1) and counts itself in the
// workspace's give-up word, which msa_decode_layer_gave_up reads.
//
// Coherence. The compute units of different XCDs have separate L2 caches, so
// a device-scope release / acquire fence writes back / invalidates the L2;
// one per workgroup costs several microseconds at the end of the scan. Here
// only device-scope relaxed atomics cross workgroups: 64-bit atomic stores
// of tagged words (written through to the coherence point) and 64-bit atomic
// loads. Every word is valid by itself (its tag says which call wrote it),
// so no ordering between words is needed, and no plain load or store
// touches them.
//
// The selection equals the two-kernel path's bit for bit; in the fused shape
// so does the output wherever that path's attention also runs 4 waves per
// item (batches with at least two items per compute unit).
// Supported: NVFP4 K/V, FP8 or NVFP4 indexer keys, q_len <= 4.
#include <atomic>

#include "indexer_impl.hpp"
#include "attn_impl.hpp"

namespace msa {

namespace {

constexpr int kLayerWaves = 4;
constexpr int kLayerThreads = 64 * kLayerWaves;
constexpr int kLayerWgsPerCu = 2;
constexpr int kSpinLimit = 1 << 20;  // polls of one chunk of tagged words (a memory round trip each)
constexpr int kSubBlocks = 1024;     // blocks per selector: one 256-block chunk per wave
constexpr int kCandWords = 1 + 3 * kTopkMax;  // words of a candidate record in use

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// Poll limit of the next launches (0: kSpinLimit); set by a debug export.
std::atomic<int> g_spin_limit{0};

struct LayerArgs {
  IndexerArgs ia;
  AttnArgs aa;            // aa.pooled: the tagged pooled words; aa.epoch: the call's tag;
                          // aa.spin_limit: polls before a wait gives up; aa.splits: S
  LayerScratch ws;
  int idx_wgs;            // workgroups running the indexer
  int nsub;               // split shape: selectors per query token (0: fused shape)
};

__device__ __forceinline__ uint64_t load_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_word(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counts one workgroup that gave up a wait in the give-up word
// (epoch << 32 | count): a word of another call restarts the count. Every
// failed exchange is another workgroup's success, so the loop ends; its
// bound only guards against the unexpected.
__device__ void report_give_up(const LayerArgs& L) {
  unsigned long long* w = L.ws.gave_up;
  const unsigned long long fresh = (unsigned long long)L.aa.epoch << 32;
  unsigned long long seen = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = 0; i < (1 << 16); i++) {
    const unsigned long long want = ((seen >> 32) == L.aa.epoch ? seen : fresh) + 1ull;
    const unsigned long long prev = atomicCAS(w, seen, want);
    if (prev == seen) break;
    seen = prev;
  }
}

// Last visible key of query token `tok` (sequence tok / Tq). The context
// length is read through the scalar cache (the constant address space: the
// array does not change during the call), so that the wait for it is not a
// wait for every vector load issued before it; under the scan's memory load
// each vector round trip costs microseconds.
__device__ __forceinline__ int query_pos(const AttnArgs& a, int tok) {
  typedef __attribute__((address_space(4))) const int32_t cint32;
  const int32_t len = *reinterpret_cast<cint32*>(reinterpret_cast<uintptr_t>(a.ctx_lens + tok / a.Tq));
  return clamp_ctx(len, a.maxb) - a.Tq + tok % a.Tq;
}

// The attention of the W waves over the LDS block lists, given the Q^T
// operand, and the merge of the wave states; wave 0 ends with the
// workgroup's state.
template <int MAXB>
__device__ __forceinline__ void attend_q(const AttnArgs& a, int g, int p, const MfmaT<true>::vec (&qb)[4],
                                         float cscale, const int32_t* blist, const int32_t* plist, int n,
                                         uint8_t* lds, int wave, int lane, SoftmaxState& st) {
  init_state(st);
  stream_blocks<true, kLayerWaves, MAXB>(a, g, p, blist, plist, n, qb, cscale, lds, wave, lane, st);
  merge_waves<kLayerWaves>(st, lds, wave, lane);
}
// The same from the raw bf16 queries.
template <int MAXB>
__device__ __forceinline__ void attend_list(const AttnArgs& a, int tok, int g, int p, const u32x4 (&qraw)[4],
                                            const int32_t* blist, const int32_t* plist, int n, uint8_t* lds,
                                            int wave, int lane, SoftmaxState& st) {
  MfmaT<true>::vec qb[4];
  float cscale;
  convert_q<true>(a, qraw, qb, cscale);
  attend_q<MAXB>(a, g, p, qb, cscale, blist, plist, n, lds, wave, lane, st);
}

// Leaves the top wave priority once the blocks are known: the later half of
// the items (by dispatch position `pos` among the items), dispatched last,
// ends the kernel, and its waves share compute units with older attention
// waves that win issue arbitration by age.
__device__ __forceinline__ void drop_priority(const AttnArgs& a, int pos) {
  if (2 * pos >= a.B * a.Tq * a.Hkv) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Fused shape: the item (token * Hkv + g) at dispatch position r. The
// q_len * Hkv items of one sequence sit 8 positions apart, so that they run
// on one XCD (workgroups go to the 8 XCDs in turn): the blocks several of
// its tokens select -- the query positions' own block always -- and the
// tokens' tagged scores, read by every KV head, can come from that XCD's L2
// (128K spec-verify: 436.3 against 443.3 MB fetched and 74.4-74.7 against
// 75.7-76.1 us per step). Groups of 8 sequences take 8 * q_len * Hkv
// positions; the sequences past the last full group keep their order.
__device__ __forceinline__ int fused_item_at(const AttnArgs& a, int r) {
  const int nit = a.Tq * a.Hkv, full = (a.B / 8) * 8;
  if (r >= full * nit) return r;
  const int grp = r / (8 * nit), rem = r - grp * 8 * nit;
  return (8 * grp + rem % 8) * nit + rem / 8;
}

// ---------------------------------------------------------------- fused shape

// Item `item` = (token, KV head), at dispatch position `pos`: selection from
// the token's tagged pooled scores, then attention over all selected blocks.
__device__ void fused_item(const LayerArgs& L, int item, int pos, uint8_t* lds) {
  const AttnArgs& a = L.aa;
  __shared__ TopkLds tk;
  __shared__ int32_t sel_lds[kTopkMax], blist[kTopkMax], plist[kTopkMax];
  __shared__ int32_t nlist;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = item % a.Hkv, tok = item / a.Hkv;
  const int b = tok / a.Tq;
  const int p = query_pos(a, tok);
  u32x4 qraw[4];
  load_q(a, tok, g, lane, qraw);  // issued first: it does not depend on the selection

  const int nvis = p < 0 ? 0 : p / kBlock + 1;
  int32_t* pages = reinterpret_cast<int32_t*>(lds);  // [nvis]: block-table entries, fetched with the scores
  const int32_t* bt_row = a.block_table + (size_t)b * a.maxb;
  const TaggedScores tw{reinterpret_cast<const uint64_t*>(a.pooled) + (size_t)tok * a.maxb, a.epoch,
                        a.spin_limit};
  const int nsel = block_topk<kLayerThreads, true>([&](int i) { return 0.0f; }, [&](int i) { return bt_row[i]; },
                                                   pages, nvis, a.top_k, a.keep_last != 0, sel_lds, tk, tw);
  bool stale = false;
#pragma unroll
  for (int w = 0; w < kLayerWaves; w++) stale |= tk.stale[w] != 0;
  if (stale) {  // the item's results are marked invalid
    write_invalid(a, tok, g, tid, kLayerThreads);
    if (g == 0 && a.sel && tid < a.top_k) a.sel[(size_t)tok * a.top_k + tid] = -1;
    if (tid == 0) report_give_up(L);
    return;
  }
  if (g == 0 && a.sel && tid < a.top_k) a.sel[(size_t)tok * a.top_k + tid] = tid < nsel ? sel_lds[tid] : -1;
  // attended blocks: selected, visible, with a page in range; ascending
  if (wave == 0) {
    bool ok = false;
    int blk = -1, page = -1;
    if (lane < nsel) {
      blk = sel_lds[lane];
      page = pages[blk];
      ok = page >= 0 && page < a.num_pages;
    }
    const uint64_t bal = __ballot(ok);
    const int pos = __popcll(bal & ((1ull << lane) - 1ull));
    if (ok) {
      blist[pos] = blk;
      plist[pos] = page;
    }
    if (lane == 0) nlist = __popcll(bal);
  }
  __syncthreads();
  drop_priority(a, pos);
  SoftmaxState st;
  attend_list<kTopkMax / kLayerWaves>(a, tok, g, p, qraw, blist, plist, __builtin_amdgcn_readfirstlane(nlist), lds,
                                      wave, lane, st);
  if (wave == 0) write_out(a, tok, g, st, lane);
}

// ---------------------------------------------------------------- split shape

__device__ __forceinline__ uint64_t* cand_record(const LayerArgs& L, int tok, int j) {
  return L.ws.records + ((size_t)tok * L.nsub + j) * kRecordWords;
}

// Selector j of query token `tok`: the top-k of the token's visible blocks
// [1024 j, 1024 (j+1)), published as a candidate record.
__device__ void select_range(const LayerArgs& L, int tok, int j, uint8_t* lds) {
  const AttnArgs& a = L.aa;
  __shared__ TopkLds tk;
  __shared__ int32_t sel_lds[kTopkMax];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = query_pos(a, tok);
  const int nvis = p < 0 ? 0 : p / kBlock + 1;
  const int lo = min(nvis, j * kSubBlocks), hi = min(nvis, lo + kSubBlocks);
  const int n = hi - lo;
  const bool forced = a.keep_last != 0 && hi == nvis;  // the range holds the query's own block
  int32_t* pages = reinterpret_cast<int32_t*>(lds);   // [n]
  const int32_t* bt_row = a.block_table + (size_t)(tok / a.Tq) * a.maxb + lo;
  const uint64_t* words = reinterpret_cast<const uint64_t*>(a.pooled) + (size_t)tok * a.maxb + lo;
  bool stale = false;
  int cnt;
  if (n > a.top_k) {
    block_topk<kLayerThreads, true>([&](int i) { return 0.0f; }, [&](int i) { return bt_row[i]; }, pages, n,
                                    a.top_k, forced, sel_lds, tk, TaggedScores{words, a.epoch, a.spin_limit});
#pragma unroll
    for (int w = 0; w < kLayerWaves; w++) stale |= tk.stale[w] != 0;
    cnt = a.top_k;  // keys of the winners: tk.fin[0 .. top_k)
  } else {
    // every block of the range is a candidate: read its score directly
    if (wave == 0) {
      uint64_t w = 0;
      bool got = true;
      if (lane < n) w = load_word(words + lane);
      for (int polls = 0;;) {
        const bool miss = lane < n && (uint32_t)(w >> 32) != a.epoch;
        if (__ballot(miss) == 0ull) break;
        if (++polls >= a.spin_limit) {
          got = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        if (miss) w = load_word(words + lane);
      }
      if (lane < n) {
        tk.fin[lane] = block_key(__uint_as_float((uint32_t)w), lane, forced && lane == n - 1);
        pages[lane] = bt_row[lane];
      }
      if (lane == 0) tk.stale[0] = got ? 0 : 1;
    }
    __syncthreads();
    stale = tk.stale[0] != 0;
    cnt = n;
  }
  if (wave != 0) return;
  const uint64_t tag = (uint64_t)a.epoch << 32;
  uint64_t* rec = cand_record(L, tok, j);
  if (!stale && lane < cnt) {
    const uint64_t key = tk.fin[lane];
    const int local = (int)(0xFFFFFFFFu - (uint32_t)key);
    const int page = pages[local];
    const bool ok = page >= 0 && page < a.num_pages;
    store_word(rec + 1 + 3 * lane, tag | (uint32_t)(key >> 32));
    store_word(rec + 2 + 3 * lane, tag | (uint32_t)(lo + local));
    store_word(rec + 3 + 3 * lane, tag | (ok ? (uint32_t)page : 0xFFFFFFFFu));
  } else if (lane < kTopkMax) {  // unused entries carry the tag too: a reader polls all of them
    store_word(rec + 1 + 3 * lane, tag);
    store_word(rec + 2 + 3 * lane, tag | 0xFFFFFFFFu);
    store_word(rec + 3 + 3 * lane, tag | 0xFFFFFFFFu);
  }
  if (lane == 0) store_word(rec, tag | (stale ? kRecordStale : 0u) | (uint32_t)(stale ? 0 : cnt));
  if (stale && lane == 0) report_give_up(L);
}

// Tagged partial softmax state of one split (kStateWords words): word
// 64 (4d + r) + lane holds O element (d, r) of the publishing wave's lane
// (h, q4) = (lane & 15, lane >> 4), i.e. head h, dim 16d + 4 q4 + r; words
// 2048 + h and 2112 + h hold m and l of head h. A reading lane loads the
// words of the same lane index, so every load and store instruction covers
// 512 contiguous bytes.
__device__ __forceinline__ uint64_t* split_state(const LayerArgs& L, int item, int split) {
  return L.ws.partials + ((size_t)item * (L.aa.splits - 1) + split) * kStateWords;
}

// Attention of KV head g of query token tok, split `split` of S.
template <int MAXB>
__device__ void split_item(const LayerArgs& L, int tok, int g, int split, uint8_t* lds) {
  const AttnArgs& a = L.aa;
  __shared__ int32_t blist[kTopkMax], plist[kTopkMax], sel_all[kTopkMax];
  __shared__ int32_t nlist, bad, gave[kLayerWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane & 15, q4 = lane >> 4;
  const int S = a.splits;
  const int item = tok * a.Hkv + g;
  const int p = query_pos(a, tok);
  const uint64_t tag = (uint64_t)a.epoch << 32;

  // Q^T operand first: it does not depend on the selection, and the
  // conversion then overlaps the wait for the candidate records
  MfmaT<true>::vec qb[4];
  float cscale;
  {
    u32x4 qraw[4];
    load_q(a, tok, g, lane, qraw);
    convert_q<true>(a, qraw, qb, cscale);
  }

  // ---- without selectors (contexts of at most one selector range): the
  // workgroup selects from the token's tagged pooled scores itself, as in
  // the fused shape, and takes its share of the blocks
  if (L.nsub == 0) {
    __shared__ TopkLds tk;
    __shared__ int32_t sel_lds[kTopkMax];
    const int nvis = p < 0 ? 0 : p / kBlock + 1;
    int32_t* pages = reinterpret_cast<int32_t*>(lds);  // [nvis]
    const int32_t* bt_row = a.block_table + (size_t)(tok / a.Tq) * a.maxb;
    const TaggedScores tw{reinterpret_cast<const uint64_t*>(a.pooled) + (size_t)tok * a.maxb, a.epoch,
                          a.spin_limit};
    const int nsel = block_topk<kLayerThreads, true>([&](int i) { return 0.0f; },
                                                     [&](int i) { return bt_row[i]; }, pages, nvis, a.top_k,
                                                     a.keep_last != 0, sel_lds, tk, tw);
    bool stale = false;
#pragma unroll
    for (int w = 0; w < kLayerWaves; w++) stale |= tk.stale[w] != 0;
    if (wave == 0) {
      // attended blocks (selected, page in range) in ascending order; this
      // split takes positions [split * per, (split + 1) * per)
      const int blk = lane < nsel ? sel_lds[lane] : -1;
      const int page = lane < nsel ? pages[blk] : -1;
      const bool ok = !stale && lane < nsel && page >= 0 && page < a.num_pages;
      const uint64_t bal = __ballot(ok);
      const int apos = __popcll(bal & ((1ull << lane) - 1ull));
      const int cnt = __popcll(bal);
      const int per = (cnt + S - 1) / S, first = split * per;
      if (ok && apos >= first && apos < first + per) {
        blist[apos - first] = blk;
        plist[apos - first] = page;
      }
      if (split == 0 && g == 0 && a.sel && lane < a.top_k)
        a.sel[(size_t)tok * a.top_k + lane] = (!stale && lane < nsel) ? blk : -1;
      if (lane == 0) {
        nlist = stale ? 0 : max(0, min(per, cnt - first));
        bad = stale ? 1 : 0;
        if (stale) report_give_up(L);
      }
    }
  }
  // ---- the token's candidate records -> the top-k blocks -> this split's share
  else if (wave == 0) {
    // candidate c = 16 r + e (record r, entry e) belongs to lane c % 64,
    // slot c / 64 (a second slot only with more than 4 records); the lane
    // reads the record's header and the entry's key, block and page words
    const int nrec = L.nsub;
    const int nslot = nrec > 4 ? 2 : 1;
    uint64_t w[2][4];
    bool got = true;
#pragma unroll
    for (int sl = 0; sl < 2; sl++) {
      const int c = lane + 64 * sl, r = c >> 4, e = c & 15;
      const bool use = sl < nslot && r < nrec;
      const uint64_t* rec = cand_record(L, tok, use ? r : 0);
#pragma unroll
      for (int f = 0; f < 4; f++) w[sl][f] = use ? load_word(rec + (f == 0 ? 0 : 3 * e + f)) : tag;
    }
    for (int polls = 0;; polls++) {
      bool miss = false;
#pragma unroll
      for (int sl = 0; sl < 2; sl++)
#pragma unroll
        for (int f = 0; f < 4; f++) miss |= (uint32_t)(w[sl][f] >> 32) != a.epoch;
      if (__ballot(miss) == 0ull) break;
      if (polls + 1 >= a.spin_limit) {
        got = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int sl = 0; sl < 2; sl++) {
        const int c = lane + 64 * sl, r = c >> 4, e = c & 15;
        const uint64_t* rec = cand_record(L, tok, r < nrec ? r : 0);
#pragma unroll
        for (int f = 0; f < 4; f++)
          if ((uint32_t)(w[sl][f] >> 32) != a.epoch) w[sl][f] = load_word(rec + (f == 0 ? 0 : 3 * e + f));
      }
    }
    // a record marked stale (its selector gave up) or malformed spoils the selection
    bool spoilt = false;
#pragma unroll
    for (int sl = 0; sl < 2; sl++) {
      const uint32_t hdr = (uint32_t)w[sl][0];
      spoilt |= (hdr & kRecordStale) != 0u || (hdr & 0xFFFFu) > (uint32_t)kTopkMax;
    }
    const bool stale = __ballot(spoilt) != 0ull || !got;
    // keys of the valid candidates: (ranking key << 32) | 1 << 20 |
    // (8191 - block) << 7 | c; bit 20 keeps every valid key nonzero
    uint64_t k[2];
    int blk[2], page[2], total = 0;
#pragma unroll
    for (int sl = 0; sl < 2; sl++) {
      const int c = lane + 64 * sl, r = c >> 4, e = c & 15;
      blk[sl] = (int)(uint32_t)w[sl][2];
      page[sl] = (int)(uint32_t)w[sl][3];
      const bool valid = !stale && sl < nslot && r < nrec && e < (int)((uint32_t)w[sl][0] & 0xFFFFu) &&
                         blk[sl] >= 0 && blk[sl] < a.maxb && blk[sl] * kBlock <= p;
      k[sl] = valid ? ((uint64_t)(uint32_t)w[sl][1] << 32) | (1ull << 20) | ((uint64_t)(8191 - blk[sl]) << 7) |
                          (uint64_t)c
                    : 0ull;
      total += __popcll(__ballot(valid));
    }
    const int K = min(a.top_k, total);
    int cnt = 0;
    if (K > 0) {
      // the rank of every key among all candidates (the number of larger
      // keys; keys are unique): at most 128 keys, read from LDS two at a
      // time by every lane at once, a fixed cost where a threshold search
      // over 64-bit keys is a long chain of dependent counts
      __shared__ __attribute__((aligned(16))) uint64_t ckey[kTopkMax * 8];
      __shared__ int32_t wblk_lds[kTopkMax], wpage_lds[kTopkMax];
      ckey[lane] = k[0];
      if (nslot > 1) ckey[lane + 64] = k[1];
      wave_lds_sync();
      const int ncand = nrec * kTopkMax;
      int rk0 = 0, rk1 = 0;
      if (nslot == 1) {
#pragma unroll 8
        for (int j = 0; j < ncand; j += 2) {
          const u64x2 two = *reinterpret_cast<const u64x2*>(ckey + j);
          rk0 += (two[0] > k[0] ? 1 : 0) + (two[1] > k[0] ? 1 : 0);
        }
      } else {
#pragma unroll 8
        for (int j = 0; j < ncand; j += 2) {
          const u64x2 two = *reinterpret_cast<const u64x2*>(ckey + j);
          rk0 += (two[0] > k[0] ? 1 : 0) + (two[1] > k[0] ? 1 : 0);
          rk1 += (two[0] > k[1] ? 1 : 0) + (two[1] > k[1] ? 1 : 0);
        }
      }
      // the winners (rank < K) to lanes 0 .. K-1, in rank order
      if (k[0] != 0ull && rk0 < K) {
        wblk_lds[rk0] = blk[0];
        wpage_lds[rk0] = page[0];
      }
      if (k[1] != 0ull && rk1 < K) {
        wblk_lds[rk1] = blk[1];
        wpage_lds[rk1] = page[1];
      }
      wave_lds_sync();
      const int wblk = lane < K ? wblk_lds[lane] : INT_MAX;
      const int wpage = lane < K ? wpage_lds[lane] : -1;
      const bool ok = lane < K && wpage >= 0 && wpage < a.num_pages;
      // ascending block order (the candidates' blocks are distinct): the
      // winner's position among all winners and among the attended ones
      // (page present)
      const int brank = rank_among16(wblk);
      const int apos = rank_among16(ok ? wblk : INT_MAX);
      if (lane < K) sel_all[brank] = wblk;
      cnt = __popcll(__ballot(ok));
      const int per = (cnt + S - 1) / S, first = split * per;
      if (ok && apos >= first && apos < first + per) {
        blist[apos - first] = wblk;
        plist[apos - first] = wpage;
      }
      if (lane == 0) nlist = max(0, min(per, cnt - first));
    } else if (lane == 0) {
      nlist = 0;
    }
    if (split == 0 && g == 0 && a.sel && lane < a.top_k) {
      wave_lds_sync();
      a.sel[(size_t)tok * a.top_k + lane] = (!stale && lane < K) ? sel_all[lane] : -1;
    }
    if (lane == 0) {
      bad = stale ? 1 : 0;
      if (!got) report_give_up(L);
    }
  }
  __syncthreads();
  if (bad) {
    write_invalid(a, tok, g, tid, kLayerThreads);
    return;
  }
  drop_priority(a, item);
  SoftmaxState st;
  attend_q<MAXB>(a, g, p, qb, cscale, blist, plist, __builtin_amdgcn_readfirstlane(nlist), lds, wave, lane, st);
  if (S == 1) {
    if (wave == 0) write_out(a, tok, g, st, lane);
    return;
  }
  if (split < S - 1) {  // publish this split's state
    if (wave != 0) return;
    uint64_t* row = split_state(L, item, split);
#pragma unroll
    for (int d = 0; d < 8; d++)
#pragma unroll
      for (int r = 0; r < 4; r++) store_word(row + 64 * (4 * d + r) + lane, tag | __float_as_uint(st.o[d][r]));
    if (q4 == 0) {
      store_word(row + 2048 + h, tag | __float_as_uint(st.m));
      store_word(row + 2112 + h, tag | __float_as_uint(st.l));
    }
    return;
  }
  // last split: wave w (1 <= w < S) reads split w-1's state into LDS slot
  // w-1 and wave 0 puts its own in slot S-1; then wave w merges dim tiles
  // 2w and 2w+1 of splits 0, 1, ..., S-1, in that order, and writes them.
  // Each reading wave first waits on one word of its split (head 0's l,
  // stored last), so that a state still being written costs one load per
  // poll, not a whole row.
  float* slots = reinterpret_cast<float*>(lds);
  __syncthreads();  // the wave-merge slots are free again
  if (wave == 0) {
    float* sl = slots + (S - 1) * kSlotFloats;
#pragma unroll
    for (int d = 0; d < 8; d++) *reinterpret_cast<f32x4*>(sl + h * kHeadDim + 16 * d + 4 * q4) = st.o[d];
    if (q4 == 0) {
      sl[16 * kHeadDim + h] = st.m;
      sl[16 * kHeadDim + 16 + h] = st.l;
    }
  } else if (wave < S) {
    const uint64_t* row = split_state(L, item, wave - 1);
    uint64_t wo[32], wm = 0, wl = 0;
    bool got = false;
    for (int polls = 0; polls < a.spin_limit; polls++) {  // head 0's l, stored last
      if ((uint32_t)(__builtin_amdgcn_readfirstlane((int)(load_word(row + 2112) >> 32))) == a.epoch) break;
      __builtin_amdgcn_s_sleep(1);
    }
    // then every word, again only the ones still missing
#pragma unroll
    for (int j = 0; j < 32; j++) wo[j] = load_word(row + 64 * j + lane);
    wm = load_word(row + 2048 + h);
    wl = load_word(row + 2112 + h);
    for (int polls = 0; polls < a.spin_limit; polls++) {
      bool miss = false;
#pragma unroll
      for (int j = 0; j < 32; j++) miss |= (uint32_t)(wo[j] >> 32) != a.epoch;
      miss |= (uint32_t)(wm >> 32) != a.epoch || (uint32_t)(wl >> 32) != a.epoch;
      if (__ballot(miss) == 0ull) {
        got = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int j = 0; j < 32; j++)
        if ((uint32_t)(wo[j] >> 32) != a.epoch) wo[j] = load_word(row + 64 * j + lane);
      if ((uint32_t)(wm >> 32) != a.epoch) wm = load_word(row + 2048 + h);
      if ((uint32_t)(wl >> 32) != a.epoch) wl = load_word(row + 2112 + h);
    }
    float* sl = slots + (wave - 1) * kSlotFloats;
#pragma unroll
    for (int d = 0; d < 8; d++)
#pragma unroll
      for (int r = 0; r < 4; r++) sl[h * kHeadDim + 16 * d + 4 * q4 + r] = __uint_as_float((uint32_t)wo[4 * d + r]);
    if (q4 == 0) {
      sl[16 * kHeadDim + h] = __uint_as_float((uint32_t)wm);
      sl[16 * kHeadDim + 16 + h] = __uint_as_float((uint32_t)wl);
    }
    if (lane == 0) gave[wave] = got ? 0 : 1;
  }
  __syncthreads();
  bool lost = false;
  for (int w = 1; w < S; w++) lost |= gave[w] != 0;
  if (lost) {
    if (wave == 0) {
      write_invalid(a, tok, g, lane, kWave);
      if (lane == 0) report_give_up(L);
    }
    return;
  }
  constexpr int ND = 8 / kLayerWaves;
  const int d0 = ND * wave;
  float m = -INFINITY, l = 0.0f;
  f32x4 o[ND];
#pragma unroll
  for (int i = 0; i < ND; i++) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < S; s++) {
    const float* sl = slots + s * kSlotFloats;
    f32x4 o2[ND];
#pragma unroll
    for (int i = 0; i < ND; i++) o2[i] = *reinterpret_cast<const f32x4*>(sl + h * kHeadDim + 16 * (d0 + i) + 4 * q4);
    merge_tiles<ND>(m, l, o, sl[16 * kHeadDim + h], sl[16 * kHeadDim + 16 + h], o2);
  }
  write_tiles<ND>(a, tok, g, m, l, o, d0, wave == 0, lane);
}

template <int KF, int HP, int TQ, int MAXB>
__global__ __launch_bounds__(kLayerThreads, kLayerWgsPerCu) void decode_layer_single_kernel(LayerArgs L) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  if ((int)blockIdx.x < L.idx_wgs) {
    // Wave priorities of the scan. Split shape: the scan's end is the
    // critical path; the second indexer workgroup of each compute unit (the
    // later-dispatched half) loses issue arbitration to the older one and
    // ends last, and one priority step evens them out (512K: 40.4 against
    // 40.7 us per step). Fused shape: the scan goes one step above the
    // attention items that start in the slots of retired indexer workgroups
    // (after their selection they run at 0 or 1), so that they do not hold
    // back the scan that the later items wait for (ragged batch: 62.2
    // against 66.4 us; 128K spec-verify unchanged). Evening out the two
    // halves there instead delays the items that the early half's end
    // lets start.
    if (L.nsub > 0 || L.aa.splits > 1) {
      if (2 * (int)blockIdx.x >= L.idx_wgs) __builtin_amdgcn_s_setprio(1);
    } else {
      __builtin_amdgcn_s_setprio(1);
    }
    indexer_body<KF, HP, TQ, false, 2, true>(L.ia, reinterpret_cast<int32_t*>(lds), blockIdx.x, L.idx_wgs,
                                             L.aa.epoch);
    return;
  }
  const int r = (int)blockIdx.x - L.idx_wgs;
  if (L.nsub == 0 && L.aa.splits == 1) {
    // In the fused shape an item runs at the highest wave priority until it
    // knows its blocks: reading the tagged scores and selecting are a chain
    // of dependent steps with little issue work, on the critical path of
    // every item, while the waves it shares a compute unit with stream keys.
    // (In the split shape the selectors and attention workgroups fit beside
    // the indexer workgroups and wait through the whole scan; at the top
    // priority their polls slowed the scan: 46.4 against 45.2 us per step
    // on the 512K workload.)
    __builtin_amdgcn_s_setprio(3);
    if constexpr (MAXB == kTopkMax / kLayerWaves) fused_item(L, fused_item_at(L.aa, r), r, lds);
    return;
  }
  const int per_tok = L.nsub + L.aa.Hkv * L.aa.splits;
  const int tok = r / per_tok, k = r - tok * per_tok;
  if (k < L.nsub) {
    select_range(L, tok, k, lds);
    return;
  }
  split_item<MAXB>(L, tok, (k - L.nsub) / L.aa.splits, (k - L.nsub) % L.aa.splits, lds);
}

template <int KF, int HP, int TQ>
void* pick_maxb(int maxb) {
  switch (maxb) {
    case 4: return reinterpret_cast<void*>(decode_layer_single_kernel<KF, HP, TQ, 4>);
    case 2: return reinterpret_cast<void*>(decode_layer_single_kernel<KF, HP, TQ, 2>);
    case 1: return reinterpret_cast<void*>(decode_layer_single_kernel<KF, HP, TQ, 1>);
  }
  return nullptr;
}

template <int KF, int HP>
void* pick_tq(int tq, int maxb) {
  switch (tq) {
    case 1: return pick_maxb<KF, HP, 1>(maxb);
    case 2: return pick_maxb<KF, HP, 2>(maxb);
    case 3: return pick_maxb<KF, HP, 3>(maxb);
    case 4: return pick_maxb<KF, HP, 4>(maxb);
  }
  return nullptr;
}

}  // namespace

void set_layer_spin_limit(int polls) { g_spin_limit.store(polls, std::memory_order_relaxed); }

int layer_selectors(int max_blocks) { return (max_blocks + kSubBlocks - 1) / kSubBlocks; }

hipError_t launch_layer_single(const IndexerArgs& ia, const AttnArgs& aa, const LayerScratch& ws, uint32_t epoch,
                               bool fused, int key_format, int hp, hipStream_t s, const KTimer* tm) {
  if (!ia.pooled || ia.scores || aa.pooled != ia.pooled || !ws.records || !ws.gave_up) return hipErrorInvalidValue;
  if (aa.splits != 1 && aa.splits != 2 && aa.splits != 4) return hipErrorInvalidValue;
  if (fused && aa.splits != 1) return hipErrorInvalidValue;
  if (aa.splits > 1 && !ws.partials) return hipErrorInvalidValue;
  if (ia.B < 1 || ia.B > kIndexerMaxSeqs || ia.cus < 1) return hipErrorInvalidValue;
  if (aa.top_k < 1 || aa.top_k > kTopkMax || aa.maxb < 1 || aa.maxb > kSelectMaxBlocks) return hipErrorInvalidValue;
  if (aa.B != ia.B || aa.Tq != ia.Tq || aa.maxb != ia.maxb || aa.ctx_lens != ia.ctx_lens) return hipErrorInvalidValue;
  if (aa.grp > 16 || aa.Tq < 1 || aa.Tq > 4) return hipErrorInvalidValue;
  // selectors only where a context spans more than one selector range; below
  // that every split item selects from the pooled scores itself
  const int nsub = (fused || aa.maxb <= kSubBlocks) ? 0 : layer_selectors(aa.maxb);
  if (nsub * kRecordWords > 7 * 64 || nsub * kTopkMax > 128) return hipErrorInvalidValue;
  const int64_t tokens = (int64_t)aa.B * aa.Tq;
  const int64_t work = fused ? tokens * aa.Hkv : tokens * (nsub + (int64_t)aa.Hkv * aa.splits);
  int64_t n_idx = (int64_t)kLayerWgsPerCu * ia.cus;
  const int64_t need = ((int64_t)ia.B * ia.maxb + 3) / 4;  // at least one block per wave
  if (n_idx > need) n_idx = need;
  if (n_idx + work > INT32_MAX || n_idx > kLayerMaxIdxWgs) return hipErrorInvalidValue;
  const int limit = g_spin_limit.load(std::memory_order_relaxed);
  LayerArgs L{ia, aa, ws, (int)n_idx, nsub};
  L.aa.epoch = epoch;
  L.aa.spin_limit = limit > 0 ? limit : kSpinLimit;
  const int maxb = kTopkMax / (kLayerWaves * aa.splits);  // blocks per wave at most
  void* kern = nullptr;
  switch (key_format) {
    case kKfFp8: kern = hp == 8 ? pick_tq<kKfFp8, 8>(aa.Tq, maxb) : pick_tq<kKfFp8, 4>(aa.Tq, maxb); break;
    case kKfNvfp4: kern = hp == 8 ? pick_tq<kKfNvfp4, 8>(aa.Tq, maxb) : pick_tq<kKfNvfp4, 4>(aa.Tq, maxb); break;
  }
  if (!kern) return hipErrorInvalidValue;
  // dynamic LDS: the indexer's prefix sums and scale stages, the selection's page table, the
  // attention's K- and V-scale stages, wave-merge slots and split states share one
  // region
  size_t lds = indexer_lds_bytes(ia.B);
  const size_t pages = (size_t)aa.maxb * sizeof(int32_t);
  const size_t stage = (size_t)kLayerWaves * 1024 * 4;
  const size_t merge = (size_t)kLayerWaves * kSlotFloats * 4;  // the last split's S <= 4 states
  lds = lds > pages ? lds : pages;
  lds = lds > stage ? lds : stage;
  lds = lds > merge ? lds : merge;
  return launch_kernel(reinterpret_cast<void (*)(LayerArgs)>(kern), dim3((unsigned)(n_idx + work)),
                       dim3(kLayerThreads), lds, s, L, tm);
}

}  // namespace msa
