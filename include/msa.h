/*
 * msa.h -- C ABI of libmsa: MiniMax Sparse Attention (MSA) decode on AMD
 * Instinct MI355X (CDNA4, gfx950).
 *
 * What the path computes [page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash
 * on NVIDIA and AMD GPUs" (ainewsbites.com), section "A model built for
 * efficient inference"]: the KV cache is cut into 128-token blocks; a
 * lightweight indexer gives every key of the context a score; the scores of
 * each block are pooled into one block score; exact attention then runs over
 * the 16 best blocks only, the block holding the newest token always being one
 * of them, so no query attends to more than 16 x 128 = 2,048 keys. K and V sit
 * in an NVFP4 cache and are dequantised inside the kernels [same page, same
 * section: the model is quantisation-aware trained for an NVFP4 KV cache;
 * page "vLLM turns MiniMax's day-zero promise into GPU-specific serving code"
 * (upstreambeat.ai), section "What changed": NVFP4 is dequantised inside the
 * sparse-attention kernels].
 *
 * The pages define no formula for the indexer or the pooling. This library
 * computes, for sequence b, query token t and key position j:
 *     s[b,t,j] = sum_h w[b,t,h] * max(0, <qi[b,t,h,:], ki[j,:]>)
 *     P[b,t,i] = max over the valid keys j of block i of s[b,t,j]
 * and selects the top_k blocks by (P desc, block index asc) after setting the
 * pooled score of the block holding the newest key to +inf (keep-last rule).
 *
 * ------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ------------------------------------------------------------------------
 * Ownership.  Every buffer is allocated and freed by the caller. The library
 *   keeps no pointer after a call returns and never allocates device memory;
 *   scratch memory comes only from the caller's workspace argument. A
 *   workspace belongs to one call at a time: calls that may run at the same
 *   time (on different streams) need workspaces of their own.
 * Pointers.  Pointers named "device" must point to device memory of the
 *   current HIP device. msa_params_t and msa_cache_t themselves are host
 *   structures read during the call only.
 * Execution.  Kernels are enqueued on `stream` (a hipStream_t passed as void*,
 *   NULL = the null stream); calls return without synchronising. Outputs are
 *   written completely (padding included). Inputs and outputs must not alias.
 * Errors.  Argument errors that the host can see are reported before anything
 *   is enqueued (MSA_ERR_INVALID_ARG / MSA_ERR_UNSUPPORTED / MSA_ERR_WORKSPACE);
 *   a failed launch reports MSA_ERR_HIP. msa_last_error() returns a
 *   thread-local text describing the last failure. Nothing aborts and no C++
 *   exception crosses the ABI.
 * Device data.  Values inside device buffers are not validated on the host.
 *   The kernels never access memory through them out of bounds: a context
 *   length above max_blocks_per_seq*128 is clamped to it, a block-table entry
 *   outside [0, num_pages) makes that block absent (its keys get score -inf
 *   and it is never attended), and a query token whose position p_t is
 *   negative (ctx_lens[b] < q_len) attends to nothing (output 0, lse -inf,
 *   no block selected).
 *
 * Positions.  ctx_lens[b] = L_b counts the q_len new tokens, whose K/V and
 *   indexer keys are already in the cache. Query token t (0-based) of
 *   sequence b sits at position p_t = L_b - q_len + t and sees keys 0..p_t
 *   (causal inside the window of new tokens).
 *
 * ------------------------------------------------------------------------
 * Paged cache layout (one page = one 128-token block)
 * ------------------------------------------------------------------------
 * NVFP4 element: 4-bit E2M1 code (sign, 2 exponent bits with bias 1,
 *   1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6). Scale: one OCP
 *   E4M3 (e4m3fn) byte per 16 consecutive head_dim elements of one token,
 *   times a per-tensor fp32 scale:  x = e2m1 * e4m3 * tensor_scale.
 *   Storage cost: 64 bytes of codes + 8 scale bytes = 72 bytes for a
 *   128-element vector, i.e. 9/16 of FP8 -- the ratio of the 34,560 and
 *   61,440 bytes per token quoted for the NVFP4 and FP8 caches on the
 *   ainewsbites page, section "A model built for efficient inference".
 *   Within a byte the element with the even index is in bits 0..3.
 *
 * kv_dtype == MSA_KV_NVFP4 (G = num_kv_heads, P = num_pages):
 *   k_data  u8[P][G][128 tok][64]   byte i of token row: d = 2i (low), 2i+1
 *   k_scale u8[P][G][128 tok][8]    scale of d in [16c, 16c+16) of that token
 *   v_data  u8[P][G][128 d][64]     DIM-MAJOR: byte i of dim row d holds
 *                                   tokens 2i (low nibble) and 2i+1 (high)
 *   v_scale u8[P][G][8 c][128 tok]  scale of V[tok][16c .. 16c+16)
 * kv_dtype == MSA_KV_BF16 (no quantisation; scales must be NULL):
 *   k_data  bf16[P][G][128 tok][128 d]
 *   v_data  bf16[P][G][128 d][128 tok]   (dim-major, as above)
 * V is stored dimension-major so that the reduction of P.V (over tokens) is
 * contiguous in memory for each lane of the matrix-core operand.
 *
 * idx_dtype == MSA_IDX_FP8_E4M3:
 *   idx_k       u8[P][128 tok][64]  OCP E4M3 codes
 *   idx_k_scale f32[P][128 tok]     key = e4m3(code) * idx_k_scale[tok]
 * idx_dtype == MSA_IDX_NVFP4 (36 bytes per token instead of 68) [ainewsbites
 *   page, section "Getting started and RL support": the NVIDIA setup runs
 *   the indexer keys in NVFP4 too]:
 *   idx_k       u8[P][128 tok][32]  E2M1 codes, dim 2i in the low nibble
 *   idx_k_scale u8[P][128 tok][4]   E4M3 scale of dims [16c, 16c+16)
 *   key = e2m1 * e4m3 * idx_k_tensor_scale
 * idx_dtype == MSA_IDX_BF16:
 *   idx_k       bf16[P][128 tok][64], idx_k_scale must be NULL.
 *
 * block_table i32[B][max_blocks_per_seq]: logical block -> page.
 * ctx_lens    i32[B].
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_BLOCK_SIZE 128   /* tokens per block / page */
#define MSA_HEAD_DIM 128     /* attention head dimension */
#define MSA_IDX_DIM 64       /* indexer key / query dimension */
#define MSA_MAX_TOP_K 16     /* blocks attended per query token */
#define MSA_MAX_BLOCKS 8192  /* max_blocks_per_seq limit (1,048,576 tokens) */
#define MSA_MAX_GROUP 16     /* num_q_heads / num_kv_heads limit */
#define MSA_MAX_SEQS 8192    /* num_seqs limit */
#define MSA_NUM_STAGES 2     /* kernels enqueued by msa_decode_layer */

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shape */
  MSA_ERR_UNSUPPORTED = 2, /* valid but outside this build's limits */
  MSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  MSA_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} msa_status_t;

typedef enum { MSA_KV_BF16 = 0, MSA_KV_NVFP4 = 1 } msa_kv_dtype_t;
typedef enum { MSA_IDX_BF16 = 0, MSA_IDX_FP8_E4M3 = 1, MSA_IDX_NVFP4 = 2 } msa_idx_dtype_t;

/* Problem description (host struct). Supported: head_dim 128, idx_dim 64,
 * block_size 128, 1 <= top_k <= 16, keep_last in {0,1},
 * num_q_heads % num_kv_heads == 0 with a group of at most 16 query heads,
 * 1 <= idx_heads, and either (q_len <= 4, idx_heads <= 8) or
 * (q_len <= 8, idx_heads <= 4); 1 <= max_blocks_per_seq <= 8192;
 * 1 <= num_seqs <= 8192. */
typedef struct {
  int32_t num_seqs;           /* B */
  int32_t q_len;              /* T_q: query tokens per sequence (same for all) */
  int32_t num_q_heads;        /* H_q */
  int32_t num_kv_heads;       /* H_kv */
  int32_t head_dim;           /* must be 128 */
  int32_t idx_heads;          /* H_i */
  int32_t idx_dim;            /* must be 64 */
  int32_t block_size;         /* must be 128 */
  int32_t top_k;              /* blocks kept per query token (16 in MSA) */
  int32_t keep_last;          /* 1: the block holding p_t is always kept */
  int32_t max_blocks_per_seq; /* columns of block_table */
  int32_t num_pages;          /* pages in the cache arrays */
  float softmax_scale;        /* <= 0 selects 1/sqrt(head_dim) */
  int32_t kv_dtype;           /* msa_kv_dtype_t */
  int32_t idx_dtype;          /* msa_idx_dtype_t */
} msa_params_t;

/* Cache description (host struct holding device pointers; layouts above). */
typedef struct {
  const void* k_data;
  const void* k_scale;        /* NULL for MSA_KV_BF16 */
  const void* v_data;
  const void* v_scale;        /* NULL for MSA_KV_BF16 */
  float k_tensor_scale;       /* per-tensor fp32 scale of K (NVFP4 only) */
  float v_tensor_scale;       /* per-tensor fp32 scale of V (NVFP4 only) */
  const void* idx_k;
  const void* idx_k_scale;    /* FP8: f32[P][128]; NVFP4: u8[P][128][4]; NULL for MSA_IDX_BF16 */
  const int32_t* block_table; /* device i32[B][max_blocks_per_seq] */
  const int32_t* ctx_lens;    /* device i32[B] */
  float idx_k_tensor_scale;   /* per-tensor fp32 scale of NVFP4 indexer keys (ignored otherwise) */
} msa_cache_t;

/* Bytes of workspace msa_decode_layer and msa_sparse_attn_decode need for
 * these parameters (0 if the parameters are invalid). */
size_t msa_workspace_size(const msa_params_t* p);

/* Indexer: every key of every sequence is scored against the indexer query
 * of every query token [ainewsbites page, section "A model built for
 * efficient inference": the indexer gives a score to each key of the whole
 * context].
 *   idx_q  device bf16[B][q_len][idx_heads][64]
 *   idx_w  device f32 [B][q_len][idx_heads]   head weights
 *   scores device f32 [B][q_len][max_blocks_per_seq*128]: s[b,t,j] for
 *          j <= p_t, -inf for j > p_t and for keys of absent blocks. */
msa_status_t msa_indexer_scores(const msa_params_t* p, const msa_cache_t* cache,
                                const void* idx_q, const float* idx_w,
                                float* scores, void* stream);

/* Pool + select [same section: one score per block, the top 16 blocks, the
 * most recent block always kept].
 *   ctx_lens device i32[B]
 *   scores   device f32[B][q_len][max_blocks_per_seq*128] (as written above)
 *   pooled   device f32[B][q_len][max_blocks_per_seq] or NULL: max of each
 *            block's valid scores; -inf past the last block of token t.
 *   sel      device i32[B][q_len][top_k]: selected logical block indices,
 *            ascending, padded with -1.
 *   nsel     device i32[B][q_len] or NULL: number of selected blocks,
 *            min(top_k, n_blk_t) with n_blk_t = ceil((p_t+1)/128).
 * Order: block i beats block i' if P_i > P_i', or P_i == P_i' and i < i'.
 * With keep_last the block of p_t is ranked first. NaN scores are not
 * supported (their rank is unspecified). */
msa_status_t msa_pool_select_blocks(const msa_params_t* p, const int32_t* ctx_lens,
                                    const float* scores, float* pooled, int32_t* sel,
                                    int32_t* nsel, void* stream);

/* Exact attention of every query head over the keys of the selected blocks
 * [same section: the attention itself is exact, restricted to the 16 best
 * blocks], keys j <= p_t only, K/V dequantised inside the kernel.
 *   q     device bf16[B][q_len][num_q_heads][128]
 *   sel   device i32[B][q_len][top_k] (as produced by msa_pool_select_blocks;
 *         entries < 0 or >= max_blocks_per_seq are skipped)
 *   out   device bf16[B][q_len][num_q_heads][128], RNE from fp32
 *   lse   device f32[B][q_len][num_q_heads] or NULL: natural log of
 *         sum_j exp(softmax_scale * <q, k_j>) over the attended keys.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads). */
msa_status_t msa_sparse_attn_decode(const msa_params_t* p, const msa_cache_t* cache,
                                    const void* q, const int32_t* sel, void* out,
                                    float* lse, void* workspace, size_t ws_bytes,
                                    void* stream);

/* The whole decode step of one MSA layer in MSA_NUM_STAGES kernels on
 * `stream`: (1) indexer + per-block max pool into the workspace, (2) per
 * (sequence, query token, KV head): selection from the pooled scores, then
 * sparse attention. The selection equals msa_pool_select_blocks' on the
 * same pooled scores.
 *   sel_out device i32[B][q_len][top_k] or NULL: the selection used.
 *   lse     as in msa_sparse_attn_decode, or NULL.
 *   workspace at least msa_workspace_size(p) bytes of device memory, 256-byte
 *   aligned; its contents on entry do not matter. */
msa_status_t msa_decode_layer(const msa_params_t* p, const msa_cache_t* cache,
                              const void* q, const void* idx_q, const float* idx_w,
                              void* out, float* lse, int32_t* sel_out,
                              void* workspace, size_t ws_bytes, void* stream);

/* msa_decode_layer with a tracing hook: when `stage_events` is not NULL it
 * holds 2 * MSA_NUM_STAGES hipEvent_t handles (created by the caller, NULL
 * entries allowed). Kernel i is dispatched so that the dispatch itself
 * records the kernel's start into event 2i and its end into event 2i+1
 * (hipExtLaunchKernel), without extra packets between the kernels; the caller
 * times kernel i with hipEventElapsedTime(event 2i, event 2i+1). */
msa_status_t msa_decode_layer_traced(const msa_params_t* p, const msa_cache_t* cache,
                                     const void* q, const void* idx_q, const float* idx_w,
                                     void* out, float* lse, int32_t* sel_out,
                                     void* workspace, size_t ws_bytes, void* stream,
                                     void* const* stage_events);

/* msa_decode_layer as ONE kernel launch on `stream` [upstreambeat page
 * "vLLM turns MiniMax's day-zero promise into GPU-specific serving code",
 * section "What changed": a single-launch ("mono") decode path on MI355X to
 * cut launch overhead]. The grid runs, in dispatch order, the indexer and
 * pooling phase, which publishes every pooled score tagged with the call's
 * epoch, then the selection and attention. With at least one (sequence,
 * token, KV head) item per compute unit, one workgroup per item reads its
 * token's tagged scores, selects and attends. With fewer items, each item
 * is split over 4 attention workgroups; where max_blocks_per_seq exceeds
 * 1,024, each token first gets selector workgroups (one per 1,024 blocks)
 * that publish their top-k candidates as tagged records for the attention
 * workgroups to merge, otherwise each attention workgroup selects itself.
 * The 4 workgroups of an item attend to a share of the selected blocks each
 * and meet through tagged partial softmax
 * states, the last one merging them in a fixed order, so results do not
 * depend on timing. Same arguments, workspace and selection as
 * msa_decode_layer; out and lse equal msa_decode_layer's bit for bit from
 * two items per compute unit up (below that the two paths merge partial
 * states in different orders and agree to rounding). Every wait is on a
 * workgroup dispatched earlier and the indexer workgroups wait on nothing,
 * so every wait ends; each wait is also bounded (see
 * msa_debug_layer_spin_limit): a workgroup that gives up marks its results
 * invalid (NaN out and lse, selection -1 when the selection itself gave up)
 * and is counted in the workspace (msa_decode_layer_gave_up).
 * Supported: kv_dtype MSA_KV_NVFP4, idx_dtype MSA_IDX_FP8_E4M3 or
 * MSA_IDX_NVFP4, q_len <= 4, and a stream that is not being captured into a
 * HIP graph (the call's epoch is drawn on the host, and a replayed graph
 * would repeat it); anything else returns MSA_ERR_UNSUPPORTED before
 * anything is enqueued. Workspace: a word counts only when its tag equals the
 * call's epoch (a per-call 32-bit value, never 0). Words the library wrote in
 * earlier calls never match; memory it never wrote matches with probability
 * about 2^-32 per word, so a workspace should be zero-filled once before its
 * first use (the Python binding's alloc_workspace does) -- no clearing is
 * needed between calls. */
msa_status_t msa_decode_layer_single(const msa_params_t* p, const msa_cache_t* cache,
                                     const void* q, const void* idx_q, const float* idx_w,
                                     void* out, float* lse, int32_t* sel_out,
                                     void* workspace, size_t ws_bytes, void* stream);

/* The number of workgroups of the latest msa_decode_layer_single call made
 * on `workspace` by this process that gave up a bounded wait, written to
 * *count (0: the call's results are complete; otherwise the affected rows
 * hold NaN). Reads one word of the workspace with a copy on `stream` and
 * synchronises `stream`. A workspace no single-launch call of this process
 * has used gives 0. p: the parameters the workspace was sized for. */
msa_status_t msa_decode_layer_gave_up(const msa_params_t* p, const void* workspace, size_t ws_bytes,
                                      void* stream, int64_t* count);

/* Bytes of device memory per GPU that msa_decode_layer_single_static uses as
 * its scratch. */
#define MSA_STATIC_SCRATCH_BYTES (32u << 20)

/* msa_decode_layer_single without a workspace, for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * allocation). Its scratch (the tagged pooled scores, selection records and
 * split states) is a fixed array of MSA_STATIC_SCRATCH_BYTES bytes in the
 * library's code object, one per GPU, held until the process ends; the call
 * itself allocates nothing. The caller still passes every input and output;
 * arguments, results and limits are msa_decode_layer_single's. A problem
 * whose scratch would exceed the array (about B * q_len * max_blocks_per_seq
 * * 8 bytes of tagged scores, plus the split items' states) returns
 * MSA_ERR_UNSUPPORTED before anything is enqueued. Every call on a GPU
 * shares that GPU's array: calls that may overlap on one GPU (different
 * streams, threads) race and must be serialised by the caller. The array
 * keeps the last call's words; nothing in it needs clearing, because every
 * word carries the epoch of the call that wrote it (and the array starts
 * zeroed). The give-up count of msa_decode_layer_gave_up is not available
 * for this entry; a give-up still shows as NaN rows and -1 selections. */
msa_status_t msa_decode_layer_single_static(const msa_params_t* p, const msa_cache_t* cache,
                                            const void* q, const void* idx_q, const float* idx_w,
                                            void* out, float* lse, int32_t* sel_out, void* stream);

/* msa_decode_layer_single with a tracing hook: when `events` is not NULL it
 * holds 2 hipEvent_t handles (NULL entries allowed) into which the kernel's
 * dispatch records its start and end (hipExtLaunchKernel). */
msa_status_t msa_decode_layer_single_traced(const msa_params_t* p, const msa_cache_t* cache,
                                            const void* q, const void* idx_q, const float* idx_w,
                                            void* out, float* lse, int32_t* sel_out,
                                            void* workspace, size_t ws_bytes, void* stream,
                                            void* const* events);

/* KV-insert: quantise the q_len new tokens of every sequence and write them
 * into the paged caches -- the step that precedes the decode of those tokens
 * [ainewsbites page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on NVIDIA
 * and AMD GPUs": section "A model built for efficient inference", the model
 * is trained for an NVFP4 KV cache; section "Kernel and serving
 * optimizations", KV-insert is fused with the kernels that produce K and V].
 * Token t of sequence b goes to position pos = ctx_lens[b] - q_len + t
 * (ctx_lens counts the new tokens, as in the decode calls): page
 * block_table[b][pos / 128], slot pos % 128. Nothing else is written; a V
 * byte shared with an older token keeps that token's nibble.
 *   new_k, new_v  device bf16[B][q_len][num_kv_heads][128]
 *   new_idx_k     device bf16[B][q_len][64]
 * NVFP4 K/V, per token, KV head and 16-element group (IEEE double, in this
 * order): y = x / tensor_scale; scale code = E4M3(max|y| / 6); code =
 * E2M1(y / decoded scale), or +0 when the scale is 0. E4M3 and E2M1 round to
 * the nearest value, ties to the even code, saturating at 448 and 6; a value
 * that rounds to zero is stored as +0.
 * FP8 indexer keys, per token: s = max|k| / 448 rounded to fp32 (1.0 when
 * the max is 0); byte = E4M3(k / s) (double quotient), idx_k_scale = s.
 * NVFP4 indexer keys: as NVFP4 K with y = k / idx_k_tensor_scale, per
 * 16-dim group.
 * bf16 caches store the values unchanged.
 * The cache buffers are written through the pointers of msa_cache_t (their
 * const qualifies the decode calls only). Tokens with pos < 0 or pos >=
 * max_blocks_per_seq*128, or whose page is outside [0, num_pages), are
 * skipped. The written slots of different sequences must not share a page
 * slot. NaN and infinite inputs are not supported. */
msa_status_t msa_kv_insert(const msa_params_t* p, const msa_cache_t* cache,
                           const void* new_k, const void* new_v,
                           const void* new_idx_k, void* stream);

/* Debug exports: run the kernels' own dequantisation helpers over a flat
 * buffer, for bit-exact tests of the decoders.
 *   msa_debug_dequant_nvfp4: codes device u8[n_groups*8] (16 elements per
 *   group, even element in the low nibble), scales device u8[n_groups] (E4M3),
 *   out device f32[n_groups*16] = e2m1 * e4m3 (the tensor scale is not
 *   applied; the kernels apply it to the dot products).
 *   msa_debug_dequant_fp8: codes device u8[n], out device f32[n] = e4m3. */
msa_status_t msa_debug_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales,
                                     int64_t n_groups, float* out, void* stream);
msa_status_t msa_debug_dequant_fp8(const uint8_t* codes, int64_t n, float* out,
                                   void* stream);

/* Measurement export: streams `bytes` of device memory at `buf` (16-byte
 * aligned, bytes a multiple of 16) with 16-byte nontemporal loads, 4 KB of
 * contiguous memory per wave and step, 16 waves per compute unit, so that
 * the time of the call on `stream` gives the
 * device's attainable read bandwidth, the ceiling that the decode kernels'
 * rates are read against beside the nominal HBM peak. `out`: 4 bytes of
 * device memory the kernel may write (a checksum of the data; stored only
 * when it equals a fixed value, so that the loads stay and nothing is
 * written in practice). Errors: MSA_ERR_INVALID_ARG for a NULL buffer
 * (bytes > 0), a misaligned buf or a size not a multiple of 16. */
msa_status_t msa_debug_read_bandwidth(const void* buf, int64_t bytes, uint32_t* out, void* stream);

/* Debug export: the number of polls after which a workgroup of
 * msa_decode_layer_single stops waiting for the pooled scores of its query
 * token (default, polls = 0: about a second of polling; with polls = 1 an
 * item gives up as soon as one score of a chunk it reads is not yet
 * published). An item that stops writes NaN to its out rows and lse entries
 * and -1 to its selection; the kernel still ends normally. Applies to later calls in this
 * process; polls < 0 returns MSA_ERR_INVALID_ARG. For tests of the bounded
 * wait. */
msa_status_t msa_debug_layer_spin_limit(int32_t polls);

/* Debug export: the shape of later msa_decode_layer_single calls in this
 * process: 1 = one workgroup per item (fused selection), 2 or 4 = selectors
 * plus that many attention workgroups per item; 0 restores the automatic
 * choice. For measurements and tests of each shape. Other values return
 * MSA_ERR_INVALID_ARG. */
msa_status_t msa_debug_layer_splits(int32_t splits);

/* Human-readable name of a status code (static string). */
const char* msa_status_string(msa_status_t s);
/* Thread-local description of the last failure in this thread ("" if none). */
const char* msa_last_error(void);
/* Library version string. */
const char* msa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H_ */
