/*
 * d2f.h -- C interface of libd2f, the hot path of one D2F (Discrete Diffusion
 * Forcing) denoising step on AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *  [D2F-wiki]    "D2F: 확산 언어 모델이 KV 캐시를 얻고 자기회귀 모델보다 2.5배
 *                빨라지는 방법 (arXiv:2508.09192)", llm-wiki.hwlabs.dev
 *  [D2F-review]  "D2F 논문 리뷰: 확산 LLM이 자기회귀 모델보다 빠른 추론을
 *                처음으로 달성한 방식", allinfo.ai.kr
 *  [dLLM-survey] "확산 언어 모델(Diffusion LLM)이란 무엇인가", discuss.pytorch.kr
 *
 * One step of D2F decoding runs, per layer, attention of the active window's
 * tokens over the frozen KV cache plus the window itself (d2f_block_attn),
 * then one pass over the vocabulary logits of the window positions that
 * decides which positions to commit (d2f_confidence_commit), and, when the
 * oldest window block is complete, moves that block's K/V into the cache
 * (d2f_kv_commit).  Around these: the active-window schedule and the step's
 * bookkeeping that turn them into pipelined multi-step decoding
 * (d2f_window_*, d2f_decode_advance), other confidence measures and Prophet's
 * early commit (d2f_confidence_commit_ex), a paged cache whose persist is a
 * table update (d2f_block_attn_paged, d2f_kv_commit_paged,
 * d2f_decode_advance_paged), and attention in segments with an exact join
 * for outside-block reuse (d2f_block_attn_range, d2f_attn_combine).
 *
 * Conventions shared by every entry point:
 *  - Pointers named *_host are host memory read synchronously during the
 *    call.  All other buffers are device memory owned by the caller; the
 *    library allocates nothing and keeps no state between calls.
 *  - Work is enqueued on `stream` (NULL = the default stream) and is complete
 *    once the stream is synchronised.  Calls on different streams are
 *    independent; calls that share buffers must be ordered by the caller.
 *  - Every entry point returns a d2f_status_t.  On any status other than
 *    D2F_OK and D2F_ERR_HIP nothing was enqueued.  D2F_ERR_HIP reports a
 *    failed launch; d2f_last_error() then holds a message (per thread).
 *  - Results are deterministic for fixed inputs: no floating-point atomics.
 *  - Device buffers must be naturally aligned for their element type; the
 *    fast paths additionally use 16-byte vector accesses when rows allow it.
 */
#ifndef D2F_H
#define D2F_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t (a pointer to the runtime's opaque stream). */
struct ihipStream_t;
typedef struct ihipStream_t* d2f_stream_t;

typedef enum {
  D2F_OK = 0,
  D2F_ERR_INVALID_ARG = 1, /* a size, pointer or enum is out of range          */
  D2F_ERR_CAPACITY = 2,    /* the cache cannot hold the requested tokens       */
  D2F_ERR_ORDER = 3,       /* kv_commit of a block other than the oldest one   */
  D2F_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required       */
  D2F_ERR_HIP = 5,         /* a HIP launch or runtime call failed              */
  D2F_ERR_UNSUPPORTED = 6  /* valid, but not a shape this library handles      */
} d2f_status_t;

typedef enum { D2F_F32 = 0, D2F_BF16 = 1 } d2f_dtype_t;

/* mask_state values (uint8 per window position) */
enum { D2F_MASKED = 0, D2F_COMMITTED = 1 };
/* block_phase values (uint8 per window block) */
enum { D2F_CONSERVATIVE = 0, D2F_AGGRESSIVE = 1 };

/* Geometry of the attention of one layer.
 *  batch           requests in the call (>= 0)
 *  n_heads_q       query heads; n_heads_kv KV heads; n_heads_q % n_heads_kv == 0
 *                  and query head h reads KV head h / (n_heads_q / n_heads_kv)
 *  head_dim        D: 64 or 128 for bf16 (the MFMA path); 32, 64 or 128 for
 *                  f32; other values return D2F_ERR_UNSUPPORTED
 *  block_size      B >= 1, tokens per D2F block
 *  max_win_blocks  window capacity in blocks; Wmax = max_win_blocks * B
 *  cache_capacity  token slots per (request, KV head) in the cache arrays
 *  dtype           element type of q, k_*, v_* and out
 *  softmax_scale   scores are scale * <q, k>; <= 0 selects 1/sqrt(head_dim)
 */
typedef struct {
  int32_t batch;
  int32_t n_heads_q;
  int32_t n_heads_kv;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_win_blocks;
  int64_t cache_capacity;
  d2f_dtype_t dtype;
  float softmax_scale;
} d2f_attn_desc_t;

/* Bytes of device workspace d2f_block_attn and d2f_block_attn_paged need for
 * these lengths (0 when no key range is split), written to *bytes_out: the
 * larger of the two calls' needs, so one size serves both.  Same argument
 * rules as d2f_block_attn.  The size comes back through an out-parameter, with a
 * status as the return value, because 0 is a valid size (no split): a size
 * returned directly could not tell "nothing needed" from "invalid
 * arguments". */
d2f_status_t d2f_block_attn_workspace_size(const d2f_attn_desc_t* desc,
                                           const int32_t* prefix_len_host,
                                           const int32_t* n_win_blocks_host,
                                           size_t* bytes_out);

/* Block-causal attention of the active window over the frozen cache.
 *
 * [D2F-wiki] section "블록 단위 인과 어텐션": the sequence is split into
 * blocks of B tokens; tokens of one block attend to each other in both
 * directions, a block attends only to the blocks before it, and completed
 * blocks' K/V sit unchanged in a KV cache.  [D2F-wiki] "인터블록 병렬
 * 디코딩" and [D2F-review] "쉽게 이해하기": later blocks are decoded while
 * earlier ones are still partly masked, so a window block also attends to
 * every earlier window block.
 *
 * For request b (P = prefix_len_host[b], W = n_win_blocks_host[b] * B), query
 * head h, KV head g = h / (n_heads_q / n_heads_kv) and window row i < W, the
 * keys are the P cached tokens followed by the W window tokens; window key j
 * is visible iff j / B <= i / B (blocks counted from the window start), and
 * every cached key is visible.  out = softmax(scale * q K^T) V over the
 * visible keys; lse = the natural-log normaliser of the same softmax.
 *
 * Layouts (row-major, dtype elements):
 *   q, out          [batch][n_heads_q][Wmax][head_dim]
 *   k_cache,v_cache [batch][n_heads_kv][cache_capacity][head_dim]
 *   k_win, v_win    [batch][n_heads_kv][Wmax][head_dim]
 *   lse             [batch][n_heads_q][Wmax] float, or NULL
 *   prefix_len_host [batch], 0 <= P and P + W <= cache_capacity
 *   n_win_blocks_host [batch], 0 <= n <= max_win_blocks (0: the request is
 *                   idle in this call, e.g. finished, and costs nothing)
 * Rows i >= W of out and lse are left untouched; cache slots >= P and window
 * rows >= W are never read.  workspace: >= d2f_block_attn_workspace_size
 * bytes of device memory, 256-byte aligned (may be NULL when that is 0).
 * Errors: D2F_ERR_INVALID_ARG (bad sizes, null required pointers, group
 * mismatch), D2F_ERR_CAPACITY (P + W > cache_capacity), D2F_ERR_WORKSPACE,
 * D2F_ERR_UNSUPPORTED (head_dim/dtype pair not built), D2F_ERR_HIP.
 */
d2f_status_t d2f_block_attn(const d2f_attn_desc_t* desc, const void* q, const void* k_cache,
                            const void* v_cache, const void* k_win, const void* v_win,
                            const int32_t* prefix_len_host, const int32_t* n_win_blocks_host,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            d2f_stream_t stream);

/* Append the oldest window block of one request to the KV cache.
 *
 * [D2F-wiki] section "블록 단위 인과 어텐션": a completed block's K/V do not
 * change any more, so an ordinary KV cache holds them exactly; section
 * "KV 캐시 관리 방식": the completion of a block is the signal to make its
 * cache entries permanent.
 *
 * For every layer l < n_layers and KV head g: rows [0, B) of window block 0
 *   k_win + l*win_layer_stride  [batch][n_heads_kv][Wmax][head_dim]
 * are copied bit for bit to cache slots [P, P + B) of
 *   k_cache + l*cache_layer_stride  [batch][n_heads_kv][cache_capacity][head_dim]
 * (likewise V), for request `request`, where P = prefix_len_host[request].
 * Strides are in elements.  Then prefix_len_host[request] += B on the host,
 * and, when prefix_len_dev is not NULL, prefix_len_dev[request] is set to the
 * new value on `stream`.  The window itself is not modified: dropping the
 * block from the window is the caller's bookkeeping.  The caller guarantees
 * the block is complete (every position committed) and that its K/V were
 * computed from the committed tokens.
 * Errors: D2F_ERR_ORDER (block != 0: only the oldest window block may join
 * the cache, which keeps the cache one contiguous prefix), D2F_ERR_CAPACITY
 * (P + B > cache_capacity), D2F_ERR_INVALID_ARG, D2F_ERR_HIP.
 */
d2f_status_t d2f_kv_commit(const d2f_attn_desc_t* desc, int32_t n_layers, void* k_cache,
                           void* v_cache, int64_t cache_layer_stride, const void* k_win,
                           const void* v_win, int64_t win_layer_stride, int32_t request,
                           int32_t block, int32_t* prefix_len_host, int32_t* prefix_len_dev,
                           d2f_stream_t stream);

/* ---- Attention in segments: outside-block reuse ----
 *
 * [dLLM-survey] section "FlashBlock: 블록 외부 어텐션 캐싱": the attention of a
 * block's queries over the keys outside the block can be cached across steps
 * (its output and normaliser, a tensor that scales with the block, not the
 * context) and joined each step with a freshly computed inside part by
 * log-space composition; when too many tokens changed since it was cached it
 * is recomputed instead.  In D2F the window's queries change every step, so
 * reusing a cached outside part is an approximation; the composition itself
 * is exact.
 *
 * d2f_block_attn_range: for request b, the window's query rows i < W_b attend
 * to the cache keys [key_lo_host[b], key_hi_host[b]) only (all of them
 * visible, no window keys).  Layouts, out, lse, scale and errors as
 * d2f_block_attn; the cache arrays must hold key_hi_host[b] rows
 * (D2F_ERR_CAPACITY otherwise); a request with an empty range or no window is
 * idle (its rows untouched).  The window-only part is d2f_block_attn with
 * prefix_len 0.  Workspace: d2f_block_attn_range_workspace_size.
 */
d2f_status_t d2f_block_attn_range_workspace_size(const d2f_attn_desc_t* desc,
                                                 const int32_t* key_lo_host,
                                                 const int32_t* key_hi_host,
                                                 const int32_t* n_win_blocks_host,
                                                 size_t* bytes_out);
d2f_status_t d2f_block_attn_range(const d2f_attn_desc_t* desc, const void* q,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* key_lo_host, const int32_t* key_hi_host,
                                  const int32_t* n_win_blocks_host, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, d2f_stream_t stream);

/* Join two attention results of the same query rows over disjoint key sets:
 * per row i < W_b of request b, L = ln(e^L_a + e^L_b) and
 * O = O_a e^(L_a - L) + O_b e^(L_b - L) (a side with L = -inf weighs 0).
 * out_* and out are [batch][n_heads_q][Wmax][head_dim] in desc's dtype,
 * lse_* and lse [batch][n_heads_q][Wmax] float; out / lse may alias out_a /
 * lse_a or out_b / lse_b; rows i >= W_b are untouched.  Errors:
 * D2F_ERR_INVALID_ARG, D2F_ERR_UNSUPPORTED (head_dim / dtype not built),
 * D2F_ERR_HIP. */
d2f_status_t d2f_attn_combine(const d2f_attn_desc_t* desc, const void* out_a, const float* lse_a,
                              const void* out_b, const float* lse_b, void* out, float* lse,
                              const int32_t* n_win_blocks_host, d2f_stream_t stream);

/* ---- Paged KV cache: block completion as the persist signal ----
 *
 * [D2F-wiki] section "운영 관점" (KV cache management): completed blocks are
 * cached permanently; a paged cache (as in PagedAttention) can be used with
 * the completion of a block as the signal that makes its entries permanent.
 * [D2F-wiki] section "블록 단위 인과 어텐션": a completed block's K/V no
 * longer change.
 *
 * A page holds the K (or V) rows of one D2F block for every KV head of one
 * layer: pools k_pages, v_pages are [n_pages][n_heads_kv][block_size][head_dim]
 * (dtype elements; one pool per layer, page ids shared by all layers).
 * Request b's cached keys are the pages page_table[b][0 .. P/B) in order
 * (page_table: device int32 [batch][table_stride]); its window block k is
 * page win_pages[b][k] (device int32 [batch][max_win_blocks]).  The model
 * writes a window block's K/V into that block's page, so when the oldest
 * window block completes, d2f_kv_commit_paged moves its page id into the page
 * table: nothing is copied.  Pages are owned and handed out by the caller.
 *
 * d2f_block_attn_paged computes exactly what d2f_block_attn computes for the
 * same keys, with q, out, lse laid out as there.  It uses the same kernels and
 * work plan, so the results are bit-identical, with one exception: a call
 * whose keys are cut into few long ranges (a long prefix over few heads),
 * which d2f_block_attn re-plans for one eight-wave workgroup per CU, keeps the
 * four-wave plan here; its ranges then differ, and so do the results, by
 * rounding.  Requirements: bf16, head_dim 64 or 128,
 * block_size a power of two >= 8 (D2F_ERR_UNSUPPORTED otherwise); every
 * prefix_len_host[b] a multiple of block_size (D2F_ERR_INVALID_ARG; the
 * cache holds whole blocks) with P/B <= table_stride (D2F_ERR_CAPACITY);
 * 0 <= n_win_blocks_host[b] <= max_win_blocks.  desc->cache_capacity is not
 * used.  The workspace is the one d2f_block_attn_workspace_size gives for the
 * same lengths (with a desc whose cache_capacity covers P + W).  Page ids
 * read outside [0, n_pages) are clamped into the pool (the results are then
 * meaningless, but nothing outside the pool is read).
 */
d2f_status_t d2f_block_attn_paged(const d2f_attn_desc_t* desc, const void* q,
                                  const void* k_pages, const void* v_pages, int32_t n_pages,
                                  const int32_t* page_table, int32_t table_stride,
                                  const int32_t* win_pages, const int32_t* prefix_len_host,
                                  const int32_t* n_win_blocks_host, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, d2f_stream_t stream);

/* Persist the oldest window block of `request` in the paged cache: on
 * `stream`, page_table[request][P/B] = win_pages[request][0], the window's page
 * list moves up by one (its last entry becomes -1; the caller puts a free page
 * there before a block is appended), and prefix_len_dev[request] = P + B when
 * prefix_len_dev is not NULL; prefix_len_host[request] += B on return.
 * Errors: D2F_ERR_INVALID_ARG (request out of range, P not a multiple of B,
 * NULL pointers), D2F_ERR_CAPACITY (P/B >= table_stride), D2F_ERR_HIP. */
d2f_status_t d2f_kv_commit_paged(const d2f_attn_desc_t* desc, int32_t* page_table,
                                 int32_t table_stride, int32_t* win_pages, int32_t request,
                                 int32_t* prefix_len_host, int32_t* prefix_len_dev,
                                 d2f_stream_t stream);

/* Bytes of device workspace d2f_confidence_commit and d2f_confidence_commit_ex
 * need (16-byte aligned; its contents need no initialisation), written to
 * *bytes_out; the status reports invalid sizes (as for
 * d2f_block_attn_workspace_size). */
d2f_status_t d2f_confidence_commit_workspace_size(int32_t n_rows, int32_t vocab,
                                                  size_t* bytes_out);

/* Confidence, argmax and the commit/remask decision over the window.
 *
 * [D2F-review] section "쉽게 이해하기": a block newly added to the window is
 * conservative and commits only positions whose confidence exceeds the
 * threshold; a block whose predecessor has progressed far enough is
 * aggressive and commits the relatively most confident positions even if
 * they are not very confident; positions not committed are masked again.
 * [dLLM-survey] sections "양방향 어텐션과 사라진 KV 캐시" (low-confidence
 * remasking) and "답을 미리 안다: 조기 확정 디코딩(Prophet)" (the maximum
 * softmax probability as the confidence).
 *
 * Row p of `logits` (float, row stride ld >= vocab elements) holds window
 * position p; rows of all requests are concatenated block by block, so
 * n_rows = n_blocks * block_size.  For each row with mask_state == MASKED:
 *   conf = max_j softmax(logits[p])_j, argmax = the smallest j reaching the max.
 * Rows already COMMITTED are not read and not changed.  For block k
 * (rows [k*B, (k+1)*B)), with the float threshold tau:
 *   CONSERVATIVE: commit p iff conf_p > tau;
 *   AGGRESSIVE:   commit p iff conf_p > tau, or p is among the k_aggr most
 *                 confident MASKED rows of the block (ties: lower p first).
 * A committed row gets mask_state = COMMITTED and tokens = argmax; a MASKED
 * row that is not committed gets tokens = mask_token_id (remask).
 * n_committed[k] = rows committed by this call; block_complete[k] = 1 iff
 * every row of block k is COMMITTED afterwards.  conf_out / argmax_out
 * (optional, NULL allowed) receive conf and argmax of the rows that were
 * MASKED on entry; other rows are untouched.
 * Buffers: mask_state uint8 [n_rows] and tokens int32 [n_rows] in/out;
 * block_phase uint8 [n_blocks]; n_committed int32 [n_blocks] and
 * block_complete uint8 [n_blocks] out.  Logits must be finite.
 * Errors: D2F_ERR_INVALID_ARG (n_rows % block_size != 0, vocab < 1,
 * ld < vocab, null required pointers, k_aggr < 0), D2F_ERR_WORKSPACE,
 * D2F_ERR_HIP.
 */
d2f_status_t d2f_confidence_commit(const float* logits, int64_t ld, int32_t n_rows,
                                   int32_t vocab, uint8_t* mask_state, int32_t* tokens,
                                   const uint8_t* block_phase, int32_t block_size, float tau,
                                   int32_t k_aggr, int32_t mask_token_id, float* conf_out,
                                   int32_t* argmax_out, int32_t* n_committed,
                                   uint8_t* block_complete, void* workspace,
                                   size_t workspace_bytes, d2f_stream_t stream);

/* d2f_confidence_commit without a workspace argument, for callers that cannot
 * allocate device memory: code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus the workspace),
 * semantics, outputs and errors as d2f_confidence_commit, computed by the
 * same kernels.  The per-(row, vocabulary chunk) partials go to a scratch
 * array of D2F_NOALLOC_SCRATCH_BYTES that the library holds on every device
 * it runs on until the process ends; nothing is allocated per call.
 * Limit: d2f_confidence_commit_workspace_size(n_rows, vocab) must not exceed
 * D2F_NOALLOC_SCRATCH_BYTES (8 MiB: e.g. 16384 rows at a vocabulary of up to
 * 262144), else D2F_ERR_WORKSPACE and nothing is launched.  Every call on a
 * device shares that device's array: calls that overlap on one device (on
 * two streams, or from two host threads without ordering) race and give
 * undefined results.  The array is used on the device of `stream` (the
 * current device for the NULL stream); its address is looked up on the first
 * call on each device. */
#define D2F_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
d2f_status_t d2f_confidence_commit_noalloc(const float* logits, int64_t ld, int32_t n_rows,
                                           int32_t vocab, uint8_t* mask_state, int32_t* tokens,
                                           const uint8_t* block_phase, int32_t block_size,
                                           float tau, int32_t k_aggr, int32_t mask_token_id,
                                           float* conf_out, int32_t* argmax_out,
                                           int32_t* n_committed, uint8_t* block_complete,
                                           d2f_stream_t stream);

/* ---- Other confidence measures and Prophet's early commit ----
 *
 * [dLLM-survey] section "신뢰도를 넘어서: 궤적 일관성 디코딩(CCD)": decoders
 * choose positions by the local confidence or by the negative entropy of the
 * predicted distribution; section "토큰 순서의 이론": the top-probability
 * order (LLaDA's default) and the top-probability margin order, Dream using
 * the negative entropy; section "답을 미리 안다: 조기 확정 디코딩(Prophet)":
 * the confidence gap between the two largest logits, and once it passes a
 * threshold (lowered 7.5, 5.0, 2.5 as decoding progresses) every remaining
 * mask is filled with its argmax.
 *
 * With p = softmax(row) and l(1) >= l(2) the two largest logits (a repeated
 * maximum counts twice):
 *   D2F_CONF_MAXPROB      conf = max_j p_j                (d2f_confidence_commit)
 *   D2F_CONF_MARGIN       conf = p(1) - p(2)
 *   D2F_CONF_NEG_ENTROPY  conf = sum_j p_j ln p_j  (<= 0)
 *   D2F_CONF_LOGIT_GAP    conf = l(1) - l(2)  (+inf for a one-entry row)
 * Every measure reads each MASKED row once, as the maximum probability does.
 */
typedef enum {
  D2F_CONF_MAXPROB = 0,
  D2F_CONF_MARGIN = 1,
  D2F_CONF_NEG_ENTROPY = 2,
  D2F_CONF_LOGIT_GAP = 3
} d2f_conf_measure_t;

/* d2f_confidence_commit with a chosen measure (same block rule, buffers and
 * errors; conf_out receives the measure) and, optionally, Prophet's early
 * commit: early_gap (device, float [n_groups], or NULL for none) holds one
 * threshold per group of early_group_blocks consecutive blocks (0: all blocks
 * form one group; n_groups = ceil(n_blocks / group)).  After the block rule,
 * a group whose smallest logit gap over the rows that were MASKED on entry is
 * strictly above its threshold has every still-MASKED row committed with its
 * argmax (n_committed includes them; block_complete becomes 1).  The early
 * commit reads the logit gap under any measure except D2F_CONF_NEG_ENTROPY
 * (D2F_ERR_INVALID_ARG).  Errors as d2f_confidence_commit, plus
 * D2F_ERR_INVALID_ARG for an unknown measure or early_group_blocks < 0. */
d2f_status_t d2f_confidence_commit_ex(const float* logits, int64_t ld, int32_t n_rows,
                                      int32_t vocab, uint8_t* mask_state, int32_t* tokens,
                                      const uint8_t* block_phase, int32_t block_size,
                                      d2f_conf_measure_t measure, float tau, int32_t k_aggr,
                                      int32_t mask_token_id, const float* early_gap,
                                      int32_t early_group_blocks, float* conf_out,
                                      int32_t* argmax_out, int32_t* n_committed,
                                      uint8_t* block_complete, void* workspace,
                                      size_t workspace_bytes, d2f_stream_t stream);

/* Prophet's threshold for a decoding progress in [0, 1] (clamped): 7.5 below
 * 1/3, 5.0 below 2/3, 2.5 from there on (the pages give the three values,
 * not where they change; thirds are this library's reading).  Host only. */
float d2f_prophet_threshold(float progress);

/* ---- Active-window schedule (host only; no device memory, no stream) ----
 *
 * [D2F-review] sections "핵심 메시지" (last point) and "쉽게 이해하기"
 * (inference paragraph): decoding keeps a window of active blocks; once the
 * progress of the last block passes a threshold a new, fully masked block is
 * added behind it; a new block starts conservative and turns aggressive once
 * the block before it has progressed far enough.  [D2F-wiki] section "운영
 * 관점" (KV cache management): a completed block is persisted to the cache.
 *
 * Rules of this implementation (the pages give no numbers or tie rules):
 * progress = committed positions / block_size; a threshold is passed when
 * committed > tau * block_size (strict, in double precision of the float tau).
 * After each commit pass (d2f_window_after_commit):
 *   1. n_committed[k] (positions committed by the pass in window block k) is
 *      added to the block's count;
 *   2. while the oldest window block is complete it is persisted (the caller
 *      then calls d2f_kv_commit for it, oldest first) and leaves the window;
 *   3. if fewer than total_blocks blocks were started and the window holds
 *      fewer than max_win_blocks blocks, one new block is appended when the
 *      window is empty or its last block's progress passes tau_add;
 *   4. phases for the next pass: the oldest block is AGGRESSIVE; block k > 0
 *      becomes AGGRESSIVE when block k - 1's progress passes tau_act; a block
 *      never returns to CONSERVATIVE.
 * d2f_window_init starts the first block (AGGRESSIVE: it is the oldest).
 * The state is a plain struct owned by the caller; window block k is absolute
 * block first + k.  Errors: D2F_ERR_INVALID_ARG (block_size < 1, max_win_blocks
 * outside 1..D2F_MAX_WINDOW, total_blocks < 1, NaN thresholds, a count that
 * would exceed block_size or is negative, a call after every block was
 * persisted).  On error the state is left unchanged. */
#define D2F_MAX_WINDOW 64

typedef struct {
  int32_t block_size;      /* positions per block */
  int32_t max_win_blocks;  /* most blocks in the window at once (1..D2F_MAX_WINDOW) */
  int32_t total_blocks;    /* blocks to decode */
  float tau_add;           /* append a block once the last one's progress passes this */
  float tau_act;           /* a block turns aggressive once its predecessor passes this */
} d2f_window_params_t;

typedef struct {
  int32_t first;       /* absolute index of the oldest window block */
  int32_t n_win;       /* blocks in the window */
  int32_t started;     /* blocks started so far */
  int32_t persisted;   /* blocks persisted so far (== total_blocks when done) */
  int32_t committed[D2F_MAX_WINDOW];  /* committed positions per window block */
  uint8_t phase[D2F_MAX_WINDOW];      /* D2F_CONSERVATIVE / D2F_AGGRESSIVE per window block */
} d2f_window_t;

d2f_status_t d2f_window_init(const d2f_window_params_t* params, d2f_window_t* state);

/* Apply one commit pass; *persisted_out = blocks persisted by step 2 (the
 * caller appends their K/V oldest first), *appended_out = 0 or 1. */
d2f_status_t d2f_window_after_commit(const d2f_window_params_t* params, d2f_window_t* state,
                                     const int32_t* n_committed, int32_t* persisted_out,
                                     int32_t* appended_out);

/* ---- One decoding step's bookkeeping after the commit pass ----
 *
 * [D2F-review] section "쉽게 이해하기" (inference paragraph): the window of
 * active blocks moves forward while later blocks are already being decoded.
 * [D2F-wiki] section "운영 관점" (KV cache management): a block's completion
 * is the signal to make its K/V permanent cache entries.
 *
 * Slot layout of the window state on the device: request b owns rows
 * [b * Wmax, (b + 1) * Wmax) of mask_state (uint8) and tokens (int32), and
 * window blocks [b * max_win_blocks, (b + 1) * max_win_blocks) of block_phase
 * (uint8) and n_committed (int32).  The commit pass runs over all
 * batch * Wmax rows; rows past a request's window are COMMITTED, so their
 * logits are never read.  Before the first step the caller sets rows
 * [0, block_size) of every slot MASKED and the rest COMMITTED, block_phase
 * slot 0 AGGRESSIVE and the rest CONSERVATIVE, and calls d2f_window_init for
 * every request.
 *
 * d2f_decode_advance, once per step after d2f_confidence_commit:
 *   1. copies n_committed to the host and synchronises `stream` (the step's
 *      one device-to-host transfer);
 *   2. applies d2f_window_after_commit to every request's window (requests
 *      whose blocks are all persisted are skipped);
 *   3. enqueues one launch per 64 requests that, for each request with p
 *      persisted blocks: appends window rows [0, p * block_size) of k_win /
 *      v_win of every layer to cache slots [P, P + p * block_size) (byte copy,
 *      as d2f_kv_commit); copies their tokens to
 *      out_tokens[b][first * block_size ...] (out_tokens is
 *      [batch][total_blocks * block_size] int32, the decoded sequence); moves
 *      the remaining window rows of mask_state / tokens to the front of the
 *      slot; sets an appended block's rows MASKED with tokens = mask_token_id
 *      and rows past the window COMMITTED; writes every block_phase slot of
 *      the request (past the window: CONSERVATIVE); stores P + p * block_size
 *      into prefix_len_dev[b] when prefix_len_dev is not NULL;
 *   4. updates windows_host, prefix_len_host, persisted_host[b] and
 *      appended_host[b] (int32 [batch] each).
 * k_win / v_win are read, not moved: the next model pass writes the window's
 * K/V for the new layout.  desc and the layer strides are as for
 * d2f_kv_commit; params must agree with desc on block_size and
 * max_win_blocks.
 * Errors: D2F_ERR_INVALID_ARG (as for d2f_kv_commit and
 * d2f_window_after_commit, mismatched params, an inconsistent window state),
 * D2F_ERR_CAPACITY (a persisted block does not fit the cache): the host state
 * is unchanged and nothing was enqueued.  D2F_ERR_HIP: the transfer or a
 * launch failed; the host state is unchanged, device buffers may be partly
 * updated when batch > 64. */
d2f_status_t d2f_decode_advance(const d2f_attn_desc_t* desc, int32_t n_layers, void* k_cache,
                                void* v_cache, int64_t cache_layer_stride, const void* k_win,
                                const void* v_win, int64_t win_layer_stride,
                                const d2f_window_params_t* params, d2f_window_t* windows_host,
                                int32_t* prefix_len_host, int32_t* prefix_len_dev,
                                const int32_t* n_committed, uint8_t* mask_state, int32_t* tokens,
                                uint8_t* block_phase, int32_t* out_tokens, int32_t mask_token_id,
                                int32_t* persisted_host, int32_t* appended_host,
                                d2f_stream_t stream);

/* d2f_decode_advance for a paged cache (see d2f_block_attn_paged): the
 * persisted blocks' pages join page_table[b] in order (no K/V is copied), the
 * window's page list win_pages[b] moves up, a block appended to request b's
 * window takes page new_pages_host[b] (host int32 [batch]; read only for
 * requests that append, which then must hold a page id >= 0), and slots past
 * the window hold -1.  Everything else (schedule, slot rows, decoded tokens,
 * prefix lengths, errors) is as d2f_decode_advance; prefix lengths must be
 * whole blocks, and P/B + persisted <= table_stride (D2F_ERR_CAPACITY).  The
 * caller knows which new pages were taken from appended_host. */
d2f_status_t d2f_decode_advance_paged(const d2f_attn_desc_t* desc, int32_t* page_table,
                                      int32_t table_stride, int32_t* win_pages,
                                      const int32_t* new_pages_host,
                                      const d2f_window_params_t* params,
                                      d2f_window_t* windows_host, int32_t* prefix_len_host,
                                      int32_t* prefix_len_dev, const int32_t* n_committed,
                                      uint8_t* mask_state, int32_t* tokens, uint8_t* block_phase,
                                      int32_t* out_tokens, int32_t mask_token_id,
                                      int32_t* persisted_host, int32_t* appended_host,
                                      d2f_stream_t stream);

/* Static text for a status code. */
const char* d2f_status_string(d2f_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* d2f_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t d2f_version(void);

#ifdef __cplusplus
}
#endif

#endif /* D2F_H */
