// Internal declarations shared by the libd2f translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "d2f.h"

namespace d2f {

// Attention work decomposition.  A work unit is one workgroup: one request,
// one KV head, one tile of kQTile query rows and one contiguous range of keys
// (a "split").  Query rows of a KV head are the (window position, head in the
// group) pairs, flattened position-major: row r <-> i = r / group,
// head = kv_head * group + r % group, so one tile covers a contiguous run of
// window positions, hence of D2F blocks.
constexpr int kQTile = 64;   // query rows per workgroup
constexpr int kKTile = 64;   // keys per K/V tile
constexpr int kMaxReqPerLaunch = 64;
constexpr int kAttnThreads = 256;
constexpr int kGqaThreads = 512;   // grouped-query kernel (attn_gqa.hip): 8 waves
constexpr int kGqaMaxRows = 256;   // its query rows per unit: 16 per block, <= 2 blocks per wave

struct ReqInfo {
  int32_t b;          // batch index of the request
  int32_t prefix;     // P: cached tokens
  int32_t win;        // W: window tokens (n_win_blocks * block_size)
  int32_t qtiles;     // ceil(group * W / qrows)
  int32_t nsplit;     // key-range splits per query tile (1 = final outputs)
  int32_t unit_base;  // first work unit of this request within the launch
  int32_t group_base; // first (kv_head, qtile) merge group within the launch
  int32_t key_off;    // key-range calls: first cache key of the range (else 0)
};

struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const void* kw;
  const void* vw;
  void* out;
  float* lse;
  float* ws_o;   // [unit][slot_rows][D] unnormalised partial outputs
  float* ws_ml;  // [unit][slot_rows][2] running max (log2 units) and sum
  int64_t cap;   // cache slots per (request, KV head)
  int32_t hq, hkv, group, wmax, bsz;
  int32_t n_req, n_units, n_groups;
  int32_t remap;  // 1: keep a request's query tiles on one XCD (xcd_remap)
  int32_t qrows;  // query rows per unit: kQTile, 32 (bf16, narrow windows) or the GQA kernel's
  int32_t slot_rows;  // partial-result rows per unit in the workspace (>= qrows)
  int32_t cache_only;  // key-range calls: the keys are cache rows [key_off, key_off + prefix)
  int32_t wide;   // bf16: 1 = eight-wave workgroups, two tile groups
  float c2;       // softmax scale * log2(e)
  // Paged K/V (bf16 only): kc/vc are page pools [n_pages][hkv][bsz][D];
  // cache key p of request b is row p % bsz of page page_table[b][p / bsz],
  // window key w is row w % bsz of page win_pages[b][w / bsz].
  const int32_t* page_table;  // [batch][table_stride]
  const int32_t* win_pages;   // [batch][wmax / bsz]
  int32_t table_stride;
  int32_t n_pages;
  int32_t page_shift;  // bsz = 1 << page_shift (paged only)
  ReqInfo req[kMaxReqPerLaunch];
};

// Locate the request of a work unit (unit_base is increasing).
__device__ __forceinline__ int find_req(const AttnArgs& a, int u) {
  int lo = 0, hi = a.n_req - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a.req[mid].unit_base <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int find_req_group(const AttnArgs& a, int g) {
  int lo = 0, hi = a.n_req - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a.req[mid].group_base <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Visible-key end of query tile qt (qrows rows per tile): the last row's
// window block bounds it.
__device__ __forceinline__ int tile_key_end(int qt, int qrows, int P, int W, int G, int B) {
  const int r_last = min((qt + 1) * qrows, G * W) - 1;
  return P + min(W, ((r_last / G) / B + 1) * B);
}
// Key-range calls see no window keys: every row's keys end at P.
__device__ __forceinline__ int unit_key_end(const AttnArgs& a, int qt, int qrows, int P, int W,
                                            int G, int B) {
  return a.cache_only ? P : tile_key_end(qt, qrows, P, W, G, B);
}

// Key tiles of a query tile.  The cache [0, P) and the visible part of the
// window [P, k_end) are tiled separately, so a tile never mixes cache and
// window rows and has one base pointer per tensor; the last tile of each part
// may be partial (nvalid < kKTile).
__device__ __forceinline__ int cache_tiles(int P) { return (P + kKTile - 1) / kKTile; }
__device__ __forceinline__ int window_tiles(int P, int k_end) {
  return (k_end - P + kKTile - 1) / kKTile;
}
__device__ __forceinline__ void tile_span(int t, int nct, int P, int k_end, int& lo, int& nvalid) {
  if (t < nct) {
    lo = t * kKTile;
    nvalid = min(kKTile, P - lo);
  } else {
    lo = P + (t - nct) * kKTile;
    nvalid = min(kKTile, k_end - lo);
  }
}
// Tiles [t_lo, t_hi) of split s: nt tiles divided as evenly as possible.
__device__ __forceinline__ void split_tiles(int nt, int s, int nsplit, int& t_lo, int& t_hi) {
  t_lo = s * nt / nsplit;
  t_hi = (s + 1) * nt / nsplit;
}

// Workgroups are dealt round-robin over the 8 XCDs (workgroup x runs on XCD
// x % 8).  Renumber so that each XCD receives a contiguous run of logical
// units: neighbouring units (the query tiles of one KV range) then share that
// XCD's L2.
__device__ __forceinline__ int xcd_remap(int x, int n) {
  const int q = n >> 3, r = n & 7, k = x & 7, j = x >> 3;
  return (k < r) ? k * (q + 1) + j : r * (q + 1) + (k - r) * q + j;
}

// Launchers (each returns hipSuccess or the launch error).
hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool paged, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, hipStream_t s);
hipError_t launch_attn_gqa(const AttnArgs& a, int head_dim, bool paged, hipStream_t s);
// Attention workgroups that fit on one CU at once (0 if unknown).
int attn_bf16_wgs_per_cu(int head_dim);
int attn_f32_wgs_per_cu(int head_dim);
hipError_t launch_attn_merge(const AttnArgs& a, int head_dim, d2f_dtype_t dt, hipStream_t s);

// Log-space composition of two attention results (combine.hip).
struct CombineArgs {
  const void* out_a;
  const float* lse_a;
  const void* out_b;
  const float* lse_b;
  void* out;
  float* lse;
  int32_t hq, wmax, b0, n_req;
  int32_t win[kMaxReqPerLaunch];  // query rows of each request of the launch
};
hipError_t launch_combine(const CombineArgs& a, int head_dim, d2f_dtype_t dt, hipStream_t s);

struct CommitArgs {
  const float* logits;
  int64_t ld;
  int32_t n_rows, vocab, n_chunks, chunk, block_size, k_aggr, mask_token_id;
  float tau;
  uint8_t* mask_state;
  int32_t* tokens;
  const uint8_t* block_phase;
  float* conf_out;
  int32_t* argmax_out;
  int32_t* n_committed;
  uint8_t* block_complete;
  float4* partial;  // [row][chunk] = {max, sum, argmax bits, aux}
  int32_t measure;       // d2f_conf_measure_t
  int32_t group_blocks;  // blocks per early-commit group
  int32_t n_groups;
  const float* early_gap;  // [n_groups] thresholds, or nullptr: no early commit
  int32_t* ws_argmax;      // [n_rows], early commit only
  uint32_t* ws_gmin;       // [n_groups] bits of the smallest logit gap, early commit only
};
// Per-chunk auxiliary accumulator of the vocabulary pass.
enum { kAuxNone = 0, kAuxSecond = 1, kAuxXlogx = 2 };
constexpr int kCommitThreads = 256;
constexpr int kCommitChunk = 8192;     // logits per workgroup (32 KiB)
constexpr int kMaxCommitBlock = 1024;  // rows per D2F block handled by one workgroup
hipError_t launch_confidence_commit(const CommitArgs& a, bool vec4, hipStream_t s);

// Record a printf-style message as the calling thread's last error (read by
// d2f_last_error) and return st.
d2f_status_t fail(d2f_status_t st, const char* fmt, ...);
d2f_status_t hip_fail(hipError_t e, const char* what);
d2f_status_t check_desc(const d2f_attn_desc_t* d);

struct KvArgs {
  void* kc;
  void* vc;
  const void* kw;
  const void* vw;
  int64_t cache_layer_stride, win_layer_stride;  // elements
  int64_t cap;
  int32_t n_layers, hkv, wmax, head_dim, bsz, esize, request, prefix, new_prefix;
  int32_t* prefix_dev;
};
hipError_t launch_kv_commit(const KvArgs& a, hipStream_t s);
hipError_t launch_kv_commit_paged(int32_t* table, int32_t* win, int32_t* prefix_dev, int b,
                                  int ts, int mw, int slot, int new_prefix, hipStream_t s);

// One decoding step's bookkeeping after the commit pass, for up to
// kMaxReqPerLaunch requests (decode.hip).
struct AdvReq {
  uint64_t phase_bits;  // phase of window blocks 0..n_win_new-1 for the next pass
  int32_t persisted;    // blocks leaving the window (appended to the cache)
  int32_t prefix;       // cache length before the append
  int32_t first;        // absolute index of the oldest window block before
  int32_t n_win_old;    // window blocks before
  int32_t n_win_new;    // window blocks after (persists and the append applied)
  int32_t copy_base;    // first KV-copy workgroup of this request
  int32_t new_page;     // paged: page of an appended block
  int32_t pad;
};
struct AdvArgs {
  void* kc;
  void* vc;
  const void* kw;
  const void* vw;
  int64_t cache_layer_stride, win_layer_stride;  // elements
  int64_t cap;
  uint8_t* mask_state;
  int32_t* tokens;
  uint8_t* block_phase;
  int32_t* out_tokens;
  int32_t* prefix_dev;
  int32_t n_layers, hkv, head_dim, bsz, esize, wmax, max_win, total_blocks;
  int32_t n_req, req0, n_copy_wgs, mask_token_id;
  int32_t* page_table;  // paged: [batch][table_stride]; nullptr for contiguous caches
  int32_t* win_pages;   // paged: [batch][max_win]
  int32_t table_stride;
  AdvReq req[kMaxReqPerLaunch];
};
hipError_t launch_decode_advance(const AdvArgs& a, hipStream_t s);

}  // namespace d2f
