// C entry points of libd2f: argument checks, work planning and launches.
// The operations themselves are documented in include/d2f.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "d2f_internal.h"

namespace d2f {

thread_local std::string g_last_error;

d2f_status_t fail(d2f_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

d2f_status_t hip_fail(hipError_t e, const char* what) {
  return fail(D2F_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

namespace {

// Work-unit sizing.  The key tiles of a (request, KV head, query tile) group
// may be cut into nsplit key ranges, one workgroup each, at the price of a
// merge pass over fp32 partial results.  A split only pays when a request's
// units would run much longer than the average load of a workgroup slot
// (a long prefix among short ones, or too few groups to occupy the device).
// With C = total key tiles / (kSlotFill x resident workgroups), a request is
// split, into ceil(tiles / C) ranges, only if its longest query tile has more
// than kSplitFactor x C tiles.  Units never get shorter than kMinChunkTiles
// tiles.  (Measured on MI355X, bf16 head_dim 128: with 512 or more groups any
// split was slower; with 32 groups, 256 to 512 units were within 3% of the
// best for a 32K prefix.  A workgroup keeps one key tile in flight, so a
// launch with few groups is bound by load latency, about 1.5 us per tile:
// with 32 heads and a 512- or 1024-token prefix, chunks of 3 tiles took 11%
// and 18% off, with 8 heads and 2048 tokens 25%; 1-2 tile chunks lost the
// gain to the merge.)
constexpr int kMinChunkTiles = 3;
constexpr double kSlotFill = 0.75;
constexpr long long kSplitFactor = 2;
constexpr int kDefaultCUs = 256;        // MI355X, used when no device is visible
constexpr int kDefaultWgsPerCU = 2;
constexpr long long kWideSplitMinTiles = 32;   // see plan_attention
constexpr long long kWideSplitMaxTiles = 128;

// Workgroups of the attention kernel resident at once on the current device.
long long resident_workgroups(d2f_dtype_t dt, int head_dim) {
  static std::atomic<int> cache[2][3];  // [dtype][head_dim 32/64/128] = resident WGs + 1
  const int di = dt == D2F_BF16 ? 1 : 0;
  const int hi = head_dim == 32 ? 0 : head_dim == 64 ? 1 : 2;
  int v = cache[di][hi].load(std::memory_order_relaxed);
  if (v > 0) return v - 1;
  int dev = 0, cus = 0;
  int per_cu = dt == D2F_BF16 ? attn_bf16_wgs_per_cu(head_dim) : attn_f32_wgs_per_cu(head_dim);
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();  // no device visible: keep the MI355X defaults
    cus = kDefaultCUs;
    per_cu = kDefaultWgsPerCU;
  }
  v = cus * per_cu;
  cache[di][hi].store(v + 1, std::memory_order_relaxed);
  return v;
}

// Compute units of the current device (the MI355X count when none is visible).
long long device_cus() {
  static std::atomic<int> cache{0};  // CUs + 1 once known
  int v = cache.load(std::memory_order_relaxed);
  if (v > 0) return v - 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();  // no device visible: keep the MI355X default
    cus = kDefaultCUs;
  }
  cache.store(cus + 1, std::memory_order_relaxed);
  return cus;
}

// Host copy of the kernel's visible-key end of query tile qt.
long long host_tile_key_end(int qt, long long qrows, long long P, long long W, long long G,
                            long long B) {
  const long long r_last = std::min<long long>((qt + 1LL) * qrows, G * W) - 1;
  return P + std::min<long long>(W, ((r_last / G) / B + 1) * B);
}

bool head_dim_supported(d2f_dtype_t dt, int d) {
  if (dt == D2F_BF16) return d == 64 || d == 128;
  if (dt == D2F_F32) return d == 32 || d == 64 || d == 128;
  return false;
}

}  // namespace

d2f_status_t check_desc(const d2f_attn_desc_t* d) {
  if (d == nullptr) return fail(D2F_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0) return fail(D2F_ERR_INVALID_ARG, "batch %d < 0", d->batch);
  if (d->n_heads_q < 1 || d->n_heads_kv < 1)
    return fail(D2F_ERR_INVALID_ARG, "head counts must be >= 1 (got %d, %d)", d->n_heads_q,
                d->n_heads_kv);
  if (d->n_heads_q % d->n_heads_kv != 0)
    return fail(D2F_ERR_INVALID_ARG, "n_heads_q %d is not a multiple of n_heads_kv %d",
                d->n_heads_q, d->n_heads_kv);
  if (d->head_dim < 1) return fail(D2F_ERR_INVALID_ARG, "head_dim %d < 1", d->head_dim);
  if (d->block_size < 1) return fail(D2F_ERR_INVALID_ARG, "block_size %d < 1", d->block_size);
  if (d->max_win_blocks < 1)
    return fail(D2F_ERR_INVALID_ARG, "max_win_blocks %d < 1", d->max_win_blocks);
  if (d->cache_capacity < 0)
    return fail(D2F_ERR_INVALID_ARG, "cache_capacity %lld < 0", (long long)d->cache_capacity);
  if (d->dtype != D2F_F32 && d->dtype != D2F_BF16)
    return fail(D2F_ERR_INVALID_ARG, "unknown dtype %d", (int)d->dtype);
  const long long wmax = (long long)d->max_win_blocks * d->block_size;
  if (wmax > (1 << 20) || d->cache_capacity > (1LL << 30) ||
      (long long)d->n_heads_q / d->n_heads_kv * wmax > (1LL << 30))
    return fail(D2F_ERR_INVALID_ARG, "window or cache too large for 32-bit row indexing");
  if (!std::isfinite(d->softmax_scale))
    return fail(D2F_ERR_INVALID_ARG, "softmax_scale is not finite");
  return D2F_OK;
}

namespace {

d2f_status_t check_lengths(const d2f_attn_desc_t* d, const int32_t* prefix, const int32_t* nwin) {
  if (d->batch == 0) return D2F_OK;
  if (prefix == nullptr || nwin == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "prefix_len_host / n_win_blocks_host is NULL");
  for (int b = 0; b < d->batch; ++b) {
    if (prefix[b] < 0) return fail(D2F_ERR_INVALID_ARG, "prefix_len[%d] = %d < 0", b, prefix[b]);
    if (nwin[b] < 0 || nwin[b] > d->max_win_blocks)
      return fail(D2F_ERR_INVALID_ARG, "n_win_blocks[%d] = %d outside [0, %d]", b, nwin[b],
                  d->max_win_blocks);
    const long long need = (long long)prefix[b] + (long long)nwin[b] * d->block_size;
    if (need > d->cache_capacity)
      return fail(D2F_ERR_CAPACITY, "request %d needs %lld cache slots, capacity %lld", b, need,
                  (long long)d->cache_capacity);
  }
  return D2F_OK;
}

struct Launch {
  std::vector<ReqInfo> req;
  int n_units = 0, n_groups = 0;
  int qrows = kQTile;  // query rows per unit
  int slot_rows = kQTile;  // partial-result rows per unit in the workspace
  bool any_split = false;
  bool remap = false;
  bool wide = false;   // eight-wave workgroups (two tile groups), bf16 only
  bool gqa = false;    // grouped-query kernel (attn_gqa.hip), bf16 only
};

// Workspace of one launch: partial outputs, then partial (max, sum).
size_t attn_partial_bytes(const Launch& L, int head_dim) {
  return (size_t)L.n_units * L.slot_rows * ((size_t)head_dim + 2) * sizeof(float);
}

// Host copy of the kernels' key-tile count: cache and window tiled apart.
long long host_key_tiles(long long P, long long k_end) {
  return (P + kKTile - 1) / kKTile + (k_end - P + kKTile - 1) / kKTile;
}

// Split the batch into launches of at most kMaxReqPerLaunch requests and size
// every request's key splits.  Within a launch, requests are ordered by unit
// size, largest first, so that the short units fill in behind the long ones.
// Returns the workspace bytes needed.
// key_off (key-range calls, else nullptr): the keys of request b are cache
// rows [key_off[b], key_off[b] + prefix[b]) and no window keys; a request with
// an empty range is idle.
// Units no shorter than min_chunk tiles, sized for `slots` workgroups.
size_t plan_pass(const d2f_attn_desc_t* d, const int32_t* prefix, const int32_t* nwin,
                 std::vector<Launch>& out, const int32_t* key_off, int min_chunk,
                 long long slots) {
  const bool cache_only = key_off != nullptr;
  auto key_end = [&](int qt, long long qrows, long long P, long long W, long long G,
                     long long B) {
    return cache_only ? P : host_tile_key_end(qt, qrows, P, W, G, B);
  };
  const int G = d->n_heads_q / d->n_heads_kv;
  const int B = d->block_size;
  // Query rows per unit: when no request has more than 32 query rows per KV
  // head, the bf16 kernel works on 32-row units (one 16-row block per wave),
  // so that all four waves of a unit have rows instead of two.
  long long max_rows = 0;
  for (int b = 0; b < d->batch; ++b) max_rows = std::max<long long>(max_rows, (long long)G * nwin[b] * B);
  const int qrows = (d->dtype == D2F_BF16 && max_rows <= 32) ? 32 : kQTile;
  long long total_tiles = 0;
  for (int b = 0; b < d->batch; ++b) {
    const long long W = (long long)nwin[b] * B;
    const int qtiles = (int)((G * W + qrows - 1) / qrows);
    for (int qt = 0; qt < qtiles; ++qt)
      total_tiles += (long long)d->n_heads_kv *
                     host_key_tiles(prefix[b], key_end(qt, qrows, prefix[b], W, G, B));
  }
  slots = std::max<long long>(1, slots);
  const long long chunk_tiles = std::max<long long>(min_chunk, (total_tiles + slots - 1) / slots);
  size_t ws = 0;
  out.clear();
  for (int b0 = 0; b0 < d->batch; b0 += kMaxReqPerLaunch) {
    Launch L;
    L.qrows = qrows;
    const int b1 = std::min(d->batch, b0 + kMaxReqPerLaunch);
    std::vector<std::pair<long long, ReqInfo>> reqs;
    for (int b = b0; b < b1; ++b) {
      if (nwin[b] == 0) continue;  // idle request: no query rows
      if (cache_only && prefix[b] == 0) continue;  // empty key range
      ReqInfo r{};
      r.b = b;
      r.prefix = prefix[b];
      r.key_off = cache_only ? key_off[b] : 0;
      r.win = nwin[b] * B;
      r.qtiles = (G * r.win + qrows - 1) / qrows;
      // The last query tile sees the most keys; it sets the split count.
      const long long tiles = host_key_tiles(
          r.prefix, key_end(r.qtiles - 1, qrows, r.prefix, r.win, G, B));
      r.nsplit = 1;
      if (tiles > kSplitFactor * chunk_tiles)
        r.nsplit = (int)std::min<long long>(tiles / min_chunk,
                                            (tiles + chunk_tiles - 1) / chunk_tiles);
      if (r.nsplit > 1) L.any_split = true;
      if (r.qtiles > 1) L.remap = true;
      reqs.push_back({(tiles + r.nsplit - 1) / r.nsplit, r});
    }
    std::stable_sort(reqs.begin(), reqs.end(),
                     [](const auto& x, const auto& y) { return x.first > y.first; });
    for (auto& pr : reqs) {
      ReqInfo r = pr.second;
      r.unit_base = L.n_units;
      r.group_base = L.n_groups;
      L.n_units += d->n_heads_kv * r.nsplit * r.qtiles;
      L.n_groups += d->n_heads_kv * r.qtiles;
      L.req.push_back(r);
    }
    if (L.n_units == 0) continue;
    if (L.any_split) ws = std::max(ws, attn_partial_bytes(L, d->head_dim));
    out.push_back(std::move(L));
  }
  return ws;
}

// Calls that go to the grouped-query kernel: bf16 grouped-query calls (on a
// contiguous or a paged cache: the plan does not depend on the layout, so
// the two give the same bits) with at least kGqaMinRowsPerCU query rows per
// CU over the call, where a unit per CU gives each K/V tile enough rows.
// Measured on MI355X with 28 query / 4 KV heads, 8 requests and 2048 cached
// keys: 1344 rows per KV head (168 per CU) 64-68 us against 81-85 us on the
// four-wave kernels; 672 rows (84 per CU, 96-row units, keys split between
// the wave groups) 43-46 vs 51.6 us; 336 rows (42 per CU, 48-row units, keys
// split) 33.7 vs 35.0 us on the eight-wave kernel, and on a paged cache 40.5
// vs 45.6 us.  (Before the key split, 48-row units took 37.5 us, and such
// calls stayed on the eight-wave kernel.)
constexpr long long kGqaMinRowsPerCU = 40;
constexpr int kGqaMinGroup = 2;  // query heads per KV head
bool use_gqa(const d2f_attn_desc_t* d, const int32_t* nwin, long long cus) {
  if (d->dtype != D2F_BF16 || (d->head_dim != 64 && d->head_dim != 128) ||
      d->n_heads_q / d->n_heads_kv < kGqaMinGroup)
    return false;
  long long rows = 0;
  for (int b = 0; b < d->batch; ++b) rows += (long long)d->n_heads_q * nwin[b] * d->block_size;
  return rows >= kGqaMinRowsPerCU * std::max<long long>(1, cus);
}

// Grouped-query plan (attn_gqa.hip): a unit is R query rows of one (request,
// KV head) over all of its keys -- R a multiple of 16, at most kGqaMaxRows
// -- one workgroup of eight waves, one workgroup per CU.  R is the launch's
// query rows per CU, so that each CU gets about one unit and every K/V tile
// it streams feeds as many rows as the launch allows.  Keys are never cut
// into ranges across units (the calls this kernel takes have at least
// kGqaMinRowsPerCU rows per CU, so the units cover the CUs; within a unit of
// at most 8 blocks the kernel's two wave groups split each tile's keys and
// join in LDS), and no workspace is needed.
size_t plan_gqa(const d2f_attn_desc_t* d, const int32_t* prefix, const int32_t* nwin,
                std::vector<Launch>& out, const int32_t* key_off, long long cus) {
  const bool cache_only = key_off != nullptr;
  const int G = d->n_heads_q / d->n_heads_kv;
  const int B = d->block_size;
  const int hkv = d->n_heads_kv;
  cus = std::max<long long>(1, cus);
  out.clear();
  for (int b0 = 0; b0 < d->batch; b0 += kMaxReqPerLaunch) {
    const int b1 = std::min(d->batch, b0 + kMaxReqPerLaunch);
    auto active = [&](int b) { return nwin[b] > 0 && !(cache_only && prefix[b] == 0); };
    long long rows = 0;
    for (int b = b0; b < b1; ++b)
      if (active(b)) rows += (long long)hkv * G * nwin[b] * B;
    if (rows == 0) continue;
    long long R = ((rows + cus - 1) / cus + 15) / 16 * 16;
    R = std::min<long long>(kGqaMaxRows, std::max<long long>(16, R));
    Launch L;
    L.qrows = (int)R;
    L.slot_rows = (int)R;
    L.gqa = true;
    std::vector<std::pair<long long, ReqInfo>> reqs;
    for (int b = b0; b < b1; ++b) {
      if (!active(b)) continue;
      ReqInfo r{};
      r.b = b;
      r.prefix = prefix[b];
      r.key_off = cache_only ? key_off[b] : 0;
      r.win = nwin[b] * B;
      r.qtiles = (int)((G * r.win + R - 1) / R);
      r.nsplit = 1;
      if (r.qtiles > 1) L.remap = true;
      const long long tiles = host_key_tiles(
          r.prefix, cache_only ? r.prefix
                               : host_tile_key_end(r.qtiles - 1, R, r.prefix, r.win, G, B));
      reqs.push_back({tiles, r});
    }
    std::stable_sort(reqs.begin(), reqs.end(),
                     [](const auto& x, const auto& y) { return x.first > y.first; });
    for (auto& pr : reqs) {
      ReqInfo r = pr.second;
      r.unit_base = L.n_units;
      r.group_base = L.n_groups;
      L.n_units += hkv * r.qtiles;
      L.n_groups += hkv * r.qtiles;
      L.req.push_back(r);
    }
    if (L.n_units == 0) continue;
    out.push_back(std::move(L));
  }
  return 0;
}

// The launches of one call.  A bf16 call whose launches all have no more
// units than the device has CUs and cut no key range runs the eight-wave
// kernel (two tile groups of four waves per unit), so that every SIMD holds
// two waves of long, unsplit units.  Measured on MI355X: 8 requests with a
// 2048-token prefix, 28 query and 4 KV heads (192 units of 33 tiles) took
// 34.4-35.1 us against 39.7-39.9 us on four-wave workgroups.  A call that is
// split to occupy the device keeps the four-wave kernel: a 512-token prefix
// with 32 heads took 13.1 us unsplit on the eight-wave kernel against
// 12.5 us for 3 key ranges and the merge (a dependent step 26.4 vs 25.3 us).
size_t plan_attention(const d2f_attn_desc_t* d, const int32_t* prefix, const int32_t* nwin,
                      std::vector<Launch>& out, const int32_t* key_off = nullptr,
                      bool paged = false) {
  if (use_gqa(d, nwin, device_cus()))
    return plan_gqa(d, prefix, nwin, out, key_off, device_cus());
  const long long resident = resident_workgroups(d->dtype, d->head_dim);
  const size_t ws = plan_pass(d, prefix, nwin, out, key_off, kMinChunkTiles,
                              (long long)(kSlotFill * (double)resident));
  if (d->dtype != D2F_BF16) return ws;
  const long long cus = device_cus();
  // A split call with few, long key ranges (a long prefix over few heads)
  // is re-planned for one eight-wave unit per CU, if that keeps every range
  // between kWideSplitMinTiles and kWideSplitMaxTiles tiles.  Measured on
  // MI355X, 32 heads over a 32768-token prefix: 8 ranges of 64 tiles on
  // eight waves 92.8-95.9 us against 97.0-99.2 us for 12 ranges on four
  // waves; with a 131072-token prefix (256-tile ranges) the four-wave plan
  // stays faster (332 vs 350 us), and 512 tokens (3-tile ranges) too.
  // Contiguous caches only: on the paged loader the same re-plan took 113
  // vs 99-101 us for the 32K prefix.  Such a paged call therefore cuts its
  // keys into other ranges than the contiguous call, and the two results
  // differ by rounding; every other plan is the same for both layouts.
  bool split = false;
  for (const Launch& L : out) split |= L.any_split;
  if (split && !paged) {
    std::vector<Launch> wide;
    const size_t ws2 = plan_pass(d, prefix, nwin, wide, key_off, kMinChunkTiles, cus);
    const int G = d->n_heads_q / d->n_heads_kv;
    bool ok = !wide.empty();
    for (const Launch& L : wide) {
      ok &= L.n_units <= cus;
      for (const ReqInfo& r : L.req) {
        const long long tiles = host_key_tiles(
            r.prefix, key_off != nullptr ? r.prefix
                                         : host_tile_key_end(r.qtiles - 1, L.qrows, r.prefix,
                                                             r.win, G, d->block_size));
        const long long len = (tiles + r.nsplit - 1) / r.nsplit;
        ok &= r.nsplit > 1 && len >= kWideSplitMinTiles && len <= kWideSplitMaxTiles;
      }
    }
    if (ok) {
      for (Launch& L : wide) L.wide = true;
      out = std::move(wide);
      return ws2;
    }
  }
  for (const Launch& L : out)
    if (L.n_units > cus || L.any_split) return ws;
  for (Launch& L : out) L.wide = true;
  return ws;
}

size_t commit_chunks(int32_t vocab) { return (size_t)((vocab + kCommitChunk - 1) / kCommitChunk); }

// Commit workspace: one (max, sum, argmax) partial per (row, chunk).
size_t commit_partial_bytes(int32_t n_rows, int32_t vocab) {
  return (size_t)n_rows * commit_chunks(vocab) * sizeof(float4);
}
// One int32 / uint32 word per row, rounded up to 16 bytes.
size_t commit_row_words_bytes(int32_t n_rows) { return ((size_t)n_rows * 4 + 15) / 16 * 16; }
// Partials, then the early commit's argmax per row and gap minimum per group
// (at most one group per row).
size_t commit_workspace_bytes(int32_t n_rows, int32_t vocab) {
  return commit_partial_bytes(n_rows, vocab) + 2 * commit_row_words_bytes(n_rows);
}

}  // namespace
}  // namespace d2f

namespace d2f {
namespace {

// Page tables of a paged call (nullptr for contiguous caches).
struct PagedRefs {
  const int32_t* page_table;
  const int32_t* win_pages;
  int32_t table_stride;
  int32_t n_pages;
};

// Plan and launch one attention call (arguments already validated).
d2f_status_t run_attention(const d2f_attn_desc_t* desc, const void* q, const void* k_cache,
                           const void* v_cache, const void* k_win, const void* v_win,
                           const int32_t* prefix_len_host, const int32_t* n_win_blocks_host,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t s, const PagedRefs* paged,
                           const int32_t* key_off = nullptr) {
  std::vector<Launch> plan;
  const size_t need =
      plan_attention(desc, prefix_len_host, n_win_blocks_host, plan, key_off, paged != nullptr);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(D2F_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                workspace == nullptr ? (size_t)0 : workspace_bytes, need);
  if (need > 0 && ((uintptr_t)workspace % 256) != 0)
    return fail(D2F_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  const float scale =
      desc->softmax_scale > 0.f ? desc->softmax_scale : 1.0f / std::sqrt((float)desc->head_dim);
  for (const Launch& L : plan) {
    AttnArgs a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.kw = k_win;
    a.vw = v_win;
    a.out = out;
    a.lse = lse;
    a.ws_o = (float*)workspace;
    a.ws_ml = L.any_split ? (float*)workspace + (size_t)L.n_units * L.slot_rows * desc->head_dim
                          : nullptr;
    a.cap = desc->cache_capacity;
    a.qrows = L.qrows;
    a.slot_rows = L.slot_rows;
    a.hq = desc->n_heads_q;
    a.hkv = desc->n_heads_kv;
    a.group = desc->n_heads_q / desc->n_heads_kv;
    a.wmax = desc->max_win_blocks * desc->block_size;
    a.bsz = desc->block_size;
    a.n_req = (int)L.req.size();
    a.n_units = L.n_units;
    a.n_groups = L.n_groups;
    a.remap = L.remap ? 1 : 0;
    a.c2 = scale * 1.4426950408889634f;
    a.cache_only = key_off != nullptr ? 1 : 0;
    a.wide = L.wide ? 1 : 0;
    if (paged != nullptr) {
      a.page_table = paged->page_table;
      a.win_pages = paged->win_pages;
      a.table_stride = paged->table_stride;
      a.n_pages = paged->n_pages;
      int sh = 0;
      while ((1 << sh) < desc->block_size) ++sh;
      a.page_shift = sh;
    }
    for (size_t i = 0; i < L.req.size(); ++i) a.req[i] = L.req[i];
    hipError_t e = L.gqa ? launch_attn_gqa(a, desc->head_dim, paged != nullptr, s)
                   : desc->dtype == D2F_BF16
                       ? launch_attn_bf16(a, desc->head_dim, paged != nullptr, s)
                       : launch_attn_f32(a, desc->head_dim, s);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    if (L.any_split) {
      e = launch_attn_merge(a, desc->head_dim, desc->dtype, s);
      if (e != hipSuccess) return hip_fail(e, "split merge launch");
    }
  }
  return D2F_OK;
}

d2f_status_t check_ranges(const d2f_attn_desc_t* d, const int32_t* lo, const int32_t* hi,
                          const int32_t* nwin, std::vector<int32_t>& len) {
  if (d->batch == 0) return D2F_OK;
  if (lo == nullptr || hi == nullptr || nwin == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "key ranges / n_win_blocks_host are NULL");
  len.resize(d->batch);
  for (int b = 0; b < d->batch; ++b) {
    if (lo[b] < 0 || hi[b] < lo[b])
      return fail(D2F_ERR_INVALID_ARG, "key range [%d, %d) of request %d is not a range", lo[b],
                  hi[b], b);
    if (hi[b] > d->cache_capacity)
      return fail(D2F_ERR_CAPACITY, "key range of request %d ends at %d > capacity %lld", b,
                  hi[b], (long long)d->cache_capacity);
    if (nwin[b] < 0 || nwin[b] > d->max_win_blocks)
      return fail(D2F_ERR_INVALID_ARG, "n_win_blocks[%d] = %d outside [0, %d]", b, nwin[b],
                  d->max_win_blocks);
    len[b] = hi[b] - lo[b];
  }
  return D2F_OK;
}

}  // namespace
}  // namespace d2f

using namespace d2f;

extern "C" {

const char* d2f_status_string(d2f_status_t s) {
  switch (s) {
    case D2F_OK: return "ok";
    case D2F_ERR_INVALID_ARG: return "invalid argument";
    case D2F_ERR_CAPACITY: return "cache capacity exceeded";
    case D2F_ERR_ORDER: return "only the oldest window block can be committed";
    case D2F_ERR_WORKSPACE: return "workspace missing or too small";
    case D2F_ERR_HIP: return "HIP runtime error";
    case D2F_ERR_UNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

const char* d2f_last_error(void) { return g_last_error.c_str(); }

int32_t d2f_version(void) { return 100; }

d2f_status_t d2f_block_attn_workspace_size(const d2f_attn_desc_t* desc,
                                           const int32_t* prefix_len_host,
                                           const int32_t* n_win_blocks_host, size_t* bytes_out) {
  if (bytes_out == nullptr) return fail(D2F_ERR_INVALID_ARG, "bytes_out is NULL");
  d2f_status_t st = check_desc(desc);
  if (st != D2F_OK) return st;
  if ((st = check_lengths(desc, prefix_len_host, n_win_blocks_host)) != D2F_OK) return st;
  std::vector<Launch> plan;
  // The size covers both the contiguous and the paged call on these lengths
  // (their plans may differ).
  *bytes_out = std::max(plan_attention(desc, prefix_len_host, n_win_blocks_host, plan),
                        plan_attention(desc, prefix_len_host, n_win_blocks_host, plan, nullptr,
                                       true));
  return D2F_OK;
}


d2f_status_t d2f_block_attn(const d2f_attn_desc_t* desc, const void* q, const void* k_cache,
                            const void* v_cache, const void* k_win, const void* v_win,
                            const int32_t* prefix_len_host, const int32_t* n_win_blocks_host,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            d2f_stream_t stream) {
  d2f_status_t st = check_desc(desc);
  if (st != D2F_OK) return st;
  if ((st = check_lengths(desc, prefix_len_host, n_win_blocks_host)) != D2F_OK) return st;
  if (!head_dim_supported(desc->dtype, desc->head_dim))
    return fail(D2F_ERR_UNSUPPORTED, "head_dim %d is not built for dtype %d", desc->head_dim,
                (int)desc->dtype);
  if (desc->batch == 0) return D2F_OK;
  bool any_prefix = false;
  for (int b = 0; b < desc->batch; ++b) any_prefix |= prefix_len_host[b] > 0;
  if (q == nullptr || k_win == nullptr || v_win == nullptr || out == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "q, k_win, v_win and out must not be NULL");
  if (any_prefix && (k_cache == nullptr || v_cache == nullptr))
    return fail(D2F_ERR_INVALID_ARG, "k_cache / v_cache is NULL but a prefix is not empty");
  const size_t esz = desc->dtype == D2F_BF16 ? 2 : 4;
  for (const void* p : {q, k_cache, v_cache, k_win, v_win, (const void*)out})
    if (p != nullptr && ((uintptr_t)p % 16) != 0)
      return fail(D2F_ERR_INVALID_ARG, "q/k/v/out buffers must be 16-byte aligned");
  if (((size_t)desc->head_dim * esz) % 16 != 0)
    return fail(D2F_ERR_UNSUPPORTED, "head_dim rows must be a multiple of 16 bytes");
  return run_attention(desc, q, k_cache, v_cache, k_win, v_win, prefix_len_host,
                       n_win_blocks_host, out, lse, workspace, workspace_bytes,
                       (hipStream_t)stream, nullptr);
}


d2f_status_t d2f_block_attn_range_workspace_size(const d2f_attn_desc_t* desc,
                                                 const int32_t* key_lo_host,
                                                 const int32_t* key_hi_host,
                                                 const int32_t* n_win_blocks_host,
                                                 size_t* bytes_out) {
  if (bytes_out == nullptr) return fail(D2F_ERR_INVALID_ARG, "bytes_out is NULL");
  d2f_status_t st = check_desc(desc);
  if (st != D2F_OK) return st;
  std::vector<int32_t> len;
  if ((st = check_ranges(desc, key_lo_host, key_hi_host, n_win_blocks_host, len)) != D2F_OK)
    return st;
  std::vector<Launch> plan;
  *bytes_out = desc->batch == 0 ? 0
                                : plan_attention(desc, len.data(), n_win_blocks_host, plan,
                                                 key_lo_host);
  return D2F_OK;
}

d2f_status_t d2f_block_attn_range(const d2f_attn_desc_t* desc, const void* q,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* key_lo_host, const int32_t* key_hi_host,
                                  const int32_t* n_win_blocks_host, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, d2f_stream_t stream) {
  d2f_status_t st = check_desc(desc);
  if (st != D2F_OK) return st;
  std::vector<int32_t> len;
  if ((st = check_ranges(desc, key_lo_host, key_hi_host, n_win_blocks_host, len)) != D2F_OK)
    return st;
  if (!head_dim_supported(desc->dtype, desc->head_dim))
    return fail(D2F_ERR_UNSUPPORTED, "head_dim %d is not built for dtype %d", desc->head_dim,
                (int)desc->dtype);
  if (desc->batch == 0) return D2F_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || out == nullptr || lse == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "q, k_cache, v_cache, out and lse must not be NULL");
  for (const void* p : {q, k_cache, v_cache, (const void*)out})
    if (((uintptr_t)p % 16) != 0)
      return fail(D2F_ERR_INVALID_ARG, "q/k/v/out buffers must be 16-byte aligned");
  const size_t esz = desc->dtype == D2F_BF16 ? 2 : 4;
  if (((size_t)desc->head_dim * esz) % 16 != 0)
    return fail(D2F_ERR_UNSUPPORTED, "head_dim rows must be a multiple of 16 bytes");
  return run_attention(desc, q, k_cache, v_cache, nullptr, nullptr, len.data(),
                       n_win_blocks_host, out, lse, workspace, workspace_bytes,
                       (hipStream_t)stream, nullptr, key_lo_host);
}

d2f_status_t d2f_attn_combine(const d2f_attn_desc_t* desc, const void* out_a, const float* lse_a,
                              const void* out_b, const float* lse_b, void* out, float* lse,
                              const int32_t* n_win_blocks_host, d2f_stream_t stream) {
  d2f_status_t st = check_desc(desc);
  if (st != D2F_OK) return st;
  if (!head_dim_supported(desc->dtype, desc->head_dim))
    return fail(D2F_ERR_UNSUPPORTED, "head_dim %d is not built for dtype %d", desc->head_dim,
                (int)desc->dtype);
  if (desc->batch == 0) return D2F_OK;
  if (out_a == nullptr || lse_a == nullptr || out_b == nullptr || lse_b == nullptr ||
      out == nullptr || lse == nullptr || n_win_blocks_host == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "a required pointer is NULL");
  for (int b = 0; b < desc->batch; ++b)
    if (n_win_blocks_host[b] < 0 || n_win_blocks_host[b] > desc->max_win_blocks)
      return fail(D2F_ERR_INVALID_ARG, "n_win_blocks[%d] = %d outside [0, %d]", b,
                  n_win_blocks_host[b], desc->max_win_blocks);
  const int wmax = desc->max_win_blocks * desc->block_size;
  for (int b0 = 0; b0 < desc->batch; b0 += kMaxReqPerLaunch) {
    CombineArgs a{};
    a.out_a = out_a;
    a.lse_a = lse_a;
    a.out_b = out_b;
    a.lse_b = lse_b;
    a.out = out;
    a.lse = lse;
    a.hq = desc->n_heads_q;
    a.wmax = wmax;
    a.b0 = b0;
    a.n_req = std::min(kMaxReqPerLaunch, desc->batch - b0);
    for (int i = 0; i < a.n_req; ++i) a.win[i] = n_win_blocks_host[b0 + i] * desc->block_size;
    hipError_t e = launch_combine(a, desc->head_dim, desc->dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return D2F_OK;
}

d2f_status_t d2f_block_attn_paged(const d2f_attn_desc_t* desc, const void* q,
                                  const void* k_pages, const void* v_pages, int32_t n_pages,
                                  const int32_t* page_table, int32_t table_stride,
                                  const int32_t* win_pages, const int32_t* prefix_len_host,
                                  const int32_t* n_win_blocks_host, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, d2f_stream_t stream) {
  d2f_status_t st = check_desc(desc);
  if (st != D2F_OK) return st;
  if (desc->dtype != D2F_BF16 || (desc->head_dim != 64 && desc->head_dim != 128))
    return fail(D2F_ERR_UNSUPPORTED, "paged attention is built for bf16, head_dim 64 or 128");
  const int B = desc->block_size;
  if (B < 8 || (B & (B - 1)) != 0)
    return fail(D2F_ERR_UNSUPPORTED, "paged attention needs a power-of-two block_size >= 8 "
                "(got %d)", B);
  if (desc->batch == 0) return D2F_OK;
  if (prefix_len_host == nullptr || n_win_blocks_host == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "prefix_len_host / n_win_blocks_host is NULL");
  if (n_pages < 1 || table_stride < 0)
    return fail(D2F_ERR_INVALID_ARG, "n_pages %d / table_stride %d out of range", n_pages,
                table_stride);
  bool any_prefix = false, any_win = false;
  for (int b = 0; b < desc->batch; ++b) {
    const int P = prefix_len_host[b], n = n_win_blocks_host[b];
    if (P < 0 || P % B != 0)
      return fail(D2F_ERR_INVALID_ARG, "prefix_len[%d] = %d is not a whole number of blocks", b,
                  P);
    if (n < 0 || n > desc->max_win_blocks)
      return fail(D2F_ERR_INVALID_ARG, "n_win_blocks[%d] = %d outside [0, %d]", b, n,
                  desc->max_win_blocks);
    if (P / B > table_stride)
      return fail(D2F_ERR_CAPACITY, "request %d: %d cached blocks, table holds %d", b, P / B,
                  table_stride);
    any_prefix |= P > 0;
    any_win |= n > 0;
  }
  if (q == nullptr || out == nullptr || k_pages == nullptr || v_pages == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "q, out and the page pools must not be NULL");
  if ((any_prefix && page_table == nullptr) || (any_win && win_pages == nullptr))
    return fail(D2F_ERR_INVALID_ARG, "page table or window pages are NULL");
  for (const void* p : {q, k_pages, v_pages, (const void*)out})
    if (((uintptr_t)p % 16) != 0)
      return fail(D2F_ERR_INVALID_ARG, "q/pages/out buffers must be 16-byte aligned");
  if ((unsigned long long)n_pages * desc->n_heads_kv * B * desc->head_dim * 2 >= (1ULL << 62))
    return fail(D2F_ERR_INVALID_ARG, "page pool too large");
  const PagedRefs refs{page_table, win_pages, table_stride, n_pages};
  return run_attention(desc, q, k_pages, v_pages, nullptr, nullptr, prefix_len_host,
                       n_win_blocks_host, out, lse, workspace, workspace_bytes,
                       (hipStream_t)stream, &refs);
}

d2f_status_t d2f_kv_commit(const d2f_attn_desc_t* desc, int32_t n_layers, void* k_cache,
                           void* v_cache, int64_t cache_layer_stride, const void* k_win,
                           const void* v_win, int64_t win_layer_stride, int32_t request,
                           int32_t block, int32_t* prefix_len_host, int32_t* prefix_len_dev,
                           d2f_stream_t stream) {
  d2f_status_t st = check_desc(desc);
  if (st != D2F_OK) return st;
  if (n_layers < 1) return fail(D2F_ERR_INVALID_ARG, "n_layers %d < 1", n_layers);
  if (request < 0 || request >= desc->batch)
    return fail(D2F_ERR_INVALID_ARG, "request %d outside [0, %d)", request, desc->batch);
  if (block != 0)
    return fail(D2F_ERR_ORDER, "block %d is not the oldest window block (0)", block);
  if (prefix_len_host == nullptr) return fail(D2F_ERR_INVALID_ARG, "prefix_len_host is NULL");
  if (k_cache == nullptr || v_cache == nullptr || k_win == nullptr || v_win == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "cache and window pointers must not be NULL");
  const int32_t P = prefix_len_host[request];
  if (P < 0) return fail(D2F_ERR_INVALID_ARG, "prefix_len[%d] = %d < 0", request, P);
  if ((long long)P + desc->block_size > desc->cache_capacity)
    return fail(D2F_ERR_CAPACITY, "cache full: %d + %d > %lld", P, desc->block_size,
                (long long)desc->cache_capacity);
  const long long wmax = (long long)desc->max_win_blocks * desc->block_size;
  const long long cache_layer = (long long)desc->batch * desc->n_heads_kv * desc->cache_capacity *
                                desc->head_dim;
  const long long win_layer = (long long)desc->batch * desc->n_heads_kv * wmax * desc->head_dim;
  if (n_layers > 1 && (cache_layer_stride < cache_layer || win_layer_stride < win_layer))
    return fail(D2F_ERR_INVALID_ARG, "layer strides smaller than one layer");
  const int esz = desc->dtype == D2F_BF16 ? 2 : 4;
  KvArgs a{};
  a.kc = k_cache;
  a.vc = v_cache;
  a.kw = k_win;
  a.vw = v_win;
  a.cache_layer_stride = cache_layer_stride;
  a.win_layer_stride = win_layer_stride;
  a.cap = desc->cache_capacity;
  a.n_layers = n_layers;
  a.hkv = desc->n_heads_kv;
  a.wmax = (int32_t)wmax;
  a.head_dim = desc->head_dim;
  a.bsz = desc->block_size;
  a.esize = esz;
  a.request = request;
  a.prefix = P;
  a.new_prefix = P + desc->block_size;
  a.prefix_dev = prefix_len_dev;
  hipError_t e = launch_kv_commit(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv commit launch");
  prefix_len_host[request] = P + desc->block_size;
  return D2F_OK;
}

d2f_status_t d2f_kv_commit_paged(const d2f_attn_desc_t* desc, int32_t* page_table,
                                 int32_t table_stride, int32_t* win_pages, int32_t request,
                                 int32_t* prefix_len_host, int32_t* prefix_len_dev,
                                 d2f_stream_t stream) {
  d2f_status_t st = check_desc(desc);
  if (st != D2F_OK) return st;
  if (request < 0 || request >= desc->batch)
    return fail(D2F_ERR_INVALID_ARG, "request %d outside [0, %d)", request, desc->batch);
  if (page_table == nullptr || win_pages == nullptr || prefix_len_host == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "page table, window pages or prefix lengths are NULL");
  const int B = desc->block_size;
  const int32_t P = prefix_len_host[request];
  if (P < 0 || P % B != 0)
    return fail(D2F_ERR_INVALID_ARG, "prefix_len[%d] = %d is not a whole number of blocks",
                request, P);
  if (P / B >= table_stride)
    return fail(D2F_ERR_CAPACITY, "page table full: %d blocks, %d slots", P / B, table_stride);
  hipError_t e = launch_kv_commit_paged(page_table, win_pages, prefix_len_dev, request,
                                        table_stride, desc->max_win_blocks, P / B, P + B,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "paged kv commit launch");
  prefix_len_host[request] = P + B;
  return D2F_OK;
}

d2f_status_t d2f_confidence_commit_workspace_size(int32_t n_rows, int32_t vocab,
                                                  size_t* bytes_out) {
  if (bytes_out == nullptr) return fail(D2F_ERR_INVALID_ARG, "bytes_out is NULL");
  if (n_rows < 0 || vocab < 1)
    return fail(D2F_ERR_INVALID_ARG, "n_rows %d / vocab %d out of range", n_rows, vocab);
  *bytes_out = commit_workspace_bytes(n_rows, vocab);
  return D2F_OK;
}

d2f_status_t d2f_confidence_commit_ex(const float* logits, int64_t ld, int32_t n_rows,
                                      int32_t vocab, uint8_t* mask_state, int32_t* tokens,
                                      const uint8_t* block_phase, int32_t block_size,
                                      d2f_conf_measure_t measure, float tau, int32_t k_aggr,
                                      int32_t mask_token_id, const float* early_gap,
                                      int32_t early_group_blocks, float* conf_out,
                                      int32_t* argmax_out, int32_t* n_committed,
                                      uint8_t* block_complete, void* workspace,
                                      size_t workspace_bytes, d2f_stream_t stream) {
  if (n_rows < 0 || vocab < 1 || ld < vocab)
    return fail(D2F_ERR_INVALID_ARG, "n_rows %d, vocab %d, ld %lld out of range", n_rows, vocab,
                (long long)ld);
  if (block_size < 1 || n_rows % block_size != 0)
    return fail(D2F_ERR_INVALID_ARG, "n_rows %d is not a multiple of block_size %d", n_rows,
                block_size);
  if (block_size > kMaxCommitBlock)
    return fail(D2F_ERR_UNSUPPORTED, "block_size %d > %d", block_size, kMaxCommitBlock);
  if (k_aggr < 0) return fail(D2F_ERR_INVALID_ARG, "k_aggr %d < 0", k_aggr);
  if (std::isnan(tau)) return fail(D2F_ERR_INVALID_ARG, "tau is NaN");
  if ((int)measure < (int)D2F_CONF_MAXPROB || (int)measure > (int)D2F_CONF_LOGIT_GAP)
    return fail(D2F_ERR_INVALID_ARG, "unknown confidence measure %d", (int)measure);
  if (early_group_blocks < 0)
    return fail(D2F_ERR_INVALID_ARG, "early_group_blocks %d < 0", early_group_blocks);
  if (early_gap != nullptr && measure == D2F_CONF_NEG_ENTROPY)
    return fail(D2F_ERR_INVALID_ARG, "the early commit needs the logit gap, which the "
                "negative-entropy pass does not keep");
  if (n_rows == 0) return D2F_OK;
  if (logits == nullptr || mask_state == nullptr || tokens == nullptr || block_phase == nullptr ||
      n_committed == nullptr || block_complete == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "a required pointer is NULL");
  const size_t n_chunks = commit_chunks(vocab);
  const size_t need = commit_workspace_bytes(n_rows, vocab);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(D2F_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                workspace == nullptr ? (size_t)0 : workspace_bytes, need);
  if (((uintptr_t)workspace % 16) != 0)
    return fail(D2F_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  if ((unsigned long long)n_rows * n_chunks > 0x7fffffffULL)
    return fail(D2F_ERR_UNSUPPORTED, "too many rows x chunks for one launch");
  const int n_blocks = n_rows / block_size;
  const int group = early_group_blocks == 0 ? n_blocks : std::min(early_group_blocks, n_blocks);
  CommitArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.n_rows = n_rows;
  a.vocab = vocab;
  a.n_chunks = (int32_t)n_chunks;
  a.chunk = kCommitChunk;
  a.block_size = block_size;
  a.k_aggr = k_aggr;
  a.mask_token_id = mask_token_id;
  a.tau = tau;
  a.mask_state = mask_state;
  a.tokens = tokens;
  a.block_phase = block_phase;
  a.conf_out = conf_out;
  a.argmax_out = argmax_out;
  a.n_committed = n_committed;
  a.block_complete = block_complete;
  a.partial = (float4*)workspace;
  a.measure = (int32_t)measure;
  a.group_blocks = group;
  a.n_groups = (n_blocks + group - 1) / group;
  a.early_gap = early_gap;
  char* extra = (char*)workspace + commit_partial_bytes(n_rows, vocab);
  a.ws_argmax = (int32_t*)extra;
  a.ws_gmin = (uint32_t*)(extra + commit_row_words_bytes(n_rows));
  const bool vec4 = ((uintptr_t)logits % 16) == 0 && (ld % 4) == 0;
  hipError_t e = launch_confidence_commit(a, vec4, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "confidence commit launch");
  return D2F_OK;
}

d2f_status_t d2f_confidence_commit(const float* logits, int64_t ld, int32_t n_rows,
                                   int32_t vocab, uint8_t* mask_state, int32_t* tokens,
                                   const uint8_t* block_phase, int32_t block_size, float tau,
                                   int32_t k_aggr, int32_t mask_token_id, float* conf_out,
                                   int32_t* argmax_out, int32_t* n_committed,
                                   uint8_t* block_complete, void* workspace,
                                   size_t workspace_bytes, d2f_stream_t stream) {
  return d2f_confidence_commit_ex(logits, ld, n_rows, vocab, mask_state, tokens, block_phase,
                                  block_size, D2F_CONF_MAXPROB, tau, k_aggr, mask_token_id,
                                  nullptr, 0, conf_out, argmax_out, n_committed, block_complete,
                                  workspace, workspace_bytes, stream);
}

float d2f_prophet_threshold(float progress) {
  const float p = std::isnan(progress) ? 0.f : std::min(1.f, std::max(0.f, progress));
  if (3.f * p < 1.f) return 7.5f;
  if (3.f * p < 2.f) return 5.0f;
  return 2.5f;
}

}  // extern "C"
