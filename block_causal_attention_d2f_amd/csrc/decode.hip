// One decoding step's bookkeeping after the commit pass: the active-window
// schedule of every request (window.hip), then one launch that appends the
// K/V of the blocks that left the window to the cache, hands their tokens to
// the decoded sequence, and lays the window rows out for the next pass.
//
// [D2F-review] section "쉽게 이해하기" (inference paragraph): the window moves
// forward block by block while later blocks are already being decoded.
// [D2F-wiki] section "운영 관점" (KV cache management): the completion of a
// block is the signal that its K/V become permanent cache entries.
//
// Window rows live in per-request slots: request b owns rows
// [b * Wmax, (b + 1) * Wmax) of mask_state / tokens and window blocks
// [b * max_win, (b + 1) * max_win) of block_phase / n_committed.  Rows past
// the window are kept COMMITTED, so the commit pass does not read their logits.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "d2f_internal.h"

namespace d2f {
namespace {

constexpr int kCopySlices = 8;  // (layer, KV head, K or V) slices per copy workgroup
constexpr int kCopyUnroll = 4;  // loads in flight per thread

// Copy workgroups of a request that persists blocks.
int copy_workgroups(int n_layers, int hkv) {
  return (2 * n_layers * hkv + kCopySlices - 1) / kCopySlices;
}

__device__ int copy_request(const AdvArgs& a, int c) {
  // Last request whose first copy workgroup is <= c (requests without a copy
  // share their base with the next one, so the last such request owns c).
  int lo = 0, hi = a.n_req - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.req[mid].copy_base <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Copy workgroup c: kCopySlices consecutive (layer, KV head, K or V) slices
// of one request.  The persisted blocks are window rows [0, p * B), contiguous
// per head, and go to cache slots [P, P + p * B).  Each thread keeps kCopyUnroll
// loads in flight before it stores.
template <bool VEC16>
__device__ void copy_blocks(const AdvArgs& a, int c) {
  using T = typename std::conditional<VEC16, uint4, uint16_t>::type;
  const int i = copy_request(a, c);
  const AdvReq& r = a.req[i];
  const size_t rb = (size_t)(a.req0 + i);
  const int n_slices = 2 * a.n_layers * a.hkv;
  const int s0 = (c - r.copy_base) * kCopySlices;
  const int s1 = min(n_slices, s0 + kCopySlices);
  const size_t esz = (size_t)a.esize;
  const uint32_t n = (uint32_t)((size_t)r.persisted * a.bsz * a.head_dim * esz / sizeof(T));
  const uint32_t total = (uint32_t)(s1 - s0) * n;
  for (uint32_t f0 = threadIdx.x; f0 < total; f0 += blockDim.x * kCopyUnroll) {
    T v[kCopyUnroll];
    T* dst[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint32_t f = f0 + (uint32_t)u * blockDim.x;
      dst[u] = nullptr;
      if (f < total) {
        const int sl = s0 + (int)(f / n);
        const uint32_t e = f % n;
        const int which = sl & 1;
        const int lh = sl >> 1;
        const int layer = lh / a.hkv, head = lh % a.hkv;
        const T* src = (const T*)((const char*)(which ? a.vw : a.kw) +
                                  ((size_t)layer * a.win_layer_stride +
                                   (rb * a.hkv + head) * (size_t)a.wmax * a.head_dim) * esz);
        T* d = (T*)((char*)(which ? a.vc : a.kc) +
                    ((size_t)layer * a.cache_layer_stride +
                     ((rb * a.hkv + head) * (size_t)a.cap + r.prefix) * a.head_dim) * esz);
        v[u] = src[e];
        dst[u] = d + e;
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (dst[u] != nullptr) *dst[u] = v[u];
  }
}

// One workgroup per request: decoded tokens out, window rows moved up by the
// persisted blocks, an appended block's rows MASKED, rows past the window
// COMMITTED, phases for the next pass, device prefix length.
__device__ void advance_window(const AdvArgs& a, int i) {
  const AdvReq& r = a.req[i];
  const size_t rb = (size_t)(a.req0 + i);
  const int B = a.bsz;
  const size_t base = rb * a.wmax;
  const int shift = r.persisted * B;
  if (shift > 0) {
    int32_t* out = a.out_tokens + rb * a.total_blocks * B + (size_t)r.first * B;
    for (int e = threadIdx.x; e < shift; e += blockDim.x) out[e] = a.tokens[base + e];
  }
  if (r.persisted > 0 || r.n_win_new != r.n_win_old) {
    const int kept = (r.n_win_old - r.persisted) * B;  // rows that stay, moved to the front
    const int live = r.n_win_new * B;                   // rows of the next pass
    const int span = max(r.n_win_old, r.n_win_new) * B; // rows that may change
    // Destinations precede sources, so reading a chunk before any thread
    // writes it (the barrier) keeps every later source intact.
    for (int c = 0; c < span; c += blockDim.x) {
      const int d = c + threadIdx.x;
      uint8_t m = D2F_COMMITTED;
      int32_t t = a.mask_token_id;
      if (d < kept) {
        m = a.mask_state[base + d + shift];
        t = a.tokens[base + d + shift];
      } else if (d < live) {
        m = D2F_MASKED;
      }
      __syncthreads();
      if (d < span) {
        a.mask_state[base + d] = m;
        a.tokens[base + d] = t;
      }
    }
  }
  for (int k = threadIdx.x; k < a.max_win; k += blockDim.x)
    a.block_phase[rb * a.max_win + k] =
        k < r.n_win_new ? (uint8_t)((r.phase_bits >> k) & 1u) : (uint8_t)D2F_CONSERVATIVE;
  if (a.page_table != nullptr && threadIdx.x == 0) {
    // Paged: the persisted blocks' pages join the page table in order, the
    // window's page list moves up, an appended block takes its new page, and
    // slots past the window hold -1.  A handful of integers, one thread, in an
    // order that reads every entry before it is overwritten.
    int32_t* w = a.win_pages + rb * a.max_win;
    int32_t* t = a.page_table + rb * a.table_stride + r.prefix / B;
    for (int j = 0; j < r.persisted; ++j) t[j] = w[j];
    const int kept_blocks = r.n_win_old - r.persisted;
    for (int k = 0; k < kept_blocks; ++k) w[k] = w[k + r.persisted];
    if (r.n_win_new > kept_blocks) w[r.n_win_new - 1] = r.new_page;
    for (int k = max(r.n_win_new, kept_blocks); k < a.max_win; ++k) w[k] = -1;
  }
  if (threadIdx.x == 0 && a.prefix_dev != nullptr) a.prefix_dev[rb] = r.prefix + shift;
}

template <bool VEC16>
__global__ __launch_bounds__(256) void decode_advance_kernel(const AdvArgs a) {
  if ((int)blockIdx.x < a.n_copy_wgs) copy_blocks<VEC16>(a, blockIdx.x);
  else advance_window(a, (int)blockIdx.x - a.n_copy_wgs);
}

}  // namespace

hipError_t launch_decode_advance(const AdvArgs& a, hipStream_t s) {
  const size_t esz = (size_t)a.esize;
  const size_t head_w = (size_t)a.wmax * a.head_dim * esz, head_c = (size_t)a.cap * a.head_dim * esz;
  const size_t lw = (size_t)a.win_layer_stride * esz, lc = (size_t)a.cache_layer_stride * esz;
  bool vec16 = head_w % 16 == 0 && head_c % 16 == 0 &&
               (a.n_layers == 1 || (lw % 16 == 0 && lc % 16 == 0)) &&
               (uintptr_t)a.kw % 16 == 0 && (uintptr_t)a.vw % 16 == 0 &&
               (uintptr_t)a.kc % 16 == 0 && (uintptr_t)a.vc % 16 == 0;
  for (int i = 0; i < a.n_req && vec16; ++i) {
    const size_t nbytes = (size_t)a.req[i].persisted * a.bsz * a.head_dim * esz;
    const size_t off = (size_t)a.req[i].prefix * a.head_dim * esz;
    vec16 = nbytes % 16 == 0 && off % 16 == 0;
  }
  const dim3 grid(a.n_copy_wgs + a.n_req), block(256);
  if (vec16) hipLaunchKernelGGL(decode_advance_kernel<true>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(decode_advance_kernel<false>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace d2f

using namespace d2f;

namespace {

// The step's bookkeeping for contiguous (paged == false) or paged caches.
d2f_status_t advance_impl(const d2f_attn_desc_t* desc, int32_t n_layers, void* k_cache,
                          void* v_cache, int64_t cache_layer_stride, const void* k_win,
                          const void* v_win, int64_t win_layer_stride, int32_t* page_table,
                          int32_t table_stride, int32_t* win_pages, const int32_t* new_pages_host,
                          const d2f_window_params_t* params, d2f_window_t* windows_host,
                          int32_t* prefix_len_host, int32_t* prefix_len_dev,
                          const int32_t* n_committed, uint8_t* mask_state, int32_t* tokens,
                          uint8_t* block_phase, int32_t* out_tokens, int32_t mask_token_id,
                          int32_t* persisted_host, int32_t* appended_host, d2f_stream_t stream,
                          bool paged) {
  d2f_status_t st = check_desc(desc);
  if (st != D2F_OK) return st;
  if (params == nullptr) return fail(D2F_ERR_INVALID_ARG, "window params are NULL");
  if (params->block_size != desc->block_size || params->max_win_blocks != desc->max_win_blocks)
    return fail(D2F_ERR_INVALID_ARG,
                "window params (block %d, window %d) differ from the desc (block %d, window %d)",
                params->block_size, params->max_win_blocks, desc->block_size,
                desc->max_win_blocks);
  if (params->max_win_blocks > D2F_MAX_WINDOW || params->total_blocks < 1)
    return fail(D2F_ERR_INVALID_ARG, "window params out of range (window %d, total %d)",
                params->max_win_blocks, params->total_blocks);
  if (n_layers < 1) return fail(D2F_ERR_INVALID_ARG, "n_layers %d < 1", n_layers);
  if (desc->batch == 0) return D2F_OK;
  if (windows_host == nullptr || prefix_len_host == nullptr || n_committed == nullptr ||
      mask_state == nullptr || tokens == nullptr || block_phase == nullptr ||
      out_tokens == nullptr || persisted_host == nullptr || appended_host == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "a required pointer is NULL");
  if (paged) {
    if (page_table == nullptr || win_pages == nullptr || new_pages_host == nullptr ||
        table_stride < 1)
      return fail(D2F_ERR_INVALID_ARG, "page table, window pages or new pages are missing");
  } else if (k_cache == nullptr || v_cache == nullptr || k_win == nullptr || v_win == nullptr) {
    return fail(D2F_ERR_INVALID_ARG, "a required pointer is NULL");
  }
  const int nb = desc->batch, B = desc->block_size, mw = desc->max_win_blocks;
  const long long wmax = (long long)mw * B;
  if (!paged) {
    const long long cache_layer = (long long)nb * desc->n_heads_kv * desc->cache_capacity *
                                  desc->head_dim;
    const long long win_layer = (long long)nb * desc->n_heads_kv * wmax * desc->head_dim;
    if (n_layers > 1 && (cache_layer_stride < cache_layer || win_layer_stride < win_layer))
      return fail(D2F_ERR_INVALID_ARG, "layer strides smaller than one layer");
    // A copy workgroup indexes its kCopySlices slices of at most Wmax rows with
    // 32-bit counters of 2-byte elements.
    if ((unsigned long long)wmax * desc->head_dim * (desc->dtype == D2F_BF16 ? 2 : 4) / 2 *
            kCopySlices >= (1ULL << 32))
      return fail(D2F_ERR_UNSUPPORTED, "window too large for the append copy");
  }
  if ((long long)params->total_blocks * B > (1LL << 30))
    return fail(D2F_ERR_INVALID_ARG, "total_blocks * block_size too large");
  for (int b = 0; b < nb; ++b) {
    const d2f_window_t& w = windows_host[b];
    if (prefix_len_host[b] < 0)
      return fail(D2F_ERR_INVALID_ARG, "prefix_len[%d] = %d < 0", b, prefix_len_host[b]);
    if (paged && prefix_len_host[b] % B != 0)
      return fail(D2F_ERR_INVALID_ARG, "prefix_len[%d] = %d is not a whole number of blocks", b,
                  prefix_len_host[b]);
    if (w.persisted < params->total_blocks &&
        (w.first < 0 || w.n_win < 1 || w.n_win > mw || w.first + w.n_win != w.started ||
         w.started > params->total_blocks))
      return fail(D2F_ERR_INVALID_ARG, "window state of request %d is inconsistent", b);
  }

  // The one device-to-host transfer of the step: per-block commit counts.
  std::vector<int32_t> nc((size_t)nb * mw);
  hipError_t e = hipMemcpyAsync(nc.data(), n_committed, nc.size() * sizeof(int32_t),
                                hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reading n_committed");

  // Schedule on copies; the caller's state changes only once everything passed.
  std::vector<d2f_window_t> win(windows_host, windows_host + nb);
  std::vector<int32_t> pers(nb, 0), app(nb, 0);
  for (int b = 0; b < nb; ++b) {
    if (win[b].persisted >= params->total_blocks) continue;  // finished request
    st = d2f_window_after_commit(params, &win[b], &nc[(size_t)b * mw], &pers[b], &app[b]);
    if (st != D2F_OK) return st;
    if (paged) {
      if (prefix_len_host[b] / B + pers[b] > table_stride)
        return fail(D2F_ERR_CAPACITY, "request %d: page table full (%d + %d > %d)", b,
                    prefix_len_host[b] / B, pers[b], table_stride);
      if (app[b] && new_pages_host[b] < 0)
        return fail(D2F_ERR_INVALID_ARG, "request %d appends a block but has no new page", b);
    } else if ((long long)prefix_len_host[b] + (long long)pers[b] * B > desc->cache_capacity) {
      return fail(D2F_ERR_CAPACITY, "request %d: cache full (%d + %d > %lld)", b,
                  prefix_len_host[b], pers[b] * B, (long long)desc->cache_capacity);
    }
  }

  const int esz = desc->dtype == D2F_BF16 ? 2 : 4;
  for (int b0 = 0; b0 < nb; b0 += kMaxReqPerLaunch) {
    AdvArgs a{};
    a.kc = k_cache;
    a.vc = v_cache;
    a.kw = k_win;
    a.vw = v_win;
    a.cache_layer_stride = cache_layer_stride;
    a.win_layer_stride = win_layer_stride;
    a.cap = desc->cache_capacity;
    a.mask_state = mask_state;
    a.tokens = tokens;
    a.block_phase = block_phase;
    a.out_tokens = out_tokens;
    a.prefix_dev = prefix_len_dev;
    a.n_layers = n_layers;
    a.hkv = desc->n_heads_kv;
    a.head_dim = desc->head_dim;
    a.bsz = B;
    a.esize = esz;
    a.wmax = (int32_t)wmax;
    a.max_win = mw;
    a.total_blocks = params->total_blocks;
    a.n_req = std::min(kMaxReqPerLaunch, nb - b0);
    a.req0 = b0;
    a.mask_token_id = mask_token_id;
    a.page_table = paged ? page_table : nullptr;
    a.win_pages = paged ? win_pages : nullptr;
    a.table_stride = table_stride;
    int copies = 0;
    for (int i = 0; i < a.n_req; ++i) {
      const int b = b0 + i;
      AdvReq& r = a.req[i];
      const bool done_before = windows_host[b].persisted >= params->total_blocks;
      r.persisted = pers[b];
      r.prefix = prefix_len_host[b];
      r.first = windows_host[b].first;
      r.n_win_old = done_before ? 0 : windows_host[b].n_win;
      r.n_win_new = done_before ? 0 : win[b].n_win;
      r.phase_bits = 0;
      for (int k = 0; k < r.n_win_new; ++k)
        if (win[b].phase[k] == D2F_AGGRESSIVE) r.phase_bits |= 1ull << k;
      r.copy_base = copies;
      r.new_page = paged ? new_pages_host[b] : -1;
      if (!paged && r.persisted > 0) copies += copy_workgroups(n_layers, desc->n_heads_kv);
    }
    a.n_copy_wgs = copies;
    e = launch_decode_advance(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode advance launch");
  }

  for (int b = 0; b < nb; ++b) {
    windows_host[b] = win[b];
    prefix_len_host[b] += pers[b] * B;
    persisted_host[b] = pers[b];
    appended_host[b] = app[b];
  }
  return D2F_OK;
}

}  // namespace

extern "C" d2f_status_t d2f_decode_advance(
    const d2f_attn_desc_t* desc, int32_t n_layers, void* k_cache, void* v_cache,
    int64_t cache_layer_stride, const void* k_win, const void* v_win, int64_t win_layer_stride,
    const d2f_window_params_t* params, d2f_window_t* windows_host, int32_t* prefix_len_host,
    int32_t* prefix_len_dev, const int32_t* n_committed, uint8_t* mask_state, int32_t* tokens,
    uint8_t* block_phase, int32_t* out_tokens, int32_t mask_token_id, int32_t* persisted_host,
    int32_t* appended_host, d2f_stream_t stream) {
  return advance_impl(desc, n_layers, k_cache, v_cache, cache_layer_stride, k_win, v_win,
                      win_layer_stride, nullptr, 0, nullptr, nullptr, params, windows_host,
                      prefix_len_host, prefix_len_dev, n_committed, mask_state, tokens,
                      block_phase, out_tokens, mask_token_id, persisted_host, appended_host,
                      stream, false);
}

extern "C" d2f_status_t d2f_decode_advance_paged(
    const d2f_attn_desc_t* desc, int32_t* page_table, int32_t table_stride, int32_t* win_pages,
    const int32_t* new_pages_host, const d2f_window_params_t* params, d2f_window_t* windows_host,
    int32_t* prefix_len_host, int32_t* prefix_len_dev, const int32_t* n_committed,
    uint8_t* mask_state, int32_t* tokens, uint8_t* block_phase, int32_t* out_tokens,
    int32_t mask_token_id, int32_t* persisted_host, int32_t* appended_host,
    d2f_stream_t stream) {
  return advance_impl(desc, 1, nullptr, nullptr, 0, nullptr, nullptr, 0, page_table,
                      table_stride, win_pages, new_pages_host, params, windows_host,
                      prefix_len_host, prefix_len_dev, n_committed, mask_state, tokens,
                      block_phase, out_tokens, mask_token_id, persisted_host, appended_host,
                      stream, true);
}
