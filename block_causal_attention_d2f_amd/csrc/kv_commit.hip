// Append the oldest window block of one request to the KV cache.
//
// [D2F-wiki] section "블록 단위 인과 어텐션": a completed block's K/V no longer
// change, so an ordinary KV cache holds them exactly; section "KV 캐시 관리
// 방식": block completion is the signal to make the entries permanent.
//
// The copy is byte-exact: for each (layer, KV head, K or V) one workgroup
// moves the block's B contiguous rows from the window to cache slots
// [P, P + B), with 16-byte accesses when every address allows it.  Workgroup
// 0 also stores the new prefix length into the optional device mirror, so it
// is ordered with the copy on the caller's stream.
#include "d2f_internal.h"

namespace d2f {
namespace {

template <bool VEC16>
__global__ __launch_bounds__(256) void kv_commit_kernel(const KvArgs a) {
  const int idx = blockIdx.x;
  const int which = idx & 1;
  const int lh = idx >> 1;
  const int layer = lh / a.hkv, head = lh % a.hkv;
  const size_t esz = (size_t)a.esize;
  const size_t nbytes = (size_t)a.bsz * a.head_dim * esz;
  const char* src = (const char*)(which ? a.vw : a.kw) +
                    ((size_t)layer * a.win_layer_stride +
                     ((size_t)a.request * a.hkv + head) * (size_t)a.wmax * a.head_dim) * esz;
  char* dst = (char*)(which ? a.vc : a.kc) +
              ((size_t)layer * a.cache_layer_stride +
               (((size_t)a.request * a.hkv + head) * (size_t)a.cap + a.prefix) * a.head_dim) * esz;
  if (VEC16) {
    const uint4* s4 = (const uint4*)src;
    uint4* d4 = (uint4*)dst;
    for (size_t e = threadIdx.x; e < nbytes / 16; e += blockDim.x) d4[e] = s4[e];
  } else {
    const uint16_t* s2 = (const uint16_t*)src;
    uint16_t* d2 = (uint16_t*)dst;
    for (size_t e = threadIdx.x; e < nbytes / 2; e += blockDim.x) d2[e] = s2[e];
  }
  if (idx == 0 && threadIdx.x == 0 && a.prefix_dev != nullptr) a.prefix_dev[a.request] = a.new_prefix;
}

// Paged persist: the page of the oldest window block joins the request's
// page table at slot `slot` and the window's page list moves up by one (its
// last entry becomes -1, to be filled by the caller when a block is
// appended).  One thread: a handful of integers.
__global__ __launch_bounds__(64) void kv_commit_paged_kernel(int32_t* table, int32_t* win,
                                                             int32_t* prefix_dev, int b, int ts,
                                                             int mw, int slot, int new_prefix) {
  if (threadIdx.x != 0) return;
  int32_t* w = win + (size_t)b * mw;
  const int32_t first = w[0];
  for (int k = 0; k + 1 < mw; ++k) w[k] = w[k + 1];
  w[mw - 1] = -1;
  table[(size_t)b * ts + slot] = first;
  if (prefix_dev != nullptr) prefix_dev[b] = new_prefix;
}

}  // namespace

hipError_t launch_kv_commit_paged(int32_t* table, int32_t* win, int32_t* prefix_dev, int b,
                                  int ts, int mw, int slot, int new_prefix, hipStream_t s) {
  hipLaunchKernelGGL(kv_commit_paged_kernel, dim3(1), dim3(64), 0, s, table, win, prefix_dev, b,
                     ts, mw, slot, new_prefix);
  return hipGetLastError();
}

hipError_t launch_kv_commit(const KvArgs& a, hipStream_t s) {
  const size_t esz = (size_t)a.esize;
  const size_t nbytes = (size_t)a.bsz * a.head_dim * esz;
  const uintptr_t src_off = (uintptr_t)(((size_t)a.request * a.hkv) * (size_t)a.wmax * a.head_dim * esz);
  const uintptr_t dst_off =
      (uintptr_t)((((size_t)a.request * a.hkv) * (size_t)a.cap + a.prefix) * a.head_dim * esz);
  const size_t head_w = (size_t)a.wmax * a.head_dim * esz, head_c = (size_t)a.cap * a.head_dim * esz;
  const size_t lw = (size_t)a.win_layer_stride * esz, lc = (size_t)a.cache_layer_stride * esz;
  const bool vec16 = nbytes % 16 == 0 && head_w % 16 == 0 && head_c % 16 == 0 &&
                     (a.n_layers == 1 || (lw % 16 == 0 && lc % 16 == 0)) &&
                     ((uintptr_t)a.kw + src_off) % 16 == 0 && ((uintptr_t)a.vw + src_off) % 16 == 0 &&
                     ((uintptr_t)a.kc + dst_off) % 16 == 0 && ((uintptr_t)a.vc + dst_off) % 16 == 0;
  const dim3 grid(2 * a.n_layers * a.hkv), block(256);
  if (vec16) hipLaunchKernelGGL(kv_commit_kernel<true>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(kv_commit_kernel<false>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace d2f
