// Exact composition of two attention results over disjoint key sets.
//
// [dLLM-survey] section "FlashBlock: 블록 외부 어텐션 캐싱": the attention over
// the keys outside a block and over the keys inside it can be computed apart
// and joined in log space, as FlashAttention joins its tiles.  For one query
// row with results (O_a, L_a) and (O_b, L_b) (L = natural-log normaliser):
//   L = log(e^L_a + e^L_b),  O = (O_a e^(L_a - L) + O_b e^(L_b - L)).
// A side with L = -inf (no keys) has weight 0.
#include "d2f_internal.h"

namespace d2f {
namespace {

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<__bf16>(const __bf16* p) { return (float)*p; }
template <typename T> __device__ __forceinline__ void st(T* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<__bf16>(__bf16* p, float v) { *p = (__bf16)v; }

// One workgroup per (request, head, 16 rows); 16 threads per row, each
// owning D / 16 dims.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  constexpr int TPR = 16, DPT = D / TPR;
  const int rows_per_wg = 256 / TPR;
  const int per_head = (a.wmax + rows_per_wg - 1) / rows_per_wg;
  const int i_blk = blockIdx.x % per_head;
  const int bh = blockIdx.x / per_head;
  const int h = bh % a.hq, ri = bh / a.hq;
  const int b = a.b0 + ri;
  const int i = i_blk * rows_per_wg + (int)threadIdx.x / TPR;
  const int sub = (int)threadIdx.x % TPR;
  if (i >= a.win[ri]) return;
  const size_t row = ((size_t)b * a.hq + h) * a.wmax + i;
  const float la = a.lse_a[row], lb = a.lse_b[row];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, L = m;
  if (m != -__builtin_inff()) {
    wa = (la == -__builtin_inff()) ? 0.f : expf(la - m);
    wb = (lb == -__builtin_inff()) ? 0.f : expf(lb - m);
    const float s = wa + wb;
    L = m + logf(s);
    wa /= s;
    wb /= s;
  }
  const T* pa = (const T*)a.out_a + row * D + sub * DPT;
  const T* pb = (const T*)a.out_b + row * D + sub * DPT;
  T* po = (T*)a.out + row * D + sub * DPT;
  float v[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) v[k] = wa * ld<T>(pa + k) + wb * ld<T>(pb + k);
#pragma unroll
  for (int k = 0; k < DPT; ++k) st<T>(po + k, v[k]);
  if (sub == 0) a.lse[row] = L;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int head_dim, d2f_dtype_t dt, hipStream_t s) {
  const int per_head = (a.wmax + 15) / 16;
  const dim3 grid((unsigned)(a.n_req * a.hq * per_head)), block(256);
  if (dt == D2F_BF16 && head_dim == 128)
    hipLaunchKernelGGL((combine_kernel<__bf16, 128>), grid, block, 0, s, a);
  else if (dt == D2F_BF16 && head_dim == 64)
    hipLaunchKernelGGL((combine_kernel<__bf16, 64>), grid, block, 0, s, a);
  else if (dt == D2F_F32 && head_dim == 128)
    hipLaunchKernelGGL((combine_kernel<float, 128>), grid, block, 0, s, a);
  else if (dt == D2F_F32 && head_dim == 64)
    hipLaunchKernelGGL((combine_kernel<float, 64>), grid, block, 0, s, a);
  else if (dt == D2F_F32 && head_dim == 32)
    hipLaunchKernelGGL((combine_kernel<float, 32>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace d2f
