// Exact merge of key-range splits of the window attention.
//
// A split s of a row's keys leaves an unnormalised output O_s, its running
// maximum m_s (base-2 scaled scores) and sum l_s.  The softmax over the union
// of the splits is recovered exactly by weighting each part by 2^(m_s - m)
// with m = max_s m_s: O = sum_s O_s 2^(m_s - m) / sum_s l_s 2^(m_s - m), and
// LSE = (m + log2 sum_s l_s 2^(m_s - m)) ln 2 (the log-space composition of
// partial attention outputs, [dLLM-survey] section "FlashBlock: 블록 외부
// 어텐션 캐싱").  A split that saw no visible key has m_s = -inf and weight 0.
//
// One workgroup per (request, KV head, query tile); four threads per row,
// each owning a contiguous quarter of head_dim.  Splits are combined in a
// fixed order, so the result is deterministic.
#include "d2f_internal.h"

namespace d2f {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

template <typename T> __device__ __forceinline__ T to_out(float x);
template <> __device__ __forceinline__ float to_out<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 to_out<__bf16>(float x) { return (__bf16)x; }

template <int D, typename OutT>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnArgs a) {
  const int g = blockIdx.x;
  const int ri = find_req_group(a, g);
  const int nsplit = a.req[ri].nsplit;
  if (nsplit == 1) return;
  const int rb = a.req[ri].b, W = a.req[ri].win, qtiles = a.req[ri].qtiles;
  const int local = g - a.req[ri].group_base;
  const int qt = local % qtiles, kvh = local / qtiles;
  const int G = a.group;
  const int r = threadIdx.x >> 2, sub = threadIdx.x & 3;
  const int row = qt * kQTile + r;
  if (row >= G * W) return;
  const int i = row / G, h = kvh * G + row % G;

  auto slot = [&](int s) {
    return ((size_t)(a.req[ri].unit_base + (kvh * nsplit + s) * qtiles + qt)) * kQTile + r;
  };
  float m = kNegInf;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, a.ws_ml[slot(s) * 2]);
  constexpr int DQ = D / 4;
  float acc[DQ];
#pragma unroll
  for (int k = 0; k < DQ; ++k) acc[k] = 0.f;
  float l = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const size_t sl = slot(s);
    const float ms = a.ws_ml[sl * 2];
    if (ms == kNegInf) continue;
    const float w = exp2f(ms - m);
    l = fmaf(a.ws_ml[sl * 2 + 1], w, l);
    const float4* src = (const float4*)(a.ws_o + sl * D + sub * DQ);
#pragma unroll
    for (int k = 0; k < DQ / 4; ++k) {
      const float4 v = src[k];
      acc[4 * k + 0] = fmaf(v.x, w, acc[4 * k + 0]);
      acc[4 * k + 1] = fmaf(v.y, w, acc[4 * k + 1]);
      acc[4 * k + 2] = fmaf(v.z, w, acc[4 * k + 2]);
      acc[4 * k + 3] = fmaf(v.w, w, acc[4 * k + 3]);
    }
  }
  const float inv = 1.0f / l;
  OutT* op = (OutT*)a.out + (((size_t)rb * a.hq + h) * a.wmax + i) * D + sub * DQ;
#pragma unroll
  for (int k = 0; k < DQ; ++k) op[k] = to_out<OutT>(acc[k] * inv);
  if (a.lse != nullptr && sub == 0)
    a.lse[((size_t)rb * a.hq + h) * a.wmax + i] = (m + log2f(l)) * kLn2;
}

}  // namespace

hipError_t launch_attn_merge(const AttnArgs& a, int head_dim, d2f_dtype_t dt, hipStream_t s) {
  const dim3 grid(a.n_groups), block(256);
  if (dt == D2F_BF16) {
    if (head_dim == 128) hipLaunchKernelGGL((attn_merge_kernel<128, __bf16>), grid, block, 0, s, a);
    else if (head_dim == 64) hipLaunchKernelGGL((attn_merge_kernel<64, __bf16>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((attn_merge_kernel<128, float>), grid, block, 0, s, a);
    else if (head_dim == 64) hipLaunchKernelGGL((attn_merge_kernel<64, float>), grid, block, 0, s, a);
    else if (head_dim == 32) hipLaunchKernelGGL((attn_merge_kernel<32, float>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace d2f
