// Exact merge of the key-range splits of one (request, KV head, query tile).
//
// A split s of a row's keys leaves an unnormalised output O_s, its running
// maximum m_s (base-2 scaled scores) and sum l_s.  The softmax over the union
// of the splits is recovered exactly by weighting each part by 2^(m_s - m)
// with m = max_s m_s: O = sum_s O_s 2^(m_s - m) / sum_s l_s 2^(m_s - m), and
// LSE = (m + log2 sum_s l_s 2^(m_s - m)) ln 2 -- the log-space composition of
// partial attention outputs ([dLLM-survey] section "FlashBlock: 블록 외부
// 어텐션 캐싱").  A split that saw no visible key has m_s = -inf and weight 0.
// Splits are combined in a fixed order, so the result is deterministic.
#pragma once

#include "d2f_internal.h"

namespace d2f {

template <typename T> __device__ __forceinline__ T to_out(float x);
template <> __device__ __forceinline__ float to_out<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 to_out<__bf16>(float x) { return (__bf16)x; }

// 256 threads: four per row, each owning a contiguous quarter of head_dim.
template <int D, typename OutT>
__device__ void merge_group(const AttnArgs& a, int ri, int kvh, int qt) {
  constexpr float kNegInf = -__builtin_inff();
  constexpr float kLn2 = 0.693147180559945309f;
  constexpr int DQ = D / 4;
  const int nsplit = a.req[ri].nsplit, qtiles = a.req[ri].qtiles;
  const int rb = a.req[ri].b, W = a.req[ri].win;
  const int G = a.group;
  const int r = threadIdx.x >> 2, sub = threadIdx.x & 3;
  const int row = qt * kQTile + r;
  if (row >= G * W) return;
  const int i = row / G, h = kvh * G + row % G;
  const size_t slot0 = ((size_t)(a.req[ri].unit_base + kvh * nsplit * qtiles + qt)) * kQTile + r;
  const size_t sstride = (size_t)qtiles * kQTile;  // slot distance between splits

  float m = kNegInf;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, a.ws_ml[(slot0 + s * sstride) * 2]);
  float acc[DQ];
#pragma unroll
  for (int k = 0; k < DQ; ++k) acc[k] = 0.f;
  float l = 0.f;
  // Loads of the next split are independent of the current accumulation, so
  // the compiler keeps several splits' reads in flight.
#pragma unroll 2
  for (int s = 0; s < nsplit; ++s) {
    const size_t sl = slot0 + s * sstride;
    const float2 ml = *(const float2*)(a.ws_ml + sl * 2);
    const float w = (ml.x == kNegInf) ? 0.f : exp2f(ml.x - m);
    l = fmaf(ml.y, w, l);
    const float4* src = (const float4*)(a.ws_o + sl * D + sub * DQ);
    float4 v[DQ / 4];
#pragma unroll
    for (int k = 0; k < DQ / 4; ++k) v[k] = src[k];
#pragma unroll
    for (int k = 0; k < DQ / 4; ++k) {
      acc[4 * k + 0] = fmaf(v[k].x, w, acc[4 * k + 0]);
      acc[4 * k + 1] = fmaf(v[k].y, w, acc[4 * k + 1]);
      acc[4 * k + 2] = fmaf(v[k].z, w, acc[4 * k + 2]);
      acc[4 * k + 3] = fmaf(v[k].w, w, acc[4 * k + 3]);
    }
  }
  const float inv = 1.0f / l;
  OutT* op = (OutT*)a.out + (((size_t)rb * a.hq + h) * a.wmax + i) * D + sub * DQ;
#pragma unroll
  for (int k = 0; k < DQ; ++k) op[k] = to_out<OutT>(acc[k] * inv);
  if (a.lse != nullptr && sub == 0)
    a.lse[((size_t)rb * a.hq + h) * a.wmax + i] = (m + log2f(l)) * kLn2;
}

}  // namespace d2f
