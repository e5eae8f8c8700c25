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

// Rows [row0, row0 + 1024 / D) of one group; D / 4 threads per row, each
// owning 4 consecutive dims (one 16-byte load per split).  Loads of all
// splits are independent, so a thread keeps many in flight.
template <int D, typename OutT>
__device__ void merge_rows(const AttnArgs& a, int ri, int kvh, int qt, int row0) {
  constexpr float kNegInf = -__builtin_inff();
  constexpr float kLn2 = 0.693147180559945309f;
  constexpr int TPR = D / 4;  // threads per row
  const int nsplit = a.req[ri].nsplit, qtiles = a.req[ri].qtiles;
  const int rb = a.req[ri].b, W = a.req[ri].win;
  const int G = a.group;
  const int r = row0 + (int)threadIdx.x / TPR, sub = (int)threadIdx.x % TPR;
  const int row = qt * a.qrows + r;
  if (r >= a.qrows || row >= G * W) return;
  const int i = row / G, h = kvh * G + row % G;
  const size_t slot0 =
      ((size_t)(a.req[ri].unit_base + kvh * nsplit * qtiles + qt)) * a.slot_rows + r;
  const size_t sstride = (size_t)qtiles * a.slot_rows;  // slot distance between splits

  // Splits are taken kBatch at a time with all their loads in flight; a
  // batch raises the running max and rescales what was accumulated before.
  constexpr int kBatch = 16;
  float m = kNegInf, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    float2 ml[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (s0 + k < nsplit) {
        const size_t sl = slot0 + (size_t)(s0 + k) * sstride;
        ml[k] = *(const float2*)(a.ws_ml + sl * 2);
        v[k] = *(const float4*)(a.ws_o + sl * D + 4 * sub);
      } else {
        ml[k] = make_float2(kNegInf, 0.f);
        v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float mb = m;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mb = fmaxf(mb, ml[k].x);
    if (mb == kNegInf) continue;  // nothing visible so far
    const float r = (m == kNegInf) ? 0.f : exp2f(m - mb);
    l *= r;
    acc.x *= r;
    acc.y *= r;
    acc.z *= r;
    acc.w *= r;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = (ml[k].x == kNegInf) ? 0.f : exp2f(ml[k].x - mb);
      l = fmaf(ml[k].y, w, l);
      acc.x = fmaf(v[k].x, w, acc.x);
      acc.y = fmaf(v[k].y, w, acc.y);
      acc.z = fmaf(v[k].z, w, acc.z);
      acc.w = fmaf(v[k].w, w, acc.w);
    }
    m = mb;
  }
  const float inv = 1.0f / l;
  OutT* op = (OutT*)a.out + (((size_t)rb * a.hq + h) * a.wmax + i) * D + 4 * sub;
  op[0] = to_out<OutT>(acc.x * inv);
  op[1] = to_out<OutT>(acc.y * inv);
  op[2] = to_out<OutT>(acc.z * inv);
  op[3] = to_out<OutT>(acc.w * inv);
  if (a.lse != nullptr && sub == 0)
    a.lse[((size_t)rb * a.hq + h) * a.wmax + i] = (m + log2f(l)) * kLn2;
}

}  // namespace d2f
