// Confidence pass over the vocabulary logits and the block commit rule.
//
// [D2F-review] section "쉽게 이해하기": a newly added (conservative) block
// commits only positions whose confidence exceeds the threshold; an
// aggressive block also commits its relatively most confident positions;
// what is not committed is masked again.  [dLLM-survey] "답을 미리 안다:
// 조기 확정 디코딩(Prophet)": the confidence is the maximum softmax
// probability, and "양방향 어텐션과 사라진 KV 캐시": low-confidence remasking.
//
// Kernel 1 (vocab_reduce): one workgroup per (row, chunk of 8192 logits).  A
// MASKED row's chunk is streamed once from HBM with 16-byte loads (8 per
// thread, all in flight together); every thread takes the max of its 32
// values and the sum of exp(x - max), the workgroup reduces the max,
// rescales and reduces the sums (wavefront shuffles, then a fixed-order
// cross-wave step), and the threads holding the maximum agree on its first
// index.  COMMITTED rows are not read.
//
// Kernel 2 (commit_decide): one workgroup per D2F block.  A thread per row
// merges the row's chunk partials (loads in flight together, folded in chunk
// order), conf = 1 / sum (the max term is exp(0) = 1) is
// compared with the threshold, the aggressive top-k ranks the block's masked
// rows (ties to the lower position), and the new mask state, tokens and
// per-block counts are written.  No floating-point atomics: results are
// deterministic.
#include <climits>

#include "d2f_internal.h"

namespace d2f {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPerThread = kCommitChunk / kCommitThreads;  // 32 logits per thread
constexpr int kWaves = kCommitThreads / 64;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Merge two (max, sum, first index) partials of disjoint index ranges.
__device__ __forceinline__ void combine(float& m, float& s, int& i, float m2, float s2, int i2) {
  const float mm = fmaxf(m, m2);
  const int ii = (m > m2) ? i : (m2 > m) ? i2 : min(i, i2);
  float ss = 0.f;
  if (mm != kNegInf)
    ss = s * __builtin_amdgcn_exp2f((m - mm) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mm) * kLog2e);
  m = mm;
  s = ss;
  i = ii;
}

// Reduce one chunk of one row; returns (max, sum, first argmax) in thread 0.
template <bool VEC>
__device__ void reduce_chunk(const CommitArgs& a, int row, int ck, float4& result) {
  __shared__ float sh_m[kWaves], sh_s[kWaves];
  __shared__ int sh_i;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = ck * kCommitChunk;
  const int n = min(kCommitChunk, a.vocab - c0);
  const float* src = a.logits + (size_t)row * a.ld + c0;

  // x[4k + c] is logit 4 * (tid + 256 k) + c (vector path) or tid + 256 k.
  float x[kPerThread];
  if (VEC && n == kCommitChunk) {
#pragma unroll
    for (int k = 0; k < kPerThread / 4; ++k) {
      const float4 v = *(const float4*)(src + 4 * (tid + kCommitThreads * k));
      x[4 * k + 0] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
    }
  } else if (VEC) {
#pragma unroll
    for (int k = 0; k < kPerThread / 4; ++k) {
      const int e0 = 4 * (tid + kCommitThreads * k);
      if (e0 + 3 < n) {
        const float4 v = *(const float4*)(src + e0);
        x[4 * k + 0] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) x[4 * k + c] = (e0 + c < n) ? src[e0 + c] : kNegInf;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int e = tid + kCommitThreads * k;
      x[k] = (e < n) ? src[e] : kNegInf;
    }
  }
  float m = kNegInf;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) m = fmaxf(m, x[k]);
  // exp(x - m) as 2^((x - m) log2 e): the difference is exact for the terms
  // near the maximum that dominate the sum, so their relative error stays at
  // a few ulp (folding m * log2 e into one fma would shift every term of the
  // thread by the rounding of that product instead).
  float s = 0.f;
  if (m != kNegInf) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) s += __builtin_amdgcn_exp2f((x[k] - m) * kLog2e);
  }
  // Workgroup maximum.
  const float wm = wave_max(m);
  if (lane == 0) sh_m[wave] = wm;
  if (tid == 0) sh_i = INT_MAX;
  __syncthreads();
  float M = sh_m[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh_m[w]);
  // First index of the maximum: only threads holding it search.
  if (m == M && M != kNegInf) {
    int first = INT_MAX;
#pragma unroll
    for (int k = kPerThread - 1; k >= 0; --k) {
      const int idx = VEC ? 4 * (tid + kCommitThreads * (k >> 2)) + (k & 3)
                          : tid + kCommitThreads * k;
      if (x[k] == M) first = idx;
    }
    atomicMin(&sh_i, c0 + first);  // integer minimum: order-independent
  }
  // Sums rescaled to the workgroup maximum, then reduced in a fixed order.
  const float sr = (M == kNegInf || m == kNegInf) ? 0.f
                                                  : s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
  const float ws = wave_sum(sr);
  if (lane == 0) sh_s[wave] = ws;
  __syncthreads();
  if (tid == 0) {
    float S = sh_s[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) S += sh_s[w];
    result = make_float4(M, S, __int_as_float(sh_i), 0.f);
  }
}

// Combine the chunk partials of every row of one block into s_conf / s_idx:
// one thread per row loads kBatch partials at a time, all in flight, and
// folds them in chunk order (a fixed order: the result does not depend on
// timing).  The loads do not wait for the mask state: a row that is not
// MASKED has no partials written, and what is read for it is discarded.
__device__ void combine_rows(const CommitArgs& a, size_t row0, int B, float* s_conf, int* s_idx) {
  constexpr int kBatch = 16;
  const int nck = a.n_chunks;
  for (int p = threadIdx.x; p < B; p += kCommitThreads) {
    const bool live = a.mask_state[row0 + p] == D2F_MASKED;
    const float4* src = a.partial + (row0 + p) * nck;
    float m = kNegInf, sm = 0.f;
    int ix = INT_MAX;
    for (int c0 = 0; c0 < nck; c0 += kBatch) {
      float4 v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        v[k] = (c0 + k < nck) ? src[c0 + k] : make_float4(kNegInf, 0.f, __int_as_float(INT_MAX), 0.f);
#pragma unroll
      for (int k = 0; k < kBatch; ++k) combine(m, sm, ix, v[k].x, v[k].y, __float_as_int(v[k].z));
    }
    s_conf[p] = live ? 1.0f / sm : 0.f;
    s_idx[p] = live ? ix : -1;
  }
}

__global__ __launch_bounds__(kCommitThreads) void commit_decide_kernel(const CommitArgs a) {
  __shared__ float s_conf[kMaxCommitBlock];
  __shared__ int s_idx[kMaxCommitBlock];
  __shared__ unsigned char s_live[kMaxCommitBlock];
  __shared__ int s_cnt, s_incomplete;
  const int blk = blockIdx.x;
  const int B = a.block_size;
  const size_t row0 = (size_t)blk * B;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_cnt = 0;
    s_incomplete = 0;
  }
  for (int p = tid; p < B; p += kCommitThreads) s_live[p] = a.mask_state[row0 + p] == D2F_MASKED;
  combine_rows(a, row0, B, s_conf, s_idx);
  __syncthreads();
  const bool aggressive = a.block_phase[blk] == D2F_AGGRESSIVE && a.k_aggr > 0;
  int cnt = 0, incomplete = 0;
  for (int p = tid; p < B; p += kCommitThreads) {
    if (!s_live[p]) continue;
    const float c = s_conf[p];
    bool commit = c > a.tau;
    if (!commit && aggressive) {
      int rank = 0;
      for (int q = 0; q < B && rank < a.k_aggr; ++q)
        if (s_live[q] && (s_conf[q] > c || (s_conf[q] == c && q < p))) ++rank;
      commit = rank < a.k_aggr;
    }
    const size_t row = row0 + p;
    if (a.conf_out) a.conf_out[row] = c;
    if (a.argmax_out) a.argmax_out[row] = s_idx[p];
    if (commit) {
      a.mask_state[row] = D2F_COMMITTED;
      a.tokens[row] = s_idx[p];
      ++cnt;
    } else {
      a.tokens[row] = a.mask_token_id;
      incomplete = 1;
    }
  }
  if (cnt) atomicAdd(&s_cnt, cnt);            // integer: order-independent
  if (incomplete) atomicOr(&s_incomplete, 1);
  __syncthreads();
  if (tid == 0) {
    a.n_committed[blk] = s_cnt;
    a.block_complete[blk] = s_incomplete ? 0 : 1;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kCommitThreads) void vocab_reduce_kernel(const CommitArgs a) {
  const int row = blockIdx.x / a.n_chunks;
  const int ck = blockIdx.x - row * a.n_chunks;
  if (a.mask_state[row] != D2F_MASKED) return;
  float4 part;
  reduce_chunk<VEC>(a, row, ck, part);
  if (threadIdx.x == 0) a.partial[(size_t)row * a.n_chunks + ck] = part;
}

}  // namespace

hipError_t launch_confidence_commit(const CommitArgs& a, bool vec4, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  const long long grid = (long long)a.n_rows * a.n_chunks;
  if (vec4)
    hipLaunchKernelGGL(vocab_reduce_kernel<true>, dim3((unsigned)grid), dim3(kCommitThreads), 0, s,
                       a);
  else
    hipLaunchKernelGGL(vocab_reduce_kernel<false>, dim3((unsigned)grid), dim3(kCommitThreads), 0,
                       s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_decide_kernel, dim3(a.n_rows / a.block_size), dim3(kCommitThreads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace d2f
