// Confidence pass over the vocabulary logits and the block commit rule.
//
// [D2F-review] section "쉽게 이해하기": a newly added (conservative) block
// commits only positions whose confidence exceeds the threshold; an
// aggressive block also commits its relatively most confident positions;
// what is not committed is masked again.  [dLLM-survey] "답을 미리 안다:
// 조기 확정 디코딩(Prophet)": the confidence is the maximum softmax
// probability, and "양방향 어텐션과 사라진 KV 캐시": low-confidence remasking.
//
// Kernel 1 (vocab_reduce) streams each MASKED row once from HBM.  A row is
// cut into chunks of 8192 logits, one workgroup per (row, chunk); every
// thread loads its 32 values with 16-byte loads, forms its own (max, first
// argmax, sum of exp(x - max)), and the workgroup combines them with 64-wide
// wavefront shuffles and a fixed-order cross-wave step.  Rows already
// COMMITTED are skipped without reading their logits.
//
// Kernel 2 (commit_decide), one wavefront per D2F block, merges a row's
// chunk partials in chunk order, takes conf = 1 / sum (the max term is
// exp(0) = 1), compares with the float threshold, ranks the block's masked
// rows for the aggressive top-k (ties to the lower position), and writes the
// new mask state, tokens and per-block counts.  No floating-point atomics:
// the result is deterministic.
#include <climits>

#include "d2f_internal.h"

namespace d2f {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

struct Part {
  float m;  // running max
  float s;  // sum of exp(x - m)
  int i;    // first index attaining m
};

__device__ __forceinline__ Part combine(Part a, Part b) {
  Part r;
  r.m = fmaxf(a.m, b.m);
  r.i = (a.m > b.m) ? a.i : (b.m > a.m) ? b.i : min(a.i, b.i);
  if (r.m == kNegInf) {
    r.s = 0.f;
  } else {
    r.s = a.s * __builtin_amdgcn_exp2f((a.m - r.m) * kLog2e) +
          b.s * __builtin_amdgcn_exp2f((b.m - r.m) * kLog2e);
  }
  return r;
}

__device__ __forceinline__ Part shfl_xor_part(Part p, int o) {
  Part q;
  q.m = __shfl_xor(p.m, o);
  q.s = __shfl_xor(p.s, o);
  q.i = __shfl_xor(p.i, o);
  return q;
}

constexpr int kPerThread = kCommitChunk / kCommitThreads;  // 32 logits per thread

template <bool VEC>
__global__ __launch_bounds__(kCommitThreads) void vocab_reduce_kernel(const CommitArgs a) {
  const int row = blockIdx.x / a.n_chunks;
  const int ck = blockIdx.x - row * a.n_chunks;
  if (a.mask_state[row] != D2F_MASKED) return;
  const int c0 = ck * kCommitChunk;
  const int n = min(kCommitChunk, a.vocab - c0);
  const float* src = a.logits + (size_t)row * a.ld + c0;
  const int tid = threadIdx.x;

  float x[kPerThread];
  int base[kPerThread];  // chunk-relative index of x[e]
  if (VEC) {
    // float4 number q = tid + 256 * k covers logits 4q .. 4q + 3.
#pragma unroll
    for (int k = 0; k < kPerThread / 4; ++k) {
      const int e0 = 4 * (tid + kCommitThreads * k);
      float4 v;
      if (e0 + 3 < n) {
        v = *(const float4*)(src + e0);
      } else {
        v.x = (e0 + 0 < n) ? src[e0 + 0] : kNegInf;
        v.y = (e0 + 1 < n) ? src[e0 + 1] : kNegInf;
        v.z = (e0 + 2 < n) ? src[e0 + 2] : kNegInf;
        v.w = (e0 + 3 < n) ? src[e0 + 3] : kNegInf;
      }
      x[4 * k + 0] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
      base[4 * k + 0] = e0; base[4 * k + 1] = e0 + 1; base[4 * k + 2] = e0 + 2;
      base[4 * k + 3] = e0 + 3;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int e = tid + kCommitThreads * k;
      x[k] = (e < n) ? src[e] : kNegInf;
      base[k] = e;
    }
  }
  // Thread-local max and first argmax (x[] is in increasing index order).
  Part p;
  p.m = kNegInf;
  p.i = INT_MAX;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    if (x[k] > p.m) {
      p.m = x[k];
      p.i = c0 + base[k];
    }
  }
  p.s = 0.f;
  if (p.m != kNegInf) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) p.s += __builtin_amdgcn_exp2f((x[k] - p.m) * kLog2e);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) p = combine(p, shfl_xor_part(p, o));

  __shared__ Part wp[kCommitThreads / 64];
  if ((tid & 63) == 0) wp[tid >> 6] = p;
  __syncthreads();
  if (tid == 0) {
    Part t = wp[0];
#pragma unroll
    for (int w = 1; w < kCommitThreads / 64; ++w) t = combine(t, wp[w]);
    a.partial[(size_t)row * a.n_chunks + ck] = make_float4(t.m, t.s, __int_as_float(t.i), 0.f);
  }
}

__global__ __launch_bounds__(64) void commit_decide_kernel(const CommitArgs a) {
  __shared__ float s_conf[kMaxCommitBlock];
  __shared__ int s_idx[kMaxCommitBlock];
  __shared__ unsigned char s_live[kMaxCommitBlock];
  const int k = blockIdx.x;
  const int B = a.block_size;
  const size_t row0 = (size_t)k * B;
  const int tid = threadIdx.x;

  for (int p = tid; p < B; p += 64) {
    const size_t row = row0 + p;
    const bool live = a.mask_state[row] == D2F_MASKED;
    float conf = 0.f;
    int idx = -1;
    if (live) {
      const float4* pp = a.partial + row * a.n_chunks;
      float4 v = pp[0];
      Part t{v.x, v.y, __float_as_int(v.z)};
      for (int c = 1; c < a.n_chunks; ++c) {
        v = pp[c];
        t = combine(t, Part{v.x, v.y, __float_as_int(v.z)});
      }
      conf = 1.0f / t.s;
      idx = t.i;
    }
    s_conf[p] = conf;
    s_idx[p] = idx;
    s_live[p] = live ? 1 : 0;
  }
  __syncthreads();

  const bool aggressive = a.block_phase[k] == D2F_AGGRESSIVE && a.k_aggr > 0;
  int cnt = 0;
  int incomplete = 0;
  for (int p = tid; p < B; p += 64) {
    if (!s_live[p]) continue;
    const float c = s_conf[p];
    bool commit = c > a.tau;
    if (!commit && aggressive) {
      int rank = 0;
      for (int q = 0; q < B && rank < a.k_aggr; ++q) {
        if (s_live[q] && (s_conf[q] > c || (s_conf[q] == c && q < p))) ++rank;
      }
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
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    cnt += __shfl_xor(cnt, o);
    incomplete |= __shfl_xor(incomplete, o);
  }
  if (tid == 0) {
    a.n_committed[k] = cnt;
    a.block_complete[k] = incomplete ? 0 : 1;
  }
}

}  // namespace

hipError_t launch_confidence_commit(const CommitArgs& a, bool vec4, hipStream_t s) {
  const int n_blocks = a.n_rows / a.block_size;
  if (n_blocks == 0) return hipSuccess;
  const long long grid1 = (long long)a.n_rows * a.n_chunks;
  if (vec4)
    hipLaunchKernelGGL(vocab_reduce_kernel<true>, dim3((unsigned)grid1), dim3(kCommitThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL(vocab_reduce_kernel<false>, dim3((unsigned)grid1), dim3(kCommitThreads), 0,
                       s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_decide_kernel, dim3(n_blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace d2f
