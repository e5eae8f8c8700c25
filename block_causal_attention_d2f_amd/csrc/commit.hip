// Confidence pass over the vocabulary logits and the block commit rule.
//
// [D2F-review] section "쉽게 이해하기": a newly added (conservative) block
// commits only positions whose confidence exceeds the threshold; an
// aggressive block also commits its relatively most confident positions;
// what is not committed is masked again.  [dLLM-survey] "답을 미리 안다:
// 조기 확정 디코딩(Prophet)": the confidence is the maximum softmax
// probability, and "양방향 어텐션과 사라진 KV 캐시": low-confidence remasking.
//
// Other measures from the same row ([dLLM-survey] sections "신뢰도를 넘어서:
// 궤적 일관성 디코딩(CCD)" and "토큰 순서의 이론": negative entropy, the
// top-probability margin; "답을 미리 안다": the logit gap and Prophet's early
// commit) need one more accumulator per chunk, so every measure moves the same
// bytes: the second-largest logit l2 (margin = (1 - exp(l2 - max)) / sum, gap
// = max - l2) or X = sum exp(x - max) (x - max) (negative entropy = X / sum -
// log sum).
//
// Kernel 1 (vocab_reduce): one workgroup per (row, chunk of 8192 logits).  A
// MASKED row's chunk is streamed once from HBM with 16-byte loads (8 per
// thread, all in flight together); every thread takes the max of its 32
// values (and the second largest, or X), the sum of exp(x - max), the
// workgroup reduces the max, rescales and reduces the sums (wavefront
// shuffles, then a fixed-order cross-wave step), and the threads holding the
// maximum agree on its first index.  COMMITTED rows are not read.
//
// Kernel 2 (commit_decide): one workgroup per D2F block.  A group of lanes
// per row merges the row's chunk partials (all loads in flight together, a
// fixed merge order), conf = 1 / sum (the max term is exp(0) = 1) is
// compared with the threshold, the aggressive top-k ranks the block's masked
// rows (ties to the lower position), and the new mask state, tokens and
// per-block counts are written.  No floating-point atomics: results are
// deterministic.
//
// Kernel 3 (commit_early, only with Prophet's early commit): one workgroup
// per block; when the smallest logit gap of the block's group (an integer
// atomic minimum over the gaps' bit patterns, which order like the
// non-negative floats they are) is above the group's threshold, the block's
// remaining MASKED rows are committed with their argmax.
#include <climits>

#include "d2f_internal.h"

namespace d2f {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPerThread = kCommitChunk / kCommitThreads;  // 32 logits per thread
constexpr int kWaves = kCommitThreads / 64;

// Logit loads are marked non-temporal: every logit is read exactly once, so
// the lines are not worth keeping in L2 or the Infinity Cache.  (Measured on
// MI355X: the batched ragged workload's 291 MB pass 56.5 -> 50.9 us, Dream's
// 934 MB pass 165 -> 145.6 us.)
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream4(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load((const f32x4_t*)p);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float load_stream(const float* p) {
  return __builtin_nontemporal_load(p);
}

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

// Merge two (max, sum, first index, aux) partials of disjoint index ranges;
// aux is the second-largest value (a repeated maximum counts again) or X,
// both taken relative to the merged maximum.
template <int AUX>
__device__ __forceinline__ void combine(float& m, float& s, int& i, float& x, float m2, float s2,
                                        int i2, float x2) {
  const float mm = fmaxf(m, m2);
  const int ii = (m > m2) ? i : (m2 > m) ? i2 : min(i, i2);
  float ss = 0.f, xx = 0.f;
  if (mm != kNegInf) {
    const float ea = __builtin_amdgcn_exp2f((m - mm) * kLog2e);
    const float eb = __builtin_amdgcn_exp2f((m2 - mm) * kLog2e);
    ss = s * ea + s2 * eb;
    if (AUX == kAuxXlogx) {
      if (m != kNegInf) xx = ea * fmaf(m - mm, s, x);
      if (m2 != kNegInf) xx += eb * fmaf(m2 - mm, s2, x2);
    }
  }
  if (AUX == kAuxSecond) x = fmaxf(fminf(m, m2), fmaxf(x, x2));
  if (AUX == kAuxXlogx) x = xx;
  m = mm;
  s = ss;
  i = ii;
}

// Reduce one chunk of one row; returns (max, sum, first argmax, aux) in
// thread 0.
template <bool VEC, int AUX>
__device__ void reduce_chunk(const CommitArgs& a, int row, int ck, float4& result) {
  __shared__ float sh_m[kWaves], sh_s[kWaves], sh_x[kWaves];
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
      const float4 v = load_stream4(src + 4 * (tid + kCommitThreads * k));
      x[4 * k + 0] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
    }
  } else if (VEC) {
#pragma unroll
    for (int k = 0; k < kPerThread / 4; ++k) {
      const int e0 = 4 * (tid + kCommitThreads * k);
      if (e0 + 3 < n) {
        const float4 v = load_stream4(src + e0);
        x[4 * k + 0] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) x[4 * k + c] = (e0 + c < n) ? load_stream(src + e0 + c) : kNegInf;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int e = tid + kCommitThreads * k;
      x[k] = (e < n) ? load_stream(src + e) : kNegInf;
    }
  }
  float m = kNegInf, m2 = kNegInf;
  if (AUX == kAuxSecond) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      m2 = fmaxf(m2, fminf(m, x[k]));
      m = fmaxf(m, x[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) m = fmaxf(m, x[k]);
  }
  // exp(x - m) as 2^((x - m) log2 e): the difference is exact for the terms
  // near the maximum that dominate the sum, so their relative error stays at
  // a few ulp (folding m * log2 e into one fma would shift every term of the
  // thread by the rounding of that product instead).
  float s = 0.f, t = 0.f;
  if (m != kNegInf) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const float d = x[k] - m;
      const float e = __builtin_amdgcn_exp2f(d * kLog2e);
      s += e;
      if (AUX == kAuxXlogx && e != 0.f) t = fmaf(e, d, t);
    }
  }
  // Workgroup maximum (and second largest: a top-two merge is associative).
  float wm, w2 = kNegInf;
  if (AUX == kAuxSecond) {
    wm = m;
    w2 = m2;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float b1 = __shfl_xor(wm, o), b2 = __shfl_xor(w2, o);
      w2 = fmaxf(fminf(wm, b1), fmaxf(w2, b2));
      wm = fmaxf(wm, b1);
    }
  } else {
    wm = wave_max(m);
  }
  if (lane == 0) {
    sh_m[wave] = wm;
    if (AUX == kAuxSecond) sh_x[wave] = w2;
  }
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
  const float r = (M == kNegInf || m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((m - M) * kLog2e);
  const float ws = wave_sum(s * r);
  float wx = 0.f;
  if (AUX == kAuxXlogx) wx = wave_sum(m == kNegInf ? 0.f : r * fmaf(m - M, s, t));
  if (lane == 0) {
    sh_s[wave] = ws;
    if (AUX == kAuxXlogx) sh_x[wave] = wx;
  }
  __syncthreads();
  if (tid == 0) {
    float S = sh_s[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) S += sh_s[w];
    float X = 0.f;
    if (AUX == kAuxSecond) {
      float a1 = sh_m[0];
      X = sh_x[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        X = fmaxf(fminf(a1, sh_m[w]), fmaxf(X, sh_x[w]));
        a1 = fmaxf(a1, sh_m[w]);
      }
    } else if (AUX == kAuxXlogx) {
      X = sh_x[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) X += sh_x[w];
    }
    result = make_float4(M, S, __int_as_float(sh_i), X);
  }
}

// Combine the chunk partials of every row of one block into s_conf / s_idx
// (and s_gap, the logit gap, when AUX is the second-largest value) and mark
// the MASKED rows in s_live.  A row's chunks go to a group of L lanes of one
// wave (L the largest power of two, at most 64, with B L <= the workgroup's
// threads): lane j of the group loads chunks j, j + L, ..., kBatch at a time
// all in flight, and folds them in chunk order; the group then merges its
// lanes' partials in a fixed butterfly (exchange partner j ^ 1, then j ^ 2,
// ...), and since the merge is symmetric every lane ends with the same
// result.  The order is fixed, so the result does not depend on timing.
// The loads do not wait for the mask state: a row that is not MASKED has no
// partials written, and what is read for it is discarded.
template <int AUX>
__device__ void combine_rows(const CommitArgs& a, size_t row0, int B, float* s_conf, int* s_idx,
                             float* s_gap, unsigned char* s_live) {
  constexpr int kBatch = 8;
  constexpr float kX0 = AUX == kAuxSecond ? kNegInf : 0.f;
  const int nck = a.n_chunks;
  int L = 1;
  while (L < 64 && 2 * L * B <= kCommitThreads) L *= 2;
  const int rows_per_pass = kCommitThreads / L;
  const int j = (int)threadIdx.x % L;
  for (int p0 = 0; p0 < B; p0 += rows_per_pass) {
    const int p = p0 + (int)threadIdx.x / L;
    const bool in_block = p < B;
    const bool live = in_block && a.mask_state[row0 + p] == D2F_MASKED;
    float m = kNegInf, sm = 0.f, xa = kX0;
    int ix = INT_MAX;
    if (in_block) {
      const float4* src = a.partial + (row0 + p) * nck;
      for (int c0 = j; c0 < nck; c0 += kBatch * L) {
        float4 v[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int c = c0 + k * L;
          v[k] = c < nck ? src[c] : make_float4(kNegInf, 0.f, __int_as_float(INT_MAX), kX0);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
          combine<AUX>(m, sm, ix, xa, v[k].x, v[k].y, __float_as_int(v[k].z), v[k].w);
      }
    }
    for (int o = 1; o < L; o <<= 1)
      combine<AUX>(m, sm, ix, xa, __shfl_xor(m, o), __shfl_xor(sm, o), __shfl_xor(ix, o),
                   __shfl_xor(xa, o));
    if (!in_block || j != 0) continue;
    float c = 1.0f / sm;  // maximum probability: the max term is exp(0) = 1
    if (AUX == kAuxSecond) {
      const float gap = m - xa;  // >= 0; +inf when the row has one entry
      if (a.measure == D2F_CONF_MARGIN)
        c = (1.0f - __builtin_amdgcn_exp2f((xa - m) * kLog2e)) / sm;
      else if (a.measure == D2F_CONF_LOGIT_GAP)
        c = gap;
      s_gap[p] = gap;
    } else if (AUX == kAuxXlogx) {
      c = xa / sm - logf(sm);  // sum p log p = X / sum - log sum
    }
    s_conf[p] = live ? c : 0.f;
    s_idx[p] = live ? ix : -1;
    s_live[p] = live;
  }
}

template <int AUX>
__global__ __launch_bounds__(kCommitThreads) void commit_decide_kernel(const CommitArgs a) {
  __shared__ float s_conf[kMaxCommitBlock];
  __shared__ float s_gap[AUX == kAuxSecond ? kMaxCommitBlock : 1];
  __shared__ int s_idx[kMaxCommitBlock];
  __shared__ unsigned char s_live[kMaxCommitBlock];
  __shared__ int s_cnt, s_incomplete;
  const int blk = blockIdx.x;
  const int B = a.block_size;
  const size_t row0 = (size_t)blk * B;
  const int tid = threadIdx.x;
  // The phase goes through a vector load issued with the partials' loads
  // (a uniform address would become a scalar load waited on at once).
  int pidx = blk;
  asm volatile("" : "+v"(pidx));
  const unsigned char phase = a.block_phase[pidx];
  if (tid == 0) {
    s_cnt = 0;
    s_incomplete = 0;
  }
  combine_rows<AUX>(a, row0, B, s_conf, s_idx, s_gap, s_live);
  __syncthreads();
  const bool aggressive = phase == D2F_AGGRESSIVE && a.k_aggr > 0;
  const bool early = AUX == kAuxSecond && a.early_gap != nullptr;
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
    if (early) {
      // Non-negative floats order like their bit patterns.
      atomicMin(&a.ws_gmin[blk / a.group_blocks], __float_as_uint(s_gap[p]));
      a.ws_argmax[row] = s_idx[p];
    }
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

// Prophet's early commit of one block: runs after commit_decide on the same
// stream, so the group minimum is final.
__global__ __launch_bounds__(kCommitThreads) void commit_early_kernel(const CommitArgs a) {
  __shared__ int s_cnt;
  const int blk = blockIdx.x;
  const int g = blk / a.group_blocks;
  if (!(__uint_as_float(a.ws_gmin[g]) > a.early_gap[g])) return;
  const int B = a.block_size;
  const size_t row0 = (size_t)blk * B;
  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();
  int cnt = 0;
  for (int p = threadIdx.x; p < B; p += kCommitThreads) {
    const size_t row = row0 + p;
    if (a.mask_state[row] != D2F_MASKED) continue;
    a.mask_state[row] = D2F_COMMITTED;
    a.tokens[row] = a.ws_argmax[row];
    ++cnt;
  }
  if (cnt) atomicAdd(&s_cnt, cnt);
  __syncthreads();
  if (threadIdx.x == 0) {
    a.n_committed[blk] += s_cnt;
    a.block_complete[blk] = 1;
  }
}

template <bool VEC, int AUX>
__global__ __launch_bounds__(kCommitThreads) void vocab_reduce_kernel(const CommitArgs a) {
  // The group minima of the early commit start at +inf on every call (this
  // kernel runs first; the grid has at least as many workgroups as groups).
  if (AUX == kAuxSecond && a.early_gap != nullptr && threadIdx.x == 0 &&
      (int)blockIdx.x < a.n_groups)
    a.ws_gmin[blockIdx.x] = 0x7f800000u;
  // Workgroups are renumbered so that each XCD streams a contiguous run of
  // rows (measured on MI355X: Dream-shaped block 64, 934 MB, 138.9 vs
  // 144.6 us per pass; the smaller passes unchanged).
  const int u = xcd_remap(blockIdx.x, gridDim.x);
  const int row = u / a.n_chunks;
  const int ck = u - row * a.n_chunks;
  if (a.mask_state[row] != D2F_MASKED) return;
  float4 part;
  reduce_chunk<VEC, AUX>(a, row, ck, part);
  if (threadIdx.x == 0) a.partial[(size_t)row * a.n_chunks + ck] = part;
}

template <int AUX>
hipError_t launch_aux(const CommitArgs& a, bool vec4, hipStream_t s) {
  const long long grid = (long long)a.n_rows * a.n_chunks;
  if (vec4)
    hipLaunchKernelGGL((vocab_reduce_kernel<true, AUX>), dim3((unsigned)grid),
                       dim3(kCommitThreads), 0, s, a);
  else
    hipLaunchKernelGGL((vocab_reduce_kernel<false, AUX>), dim3((unsigned)grid),
                       dim3(kCommitThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_decide_kernel<AUX>, dim3(a.n_rows / a.block_size),
                     dim3(kCommitThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || AUX != kAuxSecond || a.early_gap == nullptr) return e;
  hipLaunchKernelGGL(commit_early_kernel, dim3(a.n_rows / a.block_size), dim3(kCommitThreads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_confidence_commit(const CommitArgs& a, bool vec4, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  // Maximum probability needs no auxiliary accumulator unless the early
  // commit reads the logit gap.
  if (a.measure == D2F_CONF_NEG_ENTROPY) return launch_aux<kAuxXlogx>(a, vec4, s);
  if (a.measure != D2F_CONF_MAXPROB || a.early_gap != nullptr)
    return launch_aux<kAuxSecond>(a, vec4, s);
  return launch_aux<kAuxNone>(a, vec4, s);
}

}  // namespace d2f
