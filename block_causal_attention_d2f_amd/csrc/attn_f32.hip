// Block-causal window attention in fp32 on the vector ALUs.
//
// Same operation, work units and outputs as the bf16 matrix-core kernel (see
// attn_bf16.hip): each window row attends to the cached keys and to the
// window keys of its own and earlier blocks, i.e. to the key prefix
// [0, P + (qb + 1) * B) for a row of window block qb.  This path exists for
// fp32 inputs, where every product is formed in fp32 from fp32 operands.
//
// One workgroup (256 threads) holds a tile of 64 query rows in LDS; four
// threads share a row.  Per 64-key tile: each thread forms 16 scores, the
// four threads of a row reduce the max and sum with lane shuffles, the
// probabilities go to LDS, and each thread accumulates a quarter of the
// row's output dimensions.
#include "d2f_internal.h"

namespace d2f {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_f32_kernel(const AttnArgs a) {
  __shared__ float Qs[kQTile][D + 1];
  __shared__ float Ks[kKTile][D + 1];
  __shared__ float Vs[kKTile][D];
  __shared__ float Ps[kQTile][kKTile + 1];

  const int u = a.remap ? xcd_remap(blockIdx.x, a.n_units) : (int)blockIdx.x;
  const int ri = find_req(a, u);
  const int rb = a.req[ri].b, P = a.req[ri].prefix, W = a.req[ri].win;
  const int qtiles = a.req[ri].qtiles, nsplit = a.req[ri].nsplit;
  int local = u - a.req[ri].unit_base;
  const int qt = local % qtiles;
  local /= qtiles;
  const int split = local % nsplit;
  const int kvh = local / nsplit;
  const int G = a.group, B = a.bsz;
  const int rows = G * W;
  const int r0 = qt * kQTile;
  const int k_end = unit_key_end(a, qt, kQTile, P, W, G, B);
  const int nct = cache_tiles(P);
  int t_lo, t_hi;
  split_tiles(nct + window_tiles(P, k_end), split, nsplit, t_lo, t_hi);

  const size_t head_c = (((size_t)rb * a.hkv + kvh) * (size_t)a.cap + a.req[ri].key_off) * D;
  const size_t head_w = ((size_t)rb * a.hkv + kvh) * (size_t)a.wmax * D;
  const float* kc = (const float*)a.kc + head_c;
  const float* vc = (const float*)a.vc + head_c;
  const float* kw = (const float*)a.kw + head_w;
  const float* vw = (const float*)a.vw + head_w;

  const int tid = threadIdx.x;
  const int r = tid >> 2, sub = tid & 3;
  const int my_row = r0 + r;
  const bool row_ok = my_row < rows;
  const int my_i = row_ok ? my_row / G : 0;
  const int my_h = kvh * G + (row_ok ? my_row % G : 0);
  const int my_lim = a.cache_only ? P : P + min(W, (my_i / B + 1) * B);

  for (int e = tid; e < kQTile * D; e += kAttnThreads) {
    const int rr = e / D, d = e % D;
    const int row = r0 + rr;
    float v = 0.f;
    if (row < rows) {
      const int i = row / G, h = kvh * G + row % G;
      v = ((const float*)a.q)[(((size_t)rb * a.hq + h) * a.wmax + i) * D + d];
    }
    Qs[rr][d] = v;
  }

  float acc[D / 4];
#pragma unroll
  for (int k = 0; k < D / 4; ++k) acc[k] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  for (int t = t_lo; t < t_hi; ++t) {
    int tile_lo, nv;
    tile_span(t, nct, P, k_end, tile_lo, nv);
    const bool in_cache = t < nct;
    const float* ksrc = in_cache ? kc + (size_t)tile_lo * D : kw + (size_t)(tile_lo - P) * D;
    const float* vsrc = in_cache ? vc + (size_t)tile_lo * D : vw + (size_t)(tile_lo - P) * D;
    __syncthreads();  // previous tile fully consumed (and Q tile stored)
    for (int e = tid; e < kKTile * D; e += kAttnThreads) {
      const int n = e / D;
      const bool ok = n < nv;
      Ks[n][e % D] = ok ? ksrc[e] : 0.f;
      Vs[n][e % D] = ok ? vsrc[e] : 0.f;
    }
    __syncthreads();
    const int lim = min(nv, my_lim - tile_lo);  // keys of this tile the row sees

    float x[16];
    float mx = kNegInf;
#pragma unroll
    for (int uu = 0; uu < 16; ++uu) {
      const int n = sub + 4 * uu;
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) s = fmaf(Qs[r][d], Ks[n][d], s);
      float v = s * a.c2;
      if (n >= lim) v = kNegInf;
      x[uu] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float ps = 0.f;
#pragma unroll
    for (int uu = 0; uu < 16; ++uu) {
      const float p = exp2f(x[uu] - m_use);
      Ps[r][sub + 4 * uu] = p;
      ps += p;
    }
    ps += __shfl_xor(ps, 1);
    ps += __shfl_xor(ps, 2);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < D / 4; ++k) acc[k] *= alpha;
    for (int n = 0; n < kKTile; ++n) {
      const float p = Ps[r][n];
#pragma unroll
      for (int k = 0; k < D / 4; ++k) acc[k] = fmaf(p, Vs[n][sub + 4 * k], acc[k]);
    }
  }

  if (nsplit == 1) {
    if (!row_ok) return;
    const float inv = 1.0f / l_run;
    float* op = (float*)a.out + (((size_t)rb * a.hq + my_h) * a.wmax + my_i) * D;
#pragma unroll
    for (int k = 0; k < D / 4; ++k) op[sub + 4 * k] = acc[k] * inv;
    if (a.lse != nullptr && sub == 0)
      a.lse[((size_t)rb * a.hq + my_h) * a.wmax + my_i] = (m_run + log2f(l_run)) * kLn2;
    return;
  }
  if (row_ok) {
    const size_t row_slot = (size_t)u * a.slot_rows + r;
    float* wp = a.ws_o + row_slot * D;
#pragma unroll
    for (int k = 0; k < D / 4; ++k) wp[sub + 4 * k] = acc[k];
    if (sub == 0) {
      a.ws_ml[row_slot * 2 + 0] = m_run;
      a.ws_ml[row_slot * 2 + 1] = l_run;
    }
  }
}

}  // namespace

int attn_f32_wgs_per_cu(int head_dim) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (head_dim) {
    case 32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_f32_kernel<32>, kAttnThreads, 0); break;
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_f32_kernel<64>, kAttnThreads, 0); break;
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_f32_kernel<128>, kAttnThreads, 0); break;
    default: break;
  }
  return e == hipSuccess ? n : 0;
}

hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid(a.n_units), block(kAttnThreads);
  switch (head_dim) {
    case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace d2f
