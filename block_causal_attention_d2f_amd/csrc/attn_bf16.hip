// Block-causal window attention, bf16 inputs, fp32 accumulation, on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// What is computed ([D2F-wiki] "블록 단위 인과 어텐션"; [D2F-review] "쉽게
// 이해하기"): every window row attends to all cached keys and to the window
// keys of its own block and of every earlier window block.  Visible keys of a
// row in window block qb therefore form the prefix [0, P + (qb + 1) * B) of
// the key list [cache ++ window]; the kernel masks with one compare per score
// and never loads a tile that lies wholly past a tile's last visible key.
//
// Design (one workgroup = 4 waves = one work unit, see d2f_internal.h):
//  * K and V tiles of 64 keys are staged HBM -> registers -> LDS with 16-byte
//    coalesced loads, double-buffered so the next tile's loads are in flight
//    while the current one is consumed.
//  * Scores are computed transposed, S^T = K Q^T: keys run along the MFMA M
//    dimension and each wave's 16 query rows along N.  Each lane then holds
//    one query and 4 keys per 16-key block, which is exactly the B operand
//    layout (8 key slots per lane) of the next product O^T = V^T P^T, so
//    probabilities go from accumulators to the PV MFMA without a shuffle.
//  * V stays in its natural [key][dim] layout in LDS; the V^T operand is read
//    with the gfx950 LDS transpose load (ds_read_b64_tr_b16).
//  * Online softmax in base 2 with the scale folded into one multiply; row
//    statistics are reduced across the 4 lanes holding one query.
//  * A unit either covers all keys of its rows (writes O in bf16 and the LSE)
//    or one key range (writes unnormalised O, running max and sum in fp32 for
//    the merge kernel: the exact log-space composition of partial softmaxes).
#include "d2f_internal.h"

namespace d2f {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) __bf16 lds_bf16;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_bf16_kernel(const AttnArgs a) {
  constexpr int S = D + 8;             // LDS row stride in bf16 (16-byte pad)
  constexpr int KSTEPS = D / 32;       // MFMA k-steps over head_dim
  constexpr int DBLK = D / 16;         // 16-dim blocks of the output
  constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
  constexpr int RPP = kAttnThreads / CPR;  // rows loaded per pass
  constexpr int PASSES = kKTile / RPP;
  constexpr int TILE = kKTile * S;     // bf16 per K (or V) tile
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * TILE];  // [buf][K,V][key][dim]

  const int u = xcd_remap(blockIdx.x, a.n_units);
  const int ri = find_req(a, u);
  const int rb = a.req[ri].b, P = a.req[ri].prefix, W = a.req[ri].win;
  const int qtiles = a.req[ri].qtiles, nsplit = a.req[ri].nsplit, chunk = a.req[ri].chunk;
  int local = u - a.req[ri].unit_base;
  const int qt = local % qtiles;
  local /= qtiles;
  const int split = local % nsplit;
  const int kvh = local / nsplit;
  const int G = a.group, B = a.bsz;
  const int rows = G * W;
  const int r0 = qt * kQTile;
  const int r_last = min(r0 + kQTile, rows) - 1;
  const int k_end = P + min(W, ((r_last / G) / B + 1) * B);   // last key any row sees
  const int k_full = P + min(W, ((r0 / G) / B + 1) * B);      // keys every row sees
  const int k_lo = split * chunk;
  const int k_hi = min(k_lo + chunk, k_end);
  const int n_tiles = k_hi > k_lo ? (k_hi - k_lo + kKTile - 1) / kKTile : 0;
  const int mask_from = min(k_full, k_hi);

  const size_t head_c = ((size_t)rb * a.hkv + kvh) * (size_t)a.cap * D;
  const size_t head_w = ((size_t)rb * a.hkv + kvh) * (size_t)a.wmax * D;
  const __bf16* kc = (const __bf16*)a.kc + head_c;
  const __bf16* vc = (const __bf16*)a.vc + head_c;
  const __bf16* kw = (const __bf16*)a.kw + head_w;
  const __bf16* vw = (const __bf16*)a.vw + head_w;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lc = lane & 15, lg = lane >> 4;

  // Loader mapping: 16-byte chunk c of rows n0 + RPP * p.
  const int ld_c = tid % CPR, ld_n0 = tid / CPR;
  uint4 kreg[PASSES], vreg[PASSES];
  auto gload = [&](int tile_lo) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int j = tile_lo + ld_n0 + RPP * p;
      if (j < k_hi) {
        const __bf16* ks = (j < P) ? kc + (size_t)j * D : kw + (size_t)(j - P) * D;
        const __bf16* vs = (j < P) ? vc + (size_t)j * D : vw + (size_t)(j - P) * D;
        kreg[p] = *(const uint4*)(ks + 8 * ld_c);
        vreg[p] = *(const uint4*)(vs + 8 * ld_c);
      } else {
        kreg[p] = make_uint4(0, 0, 0, 0);
        vreg[p] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
    __bf16* kt = smem + buf * 2 * TILE;
    __bf16* vt = kt + TILE;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int n = ld_n0 + RPP * p;
      *(uint4*)(kt + n * S + 8 * ld_c) = kreg[p];
      *(uint4*)(vt + n * S + 8 * ld_c) = vreg[p];
    }
  };

  // This lane's query (MFMA column lc of this wave's 16 rows).
  const int my_row = r0 + 16 * wave + lc;
  const bool row_ok = my_row < rows;
  const int my_i = row_ok ? my_row / G : 0;
  const int my_h = kvh * G + (row_ok ? my_row % G : 0);
  const int my_lim = min(k_hi, P + min(W, (my_i / B + 1) * B));
  const bool wave_active = (r0 + 16 * wave) < rows;

  bf16x8 qf[KSTEPS];
  if (row_ok) {
    const __bf16* qp = (const __bf16*)a.q + (((size_t)rb * a.hq + my_h) * a.wmax + my_i) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *(const bf16x8*)(qp + 32 * s + 8 * lg);
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = bf16x8{};
  }

  f32x4 o[DBLK];
#pragma unroll
  for (int d = 0; d < DBLK; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.c2;

  if (n_tiles > 0) {
    gload(k_lo);
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int tile_lo = k_lo + t * kKTile;
    if (t + 1 < n_tiles) gload(tile_lo + kKTile);

    if (wave_active) {
      const __bf16* Ks = smem + buf * 2 * TILE;
      const lds_bf16* Vs = (const lds_bf16*)(Ks + TILE);
      f32x4 sc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const bf16x8 ka = *(const bf16x8*)(Ks + (16 * kb + lc) * S + 32 * s + 8 * lg);
          sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[s], sc[kb], 0, 0, 0);
        }
      }
      // Scale, mask, and the row maximum of this tile.
      const bool need_mask = tile_lo + kKTile > mask_from;
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = sc[kb][r] * c2;
          if (need_mask && tile_lo + 16 * kb + 4 * lg + r >= my_lim) x = kNegInf;
          sc[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(sc[kb][r] - m_use);
          sc[kb][r] = p;
          ps += p;
        }
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run = l_run * alpha + ps;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < DBLK; ++d) o[d] *= alpha;

      // O^T += V^T P^T over two 32-key halves of the tile.
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        bf16x8 pf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pf[r] = (__bf16)sc[2 * kh][r];
          pf[4 + r] = (__bf16)sc[2 * kh + 1][r];
        }
        const lds_bf16* vrow = Vs + (32 * kh + 4 * lg + (lc >> 2)) * S + 4 * (lc & 3);
#pragma unroll
        for (int d = 0; d < DBLK; ++d) {
          const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vrow + 16 * d));
          const i16x4 t1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vrow + 16 * S + 16 * d));
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          const i16x8 both = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
          o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, both), pf,
                                                          o[d], 0, 0, 0);
        }
      }
    }

    if (t + 1 < n_tiles) lstore(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active || !row_ok) return;
  if (nsplit == 1) {
    const float inv = 1.0f / l_run;
    __bf16* op = (__bf16*)a.out + (((size_t)rb * a.hq + my_h) * a.wmax + my_i) * D;
#pragma unroll
    for (int d = 0; d < DBLK; ++d) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)(o[d][r] * inv);
      *(bf16x4*)(op + 16 * d + 4 * lg) = v;
    }
    if (a.lse != nullptr && lg == 0)
      a.lse[((size_t)rb * a.hq + my_h) * a.wmax + my_i] = (m_run + log2f(l_run)) * kLn2;
  } else {
    const size_t row_slot = (size_t)u * kQTile + 16 * wave + lc;
    float* wp = a.ws_o + row_slot * D;
#pragma unroll
    for (int d = 0; d < DBLK; ++d) *(f32x4*)(wp + 16 * d + 4 * lg) = o[d];
    if (lg == 0) {
      a.ws_ml[row_slot * 2 + 0] = m_run;
      a.ws_ml[row_slot * 2 + 1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid(a.n_units), block(kAttnThreads);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, block, 0, s, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace d2f
