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
//  * K and V tiles of 64 keys go HBM -> LDS with the gfx950 direct loads
//    (global_load_lds_dwordx4: each lane's 16 bytes land in LDS without
//    passing through registers).  Two LDS stages alternate: while the waves
//    work on one tile, the next one streams into the other stage.  Each
//    stage is a separate LDS variable and the tile loop is unrolled by two,
//    so the compiler can tell the stage being read from the one being
//    filled and never waits for the in-flight tile before an LDS read.
//  * The LDS rows are unpadded and their 16-byte chunks XOR-swizzled by row,
//    which makes both LDS read patterns below free of bank conflicts.
//  * Wave w works on query rows [16 QB (w & 1), +16 QB) -- QB 16-row MFMA
//    blocks: 2 for 64-row units, 1 for the 32-row units of narrow windows --
//    and on key half (w >> 1) -- 32 keys -- of every tile, so each K or V
//    fragment read from LDS feeds QB MFMAs and each wave runs 2 QB
//    independent accumulation chains.  The two key halves are merged once,
//    through LDS, at the end of the unit.
//  * Scores are computed transposed, S^T = K Q^T: keys run along the MFMA M
//    dimension and queries along N.  Each lane then holds one query and 8
//    keys, exactly the B-operand layout of the next product O^T = V^T P^T,
//    so probabilities go from accumulators to the PV MFMA without a shuffle.
//    The V^T operand is read with the LDS transpose load ds_read_b64_tr_b16.
//  * Online softmax in base 2: the row max is taken on raw scores and the
//    scale is folded into the exp argument with one fma.  The reference max
//    is raised lazily (only when a score exceeds it by 2^8), and each lane
//    keeps its own partial sum, so the steady-state tile loop needs no
//    cross-lane reduction at all.
//  * Launches with no more units than CUs and no key split run eight waves
//    per unit (TG = 2): two groups of four take alternate key tiles, each
//    with its own stages, and their states are joined through LDS.
//  * K/V tiles that no other query tile of the launch reads are loaded with
//    the non-temporal cache policy.
//  * A unit either covers all keys of its rows (writes O in bf16 and the LSE)
//    or one key range (writes unnormalised O, running max and sum in fp32,
//    merged exactly by attn_merge.hip).
//  * Paged caches (PAGED != 0) change only the loader: the rows of each 1 KB
//    direct load are found through the page tables, with the page ids of
//    the next tile fetched while the current one is issued.  Key-range calls
//    (cache_only) read cache keys [key_off, key_off + P) and no window keys,
//    all of them visible.
#include "attn_lds.h"

namespace d2f {
namespace {

// QB: 16-row query blocks per wave (2: 64 query rows per unit, 1: 32).
// PAGED: 0 contiguous K/V; otherwise rows are found through the page tables
// (see AttnArgs): 1 for 8-row pages, 2 for pages of 16 rows or more, where the
// 16 rows a wave loads of a tile always share one page.
// TG: tile groups of four waves.  1: one group takes every tile, two
// workgroups per CU.  2: eight waves; group g takes the unit's tiles g, g + 2,
// ... with its own two LDS stages, and the groups' online-softmax states are
// joined exactly through LDS at the end.  For launches with no more units
// than CUs, this puts two waves on every SIMD without cutting the unit's keys
// into separately merged ranges.
// SHARED (a.remap): several query tiles read each KV head's tiles, so units
// are numbered XCD-contiguously and the tile loads keep the default cache
// policy; otherwise they are non-temporal.
template <int D, int QB, int PAGED, int TG, bool SHARED>
__global__ __launch_bounds__(kAttnThreads * TG, TG == 1 ? 2 : 1) void attn_bf16_kernel(
    const AttnArgs a) {
  constexpr int RS = D * 2;                // LDS row bytes
  constexpr int KSTEPS = D / 32;           // MFMA k-steps over head_dim
  constexpr int DBLK = D / 16;             // 16-dim blocks of the output
  constexpr int CPR = D / 8;               // 16-byte chunks per K/V row
  constexpr int TILE = kKTile * RS;        // bytes per K (or V) tile
  constexpr int RPB = 1024 / RS;           // rows per 1 KB direct-load block
  constexpr int LPW = TILE / 1024 / 4;     // blocks per wave per tensor per tile
  static_assert(LPW >= 1 && LPW * 4 * 1024 == TILE, "4 waves cover a tile in 1 KB blocks");
  static_assert(2 * DBLK * 64 * 4 * 2 * 4 <= 2 * TILE && 2 * 64 * 2 * 2 * 4 <= 2 * TILE,
                "merge area fits the two stages");
  static_assert(TG == 1 || TG == 2, "one or two tile groups");
  constexpr int SB = TG * 2 * TILE;  // bytes per LDS stage: [group][K tile, V tile]

  const int u = SHARED ? xcd_remap(blockIdx.x, a.n_units) : (int)blockIdx.x;
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
  constexpr int QROWS = 32 * QB;  // query rows of the unit
  const int r0 = qt * QROWS;
  const int k_end = unit_key_end(a, qt, QROWS, P, W, G, B);  // last key any row sees
  const int k_full = a.cache_only ? P : P + min(W, ((r0 / G) / B + 1) * B);  // every row sees
  const int nct = cache_tiles(P);
  int t_lo, t_hi;
  split_tiles(nct + window_tiles(P, k_end), split, nsplit, t_lo, t_hi);
  const int n_tiles = t_hi - t_lo;

  const size_t head_c = (((size_t)rb * a.hkv + kvh) * (size_t)a.cap + a.req[ri].key_off) * D;
  const size_t head_w = ((size_t)rb * a.hkv + kvh) * (size_t)a.wmax * D;
  const __bf16* kc = (const __bf16*)a.kc + head_c;
  const __bf16* vc = (const __bf16*)a.vc + head_c;
  const __bf16* kw = (const __bf16*)a.kw + head_w;
  const __bf16* vw = (const __bf16*)a.vw + head_w;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lc = lane & 15, lg = lane >> 4;
  const int qh = wave & 1, kh = (wave >> 1) & 1;
  const int tg = TG == 1 ? 0 : __builtin_amdgcn_readfirstlane(wave >> 2);  // tile group

  // Loader: tile rows are copied in 1 KB blocks, one direct load per wave
  // and block; lane l of block j carries the 16 bytes that belong at LDS
  // position (row RPB j + l / CPR, chunk l % CPR), i.e. global chunk
  // (l % CPR) ^ swz(row) of that row.  A tile's rows all come from the cache
  // or all from the window, so the base pointers are uniform.  Rows past a
  // partial tile's end re-read its last row (in bounds; the score mask gives
  // them zero weight).
  auto tile_base = [&](int t, const char*& kb, const char*& vb, int& nv) {
    int lo;
    tile_span(t, nct, P, k_end, lo, nv);
    const bool in_cache = t < nct;
    const size_t o = (size_t)(in_cache ? lo : lo - P) * D;
    kb = (const char*)((in_cache ? kc : kw) + o);
    vb = (const char*)((in_cache ? vc : vw) + o);
  };
  const int wave_u = __builtin_amdgcn_readfirstlane(wave & 3);  // wave within its tile group
  // Paged rows: a 1 KB block holds RPB consecutive rows starting at a
  // multiple of RPB, and a page holds bsz rows with bsz a multiple of RPB,
  // so the rows of one direct load lie in one page and its base stays
  // uniform (a block wholly past a partial tile's end re-reads the tile's
  // last row).  The page ids of the next tile are fetched while the current
  // one is issued: lane j of a wave holds the page of its block j and that
  // page's first row relative to the tile, and the tile barrier's wait for
  // all loads covers them, so no issue waits on a table read.  Page ids are
  // clamped to the pool, so a bad table entry reads the wrong rows, never
  // outside the pool.
  static_assert(RPB * LPW == 16, "a wave loads 16 rows of a tile");
  const size_t page_elems = (size_t)a.hkv * B * D;
  const int pshift = a.page_shift;  // bsz = 1 << pshift
  int pg_page = 0, pg_row0 = 0;  // lane j < LPW: block j of the tile issued next
  auto fetch_pages = [&](int t) {
    int lo, nv;
    tile_span(t, nct, P, k_end, lo, nv);
    const bool in_cache = t < nct;
    const int r0 = in_cache ? lo : lo - P;  // first row's index in the cache or the window
    const int32_t* table = in_cache ? a.page_table + (size_t)rb * a.table_stride
                                    : a.win_pages + (size_t)rb * (a.wmax / B);
    const int j = (PAGED == 1 && lane < LPW) ? lane : 0;
    const int key0 = r0 + min(RPB * (LPW * wave_u + j), nv - 1);
    const int pi = key0 >> pshift;
    pg_page = min(max(table[pi], 0), a.n_pages - 1);
    pg_row0 = (pi << pshift) - r0;
  };
  auto issue_paged = [&](auto J, int t) {
    const unsigned sb =
        (unsigned)(uintptr_t)stage_buf<decltype(J)::value, SB>() + tg * 2 * TILE;
    int lo, nv;
    tile_span(t, nct, P, k_end, lo, nv);
    int page = __builtin_amdgcn_readfirstlane(pg_page);
    int row0 = __builtin_amdgcn_readfirstlane(pg_row0);
    size_t pbase = ((size_t)page * page_elems + (size_t)kvh * B * D) * sizeof(__bf16);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int blk = LPW * wave_u + j;
      if (PAGED == 1 && j > 0) {
        page = __builtin_amdgcn_readlane(pg_page, j);
        row0 = __builtin_amdgcn_readlane(pg_row0, j);
        pbase = ((size_t)page * page_elems + (size_t)kvh * B * D) * sizeof(__bf16);
      }
      const int row = RPB * blk + lane / CPR;
      const int off = (min(row, nv - 1) - row0) * RS + 16 * ((lane % CPR) ^ swz<D>(row));
      load_kv16<SHARED>((const char*)a.kc + pbase, off, sb + blk * 1024);
      load_kv16<SHARED>((const char*)a.vc + pbase, off, sb + TILE + blk * 1024);
    }
    fetch_pages(min(t + TG, t_hi - 1));  // the group's next tile
  };
  auto issue = [&](auto J, int t) {
    if constexpr (PAGED != 0) {
      issue_paged(J, t);
      return;
    }
    const unsigned sb =
        (unsigned)(uintptr_t)stage_buf<decltype(J)::value, SB>() + tg * 2 * TILE;
    const char *kb, *vb;
    int nv;
    tile_base(t, kb, vb, nv);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int blk = LPW * wave_u + j;
      const int row = RPB * blk + lane / CPR;
      const int off = min(row, nv - 1) * RS + 16 * ((lane % CPR) ^ swz<D>(row));
      load_kv16<SHARED>(kb, off, sb + blk * 1024);
      load_kv16<SHARED>(vb, off, sb + TILE + blk * 1024);
    }
  };

  // The first tile is requested before the queries are loaded, so that its
  // latency and theirs overlap.  Tiles past the last re-read the last tile.
  auto tile_at = [&](int i) { return min(t_lo + i, t_hi - 1); };
  // Tiles of this wave's group: t_lo + tg, t_lo + tg + TG, ...; every group
  // runs n_steps steps (the barriers are shared), idle when it has no tile.
  [[maybe_unused]] const int n_g = (n_tiles - tg + TG - 1) / TG;
  [[maybe_unused]] const int n_steps = (n_tiles + TG - 1) / TG;
  [[maybe_unused]] auto gt = [&](int k) { return t_lo + TG * k + tg; };
  if constexpr (TG == 1) {
    if (PAGED != 0 && n_tiles > 0) fetch_pages(tile_at(0));
    if (n_tiles > 0) issue(ic<0>{}, tile_at(0));
  } else {
    if (PAGED != 0 && n_g > 0) fetch_pages(gt(0));
    if (n_g > 0) issue(ic<0>{}, gt(0));
  }

  // This lane's two queries (MFMA column lc of the wave's two row blocks).
  int my_i[QB], my_h[QB], my_lim[QB];
  bool row_ok[QB];
  bf16x8 qf[QB][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = r0 + 16 * QB * qh + 16 * qb + lc;
    row_ok[qb] = row < rows;
    my_i[qb] = row_ok[qb] ? row / G : 0;
    my_h[qb] = kvh * G + (row_ok[qb] ? row % G : 0);
    my_lim[qb] = a.cache_only ? P : P + min(W, (my_i[qb] / B + 1) * B);
    if (row_ok[qb]) {
      const __bf16* qp =
          (const __bf16*)a.q + (((size_t)rb * a.hq + my_h[qb]) * a.wmax + my_i[qb]) * D;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[qb][s] = *(const bf16x8*)(qp + 32 * s + 8 * lg);
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[qb][s] = bf16x8{};
    }
  }
  const bool wave_active = (r0 + 16 * QB * qh) < rows;
  // Retire the Q loads (and the first tile) here: left pending, they would
  // make the first use in the tile loop wait on the in-order load counter
  // every iteration, i.e. on the prefetched tiles too.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);

  f32x4 o[DBLK][QB];
#pragma unroll
  for (int d = 0; d < DBLK; ++d)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[d][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_run[qb] = kNegInf, l_run[qb] = 0.f;
  const float c2 = a.c2;

  auto compute = [&](auto J, int t) {
    const char* Ks = stage_buf<decltype(J)::value, SB>() + tg * 2 * TILE;
    const lds_char* Vs = (const lds_char*)(Ks + TILE);
    int lo, nv;
    tile_span(t, nct, P, k_end, lo, nv);
    // All LDS reads of the tile are issued first -- K fragments, then the
    // transposed V fragments -- so their latency is paid once and the V reads
    // complete while the scores and probabilities are computed.  Lane (lc, lg)
    // of a transposed read gets V[key 32kh + 4lg + e][dim 16d + lc] for e < 4
    // (and +16 keys from the second read): k-slots 8lg..8lg+7 of the PV
    // product, in the same key order as the lane's probabilities.
    bf16x8 ka[2][KSTEPS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int n = 32 * kh + 16 * kb + lc;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        ka[kb][s] = *(const bf16x8*)(Ks + n * RS + (((4 * s + lg) ^ swz<D>(n)) << 4));
    }
    bf16x8 va[DBLK];
    {
      const int vr = 32 * kh + 4 * lg + (lc >> 2);
      const int vbyte = (lc & 1) << 3;
#pragma unroll
      for (int d = 0; d < DBLK; ++d) {
        const int cidx = 2 * d + ((lc & 3) >> 1);
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(Vs + vr * RS + ((cidx ^ swz<D>(vr)) << 4) + vbyte));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(Vs + (vr + 16) * RS + ((cidx ^ swz<D>(vr + 16)) << 4) + vbyte));
        const i16x8 both = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
        va[d] = __builtin_bit_cast(bf16x8, both);
      }
    }
    // S^T for this wave's 32 keys x 16 QB queries: [key block][query block].
    f32x4 sc[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][s], qf[qb][s], sc[kb][qb], 0, 0, 0);
      }
    }
    // Masking is needed on a partial tile and where a row's visible keys end.
    const int kk0 = 32 * kh + 4 * lg;  // key within the tile of sc[0][*][0]
    if (nv < kKTile || lo + kKTile > k_full) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int lim = min(nv, my_lim[qb] - lo);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kk0 + 16 * kb + r >= lim) sc[kb][qb][r] = kNegInf;
      }
    }
    bf16x8 pf[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kb][qb][r]);
      }
      // Lazy rescaling: the reference max m_run only moves when some score
      // exceeds it by more than kSlack (base-2 units), so in the steady state
      // no cross-lane reduction is needed; probabilities then stay <= 2^kSlack.
      if (__any(mx * c2 > m_run[qb] + kSlack)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[qb], mx * c2);
        const float alpha = (m_run[qb] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
#pragma unroll
        for (int d = 0; d < DBLK; ++d) o[d][qb] *= alpha;
        l_run[qb] *= alpha;
        m_run[qb] = m_new;
      }
      const float m_use = (m_run[qb] == kNegInf) ? 0.f : m_run[qb];
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][qb][r], c2, -m_use));
          ps += p;
          pf[qb][4 * kb + r] = (__bf16)p;
        }
      }
      l_run[qb] += ps;  // this lane's keys only; lanes are summed once at the end
    }
    // O^T += V^T P^T over this wave's 32 keys.
#pragma unroll
    for (int d = 0; d < DBLK; ++d) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        o[d][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[d], pf[qb], o[d][qb], 0, 0, 0);
    }
  };

  if constexpr (TG == 2) {
    // As below, per group: stage 0 of the group holds its tile k on entry to
    // each pair of steps.  Nothing is requested past a group's last tile.
    int k = 0;
    for (; k + 2 <= n_steps; k += 2) {
      tile_barrier();
      if (k + 1 < n_g) issue(ic<1>{}, gt(k + 1));
      if (wave_active && k < n_g) compute(ic<0>{}, gt(k));
      tile_barrier();
      if (k + 2 < n_g) issue(ic<0>{}, gt(k + 2));
      if (wave_active && k + 1 < n_g) compute(ic<1>{}, gt(k + 1));
    }
    if (k < n_steps) {
      tile_barrier();
      if (wave_active && k < n_g) compute(ic<0>{}, gt(k));
    }
  } else if (n_tiles > 0) {
    // The tile after the last is issued too (re-reading the last tile, a
    // cache hit) so that every wait covers exactly one tile; it is drained
    // before the stages are reused below.
    // Stage 0 holds tile i on entry to each pair (tile 0 was requested
    // before the query loads).  The barrier at the top of
    // a step both publishes the tile every wave loaded and retires the reads
    // of the tile before it, whose stage the next load then refills.
    int i = 0;
    for (; i + 2 <= n_tiles; i += 2) {
      tile_barrier();
      issue(ic<1>{}, tile_at(i + 1));
      if (wave_active) compute(ic<0>{}, t_lo + i);
      tile_barrier();
      issue(ic<0>{}, tile_at(i + 2));
      if (wave_active) compute(ic<1>{}, t_lo + i + 1);
    }
    if (i < n_tiles) {  // odd tail
      tile_barrier();
      if (wave_active) compute(ic<0>{}, t_lo + i);
    }
  }

  // Per-lane partial sums to per-query sums (the 4 lanes of a query column).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }

  // Merge the two key halves: the wave of key half 1 hands (m, l, O) to the
  // wave of key half 0 with the same query half through LDS (same lane,
  // same register layout).
  tile_barrier();  // no load in flight, no tile read pending: the stages are free
  if constexpr (TG == 2) {
    // Three waves per query half hand their state to the wave of key half 0
    // in group 0: slot c = kh + 2 tg - 1.  Slots 0 and 1 of both query halves
    // fill stage 0; slot 2 and the (m, l) pairs go to stage 1.
    constexpr int SLOT = QB * DBLK * 64 * 4;  // floats of one wave's O
    static_assert(4 * SLOT * 4 <= SB && (2 * SLOT + 6 * QB * 64 * 2) * 4 <= SB,
                  "four-wave merge area fits the stages");
    float* xo0 = (float*)stage_buf<0, SB>();
    float* xo1 = (float*)stage_buf<1, SB>();
    float* xml = xo1 + 2 * SLOT;
    auto slot_o = [&](int c) { return c < 2 ? xo0 + (qh * 2 + c) * SLOT : xo1 + qh * SLOT; };
    auto slot_ml = [&](int c) { return xml + (qh * 3 + c) * (QB * 64 * 2); };
    const int c_me = kh + 2 * tg - 1;
    if (c_me >= 0 && wave_active) {
      float* xo = slot_o(c_me);
      float* ml = slot_ml(c_me);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d) *(f32x4*)(xo + ((qb * DBLK + d) * 64 + lane) * 4) = o[d][qb];
        ml[(qb * 64 + lane) * 2 + 0] = m_run[qb];
        ml[(qb * 64 + lane) * 2 + 1] = l_run[qb];
      }
    }
    __syncthreads();
    if (c_me >= 0 || !wave_active) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mc[3], lcs[3];
      float m = m_run[qb];
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        mc[c] = slot_ml(c)[(qb * 64 + lane) * 2 + 0];
        lcs[c] = slot_ml(c)[(qb * 64 + lane) * 2 + 1];
        m = fmaxf(m, mc[c]);
      }
      const float w0 = (m_run[qb] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m);
#pragma unroll
      for (int d = 0; d < DBLK; ++d) o[d][qb] *= w0;
      l_run[qb] *= w0;
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const float wc = (mc[c] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mc[c] - m);
        const float* xo = slot_o(c);
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
          o[d][qb] += *(const f32x4*)(xo + ((qb * DBLK + d) * 64 + lane) * 4) * wc;
        l_run[qb] += lcs[c] * wc;
      }
      m_run[qb] = m;
    }
  } else {
    float* xo = (float*)stage_buf<0, SB>() + (size_t)qh * (QB * DBLK * 64 * 4);  // [qb][d][lane][4]
    float* xml = (float*)stage_buf<1, SB>() + qh * (QB * 64 * 2);
    if (kh == 1 && wave_active) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d) *(f32x4*)(xo + ((qb * DBLK + d) * 64 + lane) * 4) = o[d][qb];
        xml[(qb * 64 + lane) * 2 + 0] = m_run[qb];
        xml[(qb * 64 + lane) * 2 + 1] = l_run[qb];
      }
    }
    __syncthreads();
    if (kh == 1 || !wave_active) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m1 = xml[(qb * 64 + lane) * 2 + 0], l1 = xml[(qb * 64 + lane) * 2 + 1];
      const float m = fmaxf(m_run[qb], m1);
      const float w0 = (m_run[qb] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m);
      const float w1 = (m1 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
        o[d][qb] = o[d][qb] * w0 + *(const f32x4*)(xo + ((qb * DBLK + d) * 64 + lane) * 4) * w1;
      l_run[qb] = l_run[qb] * w0 + l1 * w1;
      m_run[qb] = m;
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (!row_ok[qb]) continue;
    if (nsplit == 1) {
      const float inv = 1.0f / l_run[qb];
      __bf16* op =
          (__bf16*)a.out + (((size_t)rb * a.hq + my_h[qb]) * a.wmax + my_i[qb]) * D;
#pragma unroll
      for (int d = 0; d < DBLK; ++d) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)(o[d][qb][r] * inv);
        *(bf16x4*)(op + 16 * d + 4 * lg) = v;
      }
      if (a.lse != nullptr && lg == 0)
        a.lse[((size_t)rb * a.hq + my_h[qb]) * a.wmax + my_i[qb]] =
            (m_run[qb] + log2f(l_run[qb])) * kLn2;
    } else {
      const size_t row_slot = (size_t)u * a.slot_rows + 16 * QB * qh + 16 * qb + lc;
      float* wp = a.ws_o + row_slot * D;
#pragma unroll
      for (int d = 0; d < DBLK; ++d) *(f32x4*)(wp + 16 * d + 4 * lg) = o[d][qb];
      if (lg == 0) {
        a.ws_ml[row_slot * 2 + 0] = m_run[qb];
        a.ws_ml[row_slot * 2 + 1] = l_run[qb];
      }
    }
  }
}

}  // namespace

int attn_bf16_wgs_per_cu(int head_dim) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  if (head_dim == 128)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<128, 2, 0, 1, false>,
                                                     kAttnThreads, 0);
  else if (head_dim == 64)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<64, 2, 0, 1, false>,
                                                     kAttnThreads, 0);
  return e == hipSuccess ? n : 0;
}

template <int D, int QB, int PAGED, int TG>
void launch_policy(const AttnArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.remap)
    hipLaunchKernelGGL((attn_bf16_kernel<D, QB, PAGED, TG, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, QB, PAGED, TG, false>), grid, block, 0, s, a);
}

template <int PAGED, int TG>
hipError_t launch_bf16(const AttnArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid(a.n_units), block(kAttnThreads * TG);
  const bool narrow = a.qrows == 32;
  if (head_dim == 128 && !narrow) launch_policy<128, 2, PAGED, TG>(a, grid, block, s);
  else if (head_dim == 128) launch_policy<128, 1, PAGED, TG>(a, grid, block, s);
  else if (head_dim == 64 && !narrow) launch_policy<64, 2, PAGED, TG>(a, grid, block, s);
  else if (head_dim == 64) launch_policy<64, 1, PAGED, TG>(a, grid, block, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int TG>
hipError_t launch_tg(const AttnArgs& a, int head_dim, bool paged, hipStream_t s) {
  if (!paged) return launch_bf16<0, TG>(a, head_dim, s);
  return a.bsz >= 16 ? launch_bf16<2, TG>(a, head_dim, s) : launch_bf16<1, TG>(a, head_dim, s);
}

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool paged, hipStream_t s) {
  return a.wide ? launch_tg<2>(a, head_dim, paged, s) : launch_tg<1>(a, head_dim, paged, s);
}

}  // namespace d2f
