// Block-causal window attention for grouped-query launches: bf16 inputs,
// fp32 accumulation, v_mfma_f32_16x16x32_bf16, many query rows per K/V tile.
//
// What is computed is what attn_bf16.hip computes ([D2F-wiki] "블록 단위 인과
// 어텐션"; [D2F-review] "쉽게 이해하기"): window row i of a request sees every
// cached key and the window keys of its own block and of every earlier
// window block.
//
// Why a second kernel.  With grouped query heads (Hq / Hkv = G > 1) a KV
// head's keys are shared by G x W query rows, and the attention becomes
// compute-bound; the kernel in attn_bf16.hip gives each K/V tile it loads to
// 64 query rows, which leaves the matrix cores waiting on the tile stream:
// streaming tiles from L2 into LDS reaches roughly 60-100 GB/s per CU on
// MI355X, while 64 rows per 32 KB tile would need ~150 GB/s per CU to keep
// the MFMA pipes full.  Here one workgroup of eight waves gives every tile to
// up to 256 query rows (the unit's rows, a multiple of 16 chosen by the
// planner), so the same stream feeds up to 4x the MFMA work.
//
// Design (one workgroup = 8 waves = one work unit, one workgroup per CU):
//  * Units of more than 8 blocks: the unit's 16-row query blocks are dealt
//    to the waves round-robin (block b -> wave b mod 8), so a wave owns one
//    or two blocks and the two waves that share a SIMD (w and w + 4) never
//    hold more blocks between them than any other pair plus one.  Every wave
//    runs over every key of the unit: it owns its rows' online-softmax state
//    outright, and no join is needed.
//  * Units of at most 8 blocks (KS): waves 0-3 take keys 0-31 of every tile
//    and waves 4-7 keys 32-63.  Each group holds all of the unit's blocks,
//    dealt round-robin over its four waves, and the second group's deal is
//    rotated by two waves, so a SIMD's pair of waves holds one block and its
//    neighbour's two rather than two and two: a 6-block unit puts three
//    half-tile blocks on every SIMD instead of four on two of them and two
//    on the others.  Each wave keeps the online-softmax state of its keys;
//    at the end the second group hands (m, l, O) to the first through LDS
//    and the first joins the two exactly.  Measured on MI355X (Dream-7B
//    shape, block 32, 96-row units): 43.2-44.7 vs 47.0-48.1 us.  Each step
//    of this mode reads the next tile's V^T fragments at its end, before
//    the barrier.  In units of at most 3 blocks, two of the waves left
//    without a block issue all of the tile loads, and the others none.
//  * Keys are processed in halves of 32, software-pipelined within a wave:
//    while the matrix cores compute the scores of half h + 1, the vector
//    units turn the scores of half h into probabilities; then half h's PV
//    product.  The K fragments of half h + 1 are read from LDS first, then
//    the V^T fragments of half h: LDS returns reads in order, so the score
//    MFMAs wait only for theirs, and the V^T reads complete behind them.
//  * K/V tiles of 64 keys go HBM -> LDS with the direct loads through a
//    four-stage ring: two tiles stream in while one is computed, one barrier
//    per tile.  Paged caches change only the loader (see issue_paged).
//  * The reference maximum starts at -FLT_MAX and is raised only when a
//    half's probability sum exceeds 2^kSlack (see probs).
//  * Scores are computed transposed (S^T = K Q^T), so a lane holds one query
//    and the keys of its column, which is the B-operand layout of the PV
//    product O^T = V^T P^T; V^T is read with ds_read_b64_tr_b16 and the LDS
//    rows are swizzled as in attn_bf16.hip (conflict-free for both reads).
//  * Online softmax in base 2 with per-lane partial sums.
//  * A unit covers all keys of its rows and writes O in bf16 and the LSE
//    (the planner never cuts these launches' keys into ranges).
//
// Measured on MI355X (8 requests, 28 query / 4 KV heads, 2048 cached keys,
// three window blocks of 64: 1344 query rows per KV head): 64-68 us against
// 76 us for the first version of this kernel and 81-85 us for attn_bf16.hip
// on the same machines; 2-4% of that came from testing a half for masking
// against two precomputed half indices (h_cmask, h_wmask) instead of
// recomputing its tile's span, and 3-6% from the load policy being a
// template argument.  Tried and not faster: scheduling-group barriers
// that interleave one MFMA with four vector instructions (81 us), a raised
// wave priority while the scores' MFMAs issue (76 us), LDS addresses
// recomputed in every step to save registers (73 us), a ring of three or
// five tiles (within noise), the V^T reads after the scores' MFMAs instead
// of between the K reads and them (+3%), and two groups of four waves that
// split each tile's keys and join through LDS at the end, which halves the
// LDS reads per tile (no gain at 48 to 128 rows per unit).  Cutting the keys
// into ranges merged by attn_merge.hip lost to the merge pass at every
// size tried, and so did wave groups a phase apart (waves 0-3 and 4-7
// placing the tile's barrier on either side of a softmax phase: 54 vs 50 us
// for two window blocks of 32).  Also slower in the key-split mode: every
// LDS read issued a step ahead into a second register set (block 16: 33.1 vs
// 31.5 us), a barrier every second step (33.5 vs 31.1 us), and waves 4-7
// forming their probabilities before their score MFMAs (32.7 vs 31.1 us).
// What bounds it: per 64-key tile and SIMD,
// the matrix work (3 blocks x 512 cycles), the softmax's vector work
// (v_exp_f32 runs at a quarter of the VALU rate) and the LDS reads (K
// fragments through ds_read_b128 at ~237 B/clock per CU, V^T through
// ds_read_b64_tr_b16 at ~218) are of the same size.  A probe that issues the
// same instruction mix with no dependencies reaches about 1.25 PFLOP/s for
// this block layout, against 0.7 here: the rest is how the waves' matrix
// and vector phases overlap.

#include "attn_lds.h"

namespace d2f {
namespace {

constexpr int kGqaWaves = kGqaThreads / 64;
constexpr int kGqaKsMaxRows = 128;  // units up to 8 blocks split each tile's keys
constexpr int kGqaStages = 4;
constexpr float kSlackSum = 256.f;  // 2^kSlack: largest per-lane probability sum kept

// s_waitcnt immediate: vmcnt(v) and lgkmcnt(0) (expcnt not waited).
constexpr int wait_vm_lgkm0(int v) { return (v & 15) | (((v >> 4) & 3) << 14) | 0x70; }

// PAGED: K/V rows are found through the page tables (AttnArgs), in pages of
// a power of two >= 8 rows.  SHARED (a.remap): several units read each KV
// head's tiles, so units are numbered XCD-contiguously and the tile loads keep
// the default cache policy; otherwise they are non-temporal.  KS: the unit
// has at most 8 blocks and its two wave groups split each tile's keys.
template <int D, bool PAGED, bool SHARED, bool KS>
__global__ __launch_bounds__(kGqaThreads, 1) void attn_gqa_kernel(const AttnArgs a) {
  constexpr int RS = D * 2;              // LDS row bytes
  constexpr int KSTEPS = D / 32;         // MFMA k-steps over head_dim
  constexpr int DBLK = D / 16;           // 16-dim blocks of the output
  constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
  constexpr int TILE = kKTile * RS;      // bytes per K (or V) tile
  constexpr int RPB = 1024 / RS;         // rows per 1 KB direct-load block
  constexpr int NBLK = TILE / 1024;      // 1 KB blocks per tensor per tile
  constexpr int LPW = NBLK / kGqaWaves;  // blocks per wave per tensor per tile
  static_assert(LPW >= 1 && LPW * kGqaWaves == NBLK, "8 waves cover a tile in 1 KB blocks");
  constexpr int LOADS = 2 * LPW;         // direct loads per wave per tile
  constexpr int SB = 2 * TILE;           // bytes per LDS stage: [K tile][V tile]
  constexpr int NST = kGqaStages;

  const int u = SHARED ? xcd_remap(blockIdx.x, a.n_units) : (int)blockIdx.x;
  const int ri = find_req(a, u);
  const int rb = a.req[ri].b, P = a.req[ri].prefix, W = a.req[ri].win;
  const int qtiles = a.req[ri].qtiles;
  const int local = u - a.req[ri].unit_base;
  const int qt = local % qtiles;
  const int kvh = local / qtiles;
  const int G = a.group, B = a.bsz;
  const int rows = G * W;
  const int R = a.qrows;  // query rows per unit (a multiple of 16)
  const int r0 = qt * R;
  const int k_end = unit_key_end(a, qt, R, P, W, G, B);  // last key any row sees
  const int k_full = a.cache_only ? P : P + min(W, ((r0 / G) / B + 1) * B);  // every row sees
  const int nct = cache_tiles(P);
  const int n = nct + window_tiles(P, k_end);  // tiles of the unit (all its keys)
  // Halves that need a mask: those of a partial last cache tile from the
  // first one that ends past P, and the window halves from the first one
  // that ends past k_full (the key end every row of the unit reaches).
  const int h_cmask = (P & 63) ? 2 * (nct - 1) + ((P & 63) >= 32 ? 1 : 0) : 2 * nct;
  const int h_wmask = 2 * nct + (k_full - P) / 32;

  const size_t head_c = (((size_t)rb * a.hkv + kvh) * (size_t)a.cap + a.req[ri].key_off) * D;
  const size_t head_w = ((size_t)rb * a.hkv + kvh) * (size_t)a.wmax * D;
  const __bf16* kc = (const __bf16*)a.kc + head_c;
  const __bf16* vc = (const __bf16*)a.vc + head_c;
  const __bf16* kw = (const __bf16*)a.kw + head_w;
  const __bf16* vw = (const __bf16*)a.vw + head_w;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lc = lane & 15, lg = lane >> 4;
  const int nblk = (min(R, rows - r0) + 15) >> 4;  // 16-row blocks with a valid row
  // KS (units of at most 8 blocks): waves 0-3 take keys 0-31 of every tile,
  // waves 4-7 keys 32-63.  Waves 0-3 hold blocks w, w + 4; wave 4 + w holds
  // the blocks of wave (w + 2) mod 4, so the two waves of a SIMD (w and
  // w + 4) hold at most three blocks between them when a unit has six.
  const int kg = KS ? (wave >> 2) : 0;                  // key half of this wave
  const int wb = KS ? (((wave & 3) + 2 * kg) & 3) : wave;  // its first block
  constexpr int BSTRIDE = KS ? 4 : kGqaWaves;
  const int nq = (wb < nblk) + (wb + BSTRIDE < nblk);  // this wave's blocks: 0, 1, 2
  // Who issues a tile's direct loads (the load mode LM of this wave).  The
  // waves that hold the most blocks set the pace of every step, so they
  // issue none (LM 2) and lighter waves issue all of them:
  //  * key-split units of at most 3 blocks leave waves 3 and 5 without a
  //    block; those two take the even and the odd 1 KB blocks (LM 1);
  //  * otherwise, on each SIMD the wave of the pair (s, s + 4) with fewer
  //    blocks, the second one on a tie, takes blocks s, s + 4, ... (LM 3).
  // Measured on MI355X, Dream-shaped calls, before -> after: block 16
  // 30.8-31.0 -> 27.5-27.6 us, block 32 40.0-40.2 -> 37.9-38.0 us, block 64
  // 59.0-59.3 -> 56.9-57.3 us.  Paged caches keep a share of every tile on
  // every wave (LM 0): a wave's page entries cover its own 8-row group.
  auto blocks_of = [&](int w) {
    const int g = KS ? (w >> 2) : 0;
    const int b = KS ? (((w & 3) + 2 * g) & 3) : w;
    return (b < nblk) + (b + BSTRIDE < nblk);
  };
  const int simd = wave & 3;
  const bool two_loaders = KS && nblk <= 3;
  const int lmode =
      PAGED ? 0
      : two_loaders ? ((wave == 3 || wave == 5) ? 1 : 2)
                    : (wave == (blocks_of(simd) < blocks_of(simd + 4) ? simd : simd + 4) ? 3 : 2);
  const int li = wave == 3 ? 0 : 1;  // LM 1: loader index

  // Loader: wave w copies 1 KB blocks w, w + 8, ... of each of K and V (in
  // the loader mode above, loader i copies blocks i, i + 2, ...); lane
  // l of block j carries the 16 bytes that belong at LDS position (row
  // RPB j + l / CPR, chunk l % CPR), i.e. global chunk (l % CPR) ^ swz(row).
  // A tile's rows all come from the cache or all from the window, so the
  // base pointers are uniform; rows past a partial tile's end re-read its
  // last row (in bounds; the mask gives them zero weight).
  // Paged loader: wave w copies the tile's consecutive blocks LPW w ..
  // LPW w + LPW - 1, i.e. its rows 8 w .. 8 w + 7 (8 rows at either head
  // dim), which start at a multiple of 8 of the cache or the window and so
  // lie in one page: the load's base address stays uniform.  Rows past a
  // partial tile's end re-read its last row, which lies in the same 8-row
  // group or, for a group wholly past the end, is the group's only row.
  // The wave's page of tile t: row group key0 of the cache or window, page
  // index key0 >> shift, first row of that page relative to the tile.
  static_assert(RPB * LPW == 8, "a wave loads 8 rows of a tile");
  const size_t page_bytes = (size_t)a.hkv * B * D * sizeof(__bf16);
  auto page_slot = [&](int t, const int32_t*& table, int& pi, int& row0)
      __attribute__((always_inline)) {
    int lo, nv;
    tile_span(t, nct, P, k_end, lo, nv);
    const bool in_cache = t < nct;
    const int r0 = in_cache ? lo : lo - P;  // first row's index in the cache or the window
    table = in_cache ? a.page_table + (size_t)rb * a.table_stride
                     : a.win_pages + (size_t)rb * (a.wmax / B);
    const int key0 = r0 + min(RPB * LPW * wave, nv - 1);
    pi = key0 >> a.page_shift;
    row0 = (pi << a.page_shift) - r0;
  };
  // Table entries of 64 tiles at a time, one per lane (lane k: tile base +
  // k), requested 32 tiles before they are needed; a tile's entry is then
  // a lane of a register loaded long before, and is clamped to the pool
  // where it is used (a bad entry reads the wrong rows, never outside the
  // pool).  The entries are loaded by an inline-asm load that waits for it
  // in the same block: loaded by the compiler, the register made it wait
  // for every load in flight -- the tile stream included -- after each
  // barrier; this way the wait happens once per 32 tiles (measured on
  // MI355X, Dream-shaped paged calls: block 16 37.4 vs 40.2 us, block 32
  // 48.8-49.1 vs 51.5 us).
  auto entries = [&](int base) __attribute__((always_inline)) {
    const int32_t* table;
    int pi, row0;
    page_slot(min(base + lane, n - 1), table, pi, row0);
    int v;
    asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)"
                 : "=v"(v)
                 : "v"(table + pi)
                 : "memory");
    return v;
  };
  int pe_cur = 0, pe_next = 0, pe_base = 0;
  auto issue_paged = [&](auto J, int t) __attribute__((always_inline)) {
    if (t == pe_base + 64) {
      pe_cur = pe_next;
      pe_base += 64;
    }
    if (t == pe_base + 32 && pe_base + 64 < n) pe_next = entries(pe_base + 64);
    const int page =
        min(max(__builtin_amdgcn_readlane(pe_cur, t - pe_base), 0), a.n_pages - 1);
    const int32_t* table;
    int pi, row0;
    page_slot(t, table, pi, row0);
    const unsigned sb = (unsigned)(uintptr_t)stage_buf<decltype(J)::value, SB>();
    int lo, nv;
    tile_span(t, nct, P, k_end, lo, nv);
    const size_t pbase = (size_t)page * page_bytes + (size_t)kvh * B * D * sizeof(__bf16);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = LPW * wave + i;
      const int row = RPB * blk + lane / CPR;
      const int off = (min(row, nv - 1) - row0) * RS + 16 * ((lane % CPR) ^ swz<D>(row));
      load_kv16<SHARED>((const char*)a.kc + pbase, off, sb + blk * 1024);
      load_kv16<SHARED>((const char*)a.vc + pbase, off, sb + TILE + blk * 1024);
    }
  };
  auto issue = [&](auto J, int t, auto LMc) __attribute__((always_inline)) {
    constexpr int LM = decltype(LMc)::value;
    if constexpr (PAGED) {
      issue_paged(J, t);
      return;
    }
    if constexpr (LM == 2) return;
    const unsigned sb = (unsigned)(uintptr_t)stage_buf<decltype(J)::value, SB>();
    int lo, nv;
    tile_span(t, nct, P, k_end, lo, nv);
    const bool in_cache = t < nct;
    const size_t o = (size_t)(in_cache ? lo : lo - P) * D;
    const char* kb = (const char*)((in_cache ? kc : kw) + o);
    const char* vb = (const char*)((in_cache ? vc : vw) + o);
    constexpr int PER = LM == 1 ? NBLK / 2 : LM == 3 ? NBLK / 4 : LPW;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = LM == 1 ? li + 2 * i : LM == 3 ? simd + 4 * i : wave + kGqaWaves * i;
      const int row = RPB * blk + lane / CPR;
      const int off = min(row, nv - 1) * RS + 16 * ((lane % CPR) ^ swz<D>(row));
      load_kv16<SHARED>(kb, off, sb + blk * 1024);
      load_kv16<SHARED>(vb, off, sb + TILE + blk * 1024);
    }
  };
  // Workgroup barrier between phases: this wave's LDS reads have returned
  // and at most `pending` tiles of its direct loads are still in flight (1:
  // the tile requested last; 2: the last two), for a wave of load mode LM.
  auto barrier = [&](int pending, auto LMc) __attribute__((always_inline)) {
    constexpr int LM = decltype(LMc)::value;
    constexpr int NL = LM == 0 ? LOADS : LM == 1 ? NBLK : LM == 3 ? NBLK / 2 : 0;
    if (pending >= 2) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * NL));
    else if (pending == 1) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NL));
    else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Tiles 0, 1 and 2 are requested before the queries are loaded (paged:
  // after the first 64 tiles' page entries).
  if constexpr (PAGED) {
    if (n > 0) pe_cur = entries(0);
  }
  auto prologue = [&](auto LMc) __attribute__((always_inline)) {
    if (0 < n) issue(ic<0>{}, 0, LMc);
    if (1 < n) issue(ic<1>{}, 1, LMc);
    if (2 < n) issue(ic<2>{}, 2, LMc);
  };
  // Runs f with this wave's load mode as a compile-time constant.
  auto with_lm = [&](auto&& f) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      f(ic<0>{});
    } else {
      if (lmode == 1) f(ic<1>{});
      else if (lmode == 3) f(ic<3>{});
      else f(ic<2>{});
    }
  };
  with_lm(prologue);

  // The wave's query rows: block qb is the unit's block wave + 8 qb; lane
  // (lc, lg) holds row lc of it (MFMA column lc).
  int my_i[2], my_h[2], my_lim[2];
  bool row_ok[2];
  bf16x8 qf[2][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = r0 + 16 * (wb + BSTRIDE * qb) + lc;
    row_ok[qb] = qb < nq && row < r0 + R && row < rows;
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
  // Retire the query loads and the first tiles here, so that no wait in the
  // loop has to count them; the barrier publishes tile 0 (and 1, 2).
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  if (n > 0) barrier(0, ic<0>{});

  f32x4 o[DBLK][2];
#pragma unroll
  for (int d = 0; d < DBLK; ++d) o[d][0] = o[d][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Reference maxima start at the finite sentinel -FLT_MAX (see probs).
  float m_run[2] = {-__FLT_MAX__, -__FLT_MAX__}, l_run[2] = {0.f, 0.f};
  const float c2 = a.c2;
  // The keys are processed in halves of 32 (half h: keys 32 (h & 1) ..
  // 32 (h & 1) + 31 of tile h >> 1), software-pipelined within each wave:
  // step h computes the scores of half h + 1 on the matrix cores while the
  // vector units turn the scores of half h into probabilities, then adds
  // half h's P V product, then masks half h + 1 and raises its reference
  // maximum when needed.  Scores: key block kb (16 keys) x query block qb;
  // lane (lc, lg) holds keys 16 kb + 4 lg + r of the half for query column
  // lc.  Probabilities in the PV B-operand layout: k-slot 8 lg + 4 kb + r is
  // key 16 kb + 4 lg + r of the half.
  f32x4 sa[2][2], sb[2][2];  // scores of alternate halves: [kb][qb]
  bf16x8 pf[2];              // probabilities of the half whose PV is next: [qb]

  // K fragments of half h (its tile in stage J): key block kb, k-step st.
  auto kread = [&](auto J, auto QBc, int h, bf16x8 (&ka)[2][KSTEPS]) __attribute__((always_inline)) {
    constexpr int QB = decltype(QBc)::value;
    if constexpr (QB > 0) {
      const char* Ks = stage_buf<decltype(J)::value, SB>();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * (h & 1) + 16 * kb + lc;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
          ka[kb][st] = *(const bf16x8*)(Ks + row * RS + (((4 * st + lg) ^ swz<D>(row)) << 4));
      }
    }
  };
  // S^T of a half from its K fragments into s.
  auto smma = [&](auto QBc, const bf16x8 (&ka)[2][KSTEPS], f32x4 (&s)[2][2])
      __attribute__((always_inline)) {
    constexpr int QB = decltype(QBc)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][st], qf[qb][st], s[kb][qb], 0, 0, 0);
      }
  };
  // Mask half h's scores where needed (a partial tile, a row's visible keys
  // ending).
  auto prepare = [&](auto QBc, int h, f32x4 (&s)[2][2]) __attribute__((always_inline)) {
    constexpr int QB = decltype(QBc)::value;
    if constexpr (QB > 0) {
      if ((h >= h_cmask && h < 2 * nct) || h >= h_wmask) {
        int lo, nv;
        tile_span(h >> 1, nct, P, k_end, lo, nv);
        const int klo = lo + 32 * (h & 1), nvh = nv - 32 * (h & 1);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int lim = min(nvh, my_lim[qb] - klo);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * kb + 4 * lg + r >= lim) s[kb][qb][r] = kNegInf;
        }
      }
    }
  };
  // Probabilities of a half from its scores s against the reference maximum
  // m_run (base-2 units), in straight-line code; a lane's sum ps bounds each
  // of its probabilities.  Only when some lane's sum exceeds 2^kSlack (so a
  // probability may have) -- and on the first half, where m_run is still the
  // finite sentinel -FLT_MAX and every visible score gives +inf -- is the
  // reference raised to the half's true maximum, O and l rescaled and the
  // probabilities recomputed.  The reference only moves to maxima actually
  // seen, so the row's largest score keeps a probability >= 1.
  auto probs = [&](auto QBc, f32x4 (&s)[2][2]) __attribute__((always_inline)) {
    constexpr int QB = decltype(QBc)::value;
    float ps[QB > 0 ? QB : 1];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ps[qb] = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], c2, -m_run[qb]));
          ps[qb] += p;
          pf[qb][4 * kb + r] = (__bf16)p;
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (__any(!(ps[qb] <= kSlackSum))) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[qb], mx * c2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
#pragma unroll
        for (int d = 0; d < DBLK; ++d) o[d][qb] *= alpha;
        l_run[qb] *= alpha;
        m_run[qb] = m_new;
        ps[qb] = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], c2, -m_new));
            ps[qb] += p;
            pf[qb][4 * kb + r] = (__bf16)p;
          }
        }
      }
      l_run[qb] += ps[qb];
    }
  };
  // V^T fragments of half h (its tile in stage J): lane (lc, lg) of a
  // transposed read gets V[key 4 lg + e][dim 16 d + lc] of the half (e < 4),
  // and 16 keys on from the second read, i.e. k-slots 8 lg .. 8 lg + 7 in
  // the probabilities' key order.
  auto vload = [&](auto J, auto QBc, int h, bf16x8 (&va)[DBLK]) __attribute__((always_inline)) {
    constexpr int QB = decltype(QBc)::value;
    if constexpr (QB > 0) {
      const lds_char* Vs =
          (const lds_char*)(stage_buf<decltype(J)::value, SB>() + TILE);
      const int vr = 32 * (h & 1) + 4 * lg + (lc >> 2);
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
  };
  // O^T += V^T P^T with the fragments of vload.
  auto pv = [&](auto QBc, const bf16x8 (&va)[DBLK]) __attribute__((always_inline)) {
    constexpr int QB = decltype(QBc)::value;
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        o[d][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[d], pf[qb], o[d][qb], 0, 0, 0);
  };

  // Tile t sits in stage t mod 4.  Step 2t (half 0 of tile t) reads only
  // tile t.  Step 2t + 1 reads tile t (V of half 1) and tile t + 1 (K of its
  // half 0): it starts with a barrier after which tile t + 1 is in LDS (this
  // wave waits for its own loads of it; tile t + 2 may stay in flight) and
  // every wave is past step 2t - 1, the last to read tile t - 1, whose stage
  // then receives tile t + 3.
  // Within a step the K fragments of the next half are requested before
  // the V^T fragments of this one: LDS returns reads in order, and the
  // scores' MFMAs, which come first, then wait only for the K reads.
  auto run = [&](auto QBc, auto LMc) __attribute__((always_inline)) {
    {
      bf16x8 ka[2][KSTEPS];
      kread(ic<0>{}, QBc, 0, ka);
      smma(QBc, ka, sa);
    }
    prepare(QBc, 0, sa);
    auto tile = [&](auto J, int t) __attribute__((always_inline)) {
      constexpr int JK = decltype(J)::value;
      bf16x8 va[DBLK];
      // step 2t: scores of half 1 (same tile) while half 0 becomes P.
      {
        bf16x8 ka[2][KSTEPS];
        kread(J, QBc, 2 * t + 1, ka);
        vload(J, QBc, 2 * t, va);
        smma(QBc, ka, sb);
      }
      probs(QBc, sa);
      pv(QBc, va);
      prepare(QBc, 2 * t + 1, sb);
      // step 2t + 1: the next tile's first half.
      barrier(t + 2 < n ? 1 : 0, LMc);
      if (t + 3 < n) issue(ic<(JK + 3) % NST>{}, t + 3, LMc);
      if (t + 1 < n) {
        bf16x8 ka[2][KSTEPS];
        kread(ic<(JK + 1) % NST>{}, QBc, 2 * t + 2, ka);
        vload(J, QBc, 2 * t + 1, va);
        smma(QBc, ka, sa);
      } else {
        vload(J, QBc, 2 * t + 1, va);
      }
      probs(QBc, sb);
      pv(QBc, va);
      if (t + 1 < n) prepare(QBc, 2 * t + 2, sa);
    };
    for (int t = 0; t < n; t += NST) {
      tile(ic<0>{}, t);
      if (t + 1 < n) tile(ic<1>{}, t + 1);
      if (t + 2 < n) tile(ic<2>{}, t + 2);
      if (t + 3 < n) tile(ic<3>{}, t + 3);
    }
  };
  // KS: one half per tile.  Step t reads K of tile t + 1 (landed at barrier
  // t) after the barrier, and at its end, before barrier t + 1, the V^T
  // fragments of tile t + 1 that step t + 1 multiplies, so only the K reads
  // queue at the LDS behind the barrier (measured on MI355X, Dream-shaped
  // calls: block 16 31.1-31.3 vs 31.4-31.5 us, block 32 39.7-39.9 vs
  // 40.8-40.9 us).  Tile t - 1 is last read in step t - 2, so after barrier
  // t its stage receives tile t + 3.
  auto run_ks = [&](auto QBc, auto LMc) __attribute__((always_inline)) {
    bf16x8 va[DBLK];
    {
      bf16x8 ka[2][KSTEPS];
      kread(ic<0>{}, QBc, kg, ka);
      vload(ic<0>{}, QBc, kg, va);
      smma(QBc, ka, sa);
    }
    prepare(QBc, kg, sa);
    auto tile = [&](auto J, int t) __attribute__((always_inline)) {
      constexpr int JK = decltype(J)::value;
      f32x4 (&scur)[2][2] = (JK & 1) ? sb : sa;
      f32x4 (&snext)[2][2] = (JK & 1) ? sa : sb;
      barrier(t + 2 < n ? 1 : 0, LMc);
      if (t + 3 < n) issue(ic<(JK + 3) % NST>{}, t + 3, LMc);
      if (t + 1 < n) {
        bf16x8 ka[2][KSTEPS];
        kread(ic<(JK + 1) % NST>{}, QBc, 2 * t + 2 + kg, ka);
        smma(QBc, ka, snext);
      }
      probs(QBc, scur);
      pv(QBc, va);
      if (t + 1 < n) {
        vload(ic<(JK + 1) % NST>{}, QBc, 2 * t + 2 + kg, va);
        prepare(QBc, 2 * t + 2 + kg, snext);
      }
    };
    for (int t = 0; t < n; t += NST) {
      tile(ic<0>{}, t);
      if (t + 1 < n) tile(ic<1>{}, t + 1);
      if (t + 2 < n) tile(ic<2>{}, t + 2);
      if (t + 3 < n) tile(ic<3>{}, t + 3);
    }
  };
  if (n > 0) {
    with_lm([&](auto LMc) __attribute__((always_inline)) {
      constexpr int LM = decltype(LMc)::value;
      if constexpr (LM == 1) {
        if constexpr (KS) run_ks(ic<0>{}, LMc);  // the two loaders hold no block
      } else if constexpr (KS) {
        if (nq == 2) run_ks(ic<2>{}, LMc);
        else if (nq == 1) run_ks(ic<1>{}, LMc);
        else run_ks(ic<0>{}, LMc);
      } else {
        if (nq == 2) run(ic<2>{}, LMc);
        else if (nq == 1) run(ic<1>{}, LMc);
        else run(ic<0>{}, LMc);
      }
    });
  }

  // KS: waves 4-7 hand (m, l, O) of each block to the wave of keys 0-31
  // through LDS (same lane, same register layout); it joins the two exactly.
  if constexpr (KS) {
    constexpr int OB = DBLK * 4 * 64;  // floats of one block's O
    static_assert(4 * OB * 4 <= SB, "four blocks' O fit one stage");
    __builtin_amdgcn_s_waitcnt(kVmLgkmZero);
    __builtin_amdgcn_s_barrier();  // every wave is past its last read of the stages
    auto oslot = [&](int b) {
      return (b < 4 ? (float*)stage_buf<0, SB>() : (float*)stage_buf<1, SB>()) + (b & 3) * OB;
    };
    float* mlslot = (float*)stage_buf<2, SB>();
    if (kg == 1) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (qb >= nq) continue;
        const int b = wb + 4 * qb;
        float* xo = oslot(b);
#pragma unroll
        for (int d = 0; d < DBLK; ++d) *(f32x4*)(xo + (d * 64 + lane) * 4) = o[d][qb];
        mlslot[(b * 64 + lane) * 2 + 0] = m_run[qb];
        mlslot[(b * 64 + lane) * 2 + 1] = l_run[qb];
      }
    }
    __builtin_amdgcn_s_waitcnt(kVmLgkmZero);
    __builtin_amdgcn_s_barrier();
    if (kg == 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (qb >= nq) continue;
        const int b = wb + 4 * qb;
        const float* xo = oslot(b);
        const float m1 = mlslot[(b * 64 + lane) * 2 + 0];
        const float l1 = mlslot[(b * 64 + lane) * 2 + 1];
        const float m = fmaxf(m_run[qb], m1);
        const float w0 = __builtin_amdgcn_exp2f(m_run[qb] - m);
        const float w1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
          o[d][qb] = o[d][qb] * w0 + *(const f32x4*)(xo + (d * 64 + lane) * 4) * w1;
        l_run[qb] = l_run[qb] * w0 + l1 * w1;
        m_run[qb] = m;
      }
    }
  }

  // Per-lane partial sums to per-query sums (the 4 lanes of a query column),
  // then the rows' outputs.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!row_ok[qb] || kg != 0) continue;
    const float inv = 1.0f / l_run[qb];
    __bf16* op = (__bf16*)a.out + (((size_t)rb * a.hq + my_h[qb]) * a.wmax + my_i[qb]) * D;
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
  }
}

}  // namespace

template <int D, bool PAGED, bool KS>
void launch_gqa_ks(const AttnArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.remap) hipLaunchKernelGGL((attn_gqa_kernel<D, PAGED, true, KS>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((attn_gqa_kernel<D, PAGED, false, KS>), grid, block, 0, s, a);
}
// Units of at most kGqaKsMaxRows rows split each tile's keys between the two
// wave groups (KS); larger units give every wave all the keys of its blocks.
template <int D, bool PAGED>
void launch_gqa_policy(const AttnArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.qrows <= kGqaKsMaxRows) launch_gqa_ks<D, PAGED, true>(a, grid, block, s);
  else launch_gqa_ks<D, PAGED, false>(a, grid, block, s);
}

hipError_t launch_attn_gqa(const AttnArgs& a, int head_dim, bool paged, hipStream_t s) {
  const dim3 grid(a.n_units), block(kGqaThreads);
  if (head_dim == 128) {
    if (paged) launch_gqa_policy<128, true>(a, grid, block, s);
    else launch_gqa_policy<128, false>(a, grid, block, s);
  } else if (head_dim == 64) {
    if (paged) launch_gqa_policy<64, true>(a, grid, block, s);
    else launch_gqa_policy<64, false>(a, grid, block, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace d2f
