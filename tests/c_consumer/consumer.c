/* A consumer of libd2f written in plain C99: it uses only d2f.h and the HIP
 * runtime API (device memory and copies), no Python and no C++.  It runs one
 * D2F step on a small synthetic problem -- block-causal attention with a
 * split key range, the commit pass, the KV append -- plus error calls, and
 * writes every result to a file that tests/test_gpu_c_consumer.py compares
 * with the fp64 oracle on the same inputs.
 *
 * Inputs come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; the 64-bit finaliser as
 * published by Vigna), one stream per tensor; the test regenerates them
 * from the same definition.  A draw x gives u = (x >> 40) / 2^24 in [0, 1)
 * and the value 2u - 1, exact in float32, rounded to bf16 to nearest even.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "d2f.h"

enum { NB = 2, HQ = 4, HKV = 2, D = 64, BS = 16, MAXW = 2, CAP = 2048, WMAX = MAXW * BS };
enum { ROWS = 32, VOCAB = 1000, MASK_ID = 1000 };
static const int32_t PREFIX[NB] = {37, 2000};
static const int32_t NWIN[NB] = {2, 1};

static uint64_t splitmix64(uint64_t* s) {
  uint64_t z = (*s += 0x9e3779b97f4a7c15ULL);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}
static float unit_value(uint64_t* s) {
  return (float)(splitmix64(s) >> 40) * (1.0f / 16777216.0f) * 2.0f - 1.0f;
}
static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* n bf16 values of stream `seed`, in row-major order */
static void fill_bf16(uint16_t* dst, size_t n, uint64_t seed) {
  for (size_t i = 0; i < n; ++i) dst[i] = bf16_rne(unit_value(&seed));
}

#define CHECK_HIP(x)                                 \
  do {                                               \
    if ((x) != hipSuccess) {                         \
      fprintf(stderr, "HIP error at %s\n", #x);      \
      return 100;                                    \
    }                                                \
  } while (0)

static int put(FILE* f, const void* p, size_t bytes) { return fwrite(p, 1, bytes, f) == bytes ? 0 : 1; }

int d2f_consumer_run(const char* path) {
  const uint16_t NAN_BF16 = 0x7fc0, FILL = 0x7f7f;
  const size_t nq = (size_t)NB * HQ * WMAX * D, nc = (size_t)NB * HKV * CAP * D,
               nw = (size_t)NB * HKV * WMAX * D, nl = (size_t)NB * HQ * WMAX;
  uint16_t *q = malloc(nq * 2), *kc = malloc(nc * 2), *vc = malloc(nc * 2), *kw = malloc(nw * 2),
           *vw = malloc(nw * 2), *out = malloc(nq * 2);
  float *lse = malloc(nl * 4), *logits = malloc((size_t)ROWS * VOCAB * 4), conf[ROWS];
  int32_t argmax[ROWS], tokens[ROWS], n_committed[ROWS / BS], status[8], prefix[NB];
  uint8_t mask[ROWS], phase[ROWS / BS], complete[ROWS / BS];
  if (!q || !kc || !vc || !kw || !vw || !out || !lse || !logits) return 101;

  fill_bf16(q, nq, 1);
  fill_bf16(kc, nc, 2);
  fill_bf16(vc, nc, 3);
  fill_bf16(kw, nw, 4);
  fill_bf16(vw, nw, 5);
  /* slots a step must not read are NaN: cache rows past the prefix, window
   * and query rows past the window */
  for (int b = 0; b < NB; ++b)
    for (int h = 0; h < HKV; ++h) {
      for (size_t r = (size_t)PREFIX[b]; r < CAP; ++r)
        for (int d = 0; d < D; ++d)
          kc[(((size_t)b * HKV + h) * CAP + r) * D + d] = vc[(((size_t)b * HKV + h) * CAP + r) * D + d] = NAN_BF16;
      for (size_t r = (size_t)NWIN[b] * BS; r < WMAX; ++r)
        for (int d = 0; d < D; ++d)
          kw[(((size_t)b * HKV + h) * WMAX + r) * D + d] = vw[(((size_t)b * HKV + h) * WMAX + r) * D + d] = NAN_BF16;
    }
  for (int b = 0; b < NB; ++b)
    for (int h = 0; h < HQ; ++h)
      for (size_t r = (size_t)NWIN[b] * BS; r < WMAX; ++r)
        for (int d = 0; d < D; ++d) q[(((size_t)b * HQ + h) * WMAX + r) * D + d] = NAN_BF16;
  for (size_t i = 0; i < nq; ++i) out[i] = FILL;
  for (size_t i = 0; i < nl; ++i) lse[i] = 7.0f;

  /* commit inputs: logits 4 u, every third row with one entry raised by 10;
   * a quarter of the positions COMMITTED with a drawn token */
  uint64_t s = 6, sm = 7, st = 8;
  for (int r = 0; r < ROWS; ++r) {
    for (int j = 0; j < VOCAB; ++j) logits[(size_t)r * VOCAB + j] = 4.0f * unit_value(&s);
    if (r % 3 == 0) logits[(size_t)r * VOCAB + (r * 37) % VOCAB] += 10.0f;
    const uint64_t xm = splitmix64(&sm), xt = splitmix64(&st);
    mask[r] = (xm >> 62) == 0 ? D2F_COMMITTED : D2F_MASKED;
    tokens[r] = mask[r] == D2F_COMMITTED ? (int32_t)(xt % VOCAB) : MASK_ID;
  }
  phase[0] = D2F_AGGRESSIVE;
  phase[1] = D2F_CONSERVATIVE;

  void *dq, *dkc, *dvc, *dkw, *dvw, *dout, *dlse, *dlog, *dconf, *darg, *dmask, *dtok, *dphase,
      *dncom, *dcomp, *dws = NULL, *dcws = NULL;
  CHECK_HIP(hipMalloc(&dq, nq * 2));
  CHECK_HIP(hipMalloc(&dkc, nc * 2));
  CHECK_HIP(hipMalloc(&dvc, nc * 2));
  CHECK_HIP(hipMalloc(&dkw, nw * 2));
  CHECK_HIP(hipMalloc(&dvw, nw * 2));
  CHECK_HIP(hipMalloc(&dout, nq * 2));
  CHECK_HIP(hipMalloc(&dlse, nl * 4));
  CHECK_HIP(hipMalloc(&dlog, (size_t)ROWS * VOCAB * 4));
  CHECK_HIP(hipMalloc(&dconf, ROWS * 4));
  CHECK_HIP(hipMalloc(&darg, ROWS * 4));
  CHECK_HIP(hipMalloc(&dmask, ROWS));
  CHECK_HIP(hipMalloc(&dtok, ROWS * 4));
  CHECK_HIP(hipMalloc(&dphase, ROWS / BS));
  CHECK_HIP(hipMalloc(&dncom, ROWS / BS * 4));
  CHECK_HIP(hipMalloc(&dcomp, ROWS / BS));
  CHECK_HIP(hipMemcpy(dq, q, nq * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dkc, kc, nc * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dvc, vc, nc * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dkw, kw, nw * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dvw, vw, nw * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dout, out, nq * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dlse, lse, nl * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dlog, logits, (size_t)ROWS * VOCAB * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dmask, mask, ROWS, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dtok, tokens, ROWS * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dphase, phase, ROWS / BS, hipMemcpyHostToDevice));

  d2f_attn_desc_t desc;
  desc.batch = NB;
  desc.n_heads_q = HQ;
  desc.n_heads_kv = HKV;
  desc.head_dim = D;
  desc.block_size = BS;
  desc.max_win_blocks = MAXW;
  desc.cache_capacity = CAP;
  desc.dtype = D2F_BF16;
  desc.softmax_scale = 0.0f;

  size_t ws = 0, cws = 0;
  status[0] = d2f_block_attn_workspace_size(&desc, PREFIX, NWIN, &ws);
  /* a workspace one byte short is refused before anything is launched */
  if (ws > 0) CHECK_HIP(hipMalloc(&dws, ws));
  status[1] = ws > 0 ? (int32_t)d2f_block_attn(&desc, dq, dkc, dvc, dkw, dvw, PREFIX, NWIN, dout,
                                               dlse, dws, ws - 1, NULL)
                     : -1;
  status[2] = d2f_block_attn(&desc, dq, dkc, dvc, dkw, dvw, PREFIX, NWIN, dout, dlse, dws, ws, NULL);
  status[3] = d2f_confidence_commit_workspace_size(ROWS, VOCAB, &cws);
  CHECK_HIP(hipMalloc(&dcws, cws));
  status[4] = d2f_confidence_commit(dlog, VOCAB, ROWS, VOCAB, dmask, dtok, dphase, BS, 0.5f, 1,
                                    MASK_ID, dconf, darg, dncom, dcomp, dcws, cws, NULL);
  prefix[0] = PREFIX[0];
  prefix[1] = PREFIX[1];
  /* only the oldest window block may join the cache */
  status[5] = d2f_kv_commit(&desc, 1, dkc, dvc, (int64_t)nc, dkw, dvw, (int64_t)nw, 0, 1, prefix,
                            NULL, NULL);
  status[6] = d2f_kv_commit(&desc, 1, dkc, dvc, (int64_t)nc, dkw, dvw, (int64_t)nw, 0, 0, prefix,
                            NULL, NULL);
  status[7] = d2f_status_string(D2F_ERR_ORDER) != NULL && d2f_last_error() != NULL ? 0 : -1;
  CHECK_HIP(hipDeviceSynchronize());

  CHECK_HIP(hipMemcpy(out, dout, nq * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(lse, dlse, nl * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(conf, dconf, ROWS * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(argmax, darg, ROWS * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(mask, dmask, ROWS, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(tokens, dtok, ROWS * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(n_committed, dncom, ROWS / BS * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(complete, dcomp, ROWS / BS, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(kc, dkc, nc * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(vc, dvc, nc * 2, hipMemcpyDeviceToHost));

  FILE* f = fopen(path, "wb");
  if (!f) return 102;
  int bad = put(f, status, sizeof status) | put(f, out, nq * 2) | put(f, lse, nl * 4) |
            put(f, conf, sizeof conf) | put(f, argmax, sizeof argmax) | put(f, mask, sizeof mask) |
            put(f, tokens, sizeof tokens) | put(f, n_committed, ROWS / BS * 4) |
            put(f, complete, ROWS / BS) | put(f, kc, nc * 2) | put(f, vc, nc * 2) |
            put(f, prefix, sizeof prefix);
  fclose(f);

  void* dev[] = {dq, dkc, dvc, dkw, dvw, dout, dlse, dlog, dconf, darg, dmask, dtok, dphase,
                 dncom, dcomp, dws, dcws};
  for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i)
    if (dev[i]) (void)hipFree(dev[i]);
  free(q); free(kc); free(vc); free(kw); free(vw); free(out); free(lse); free(logits);
  return bad ? 103 : 0;
}
