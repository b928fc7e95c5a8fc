/* Runs every oracle entry point on small seeded inputs (ragged requests,
 * shuffled pages, -1 and out-of-range ids, an empty request, prefill
 * positions, a window with row scales) so that a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer sees every path. Prints "oracle ok". */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/csa2_oracle.h"

static unsigned long long g_state = 0x9E3779B97F4A7C15ull;
static unsigned rnd(void) {  /* xorshift64*: the driver's own inputs */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (unsigned)((g_state * 2685821657736338717ull) >> 32);
}
static float frnd(void) { return (float)((double)rnd() / 4294967296.0 * 4.0 - 2.0); }

int main(void) {
  enum { B = 3, PAGE = 16, MAXP = 12, NP = 30, NQ = 2, K = 40, POOL = 64, WROWS = 24 };
  const int32_t n_ent[B] = {150, 0, 37};
  static uint8_t kvc[NP * PAGE * 256], kvs[NP * PAGE * 32], ixc[NP * PAGE * 32], ixs[NP * PAGE * 4];
  for (size_t i = 0; i < sizeof kvc; ++i) kvc[i] = (uint8_t)rnd();
  for (size_t i = 0; i < sizeof kvs; ++i) kvs[i] = (uint8_t)(0x20 + rnd() % 40);
  for (size_t i = 0; i < sizeof ixc; ++i) ixc[i] = (uint8_t)rnd();
  for (size_t i = 0; i < sizeof ixs; ++i) ixs[i] = (uint8_t)(0x20 + rnd() % 40);
  int32_t bt[B * MAXP];
  int perm[NP];
  for (int i = 0; i < NP; ++i) perm[i] = i;
  for (int i = NP - 1; i > 0; --i) {
    int j = (int)(rnd() % (unsigned)(i + 1)), t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  for (int i = 0; i < B * MAXP; ++i) bt[i] = (i < NP) ? perm[i] : -1;
  orc_cache c = {kvc, kvs, ixc, ixs, bt, n_ent, PAGE, MAXP, NP};

  uint8_t wcodes[B * WROWS * 512];
  float wrs[B * WROWS];
  for (size_t i = 0; i < sizeof wcodes; ++i) wcodes[i] = (uint8_t)(rnd() % 0x7E);
  for (int i = 0; i < B * WROWS; ++i) wrs[i] = 0.5f + (float)(rnd() % 100) / 100.0f;
  const int32_t wlen[B] = {24, 0, 7};
  orc_window win = {wcodes, wrs, wlen, NULL, WROWS, 128};

  float q[B * NQ * 16 * 512], w[B * NQ * 4];
  uint8_t qc[B * NQ * 4 * 32], qs[B * NQ * 4 * 4];
  for (size_t i = 0; i < sizeof q / sizeof q[0]; ++i) q[i] = frnd();
  for (size_t i = 0; i < sizeof w / sizeof w[0]; ++i) w[i] = 0.5f + (float)(rnd() % 100) / 100.0f;
  for (size_t i = 0; i < sizeof qc; ++i) qc[i] = (uint8_t)rnd();
  for (size_t i = 0; i < sizeof qs; ++i) qs[i] = (uint8_t)(0x28 + rnd() % 16);

  static double scores[B * NQ * MAXP * PAGE], out[B * NQ * 16 * 512], lse[B * NQ * 16], psum[B * NQ * 16];
  int32_t idx[B * NQ * K], pool[B * NQ * POOL], idx2[B * NQ * K];
  const int32_t qpos[B * NQ] = {590, 599, 3, 10, 140, 147};

  /* decode and prefill positions, Full with a pool, Reindex over the pool, Reuse */
  for (int pf = 0; pf < 2; ++pf) {
    const int32_t *qp = pf ? qpos : NULL;
    orc_layer_step(0, &c, &win, q, qc, qs, w, qp, B, NQ, K, POOL, NULL, idx, pool, 0.044, out, lse, scores);
    orc_layer_step(1, &c, &win, q, qc, qs, w, qp, B, NQ, K, POOL, pool, idx2, NULL, 0.044, out, lse, NULL);
    orc_layer_step(2, &c, &win, q, NULL, NULL, NULL, qp, B, NQ, K, 0, idx2, NULL, NULL, 0.044, out, lse, NULL);
  }
  /* candidate lists with pads and ids past the entries; selection with a map */
  int32_t cand[B * NQ * 20];
  for (int i = 0; i < B * NQ * 20; ++i) cand[i] = (int32_t)(rnd() % 200) - 20;
  orc_index_score(&c, qc, qs, w, NULL, cand, 20, B, NQ, 20, scores);
  orc_topk(scores, cand, B, NQ, 20, 7, idx);
  orc_topk(scores, cand, B, NQ, 20, 25, idx);
  /* attention with ids out of range, -1 pads, no window */
  for (int i = 0; i < B * NQ * K; ++i) idx[i] = (int32_t)(rnd() % 400) - 100;
  orc_sparse_attend(&c, idx, K, q, NULL, NULL, 0.044, B, NQ, out, lse, psum);
  orc_sparse_attend(&c, idx, K, q, &win, NULL, 0.044, B, NQ, out, lse, psum);

  /* formats and the write side */
  for (int i = 0; i < 16; ++i) (void)orc_e2m1(i);
  for (int i = 0; i < 256; ++i) (void)orc_e4m3(i);
  double dq[4 * 64];
  uint8_t codes[4 * 32], sc[4 * 4], e8[4 * 64];
  float x[4 * 64];
  for (int i = 0; i < 4 * 64; ++i) x[i] = frnd() * (i % 7 == 0 ? 1000.0f : 1.0f);
  x[5] = 0.0f;
  orc_quantize_fp4(x, 4, 64, codes, sc);
  orc_dequant_fp4(codes, sc, 4, 64, dq);
  orc_e4m3_encode_n(x, 4 * 64, e8);
  orc_dequant_e4m3(e8, NULL, 4, 64, dq);
  static uint8_t wkvc[NP * PAGE * 256], wkvs[NP * PAGE * 32], wixc[NP * PAGE * 32], wixs[NP * PAGE * 4];
  orc_cache_w cw = {wkvc, wkvs, wixc, wixs, bt, PAGE, MAXP, NP};
  static float kv[B * 2 * 512], ixv[B * 2 * 64];
  for (int i = 0; i < B * 2 * 512; ++i) kv[i] = frnd();
  for (int i = 0; i < B * 2 * 64; ++i) ixv[i] = frnd();
  const int32_t ent[B * 2] = {0, 149, -1, 5000, 36, 12};
  orc_kv_append(&cw, kv, ixv, ent, B, 2);
  const int32_t wrow[B * 2] = {0, 23, -1, 24, 6, 3};
  orc_window_append(wcodes, wrs, WROWS, kv, wrow, B, 2);
  orc_window_append(wcodes, NULL, WROWS, kv, wrow, B, 2);
  printf("oracle ok\n");
  return 0;
}
