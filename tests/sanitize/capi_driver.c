/* The host side of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer, with no GPU: workspace sizing over many shapes
 * and every argument check that returns before a launch. Prints "capi ok". */
#include <stdio.h>
#include <string.h>

#include "../../include/csa2.h"
#include "../../include/csa2_probe.h"

#define EXPECT(cond)                                         \
  do {                                                       \
    if (!(cond)) {                                           \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                              \
    }                                                        \
  } while (0)

int main(void) {
  /* fake, never dereferenced device addresses (every call below fails its
     checks before it would launch anything) */
  const uint8_t *p8 = (const uint8_t *)0x100000;
  const int32_t *p32 = (const int32_t *)0x200000;
  float *pf = (float *)0x300000;
  int32_t *po = (int32_t *)0x400000;
  size_t total = 0;
  const int32_t batches[] = {1, 8, 32, 64, 4096};
  const int32_t cols[] = {0, 100, 4096, 4097, 16384, 16385, 262144, 524288};
  const int32_t ks[] = {1, 256, 2048, 4096};
  for (int m = 0; m < 3; ++m)
    for (int bi = 0; bi < 5; ++bi)
      for (int ci = 0; ci < 8; ++ci)
        for (int ki = 0; ki < 4; ++ki)
          for (int pool = 0; pool <= 16384; pool += 16384)
            for (int wc = 0; wc <= 128; wc += 128)
              total += csa2_workspace_bytes((csa2_mode)m, batches[bi], 1, cols[ci], ks[ki], pool, wc);
  EXPECT(total > 0);
  EXPECT(csa2_workspace_bytes(CSA2_FULL, 0, 1, 100, 16, 0, 0) == 0);

  csa2_cache c;
  memset(&c, 0, sizeof c);
  c.kv_codes = p8; c.kv_scales = p8; c.ix_codes = p8; c.ix_scales = p8;
  c.block_table = p32; c.n_entries = p32;
  c.page_size = 64; c.max_pages = 4; c.num_pages = 8;
  csa2_window w;
  memset(&w, 0, sizeof w);
  w.codes = p8; w.length = p32; w.rows = 128; w.window = 128;

  csa2_layer_args a;
  memset(&a, 0, sizeof a);
  a.mode = CSA2_FULL; a.cache = &c; a.win = &w; a.q = pf; a.qix_codes = p8; a.qix_scales = p8;
  a.w = pf; a.batch = 2; a.nq = 1; a.k = 16; a.idx_out = po; a.sm_scale = 0.04f; a.out = pf; a.lse = pf;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EWORKSPACE);   /* no workspace */
  EXPECT(strlen(csa2_last_error()) > 0);
  a.ws = (void *)0x10010; a.ws_bytes = 1u << 30;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EWORKSPACE);   /* misaligned */
  a.ws = NULL; a.ws_bytes = 0;
  a.k = 0;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EINVAL);
  a.k = 5000;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EINVAL);
  a.k = 16; a.mode = (csa2_mode)7;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EINVAL);
  a.mode = CSA2_REINDEX;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EINVAL);       /* no pool in idx_in */
  a.mode = CSA2_REUSE; a.idx_in = NULL;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EINVAL);
  a.mode = CSA2_FULL; a.pool = 8;                          /* pool < k */
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EINVAL);
  a.pool = 0; c.page_size = 48;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EUNSUPPORTED);
  c.page_size = 64; w.rows = 70000;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EINVAL);
  w.rows = 128; a.sm_scale = 1.0f / 0.0f;
  EXPECT(csa2_layer_step(&a, NULL) == CSA2_EINVAL);
  EXPECT(csa2_layer_step(NULL, NULL) == CSA2_EINVAL);

  EXPECT(csa2_topk(NULL, NULL, 1, 1, 10, 2, po, NULL, 0, NULL) == CSA2_EINVAL);
  EXPECT(csa2_topk(pf, NULL, 1, 1, 600000, 2, po, NULL, 0, NULL) == CSA2_EUNSUPPORTED);
  EXPECT(csa2_topk(pf, NULL, 1, 1, 300000, 2, po, NULL, 0, NULL) == CSA2_EWORKSPACE);
  EXPECT(csa2_sparse_attend(&c, p32, 0, pf, &w, NULL, 0.04f, 1, 1, pf, pf, NULL, 0, NULL) == CSA2_EINVAL);
  EXPECT(csa2_sparse_attend(&c, p32, 16, pf, &w, NULL, 0.04f, 300, 1, pf, pf, NULL, 0, NULL) == CSA2_EWORKSPACE);
  EXPECT(csa2_sparse_attend_noalloc(&c, p32, 16, pf, &w, NULL, 0.04f, 1, 1, NULL, pf, NULL) == CSA2_EINVAL);
  EXPECT(csa2_sparse_attend_noalloc(&c, p32, 5000, pf, &w, NULL, 0.04f, 1, 1, pf, pf, NULL) == CSA2_EINVAL);
  EXPECT(csa2_index_score(&c, NULL, p8, pf, NULL, NULL, 0, 1, 1, pf, NULL, NULL) == CSA2_EINVAL);
  EXPECT(csa2_index_score(&c, p8, p8, pf, NULL, p32, 0, 1, 1, pf, NULL, NULL) == CSA2_EINVAL);
  EXPECT(csa2_index_topk(&c, p8, p8, pf, NULL, 1, 1, 16, 8, po, po, NULL, 0, NULL) == CSA2_EINVAL);
  EXPECT(csa2_quantize_fp4(pf, 4, 20, (uint8_t *)po, (uint8_t *)po, NULL) == CSA2_EINVAL);
  EXPECT(csa2_kv_append(NULL, pf, NULL, p32, 1, 1, NULL) == CSA2_EINVAL);
  EXPECT(csa2_window_append((uint8_t *)po, NULL, 0, pf, p32, 1, 1, NULL) == CSA2_EINVAL);
  EXPECT(csa2_dequant_fp4(p8, p8, 4, 20, (uint16_t *)po, NULL) == CSA2_EINVAL);
  EXPECT(csa2_dequant_e4m3(p8, -1, pf, NULL) == CSA2_EINVAL);
  EXPECT(csa2_stream_read(p8, 15, (uint32_t *)po, 8, NULL) == CSA2_EINVAL);
  for (int s = 0; s < 6; ++s) EXPECT(csa2_status_string((csa2_status)s) != NULL);
  EXPECT(strstr(csa2_version(), "gfx950") != NULL);
  printf("capi ok\n");
  return 0;
}
