/* Host sanitizer driver for the C-ABI's validation paths: the library's host
 * code is built with AddressSanitizer and UndefinedBehaviorSanitizer (no
 * device code: every call below is rejected on the host before any launch),
 * then each entry point gets arguments that its checks must refuse, and the
 * workspace-size functions get extreme shapes.  A memory error, an integer
 * overflow or a wrong return code fails the run. */
#include <stdint.h>
#include <stdio.h>

#include "../../include/csa.h"

static int fails = 0;
#define EXPECT(call, code)                                                                                  \
  do {                                                                                                      \
    int rc_ = (call);                                                                                       \
    if (rc_ != (code)) {                                                                                    \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #call, rc_, (code), \
              csa_last_error());                                                                            \
      ++fails;                                                                                              \
    }                                                                                                       \
  } while (0)

int main(void) {
  void* P = (void*)(uintptr_t)4096;       /* a non-null, aligned stand-in: never dereferenced here */
  void* MIS = (void*)(uintptr_t)(4096 + 4);
  const int BF = CSA_BF16;

  if (csa_version() < 1) ++fails;
  for (int c = -10; c <= 1; ++c)
    if (!csa_error_string(c)) ++fails;

  /* compressors */
  EXPECT(csa_compress(NULL, P, P, P, P, 2, 8, 512, 64, 4, 1, 16, 1e-6f, 1e4f, BF, NULL), CSA_ERR_NULL);
  EXPECT(csa_compress(P, P, P, MIS, P, 2, 8, 512, 64, 4, 1, 16, 1e-6f, 1e4f, BF, NULL), CSA_ERR_ALIGN);
  EXPECT(csa_compress(P, P, P, P, P, 2, 8, 513, 64, 4, 1, 16, 1e-6f, 1e4f, BF, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_compress(P, P, P, P, P, 2, 8, 512, 64, 0, 1, 16, 1e-6f, 1e4f, BF, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_compress(P, P, P, P, P, 2, 2147483647, 512, 64, 1, 1, 16, 1e-6f, 1e4f, BF, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_compress(P, P, P, P, P, 2, 8, 512, 64, 4, 1, 16, 1e-6f, 1e4f, 7, NULL), CSA_ERR_DTYPE);
  EXPECT(csa_compress_kv_index(P, P, P, P, 512, 64, 1, 16, P, P, P, P, 131, 64, 16, P, 2, 8, 4, 1e-6f, 1e4f, BF, NULL),
         CSA_ERR_SHAPE);

  /* indexer and top-k */
  EXPECT(csa_index_scores(NULL, P, P, P, P, 1, 1, 64, 128, 100, 4, 0, BF, NULL), CSA_ERR_NULL);
  EXPECT(csa_index_scores(P, P, P, P, P, 1, 1, 64, 128, 100, 4, 8u, BF, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_topk(P, P, P, NULL, NULL, 0, 1, 1, 100, 0, 4, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_topk(P, P, P, NULL, NULL, 0, 1, 1, 100, 5000, 4, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_topk(P, P, P, NULL, NULL, 0, 8, 1, 262144, 1024, 4, NULL), CSA_ERR_WORKSPACE);
  EXPECT(csa_index_topk(P, P, P, P, P, NULL, NULL, 0, 1, 1, 64, 128, 100, 16, 4, 0, BF, NULL), CSA_ERR_WORKSPACE);
  (void)csa_topk_workspace_size(65535, 65535, 2147483647, 4096);
  (void)csa_index_topk_workspace_size(65535, 65535, 2147483647, 4096);
  if (csa_topk_workspace_size(-1, -1, -1, -1) != 0 || csa_topk_workspace_size(1, 1, 100, 0) != 0 ||
      csa_index_topk_workspace_size(1, 1, 100, 5000) != 0)
    ++fails;

  /* attention */
  EXPECT(csa_sparse_attn(NULL, P, P, P, NULL, P, P, P, NULL, NULL, 0, 1, 1, 16, 512, 64, 100, 16, 128, 128, 0.f,
                         1e4f, BF, NULL),
         CSA_ERR_NULL);
  EXPECT(csa_sparse_attn(P, P, P, P, NULL, P, P, P, NULL, NULL, 0, 1, 1, 16, 512, 65, 100, 16, 128, 128, 0.f, 1e4f, BF,
                         NULL),
         CSA_ERR_SHAPE);
  EXPECT(csa_sparse_attn(P, P, P, P, NULL, P, P, P, NULL, NULL, 0, 1, 1, 16, 512, 64, 100, 16, 128, 129, 0.f, 1e4f, BF,
                         NULL),
         CSA_ERR_SHAPE);
  EXPECT(csa_sparse_attn(P, P, P, P, NULL, P, P, P, NULL, NULL, 0, 1, 1, 15, 512, 64, 100, 16, 128, 128, 0.f, 1e4f,
                         CSA_BF16_KV_FP8, NULL),
         CSA_ERR_UNSUPPORTED);
  EXPECT(hca_attn(P, P, P, NULL, P, P, P, NULL, NULL, 0, 1, 1, 16, 512, 64, 100, 0, 128, 128, 0.f, 1e4f, BF, NULL),
         CSA_ERR_SHAPE);
  EXPECT(swa_attn(P, P, NULL, P, P, P, NULL, NULL, 0, 1, 1, 16, 512, 64, 128, 0, 0.f, 1e4f, BF, NULL), CSA_ERR_SHAPE);
  if (csa_attn_workspace_size(65535, 65535, 2147483632, 512, 2147483647) != 0) ++fails;  /* B*S*H too large */
  if (csa_attn_workspace_size(0, 1, 16, 512, 100) != 0 || csa_attn_workspace_size(1, 1, 16, 512, -5) != 0) ++fails;
  (void)csa_attn_workspace_size(1, 1, 16, 512, 0);
  (void)csa_attn_workspace_size(1, 1, 32, 512, 2147483647);

  /* FP8 rows, weights, projections */
  EXPECT(csa_quantize_rows(P, P, 4, 256, 64, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_dequantize_rows(P, P, -1, 512, 64, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_pack_weights(P, P, 1, 100, 512, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_q_proj(P, P, P, P, P, P, P, NULL, 0, 4, 1, 7168, 1536, 128, 512, 64, 1e-6f, 1e4f, NULL), CSA_ERR_WORKSPACE);
  EXPECT(csa_q_proj(P, P, P, P, P, P, P, NULL, 0, 4, 1, 7000, 1536, 128, 512, 64, 1e-6f, 1e4f, NULL), CSA_ERR_SHAPE);
  EXPECT(csa_o_proj(P, P, P, P, P, NULL, 0, 4, 128, 512, 3, 1024, 7168, NULL), CSA_ERR_SHAPE);
  if (csa_q_proj_workspace_size(2147483647, 2147483647, 2048, 2147483647, 2048) != 0) ++fails;
  if (csa_o_proj_workspace_size(2147483647, 2147483647, 2048, 1, 2147483647, 2147483647) != 0) ++fails;
  (void)csa_q_proj_workspace_size(1 << 20, 1 << 20, 2048, 512, 2048);
  (void)csa_o_proj_workspace_size(1 << 20, 512, 2048, 1, 1 << 20, 1 << 20);

  if (fails) {
    fprintf(stderr, "abi driver: %d check(s) failed\n", fails);
    return 1;
  }
  printf("abi driver: ok\n");
  return 0;
}
