/* The C ABI from plain C99: the header compiles as C, the library links and answers the calls
 * that need no GPU (version, workspace queries, argument validation). */
#include <stdio.h>
#include <string.h>

#include "awq.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
              __LINE__, #cond);                                        \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

int main(void) {
  awq_cfg cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.bits = 4;
  cfg.group = 128;
  cfg.n_grid = 20;
  cfg.s_floor = 1e-5f;
  cfg.form = AWQ_FORM_GRAM;
  cfg.n_clip = 11;
  cfg.clip_min = 0.5f;
  cfg.zero_point = 0;

  EXPECT(awq_version() >= 10600);
  EXPECT(strncmp(awq_status_string(AWQ_ERR_SHAPE), "AWQ_ERR_SHAPE", 13) == 0);
  EXPECT(awq_act_stats_workspace_bytes(65536, 4096) > 0);
  EXPECT(awq_search_workspace_bytes(65536, 4096, 4096, AWQ_F16, &cfg) > 0);
  EXPECT(awq_clip_search_gram_ws_bytes(4096, &cfg) > 0);
  EXPECT(awq_clip_search_gram_ws_bytes(4096, &cfg) <=
         awq_search_workspace_bytes(65536, 4096, 4096, AWQ_F16, &cfg));
  cfg.bits = 5;
  EXPECT(awq_search_workspace_bytes(65536, 4096, 4096, AWQ_F16, &cfg) == 0);
  cfg.bits = 4;

  /* validation happens before any HIP call */
  float sx[16];
  uint32_t flags = 0;
  EXPECT(awq_act_stats(NULL, AWQ_F16, 16, 16, 16, sx, &flags, NULL, 0, NULL) == AWQ_ERR_NULL);
  EXPECT(w4a16_gemm(NULL, 1, 16, 128, 128, NULL, NULL, NULL, NULL, NULL, NULL) == AWQ_ERR_NULL);
  EXPECT(w4a16_gemm_workspace_bytes(64, 4096, 4096, 128) > 0);
  EXPECT(w4a16_gemm_ws(NULL, 16, 4096, 4096, 128, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
         AWQ_ERR_NULL);

  if (failures) return 1;
  printf("C ABI ok (version %d)\n", (int)awq_version());
  return 0;
}
