/* A plain C consumer of the library: compiled against include/dflash.h and
 * linked with libdflash.so by tests/test_c_consumer.py.  It makes only the
 * host-side calls (no device needed): version, workspace sizing for a valid
 * and an invalid configuration, and argument rejection with its message.
 * Exit status 0 = every check held. */
#include <stdio.h>
#include <string.h>

#include "dflash.h"

static int fails = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++fails;                                                   \
    }                                                            \
  } while (0)

int main(void) {
  const char* v = dflash_version();
  CHECK(v != NULL && strstr(v, "gfx950") != NULL);

  dflash_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.hidden = 4096;
  cfg.n_q_heads = 32;
  cfg.n_kv_heads = 8;
  cfg.head_dim = 128;
  cfg.n_layers = 5;
  cfg.ffn = 12288;
  cfg.vocab = 151936;
  cfg.block = 16;
  cfg.n_target_layers = 5;
  cfg.max_batch = 1;
  cfg.max_ctx = 4160;
  cfg.max_fuse_rows = 17;
  cfg.conv_width = 0;
  cfg.dtype = DFLASH_DTYPE_BF16;
  cfg.rms_eps = 1e-6f;
  cfg.rope_theta = 1e6f;
  const size_t ws = dflash_workspace_bytes(&cfg);
  CHECK(ws > 0);

  dflash_config bad = cfg;
  bad.head_dim = 96;
  CHECK(dflash_workspace_bytes(&bad) == 0);

  dflash_ctx* ctx = NULL;
  CHECK(dflash_create(&cfg, NULL, NULL, NULL, NULL, NULL, 0, &ctx) == DFLASH_EINVAL);
  CHECK(ctx == NULL);
  CHECK(strstr(dflash_last_error(), "null") != NULL);
  CHECK(dflash_create(&bad, NULL, NULL, NULL, NULL, NULL, 0, &ctx) == DFLASH_EUNSUPPORTED);
  CHECK(dflash_fuse_ctx(NULL, 1, NULL, 1, 0, NULL, NULL) == DFLASH_EINVAL);
  CHECK(dflash_reload_weights(NULL, NULL) == DFLASH_EINVAL);
  dflash_destroy(NULL);

  printf("abi consumer: workspace %zu bytes, %d failed checks\n", ws, fails);
  return fails == 0 ? 0 : 1;
}
