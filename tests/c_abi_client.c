/* A C11 client of libspecverify: it includes only sv.h, takes the address of
 * every entry point the header declares (so each must link from C), and
 * exercises the host-only paths, which need no GPU: version, error strings,
 * workspace sizes, tree depths, probe sizing, and the argument checks of
 * every compute entry point, which return a status and enqueue nothing.
 * One "name value" line per result on stdout. */
#include <stdio.h>

#include "sv.h"

typedef void (*any_fn)(void);

int main(void) {
  const struct {
    const char *name;
    any_fn fn;
  } entry[] = {
      {"sv_version", (any_fn)sv_version},
      {"sv_strerror", (any_fn)sv_strerror},
      {"sv_workspace_size", (any_fn)sv_workspace_size},
      {"sv_verify_window", (any_fn)sv_verify_window},
      {"sv_verify_window_noalloc", (any_fn)sv_verify_window_noalloc},
      {"sv_verify_window_part", (any_fn)sv_verify_window_part},
      {"sv_verify_window_early_exit", (any_fn)sv_verify_window_early_exit},
      {"sv_verify_greedy", (any_fn)sv_verify_greedy},
      {"sv_tree_max_depth", (any_fn)sv_tree_max_depth},
      {"sv_verify_tree", (any_fn)sv_verify_tree},
      {"sv_rollback", (any_fn)sv_rollback},
      {"sv_probe_blocks", (any_fn)sv_probe_blocks},
      {"sv_probe_read", (any_fn)sv_probe_read},
      {"sv_verify_window_lmhead", (any_fn)sv_verify_window_lmhead},
  };
  for (size_t k = 0; k < sizeof(entry) / sizeof(entry[0]); ++k)
    printf("linked %s %d\n", entry[k].name, entry[k].fn != NULL);

  printf("version %d\n", sv_version());
  for (int s = 0; s >= -7; --s) printf("strerror %d %s\n", s, sv_strerror(s));

  printf("ws_window %zu\n", sv_workspace_size(SV_OP_WINDOW, 256, 8, 128256, SV_DT_BF16));
  printf("ws_greedy %zu\n", sv_workspace_size(SV_OP_GREEDY, 256, 8, 128256, SV_DT_BF16));
  printf("ws_tree %zu\n", sv_workspace_size(SV_OP_TREE, 4, 41, 50257, SV_DT_F16));
  printf("ws_lmhead %zu\n", sv_workspace_size(SV_OP_LMHEAD, 256, 8, 128256, SV_DT_BF16));
  printf("ws_bad_dtype %zu\n", sv_workspace_size(SV_OP_WINDOW, 4, 4, 1000, 7));

  const int32_t chain[5] = {-1, 0, 1, 2, 3}, bushy[6] = {-1, 0, 0, 1, 1, 2}, bad[3] = {-1, 2, 0};
  printf("depth_chain %d\n", sv_tree_max_depth(chain, 5));
  printf("depth_bushy %d\n", sv_tree_max_depth(bushy, 6));
  printf("depth_bad %d\n", sv_tree_max_depth(bad, 3));
  printf("probe_blocks %d\n", sv_probe_blocks((size_t)1 << 30));

  /* argument checks: null device pointers, unknown dtype, bad sizes */
  printf("window_null %d\n", sv_verify_window(NULL, 0, NULL, 0, SV_DT_BF16, NULL, NULL, 4, 8, 1000, 0, 0, NULL,
                                              NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL));
  printf("window_dtype %d\n", sv_verify_window(NULL, 0, NULL, 0, 9, NULL, NULL, 4, 8, 1000, 0, 0, NULL, NULL, NULL,
                                               NULL, NULL, NULL, NULL, 0, NULL));
  printf("noalloc_null %d\n", sv_verify_window_noalloc(NULL, 0, NULL, 0, SV_DT_F32, NULL, NULL, 4, 8, 1000, 0, 0,
                                                       NULL, NULL, NULL, NULL, NULL, NULL, NULL));
  printf("part_bad %d\n", sv_verify_window_part(3, NULL, 0, NULL, 0, SV_DT_BF16, NULL, NULL, 4, 8, 1000, 0, 0, NULL,
                                                NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL));
  printf("early_null %d\n", sv_verify_window_early_exit(NULL, 0, NULL, 0, SV_DT_F16, NULL, NULL, 4, 8, 1000, 0, 0,
                                                        NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL));
  printf("greedy_null %d\n", sv_verify_greedy(NULL, 0, SV_DT_BF16, NULL, NULL, 4, 8, 1000, NULL, NULL, NULL, 0, NULL));
  printf("tree_bad_parent %d\n", sv_verify_tree(NULL, NULL, SV_DT_F16, NULL, bad, 4, 3, 1000, SV_TREE_STOCHASTIC, 0,
                                                0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL));
  printf("rollback_null %d\n", sv_rollback(NULL, NULL, 4, 3, 16, 1, NULL, 0, NULL, 0, NULL));
  printf("probe_null %d\n", sv_probe_read(NULL, 1024, NULL, NULL));
  printf("lmhead_null %d\n", sv_verify_window_lmhead(NULL, NULL, 128, NULL, NULL, 64, NULL, NULL, 4, 4, 1000, 0, 0,
                                                     NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL));
  return 0;
}
