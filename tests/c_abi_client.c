/* A plain C99 client of the library: it includes only include/relbias_attn.h, links the shared
 * library and calls entry points whose outcome needs no device: argument errors (returned before
 * any HIP call, with a message), empty problems, the host-only workspace-size functions and the
 * version string.  Exit status 0 and "ok" on success. */

#include <stdio.h>
#include <string.h>

#include "relbias_attn.h"

static int fails = 0;

static void check(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAIL %s (last error: \"%s\")\n", what, relbias_attn_last_error());
    ++fails;
  }
}

int main(void) {
  /* stand-ins for device buffers: only their alignment is inspected before the errors below */
  static unsigned char buf[256] __attribute__((aligned(256)));
  void* p = buf;
  int st;

  const char* v = relbias_attn_version();
  check(v != NULL && strstr(v, "gfx950") != NULL, "version names gfx950");

  st = relbias_attn_fwd(RBA_BF16, p, p, p, p, NULL, 1, 16, 4, 3, 128, 0, 8, RBA_BIAS_NONE, NULL,
                        NULL, NULL, 0, 0.1f, 0, NULL, 0, NULL);
  check(st == RBA_EINVAL && strstr(relbias_attn_last_error(), "multiple") != NULL,
        "Hq not a multiple of Hkv is RBA_EINVAL");
  st = relbias_attn_fwd(RBA_BF16, p, p, p, p, NULL, 1, 16, 4, 2, 96, 0, 8, RBA_BIAS_NONE, NULL,
                        NULL, NULL, 0, 0.1f, 0, NULL, 0, NULL);
  check(st == RBA_ENOTSUP && strstr(relbias_attn_last_error(), "head_dim") != NULL,
        "head_dim 96 is RBA_ENOTSUP");
  st = relbias_attn_fwd(RBA_BF16, p, p, p, p, NULL, 1, 16, 4, 2, 128, 0, 8, RBA_BIAS_TABLE, NULL,
                        NULL, NULL, 0, 0.1f, 0, NULL, 0, NULL);
  check(st == RBA_EINVAL && strstr(relbias_attn_last_error(), "table") != NULL,
        "table mode without a table is RBA_EINVAL");
  st = relbias_attn_decode(RBA_BF16, p, p, p, p, NULL, 2, 100, 0, 8, 2, 128, 0, 8, RBA_BIAS_NONE,
                           NULL, NULL, NULL, 0, 0.1f, 0, NULL, 0, NULL);
  check(st == RBA_EINVAL && strstr(relbias_attn_last_error(), "kv_len") != NULL,
        "decode with kv_len 0 is RBA_EINVAL");
  st = relbias_attn_bwd(7, p, p, p, p, (float*)p, p, p, p, p, NULL, NULL, NULL, 1, 16, 4, 2, 128,
                        0, 8, RBA_BIAS_NONE, NULL, NULL, NULL, 0, 0.1f, 0, p, 256, NULL);
  check(st == RBA_EINVAL && strstr(relbias_attn_last_error(), "dtype") != NULL,
        "backward with an unknown dtype is RBA_EINVAL");

  /* empty problems succeed without touching any pointer, and clear the message */
  st = relbias_attn_fwd(RBA_BF16, NULL, NULL, NULL, NULL, NULL, 0, 16, 4, 2, 128, 0, 8,
                        RBA_BIAS_NONE, NULL, NULL, NULL, 0, 0.1f, 0, NULL, 0, NULL);
  check(st == RBA_OK && relbias_attn_last_error()[0] == '\0', "B = 0 prefill is RBA_OK");
  st = relbias_attn_decode(RBA_BF16, NULL, NULL, NULL, NULL, NULL, 0, 100, 50, 8, 2, 128, 0, 8,
                           RBA_BIAS_NONE, NULL, NULL, NULL, 0, 0.1f, 0, NULL, 0, NULL);
  check(st == RBA_OK, "B = 0 decode is RBA_OK");

  /* host-only sizes */
  check(relbias_attn_fwd_workspace_size(RBA_BF16, 2, 4096, 32, 8, 128, 512, 512, RBA_BIAS_NONE, 0,
                                        0.088f) == 0, "no workspace without the r.E bias");
  check(relbias_attn_decode_workspace_size(64, 32, 8, 128, 65536, 0) > 0,
        "split decode needs a workspace");
  check(relbias_attn_decode_paged_workspace_size(64, 32, 8, 128, 65536, 0) ==
            relbias_attn_decode_workspace_size(64, 32, 8, 128, 65536, 0),
        "paged decode workspace equals the contiguous one at the bound");
  check(relbias_attn_bwd_workspace_size(2, 100, 8, RBA_BIAS_RPROJ, 512) ==
            (size_t)6400 + (size_t)8 * 641 * 32 * 2,
        "backward workspace: rowsum plus the converted E");

  if (fails) return 1;
  printf("ok\n");
  return 0;
}
