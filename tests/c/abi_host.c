/* A C99 consumer of libkvc.so: drives a host-only cache (no device pools)
 * through create, appends, visible tables, rollback and destroy, and checks
 * the invariants "LingBot-Map Paged KV Cache" states (section 2: patch pages
 * constant once the window is full, special pages packing 42 frames of 6
 * tokens, the last page described by its length; section 3: a rollback
 * restores the table; single-level undo).  Built and run by
 * tests/test_c_abi.py; prints "OK" on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvc.h"

#define S_UNITS 8
#define W_UNITS 64
#define FRAMES 150
#define CAP 256

static int fails = 0;

static void check(int ok, const char* what, int t) {
  if (!ok) {
    printf("FAIL %s at frame %d (%s)\n", what, t, kvc_last_error());
    ++fails;
  }
}

static int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

int main(void) {
  kvc_config cfg;
  kvc_t* c = NULL;
  int32_t ids[CAP], lens[CAP], ids0[CAP], lens0[CAP];
  int32_t n = 0, last = 0, n0 = 0, pages = 0;
  int t;
  memset(&cfg, 0, sizeof cfg);
  cfg.num_heads = 1;
  cfg.head_dim = 64;
  cfg.page_size = 256;
  cfg.dtype = KVC_DTYPE_BF16;
  cfg.patch_tokens = 256;
  cfg.special_tokens = 6;
  cfg.num_scale_units = S_UNITS;
  cfg.window_units = W_UNITS;
  cfg.special_packing = KVC_SPECIAL_FRAME_ALIGNED;
  cfg.max_units = FRAMES + 1;
  cfg.num_pages = 0;
  check(kvc_required_pages(&cfg, &pages) == KVC_OK, "kvc_required_pages", -1);
  /* scale and window units, one spare unit, ceil(151 / 42) special pages */
  check(pages == S_UNITS + W_UNITS + 1 + ceil_div(FRAMES + 1, 42), "required page count", -1);
  check(kvc_create(&cfg, NULL, NULL, &c) == KVC_OK, "kvc_create", -1);
  for (t = 1; t <= FRAMES; ++t) {
    int32_t patch, special, i, in_special;
    check(kvc_append_frame(c, NULL, NULL, NULL) == KVC_OK, "kvc_append_frame", t);
    check(kvc_build_visible_table(c, ids, lens, CAP, &n, &last) == KVC_OK, "kvc_build_visible_table", t);
    patch = t < S_UNITS + W_UNITS ? t : S_UNITS + W_UNITS;
    special = ceil_div(t, 42);
    check(n == patch + special, "visible page count", t);
    check(last == 6 * (t - 42 * (special - 1)), "last_page_len", t);
    in_special = 0;
    for (i = 0; i < n; ++i) {
      if (i < patch) in_special += lens[i] != 256;
      else if (i < n - 1) in_special += lens[i] != 252;
    }
    check(in_special == 0, "page lengths (256 per patch page, 252 per full special page)", t);
  }
  /* append, roll back: the table is restored exactly; a second rollback fails */
  check(kvc_build_visible_table(c, ids0, lens0, CAP, &n0, NULL) == KVC_OK, "table before", FRAMES);
  check(kvc_append_frame(c, NULL, NULL, NULL) == KVC_OK, "append before rollback", FRAMES + 1);
  check(kvc_rollback_last_frame(c) == KVC_OK, "rollback", FRAMES + 1);
  check(kvc_build_visible_table(c, ids, lens, CAP, &n, NULL) == KVC_OK, "table after", FRAMES + 1);
  check(n == n0 && memcmp(ids, ids0, sizeof(int32_t) * (size_t)n) == 0 &&
            memcmp(lens, lens0, sizeof(int32_t) * (size_t)n) == 0,
        "rollback restores the table", FRAMES + 1);
  check(kvc_rollback_last_frame(c) == KVC_ERR_NO_UNDO, "second rollback refused", FRAMES + 1);
  check(strlen(kvc_strerror(KVC_ERR_NO_UNDO)) > 0, "kvc_strerror", FRAMES + 1);
  /* a host-only handle refuses device data */
  check(kvc_append_frame(c, (const void*)16, (const void*)16, NULL) == KVC_ERR_INVALID_ARGUMENT,
        "host-only handle refuses data pointers", FRAMES + 1);
  check(kvc_destroy(c) == KVC_OK, "kvc_destroy", FRAMES + 1);
  if (fails == 0) printf("OK %d frames\n", FRAMES);
  return fails == 0 ? 0 : 1;
}
