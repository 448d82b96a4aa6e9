/* A C99 consumer of libkvc.so on the GPU, with no Python in the process:
 * reads a stream of units (K/V) and one query block from a file, creates a
 * bf16 cache with device pools from hipMalloc, appends every unit through
 * kvc_append_frame, rolls back the units that are not keyframes
 * ("LingBot-Map Paged KV Cache", section 3: append, attend, roll back),
 * attends the last unit's queries with kvc_attend, and writes the visible
 * table, O and lse to a file.  tests/test_gpu_c_abi.py writes the input,
 * runs this program and checks its output against the oracle.
 *
 * Input (little-endian int32 header, then bf16 bit patterns):
 *   H, patch_tokens, special_tokens, S, W, units, interval;
 *   per unit: K [T][H][64], V [T][H][64] (T = patch + special tokens);
 *   then Q [T][H][64] of the last unit.
 * Output: int32 n; int32 page_ids[n]; int32 page_lens[n]; O [T][H][64] bf16;
 *   lse [T][H] fp32.  Prints "OK" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvc.h"

#define D 64
#define CAP 1024

static int die(const char* what, int status) {
  printf("FAIL %s: status %d (%s) %s\n", what, status, kvc_strerror(status), kvc_last_error());
  return 1;
}

static int hip_die(const char* what, hipError_t e) {
  printf("FAIL %s: %s\n", what, hipGetErrorString(e));
  return 1;
}

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  int32_t hdr[7];
  FILE* f;
  kvc_config cfg;
  kvc_t* c = NULL;
  size_t pool_bytes = 0, ws_bytes = 0, unit_bytes, lse_bytes;
  void *kp = NULL, *vp = NULL, *dk = NULL, *dv = NULL, *dq = NULL, *dout = NULL, *dws = NULL;
  float* dlse = NULL;
  uint16_t *hk, *hv, *hq, *hout;
  float* hlse;
  hipStream_t st;
  hipError_t e;
  int32_t ids[CAP], lens[CAP], n = 0, last = 0, H, T, S, units, interval, t;
  int s;

  if (argc != 3) {
    printf("usage: %s input output\n", argv[0]);
    return 2;
  }
  f = fopen(argv[1], "rb");
  if (!f || !read_all(f, hdr, sizeof hdr)) {
    printf("FAIL reading %s\n", argv[1]);
    return 1;
  }
  H = hdr[0];
  T = hdr[1] + hdr[2];
  S = hdr[3];
  units = hdr[5];
  interval = hdr[6];
  memset(&cfg, 0, sizeof cfg);
  cfg.num_heads = H;
  cfg.head_dim = D;
  cfg.page_size = 256;
  cfg.dtype = KVC_DTYPE_BF16;
  cfg.patch_tokens = hdr[1];
  cfg.special_tokens = hdr[2];
  cfg.num_scale_units = S;
  cfg.window_units = hdr[4];
  cfg.special_packing = KVC_SPECIAL_FRAME_ALIGNED;
  cfg.max_units = units;
  unit_bytes = (size_t)T * H * D * sizeof(uint16_t);
  lse_bytes = (size_t)T * H * sizeof(float);
  hk = (uint16_t*)malloc(unit_bytes);
  hv = (uint16_t*)malloc(unit_bytes);
  hq = (uint16_t*)malloc(unit_bytes);
  hout = (uint16_t*)malloc(unit_bytes);
  hlse = (float*)malloc(lse_bytes);
  if (!hk || !hv || !hq || !hout || !hlse) {
    printf("FAIL host allocation\n");
    return 1;
  }

  if ((s = kvc_pool_bytes(&cfg, &pool_bytes))) return die("kvc_pool_bytes", s);
  if ((e = hipMalloc(&kp, pool_bytes)) != hipSuccess) return hip_die("hipMalloc k_pool", e);
  if ((e = hipMalloc(&vp, pool_bytes)) != hipSuccess) return hip_die("hipMalloc v_pool", e);
  if ((s = kvc_create(&cfg, kp, vp, &c))) return die("kvc_create", s);
  if ((s = kvc_attend_workspace_size(c, T, &ws_bytes))) return die("kvc_attend_workspace_size", s);
  if ((e = hipMalloc(&dk, unit_bytes)) != hipSuccess) return hip_die("hipMalloc k", e);
  if ((e = hipMalloc(&dv, unit_bytes)) != hipSuccess) return hip_die("hipMalloc v", e);
  if ((e = hipMalloc(&dq, unit_bytes)) != hipSuccess) return hip_die("hipMalloc q", e);
  if ((e = hipMalloc(&dout, unit_bytes)) != hipSuccess) return hip_die("hipMalloc o", e);
  if ((e = hipMalloc((void**)&dlse, lse_bytes)) != hipSuccess) return hip_die("hipMalloc lse", e);
  if (ws_bytes && (e = hipMalloc(&dws, ws_bytes)) != hipSuccess) return hip_die("hipMalloc workspace", e);
  if ((e = hipStreamCreate(&st)) != hipSuccess) return hip_die("hipStreamCreate", e);

  for (t = 0; t < units; ++t) {
    const int keep = t < S || interval <= 1 || (t - S) % interval == 0;
    if (!read_all(f, hk, unit_bytes) || !read_all(f, hv, unit_bytes)) {
      printf("FAIL reading unit %d\n", t);
      return 1;
    }
    /* the previous append has read the unit buffers before they are written again */
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_die("hipStreamSynchronize", e);
    if ((e = hipMemcpy(dk, hk, unit_bytes, hipMemcpyHostToDevice)) != hipSuccess) return hip_die("copy k", e);
    if ((e = hipMemcpy(dv, hv, unit_bytes, hipMemcpyHostToDevice)) != hipSuccess) return hip_die("copy v", e);
    if ((s = kvc_append_frame(c, dk, dv, (kvc_stream_t)st))) return die("kvc_append_frame", s);
    if (t == units - 1) break; /* the last unit is attended before any rollback */
    if (!keep && (s = kvc_rollback_last_frame(c))) return die("kvc_rollback_last_frame", s);
  }
  if (!read_all(f, hq, unit_bytes)) {
    printf("FAIL reading q\n");
    return 1;
  }
  fclose(f);
  if ((e = hipMemcpy(dq, hq, unit_bytes, hipMemcpyHostToDevice)) != hipSuccess) return hip_die("copy q", e);
  if ((s = kvc_attend(c, dq, T, 0.f, dout, dlse, dws, ws_bytes, (kvc_stream_t)st))) return die("kvc_attend", s);
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_die("hipStreamSynchronize", e);
  if ((e = hipMemcpy(hout, dout, unit_bytes, hipMemcpyDeviceToHost)) != hipSuccess) return hip_die("copy o", e);
  if ((e = hipMemcpy(hlse, dlse, lse_bytes, hipMemcpyDeviceToHost)) != hipSuccess) return hip_die("copy lse", e);
  if ((s = kvc_build_visible_table(c, ids, lens, CAP, &n, &last))) return die("kvc_build_visible_table", s);
  if (n > 0 && lens[n - 1] != last) {
    printf("FAIL last_page_len %d against the table's %d\n", last, lens[n - 1]);
    return 1;
  }

  f = fopen(argv[2], "wb");
  if (!f || fwrite(&n, sizeof n, 1, f) != 1 || fwrite(ids, sizeof(int32_t), (size_t)n, f) != (size_t)n ||
      fwrite(lens, sizeof(int32_t), (size_t)n, f) != (size_t)n || fwrite(hout, 1, unit_bytes, f) != unit_bytes ||
      fwrite(hlse, 1, lse_bytes, f) != lse_bytes) {
    printf("FAIL writing %s\n", argv[2]);
    return 1;
  }
  fclose(f);

  if ((s = kvc_destroy(c))) return die("kvc_destroy", s);
  hipStreamDestroy(st);
  hipFree(kp);
  hipFree(vp);
  hipFree(dk);
  hipFree(dv);
  hipFree(dq);
  hipFree(dout);
  hipFree(dlse);
  if (dws) hipFree(dws);
  free(hk);
  free(hv);
  free(hq);
  free(hout);
  free(hlse);
  printf("OK %d pages\n", n);
  return 0;
}
