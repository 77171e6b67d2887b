/* A plain C caller of the MoE layer library: device buffers from hipMalloc,
 * a HIP stream of its own, the workspace sized by moe_workspace_bytes, and one
 * moe_forward call.  No Python and no torch anywhere in the process.
 *
 *   moe_c_caller DIR T d E d_ff k
 *
 * reads DIR/x.bin [T][d], DIR/Wg.bin [E][d], DIR/W1.bin and DIR/W3.bin
 * [E][d_ff][d], DIR/W2.bin [E][d][d_ff] (raw bf16 bit patterns, little
 * endian), runs the layer on device 0 and writes DIR/y.bin [T][d] (bf16).
 * Exit status 0 on success; a library or HIP error is printed with its text. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/moe_mi355x.h"

static int hip_ok(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

/* read n bytes of DIR/name into a new device buffer */
static void *load(const char *dir, const char *name, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return NULL;
  }
  void *h = malloc(n), *d = NULL;
  const size_t got = h ? fread(h, 1, n, f) : 0;
  fclose(f);
  if (got != n) {
    fprintf(stderr, "%s: read %zu of %zu bytes\n", path, got, n);
    free(h);
    return NULL;
  }
  if (!hip_ok(hipMalloc(&d, n), "hipMalloc") || !hip_ok(hipMemcpy(d, h, n, hipMemcpyHostToDevice), "copy in"))
    d = NULL;
  free(h);
  return d;
}

int main(int argc, char **argv) {
  if (argc != 7) {
    fprintf(stderr, "usage: %s DIR T d E d_ff k\n", argv[0]);
    return 2;
  }
  const char *dir = argv[1];
  const int T = atoi(argv[2]), d = atoi(argv[3]), E = atoi(argv[4]), dff = atoi(argv[5]),
            k = atoi(argv[6]);
  if (T <= 0 || d <= 0 || E <= 0 || dff <= 0 || k <= 0) return 2;
  if (!hip_ok(hipSetDevice(0), "hipSetDevice")) return 1;
  const size_t bx = (size_t)T * d * 2, bw = (size_t)E * dff * d * 2;
  void *x = load(dir, "x.bin", bx), *Wg = load(dir, "Wg.bin", (size_t)E * d * 2);
  void *W1 = load(dir, "W1.bin", bw), *W3 = load(dir, "W3.bin", bw), *W2 = load(dir, "W2.bin", bw);
  if (!x || !Wg || !W1 || !W3 || !W2) return 1;
  const size_t wsb = moe_workspace_bytes(T, d, dff, E, k, 0, MOE_BF16);
  void *ws = NULL, *y = NULL;
  hipStream_t s;
  if (!hip_ok(hipMalloc(&ws, wsb), "hipMalloc workspace") || !hip_ok(hipMalloc(&y, bx), "hipMalloc y") ||
      !hip_ok(hipStreamCreate(&s), "hipStreamCreate"))
    return 1;
  const int rc = moe_forward(x, Wg, NULL, W1, W3, W2, NULL, NULL, NULL, 0, T, E, k, d, dff, MOE_BF16,
                             ws, wsb, y, (void *)s);
  if (rc != MOE_OK) {
    fprintf(stderr, "moe_forward: %s\n", moe_strerror(rc));
    return 1;
  }
  if (!hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return 1;
  void *hy = malloc(bx);
  if (!hy || !hip_ok(hipMemcpy(hy, y, bx, hipMemcpyDeviceToHost), "copy out")) return 1;
  char path[4096];
  snprintf(path, sizeof path, "%s/y.bin", dir);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(hy, 1, bx, f) != bx) {
    fprintf(stderr, "cannot write %s\n", path);
    return 1;
  }
  fclose(f);
  free(hy);
  hipFree(x);
  hipFree(Wg);
  hipFree(W1);
  hipFree(W3);
  hipFree(W2);
  hipFree(ws);
  hipFree(y);
  hipStreamDestroy(s);
  printf("moe_c_caller: T=%d d=%d E=%d d_ff=%d k=%d workspace %zu bytes: ok\n", T, d, E, dff, k, wsb);
  return 0;
}
