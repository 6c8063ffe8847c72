/*
 * A plain C99 consumer of the library's C ABI (include/moe.h): one bf16 MoE
 * layer, forward and backward, with device memory from the HIP runtime's C
 * API and nothing else. It exists to show that the boundary needs no C++,
 * no Python and no torch: plain pointers, sizes and a stream handle.
 *
 *   moe_layer --host     no GPU: version, a workspace query and a rejected
 *                        shape (k > E), printed one per line
 *   moe_layer IN OUT     route (logits given), permute, grouped FFN forward,
 *                        combine, then their backward, on the default stream
 *
 * IN (little-endian): int64 T; int32 d, E, k, F; then bf16 bit patterns of
 * x [T,d], fp32 logits [T,E], bf16 w_gu [E,2F,d], bf16 w_down [E,d,F], bf16
 * dout [T,d]. OUT: the raw arrays topk_idx, topk_w, counts, offsets,
 * row_of_slot, src_of_row, x_perm, h, a, y, out, dy, dtopk_w, dlogits,
 * dx_perm, dh, dx, dw_gu, dw_down in that order (dh is the first R*2F*2 bytes
 * of the backward workspace, where the grouped backward keeps it).
 *
 * Exit status: 0 on success, 2 usage, 3 HIP error, 4 library error, 5 I/O.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

#define CHECK_HIP(call)                                                                          \
  do {                                                                                           \
    hipError_t e_ = (call);                                                                      \
    if (e_ != hipSuccess) {                                                                      \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_));      \
      exit(3);                                                                                   \
    }                                                                                            \
  } while (0)

#define CHECK_MOE(call)                                                                          \
  do {                                                                                           \
    moe_status s_ = (call);                                                                      \
    if (s_ != MOE_OK) {                                                                          \
      fprintf(stderr, "%s:%d: %s: %s (%s)\n", __FILE__, __LINE__, #call, moe_status_string(s_),  \
              moe_last_error());                                                                 \
      exit(4);                                                                                   \
    }                                                                                            \
  } while (0)

static void *dev_alloc(size_t n) {
  void *p = NULL;
  if (n > 0) CHECK_HIP(hipMalloc(&p, n));
  return p;
}

static void read_exact(FILE *f, void *host, size_t n) {
  if (n > 0 && fread(host, 1, n, f) != n) {
    fprintf(stderr, "short read (%zu bytes wanted)\n", n);
    exit(5);
  }
}

/* n bytes from the file into device memory */
static void read_dev(FILE *f, void *dev, size_t n) {
  void *h;
  if (n == 0) return;
  h = malloc(n);
  if (!h) exit(5);
  read_exact(f, h, n);
  CHECK_HIP(hipMemcpy(dev, h, n, hipMemcpyHostToDevice));
  free(h);
}

/* n bytes of device memory to the file */
static void write_dev(FILE *f, const void *dev, size_t n) {
  void *h;
  if (n == 0) return;
  h = malloc(n);
  if (!h) exit(5);
  CHECK_HIP(hipMemcpy(h, dev, n, hipMemcpyDeviceToHost));
  if (fwrite(h, 1, n, f) != n) exit(5);
  free(h);
}

static int host_only(void) {
  moe_shape s;
  size_t r = 0, g = 0, b = 0;
  moe_status st;
  memset(&s, 0, sizeof s);
  s.T = 4096;
  s.d = 1024;
  s.E = 8;
  s.k = 2;
  s.F = 2816;
  s.dtype = MOE_DTYPE_BF16;
  printf("version %s\n", moe_version());
  st = moe_workspace_size(&s, &r, &g, &b);
  printf("workspace %d %zu %zu %zu\n", (int)st, r, g, b);
  s.k = 9; /* k > E */
  st = moe_workspace_size(&s, &r, &g, &b);
  printf("rejected %d %s\n", (int)st, moe_status_string(st));
  return 0;
}

int main(int argc, char **argv) {
  FILE *in, *out;
  int64_t T;
  int32_t dims[4];
  moe_shape sh;
  size_t R, d, E, k, F, ws_route = 0, ws_fwd = 0, ws_bwd = 0;
  void *x, *w_gu, *w_down, *dout, *x_perm, *h, *a, *y, *o, *dy, *dx_perm, *dx, *ws_r, *ws_f, *ws_b;
  float *logits, *topk_w, *dtopk_w, *dlogits, *dw_gu, *dw_down;
  int32_t *topk_idx, *counts, *offsets, *row_of_slot, *src_of_row;

  if (argc == 2 && strcmp(argv[1], "--host") == 0) return host_only();
  if (argc != 3) {
    fprintf(stderr, "usage: %s --host | %s IN OUT\n", argv[0], argv[0]);
    return 2;
  }
  in = fopen(argv[1], "rb");
  if (!in) return 5;
  read_exact(in, &T, sizeof T);
  read_exact(in, dims, sizeof dims);
  memset(&sh, 0, sizeof sh);
  sh.T = T;
  sh.d = dims[0];
  sh.E = dims[1];
  sh.k = dims[2];
  sh.F = dims[3];
  sh.dtype = MOE_DTYPE_BF16;
  d = (size_t)sh.d;
  E = (size_t)sh.E;
  k = (size_t)sh.k;
  F = (size_t)sh.F;
  R = (size_t)T * k;
  CHECK_MOE(moe_workspace_size(&sh, &ws_route, &ws_fwd, &ws_bwd));

  x = dev_alloc((size_t)T * d * 2);
  logits = (float *)dev_alloc((size_t)T * E * 4);
  w_gu = dev_alloc(E * 2 * F * d * 2);
  w_down = dev_alloc(E * d * F * 2);
  dout = dev_alloc((size_t)T * d * 2);
  topk_idx = (int32_t *)dev_alloc(R * 4);
  topk_w = (float *)dev_alloc(R * 4);
  counts = (int32_t *)dev_alloc(E * 4);
  offsets = (int32_t *)dev_alloc((E + 1) * 4);
  row_of_slot = (int32_t *)dev_alloc(R * 4);
  src_of_row = (int32_t *)dev_alloc(R * 4);
  x_perm = dev_alloc(R * d * 2);
  h = dev_alloc(R * 2 * F * 2);
  a = dev_alloc(R * F * 2);
  y = dev_alloc(R * d * 2);
  o = dev_alloc((size_t)T * d * 2);
  dy = dev_alloc(R * d * 2);
  dtopk_w = (float *)dev_alloc(R * 4);
  dlogits = (float *)dev_alloc((size_t)T * E * 4);
  dx_perm = dev_alloc(R * d * 2);
  dx = dev_alloc((size_t)T * d * 2);
  dw_gu = (float *)dev_alloc(E * 2 * F * d * 4);
  dw_down = (float *)dev_alloc(E * d * F * 4);
  ws_r = dev_alloc(ws_route);
  ws_f = dev_alloc(ws_fwd);
  ws_b = dev_alloc(ws_bwd);
  CHECK_HIP(hipMemset(dw_gu, 0, E * 2 * F * d * 4));
  CHECK_HIP(hipMemset(dw_down, 0, E * d * F * 4));

  read_dev(in, x, (size_t)T * d * 2);
  read_dev(in, logits, (size_t)T * E * 4);
  read_dev(in, w_gu, E * 2 * F * d * 2);
  read_dev(in, w_down, E * d * F * 2);
  read_dev(in, dout, (size_t)T * d * 2);
  fclose(in);

  /* forward */
  CHECK_MOE(moe_route(&sh, NULL, NULL, NULL, logits, topk_idx, topk_w, counts, offsets, row_of_slot, src_of_row,
                      ws_r, ws_route, NULL));
  CHECK_MOE(moe_permute(&sh, x, row_of_slot, x_perm, NULL));
  CHECK_MOE(moe_grouped_gemm_fwd(&sh, x_perm, w_gu, w_down, offsets, h, a, y, ws_f, ws_fwd, NULL));
  CHECK_MOE(moe_unpermute_combine(&sh, y, topk_w, row_of_slot, o, NULL));
  /* backward */
  CHECK_MOE(moe_unpermute_combine_bwd(&sh, dout, y, topk_w, row_of_slot, dy, dtopk_w, NULL));
  CHECK_MOE(moe_route_bwd(&sh, dtopk_w, logits, topk_idx, topk_w, NULL, NULL, dlogits, NULL, NULL, ws_r, ws_route,
                          NULL));
  CHECK_MOE(moe_grouped_gemm_bwd(&sh, dy, x_perm, h, a, w_gu, w_down, offsets, dx_perm, dw_gu, dw_down, ws_b,
                                 ws_bwd, NULL));
  CHECK_MOE(moe_permute_bwd(&sh, dx_perm, row_of_slot, NULL, dx, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  out = fopen(argv[2], "wb");
  if (!out) return 5;
  write_dev(out, topk_idx, R * 4);
  write_dev(out, topk_w, R * 4);
  write_dev(out, counts, E * 4);
  write_dev(out, offsets, (E + 1) * 4);
  write_dev(out, row_of_slot, R * 4);
  write_dev(out, src_of_row, R * 4);
  write_dev(out, x_perm, R * d * 2);
  write_dev(out, h, R * 2 * F * 2);
  write_dev(out, a, R * F * 2);
  write_dev(out, y, R * d * 2);
  write_dev(out, o, (size_t)T * d * 2);
  write_dev(out, dy, R * d * 2);
  write_dev(out, dtopk_w, R * 4);
  write_dev(out, dlogits, (size_t)T * E * 4);
  write_dev(out, dx_perm, R * d * 2);
  write_dev(out, ws_b, R * 2 * F * 2);
  write_dev(out, dx, (size_t)T * d * 2);
  write_dev(out, dw_gu, E * 2 * F * d * 4);
  write_dev(out, dw_down, E * d * F * 4);
  if (fclose(out) != 0) return 5;

  hipFree(x);
  hipFree(logits);
  hipFree(w_gu);
  hipFree(w_down);
  hipFree(dout);
  hipFree(topk_idx);
  hipFree(topk_w);
  hipFree(counts);
  hipFree(offsets);
  hipFree(row_of_slot);
  hipFree(src_of_row);
  hipFree(x_perm);
  hipFree(h);
  hipFree(a);
  hipFree(y);
  hipFree(o);
  hipFree(dy);
  hipFree(dtopk_w);
  hipFree(dlogits);
  hipFree(dx_perm);
  hipFree(dx);
  hipFree(dw_gu);
  hipFree(dw_down);
  hipFree(ws_r);
  hipFree(ws_f);
  hipFree(ws_b);
  return 0;
}
