/*
 * A plain C caller of libmxq: no PyTorch and no Python binding, only include/mxq.h and
 * the HIP runtime. It reads a row-major bf16 tensor [rows, cols] from a file, copies it
 * to device memory from hipMalloc, quantises it to MXFP4 row- and column-wise in one
 * call (nearest even), dequantises the row-wise codes back to bf16, quantises it to
 * NVFP4 row-wise with no amax given (the library computes the tensor amax and s_t),
 * and writes every output to <prefix>.codes_row, .scales_row, .codes_col,
 * .scales_col, .deq_row, .nv_codes, .nv_scales and .nv_st. Given token offsets of
 * experts (offsets[0] = 0, ..., offsets[E] = rows), it also converts the MXFP4 rows
 * to FP8 columns per 128-token expert group: <prefix>.fc_q8 (E4M3 [cols, ld_q8],
 * ld_q8 = rows rounded up to 16) and .fc_s (fp32 [cols, (rows + 127 E) / 128]).
 *
 * usage: mxq_c_caller rows cols input.bin prefix [offsets...]
 *        (rows % 32 == 0, cols % 32 == 0)
 * Exit status: 0 on success, 1 on a usage or I/O error, 2 on a library or HIP error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "mxq.h"

static int hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return 1;
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 0;
}

static int write_file(const char* prefix, const char* ext, const void* p, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s.%s", prefix, ext);
  FILE* f = fopen(path, "wb");
  if (!f) return 0;
  const size_t w = fwrite(p, 1, n, f);
  fclose(f);
  return w == n;
}

int main(int argc, char** argv) {
  if (argc < 5 || argc == 6) {
    fprintf(stderr, "usage: %s rows cols input.bin prefix [offsets...]\n", argv[0]);
    return 1;
  }
  const int64_t rows = atoll(argv[1]), cols = atoll(argv[2]);
  if (rows <= 0 || cols <= 0 || rows % 32 || cols % 32) {
    fprintf(stderr, "rows and cols must be positive multiples of 32\n");
    return 1;
  }
  const size_t n = (size_t)rows * (size_t)cols;
  const int64_t n_experts = argc > 5 ? argc - 6 : 0;
  int64_t* offsets = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_experts + 1));
  for (int64_t e = 0; e <= n_experts && n_experts > 0; ++e) offsets[e] = atoll(argv[5 + e]);
  const int64_t ld_q8 = (rows + 15) / 16 * 16, ld_s = (rows + 127 * n_experts) / 128;
  const size_t fc_sizes[3] = {(size_t)cols * (size_t)ld_q8, (size_t)cols * (size_t)ld_s * sizeof(float),
                              sizeof(int64_t) * (size_t)(n_experts + 1)};
  void* dfc[3] = {0, 0, 0};  /* FP8 columns, their scales, the offsets */
  uint8_t* fc_host[2] = {0, 0};
  const size_t sizes[5] = {n * 2, n / 2, n / 32, n / 2, n / 32};  /* x, codes/scales row, codes/scales col */
  uint8_t* host[5];
  int have = 1;
  for (int i = 0; i < 5; ++i) have &= (host[i] = (uint8_t*)malloc(sizes[i])) != NULL;
  uint16_t* deq = (uint16_t*)malloc(n * 2);
  FILE* f = have && deq ? fopen(argv[3], "rb") : NULL;
  const int read_ok = f && fread(host[0], 1, sizes[0], f) == sizes[0];
  if (f) fclose(f);
  if (!read_ok) {
    fprintf(stderr, "cannot read %zu bytes from %s\n", sizes[0], argv[3]);
    for (int i = 0; i < 5; ++i) free(host[i]);
    free(deq);
    free(offsets);
    return 1;
  }

  void* dev[5] = {0, 0, 0, 0, 0};
  void* ddeq = 0;
  void* dnv[3] = {0, 0, 0};  /* NVFP4 codes, block scales, tensor scale */
  const size_t nv_sizes[3] = {n / 2, n / 16, sizeof(float)};
  uint8_t* nv_host[3] = {0, 0, 0};
  int ok = 1;
  for (int i = 0; i < 5 && ok; ++i) ok = hip_ok(hipMalloc(&dev[i], sizes[i]), "hipMalloc");
  if (ok) ok = hip_ok(hipMalloc(&ddeq, n * 2), "hipMalloc");
  for (int i = 0; i < 3 && ok; ++i) ok = hip_ok(hipMalloc(&dnv[i], nv_sizes[i]), "hipMalloc");
  for (int i = 0; i < 3 && ok; ++i) ok = (nv_host[i] = (uint8_t*)malloc(nv_sizes[i])) != NULL;
  if (n_experts > 0) {
    for (int i = 0; i < 3 && ok; ++i) ok = hip_ok(hipMalloc(&dfc[i], fc_sizes[i]), "hipMalloc");
    for (int i = 0; i < 2 && ok; ++i) ok = (fc_host[i] = (uint8_t*)malloc(fc_sizes[i])) != NULL;
    if (ok) ok = hip_ok(hipMemcpy(dfc[2], offsets, fc_sizes[2], hipMemcpyHostToDevice), "hipMemcpy offsets");
  }
  if (ok) ok = hip_ok(hipMemcpy(dev[0], host[0], sizes[0], hipMemcpyHostToDevice), "hipMemcpy in");
  if (ok) {
    /* a null stream: the device's default stream */
    mxq_status s = mxq_quantize(dev[0], MXQ_BF16, rows, cols, cols, MXQ_MXFP4, MXQ_BOTH, MXQ_RNE, 0, 0,
                                (uint8_t*)dev[1], (uint8_t*)dev[2], (uint8_t*)dev[3], (uint8_t*)dev[4], NULL,
                                NULL, NULL);
    if (s == MXQ_OK)
      s = mxq_dequantize((const uint8_t*)dev[1], (const uint8_t*)dev[2], MXQ_MXFP4, rows, cols, NULL, ddeq,
                         MXQ_BF16, NULL);
    /* amax NULL: the tensor amax is computed into the tensor-scale slot first */
    if (s == MXQ_OK)
      s = mxq_quantize(dev[0], MXQ_BF16, rows, cols, cols, MXQ_NVFP4, MXQ_ROWWISE, MXQ_RNE, 0, 0,
                       (uint8_t*)dnv[0], (uint8_t*)dnv[1], NULL, NULL, NULL, (float*)dnv[2], NULL);
    /* the MXFP4 rows just written, as FP8 columns per expert group */
    if (s == MXQ_OK && n_experts > 0)
      s = mxq_fp4_row_to_fp8_col((const uint8_t*)dev[1], (const uint8_t*)dev[2], rows, cols,
                                 (const int64_t*)dfc[2], n_experts, (uint8_t*)dfc[0], ld_q8, (float*)dfc[1],
                                 ld_s, NULL);
    if (s != MXQ_OK) {
      fprintf(stderr, "libmxq: %s\n", mxq_status_string(s));
      ok = 0;
    }
  }
  if (ok) ok = hip_ok(hipDeviceSynchronize(), "kernels");
  for (int i = 1; i < 5 && ok; ++i) ok = hip_ok(hipMemcpy(host[i], dev[i], sizes[i], hipMemcpyDeviceToHost), "hipMemcpy out");
  if (ok) ok = hip_ok(hipMemcpy(deq, ddeq, n * 2, hipMemcpyDeviceToHost), "hipMemcpy out");
  for (int i = 0; i < 3 && ok; ++i)
    ok = hip_ok(hipMemcpy(nv_host[i], dnv[i], nv_sizes[i], hipMemcpyDeviceToHost), "hipMemcpy out");
  for (int i = 0; i < 5; ++i)
    if (dev[i]) hipFree(dev[i]);
  if (ddeq) hipFree(ddeq);
  for (int i = 0; i < 2 && ok && n_experts > 0; ++i)
    ok = hip_ok(hipMemcpy(fc_host[i], dfc[i], fc_sizes[i], hipMemcpyDeviceToHost), "hipMemcpy out");
  for (int i = 0; i < 3; ++i)
    if (dnv[i]) hipFree(dnv[i]);
  for (int i = 0; i < 3; ++i)
    if (dfc[i]) hipFree(dfc[i]);

  int status = ok ? 0 : 2;
  const char* ext[5] = {"", "codes_row", "scales_row", "codes_col", "scales_col"};
  for (int i = 1; i < 5 && status == 0; ++i)
    if (!write_file(argv[4], ext[i], host[i], sizes[i])) status = 1;
  if (status == 0 && !write_file(argv[4], "deq_row", deq, n * 2)) status = 1;
  const char* nv_ext[3] = {"nv_codes", "nv_scales", "nv_st"};
  for (int i = 0; i < 3 && status == 0; ++i)
    if (!write_file(argv[4], nv_ext[i], nv_host[i], nv_sizes[i])) status = 1;
  const char* fc_ext[2] = {"fc_q8", "fc_s"};
  for (int i = 0; i < 2 && status == 0 && n_experts > 0; ++i)
    if (!write_file(argv[4], fc_ext[i], fc_host[i], fc_sizes[i])) status = 1;
  for (int i = 0; i < 2; ++i) free(fc_host[i]);
  free(offsets);
  for (int i = 0; i < 3; ++i) free(nv_host[i]);
  for (int i = 0; i < 5; ++i) free(host[i]);
  free(deq);
  if (status == 0) printf("ok %lld x %lld\n", (long long)rows, (long long)cols);
  return status;
}
