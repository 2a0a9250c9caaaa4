/* A plain C caller of libattnres.so: no Python, no torch -- the HIP runtime for
 * device memory and the C ABI of include/attnres.h, nothing else.  It reads one
 * aggregation problem from a file, runs attnres_aggregate on the current GPU
 * (null stream) and writes the results to a file.
 *
 *   capi_client <in> <out>
 *
 *   in:  int32 S, T, d, dtype (ATTNRES_BF16 = 0, ATTNRES_F32 = 1); then the
 *        S x T x d source elements, source-major, 2 or 4 bytes each; then the
 *        d float32 elements of the query.
 *   out: the T x d residual elements (the sources' dtype), then the T x S
 *        float32 weights.
 *
 * Exit status 0 on success; otherwise 1, with the reason (the library's
 * status text where the library refused the call) on stderr.  All of the
 * method's arithmetic happens in the library. */
#define __HIP_PLATFORM_AMD__
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "attnres.h"

static int fail(const char* what) {
  fprintf(stderr, "capi_client: %s\n", what);
  return 1;
}

int main(int argc, char** argv) {
  if (argc != 3) return fail("usage: capi_client <in> <out>");
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) return fail("cannot open the input file");
  int32_t hdr[4];
  if (fread(hdr, sizeof(int32_t), 4, in) != 4) return fail("short header");
  const int32_t S = hdr[0], d = hdr[2], dtype = hdr[3];
  const int64_t T = hdr[1];
  if (S < 1 || S > ATTNRES_MAX_SOURCES_FULL || T < 1 || d < 1 || (dtype != ATTNRES_BF16 && dtype != ATTNRES_F32))
    return fail("bad header");
  const size_t es = dtype == ATTNRES_BF16 ? 2 : 4;
  const size_t n_src = (size_t)S * (size_t)T * (size_t)d, n_out = (size_t)T * (size_t)d;
  const size_t n_wt = (size_t)T * (size_t)S;
  void* h_src = malloc(n_src * es);
  float* h_w = malloc((size_t)d * sizeof(float));
  void* h_out = malloc(n_out * es);
  float* h_wt = malloc(n_wt * sizeof(float));
  if (h_src == NULL || h_w == NULL || h_out == NULL || h_wt == NULL) return fail("out of host memory");
  if (fread(h_src, es, n_src, in) != n_src || fread(h_w, sizeof(float), (size_t)d, in) != (size_t)d)
    return fail("short input");
  fclose(in);

  void *d_src = NULL, *d_out = NULL, *d_w = NULL, *d_wt = NULL;
  if (hipMalloc(&d_src, n_src * es) != hipSuccess || hipMalloc(&d_w, (size_t)d * sizeof(float)) != hipSuccess ||
      hipMalloc(&d_out, n_out * es) != hipSuccess || hipMalloc(&d_wt, n_wt * sizeof(float)) != hipSuccess)
    return fail("hipMalloc failed");
  if (hipMemcpy(d_src, h_src, n_src * es, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(d_w, h_w, (size_t)d * sizeof(float), hipMemcpyHostToDevice) != hipSuccess)
    return fail("copy to the device failed");

  /* src_stride 0: the S rows of [T][d] are contiguous; NULL: the null stream */
  const int rc = attnres_aggregate(d_src, S, T, d, 0, (const float*)d_w, d_out, (float*)d_wt, 1e-5f, dtype, NULL);
  if (rc != ATTNRES_OK) {
    fprintf(stderr, "capi_client: attnres_aggregate: %s\n", attnres_strerror(rc));
    return 1;
  }
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(h_out, d_out, n_out * es, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(h_wt, d_wt, n_wt * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
    return fail("the aggregation or the copy back failed");

  FILE* out = fopen(argv[2], "wb");
  if (out == NULL) return fail("cannot open the output file");
  if (fwrite(h_out, es, n_out, out) != n_out || fwrite(h_wt, sizeof(float), n_wt, out) != n_wt)
    return fail("short write");
  fclose(out);
  (void)hipFree(d_src);
  (void)hipFree(d_w);
  (void)hipFree(d_out);
  (void)hipFree(d_wt);
  free(h_src);
  free(h_w);
  free(h_out);
  free(h_wt);
  return 0;
}
