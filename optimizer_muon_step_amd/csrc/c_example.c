/*
 * A plain C caller of the library: one Muon step (muon_step_ex) over the
 * matrices described in an input file, with device memory from the HIP
 * runtime and the results written to an output file.  It shows the C ABI in
 * use without Python, and the test suite runs it against the Python binding.
 *
 * Input file (native byte order):
 *   int32 n; float lr, beta; int32 ns_steps; float a, b, c;
 *   n x { int64 rows, int64 cols };
 *   for each matrix: W, G, M as rows*cols fp32 each.
 * Output file: for each matrix, W and M (fp32) and the applied bf16 update
 * (rows*cols uint16 each).
 *
 * Usage: muon_c_example IN OUT.  Exit status 0 on success, 1 with a message
 * on stderr otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "muon.h"

static int fail(const char* what, const char* detail) {
  fprintf(stderr, "muon_c_example: %s%s%s\n", what, detail ? ": " : "", detail ? detail : "");
  return 1;
}

#define HIP_TRY(call)                                              \
  do {                                                             \
    hipError_t e_ = (call);                                        \
    if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_)); \
  } while (0)

static int read_all(FILE* f, void* p, size_t bytes) { return fread(p, 1, bytes, f) == bytes; }
static int write_all(FILE* f, const void* p, size_t bytes) { return fwrite(p, 1, bytes, f) == bytes; }

int main(int argc, char** argv) {
  if (argc != 3) return fail("usage", "muon_c_example IN OUT");
  FILE* in = fopen(argv[1], "rb");
  if (!in) return fail("cannot open", argv[1]);
  int32_t n = 0, ns_steps = 0;
  float lr = 0.f, beta = 0.f, coeffs[3];
  if (!read_all(in, &n, 4) || !read_all(in, &lr, 4) || !read_all(in, &beta, 4) || !read_all(in, &ns_steps, 4) ||
      !read_all(in, coeffs, sizeof coeffs) || n < 1 || n > 1024)
    return fail("bad header", argv[1]);
  muon_shape_t* shapes = (muon_shape_t*)calloc((size_t)n, sizeof *shapes);
  float** W = (float**)calloc((size_t)n, sizeof *W);
  float** G = (float**)calloc((size_t)n, sizeof *G);
  float** M = (float**)calloc((size_t)n, sizeof *M);
  uint16_t** U = (uint16_t**)calloc((size_t)n, sizeof *U);
  if (!shapes || !W || !G || !M || !U) return fail("out of host memory", NULL);
  for (int i = 0; i < n; ++i)
    if (!read_all(in, &shapes[i].rows, 8) || !read_all(in, &shapes[i].cols, 8)) return fail("bad shapes", argv[1]);

  size_t max_elems = 0;
  for (int i = 0; i < n; ++i) {
    const size_t e = (size_t)(shapes[i].rows * shapes[i].cols);
    if (e > max_elems) max_elems = e;
  }
  float* host = (float*)malloc(max_elems * sizeof(float));
  if (!host) return fail("out of host memory", NULL);
  for (int i = 0; i < n; ++i) {
    const size_t e = (size_t)(shapes[i].rows * shapes[i].cols);
    float** dst[3] = {&W[i], &G[i], &M[i]};
    for (int k = 0; k < 3; ++k) {
      if (!read_all(in, host, e * sizeof(float))) return fail("short input", argv[1]);
      HIP_TRY(hipMalloc((void**)dst[k], e * sizeof(float)));
      HIP_TRY(hipMemcpy(*dst[k], host, e * sizeof(float), hipMemcpyHostToDevice));
    }
    HIP_TRY(hipMalloc((void**)&U[i], e * sizeof(uint16_t)));
  }
  fclose(in);

  hipStream_t stream;
  HIP_TRY(hipStreamCreate(&stream));
  const int rc = muon_step_ex(W, (const float* const*)G, M, shapes, n, lr, beta, ns_steps, coeffs, U, stream);
  if (rc != MUON_OK) return fail("muon_step_ex", muon_last_error());
  HIP_TRY(hipStreamSynchronize(stream));

  FILE* out = fopen(argv[2], "wb");
  if (!out) return fail("cannot open", argv[2]);
  for (int i = 0; i < n; ++i) {
    const size_t e = (size_t)(shapes[i].rows * shapes[i].cols);
    HIP_TRY(hipMemcpy(host, W[i], e * sizeof(float), hipMemcpyDeviceToHost));
    if (!write_all(out, host, e * sizeof(float))) return fail("write failed", argv[2]);
    HIP_TRY(hipMemcpy(host, M[i], e * sizeof(float), hipMemcpyDeviceToHost));
    if (!write_all(out, host, e * sizeof(float))) return fail("write failed", argv[2]);
    HIP_TRY(hipMemcpy(host, U[i], e * sizeof(uint16_t), hipMemcpyDeviceToHost));
    if (!write_all(out, host, e * sizeof(uint16_t))) return fail("write failed", argv[2]);
    HIP_TRY(hipFree(W[i]));
    HIP_TRY(hipFree(G[i]));
    HIP_TRY(hipFree(M[i]));
    HIP_TRY(hipFree(U[i]));
  }
  if (fclose(out) != 0) return fail("close failed", argv[2]);
  HIP_TRY(hipStreamDestroy(stream));
  muon_release();
  free(host);
  free(shapes);
  free(W);
  free(G);
  free(M);
  free(U);
  return 0;
}
