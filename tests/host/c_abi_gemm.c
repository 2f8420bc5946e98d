/* The library driven from plain C through include/patch.h and the HIP runtime's
 * C API: no C++, no Python binding, no torch.  Used by tests/test_gpu_c_abi.py,
 * which writes the input file, runs this program and checks its output against
 * the oracle.
 *
 *   c_abi_gemm IN OUT
 *
 * IN:  int64 n, k, m, tile_n, tile_k; then W bf16 [n][k], the keep mask bits
 *      (MSB first) ceil(n*k/8) bytes, X bf16 [m][k].
 * OUT: int64 n_dense, n_sparse; Y bf16 [m][n]; Y fp32 [m][n]; then the exported
 *      tile_map, tile_slot (int32), dense_vals, sparse_vals, sparse_meta.
 * Exit status 0 on success; otherwise the failing call and patch_last_error()
 * go to stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "patch.h"

#define CHECK_HIP(call)                                                         \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                \
      return 2;                                                                 \
    }                                                                           \
  } while (0)
#define CHECK_PATCH(call)                                                       \
  do {                                                                          \
    patch_status s_ = (call);                                                   \
    if (s_ != PATCH_OK) {                                                       \
      fprintf(stderr, "%s: status %d: %s\n", #call, (int)s_, patch_last_error()); \
      return 3;                                                                 \
    }                                                                           \
  } while (0)

static int read_all(FILE* f, void* p, size_t bytes) { return fread(p, 1, bytes, f) == bytes; }
static int write_all(FILE* f, const void* p, size_t bytes) { return fwrite(p, 1, bytes, f) == bytes; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 1;
  int64_t hdr[5];
  if (!read_all(in, hdr, sizeof hdr)) return 1;
  const int64_t n = hdr[0], k = hdr[1], m = hdr[2];
  const int32_t tn = (int32_t)hdr[3], tk = (int32_t)hdr[4];
  const size_t w_bytes = (size_t)(n * k * 2), bit_bytes = (size_t)((n * k + 7) / 8), x_bytes = (size_t)(m * k * 2);
  const size_t y16_bytes = (size_t)(m * n * 2), y32_bytes = (size_t)(m * n * 4);
  uint16_t* w = malloc(w_bytes);
  uint8_t* bits = malloc(bit_bytes);
  uint16_t* x = malloc(x_bytes);
  uint16_t* y16 = malloc(y16_bytes);
  float* y32 = malloc(y32_bytes);
  if (!w || !bits || !x || !y16 || !y32) return 1;
  if (!read_all(in, w, w_bytes) || !read_all(in, bits, bit_bytes) || !read_all(in, x, x_bytes)) return 1;
  fclose(in);

  void *dw, *dbits, *dx, *dy16, *dy32;
  CHECK_HIP(hipMalloc(&dw, w_bytes));
  CHECK_HIP(hipMalloc(&dbits, bit_bytes));
  CHECK_HIP(hipMalloc(&dx, x_bytes));
  CHECK_HIP(hipMalloc(&dy16, y16_bytes));
  CHECK_HIP(hipMalloc(&dy32, y32_bytes));
  CHECK_HIP(hipMemcpy(dw, w, w_bytes, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dbits, bits, bit_bytes, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dx, x, x_bytes, hipMemcpyHostToDevice));

  patch_weight* pw = NULL;
  patch_info info;
  CHECK_PATCH(patch_pack((const uint16_t*)dw, n, k, k, (const uint8_t*)dbits, PATCH_BITS_MSB_FIRST, tn, tk, NULL, &pw,
                         &info));
  CHECK_PATCH(patch_gemm(pw, (const uint16_t*)dx, m, k, dy16, n, PATCH_OUT_BF16, NULL));
  CHECK_PATCH(patch_gemm(pw, (const uint16_t*)dx, m, k, dy32, n, PATCH_OUT_F32, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(y16, dy16, y16_bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(y32, dy32, y32_bytes, hipMemcpyDeviceToHost));

  patch_info again;
  CHECK_PATCH(patch_get_info(pw, &again));
  if (again.n_dense != info.n_dense || again.n_sparse != info.n_sparse) {
    fprintf(stderr, "patch_get_info disagrees with patch_pack\n");
    return 4;
  }
  const int64_t tiles = info.tiles_n * info.tiles_k;
  uint8_t* tile_map = malloc((size_t)tiles + 1);
  int32_t* tile_slot = malloc((size_t)tiles * 4 + 4);
  uint16_t* dense_vals = malloc((size_t)info.bytes_dense + 2);
  uint16_t* sparse_vals = malloc((size_t)info.bytes_sparse_vals + 2);
  uint8_t* sparse_meta = malloc((size_t)info.bytes_sparse_meta + 1);
  if (!tile_map || !tile_slot || !dense_vals || !sparse_vals || !sparse_meta) return 1;
  CHECK_PATCH(patch_export(pw, tile_map, tile_slot, dense_vals, sparse_vals, sparse_meta));
  patch_destroy(pw);

  FILE* out = fopen(argv[2], "wb");
  if (!out) return 1;
  const int64_t counts[2] = {info.n_dense, info.n_sparse};
  if (!write_all(out, counts, sizeof counts) || !write_all(out, y16, y16_bytes) || !write_all(out, y32, y32_bytes) ||
      !write_all(out, tile_map, (size_t)tiles) || !write_all(out, tile_slot, (size_t)tiles * 4) ||
      !write_all(out, dense_vals, (size_t)info.bytes_dense) ||
      !write_all(out, sparse_vals, (size_t)info.bytes_sparse_vals) ||
      !write_all(out, sparse_meta, (size_t)info.bytes_sparse_meta))
    return 1;
  fclose(out);
  CHECK_HIP(hipFree(dw));
  CHECK_HIP(hipFree(dbits));
  CHECK_HIP(hipFree(dx));
  CHECK_HIP(hipFree(dy16));
  CHECK_HIP(hipFree(dy32));
  free(w);
  free(bits);
  free(x);
  free(y16);
  free(y32);
  free(tile_map);
  free(tile_slot);
  free(dense_vals);
  free(sparse_vals);
  free(sparse_meta);
  printf("c_abi_gemm ok: %lld dense, %lld 2:4 tiles\n", (long long)counts[0], (long long)counts[1]);
  return 0;
}
