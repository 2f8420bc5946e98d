// C ABI of libpatch.so (declared in include/patch.h): argument checks, the
// packed-weight handle, status codes and stream-ordered kernel launches.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <new>
#include <string>
#include <vector>

#include "layout.h"
using namespace patch_layout;
#include "patch_internal.h"

namespace {

// The calling thread's last error text: a fixed buffer, so that reporting an
// error allocates nothing (patch_pack_noalloc promises no host allocation).
constexpr size_t ERR_BYTES = 512;
thread_local char g_err[ERR_BYTES];

patch_status fail(patch_status st, const char* fmt, ...) {
  char buf[ERR_BYTES];  // formatted apart from g_err: an argument may point into it
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  memcpy(g_err, buf, sizeof(buf));
  return st;
}

patch_status ok() {
  g_err[0] = 0;
  return PATCH_OK;
}

patch_status hip_fail(hipError_t e, const char* what) {
  return fail(PATCH_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The integer a C caller passed for an enum argument.  Any int may arrive, and
// reading a value outside the enumerators as the enum type is undefined in
// C++, so the checks below work on the argument's bits.
template <typename E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

// Device allocation with a test hook: PATCH_TEST_FAIL_ALLOC=<n> makes the n-th
// allocation (1-based) of the calling process fail, to exercise clean-up paths.
hipError_t dev_alloc(void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return hipSuccess;
  static std::atomic<int> counter{0};
  const char* env = getenv("PATCH_TEST_FAIL_ALLOC");
  if (env && *env) {
    const int nth = atoi(env);
    if (nth > 0 && ++counter == nth) {
      counter = 0;
      return hipErrorOutOfMemory;
    }
  }
  return hipMalloc(p, bytes);
}

void dev_free(void* p) {
  if (p) (void)hipFree(p);
}

// gfx950 check, cached per device ordinal.
patch_status check_device(int* dev_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  static std::atomic<int> cache[64];  // 0 unknown, 1 supported, 2 unsupported
  if (dev >= 0 && dev < 64 && cache[dev].load(std::memory_order_relaxed) == 1) {
    *dev_out = dev;
    return PATCH_OK;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  const bool supported = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) cache[dev].store(supported ? 1 : 2, std::memory_order_relaxed);
  if (!supported) return fail(PATCH_E_UNSUPPORTED, "device %d is %s; only gfx950 is supported", dev, prop.gcnArchName);
  *dev_out = dev;
  return PATCH_OK;
}

// Compute units of a device, cached per device ordinal.
hipError_t compute_units(int dev, int* cus) {
  static std::atomic<int> cache[64];
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  const hipError_t e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && dev >= 0 && dev < 64) cache[dev].store(*cus, std::memory_order_relaxed);
  return e;
}

patch_status check_tile(int64_t n, int64_t k, int32_t tn, int32_t tk) {
  if ((tn != 64 && tn != 128) || (tk != 64 && tk != 128))
    return fail(PATCH_E_SHAPE, "tile %dx%d: each side must be 64 or 128", tn, tk);
  if (n < 0 || k < 0) return fail(PATCH_E_SHAPE, "negative shape %lldx%lld", (long long)n, (long long)k);
  if (n % tn || k % tk)
    return fail(PATCH_E_SHAPE, "W %lldx%lld is not a whole number of %dx%d tiles", (long long)n, (long long)k, tn,
                tk);
  // the GEMM kernels address the packed pools with 32-bit byte offsets; the
  // product is tested by division, so that no shape can overflow it
  if (n > 0 && k > PATCH_MAX_WEIGHTS / n)
    return fail(PATCH_E_SHAPE, "W %lldx%lld has more than 2^31 - 1 weights", (long long)n, (long long)k);
  return PATCH_OK;
}

void fill_info(const patch_weight* w, patch_info* info) {
  info->n = w->n;
  info->k = w->k;
  info->tile_n = w->tn;
  info->tile_k = w->tk;
  info->tiles_n = w->tiles_n;
  info->tiles_k = w->tiles_k;
  info->n_dense = w->n_dense;
  info->n_sparse = w->n_sparse;
  info->bytes_dense = w->n_dense * w->tn * w->tk * 2;
  info->bytes_sparse_vals = w->n_sparse * w->tn * w->tk;
  info->bytes_sparse_meta = w->n_sparse * w->tn * w->tk / 8;
  info->sparsity = w->tiles ? 0.5 * (double)w->n_sparse / (double)w->tiles : 0.0;
  info->bad_tile = info->bad_row = info->bad_group = -1;
}

void free_weight(patch_weight* w) {
  if (!w || w->borrowed) return;
  delete[] w->row_dense_prefix;
  dev_free(w->tile_map);
  dev_free(w->tile_desc);
  dev_free(w->dense_vals);
  dev_free(w->sparse_vals);
  dev_free(w->sparse_meta);
  delete w;
}

}  // namespace

bool set_cost_prefix(patch_weight* w, const uint8_t* tile_map_host) {
  int64_t* p = new (std::nothrow) int64_t[w->tiles_n + 1];
  if (!p) return false;
  p[0] = 0;
  for (int64_t i = 0; i < w->tiles_n; ++i) {
    int64_t d = 0;
    for (int64_t j = 0; j < w->tiles_k; ++j) d += tile_map_host[i * w->tiles_k + j] == PATCH_TILE_DENSE;
    p[i + 1] = p[i] + d;
  }
  delete[] w->row_dense_prefix;
  w->row_dense_prefix = p;
  return true;
}

double row_cost(const patch_weight* w, int64_t r0, int64_t r1) {
  if (r1 > w->tiles_n) r1 = w->tiles_n;
  if (r0 >= r1 || w->tiles_k == 0) return PATCH_STEP_COST_DENSE;
  if (!w->row_dense_prefix) {  // no per-row counts: the weight's mean mix
    const double t = (double)(w->n_dense + w->n_sparse);
    return t > 0 ? (w->n_dense * PATCH_STEP_COST_DENSE + w->n_sparse * PATCH_STEP_COST_24) / t : PATCH_STEP_COST_DENSE;
  }
  const double tiles = (double)(r1 - r0) * (double)w->tiles_k;
  const double dense = (double)(w->row_dense_prefix[r1] - w->row_dense_prefix[r0]);
  return (dense * PATCH_STEP_COST_DENSE + (tiles - dense) * PATCH_STEP_COST_24) / tiles;
}

extern "C" {

const char* patch_last_error(void) { return g_err; }

patch_status patch_pack(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, const uint8_t* mask_bits,
                        patch_bit_order order, int32_t tile_n, int32_t tile_k, void* stream, patch_weight** out,
                        patch_info* info) {
  if (!out) return fail(PATCH_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const int ord = enum_value(order);
  if (ord != PATCH_BITS_MSB_FIRST && ord != PATCH_BITS_LSB_FIRST)
    return fail(PATCH_E_INVALID_ARG, "bad bit order %d", ord);
  patch_status st = check_tile(n, k, tile_n, tile_k);
  if (st != PATCH_OK) return st;
  const int64_t tiles = (n / tile_n) * (k / tile_k);
  if (tiles > 0) {
    if (!w || !mask_bits) return fail(PATCH_E_INVALID_ARG, "w or mask_bits is NULL");
    if (!aligned16(w) || !aligned16(mask_bits))
      return fail(PATCH_E_INVALID_ARG, "w and mask_bits must be 16-byte aligned");
    if (ldw < k || ldw % 8) return fail(PATCH_E_INVALID_ARG, "ldw %lld must be >= k and a multiple of 8", (long long)ldw);
  }
  int dev = 0;
  st = check_device(&dev);
  if (st != PATCH_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  patch_weight* pw = new (std::nothrow) patch_weight();
  if (!pw) return fail(PATCH_E_NOMEM, "host allocation failed");
  pw->device = dev;
  pw->n = n;
  pw->k = k;
  pw->tn = tile_n;
  pw->tk = tile_k;
  pw->tiles_n = n / tile_n;
  pw->tiles_k = k / tile_k;
  pw->tiles = tiles;

  if (tiles == 0) {
    if (!set_cost_prefix(pw, nullptr)) {
      free_weight(pw);
      return fail(PATCH_E_NOMEM, "host allocation failed");
    }
    if (info) fill_info(pw, info);
    *out = pw;
    return ok();
  }

  // Scratch for validation: [0] first bad location, [1] dense count, [2] sparse count.
  unsigned long long* scratch = nullptr;
  hipError_t e;
#define PATCH_TRY_ALLOC(ptr, bytes)                                                              \
  do {                                                                                           \
    e = dev_alloc(reinterpret_cast<void**>(&(ptr)), (bytes));                                    \
    if (e != hipSuccess) {                                                                       \
      dev_free(scratch);                                                                         \
      free_weight(pw);                                                                           \
      return fail(PATCH_E_NOMEM, "device allocation of %lld bytes failed: %s", (long long)(bytes), \
                  hipGetErrorString(e));                                                         \
    }                                                                                            \
  } while (0)
#define PATCH_TRY_HIP(expr, what)     \
  do {                                \
    e = (expr);                       \
    if (e != hipSuccess) {            \
      dev_free(scratch);              \
      free_weight(pw);                \
      return hip_fail(e, what);       \
    }                                 \
  } while (0)

  PATCH_TRY_ALLOC(scratch, 3 * sizeof(unsigned long long));
  PATCH_TRY_ALLOC(pw->tile_map, (size_t)tiles);
  PATCH_TRY_ALLOC(pw->tile_desc, (size_t)tiles * sizeof(int32_t));

  PATCH_TRY_HIP(launch_fill_u64(scratch, 1, PATCH_NO_ERROR_LOC, s), "fill");
  PATCH_TRY_HIP(launch_classify(mask_bits, k, ord, tile_n, tile_k, pw->tiles_n, pw->tiles_k, pw->tile_map,
                                scratch, s),
                "classify launch");
  PATCH_TRY_HIP(launch_slot_scan(pw->tile_map, tiles, pw->tile_desc, reinterpret_cast<long long*>(scratch + 1), s),
                "slot scan launch");
  unsigned long long host[3] = {0, 0, 0};
  std::vector<uint8_t> map_host;
  try {
    map_host.resize((size_t)tiles);
  } catch (const std::bad_alloc&) {
    dev_free(scratch);
    free_weight(pw);
    return fail(PATCH_E_NOMEM, "host allocation failed");
  }
  PATCH_TRY_HIP(hipMemcpyAsync(host, scratch, sizeof(host), hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
  PATCH_TRY_HIP(hipMemcpyAsync(map_host.data(), pw->tile_map, (size_t)tiles, hipMemcpyDeviceToHost, s),
                "hipMemcpyAsync");
  PATCH_TRY_HIP(hipStreamSynchronize(s), "hipStreamSynchronize");

  if (host[0] != PATCH_NO_ERROR_LOC) {
    const int64_t per_tile = (int64_t)tile_n * tile_k / 4;
    const int64_t loc = (int64_t)host[0];
    const int64_t bt = loc / per_tile, rem = loc % per_tile;
    const int64_t br = rem / (tile_k / 4), bg = rem % (tile_k / 4);
    if (info) {
      fill_info(pw, info);
      info->n_dense = info->n_sparse = 0;
      info->bad_tile = bt;
      info->bad_row = br;
      info->bad_group = bg;
    }
    dev_free(scratch);
    free_weight(pw);
    return fail(PATCH_E_MASK,
                "mask is not tile-wise dense / 2:4: tile %lld (tile row %lld, tile col %lld), row %lld in tile, "
                "group %lld along K",
                (long long)bt, (long long)(bt / (k / tile_k)), (long long)(bt % (k / tile_k)), (long long)br,
                (long long)bg);
  }
  pw->n_dense = (int64_t)host[1];
  pw->n_sparse = (int64_t)host[2];
  if (!set_cost_prefix(pw, map_host.data())) {
    dev_free(scratch);
    free_weight(pw);
    return fail(PATCH_E_NOMEM, "host allocation failed");
  }

  PATCH_TRY_ALLOC(pw->dense_vals, (size_t)pw->n_dense * tile_n * tile_k * 2);
  PATCH_TRY_ALLOC(pw->sparse_vals, (size_t)pw->n_sparse * tile_n * tile_k);
  // +16 B: the streaming kernel reads 16 bytes at each lane's 8-byte code slot
  PATCH_TRY_ALLOC(pw->sparse_meta, (size_t)pw->n_sparse * tile_n * tile_k / 8 + 16);
  PATCH_TRY_HIP(launch_compress(w, ldw, mask_bits, k, ord, tile_n, tile_k, pw->tiles_n, pw->tiles_k,
                                pw->tile_desc, pw->dense_vals, pw->sparse_vals, pw->sparse_meta, s),
                "compress launch");
  // W and the mask belong to the caller and may be released as soon as we return.
  PATCH_TRY_HIP(hipStreamSynchronize(s), "hipStreamSynchronize");
  dev_free(scratch);
#undef PATCH_TRY_ALLOC
#undef PATCH_TRY_HIP
  if (info) fill_info(pw, info);
  *out = pw;
  return ok();
}

// Whether the streaming kernel should run a product of m rows on w.  Decode
// (m <= 16) always streams.  Up to PATCH_STREAM_MAX_M rows both kernels can,
// and their estimated times (us) decide.  Both launches are bound by latency
// here, so the estimates count serial steps, with the plain HBM read of the
// packed W (5.5 TB/s, plus the launch) as a floor.  Streaming: 5.7, plus the X
// copies (every workgroup copies all of X, rounded up to its 16-row X blocks)
// at 50 TB/s, plus 0.54 per chunk a wave waits for in turn (one in flight), plus
// 0.085 per 16 x 16 x 64 block of products a wave issues.  Tiled: these m give
// it one or two 64-row blocks per 128 W rows, so 5.4 plus 0.285 per 64-wide K
// step, per round of 256 workgroups.  Fitted on MI355X to timings with the
// weights read from HBM (90% 2:4 tiles, ten products from 2048 x 8192 to
// 14336 x 4096, m = 17 .. 128): the choice was the faster kernel in all 52
// cases.
static bool stream_wins(const patch_weight* w, int64_t m) {
  if (m <= 16) return true;
  const int xb = stream_x_blocks(m);
  if (xb == 0) return false;
  const int nblk = stream_w_blocks(w->n), waves = stream_waves(m, w->n);  // one chunk in flight per wave
  const double tile = (double)w->tn * (double)w->tk;
  const double w_floor = tile * (2.0 * (double)w->n_dense + 1.125 * (double)w->n_sparse) / 5.5e6;
  const double chunks = (double)(w->k / 64);
  const double x_bytes = (double)(w->n / (16 * nblk)) * (16.0 * xb) * (double)w->k * 2.0;
  const double per_wave = std::ceil(chunks / waves);
  const double t_stream = std::max(5.7 + x_bytes / 50e6 + 0.54 * per_wave + 0.085 * per_wave * xb * nblk, 3.0 + w_floor);
  const double wgs = (double)(w->n / 128) * (double)((m + 63) / 64);
  const double rounds = wgs > 256 ? (double)(int64_t)((wgs + 255) / 256) : 1.0;
  const double t_tiled = std::max(5.4 + 0.285 * chunks * rounds, 4.0 + w_floor);
  return t_stream < t_tiled;
}

// Checks one product's arguments; sets *skip when it has nothing to compute
// (m = 0 or n = 0).
static patch_status check_product(const patch_weight* w, const uint16_t* x, int64_t m, int64_t ldx, void* y,
                                  int64_t ldy, bool* skip) {
  *skip = false;
  if (!w) return fail(PATCH_E_INVALID_ARG, "weight handle is NULL");
  if (m < 0) return fail(PATCH_E_INVALID_ARG, "m = %lld < 0", (long long)m);
  if (m == 0 || w->n == 0) {
    *skip = true;
    return ok();
  }
  if (!y) return fail(PATCH_E_INVALID_ARG, "y is NULL");
  if (!aligned16(y)) return fail(PATCH_E_INVALID_ARG, "y must be 16-byte aligned");
  if (ldy < w->n || ldy % 8) return fail(PATCH_E_INVALID_ARG, "ldy %lld must be >= n and a multiple of 8", (long long)ldy);
  if (w->k > 0) {  // with K = 0, X is never read and Y is all zeros
    if (!x) return fail(PATCH_E_INVALID_ARG, "x is NULL");
    if (!aligned16(x)) return fail(PATCH_E_INVALID_ARG, "x must be 16-byte aligned");
    if (ldx < w->k || ldx % 8) return fail(PATCH_E_INVALID_ARG, "ldx %lld must be >= k and a multiple of 8", (long long)ldx);
    // the tiled kernel addresses a block's X rows with 32-bit byte offsets
    if (ldx > PATCH_MAX_LDX)
      return fail(PATCH_E_INVALID_ARG, "ldx %lld exceeds %lld", (long long)ldx, (long long)PATCH_MAX_LDX);
  }
  return ok();
}

// Runs up to PATCH_MAX_GROUP products: those with K = 0 get a zero fill, the
// rest one launch of the streaming kernel (m <= 16) and/or one of the tiled
// kernel.  kernel / variant as in patch_gemm_kernel.
// Bytes of fp32 partials a split of the product of m rows on w needs (0: no split).
static int64_t split_bytes(const patch_weight* w, int64_t m) {
  if (m < 1 || m > PATCH_STREAM_MAX_M || w->k == 0 || w->n == 0 || !stream_wins(w, m)) return 0;
  const int split = stream_k_split(m, w->n, w->k);
  return split > 1 ? (int64_t)split * m * w->n * 4 : 0;
}

// `workspace` (one product only, AUTO): when it holds split_bytes, a streamed
// product splits its K (launch_stream_split).
static patch_status gemm_group_common(const patch_gemm_item* items, int32_t count, int y_dtype, int kernel,
                                      int32_t variant, void* stream, void* workspace = nullptr,
                                      int64_t workspace_bytes = 0) {
  if (count < 0 || count > PATCH_MAX_GROUP)
    return fail(PATCH_E_INVALID_ARG, "group of %d products, must be 0..%d", (int)count, PATCH_MAX_GROUP);
  if (count > 0 && !items) return fail(PATCH_E_INVALID_ARG, "items is NULL");
  if (y_dtype != PATCH_OUT_BF16 && y_dtype != PATCH_OUT_F32)
    return fail(PATCH_E_INVALID_ARG, "bad output dtype %d", y_dtype);
  if (kernel != PATCH_KERNEL_AUTO && kernel != PATCH_KERNEL_TILED && kernel != PATCH_KERNEL_STREAM)
    return fail(PATCH_E_INVALID_ARG, "bad kernel %d", kernel);
  if (kernel == PATCH_KERNEL_TILED && variant > 0 && variant != 256 && variant != 192 && variant != 128 && variant != 64)
    return fail(PATCH_E_INVALID_ARG, "tiled block rows must be 256, 192, 128 or 64, got %d", (int)variant);
  if (count == 0) return ok();
  bool skip[PATCH_MAX_GROUP];
  for (int i = 0; i < count; ++i) {
    const patch_gemm_item& it = items[i];
    const patch_status st = check_product(it.w, it.x, it.m, it.ldx, it.y, it.ldy, &skip[i]);
    if (st != PATCH_OK) {
      if (count == 1) return st;
      return fail(st, "product %d: %s", i, g_err);  // fail() formats before it rewrites g_err
    }
    if (kernel == PATCH_KERNEL_STREAM && it.m > PATCH_STREAM_MAX_M) {
      if (count == 1)
        return fail(PATCH_E_INVALID_ARG, "the streaming kernel takes m <= %d, got %lld", PATCH_STREAM_MAX_M,
                    (long long)it.m);
      return fail(PATCH_E_INVALID_ARG, "product %d: the streaming kernel takes m <= %d, got %lld", i,
                  PATCH_STREAM_MAX_M, (long long)it.m);
    }
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  for (int i = 0; i < count; ++i)
    if (!skip[i] && items[i].w->device != dev)
      return fail(PATCH_E_INVALID_ARG, "product %d: weight lives on device %d, current device is %d", i,
                  items[i].w->device, dev);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int f32 = y_dtype == PATCH_OUT_F32;
  gemm_group streamed = {}, tiled = {};
  for (int i = 0; i < count; ++i) {
    if (skip[i]) continue;
    const patch_gemm_item& it = items[i];
    if (it.w->k == 0) {
      e = launch_fill_zero_y(it.y, it.m, it.w->n, it.ldy, f32, s);
      if (e != hipSuccess) return hip_fail(e, "zero-fill launch");
      continue;
    }
    const bool st = kernel == PATCH_KERNEL_STREAM || (kernel == PATCH_KERNEL_AUTO && stream_wins(it.w, it.m));
    const int64_t need = workspace && kernel == PATCH_KERNEL_AUTO ? split_bytes(it.w, it.m) : 0;
    if (st && need > 0 && workspace_bytes >= need) {
      gemm_problem p = make_problem(it.w, it.x, it.m, it.ldx, it.y, it.ldy);
      p.ksplit = stream_k_split(it.m, it.w->n, it.w->k);
      p.part = static_cast<float*>(workspace);
      e = launch_stream_split(p, f32, s);
      if (e != hipSuccess) return hip_fail(e, "gemm launch (streaming kernel, split K)");
      continue;
    }
    gemm_group& g = st ? streamed : tiled;
    g.p[g.count++] = make_problem(it.w, it.x, it.m, it.ldx, it.y, it.ldy);
  }
  if (streamed.count) {
    e = launch_stream_group(streamed, f32, s);
    if (e != hipSuccess) return hip_fail(e, "gemm launch (streaming kernel)");
  }
  if (tiled.count > 1 && kernel == PATCH_KERNEL_AUTO) {
    // A product with at least one 256 x 256 block per CU fills the GPU on its
    // own: it gets a launch of its own, with its own block height and tail
    // plan, as a solo patch_gemm would.  Only the under-filled products share a
    // launch, which is where sharing gains (measured on the 32-layer LLaMA-2-7B
    // prefill stack: sharing launches between its full-size products was 4%
    // slower than launching them one by one).
    int cus = 0;
    e = compute_units(dev, &cus);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    gemm_group small = {};
    for (int i = 0; i < tiled.count; ++i) {
      const gemm_problem& p = tiled.p[i];
      if (((p.n + 255) / 256) * ((p.m + 255) / 256) >= cus) {
        gemm_group one = {};
        one.p[one.count++] = p;
        e = launch_tiled_group(one, f32, 0, s);
        if (e != hipSuccess) return hip_fail(e, "gemm launch (tiled kernel)");
      } else {
        small.p[small.count++] = p;
      }
    }
    tiled = small;
  }
  if (tiled.count) {
    e = launch_tiled_group(tiled, f32, kernel == PATCH_KERNEL_AUTO ? 0 : variant, s);
    if (e != hipSuccess) return hip_fail(e, "gemm launch (tiled kernel)");
  }
  return ok();
}

patch_status patch_gemm(const patch_weight* w, const uint16_t* x, int64_t m, int64_t ldx, void* y, int64_t ldy,
                        patch_out_dtype y_dtype, void* stream) {
  const patch_gemm_item it = {w, x, m, ldx, y, ldy};
  return gemm_group_common(&it, 1, enum_value(y_dtype), PATCH_KERNEL_AUTO, 0, stream);
}

patch_status patch_gemm_kernel(const patch_weight* w, const uint16_t* x, int64_t m, int64_t ldx, void* y,
                               int64_t ldy, patch_out_dtype y_dtype, patch_kernel kernel, int32_t variant,
                               void* stream) {
  const patch_gemm_item it = {w, x, m, ldx, y, ldy};
  return gemm_group_common(&it, 1, enum_value(y_dtype), enum_value(kernel), variant, stream);
}

patch_status patch_gemm_with_workspace(const patch_weight* w, const uint16_t* x, int64_t m, int64_t ldx, void* y,
                                       int64_t ldy, patch_out_dtype y_dtype, void* workspace, int64_t workspace_bytes,
                                       void* stream) {
  if (workspace && !aligned16(workspace)) return fail(PATCH_E_INVALID_ARG, "workspace must be 16-byte aligned");
  if (workspace_bytes < 0) return fail(PATCH_E_INVALID_ARG, "workspace_bytes %lld < 0", (long long)workspace_bytes);
  const patch_gemm_item it = {w, x, m, ldx, y, ldy};
  return gemm_group_common(&it, 1, enum_value(y_dtype), PATCH_KERNEL_AUTO, 0, stream, workspace, workspace_bytes);
}

patch_status patch_gemm_workspace_size(const patch_weight* w, int64_t m, int64_t* bytes) {
  if (!w) return fail(PATCH_E_INVALID_ARG, "weight handle is NULL");
  if (!bytes) return fail(PATCH_E_INVALID_ARG, "bytes is NULL");
  if (m < 0) return fail(PATCH_E_INVALID_ARG, "m = %lld < 0", (long long)m);
  *bytes = split_bytes(w, m);
  return ok();
}

patch_status patch_gemm_grouped(const patch_gemm_item* items, int32_t count, patch_out_dtype y_dtype,
                                void* stream) {
  return gemm_group_common(items, count, enum_value(y_dtype), PATCH_KERNEL_AUTO, 0, stream);
}

patch_status patch_gemm_grouped_kernel(const patch_gemm_item* items, int32_t count, patch_out_dtype y_dtype,
                                       patch_kernel kernel, int32_t variant, void* stream) {
  return gemm_group_common(items, count, enum_value(y_dtype), enum_value(kernel), variant, stream);
}

patch_status patch_unpack(const patch_weight* w, uint16_t* w_out, int64_t ldw, void* stream) {
  if (!w) return fail(PATCH_E_INVALID_ARG, "weight handle is NULL");
  if (w->tiles == 0) return ok();
  if (!w_out) return fail(PATCH_E_INVALID_ARG, "w_out is NULL");
  if (!aligned16(w_out)) return fail(PATCH_E_INVALID_ARG, "w_out must be 16-byte aligned");
  if (ldw < w->k || ldw % 8) return fail(PATCH_E_INVALID_ARG, "ldw %lld must be >= k and a multiple of 8", (long long)ldw);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != w->device) return fail(PATCH_E_INVALID_ARG, "weight lives on device %d, current device is %d", w->device, dev);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  e = launch_decompress(w, w_out, ldw, s);
  if (e != hipSuccess) return hip_fail(e, "unpack launch");
  return ok();
}

patch_status patch_mask_unpack(const uint8_t* bits, int64_t count, patch_bit_order order, uint8_t* out,
                               void* stream) {
  const int ord = enum_value(order);
  if (ord != PATCH_BITS_MSB_FIRST && ord != PATCH_BITS_LSB_FIRST)
    return fail(PATCH_E_INVALID_ARG, "bad bit order %d", ord);
  if (count < 0) return fail(PATCH_E_INVALID_ARG, "count < 0");
  if (count == 0) return ok();
  if (!bits || !out) return fail(PATCH_E_INVALID_ARG, "bits or out is NULL");
  int dev = 0;
  patch_status st = check_device(&dev);
  if (st != PATCH_OK) return st;
  hipError_t e = launch_mask_unpack(bits, count, ord, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mask unpack launch");
  return ok();
}

patch_status patch_get_info(const patch_weight* w, patch_info* info) {
  if (!w || !info) return fail(PATCH_E_INVALID_ARG, "NULL argument");
  fill_info(w, info);
  return ok();
}

static patch_status export_impl(const patch_weight* w, uint8_t* tile_map, int32_t* tile_slot, uint16_t* dense_vals,
                                uint16_t* sparse_vals, uint8_t* sparse_meta);

patch_status patch_export(const patch_weight* w, uint8_t* tile_map, int32_t* tile_slot, uint16_t* dense_vals,
                          uint16_t* sparse_vals, uint8_t* sparse_meta) {
  try {
    return export_impl(w, tile_map, tile_slot, dense_vals, sparse_vals, sparse_meta);
  } catch (const std::bad_alloc&) {
    return fail(PATCH_E_NOMEM, "host staging allocation failed");
  }
}

static patch_status export_impl(const patch_weight* w, uint8_t* tile_map, int32_t* tile_slot, uint16_t* dense_vals,
                                uint16_t* sparse_vals, uint8_t* sparse_meta) {
  if (!w) return fail(PATCH_E_INVALID_ARG, "weight handle is NULL");
  if (w->tiles == 0) return ok();
  // The pools never change once patch_pack / patch_import have returned (both
  // block until they are complete), so no stream needs waiting for here.
  hipError_t e = hipSuccess;
  if (tile_map) {
    e = hipMemcpy(tile_map, w->tile_map, (size_t)w->tiles, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy tile_map");
  }
  if (tile_slot) {
    e = hipMemcpy(tile_slot, w->tile_desc, (size_t)w->tiles * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy tile_desc");
    for (int64_t t = 0; t < w->tiles; ++t) tile_slot[t] >>= 1;  // desc = (slot << 1) | type
  }
  const int64_t tn = w->tn, tk = w->tk;
  const size_t dv = (size_t)w->n_dense * tn * tk * 2, sv = (size_t)w->n_sparse * tn * tk,
               sm = (size_t)w->n_sparse * tn * tk / 8;
  // The device pools are in operand order (layout.h); convert to the row-major
  // format of the header.
  if (dense_vals && dv) {
    std::vector<uint16_t> tmp(dv / 2);
    e = hipMemcpy(tmp.data(), w->dense_vals, dv, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy dense_vals");
    dense_to_row_major(tmp.data(), dense_vals, w->n_dense, tn, tk);
  }
  if (sparse_vals && sv) {
    std::vector<uint16_t> tmp(sv / 2);
    e = hipMemcpy(tmp.data(), w->sparse_vals, sv, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy sparse_vals");
    sparse_values_to_row_major(tmp.data(), sparse_vals, w->n_sparse, tn, tk);
  }
  if (sparse_meta && sm) {
    std::vector<uint8_t> tmp(sm);
    e = hipMemcpy(tmp.data(), w->sparse_meta, sm, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy sparse_meta");
    sparse_codes_to_row_major(tmp.data(), sparse_meta, w->n_sparse, tn, tk);
  }
  return ok();
}

patch_status patch_sample_mask(const float* tile_logits, const float* tile_noise, const float* group_logits,
                               const float* group_noise, int64_t n, int64_t k, int32_t tile_n, int32_t tile_k,
                               float kappa, patch_bit_order order, uint8_t* mask_bits, void* stream) {
  const int ord = enum_value(order);
  if (ord != PATCH_BITS_MSB_FIRST && ord != PATCH_BITS_LSB_FIRST)
    return fail(PATCH_E_INVALID_ARG, "bad bit order %d", ord);
  patch_status st = check_tile(n, k, tile_n, tile_k);
  if (st != PATCH_OK) return st;
  if (n * k == 0) return ok();
  if (!tile_logits || !group_logits || !mask_bits)
    return fail(PATCH_E_INVALID_ARG, "tile_logits, group_logits and mask_bits must not be NULL");
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; };
  if (misaligned(tile_logits) || misaligned(group_logits) || misaligned(tile_noise) || misaligned(group_noise))
    return fail(PATCH_E_INVALID_ARG, "logits and noise must be 4-byte aligned");
  int dev = 0;
  st = check_device(&dev);
  if (st != PATCH_OK) return st;
  const hipError_t e = launch_sample_mask(tile_logits, tile_noise, group_logits, group_noise, n, k, tile_n, tile_k,
                                          kappa, ord == PATCH_BITS_LSB_FIRST, mask_bits,
                                          reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sample launch");
  return ok();
}

patch_status patch_import(int64_t n, int64_t k, int32_t tile_n, int32_t tile_k, const uint8_t* tile_map,
                          const uint16_t* dense_vals, const uint16_t* sparse_vals, const uint8_t* sparse_meta,
                          void* stream, patch_weight** out, patch_info* info) {
  if (!out) return fail(PATCH_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  patch_status st = check_tile(n, k, tile_n, tile_k);
  if (st != PATCH_OK) return st;
  const int64_t tiles_n = n / tile_n, tiles_k = k / tile_k, tiles = tiles_n * tiles_k;
  const int64_t tn = tile_n, tk = tile_k;
  if (tiles > 0 && !tile_map) return fail(PATCH_E_INVALID_ARG, "tile_map is NULL");
  // Host-side validation of the exported format, before any device work.
  int64_t nd = 0, ns = 0;
  for (int64_t t = 0; t < tiles; ++t) {
    if (tile_map[t] == PATCH_TILE_DENSE) ++nd;
    else if (tile_map[t] == PATCH_TILE_SPARSE24) ++ns;
    else return fail(PATCH_E_INVALID_ARG, "tile_map[%lld] = %d is neither dense (0) nor 2:4 (1)", (long long)t,
                     (int)tile_map[t]);
  }
  if (nd > 0 && !dense_vals) return fail(PATCH_E_INVALID_ARG, "dense_vals is NULL but %lld tiles are dense", (long long)nd);
  if (ns > 0 && (!sparse_vals || !sparse_meta))
    return fail(PATCH_E_INVALID_ARG, "sparse_vals or sparse_meta is NULL but %lld tiles are 2:4", (long long)ns);
  {
    // every code must name two distinct kept positions i0 < i1
    static const bool legal[16] = {false, false, false, false, true,  false, false, false,
                                   true,  true,  false, false, true,  true,  true,  false};
    int64_t slot = 0;
    for (int64_t t = 0; t < tiles; ++t) {
      if (tile_map[t] != PATCH_TILE_SPARSE24) continue;
      const uint8_t* m = sparse_meta + slot * tn * tk / 8;
      for (int64_t row = 0; row < tn; ++row)
        for (int64_t g = 0; g < tk / 4; ++g) {
          const int code = (m[row * (tk / 8) + g / 2] >> (4 * (g & 1))) & 15;
          if (!legal[code]) {
            if (info) {
              memset(info, 0, sizeof(*info));
              info->n = n;
              info->k = k;
              info->tile_n = tile_n;
              info->tile_k = tile_k;
              info->tiles_n = tiles_n;
              info->tiles_k = tiles_k;
              info->bad_tile = t;
              info->bad_row = row;
              info->bad_group = g;
            }
            return fail(PATCH_E_MASK, "2:4 code %d of tile %lld, row %lld, group %lld is not i0 | i1 << 2 with i0 < i1",
                        code, (long long)t, (long long)row, (long long)g);
          }
        }
      ++slot;
    }
  }
  int dev = 0;
  st = check_device(&dev);
  if (st != PATCH_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  patch_weight* pw = new (std::nothrow) patch_weight();
  if (!pw) return fail(PATCH_E_NOMEM, "host allocation failed");
  pw->device = dev;
  pw->n = n;
  pw->k = k;
  pw->tn = tile_n;
  pw->tk = tile_k;
  pw->tiles_n = tiles_n;
  pw->tiles_k = tiles_k;
  pw->tiles = tiles;
  pw->n_dense = nd;
  pw->n_sparse = ns;
  if (!set_cost_prefix(pw, tile_map)) {
    free_weight(pw);
    return fail(PATCH_E_NOMEM, "host allocation failed");
  }
  if (tiles == 0) {
    if (info) fill_info(pw, info);
    *out = pw;
    return ok();
  }
  hipError_t e;
#define PATCH_TRY(expr, what, status)                                    \
  do {                                                                   \
    e = (expr);                                                          \
    if (e != hipSuccess) {                                               \
      free_weight(pw);                                                   \
      return status == PATCH_E_NOMEM                                     \
                 ? fail(PATCH_E_NOMEM, "%s: %s", what, hipGetErrorString(e)) \
                 : hip_fail(e, what);                                    \
    }                                                                    \
  } while (0)
  const size_t dv = (size_t)nd * tn * tk * 2, sv = (size_t)ns * tn * tk, sm = (size_t)ns * tn * tk / 8;
  PATCH_TRY(dev_alloc(reinterpret_cast<void**>(&pw->tile_map), (size_t)tiles), "device allocation", PATCH_E_NOMEM);
  PATCH_TRY(dev_alloc(reinterpret_cast<void**>(&pw->tile_desc), (size_t)tiles * 4), "device allocation", PATCH_E_NOMEM);
  PATCH_TRY(dev_alloc(reinterpret_cast<void**>(&pw->dense_vals), dv), "device allocation", PATCH_E_NOMEM);
  PATCH_TRY(dev_alloc(reinterpret_cast<void**>(&pw->sparse_vals), sv), "device allocation", PATCH_E_NOMEM);
  // +16 B: the streaming kernel reads 16 bytes at each lane's 8-byte code slot
  PATCH_TRY(dev_alloc(reinterpret_cast<void**>(&pw->sparse_meta), sm + 16), "device allocation", PATCH_E_NOMEM);

  // Descriptors (slot << 1 | type) and the pools in operand order: the inverse
  // of the conversion in patch_export.
  std::vector<int32_t> desc;
  std::vector<uint16_t> dtmp, stmp;
  std::vector<uint8_t> mtmp;
  try {
    desc.resize(tiles);
    dtmp.resize(dv / 2);
    stmp.resize(sv / 2);
    mtmp.assign(sm + 16, 0);
  } catch (const std::bad_alloc&) {
    free_weight(pw);
    return fail(PATCH_E_NOMEM, "host staging allocation failed");
  }
  {
    int64_t cd = 0, cs = 0;
    for (int64_t t = 0; t < tiles; ++t)
      desc[t] = tile_map[t] == PATCH_TILE_DENSE ? (int32_t)((cd++) << 1) : (int32_t)(((cs++) << 1) | 1);
  }
  dense_from_row_major(dense_vals, dtmp.data(), nd, tn, tk);
  sparse_values_from_row_major(sparse_vals, stmp.data(), ns, tn, tk);
  sparse_codes_from_row_major(sparse_meta, mtmp.data(), ns, tn, tk);
  PATCH_TRY(hipMemcpyAsync(pw->tile_map, tile_map, (size_t)tiles, hipMemcpyHostToDevice, s), "copy tile_map", 0);
  PATCH_TRY(hipMemcpyAsync(pw->tile_desc, desc.data(), (size_t)tiles * 4, hipMemcpyHostToDevice, s), "copy descriptors", 0);
  if (dv) PATCH_TRY(hipMemcpyAsync(pw->dense_vals, dtmp.data(), dv, hipMemcpyHostToDevice, s), "copy dense_vals", 0);
  if (sv) PATCH_TRY(hipMemcpyAsync(pw->sparse_vals, stmp.data(), sv, hipMemcpyHostToDevice, s), "copy sparse_vals", 0);
  if (sm) PATCH_TRY(hipMemcpyAsync(pw->sparse_meta, mtmp.data(), sm + 16, hipMemcpyHostToDevice, s), "copy sparse_meta", 0);
  // the host staging buffers die on return
  PATCH_TRY(hipStreamSynchronize(s), "hipStreamSynchronize", 0);
#undef PATCH_TRY
  if (info) fill_info(pw, info);
  *out = pw;
  return ok();
}

void patch_destroy(patch_weight* w) { free_weight(w); }

}  // extern "C"

// ---- allocation-free packing ------------------------------------------------
// Validation scratch of patch_pack_noalloc: [0] first invalid group, [1] dense
// tiles, [2] 2:4 tiles.  One copy per GPU, held until the process ends; every
// call on a GPU reuses it (so calls that overlap on one GPU race).  In host code
// the array's name is only a stand-in: kernels get the per-device address
// hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned long long scratch[PATCH_PACK_SCRATCH_WORDS];

namespace {

// Device address of `scratch` on device dev, looked up once per device (with
// that device current, as here: every entry point runs on the current device).
hipError_t scratch_address(int dev, unsigned long long** out) {
  static std::atomic<unsigned long long*> addr[64] = {};
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  unsigned long long* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    p = static_cast<unsigned long long*>(q);
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

patch_status patch_pack_noalloc(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, const uint8_t* mask_bits,
                                patch_bit_order order, int32_t tile_n, int32_t tile_k, void* stream,
                                uint8_t* tile_map, int32_t* tile_desc, uint16_t* dense_vals, int64_t dense_bytes,
                                uint16_t* sparse_vals, int64_t sparse_bytes, uint8_t* sparse_meta,
                                int64_t meta_bytes, patch_weight_storage* storage, patch_weight** out,
                                patch_info* info) {
  static_assert(sizeof(patch_weight) <= sizeof(patch_weight_storage), "handle fits the caller's storage");
  static_assert(alignof(patch_weight) <= alignof(patch_weight_storage), "handle alignment");
  if (!out) return fail(PATCH_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!storage) return fail(PATCH_E_INVALID_ARG, "storage is NULL");
  const int ord = enum_value(order);
  if (ord != PATCH_BITS_MSB_FIRST && ord != PATCH_BITS_LSB_FIRST)
    return fail(PATCH_E_INVALID_ARG, "bad bit order %d", ord);
  patch_status st = check_tile(n, k, tile_n, tile_k);
  if (st != PATCH_OK) return st;
  const int64_t tiles = (n / tile_n) * (k / tile_k);
  if (tiles > 0) {
    if (!w || !mask_bits || !tile_map || !tile_desc) return fail(PATCH_E_INVALID_ARG, "NULL pointer");
    if (!aligned16(w) || !aligned16(mask_bits) || !aligned16(tile_desc))
      return fail(PATCH_E_INVALID_ARG, "w, mask_bits and tile_desc must be 16-byte aligned");
    if (ldw < k || ldw % 8) return fail(PATCH_E_INVALID_ARG, "ldw %lld must be >= k and a multiple of 8", (long long)ldw);
    if (dense_bytes < 0 || sparse_bytes < 0 || meta_bytes < 0) return fail(PATCH_E_INVALID_ARG, "negative pool size");
    if ((dense_bytes && (!dense_vals || !aligned16(dense_vals))) ||
        (sparse_bytes && (!sparse_vals || !aligned16(sparse_vals))) ||
        (meta_bytes && (!sparse_meta || !aligned16(sparse_meta))))
      return fail(PATCH_E_INVALID_ARG, "pools must be 16-byte aligned and non-NULL when their size is not 0");
  }
  int dev = 0;
  st = check_device(&dev);
  if (st != PATCH_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  patch_weight* pw = new (storage) patch_weight();
  pw->borrowed = true;
  pw->device = dev;
  pw->n = n;
  pw->k = k;
  pw->tn = tile_n;
  pw->tk = tile_k;
  pw->tiles_n = n / tile_n;
  pw->tiles_k = k / tile_k;
  pw->tiles = tiles;
  if (tiles == 0) {
    if (info) fill_info(pw, info);
    *out = pw;
    return ok();
  }
  unsigned long long* sc = nullptr;
  hipError_t e = scratch_address(dev, &sc);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress");
  pw->tile_map = tile_map;
  pw->tile_desc = tile_desc;
  // the first-error word must start at "no error"; the counts are written, not accumulated
  if ((e = launch_fill_u64(sc, 1, PATCH_NO_ERROR_LOC, s)) != hipSuccess) return hip_fail(e, "fill launch");
  if ((e = launch_classify(mask_bits, k, ord, tile_n, tile_k, pw->tiles_n, pw->tiles_k, tile_map, sc, s)) != hipSuccess)
    return hip_fail(e, "classify launch");
  if ((e = launch_slot_scan(tile_map, tiles, tile_desc, reinterpret_cast<long long*>(sc + 1), s)) != hipSuccess)
    return hip_fail(e, "slot scan launch");
  unsigned long long host[3] = {0, 0, 0};
  if ((e = hipMemcpyAsync(host, sc, sizeof(host), hipMemcpyDeviceToHost, s)) != hipSuccess)
    return hip_fail(e, "hipMemcpyAsync");
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  if (host[0] != PATCH_NO_ERROR_LOC) {
    const int64_t per_tile = (int64_t)tile_n * tile_k / 4;
    const int64_t loc = (int64_t)host[0];
    if (info) {
      fill_info(pw, info);
      info->n_dense = info->n_sparse = 0;
      info->bad_tile = loc / per_tile;
      info->bad_row = (loc % per_tile) / (tile_k / 4);
      info->bad_group = (loc % per_tile) % (tile_k / 4);
    }
    return fail(PATCH_E_MASK, "mask is not tile-wise dense / 2:4: tile %lld, row %lld in tile, group %lld along K",
                (long long)(loc / per_tile), (long long)((loc % per_tile) / (tile_k / 4)),
                (long long)((loc % per_tile) % (tile_k / 4)));
  }
  pw->n_dense = (int64_t)host[1];
  pw->n_sparse = (int64_t)host[2];
  const int64_t need_d = pw->n_dense * tile_n * tile_k * 2, need_s = pw->n_sparse * tile_n * tile_k,
                need_m = pw->n_sparse * tile_n * tile_k / 8 + (pw->n_sparse ? 16 : 0);
  if (dense_bytes < need_d || sparse_bytes < need_s || meta_bytes < need_m)
    return fail(PATCH_E_INVALID_ARG,
                "pools too small for %lld dense and %lld 2:4 tiles: need %lld, %lld and %lld bytes, have %lld, %lld "
                "and %lld", (long long)pw->n_dense, (long long)pw->n_sparse, (long long)need_d, (long long)need_s,
                (long long)need_m, (long long)dense_bytes, (long long)sparse_bytes, (long long)meta_bytes);
  pw->dense_vals = dense_vals;
  pw->sparse_vals = sparse_vals;
  pw->sparse_meta = sparse_meta;
  if ((e = launch_compress(w, ldw, mask_bits, k, ord, tile_n, tile_k, pw->tiles_n, pw->tiles_k, tile_desc, dense_vals,
                           sparse_vals, sparse_meta, s)) != hipSuccess)
    return hip_fail(e, "compress launch");
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  if (info) fill_info(pw, info);
  *out = pw;
  return ok();
}

}  // extern "C"
