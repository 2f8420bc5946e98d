// Internal declarations shared by the libpatch HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/patch.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Handle.  All pointers are device memory owned by the handle.
struct patch_weight {
  int device;
  int64_t n, k;
  int32_t tn, tk;
  int64_t tiles_n, tiles_k, tiles, n_dense, n_sparse;
  uint8_t* tile_map;     // [tiles]  PATCH_TILE_DENSE / PATCH_TILE_SPARSE24
  int32_t* tile_desc;    // [tiles]  (slot << 1) | type: one load gives the tile's address
  uint16_t* dense_vals;  // [D][TN][TK]
  uint16_t* sparse_vals; // [S][TN][TK/2]
  uint8_t* sparse_meta;  // [S][TN][TK/8]
  // Host: row_dense_prefix[i] = dense tiles in tile rows 0 .. i-1 (tiles_n + 1
  // entries), the cost prefix the GEMM launcher schedules by (NULL for a handle
  // made by patch_pack_noalloc: its rows then count at the weight's mean mix).
  int64_t* row_dense_prefix;
  // Made by patch_pack_noalloc: the struct and the pools belong to the caller,
  // and patch_destroy frees nothing.
  bool borrowed;
};

// Relative time of one 64-wide K step of a 64-row W group in the tiled
// kernels: dense 1, 2:4 0.84 (in-kernel timestamps on MI355X, 256-row blocks,
// 90% against 0% 2:4 tiles: 2 650 against 3 150 clocks per step).
#define PATCH_STEP_COST_DENSE 1.0
#define PATCH_STEP_COST_24 0.84
// Mean relative step cost of tile rows [r0, r1) of w (1 = all dense).
double row_cost(const patch_weight* w, int64_t r0, int64_t r1);
// Fills w->row_dense_prefix from a host copy of the tile map; false if the
// host allocation fails.
bool set_cost_prefix(patch_weight* w, const uint8_t* tile_map_host);

// Words of the per-GPU validation scratch of patch_pack_noalloc.
#define PATCH_PACK_SCRATCH_WORDS 4

// Sentinel for "no invalid group found".
#define PATCH_NO_ERROR_LOC 0xFFFFFFFFFFFFFFFFull

// ---- pack kernels (pack.hip) ----
// Writes tile_map and atomically lowers *err_loc to the first invalid group
// (t * TN*TK/4 + row * TK/4 + group).  *err_loc must start at PATCH_NO_ERROR_LOC.
hipError_t launch_classify(const uint8_t* bits, int64_t k, int order, int tn, int tk,
                           int64_t tiles_n, int64_t tiles_k, uint8_t* tile_map,
                           unsigned long long* err_loc, hipStream_t s);
hipError_t launch_fill_u64(unsigned long long* p, int64_t count, unsigned long long v, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t v, hipStream_t s);
// Exclusive per-type slot scan; counts[0] = D, counts[1] = S.
hipError_t launch_slot_scan(const uint8_t* tile_map, int64_t tiles, int32_t* tile_desc,
                            long long* counts, hipStream_t s);
hipError_t launch_compress(const uint16_t* w, int64_t ldw, const uint8_t* bits, int64_t k, int order,
                           int tn, int tk, int64_t tiles_n, int64_t tiles_k, const int32_t* tile_desc,
                           uint16_t* dense_vals, uint16_t* sparse_vals, uint8_t* sparse_meta,
                           hipStream_t s);
hipError_t launch_decompress(const patch_weight* pw, uint16_t* w_out, int64_t ldw, hipStream_t s);
hipError_t launch_mask_unpack(const uint8_t* bits, int64_t count, int order, uint8_t* out, hipStream_t s);
// ---- hard tile-configuration sample (sample.hip) ----
hipError_t launch_sample_mask(const float* tile_logits, const float* tile_noise, const float* group_logits,
                              const float* group_noise, int64_t n, int64_t k, int tn, int tk, float kappa,
                              int lsb_first, uint8_t* bits, hipStream_t s);

// ---- GEMM kernels ----
// One product Y = X . Wm^T of a launch; a launch runs up to PATCH_MAX_GROUP of
// them, passed by value as a kernel argument.
#define PATCH_MAX_GROUP 16
struct gemm_problem {
  const int32_t* tile_desc;
  const uint16_t* dense_vals;
  const uint16_t* sparse_vals;
  const uint8_t* sparse_meta;
  const uint16_t* x;
  void* y;
  int64_t tiles_k, n, k, m, ldx, ldy;
  int32_t tn, tk;
  int32_t block0;  // first workgroup of this product in the launch
  int32_t blocks;  // its workgroups (the launch may pad after them)
  float w_bytes;   // packed bytes per weight element (2 dense, 1.125 for 2:4, mean over tiles)
  int32_t group_n; // tiled kernels: block columns per group of the block order
  int64_t n_begin; // this entry covers W rows / Y columns n_begin .. n - 1
  int32_t bm;      // tiled kernels: X rows per block of this entry (set by the launcher)
  float mix;       // mean relative step cost of the entry's W rows (host scheduling only)
  int32_t ksplit;  // streaming kernel: workgroups that share each W block's K range (1: no split, or 4)
  float* part;     // ksplit > 1: fp32 partial sums [ksplit][m][n], one per share of K
};
struct gemm_group {
  int32_t count;
  int32_t total;  // workgroup slots of the whole launch (tiled kernels)
  gemm_problem p[PATCH_MAX_GROUP];
};
// The product of handle w with X [m][ldx] into Y [m][ldy] (block fields unset).
gemm_problem make_problem(const patch_weight* w, const uint16_t* x, int64_t m, int64_t ldx, void* y, int64_t ldy);
// PATCH_STREAM_MAX_M (patch.h): 8 blocks of 16 X rows per wave.
// 16-row X blocks per wave of the streaming kernel for m rows (0 past PATCH_STREAM_MAX_M).
int stream_x_blocks(int64_t m);
// 16-row W blocks per workgroup of the streaming kernel for an n-row W (1, 2 or 4).
int stream_w_blocks(int64_t n);
// Waves that split K in the streaming kernel for an m x n product (16 or 8).
int stream_waves(int64_t m, int64_t n);
// Workgroups that share one W block's K range of an m x n x k product when
// the caller gives a workspace (1: it runs unsplit; else 4), and the W blocks
// per workgroup then.
int stream_k_split(int64_t m, int64_t n, int64_t k);
int stream_split_w_blocks(int64_t n);
// One product on the streaming kernel with its K split p.ksplit ways: fp32
// partials into p.part, then a second launch that sums them in order into Y.
hipError_t launch_stream_split(const gemm_problem& p, int out_f32, hipStream_t s);
// One launch of the streaming kernel (every m <= PATCH_STREAM_MAX_M) / the
// tiled kernel over a group.  block_m > 0 forces the tiled block height (256,
// 192, 128, 64).
hipError_t launch_stream_group(gemm_group& g, int out_f32, hipStream_t s);
hipError_t launch_tiled_group(gemm_group& g, int out_f32, int block_m, hipStream_t s);
// The tiled block height the launcher would pick for a group.
int tiled_block_m(const gemm_group& g);
hipError_t launch_fill_zero_y(void* y, int64_t m, int64_t n, int64_t ldy, int out_f32, hipStream_t s);

// ---- device helpers ----
// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
