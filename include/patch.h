/*
 * patch.h -- C ABI of libpatch.so: the PATCH hybrid dense / 2:4 tile GEMM on
 * AMD Instinct MI355X (gfx950).
 *
 * In PATCH each tile of a weight matrix keeps all its weights or is pruned 2:4
 * (half of them), so the matrix's sparsity can take any value from 0% to 50%
 * ("PATCH: Learnable Tile-level Hybrid Sparsity for LLMs", Abstract).  The
 * released artifact is a bit-packed binary keep/prune mask over frozen base
 * weights, and applying it zeroes the pruned weights (model card
 * "llama_3.2_1b-PATCH-45Sparse", description and "How to use").  Hardware tiles
 * are 128x128, 128x64, 64x128 and 64x64 (same card, "Training
 * hyper-parameters").
 *
 * This library takes W (bf16, nn.Linear layout [N][K]) plus such a mask,
 * validates that every tile is dense or 2:4 along K, compresses W into a packed
 * weight, and computes Y = X . W_masked^T on the matrix cores: 2:4 tiles on the
 * sparse MFMA instruction (smfmac 16x16x64, bf16), dense tiles on the same
 * instruction twice per 64-wide K step with fixed index words (kept positions
 * 0, 1 and then 2, 3 of every group of four), which does the dense bf16 MFMA's
 * work per instruction at its rate.
 *
 * Conventions for every call:
 *   - Pointers marked "device" are HIP device pointers on the current device;
 *     "host" pointers are ordinary host memory.  Device pointers must be
 *     16-byte aligned.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued on
 *     it in order; only patch_pack, patch_import and patch_export block the
 *     host.
 *   - Every call returns a patch_status.  Nothing aborts and no C++ exception
 *     crosses the ABI.  On failure patch_last_error() returns a message (per
 *     thread, valid until the next call on that thread).
 *   - Only gfx950 devices are supported (PATCH_E_UNSUPPORTED otherwise).
 */
#ifndef PATCH_H_
#define PATCH_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PATCH_OK = 0,
  PATCH_E_INVALID_ARG = 1, /* null / misaligned pointer, bad enum, bad leading dimension */
  PATCH_E_SHAPE = 2,       /* tile not in {64,128}^2, N % TN != 0, K % TK != 0, or N*K > 2^31 - 1 */
  PATCH_E_MASK = 3,        /* some tile is neither all-dense nor exactly 2:4 along K */
  PATCH_E_HIP = 4,         /* a HIP runtime call failed (message has hipGetErrorString) */
  PATCH_E_NOMEM = 5,       /* device allocation failed; nothing is leaked */
  PATCH_E_UNSUPPORTED = 6  /* device is not gfx950 */
} patch_status;

/* Bit order of the packed mask: bit i of the row-major flattened [N][K] mask is
 * bit (7 - i%8) (MSB first, numpy.packbits default) or bit (i%8) (LSB first)
 * of byte i/8.  1 = keep. */
typedef enum { PATCH_BITS_MSB_FIRST = 0, PATCH_BITS_LSB_FIRST = 1 } patch_bit_order;

typedef enum { PATCH_OUT_BF16 = 0, PATCH_OUT_F32 = 1 } patch_out_dtype;

/* Largest X leading dimension (elements) patch_gemm accepts: 2^22. */
#define PATCH_MAX_LDX 4194304LL

/* Largest weight (N * K elements) patch_pack, patch_pack_noalloc, patch_import
 * and patch_sample_mask accept: 2^31 - 1.  The GEMM kernels address the packed
 * pools with 32-bit byte offsets; the largest linear of a 70B-class model holds
 * about 2^28 weights. */
#define PATCH_MAX_WEIGHTS 2147483647LL

typedef enum { PATCH_TILE_DENSE = 0, PATCH_TILE_SPARSE24 = 1 } patch_tile_type;

/* Largest M the STREAM kernel takes. */
#define PATCH_STREAM_MAX_M 128

/* Kernel selection for patch_gemm_kernel.  AUTO picks STREAM for M <= 16 and
 * TILED for M > PATCH_STREAM_MAX_M; in between it estimates both kernels' time
 * from the weight's shape and packed bytes and picks the faster.  Forcing one
 * is for tests and measurements. */
typedef enum {
  PATCH_KERNEL_AUTO = 0,
  PATCH_KERNEL_TILED = 1,  /* LDS-staged MFMA tiles, for prefill-sized M */
  PATCH_KERNEL_STREAM = 2  /* weight streaming, one workgroup per 16, 32 or 64 rows of W (wider
                              weights take more), each W chunk applied to all M rows: decode and
                              batches up to PATCH_STREAM_MAX_M rows */
} patch_kernel;

typedef struct patch_weight patch_weight; /* opaque, owned by the library */

typedef struct {
  int64_t n, k;                 /* W is [n][k] */
  int32_t tile_n, tile_k;       /* TN x TK */
  int64_t tiles_n, tiles_k;     /* n / TN, k / TK */
  int64_t n_dense, n_sparse;    /* D and S; D + S = tiles_n * tiles_k */
  int64_t bytes_dense;          /* D * TN * TK * 2 */
  int64_t bytes_sparse_vals;    /* S * TN * TK     (TK/2 bf16 per row) */
  int64_t bytes_sparse_meta;    /* S * TN * TK / 8 (one 4-bit code per group) */
  double sparsity;              /* 0.5 * S / (D + S): fraction of pruned weights */
  int64_t bad_tile, bad_row, bad_group; /* first invalid group, or -1 (see patch_pack) */
} patch_info;

/*
 * patch_pack -- validate a keep mask and compress W into a packed weight.
 *
 * Semantics: the mask is the bit-packed keep/prune mask of the card's
 * description; each TN x TK tile must be dense (every aligned group of four
 * along K keeps 4) or 2:4 (every group keeps exactly 2).  A tile's type is set
 * by its first group; the first group (tiles in row-major order, then rows,
 * then groups along K) whose count differs, or a first group that keeps 0, 1
 * or 3, is reported.
 *
 *   w          device, bf16 [n][ldw], ldw >= k, ldw % 8 == 0.  Read only.
 *   n, k       W shape; n % tile_n == 0, k % tile_k == 0; n, k >= 0.
 *   mask_bits  device, ceil(n*k/8) bytes, bit order `order`.  Read only.
 *   tile_n/k   each 64 or 128.
 *   out        receives the new handle (NULL on any failure).
 *   info       host, may be NULL; filled on success and on PATCH_E_MASK
 *              (bad_tile = row-major tile index, bad_row = row inside the tile,
 *              bad_group = group of four inside that tile row).
 *
 * Packed format (exported by patch_export, bit-exact):
 *   tile_map[t]  PATCH_TILE_DENSE / PATCH_TILE_SPARSE24, t = i*tiles_k + j.
 *   tile_slot[t] number of earlier tiles of the same type.
 *   dense_vals   [D][TN][TK] bf16, the tile copied row-major.
 *   sparse_vals  [S][TN][TK/2] bf16: per row, per group, the two kept values
 *                in ascending k.
 *   sparse_meta  [S][TN][TK/8] bytes: per group the code i0 | i1 << 2 of the
 *                kept positions (i0 < i1), two groups per byte, even group in
 *                the low nibble.
 *
 * Ownership: W and the mask may be freed once this returns; the handle owns
 * copies of everything it needs.  Blocks the host until validation is known
 * (one device-to-host copy).
 */
patch_status patch_pack(const uint16_t* w, int64_t n, int64_t k, int64_t ldw,
                        const uint8_t* mask_bits, patch_bit_order order,
                        int32_t tile_n, int32_t tile_k, void* stream,
                        patch_weight** out, patch_info* info);

/*
 * patch_gemm -- Y = X . W_masked^T, the linear layer over the packed weight.
 *
 * Y[m][n] = sum_k X[m][k] * Wm[n][k] with bf16 inputs and fp32 accumulation;
 * Wm is W with the pruned weights zeroed (card "How to use").  2:4 tiles run
 * on smfmac with their stored indices, dense tiles on smfmac twice with fixed
 * indices (dense bf16 MFMA work and rate), so only kept weights are multiplied.
 *
 *   x      device, bf16 [m][ldx], k <= ldx <= PATCH_MAX_LDX, ldx % 8 == 0.
 *   m      >= 0 rows of X (0 is a no-op).
 *   y      device, [m][ldy] of bf16 (round to nearest even) or fp32,
 *          ldy >= n, ldy % 8 == 0.  Written, never read.  Must not alias x.
 *
 * Never allocates, never blocks the host and keeps no state between calls:
 * calls on the same handle may overlap on different streams (they only read
 * the handle).  Y is deterministic: the same inputs give the same bits.
 */
patch_status patch_gemm(const patch_weight* w, const uint16_t* x, int64_t m, int64_t ldx,
                        void* y, int64_t ldy, patch_out_dtype y_dtype, void* stream);

/* patch_gemm with the kernel chosen by the caller, for tests and measurements.
 * `variant` <= 0 lets the library choose; for PATCH_KERNEL_TILED a positive
 * value forces the X rows per workgroup, 256, 192, 128 or 64 (other values:
 * PATCH_E_INVALID_ARG).  It is ignored by PATCH_KERNEL_STREAM and
 * PATCH_KERNEL_AUTO.  PATCH_KERNEL_STREAM needs m <= PATCH_STREAM_MAX_M. */
patch_status patch_gemm_kernel(const patch_weight* w, const uint16_t* x, int64_t m, int64_t ldx,
                               void* y, int64_t ldy, patch_out_dtype y_dtype,
                               patch_kernel kernel, int32_t variant, void* stream);

/*
 * patch_gemm_with_workspace -- patch_gemm that may split K across workgroups.
 *
 * The same product as patch_gemm (card "How to use": Y = X . W_masked^T).
 * When AUTO runs it on the streaming kernel (m <= PATCH_STREAM_MAX_M) and the
 * weight is narrow with a long K (fewer than 5120 rows of W, at least 2048,
 * and below 4096 for m <= 16; K >= 8192), four workgroups share each block of
 * W rows, each taking a quarter of K: they write fp32 partial sums into the
 * workspace, and a second launch adds the four in a fixed order into Y.
 * Otherwise it is patch_gemm.
 *
 *   workspace        device, 16-byte aligned, workspace_bytes long, or NULL.
 *                    Scratch: its contents are not kept.  The product is split
 *                    only if workspace_bytes >= patch_gemm_workspace_size.
 *   other arguments  as for patch_gemm.
 *
 * Never allocates and never blocks the host.  Calls that share a workspace
 * must not overlap (order them on one stream).  Y is deterministic; a split
 * product's Y sums K in another order than patch_gemm's, so the two may
 * differ in the last bits (both are within the same error bound).
 */
patch_status patch_gemm_with_workspace(const patch_weight* w, const uint16_t* x, int64_t m, int64_t ldx,
                                       void* y, int64_t ldy, patch_out_dtype y_dtype, void* workspace,
                                       int64_t workspace_bytes, void* stream);

/* Bytes of workspace with which patch_gemm_with_workspace splits the product
 * of m rows on w (0: it would not split).  *bytes is written on success;
 * PATCH_E_INVALID_ARG for a NULL handle or pointer, or m < 0. */
patch_status patch_gemm_workspace_size(const patch_weight* w, int64_t m, int64_t* bytes);

/*
 * patch_gemm_grouped -- several independent linear layers in one launch.
 *
 * A transformer layer applies several linears to the same or to different
 * inputs (the card's model is LLaMA-3.2-1B: q, k, v, o, gate, up and down
 * projections per layer, each with its own PATCH mask).  Each item is the
 * patch_gemm of its own handle, X and Y.  Items that run on the STREAM kernel
 * (as their solo patch_gemm would) share a launch of it with the items that
 * split K among as many waves and carry as many W blocks per workgroup (both
 * set by the item's own m and n), so each item's Y equals its solo result;
 * TILED items that fill the GPU on their own (at least
 * one 256 x 256 output block per compute unit) get a launch each, and the
 * other TILED items share one launch, so small projections share the chip
 * instead of running one after another; an item with K = 0 gets a zero fill.
 * With patch_gemm_grouped_kernel and a forced kernel, all items of that
 * kernel share one launch.
 *
 *   items    host, `count` items; read during the call only.
 *   count    0 .. 16 (0 is a no-op).
 *   y_dtype  applies to every item.
 *
 * Each item obeys patch_gemm's rules (the first failing item is named in the
 * message, and nothing is launched).  The Y buffers must not overlap one
 * another or any X of the group; X buffers and handles may be shared.  Each
 * item's Y equals, bit for bit, what patch_gemm gives for it alone.  Never
 * allocates and never blocks the host.
 */
typedef struct {
  const patch_weight* w;
  const uint16_t* x; /* device, bf16 [m][ldx] */
  int64_t m;
  int64_t ldx;
  void* y;           /* device, [m][ldy] of y_dtype */
  int64_t ldy;
} patch_gemm_item;

patch_status patch_gemm_grouped(const patch_gemm_item* items, int32_t count, patch_out_dtype y_dtype,
                                void* stream);

/* patch_gemm_grouped with the kernel chosen by the caller (`kernel` and
 * `variant` as in patch_gemm_kernel, applied to every item). */
patch_status patch_gemm_grouped_kernel(const patch_gemm_item* items, int32_t count, patch_out_dtype y_dtype,
                                       patch_kernel kernel, int32_t variant, void* stream);

/*
 * patch_unpack -- rebuild the masked dense weight: the card's "apply the mask"
 * (pruned weights zeroed).  Kept weights get their bf16 bits back exactly;
 * pruned ones get +0.0 (0x0000).
 *
 *   w_out  device, bf16 [n][ldw], ldw >= k, ldw % 8 == 0.  Written.
 */
patch_status patch_unpack(const patch_weight* w, uint16_t* w_out, int64_t ldw, void* stream);

/*
 * patch_mask_unpack -- expand `count` packed mask bits into bytes 0/1
 * (out[i] = bit i in `order`).  Pad bits past `count` are ignored.
 *
 * The released artifact of the method is a binary keep/prune mask stored
 * bit-packed in mask.npz (model card "llama_3.2_1b-PATCH-45Sparse",
 * description; the MaskLLM card "gemma_3_1b-MaskLLM-50Sparse", description,
 * ships its mask the same way).  The pages do not state the bit order; both
 * orders are accepted, 1 = keep.
 *
 *   bits   device, at least ceil(count/8) bytes.  Read only.
 *   count  number of mask bits, >= 0 (0 is a no-op).
 *   out    device, at least count bytes, written.  May have any alignment.
 *
 * Errors: PATCH_E_INVALID_ARG for a bad order, count < 0 or a NULL pointer
 * when count > 0; PATCH_E_UNSUPPORTED off gfx950.  Buffer sizes cannot be
 * checked here: a short `bits` or `out` is read or written out of bounds.
 * Never allocates, never blocks the host.
 */
patch_status patch_mask_unpack(const uint8_t* bits, int64_t count, patch_bit_order order,
                               uint8_t* out, void* stream);

/*
 * patch_get_info -- shape, tile counts, pool sizes and sparsity of a packed
 * weight.  `sparsity` is the fraction of pruned weights, 0.5 * S / (D + S):
 * the pages report the measured mask sparsity this way, 44.99% for a 45%
 * target (model card "llama_3.2_1b-PATCH-45Sparse", description) and 50.00%
 * when every tile is 2:4 (card "gemma_3_1b-MaskLLM-50Sparse", description).
 *
 *   w     handle.   info  host struct, written (bad_* are -1).
 *
 * Errors: PATCH_E_INVALID_ARG for a NULL argument.  No device work.
 */
patch_status patch_get_info(const patch_weight* w, patch_info* info);

/*
 * patch_export -- copy the packed arrays to host buffers in the format
 * described under patch_pack.  The pages define the tile types (dense or 2:4,
 * "PATCH: Learnable Tile-level Hybrid Sparsity for LLMs", Abstract) but give
 * no storage format for a packed weight; the exported format is this
 * library's own (kept values in ascending k, 4-bit codes, separate pools), and
 * it is what the CPU oracle produces, so the two can be compared bit for bit.
 *
 *   tile_map, tile_slot   host, tiles = tiles_n * tiles_k entries (u8, i32).
 *   dense_vals, sparse_vals, sparse_meta   host, bytes_dense,
 *                         bytes_sparse_vals and bytes_sparse_meta bytes.
 *   Any of them may be NULL to skip that array.
 *
 * Errors: PATCH_E_INVALID_ARG for a NULL handle, PATCH_E_HIP if a copy fails,
 * PATCH_E_NOMEM if host staging memory runs out.  Blocks the host until the
 * copies are done.  The packed arrays never change after patch_pack or
 * patch_import returns, so GEMMs on the handle may still be in flight.
 */
patch_status patch_export(const patch_weight* w, uint8_t* tile_map, int32_t* tile_slot,
                          uint16_t* dense_vals, uint16_t* sparse_vals, uint8_t* sparse_meta);

/*
 * patch_sample_mask -- the hard sample of a tile configuration: per tile the
 * choice dense / 2:4, per group of four along K one of the six 2:4 patterns,
 * written as a bit-packed keep mask that patch_pack accepts.
 *
 * PATCH learns a per-tile dense / 2:4 choice ("PATCH: Learnable Tile-level
 * Hybrid Sparsity for LLMs", Abstract) from logits sampled with Gumbel noise
 * under a scaling kappa and a temperature tau (model card
 * "llama_3.2_1b-PATCH-45Sparse", "Training hyper-parameters": kappa 25 -> 350,
 * tau 4 -> 0.05, logits initialised from N(0, 0.014)); the pattern inside a
 * 2:4 group comes from logits over its candidate patterns (card
 * "gemma_3_1b-MaskLLM-50Sparse", description).  Each choice takes the index
 * of the largest score fl(fl(kappa * logit) + noise), computed in fp32 with
 * one rounding per operation; the first maximum wins and a NaN score never
 * wins (all-NaN or all -inf picks index 0).  tau divides every score of a
 * choice by the same positive number, so it does not change a hard sample and
 * is not an argument.
 *
 *   tile_logits   device f32 [tiles][2] (dense, 2:4), row-major tile order,
 *                 tiles = (n/tile_n)*(k/tile_k).
 *   tile_noise    device f32 [tiles][2], or NULL for no noise.
 *   group_logits  device f32 [n][k/4][6]: per group, the patterns with kept
 *                 positions (0,1) (0,2) (0,3) (1,2) (1,3) (2,3) in that order.
 *   group_noise   device f32 [n][k/4][6], or NULL.
 *   n, k, tile_n/k  as for patch_pack (PATCH_E_SHAPE otherwise).
 *   kappa         scale of the logits.
 *   mask_bits     device, n*k/8 bytes, written (bit order `order`; 1 = keep):
 *                 dense tiles keep everything, 2:4 tiles the chosen pattern.
 *
 * All float pointers 4-byte aligned.  Never allocates, never blocks the host.
 */
patch_status patch_sample_mask(const float* tile_logits, const float* tile_noise, const float* group_logits,
                               const float* group_noise, int64_t n, int64_t k, int32_t tile_n, int32_t tile_k,
                               float kappa, patch_bit_order order, uint8_t* mask_bits, void* stream);

/*
 * patch_import -- build a packed weight from the exported format: the inverse
 * of patch_export, e.g. for a packed weight saved to a file and read back.
 * The released artifact of the method is a mask over frozen base weights
 * (model card "llama_3.2_1b-PATCH-45Sparse", description); this lets a model
 * be packed once and loaded later without the dense W or the mask.
 *
 *   n, k, tile_n/k  as for patch_pack.
 *   tile_map     host, (n/tile_n)*(k/tile_k) bytes, each PATCH_TILE_DENSE or
 *                PATCH_TILE_SPARSE24; D and S are the counts of each.
 *   dense_vals   host, D*tile_n*tile_k bf16 (may be NULL when D = 0).
 *   sparse_vals  host, S*tile_n*tile_k/2 bf16.   sparse_meta  host,
 *                S*tile_n*tile_k/8 bytes (both may be NULL when S = 0).
 *                Layouts exactly as in the packed-format notes of patch_pack;
 *                slots follow from the tile order.
 *   stream, out, info  as for patch_pack.
 *
 * Errors, all found on the host before any device work: PATCH_E_SHAPE as for
 * patch_pack; PATCH_E_INVALID_ARG for a tile_map byte other than 0 or 1, or a
 * NULL pool that must hold data; PATCH_E_MASK for a 2:4 code that is not
 * i0 | i1 << 2 with i0 < i1 (info->bad_tile / bad_row / bad_group locate it,
 * as for patch_pack).  Ownership as for patch_pack: the host arrays may be
 * freed on return.  Blocks the host until the copies are done.
 * patch_export of the result returns the same arrays bit for bit.
 */
patch_status patch_import(int64_t n, int64_t k, int32_t tile_n, int32_t tile_k, const uint8_t* tile_map,
                          const uint16_t* dense_vals, const uint16_t* sparse_vals, const uint8_t* sparse_meta,
                          void* stream, patch_weight** out, patch_info* info);

/*
 * patch_pack_noalloc -- patch_pack for callers that cannot allocate memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the caller provides the device pools and the host storage of the
 * handle, and the library allocates nothing, on the device or the host.
 *
 * Same validation, packed format, status codes and blocking as patch_pack,
 * with these differences:
 *   tile_map, tile_desc  device, tiles and 4 * tiles bytes (tiles =
 *            (n/tile_n) * (k/tile_k)); tile_desc 16-byte aligned.
 *   dense_vals / sparse_vals / sparse_meta  device pools of dense_bytes,
 *            sparse_bytes and meta_bytes bytes, 16-byte aligned.  After
 *            classification they must hold 2 D TN TK, S TN TK and S TN TK / 8 +
 *            16 bytes (D, S: dense and 2:4 tiles; sizes for every tile dense,
 *            2 n k, and every tile 2:4, n k and n k / 8 + 16, always suffice);
 *            otherwise PATCH_E_INVALID_ARG and nothing is compressed.
 *   storage  host memory the handle is built in; *out points into it.
 * The caller owns storage and every pool and must keep them alive while the
 * handle is used; patch_destroy on this handle frees nothing.  The handle
 * works with every other entry point.  Its rows are scheduled at the weight's
 * mean dense / 2:4 mix (patch_pack keeps a per-row count on the host).
 *
 * Validation uses a fixed 32-byte scratch in device memory, one per GPU,
 * reserved when the library is loaded and held until the process ends; it does
 * not grow with the weight, so no size is refused for it.  Every call on one
 * GPU reuses it: calls that overlap on the same GPU (different host threads or
 * streams) race and must be serialised by the caller.
 */
typedef struct {
  uint64_t words[64];
} patch_weight_storage;

patch_status patch_pack_noalloc(const uint16_t* w, int64_t n, int64_t k, int64_t ldw,
                                const uint8_t* mask_bits, patch_bit_order order,
                                int32_t tile_n, int32_t tile_k, void* stream,
                                uint8_t* tile_map, int32_t* tile_desc,
                                uint16_t* dense_vals, int64_t dense_bytes,
                                uint16_t* sparse_vals, int64_t sparse_bytes,
                                uint8_t* sparse_meta, int64_t meta_bytes,
                                patch_weight_storage* storage, patch_weight** out,
                                patch_info* info);

/* Free a handle and its device memory (NULL is a no-op; a handle made by
 * patch_pack_noalloc owns nothing and is left alone).  The caller must make
 * sure no work using it is still in flight. */
void patch_destroy(patch_weight* w);

/* Message for the last failing call on this thread ("" if none). */
const char* patch_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PATCH_H_ */
