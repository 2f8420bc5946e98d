// Mask bit-unpack, tile classification / validation, slot scan, compression
// and decompression for the PATCH packed-weight format.
//
// Semantics: each TN x TK tile of W is either dense or 2:4 sparse along K
// ("PATCH: Learnable Tile-level Hybrid Sparsity for LLMs", Abstract); the mask
// is a bit-packed binary keep/prune mask and applying it zeroes the pruned
// weights (model card "llama_3.2_1b-PATCH-45Sparse", description and "How to
// use").  All of these kernels move bits and bytes only; none does floating
// point arithmetic, so their results are bit-exact by construction.
//
// Mask geometry: bit i of the row-major [N][K] mask; K % 64 == 0 and
// TK in {64, 128}, so every tile row starts on an 8-byte boundary of the
// packed stream and one byte holds exactly two groups of four.
#include "patch_internal.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t rev4(uint32_t x) {
  return ((x & 1u) << 3) | ((x & 2u) << 1) | ((x & 4u) >> 1) | ((x & 8u) >> 3);
}

// Keep flags of the two groups held by one mask byte, in k order (bit p of the
// result = keep flag of position p inside the group).
__device__ __forceinline__ void byte_to_groups(uint32_t byte, int order, uint32_t& g0, uint32_t& g1) {
  if (order == PATCH_BITS_MSB_FIRST) {  // first k of the byte is bit 7
    g0 = rev4(byte >> 4);
    g1 = rev4(byte & 0xFu);
  } else {                              // first k of the byte is bit 0
    g0 = byte & 0xFu;
    g1 = byte >> 4;
  }
}

__global__ void k_fill_u64(unsigned long long* p, int64_t count, unsigned long long v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = v;
}

__global__ void k_fill_u32(uint32_t* p, int64_t count, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = v;
}

// One workgroup per tile.  The tile's type is set by its first group; every
// group must keep the same count (4 = dense, 2 = 2:4).  The first offending
// group, linearised as t * (TN*TK/4) + row * (TK/4) + group, lowers *err_loc.
__global__ __launch_bounds__(kThreads) void k_classify(const uint8_t* __restrict__ bits, int64_t k, int order,
                                                       int tn, int tk, int64_t tiles_k,
                                                       uint8_t* __restrict__ tile_map,
                                                       unsigned long long* __restrict__ err_loc) {
  const int64_t t = blockIdx.x;
  const int64_t ti = t / tiles_k, tj = t % tiles_k;
  const int64_t row_bytes = k >> 3;
  const int words_per_row = tk >> 6;  // 8-byte words per tile row: 1 or 2
  const int words = tn * words_per_row;
  const int groups_per_row = tk >> 2;
  const uint8_t* base = bits + ti * tn * row_bytes + tj * (tk >> 3);

  uint32_t f0, f1;
  byte_to_groups(base[0], order, f0, f1);
  const int want = __popc(f0);

  __shared__ uint32_t s_bad;
  if (threadIdx.x == 0) s_bad = 0xFFFFFFFFu;
  __syncthreads();

  uint32_t bad = 0xFFFFFFFFu;
  if (want != 2 && want != 4) {
    bad = 0;
  } else {
    for (int wd = threadIdx.x; wd < words; wd += kThreads) {
      const int r = wd / words_per_row, c = wd % words_per_row;
      const uint64_t v = *reinterpret_cast<const uint64_t*>(base + r * row_bytes + c * 8);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        uint32_t g0, g1;
        byte_to_groups((uint32_t)(v >> (8 * b)) & 0xFFu, order, g0, g1);
        const uint32_t g = (uint32_t)(r * groups_per_row + (c * 8 + b) * 2);
        if (__popc(g0) != want) bad = min(bad, g);
        if (__popc(g1) != want) bad = min(bad, g + 1);
      }
    }
  }
  if (bad != 0xFFFFFFFFu) atomicMin(&s_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    tile_map[t] = (want == 4) ? PATCH_TILE_DENSE : PATCH_TILE_SPARSE24;
    if (s_bad != 0xFFFFFFFFu)
      atomicMin(err_loc, (unsigned long long)t * (unsigned long long)(tn * tk / 4) + s_bad);
  }
}

// Single workgroup: exclusive count of earlier tiles of the same type.
// tile_desc[t] = (slot << 1) | type.  counts[0] = dense tiles, counts[1] = 2:4 tiles.
__global__ __launch_bounds__(1024) void k_slot_scan(const uint8_t* __restrict__ tile_map, int64_t tiles,
                                                    int32_t* __restrict__ tile_desc,
                                                    long long* __restrict__ counts) {
  __shared__ int s_wave[16];
  __shared__ long long s_carry;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < tiles; base += 1024) {
    const int64_t t = base + threadIdx.x;
    const int sp = (t < tiles) ? (tile_map[t] & 1) : 0;
    int v = sp;  // inclusive scan inside the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (lane == 63) s_wave[wave] = v;
    __syncthreads();
    int wave_prefix = 0;
    for (int w = 0; w < wave; ++w) wave_prefix += s_wave[w];
    const long long carry = s_carry;
    const long long incl = carry + wave_prefix + v;
    if (t < tiles) {
      const long long excl_sparse = incl - sp;
      const long long slot = sp ? excl_sparse : (t - excl_sparse);
      tile_desc[t] = (int32_t)((slot << 1) | sp);
    }
    __syncthreads();
    if (threadIdx.x == 1023) s_carry = incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    counts[1] = s_carry;
    counts[0] = tiles - s_carry;
  }
}

// Device layout of the packed pools ("operand order").  The GEMM feeds W to
// smfmac 16x16x64 as the A operand, one 16-row block and one 64-wide K step at
// a time; lane l = 16 q + r of such an operand covers row r of the block and
// dense k = 16 q .. 16 q + 15 of the step.  Each (step, block) unit of a tile
// is stored as exactly those 64 lane values, in lane order, so one 16-byte load
// per lane fetches a whole operand (1 KiB contiguous per wave):
//   unit u = step * (TN / 16) + block, for step < TK / 64, block < TN / 16
//   2:4 values  [slot] [u] [lane] 8 bf16: the 8 kept values of the lane's 16 k
//                                         (two per group of four, ascending k)
//   2:4 codes   [slot] [u / 4] [lane] [u % 4] u16: code of group g at bits
//                                         4 g .. 4 g + 3; the codes of the four
//                                         blocks of a 64-row group sit together,
//                                         8 bytes per lane
//   dense       [slot] [u] [0/1] [lane] 8 bf16: the lane's 16 k split into
//                                         dwords 0, 2, 4, 6 (positions 0 and 1
//                                         of each group) and dwords 1, 3, 5, 7
//                                         (positions 2 and 3)
// Pool sizes equal those of the row-major format; patch_export converts.

// One workgroup per tile; one work item per (unit, lane).
__global__ __launch_bounds__(kThreads) void k_compress(const uint16_t* __restrict__ w, int64_t ldw,
                                                       const uint8_t* __restrict__ bits, int64_t k, int order,
                                                       int tn, int tk, int64_t tiles_k,
                                                       const int32_t* __restrict__ tile_desc,
                                                       uint16_t* __restrict__ dense_vals,
                                                       uint16_t* __restrict__ sparse_vals,
                                                       uint8_t* __restrict__ sparse_meta) {
  const int64_t t = blockIdx.x;
  const int64_t ti = t / tiles_k, tj = t % tiles_k;
  const int32_t d = tile_desc[t];
  const int64_t slot = d >> 1;
  const int bt = tn >> 4;                   // 16-row blocks per tile
  const int items = (tk >> 6) * bt * 64;
  const int64_t row_bytes = k >> 3;
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int u = it >> 6, l = it & 63;
    const int step = u / bt, blk = u % bt, q = l >> 4, r = l & 15;
    const int64_t row = ti * tn + blk * 16 + r;
    const int64_t col = tj * tk + step * 64 + 16 * q;
    const uint16_t* src = w + row * ldw + col;
    const uint4 lo = *reinterpret_cast<const uint4*>(src);
    const uint4 hi = *reinterpret_cast<const uint4*>(src + 8);
    if ((d & 1) == PATCH_TILE_DENSE) {
      uint8_t* dst = reinterpret_cast<uint8_t*>(dense_vals) + (slot * tn * tk + (int64_t)u * 1024) * 2 + l * 16;
      *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.z, hi.x, hi.z);
      *reinterpret_cast<uint4*>(dst + 1024) = make_uint4(lo.y, lo.w, hi.y, hi.w);
      continue;
    }
    const uint32_t wv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    auto elem = [&](uint32_t e) -> uint32_t { return (wv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu; };
    const uint8_t* mb = bits + row * row_bytes + (col >> 3);  // 16 mask bits = 4 groups
    uint32_t vals[4], meta = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t g0, g1;
      byte_to_groups(mb[h], order, g0, g1);
      const uint32_t a0 = __builtin_ctz(g0), b0 = 31 - __builtin_clz(g0);
      const uint32_t a1 = __builtin_ctz(g1), b1 = 31 - __builtin_clz(g1);
      const uint32_t base = 8 * h;
      vals[2 * h] = elem(base + a0) | (elem(base + b0) << 16);
      vals[2 * h + 1] = elem(base + 4 + a1) | (elem(base + 4 + b1) << 16);
      meta |= ((a0 | (b0 << 2)) | ((a1 | (b1 << 2)) << 4)) << (8 * h);
    }
    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(sparse_vals) + slot * tn * tk + (int64_t)u * 1024 + l * 16) =
        make_uint4(vals[0], vals[1], vals[2], vals[3]);
    *reinterpret_cast<uint16_t*>(sparse_meta + slot * tn * (tk >> 3) + (int64_t)(u >> 2) * 512 + l * 8 + (u & 3) * 2) =
        (uint16_t)meta;
  }
}

// Inverse of k_compress into a dense [N][ldw] buffer; pruned weights get 0x0000.
__global__ __launch_bounds__(kThreads) void k_decompress(const int32_t* __restrict__ tile_desc, int tn, int tk,
                                                         int64_t tiles_k,
                                                         const uint16_t* __restrict__ dense_vals,
                                                         const uint16_t* __restrict__ sparse_vals,
                                                         const uint8_t* __restrict__ sparse_meta,
                                                         uint16_t* __restrict__ out, int64_t ldw) {
  const int64_t t = blockIdx.x;
  const int64_t ti = t / tiles_k, tj = t % tiles_k;
  const int32_t d = tile_desc[t];
  const int64_t slot = d >> 1;
  const int bt = tn >> 4;
  const int items = (tk >> 6) * bt * 64;
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int u = it >> 6, l = it & 63;
    const int step = u / bt, blk = u % bt, q = l >> 4, r = l & 15;
    uint16_t* dst = out + (ti * tn + blk * 16 + r) * ldw + tj * tk + step * 64 + 16 * q;
    if ((d & 1) == PATCH_TILE_DENSE) {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(dense_vals) + (slot * tn * tk + (int64_t)u * 1024) * 2 + l * 16;
      const uint4 e = *reinterpret_cast<const uint4*>(src);
      const uint4 o = *reinterpret_cast<const uint4*>(src + 1024);
      *reinterpret_cast<uint4*>(dst) = make_uint4(e.x, o.x, e.y, o.y);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(e.z, o.z, e.w, o.w);
      continue;
    }
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(sparse_vals) + slot * tn * tk +
                                                     (int64_t)u * 1024 + l * 16);
    const uint32_t meta = *reinterpret_cast<const uint16_t*>(sparse_meta + slot * tn * (tk >> 3) +
                                                            (int64_t)(u >> 2) * 512 + l * 8 + (u & 3) * 2);
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
    uint32_t e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t code = (meta >> (4 * g)) & 0xFu;
      e[4 * g + (code & 3u)] = vv[g] & 0xFFFFu;
      e[4 * g + (code >> 2)] = vv[g] >> 16;
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                                e[6] | (e[7] << 16));
    *reinterpret_cast<uint4*>(dst + 8) = make_uint4(e[8] | (e[9] << 16), e[10] | (e[11] << 16),
                                                    e[12] | (e[13] << 16), e[14] | (e[15] << 16));
  }
}

// One thread per packed byte: up to 8 output bytes.
__global__ void k_mask_unpack(const uint8_t* __restrict__ bits, int64_t count, int order,
                              uint8_t* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t first = b * 8;
  if (first >= count) return;
  const uint32_t byte = bits[b];
  uint64_t v = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t bit = (order == PATCH_BITS_MSB_FIRST) ? (byte >> (7 - j)) & 1u : (byte >> j) & 1u;
    v |= (uint64_t)bit << (8 * j);
  }
  if (first + 8 <= count && (reinterpret_cast<uintptr_t>(out + first) & 7) == 0) {
    *reinterpret_cast<uint64_t*>(out + first) = v;
  } else {
    const int64_t n = (count - first < 8) ? count - first : 8;
    for (int64_t j = 0; j < n; ++j) out[first + j] = (uint8_t)((v >> (8 * j)) & 1u);
  }
}

inline unsigned grid_for(int64_t n, int per_block) { return (unsigned)((n + per_block - 1) / per_block); }

}  // namespace

hipError_t launch_fill_u64(unsigned long long* p, int64_t count, unsigned long long v, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(count, 256)), dim3(256), 0, s, p, count, v);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t v, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(count, 256)), dim3(256), 0, s, p, count, v);
  return hipGetLastError();
}

hipError_t launch_classify(const uint8_t* bits, int64_t k, int order, int tn, int tk, int64_t tiles_n,
                           int64_t tiles_k, uint8_t* tile_map, unsigned long long* err_loc, hipStream_t s) {
  const int64_t tiles = tiles_n * tiles_k;
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_classify, dim3((unsigned)tiles), dim3(kThreads), 0, s, bits, k, order, tn, tk, tiles_k,
                     tile_map, err_loc);
  return hipGetLastError();
}

hipError_t launch_slot_scan(const uint8_t* tile_map, int64_t tiles, int32_t* tile_desc, long long* counts,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_slot_scan, dim3(1), dim3(1024), 0, s, tile_map, tiles, tile_desc, counts);
  return hipGetLastError();
}

hipError_t launch_compress(const uint16_t* w, int64_t ldw, const uint8_t* bits, int64_t k, int order, int tn,
                           int tk, int64_t tiles_n, int64_t tiles_k, const int32_t* tile_desc,
                           uint16_t* dense_vals, uint16_t* sparse_vals, uint8_t* sparse_meta, hipStream_t s) {
  const int64_t tiles = tiles_n * tiles_k;
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_compress, dim3((unsigned)tiles), dim3(kThreads), 0, s, w, ldw, bits, k, order, tn, tk,
                     tiles_k, tile_desc, dense_vals, sparse_vals, sparse_meta);
  return hipGetLastError();
}

hipError_t launch_decompress(const patch_weight* pw, uint16_t* w_out, int64_t ldw, hipStream_t s) {
  if (pw->tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_decompress, dim3((unsigned)pw->tiles), dim3(kThreads), 0, s, pw->tile_desc, pw->tn,
                     pw->tk, pw->tiles_k, pw->dense_vals, pw->sparse_vals, pw->sparse_meta, w_out, ldw);
  return hipGetLastError();
}

hipError_t launch_mask_unpack(const uint8_t* bits, int64_t count, int order, uint8_t* out, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int64_t nbytes = (count + 7) / 8;
  hipLaunchKernelGGL(k_mask_unpack, dim3(grid_for(nbytes, 256)), dim3(256), 0, s, bits, count, order, out);
  return hipGetLastError();
}
