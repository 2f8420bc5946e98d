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

// One workgroup per tile.  Dense: copy the tile row-major.  2:4: each thread
// takes 8 consecutive k of one row (two groups): two kept values per group in
// ascending k, and one byte of codes (i0 | i1 << 2), even group low.
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
  const uint16_t* wt = w + ti * tn * ldw + tj * tk;
  const int units_per_row = tk >> 3;  // 8 bf16 = 16 bytes per unit
  const int units = tn * units_per_row;
  if ((d & 1) == PATCH_TILE_DENSE) {
    uint16_t* dst = dense_vals + slot * tn * tk;
    for (int u = threadIdx.x; u < units; u += kThreads) {
      const int r = u / units_per_row, c = u % units_per_row;
      *reinterpret_cast<uint4*>(dst + r * tk + c * 8) = *reinterpret_cast<const uint4*>(wt + r * ldw + c * 8);
    }
    return;
  }
  uint16_t* vdst = sparse_vals + slot * tn * (tk >> 1);
  uint8_t* mdst = sparse_meta + slot * tn * (tk >> 3);
  const int64_t row_bytes = k >> 3;
  const uint8_t* bt = bits + ti * tn * row_bytes + tj * (tk >> 3);
  for (int u = threadIdx.x; u < units; u += kThreads) {
    const int r = u / units_per_row, c = u % units_per_row;
    const uint4 raw = *reinterpret_cast<const uint4*>(wt + r * ldw + c * 8);
    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t g0, g1;
    byte_to_groups(bt[r * row_bytes + c], order, g0, g1);
    const uint32_t a0 = __builtin_ctz(g0), b0 = 31 - __builtin_clz(g0);
    const uint32_t a1 = __builtin_ctz(g1), b1 = 31 - __builtin_clz(g1);
    auto elem = [&](uint32_t e) -> uint32_t { return (wv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu; };
    uint2 out;
    out.x = elem(a0) | (elem(b0) << 16);
    out.y = elem(4 + a1) | (elem(4 + b1) << 16);
    *reinterpret_cast<uint2*>(vdst + r * (tk >> 1) + c * 4) = out;
    mdst[r * (tk >> 3) + c] = (uint8_t)((a0 | (b0 << 2)) | ((a1 | (b1 << 2)) << 4));
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
  uint16_t* ot = out + ti * tn * ldw + tj * tk;
  const int units_per_row = tk >> 3;
  const int units = tn * units_per_row;
  if ((d & 1) == PATCH_TILE_DENSE) {
    const uint16_t* src = dense_vals + slot * tn * tk;
    for (int u = threadIdx.x; u < units; u += kThreads) {
      const int r = u / units_per_row, c = u % units_per_row;
      *reinterpret_cast<uint4*>(ot + r * ldw + c * 8) = *reinterpret_cast<const uint4*>(src + r * tk + c * 8);
    }
    return;
  }
  const uint16_t* vsrc = sparse_vals + slot * tn * (tk >> 1);
  const uint8_t* msrc = sparse_meta + slot * tn * (tk >> 3);
  for (int u = threadIdx.x; u < units; u += kThreads) {
    const int r = u / units_per_row, c = u % units_per_row;
    const uint2 v = *reinterpret_cast<const uint2*>(vsrc + r * (tk >> 1) + c * 4);
    const uint32_t code = msrc[r * (tk >> 3) + c];
    uint32_t e[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    e[code & 3u] = v.x & 0xFFFFu;
    e[(code >> 2) & 3u] = v.x >> 16;
    e[4 + ((code >> 4) & 3u)] = v.y & 0xFFFFu;
    e[4 + ((code >> 6) & 3u)] = v.y >> 16;
    uint4 o;
    o.x = e[0] | (e[1] << 16);
    o.y = e[2] | (e[3] << 16);
    o.z = e[4] | (e[5] << 16);
    o.w = e[6] | (e[7] << 16);
    *reinterpret_cast<uint4*>(ot + r * ldw + c * 8) = o;
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
