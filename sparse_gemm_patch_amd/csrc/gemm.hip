// Hybrid dense / 2:4 tile GEMM:  Y[m][n] = sum_k X[m][k] * Wm[n][k].
//
// Every TN x TK tile of W is dense or 2:4 along K ("PATCH: Learnable
// Tile-level Hybrid Sparsity for LLMs", Abstract; tile sizes from model card
// "llama_3.2_1b-PATCH-45Sparse", "Training hyper-parameters").  W is the MFMA
// "A" operand, because the gfx950 sparse MFMA (smfmac) takes its 2:4 operand
// there; X rows are the "B" operand; each wave accumulates a block of Y^T in
// fp32 and the epilogue writes Y[m][n].
//
// gfx950 operand layouts used here (lane l, register j; R = 16 or 32 rows):
//   dense  16x16x32 / 32x32x16 bf16: A[l%R][8*(l/R)+j], B[8*(l/R)+j][l%R]
//   smfmac 16x16x64 / 32x32x32 bf16: compressed A row l%R holds the kept
//          values of dense k = 16*(l/R) .. +15 (8 values, 2 per group of four);
//          the 2-bit position of value j is bits [2j+1:2j] of the index VGPR;
//          B register j holds k = 8*(l/R)+j (j < 8) or KK/2 + 8*(l/R)+j-8.
//   C: 16x16 -> row 4*(l/16)+r, col l%16;  32x32 -> row 8*(r/4)+4*(l/32)+r%4, col l%32.
// So a K chunk of X loaded as two 16-byte pieces (k = 8q.. and KK/2 + 8q..)
// feeds both the pair of dense MFMAs and the single smfmac over that chunk,
// and the packed 2:4 format (two kept values per group in ascending k, code
// i0 | i1 << 2 with the even group in the low nibble) is exactly the smfmac
// operand: 16 contiguous bytes of values plus one little-endian u16 of codes.
#include "patch_internal.h"

namespace {

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x16 cat16(bf16x8 a, bf16x8 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

// Store four consecutive n of one row of Y.
template <bool F32>
__device__ __forceinline__ void store4(void* y, int64_t ldy, int64_t m, int64_t n, float a, float b, float c,
                                       float d) {
  if (F32) {
    float4 v = make_float4(a, b, c, d);
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + m * ldy + n) = v;
  } else {
    uint2 v;
    v.x = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
    v.y = (uint32_t)f32_to_bf16_rne(c) | ((uint32_t)f32_to_bf16_rne(d) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + m * ldy + n) = v;
  }
}

// ------------------------------------------------------------------------
// Streaming kernel for M <= 16 (decode).  The weight is read once, so the
// kernel is bound by HBM bandwidth; it spreads W over the whole chip with a
// split along K.  Grid (N/64, splits), 256 threads.  Workgroup (nb, s) owns
// rows [64 nb, 64 nb + 64) and a contiguous range of 64-wide K chunks; its four
// waves take every fourth chunk of that range, each accumulating 64 x 16 of
// Y^T with four 16-row blocks.  The waves are summed through LDS in a fixed
// order; with splits > 1 each workgroup writes a partial, and the last one to
// arrive for a row block (arrival counter) adds the partials in split order,
// so the result does not depend on scheduling.
// ------------------------------------------------------------------------
template <bool F32>
__global__ __launch_bounds__(256) void k_gemm_stream(
    const int32_t* __restrict__ tile_desc, const uint16_t* __restrict__ dense_vals,
    const uint16_t* __restrict__ sparse_vals, const uint8_t* __restrict__ sparse_meta, int tn, int tk,
    int64_t tiles_k, int64_t n, int64_t k, const uint16_t* __restrict__ x, int64_t m, int64_t ldx,
    void* __restrict__ y, int64_t ldy, int splits, float* __restrict__ ws, uint32_t* __restrict__ counters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t nb = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t chunks = k >> 6;
  const int64_t c_begin = chunks * s / splits, c_end = chunks * (s + 1) / splits;

  const int64_t n0 = nb * 64;
  const int64_t ti = n0 / tn;
  const int row0 = (int)(n0 % tn);  // first row of this block inside its tile row
  const int64_t tile_row_base = ti * tiles_k;

  const bool m_ok = r16 < m;
  const uint16_t* xrow = x + (int64_t)r16 * ldx;

  f32x4 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t c = c_begin + wave; c < c_end; c += 4) {
    const int64_t k0 = c << 6;
    const bf16x8 xb0 = m_ok ? ld8(xrow + k0 + 8 * q) : zero8();
    const bf16x8 xb1 = m_ok ? ld8(xrow + k0 + 32 + 8 * q) : zero8();
    const int32_t d = tile_desc[tile_row_base + k0 / tk];
    const int64_t slot = d >> 1;
    const int kin = (int)(k0 % tk);
    if ((d & 1) == PATCH_TILE_DENSE) {
      const uint16_t* wt = dense_vals + slot * tn * tk + kin + 8 * q;
      bf16x8 a0[4], a1[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint16_t* p = wt + (int64_t)(row0 + 16 * b + r16) * tk;
        a0[b] = ld8(p);
        a1[b] = ld8(p + 32);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[b], xb0, acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[b], xb1, acc[b], 0, 0, 0);
      }
    } else {
      const uint16_t* vt = sparse_vals + slot * tn * (tk >> 1) + (kin >> 1) + 8 * q;
      const uint8_t* mt = sparse_meta + slot * tn * (tk >> 3) + (kin >> 3) + 2 * q;
      bf16x8 a[4];
      int idx[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int row = row0 + 16 * b + r16;
        a[b] = ld8(vt + (int64_t)row * (tk >> 1));
        idx[b] = *reinterpret_cast<const uint16_t*>(mt + (int64_t)row * (tk >> 3));
      }
      const bf16x16 xb = cat16(xb0, xb1);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a[b], xb, acc[b], idx[b], 0, 0);
    }
  }

  // Sum the four waves in a fixed order: red[wave][n_local][m] in LDS.
  __shared__ float red[4][64][17];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][16 * b + 4 * q + r][r16] = acc[b][r];
  __syncthreads();

  // Thread t handles (n_local = t / 4, m quarter = t % 4 -> m = 4*(t%4) .. +3).
  const int nl = threadIdx.x >> 2, mq = (threadIdx.x & 3) * 4;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = red[0][nl][mq + j] + red[1][nl][mq + j] + red[2][nl][mq + j] + red[3][nl][mq + j];

  if (splits == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t mm = mq + j;
      if (mm < m) {
        if (F32) reinterpret_cast<float*>(y)[mm * ldy + n0 + nl] = v[j];
        else reinterpret_cast<uint16_t*>(y)[mm * ldy + n0 + nl] = f32_to_bf16_rne(v[j]);
      }
    }
    return;
  }

  // ws layout [split][16][n]; only rows m < M are written and read.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t mm = mq + j;
    if (mm < m) ws[((int64_t)s * 16 + mm) * n + n0 + nl] = v[j];
  }
  __threadfence();
  __syncthreads();
  __shared__ uint32_t s_last;
  if (threadIdx.x == 0) s_last = (atomicAdd(&counters[nb], 1u) == (uint32_t)(splits - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t mm = mq + j;
    if (mm >= m) continue;
    float acc_s = 0.f;
    for (int t = 0; t < splits; ++t) acc_s += __builtin_nontemporal_load(&ws[((int64_t)t * 16 + mm) * n + n0 + nl]);
    if (F32) reinterpret_cast<float*>(y)[mm * ldy + n0 + nl] = acc_s;
    else reinterpret_cast<uint16_t*>(y)[mm * ldy + n0 + nl] = f32_to_bf16_rne(acc_s);
  }
  if (threadIdx.x == 0) counters[nb] = 0;  // ready for the next call on this handle
}

// ------------------------------------------------------------------------
// Tiled kernel, first version: 128 x 128 block of Y^T per workgroup, four
// waves of 64 (n) x 64 (m), 32x32 MFMA shapes, operands straight from global
// memory (no LDS staging).  Correct for any M; kept as the simple baseline.
// ------------------------------------------------------------------------
template <bool F32>
__global__ __launch_bounds__(256) void k_gemm_tiled_direct(
    const int32_t* __restrict__ tile_desc, const uint16_t* __restrict__ dense_vals,
    const uint16_t* __restrict__ sparse_vals, const uint8_t* __restrict__ sparse_meta, int tn, int tk,
    int64_t tiles_k, int64_t n, int64_t k, const uint16_t* __restrict__ x, int64_t m, int64_t ldx,
    void* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 5, r32 = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * 128 + 64 * (wave >> 1);
  const int64_t m0 = (int64_t)blockIdx.y * 128 + 64 * (wave & 1);
  if (n0 >= n) return;  // N % 128 == 64: the second strip of the last block is empty
  const int64_t ti = n0 / tn;
  const int row0 = (int)(n0 % tn);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const bool mok0 = m0 + r32 < m, mok1 = m0 + 32 + r32 < m;
  const uint16_t* xr0 = x + (m0 + r32) * ldx + 8 * q;
  const uint16_t* xr1 = x + (m0 + 32 + r32) * ldx + 8 * q;

  for (int64_t k0 = 0; k0 < k; k0 += 32) {
    bf16x8 xb[2][2];
    xb[0][0] = mok0 ? ld8(xr0 + k0) : zero8();
    xb[0][1] = mok0 ? ld8(xr0 + k0 + 16) : zero8();
    xb[1][0] = mok1 ? ld8(xr1 + k0) : zero8();
    xb[1][1] = mok1 ? ld8(xr1 + k0 + 16) : zero8();
    const int32_t d = tile_desc[ti * tiles_k + k0 / tk];
    const int64_t slot = d >> 1;
    const int kin = (int)(k0 % tk);
    if ((d & 1) == PATCH_TILE_DENSE) {
      const uint16_t* wt = dense_vals + slot * tn * tk + kin + 8 * q;
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
        const uint16_t* p = wt + (int64_t)(row0 + 32 * bn + r32) * tk;
        const bf16x8 a0 = ld8(p), a1 = ld8(p + 16);
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) {
          acc[bn][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, xb[bm][0], acc[bn][bm], 0, 0, 0);
          acc[bn][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, xb[bm][1], acc[bn][bm], 0, 0, 0);
        }
      }
    } else {
      const uint16_t* vt = sparse_vals + slot * tn * (tk >> 1) + (kin >> 1) + 8 * q;
      const uint8_t* mt = sparse_meta + slot * tn * (tk >> 3) + (kin >> 3) + 2 * q;
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
        const int row = row0 + 32 * bn + r32;
        const bf16x8 a = ld8(vt + (int64_t)row * (tk >> 1));
        const int idx = *reinterpret_cast<const uint16_t*>(mt + (int64_t)row * (tk >> 3));
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
          acc[bn][bm] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, cat16(xb[bm][0], xb[bm][1]), acc[bn][bm],
                                                                  idx, 0, 0);
      }
    }
  }

#pragma unroll
  for (int bn = 0; bn < 2; ++bn)
#pragma unroll
    for (int bm = 0; bm < 2; ++bm) {
      const int64_t mm = m0 + 32 * bm + r32;
      if (mm >= m) continue;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int64_t nn = n0 + 32 * bn + 8 * rg + 4 * q;
        const f32x16& a = acc[bn][bm];
        store4<F32>(y, ldy, mm, nn, a[4 * rg], a[4 * rg + 1], a[4 * rg + 2], a[4 * rg + 3]);
      }
    }
}

template <bool F32>
__global__ void k_fill_zero_y(void* y, int64_t m, int64_t n, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m * n) return;
  const int64_t r = i / n, c = i % n;
  if (F32) reinterpret_cast<float*>(y)[r * ldy + c] = 0.f;
  else reinterpret_cast<uint16_t*>(y)[r * ldy + c] = 0;
}

}  // namespace

int stream_default_splits(const patch_weight* pw, int64_t m) {
  (void)m;
  const int64_t nblocks = pw->n / 64;
  const int64_t chunks = pw->k / 64;
  int64_t splits = (1024 + nblocks - 1) / nblocks;  // aim at ~1024 workgroups
  const int64_t max_by_k = chunks / 4 > 0 ? chunks / 4 : 1;  // keep >= 1 chunk per wave
  if (splits > max_by_k) splits = max_by_k;
  if (splits > pw->max_splits) splits = pw->max_splits;
  if (splits < 1) splits = 1;
  return (int)splits;
}

hipError_t launch_gemm_stream(const patch_weight* pw, const uint16_t* x, int64_t m, int64_t ldx, void* y,
                              int64_t ldy, int out_f32, int split_k, hipStream_t s) {
  const int64_t chunks = pw->k / 64;
  int splits = split_k > 0 ? split_k : stream_default_splits(pw, m);
  if (splits > chunks) splits = (int)chunks;
  if (splits > pw->max_splits) splits = pw->max_splits;
  if (splits < 1) splits = 1;
  dim3 grid((unsigned)(pw->n / 64), (unsigned)splits);
  if (out_f32)
    hipLaunchKernelGGL(k_gemm_stream<true>, grid, dim3(256), 0, s, pw->tile_desc, pw->dense_vals, pw->sparse_vals,
                       pw->sparse_meta, pw->tn, pw->tk, pw->tiles_k, pw->n, pw->k, x, m, ldx, y, ldy, splits, pw->ws,
                       pw->counters);
  else
    hipLaunchKernelGGL(k_gemm_stream<false>, grid, dim3(256), 0, s, pw->tile_desc, pw->dense_vals,
                       pw->sparse_vals, pw->sparse_meta, pw->tn, pw->tk, pw->tiles_k, pw->n, pw->k, x, m, ldx, y,
                       ldy, splits, pw->ws, pw->counters);
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(const patch_weight* pw, const uint16_t* x, int64_t m, int64_t ldx, void* y,
                             int64_t ldy, int out_f32, hipStream_t s) {
  dim3 grid((unsigned)((pw->n + 127) / 128), (unsigned)((m + 127) / 128));
  if (out_f32)
    hipLaunchKernelGGL(k_gemm_tiled_direct<true>, grid, dim3(256), 0, s, pw->tile_desc, pw->dense_vals,
                       pw->sparse_vals, pw->sparse_meta, pw->tn, pw->tk, pw->tiles_k, pw->n, pw->k, x, m, ldx, y, ldy);
  else
    hipLaunchKernelGGL(k_gemm_tiled_direct<false>, grid, dim3(256), 0, s, pw->tile_desc, pw->dense_vals,
                       pw->sparse_vals, pw->sparse_meta, pw->tn, pw->tk, pw->tiles_k, pw->n, pw->k, x, m, ldx, y, ldy);
  return hipGetLastError();
}

hipError_t launch_fill_zero_y(void* y, int64_t m, int64_t n, int64_t ldy, int out_f32, hipStream_t s) {
  const int64_t total = m * n;
  if (total <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (out_f32) hipLaunchKernelGGL(k_fill_zero_y<true>, dim3(grid), dim3(256), 0, s, y, m, n, ldy);
  else hipLaunchKernelGGL(k_fill_zero_y<false>, dim3(grid), dim3(256), 0, s, y, m, n, ldy);
  return hipGetLastError();
}
