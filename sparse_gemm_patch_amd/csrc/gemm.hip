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

__device__ __forceinline__ bf16x8 lo8(bf16x16 v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ __forceinline__ bf16x8 hi8(bf16x16 v) {
  return __builtin_shufflevector(v, v, 8, 9, 10, 11, 12, 13, 14, 15);
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
  const int ks = tk == 128;          // 64-wide K chunks per tile column: 1 << ks
  const int64_t ti = n0 >> (tn == 128 ? 7 : 6);
  const int row0 = (int)(n0 & (tn - 1));  // first row of this block inside its tile row
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
    const int32_t d = tile_desc[tile_row_base + (c >> ks)];
    const int64_t slot = d >> 1;
    const int kin = (int)(c & ks) << 6;
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
// Tiled kernel for prefill-sized M.
//
// Workgroup = 6 waves: 4 consumers (MFMA) and 2 producers (global -> LDS).
// The block of Y^T is 256 W rows (n) x 128 X rows (m); consumer wave w owns the
// 64 W rows of group w and all 128 columns, as 4 x 8 blocks of 16 x 16
// (128 fp32 accumulators per lane).  K advances 64 at a time; a 64-wide K step
// never crosses a tile and a 64-row group never crosses a tile row, so a
// consumer meets one tile type per step.
//
// Everything runs on smfmac 16x16x64, which issues at twice the dense MFMA
// rate: a 2:4 step is one smfmac per block with the stored 2-bit codes; a dense
// step is two, fed kept positions (0,1) and (2,3) of every group of four with
// constant codes 0x4444 and 0xEEEE.  Two of them cost what dense MFMAs over the
// same K cost, and every accumulator update is the same instruction.
//
// LDS holds a ring of 3 stages of 48 KiB:
//   X:  128 rows x 128 B; 16-byte chunk c of row r at position c ^ h(r),
//       h(r) = (r & 7) ^ ((r >> 3) & 1)
//   W:  four 64-row groups of 8 KiB, each in its tile's own format:
//       dense  64 rows x 128 B, chunk c at c ^ h(r)
//       2:4    64 rows x 64 B of kept values, chunk c at c ^ (((r >> 1) ^ (r >> 3)) & 3),
//              then 64 rows x 8 B of 2-bit codes at +4 KiB
// The swizzles keep the 16-byte reads of 16 consecutive lanes (16 consecutive
// rows, one logical chunk) on distinct banks whether the LDS serves 128 or
// 256 bytes per clock.
//
// Producers load with global_load_lds_dwordx4 (lane i of a wave writes bytes
// 16 i .. 16 i + 15 of a 1 KiB LDS block, so a lane fetches the global chunk
// that belongs at its LDS position; 8 lanes still cover one 128-byte row
// segment).  Producer p loads the steps with parity p, two steps ahead, and
// waits for its own loads only before the barrier at which they are consumed.
// Consumers issue no global->LDS loads, so none of their LDS reads waits on one.
// Every wave passes exactly one barrier per step.
// ------------------------------------------------------------------------
namespace tiled {
constexpr int BN = 256, BM = 128, BK = 64;
constexpr int X_BYTES = BM * 128;          // 16 KiB
constexpr int G_BYTES = 64 * 128;          // 8 KiB per 64-row W group
constexpr int STAGE_BYTES = X_BYTES + 4 * G_BYTES;
constexpr int STAGES = 3;
constexpr int CONSUMERS = 4, PRODUCERS = 2;
constexpr int GROUP_N = 4;  // block columns per group of the block order
constexpr int THREADS = 64 * (CONSUMERS + PRODUCERS);
}  // namespace tiled

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void g2l16(const void* src, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 16, 0, 0);
}
__device__ __forceinline__ void g2l4(const void* src, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 4, 0, 0);
}
__device__ __forceinline__ bf16x8 lds8(const uint8_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Workgroup barrier without the implied memory fences: the producers wait for
// their own loads explicitly, and the "memory" clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Output block of this workgroup.  The dispatcher deals workgroup i to XCD
// i % 8; renumbering so that each XCD owns a contiguous range of blocks, walked
// in groups of GROUP_N block columns (m fastest inside a group), makes the
// ~32 workgroups resident on one XCD cover about 4 x 8 blocks and share their W
// and X slabs in that XCD's L2.
__device__ __forceinline__ void block_origin(int64_t n, int64_t m, int64_t& n0, int64_t& m0) {
  using namespace tiled;
  const int nbn = (int)((n + BN - 1) / BN), nbm = (int)((m + BM - 1) / BM);
  const int total = nbn * nbm;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3, base = total >> 3, rem = total & 7;
  const int id = xcd < rem ? xcd * (base + 1) + local : rem * (base + 1) + (xcd - rem) * base + local;
  const int per_group = GROUP_N * nbm;
  const int group = id / per_group, in_group = id % per_group;
  const int first = group * GROUP_N;
  const int width = nbn - first < GROUP_N ? nbn - first : GROUP_N;
  n0 = (int64_t)(first + in_group % width) * BN;
  m0 = (int64_t)(in_group / width) * BM;
}

template <bool F32>
__global__ __launch_bounds__(tiled::THREADS, 1) void k_gemm_tiled(
    const int32_t* __restrict__ tile_desc, const uint16_t* __restrict__ dense_vals,
    const uint16_t* __restrict__ sparse_vals, const uint8_t* __restrict__ sparse_meta, int tn, int tk,
    int64_t tiles_k, int64_t n, int64_t k, const uint16_t* __restrict__ x, int64_t m, int64_t ldx,
    void* __restrict__ y, int64_t ldy) {
  using namespace tiled;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t n0, m0;
  block_origin(n, m, n0, m0);
  const int nsteps = (int)(k / BK);
  const int ks = tk == 128;           // 64-wide K steps per tile column: 1 << ks
  const int ns = tn == 128 ? 7 : 6;   // log2(TN)

  if (wave >= CONSUMERS) {
    // ------------------------------ producer ------------------------------
    // Per-lane byte offsets are fixed for the whole K loop; each step only moves
    // the uniform base pointers (tile slot and K position), so every load is a
    // scalar-base + 32-bit-offset global_load_lds with no per-step vector math.
    const int p = wave - CONSUMERS;
    const int lrow8 = lane >> 3;   // row within a 1 KiB block of 128-byte rows
    const int lpos8 = lane & 7;    // 16-byte position within the row
    uint32_t xoff[BM / 8];
#pragma unroll
    for (int j = 0; j < BM / 8; ++j) {
      const int row = 8 * j + lrow8;
      int64_t gm = m0 + row;
      if (gm > m - 1) gm = m - 1;  // rows past M only feed Y rows that are never stored
      xoff[j] = (uint32_t)((gm - m0) * ldx * 2) + 16u * (uint32_t)(lpos8 ^ swz8(row));
    }
    uint32_t doff[8], soff[4], moff[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 8 * j + lrow8;
      doff[j] = 2u * (uint32_t)(row * tk + 8 * (lpos8 ^ swz8(row)));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // 16 rows of 64 bytes per 1 KiB block
      const int row = 16 * j + (lane >> 2);
      soff[j] = 2u * (uint32_t)(row * (tk >> 1) + 8 * ((lane & 3) ^ swz4(row)));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // 32 rows of 8 bytes per 256 B block, 4 bytes per lane
      const int row = 32 * j + (lane >> 1);
      moff[j] = (uint32_t)(row * (tk >> 3) + 4 * (lane & 1));
    }
    const uint8_t* xbase = reinterpret_cast<const uint8_t*>(x + m0 * ldx);
    auto load_step = [&](int step) {
      uint8_t* st = lds + (step % STAGES) * STAGE_BYTES;
      const uint8_t* xb = xbase + (int64_t)step * BK * 2;
#pragma unroll
      for (int j = 0; j < BM / 8; ++j) g2l16(xb + xoff[j], st + 1024 * j);
      const int kin = (step & ks) << 6;
#pragma unroll 1
      for (int grp = 0; grp < 4; ++grp) {
        const int64_t gn0 = n0 + 64 * grp;
        if (gn0 >= n) break;
        const int32_t d = tile_desc[(gn0 >> ns) * tiles_k + (step >> ks)];
        const int64_t slot = d >> 1;
        const int64_t r0 = gn0 & (tn - 1);
        uint8_t* g = st + X_BYTES + grp * G_BYTES;
        if ((d & 1) == PATCH_TILE_DENSE) {
          const uint8_t* src = reinterpret_cast<const uint8_t*>(dense_vals + slot * tn * tk + r0 * tk + kin);
#pragma unroll
          for (int j = 0; j < 8; ++j) g2l16(src + doff[j], g + 1024 * j);
        } else {
          const uint8_t* src =
              reinterpret_cast<const uint8_t*>(sparse_vals + slot * tn * (tk >> 1) + r0 * (tk >> 1) + (kin >> 1));
#pragma unroll
          for (int j = 0; j < 4; ++j) g2l16(src + soff[j], g + 1024 * j);
          const uint8_t* msrc = sparse_meta + slot * tn * (tk >> 3) + r0 * (tk >> 3) + (kin >> 3);
#pragma unroll
          for (int j = 0; j < 2; ++j) g2l4(msrc + moff[j], g + 4096 + 256 * j);
        }
      }
    };
    if (p < nsteps) load_step(p);
    for (int i = 0; i < nsteps; ++i) {
      if ((i & 1) == p) wait_loads();  // step i is mine: it must have landed
      wg_barrier();
      if (i + 2 < nsteps && ((i + 2) & 1) == p) load_step(i + 2);  // into the stage step i - 1 used
    }
    return;
  }

  // ------------------------------ consumer ------------------------------
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t gn0 = n0 + 64 * wave;
  const bool group_ok = gn0 < n;
  const int64_t desc_row = (gn0 >> ns) * tiles_k;

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < nsteps; ++i) {
    wg_barrier();  // step i has landed; step i - 1's stage may now be refilled
    if (!group_ok) continue;
    const uint8_t* cur = lds + (i % STAGES) * STAGE_BYTES;
    const uint8_t* g = cur + X_BYTES + wave * G_BYTES;
    const bool dense = (tile_desc[desc_row + (i >> ks)] & 1) == PATCH_TILE_DENSE;
    // W operands of the 4 row blocks: a lane covers dense k = 16q .. 16q + 15 of the step
    bf16x8 a0[4], a1[4];
    int i0[4];
    if (dense) {
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
        const int r = 16 * bn + r16;
        // 32 contiguous bytes: dword 2g = positions (0,1) of group g, dword 2g + 1 = (2,3)
        const uint4 lo = *reinterpret_cast<const uint4*>(g + r * 128 + (((2 * q) ^ swz8(r)) << 4));
        const uint4 hi = *reinterpret_cast<const uint4*>(g + r * 128 + (((2 * q + 1) ^ swz8(r)) << 4));
        const uint4 e = make_uint4(lo.x, lo.z, hi.x, hi.z), o = make_uint4(lo.y, lo.w, hi.y, hi.w);
        a0[bn] = *reinterpret_cast<const bf16x8*>(&e);
        a1[bn] = *reinterpret_cast<const bf16x8*>(&o);
        i0[bn] = 0x4444;  // kept positions 0 and 1 of every group
      }
    } else {
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
        const int r = 16 * bn + r16;
        a0[bn] = lds8(g + r * 64 + ((q ^ swz4(r)) << 4));
        i0[bn] = *reinterpret_cast<const uint16_t*>(g + 4096 + r * 8 + 2 * q);
      }
    }
    // X operands streamed per 16-column block: k = 8q .. (regs 0-7) and 32 + 8q .. (regs 8-15)
#pragma unroll
    for (int bm = 0; bm < 8; ++bm) {
      const int r = 16 * bm + r16;
      const bf16x16 b = cat16(lds8(cur + r * 128 + ((q ^ swz8(r)) << 4)),
                              lds8(cur + r * 128 + (((4 + q) ^ swz8(r)) << 4)));
#pragma unroll
      for (int bn = 0; bn < 4; ++bn)
        acc[bn][bm] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a0[bn], b, acc[bn][bm], i0[bn], 0, 0);
      if (dense) {
#pragma unroll
        for (int bn = 0; bn < 4; ++bn)  // kept positions 2 and 3 of every group
          acc[bn][bm] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a1[bn], b, acc[bn][bm], 0xEEEE, 0, 0);
      }
    }
  }

  // epilogue: per block, lane holds rows n = 4 q + (0..3) of column m = r16
  if (!group_ok) return;
#pragma unroll
  for (int bm = 0; bm < 8; ++bm) {
    const int64_t mm = m0 + 16 * bm + r16;
    if (mm >= m) continue;
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const f32x4 v = acc[bn][bm];
      store4<F32>(y, ldy, mm, gn0 + 16 * bn + 4 * q, v[0], v[1], v[2], v[3]);
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
  constexpr int lds_bytes = tiled::STAGES * tiled::STAGE_BYTES;  // 144 KiB: opt in above 64 KiB, once
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_tiled<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_tiled<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)(((pw->n + tiled::BN - 1) / tiled::BN) * ((m + tiled::BM - 1) / tiled::BM)));
  if (out_f32)
    hipLaunchKernelGGL(k_gemm_tiled<true>, grid, dim3(tiled::THREADS), lds_bytes, s, pw->tile_desc, pw->dense_vals,
                       pw->sparse_vals, pw->sparse_meta, pw->tn, pw->tk, pw->tiles_k, pw->n, pw->k, x, m, ldx, y, ldy);
  else
    hipLaunchKernelGGL(k_gemm_tiled<false>, grid, dim3(tiled::THREADS), lds_bytes, s, pw->tile_desc, pw->dense_vals,
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
