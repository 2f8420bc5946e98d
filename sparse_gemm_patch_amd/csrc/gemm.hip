// Hybrid dense / 2:4 tile GEMM:  Y[m][n] = sum_k X[m][k] * Wm[n][k].
//
// Every TN x TK tile of W is dense or 2:4 along K ("PATCH: Learnable
// Tile-level Hybrid Sparsity for LLMs", Abstract; tile sizes from model card
// "llama_3.2_1b-PATCH-45Sparse", "Training hyper-parameters").  W is the A
// operand of smfmac 16x16x64 (the gfx950 sparse MFMA takes its 2:4 operand
// there); X rows are the B operand; each wave accumulates blocks of Y^T in fp32
// and the epilogue writes Y[m][n].
//
// smfmac 16x16x64 bf16 on gfx950 (lane l = 16 q + r, register j):
//   A: row r, the 8 kept values of dense k = 16 q .. 16 q + 15 (two per group of
//      four); the 2-bit position of value j is bits [2j+1:2j] of the index VGPR
//   B: column r, k = 8 q + j (j < 8) and 32 + 8 q + j - 8 (j >= 8)
//   C: row 4 q + i (i = 0..3), column r
// smfmac issues at twice the dense MFMA rate, so a dense 64-wide K step is run
// as two smfmacs, fed kept positions (0,1) and (2,3) of every group of four
// with the constant index words 0x4444 and 0xEEEE; that costs what the dense
// MFMAs over the same K cost, and one instruction serves both tile types.
// The packed pools are stored in this operand order (see pack.hip), so a
// lane's A operand is one 16-byte load and a wave's is 1 KiB contiguous.
#include "patch_internal.h"

#include <atomic>
#include <climits>
#include <cstdio>
#include <cstdlib>

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

// global -> LDS copy of 16 (or 4) bytes per lane from base + off (base
// wave-uniform, off a 32-bit per-lane byte offset); lane i writes LDS bytes
// lds_addr + 16 i (4 i).  lds_addr must be wave-uniform.  A scalar base keeps
// one VGPR per copy stream instead of a 64-bit address.  The LDS address goes
// in M0, which the asm declares clobbered (the compiler sets it again where it
// needs it) instead of saving and restoring it around every copy.
__device__ __forceinline__ bf16x8 lds8(const uint8_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               : : "s"(lds_addr), "v"(off), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               : : "s"(lds_addr), "v"(off), "s"(base) : "memory", "m0");
}
// The same copy with M0 saved and restored around it: three more scalar
// instructions per copy.  k_gemm_tiled issues its X and dense-tile copies this
// way: issued back to back with one M0 write each, they made all-dense steps
// 4-8% slower (the 8192 x 2048 product at M = 4096, the 13824 x 5120 one at
// M = 2048), with no gain on 2:4 steps; spread out, a wave reaches a full fill
// queue later.
__device__ __forceinline__ void dma16_paced(const void* base, uint32_t off, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds_addr), "v"(off), "s"(base) : "memory");
}
// A run of copies that share one M0: the instruction's immediate offset moves
// the global and the LDS address alike, so consecutive 1 KiB blocks of a pool
// need one M0 write between them.  set_m0 must precede the first dma*_at of
// the run, with no other copy in between.
__device__ __forceinline__ void set_m0(uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" : : "s"(lds_addr) : "memory", "m0");
}
template <int IMM>
__device__ __forceinline__ void dma16_at(const void* base, uint32_t off) {
  static_assert(IMM >= 0 && IMM < 4096, "immediate offset range");
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" : : "v"(off), "s"(base), "i"(IMM) : "memory", "m0");
}
template <int IMM>
__device__ __forceinline__ void dma4_at(const void* base, uint32_t off) {
  static_assert(IMM >= 0 && IMM < 4096, "immediate offset range");
  asm volatile("global_load_lds_dword %0, %1 offset:%2" : : "v"(off), "s"(base), "i"(IMM) : "memory", "m0");
}
// ------------------------------------------------------------------------
// Streaming kernel for small M (decode, and batches up to 16 MB rows).
//
// The weight is read once, so this kernel is bound by HBM bandwidth.  One
// workgroup of WAVES waves per NBLK 16-row blocks of W (grid N / (16 NBLK)):
// the waves take every WAVES-th 64-wide K chunk, each keeping NBLK x MB
// 16 x 16 accumulator blocks of Y^T (MB = one per 16 rows of X), and are
// summed through LDS in a fixed order.  No workgroup depends on another (a
// cross-workgroup reduction would need device-scope fences, which write back
// a whole XCD's L2 on this chip).  Per chunk a wave loads its A operands once
// (1 KiB of 2:4 values or 2 KiB of dense positions per W block, contiguous,
// with non-temporal loads) and copies the MB x 16 X rows into its own LDS
// slot (two global_load_lds copies of 8 rows x 128 bytes per X block; rows
// past M repeat row M - 1), BATCH chunks at a time; every A operand then
// meets every X block.  MB = 1 serves decode (M <= 16).
//
// Every workgroup copies all of X, so NBLK divides that traffic and MB
// multiplies it; NBLK also divides the grid, and a grid of fewer than about
// 160 workgroups leaves the chip's fetch latency exposed (stream_w_blocks).
// ------------------------------------------------------------------------
namespace streamk {
// the decode instance with one W block per workgroup
constexpr int WAVES = 16;
constexpr int BATCH = 2;  // chunks per wave in flight together (1: 7-20% slower; 4: up to 19% slower, one workgroup per CU)
}  // namespace streamk

// The product a workgroup belongs to (a short scalar scan over the group) and
// the workgroup's index inside it; -1 for padding.
__device__ __forceinline__ int find_problem(const gemm_group& g, int bid, int& local) {
  for (int i = 0; i < g.count; ++i) {
    const int b0 = g.p[i].block0;
    if (bid >= b0 && bid < b0 + g.p[i].blocks) {
      local = bid - b0;
      return i;
    }
  }
  return -1;
}

template <bool F32, int MB, int NBLK, int WAVES, int BATCH, int SPLIT>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_stream(const gemm_group g) {
  static_assert(MB >= 1 && MB <= 8, "X blocks per wave");
  static_assert(SPLIT == 1 || SPLIT == 2 || SPLIT == 4, "workgroups per W block's K range");
  static_assert(NBLK == 1 || NBLK == 2 || NBLK == 4, "16-row W blocks per workgroup");
  int local;
  const int pi = find_problem(g, blockIdx.x, local);
  if (pi < 0) return;
  const gemm_problem& P = g.p[pi];
  const int32_t* __restrict__ tile_desc = P.tile_desc;
  const uint16_t* __restrict__ dense_vals = P.dense_vals;
  const uint16_t* __restrict__ sparse_vals = P.sparse_vals;
  const uint8_t* __restrict__ sparse_meta = P.sparse_meta;
  const int tn = P.tn, tk = P.tk;
  const int64_t tiles_k = P.tiles_k, k = P.k, m = P.m, ldx = P.ldx, ldy = P.ldy;
  const uint16_t* __restrict__ x = P.x;
  void* __restrict__ y = P.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  // Blocks of 16 NBLK W rows in XCD-contiguous order (workgroup i runs on XCD
  // i % 8 and each product starts on a multiple of 8): the 16-row blocks that
  // share a 512-byte group of 2:4 codes run on one XCD and read the codes from
  // its L2 once; dealt round-robin, every XCD fetched them from memory.  A
  // block's NBLK 16-row blocks lie in one tile (16 NBLK divides TN), so they
  // share each chunk's tile descriptor and code group.
  // With a K split, the SPLIT workgroups of one W block are consecutive in
  // this order (one XCD), share s taking chunks [C s / SPLIT, C (s + 1) /
  // SPLIT).  SPLIT is a template argument: computed at run time, this
  // arithmetic sits before every workgroup's first descriptor load and cost
  // the unsplit decode launches 0.1-0.5 us.
  constexpr int LG = SPLIT == 4 ? 2 : SPLIT == 2 ? 1 : 0;
  const int nb = P.blocks, xcd = local & 7, base_b = nb >> 3, rem_b = nb & 7;
  const int pos = xcd * base_b + (xcd < rem_b ? xcd : rem_b) + (local >> 3);
  const int share = pos & (SPLIT - 1);
  const int64_t n0 = (int64_t)(pos >> LG) * (16 * NBLK);
  const int64_t first_chunk = ((k >> 6) * share) >> LG;
  const int64_t chunks = ((k >> 6) * (share + 1)) >> LG;  // one past this workgroup's last chunk
  const int ks = tk == 128;                      // 64-wide K chunks per tile column: 1 << ks
  const int ns = tn == 128 ? 7 : 6;              // log2(TN)
  const int64_t desc_row = (n0 >> ns) * tiles_k;
  const int blk = (int)((n0 & (tn - 1)) >> 4);   // first 16-row block of this block inside its tile
  const int bt = tn >> 4;

  // X goes through LDS: per chunk and X block two copies of 8 rows x 128
  // bytes (whole lines), 16-byte chunk c of row r at position c ^ (r & 7),
  // into this wave's slot of the batch; rows past M repeat row M - 1 (they
  // only feed Y rows that are never stored).  Read straight into the B
  // operand, every load touched 16 rows x 64 bytes.
  constexpr int SLOT = MB * 2048;  // one chunk's X blocks
  __shared__ __attribute__((aligned(1024))) uint8_t smem[WAVES * BATCH * SLOT];
  const uint32_t slot0 = (uint32_t)(uintptr_t)smem + (uint32_t)(wave * BATCH * SLOT);
  uint32_t xoff[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * mb + 8 * h + (lane >> 3);
      const int64_t rc = row < m ? row : m - 1;
      xoff[mb][h] = (uint32_t)((rc * ldx + 8 * ((lane & 7) ^ (row & 7))) * 2);
    }
  const uint8_t* dbase = reinterpret_cast<const uint8_t*>(dense_vals) + lane * 16;
  const uint8_t* sbase = reinterpret_cast<const uint8_t*>(sparse_vals) + lane * 16;
  const uint8_t* mbase = sparse_meta + lane * 8;

  f32x4 acc[NBLK][MB];
#pragma unroll
  for (int b = 0; b < NBLK; ++b)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[b][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // This wave's chunks are c = wave + WAVES j.  Their tile descriptors arrive
  // with one load (lane j holds chunk j's), so that the operand loads of a
  // batch of chunks can be issued back to back before their MFMAs.
  for (int64_t base = first_chunk + wave; base < chunks; base += (int64_t)WAVES * 64) {
    const int nj = (int)min((int64_t)64, (chunks - base + WAVES - 1) / WAVES);
    const int64_t cl = base + (int64_t)WAVES * lane;
    const int32_t dl = lane < nj ? tile_desc[desc_row + (cl >> ks)] : 0;
    for (int j = 0; j < nj; j += BATCH) {
      // BATCH chunks, past the last one clamped to it (loaded, not used): every
      // chunk issues the same loads whatever its tile type, so the waits the
      // compiler places stay exact.
      int32_t d[BATCH];
#pragma unroll
      for (int t = 0; t < BATCH; ++t) d[t] = __builtin_amdgcn_readlane(dl, min(j + t, nj - 1));
      bf16x8 a0[BATCH][NBLK];
      u32x4 w2[BATCH][NBLK];
#pragma unroll
      for (int t = 0; t < BATCH; ++t) {
        const int64_t c = base + (int64_t)WAVES * min(j + t, nj - 1);
        const uint16_t* xc = x + (c << 6);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          dma16(xc, xoff[mb][0], slot0 + t * SLOT + mb * 2048);
          dma16(xc, xoff[mb][1], slot0 + t * SLOT + mb * 2048 + 1024);
        }
        const int64_t slot = d[t] >> 1;
        const int64_t u = (c & ks) * bt + blk;  // operand unit of the first 16-row block and this chunk
        const bool dn = (d[t] & 1) == PATCH_TILE_DENSE;
        const uint8_t* dw = dbase + (slot * tn * tk + u * 1024) * 2;
        const uint8_t* sw = sbase + slot * tn * tk + u * 1024;
        const uint8_t* cw = mbase + slot * tn * (tk >> 3) + (u >> 2) * 512;  // lane's 8 bytes of codes (all NBLK blocks)
        // W is read once: non-temporal loads keep it from displacing X in the caches
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
          a0[t][b] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                                                    reinterpret_cast<const u32x4*>(dn ? dw + 2048 * b : sw + 1024 * b)));
          w2[t][b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dn ? dw + 2048 * b + 1024 : cw));
        }
      }
      // the X copies are not loads the compiler knows of: wait for them here
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int t = 0; t < BATCH; ++t) {
        if (j + t >= nj) continue;
        const int64_t c = base + (int64_t)WAVES * (j + t);
        const int u0 = (int)((c & ks) * bt + blk);
        const bool dn = (d[t] & 1) == PATCH_TILE_DENSE;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint8_t* sl = smem + (wave * BATCH + t) * SLOT + mb * 2048 + r16 * 128;
          const bf16x16 xb = cat16(lds8(sl + ((q ^ (r16 & 7)) << 4)), lds8(sl + (((4 + q) ^ (r16 & 7)) << 4)));
#pragma unroll
          for (int b = 0; b < NBLK; ++b) {
            const int ub = (u0 + b) & 3;  // block within its 4-block code group
            const uint32_t word = ub < 2 ? w2[t][0].x : w2[t][0].y;  // codes of blocks (0,1) or (2,3)
            if (dn) {
              acc[b][mb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a0[t][b], xb, acc[b][mb], 0x4444, 0, 0);
              acc[b][mb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, w2[t][b]), xb,
                                                                     acc[b][mb], 0xEEEE, 0, 0);
            } else {
              acc[b][mb] = ub & 1 ? __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a0[t][b], xb, acc[b][mb], (int)word, 0, 1)
                                  : __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a0[t][b], xb, acc[b][mb], (int)word, 0, 0);
            }
          }
        }
      }
    }
  }

  // Sum the waves in a fixed order, one 16-row W block at a time: lane holds
  // rows 4 q + i of column m = r16 of each X block.  The X slots are free once
  // every wave is past its last chunk.
  static_assert(WAVES * MB * 16 * 17 * 4 <= WAVES * BATCH * SLOT, "reduction fits the X slots");
  float(*red)[MB][16][17] = reinterpret_cast<float(*)[MB][16][17]>(smem);
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][mb][4 * q + i][r16] = acc[b][mb][i];
    __syncthreads();
    for (int o = threadIdx.x; o < 256 * MB; o += 64 * WAVES) {
      const int mb = o >> 8, nl = (o >> 4) & 15, mm = 16 * mb + (o & 15);
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) v += red[w][mb][nl][o & 15];
      if (mm < m) {
        const int64_t col = n0 + 16 * b + nl;
        if constexpr (SPLIT > 1) P.part[(share * m + mm) * P.n + col] = v;
        else if (F32) reinterpret_cast<float*>(y)[mm * ldy + col] = v;
        else reinterpret_cast<uint16_t*>(y)[mm * ldy + col] = f32_to_bf16_rne(v);
      }
    }
  }
}

// ------------------------------------------------------------------------
// Tiled kernel for prefill-sized M: 256 or 192 X rows per block, and 64 when
// two workgroups share each CU (other 128- and 64-row blocks run on k_gemm_ws
// below).  192-row blocks fill the chip where 256-row ones leave many CUs
// idle and 128-row ones leave a ragged second round (5120-wide products at
// M = 2048: 220 against 160 or 320 workgroups, 11% faster).
//
// Workgroup = 8 waves in a 2 x 4 grid; the block of Y^T is 256 W rows (n) x
// BM X rows (m).  Wave (wn, wm) owns W rows 128 wn .. +127 (8 row blocks of
// 16, in two 64-row groups that each lie in one tile row) and X rows
// BM/4 wm .. +BM/4-1 (BM/64 column blocks): up to 8 x 4 accumulator blocks of
// 16 x 16, 128 fp32 accumulators per lane, two waves per SIMD.  K advances 64
// at a time; a step never crosses a tile.  The smaller blocks exist for
// shapes whose 256 x 256 blocks would leave CUs idle: no block is split along
// K (a cross-workgroup reduction needs device-scope fences, which on this chip
// write back the whole L2 of an XCD).
//
// Per 256 x 256 step a CU copies 50 KiB (2:4) to 64 KiB (dense) into LDS,
// its waves read 136 to 192 KiB back, and each SIMD runs 64 (2:4) to 128
// (dense) smfmacs.  Measured on MI355X: the global -> LDS copies move 40-48
// bytes per clock per CU while they are issued, without ever filling the
// fill-path FIFOs (hardware counters), so a copy phase is set by the copy
// instructions and the scalar instructions around them (M0 writes, address
// arithmetic; scalar issue takes about 16% of the waves' cycles); LDS operand
// reads run at 128 bytes per clock with one reading wave per SIMD and about
// 165 with two; an smfmac takes 17-19 clocks.  So a 90% 2:4 step needs about
// 1 150 clocks of copy issue, 850 of LDS reads and 1 380 of matrix work per
// SIMD, and the schedule decides how much of that overlaps (in-kernel
// timestamps: about 2 550-2 650 clocks per step at 256 rows).
//
// LDS holds two stages of BM * 128 + 32 KiB:
//   X  BM rows x 128 B; 16-byte chunk c of row r at position c ^ (r & 7), so
//      that the B-operand reads (16 rows, one chunk per 16 lanes) are free of
//      bank conflicts; without the swizzle they run at a quarter of the rate.
//   W  four 64-row groups of 8 KiB.  A group's operands for one step are
//      contiguous in the operand-order pools and are copied verbatim: dense 4
//      blocks x [a0 | a1] x 1 KiB; 2:4 4 blocks x 1 KiB of values, then 512 B
//      of codes at +4 KiB, 8 bytes per lane (one code word per block).  Lane l
//      reads bytes 16 l .. 16 l + 15 of a block (or 8 l .. 8 l + 7 of the
//      codes): consecutive lanes, consecutive addresses.
// Every wave copies an eighth of the next step (BM/8 X rows and half of one W
// group) straight from global memory into LDS with global_load_lds.  The two
// waves of a SIMD run half a step apart: waves 0-3 copy, read and multiply
// step i; waves 4-7 multiply step i - 1 (read at the end of the previous
// step), then copy and read step i, so that one wave of each SIMD keeps the
// matrix unit busy while the other issues copies or waits for LDS reads.  Against
// four dedicated copy waves that copy the whole step before multiplying their
// own share this is 2-5% faster on the 256-row products (timestamps: the copy
// waves spent about 1 000 clocks issuing before their first smfmac).  Measured
// and dropped: the lagging waves copying before they multiply (13% slower:
// both waves of a SIMD are then busy with copies at once), copies interleaved
// between the smfmacs (35-40% slower), and three X stages with X copied two
// steps ahead (160 KiB of LDS, 9% slower).  The copies are issued from inline assembly: the compiler
// cannot tell that they target the other stage, and as builtins every LDS read
// after them would wait for them to land.  The two 1 KiB value blocks of a 2:4
// group share one write of M0 (the LDS address register) through the
// instruction's immediate offset: with about 40% fewer scalar instructions per
// step the 2:4-heavy products run 2-4% faster.  X and dense-tile copies keep
// one M0 write per copy, with M0 saved and restored (see dma16_paced).  Its only other vector-memory loads are the
// descriptor windows, waited for where they are loaded, so the explicit waits
// are the only ones these copies need.
// ------------------------------------------------------------------------
namespace tiled {
constexpr int BN = 256, BK = 64;
constexpr int G_BYTES = 64 * 128;          // 8 KiB per 64-row W group
constexpr int STAGES = 2;
template <int BM> constexpr int x_bytes() { return BM * 128; }
template <int BM> constexpr int stage_bytes() { return x_bytes<BM>() + 4 * G_BYTES; }
}  // namespace tiled

// Wait for this wave's copies and LDS reads, then synchronise the workgroup.
__device__ __forceinline__ void step_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ int xswz(int r) { return r & 7; }

// Output block of this workgroup (W rows from n_begin on).  The dispatcher deals workgroup i to XCD
// i % 8; renumbering so that each XCD owns a contiguous range of blocks, walked
// in groups of group_n block columns (m fastest inside a group), makes the
// workgroups resident on one XCD cover a compact region and share their W and
// X in that XCD's L2 (group_n is chosen by the launch, see group_width).
// bid: the workgroup's index inside its product, whose first workgroup is a
// multiple of 8 in the launch (so bid % 8 is still its XCD).
template <int BM, int BN>
__device__ __forceinline__ void block_origin(int64_t n_begin, int64_t n, int64_t m, int bid, int group_n,
                                             int64_t& n0, int64_t& m0) {
  const int nbn = (int)((n - n_begin + BN - 1) / BN), nbm = (int)((m + BM - 1) / BM);
  const int total = nbn * nbm;
  const int xcd = bid & 7, local = bid >> 3, base = total >> 3, rem = total & 7;
  const int id = xcd < rem ? xcd * (base + 1) + local : rem * (base + 1) + (xcd - rem) * base + local;
  const int per_group = group_n * nbm;
  const int group = id / per_group, in_group = id % per_group;
  const int first = group * group_n;
  const int width = nbn - first < group_n ? nbn - first : group_n;
  n0 = n_begin + (int64_t)(first + in_group % width) * BN;
  m0 = (int64_t)(in_group / width) * BM;
}

// Tile descriptors seen through the constant address space: nothing writes the
// packed weight while a GEMM runs, and saying so lets the wave-uniform reads go
// through the scalar cache (a pointer taken from a kernel-argument array is
// otherwise assumed to alias Y, which forces vector loads).
typedef const __attribute__((address_space(4))) int32_t* const_desc_ptr;

// A window of 64 tile columns of one tile row's descriptors, lane j holding
// column 64 win + j (0 past the row).  k_gemm_tiled keeps the window in a
// register and takes a step's descriptor with readlane (copies) or a bit of a
// ballot mask (dense or 2:4, for the smfmacs) instead of a scalar load per
// step: 2-3% faster at 256 rows.  In k_gemm_ws, whose copy waves run two
// steps ahead and whose computing waves overlap each other, the scalar loads'
// latency is already hidden and the window only costs registers.
__device__ __forceinline__ int32_t desc_window(const_desc_ptr tile_desc, int64_t row_base, int64_t tiles_k, int win,
                                               int lane) {
  const int64_t c = (int64_t)win * 64 + lane;
  return c < tiles_k ? tile_desc[row_base + c] : 0;
}

// Epilogue of a computing wave: its block of Y^T, W rows wrow0 .. +64 GW - 1
// (GW 64-row groups) by X rows mrow0 .. +RW-1, where lane (q, r16) of
// accumulator block (bn, bm) holds rows n = 16 bn + 4 q .. +3 of column
// m = 16 bm + r16.  For bf16 Y each group goes through `region` (RW x 128 bytes of LDS that no
// other wave touches; 16-byte chunk c of row r at position c ^ (r & 7)) and
// leaves as 16-byte non-temporal stores, eight whole 128-byte row segments of
// Y per instruction.  Written straight from the accumulators, each store
// would cover 16 rows x 32 bytes: on the 8192 x 2048 product at M = 4096 that
// costs 5% more, and as non-temporal stores twice the kernel time.  Whole
// lines stored non-temporally stream out while other workgroups compute
// (2-8% faster than ordinary stores of the same lines).  fp32 Y is stored
// directly (16 bytes per lane).
template <bool F32, int RW, int XB, int GW>
__device__ __forceinline__ void store_block(const f32x4 (&acc)[4 * GW][XB], uint8_t* region, void* __restrict__ y,
                                            int64_t ldy, int64_t m, int64_t mrow0, int64_t wrow0,
                                            const bool (&hok)[GW], int lane) {
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    if (!hok[h]) continue;
    if (F32) {
#pragma unroll
      for (int bm = 0; bm < XB; ++bm) {
        const int64_t mm = mrow0 + 16 * bm + r16;
        if (mm >= m) continue;
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const f32x4 v = acc[4 * h + b4][bm];
          store4<true>(y, ldy, mm, wrow0 + 64 * h + 16 * b4 + 4 * q, v[0], v[1], v[2], v[3]);
        }
      }
      continue;
    }
#pragma unroll
    for (int bm = 0; bm < XB; ++bm)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const f32x4 v = acc[4 * h + b4][bm];
        const int r = 16 * bm + r16, c = 2 * b4 + (q >> 1);
        uint2 w;
        w.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        w.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<uint2*>(region + r * 128 + ((c ^ (r & 7)) << 4) + ((q & 1) << 3)) = w;
      }
#pragma unroll
    for (int j = 0; j < RW / 8; ++j) {
      const int r = 8 * j + (lane >> 3), c = lane & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(region + r * 128 + ((c ^ (r & 7)) << 4));
      const int64_t mm = mrow0 + r;
      if (mm < m)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + mm * ldy + wrow0 + 64 * h + 8 * c));
    }
  }
}

// One output block of k_gemm_tiled: block `local` of entry P of the launch.
template <bool F32, int BM>
__device__ __forceinline__ void tiled_block(const gemm_problem& P, int local) {
  using namespace tiled;
  const const_desc_ptr tile_desc = (const_desc_ptr)P.tile_desc;
  const uint16_t* __restrict__ dense_vals = P.dense_vals;
  const uint16_t* __restrict__ sparse_vals = P.sparse_vals;
  const uint8_t* __restrict__ sparse_meta = P.sparse_meta;
  const int tn = P.tn, tk = P.tk;
  const int64_t tiles_k = P.tiles_k, n = P.n, k = P.k, m = P.m, ldx = P.ldx, ldy = P.ldy;
  const uint16_t* __restrict__ x = P.x;
  void* __restrict__ y = P.y;
  constexpr int XB = BM / 64;                        // X blocks of 16 rows per wave
  constexpr int X_BYTES = x_bytes<BM>(), STAGE_BYTES = stage_bytes<BM>();
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // Opaque per block, so that the compiler recomputes the lane-dependent
  // offsets for every block instead of holding them across the block loop.
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 2, wm = wave & 3;
  const int q = lane >> 4, r16 = lane & 15;
  int64_t n0, m0;
  block_origin<BM, BN>(P.n_begin, n, m, local, P.group_n, n0, m0);
  const int nsteps = (int)(k / BK);
  const int ks = tk == 128;           // 64-wide K steps per tile column: 1 << ks
  const int ns = tn == 128 ? 7 : 6;   // log2(TN)
  const int bt = tn >> 4;             // 16-row blocks per tile

  // ---- copy roles: every wave copies an eighth of the next step.  Wave w:
  // X rows BM/8 w .. +BM/8-1 (8 rows per 1 KiB copy), and half (w >> 2) of W
  // group (w & 3): dense 4 of its 8 KiB, 2:4 two value blocks and 256 B of codes.
  const int cw = wave & 3, chalf = wave >> 2;
  constexpr int XC = BM / 64;  // X copies per wave
  const uint8_t* xblk = reinterpret_cast<const uint8_t*>(x + m0 * ldx);
  // byte offset of this lane's 16 bytes in X copy j: row BM/8 wave + 8 j + lane / 8
  // of the block (rows past M read row M - 1: they only feed Y rows that are never
  // stored), logical chunk (lane & 7) ^ (row & 7); recomputed per copy, which
  // costs a few VALU operations and saves the registers of a table
  auto xoff = [&](int j) -> uint32_t {
    const int row = BM / 8 * wave + 8 * j + (lane >> 3);
    int64_t gm = m0 + row;
    if (gm > m - 1) gm = m - 1;
    return (uint32_t)(((gm - m0) * ldx + 8 * ((lane & 7) ^ xswz(row))) * 2);
  };
  const int64_t gn0 = n0 + 64 * cw;
  const bool g_ok = gn0 < n;
  const int64_t g_desc = (gn0 >> ns) * tiles_k;
  const int g_blk = (int)((gn0 & (tn - 1)) >> 4);
  const uint8_t* dsrc = reinterpret_cast<const uint8_t*>(dense_vals);
  const uint8_t* ssrc = reinterpret_cast<const uint8_t*>(sparse_vals);
  const uint32_t loff16 = lane * 16, loff4 = lane * 4;
  const uint32_t tile_elems = (uint32_t)(tn * tk);

  int32_t gd = 0;  // descriptor window of the copy group's tile row
  int gwin = -1;
  // descriptor window for the copies of `step`; loaded (and waited for) before any copy of the step
  auto copy_desc = [&](int step) -> int32_t {
    const int col = step >> ks;
    if (g_ok && (col >> 6) != gwin) {
      gwin = col >> 6;
      gd = desc_window(tile_desc, g_desc, tiles_k, gwin, lane);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      asm volatile("" : "+v"(gd));
    }
    return __builtin_amdgcn_readlane(gd, col & 63);
  };
  auto issue_x = [&](int step, int stage) {
    const uint32_t st = lds_base + stage * STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < XC; ++j) dma16_paced(xblk + step * 128, xoff(j), st + (BM / 8 * wave + 8 * j) * 128);
  };
  auto issue_w = [&](int step, int stage, int32_t d) {
    const uint32_t st = lds_base + stage * STAGE_BYTES;
    const uint32_t g = st + X_BYTES + cw * G_BYTES;
    if (!g_ok) return;  // group past N
    // pool offsets in 32 bits: every pool is below 4 GiB (checked at pack and import)
    const uint32_t slot = (uint32_t)d >> 1;
    const uint32_t u0 = (uint32_t)((step & ks) * bt + g_blk);  // first operand unit of the group
    if ((d & 1) == PATCH_TILE_DENSE) {
      const uint8_t* src = dsrc + (slot * tile_elems + u0 * 1024u) * 2u + 4096u * chalf;
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16_paced(src + 1024 * j, loff16, g + 4096 * chalf + 1024 * j);
    } else {
      const uint8_t* src = ssrc + slot * tile_elems + u0 * 1024u + 2048u * chalf;
      set_m0(g + 2048 * chalf);
      dma16_at<0>(src, loff16);
      dma16_at<1024>(src, loff16);
      const uint8_t* mp = sparse_meta + slot * (tile_elems >> 3) + (u0 >> 2) * 512u + 256u * chalf;
      dma4(mp, loff4, g + 4096 + 256 * chalf);
    }
  };
  auto issue = [&](int step, int stage, int32_t d) {
    issue_x(step, stage);
    issue_w(step, stage, d);
  };

  // ---- compute role: W rows 128 wn .. +127 (groups 2 wn, 2 wn + 1), X rows BM/4 wm .. +BM/4-1
  const int64_t wrow0 = n0 + 128 * wn;
  const bool hok0 = wrow0 < n, hok1 = wrow0 + 64 < n;
  const int64_t hdesc0 = (wrow0 >> ns) * tiles_k, hdesc1 = ((wrow0 + 64) >> ns) * tiles_k;

  f32x4 acc[8][XB];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < XB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint64_t dn0 = 0, dn1 = 0;  // bit j: column 64 cwin + j of this wave's tile rows is dense
  int cwin = -1;
  int d0 = -1, d1 = -1;
  bf16x16 b[XB];
  bf16x8 a0[8], a1[8];
  int ix[2][2];  // per W group: the code words of blocks (0, 1) and (2, 3)
  // dense / 2:4 bits of the window of tile columns holding `col`
  auto compute_window = [&](int col) {
    if ((col >> 6) != cwin) {
      cwin = col >> 6;
      const int32_t v0 = hok0 ? desc_window(tile_desc, hdesc0, tiles_k, cwin, lane) : 1;
      const int32_t v1 = hok1 ? desc_window(tile_desc, hdesc1, tiles_k, cwin, lane) : 1;
      dn0 = __builtin_amdgcn_ballot_w64((v0 & 1) == PATCH_TILE_DENSE);
      dn1 = __builtin_amdgcn_ballot_w64((v1 & 1) == PATCH_TILE_DENSE);
    }
  };
  // Step 0: the three descriptor windows (copies and both compute groups) are
  // loaded together and step 0's X copies issued behind them, so that their
  // latencies overlap; the first use of a window waits for all of it (the
  // compiler does not count the copies, so it waits for them too), then the W
  // copies follow.  Loaded one after the other, the windows cost two more
  // memory round trips before the first copy.
  auto prologue = [&]() {
    cwin = gwin = 0;
    gd = g_ok ? desc_window(tile_desc, g_desc, tiles_k, 0, lane) : 0;
    const int32_t v0 = hok0 ? desc_window(tile_desc, hdesc0, tiles_k, 0, lane) : 1;
    const int32_t v1 = hok1 ? desc_window(tile_desc, hdesc1, tiles_k, 0, lane) : 1;
    issue_x(0, 0);
    dn0 = __builtin_amdgcn_ballot_w64((v0 & 1) == PATCH_TILE_DENSE);
    dn1 = __builtin_amdgcn_ballot_w64((v1 & 1) == PATCH_TILE_DENSE);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("" : "+v"(gd));
    issue_w(0, 0, __builtin_amdgcn_readlane(gd, 0));
  };
  auto load_ops = [&](int step, int stage) {
    const uint8_t* cur = lds + stage * STAGE_BYTES;
    const int col = step >> ks;
    compute_window(col);
    d0 = hok0 ? (int)((dn0 >> (col & 63)) & 1) : -1;
    d1 = hok1 ? (int)((dn1 >> (col & 63)) & 1) : -1;
#pragma unroll
    for (int bm = 0; bm < XB; ++bm) {
      const int r = BM / 4 * wm + 16 * bm + r16;
      b[bm] = cat16(lds8(cur + r * 128 + ((q ^ xswz(r)) << 4)), lds8(cur + r * 128 + (((4 + q) ^ xswz(r)) << 4)));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int dh = h ? d1 : d0;
      const uint8_t* g = cur + X_BYTES + (2 * wn + h) * G_BYTES;
      if (dh > 0) {
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          a0[4 * h + b4] = lds8(g + 2048 * b4 + lane * 16);
          a1[4 * h + b4] = lds8(g + 2048 * b4 + 1024 + lane * 16);
        }
        ix[h][0] = ix[h][1] = 0x44444444;  // kept positions 0 and 1 of every group, in both halves
      } else if (dh == 0) {
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) a0[4 * h + b4] = lds8(g + 1024 * b4 + lane * 16);
        const uint2 c = *reinterpret_cast<const uint2*>(g + 4096 + 8 * lane);
        ix[h][0] = (int)c.x;
        ix[h][1] = (int)c.y;
      }
    }
  };
  auto mma = [&]() {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int dh = h ? d1 : d0;
      if (dh < 0) continue;
#pragma unroll
      for (int bm = 0; bm < XB; ++bm)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int bn = 4 * h + b4;
          acc[bn][bm] = b4 & 1 ? __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a0[bn], b[bm], acc[bn][bm], ix[h][b4 >> 1], 0, 1)
                               : __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a0[bn], b[bm], acc[bn][bm], ix[h][b4 >> 1], 0, 0);
        }
      if (dh > 0) {  // kept positions 2 and 3 of every group
#pragma unroll
        for (int bm = 0; bm < XB; ++bm)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const int bn = 4 * h + b4;
            acc[bn][bm] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a1[bn], b[bm], acc[bn][bm], 0xEEEE, 0, 0);
          }
      }
    }
  };

  // Two waves per SIMD (wave w and w + 4) run half a step apart: after the
  // barrier of step i, waves 0-3 issue their copies of step i + 1, read step i
  // and multiply it; waves 4-7 multiply step i - 1 (read before the barrier),
  // issue their copies and read step i.  Copies of step i + 1 go to the stage
  // that every wave finished reading before the barrier.
  // 64-row blocks run two workgroups per CU (128 VGPRs): both wave groups keep
  // the same order there, and the other workgroup on the CU fills the gaps.
  constexpr bool LAG = BM > 64;
  if (nsteps > 0) prologue();
  if (!LAG || wn == 0) {
    for (int i = 0; i < nsteps; ++i) {
      const int32_t dnext = i + 1 < nsteps ? copy_desc(i + 1) : 0;
      step_barrier();
      if (i + 1 < nsteps) issue(i + 1, (i + 1) & 1, dnext);
      load_ops(i, i & 1);
      mma();
    }
  } else if (nsteps > 0) {
    for (int i = 0; i < nsteps; ++i) {
      const int32_t dnext = i + 1 < nsteps ? copy_desc(i + 1) : 0;
      step_barrier();
      if (i > 0) mma();
      if (i + 1 < nsteps) issue(i + 1, (i + 1) & 1, dnext);
      load_ops(i, i & 1);
    }
    mma();
  }

  // After the last barrier every wave is done with step nsteps - 2, and no copy
  // targets its stage any more: each wave stages its Y block there.
  static_assert(8 * (BM / 4) * 128 <= STAGE_BYTES, "Y staging fits one stage");
  uint8_t* region = lds + (nsteps & 1) * STAGE_BYTES + wave * (BM / 4 * 128);
  const bool hok[2] = {hok0, hok1};
  store_block<F32, BM / 4, XB, 2>(acc, region, y, ldy, m, m0 + BM / 4 * wm, wrow0, hok, lane);
}

// Persistent: each workgroup takes slots blockIdx.x, + gridDim.x, ...  The
// grid is a multiple of 8, so every slot stays on the XCD its number maps to,
// and a block's Y stores drain while the same workgroup copies and multiplies
// its next block.  The barrier between blocks keeps the next block's first
// copies off LDS that slower waves still read.
//
// The 256-row instance also runs entries of 192-row blocks (gemm_problem.bm):
// the launcher may cut a product's last, ragged round of 256-row blocks into a
// round of 192-row ones in the same launch (see plan_tail).
template <bool F32, int BM>
__global__ __launch_bounds__(512, BM == 64 ? 4 : 1) void k_gemm_tiled(const gemm_group g) {
  for (int slot = blockIdx.x; slot < g.total; slot += gridDim.x) {
    int local;
    const int pi = find_problem(g, slot, local);
    if (pi >= 0) {
      if constexpr (BM == 256) {
        if (g.p[pi].bm == 192) tiled_block<F32, 192>(g.p[pi], local);
        else tiled_block<F32, 256>(g.p[pi], local);
      } else {
        tiled_block<F32, BM>(g.p[pi], local);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// ------------------------------------------------------------------------
// Warp-specialised kernel for 128 X rows per block, and for 64 when the grid
// gives each CU at most one workgroup: 12 waves.  Waves 0-7 compute exactly as
// in k_gemm_tiled (2 x 4 grid, 128 W rows x BM/4 X rows each, two per SIMD);
// waves 8-11 (one per SIMD) only copy, two steps ahead through three LDS
// stages (48 KiB each at 128 rows, 40 at 64).  Issuing copies takes a wave
// hundreds of clocks per step; here no computing wave ever does, and the third
// stage hides the copies' latency.  A copy wave writes M0 once
// per run of consecutive 1 KiB pool blocks (immediate offsets for the rest), so
// it issues its copies with fewer scalar instructions: 6-16% faster on the
// 512 x 2048 products at M = 4096, 1-2% on the 2048-wide ones.
// ------------------------------------------------------------------------
namespace wsk {
constexpr int STAGES = 3, WAVES = 12;
template <int BM, int NG> constexpr int step_bytes() { return BM * 128 + NG * tiled::G_BYTES; }
}  // namespace wsk

// Wait until at most n of this wave's copies are outstanding, and for its LDS
// reads.  n is the copy count of one stage: per K step XC (2 or 4) X copies
// plus 0, 6 or 8 W copies, one or two K steps, so an even number up to 24.
__device__ __forceinline__ void wait_copies_but(int n) {
#define PATCH_WAIT_CASE(c) \
  case c: asm volatile("s_waitcnt vmcnt(" #c ") lgkmcnt(0)" ::: "memory"); break;
  switch (n) {
    PATCH_WAIT_CASE(24) PATCH_WAIT_CASE(22) PATCH_WAIT_CASE(20) PATCH_WAIT_CASE(18) PATCH_WAIT_CASE(16)
    PATCH_WAIT_CASE(14) PATCH_WAIT_CASE(12) PATCH_WAIT_CASE(10) PATCH_WAIT_CASE(8) PATCH_WAIT_CASE(6)
    PATCH_WAIT_CASE(4) PATCH_WAIT_CASE(2)
    default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); break;
  }
#undef PATCH_WAIT_CASE
}

// One output block of k_gemm_ws: workgroup slot `slot` of the launch; the
// block is NG 64-row W groups (BN = 64 NG rows of W) by BM rows of X.  A stage
// holds KS consecutive 64-wide K steps (one barrier per stage): two halve the
// barriers of the small 64 x 128 blocks, whose steps carry little work.
template <bool F32, int BM, int NG, int KS>
__device__ __forceinline__ void ws_block(const gemm_group& g, int slot) {
  using namespace wsk;
  using tiled::G_BYTES;
  static_assert(NG == 2 || NG == 4, "128 or 256 W rows per block");
  static_assert(KS == 1 || KS == 2, "one or two K steps per stage");
  constexpr int BN = 64 * NG, GW = NG / 2;  // GW: W groups per computing wave
  constexpr int X_BYTES = BM * 128, STEP_BYTES = step_bytes<BM, NG>(), STAGE_BYTES = KS * STEP_BYTES;
  constexpr int RW = BM / 4;   // X rows per copy wave and per compute wave
  constexpr int XC = RW / 8;   // X copies per copy wave
  constexpr int XB = RW / 16;  // X blocks of 16 rows per compute wave
  int local;
  const int pi = find_problem(g, slot, local);
  if (pi < 0) return;
  const gemm_problem& P = g.p[pi];
  const const_desc_ptr tile_desc = (const_desc_ptr)P.tile_desc;
  const int tn = P.tn, tk = P.tk;
  const int64_t tiles_k = P.tiles_k, n = P.n, k = P.k, m = P.m;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // Opaque per block, so that the compiler recomputes the lane-dependent
  // offsets for every block instead of holding them across the block loop.
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t n0, m0;
  block_origin<BM, BN>(P.n_begin, n, m, local, P.group_n, n0, m0);
  const int nsteps = (int)(k / 64);
  const int nstages = (nsteps + KS - 1) / KS;  // stage loads, KS K steps each (the last may hold fewer)
  const int ks = tk == 128;
  const int ns = tn == 128 ? 7 : 6;
  const int bt = tn >> 4;

  if (wave >= 8) {
    // ---- copy waves: X rows RW c .. RW c + RW - 1 and W group c (rows n0 + 64 c ..) if c < NG
    const int cw = wave - 8;
    // The narrow instance's steps carry little matrix work; its copies keep the
    // pace, so its copy waves issue ahead of the computing waves (7% faster on
    // the 512 x 2048 product at M = 4096; the 128 x 256 instance is slower so).
    if constexpr (NG == 2) __builtin_amdgcn_s_setprio(3);
    const int64_t ldx = P.ldx;
    const uint8_t* xblk = reinterpret_cast<const uint8_t*>(P.x + m0 * ldx);
    uint32_t xoff[XC];
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      const int row = RW * cw + 8 * j + (lane >> 3);
      int64_t gm = m0 + row;
      if (gm > m - 1) gm = m - 1;  // rows past M only feed Y rows that are never stored
      xoff[j] = (uint32_t)(((gm - m0) * ldx + 8 * ((lane & 7) ^ xswz(row))) * 2);
    }
    const int64_t gn0 = n0 + 64 * cw;
    const bool g_ok = cw < NG && gn0 < n;
    const int64_t g_desc = (gn0 >> ns) * tiles_k;
    const int g_blk = (int)((gn0 & (tn - 1)) >> 4);
    const uint8_t* dsrc = reinterpret_cast<const uint8_t*>(P.dense_vals);
    const uint8_t* ssrc = reinterpret_cast<const uint8_t*>(P.sparse_vals);
    const uint8_t* msrc = P.sparse_meta;
    const uint32_t loff16 = lane * 16, loff4 = lane * 4;
    const uint32_t tile_elems = (uint32_t)(tn * tk);
    // copies of K step `step` into the LDS bytes at st
    auto issue_step = [&](int step, uint32_t st) -> int {
#pragma unroll
      for (int j = 0; j < XC; ++j) dma16(xblk + step * 128, xoff[j], st + (RW * cw + 8 * j) * 128);
      const uint32_t gl = st + X_BYTES + cw * G_BYTES;
      if (!g_ok) return XC;
      const int32_t d = tile_desc[g_desc + (step >> ks)];
      const uint32_t slot = (uint32_t)d >> 1;  // pools are below 4 GiB
      const uint32_t u0 = (uint32_t)((step & ks) * bt + g_blk);
      if ((d & 1) == PATCH_TILE_DENSE) {
        const uint8_t* src = dsrc + (slot * tile_elems + u0 * 1024u) * 2u;
        set_m0(gl);
        dma16_at<0>(src, loff16);
        dma16_at<1024>(src, loff16);
        dma16_at<2048>(src, loff16);
        dma16_at<3072>(src, loff16);
        set_m0(gl + 4096);
        dma16_at<0>(src + 4096, loff16);
        dma16_at<1024>(src + 4096, loff16);
        dma16_at<2048>(src + 4096, loff16);
        dma16_at<3072>(src + 4096, loff16);
        return XC + 8;
      }
      const uint8_t* src = ssrc + slot * tile_elems + u0 * 1024u;
      set_m0(gl);
      dma16_at<0>(src, loff16);
      dma16_at<1024>(src, loff16);
      dma16_at<2048>(src, loff16);
      dma16_at<3072>(src, loff16);
      const uint8_t* mp = msrc + slot * (tile_elems >> 3) + (u0 >> 2) * 512u;
      set_m0(gl + 4096);
      dma4_at<0>(mp, loff4);
      dma4_at<256>(mp, loff4);
      return XC + 6;
    };
    // copies of stage load t (K steps KS t ..) into LDS stage `stage`
    auto issue = [&](int t, int stage) -> int {
      int c = 0;
#pragma unroll
      for (int j = 0; j < KS; ++j)
        if (KS * t + j < nsteps) c += issue_step(KS * t + j, lds_base + stage * STAGE_BYTES + j * STEP_BYTES);
      return c;
    };
    // Two stage loads ahead.  Before the barrier of load i this wave waits only
    // for its copies of load i (those of load i + 1 were issued after them;
    // vmcnt counts in issue order).  After it, every wave is done with load
    // i - 1, whose stage takes load i + 2.
    int pending = 0;
    if (nstages > 0) issue(0, 0);
    if (nstages > 1) pending = issue(1, 1);
    int stage = 0;
    for (int i = 0; i < nstages; ++i) {
      wait_copies_but(i + 1 < nstages ? pending : 0);
      barrier();
      if (i + 2 < nstages) pending = issue(i + 2, stage == 0 ? 2 : stage - 1);
      stage = stage == 2 ? 0 : stage + 1;
    }
    return;
  }

  // ---- compute waves: W groups GW wn .. GW wn + GW - 1, X rows RW wm .. +RW-1
  const int wn = wave >> 2, wm = wave & 3;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t wrow0 = n0 + 64 * GW * wn;
  bool hok[GW];
  int64_t hdesc[GW];
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    hok[h] = wrow0 + 64 * h < n;
    hdesc[h] = ((wrow0 + 64 * h) >> ns) * tiles_k;
  }
  f32x4 acc[4 * GW][XB];
#pragma unroll
  for (int i = 0; i < 4 * GW; ++i)
#pragma unroll
    for (int j = 0; j < XB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Operands of one step: read by load_ops, consumed by mma.
  int dg[GW];  // per 64-row group: 1 dense, 0 2:4, -1 past N
  bf16x16 b[XB];
  bf16x8 a0[4 * GW], a1[4 * GW];
  int ix[4 * GW];
  // operands of K step `step`, held in LDS stage `stage` at position step % KS
  auto load_ops = [&](int step, int stage) {
    const uint8_t* cur = lds + stage * STAGE_BYTES + (step % KS) * STEP_BYTES;
#pragma unroll
    for (int h = 0; h < GW; ++h)
      dg[h] = hok[h] ? ((tile_desc[hdesc[h] + (step >> ks)] & 1) == PATCH_TILE_DENSE) : -1;
#pragma unroll
    for (int bm = 0; bm < XB; ++bm) {
      const int r = RW * wm + 16 * bm + r16;
      b[bm] = cat16(lds8(cur + r * 128 + ((q ^ xswz(r)) << 4)), lds8(cur + r * 128 + (((4 + q) ^ xswz(r)) << 4)));
    }
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      const uint8_t* gp = cur + X_BYTES + (GW * wn + h) * G_BYTES;
      if (dg[h] > 0) {
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          a0[4 * h + b4] = lds8(gp + 2048 * b4 + lane * 16);
          a1[4 * h + b4] = lds8(gp + 2048 * b4 + 1024 + lane * 16);
          ix[4 * h + b4] = 0x44444444;
        }
      } else if (dg[h] == 0) {
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) a0[4 * h + b4] = lds8(gp + 1024 * b4 + lane * 16);
        const uint2 c = *reinterpret_cast<const uint2*>(gp + 4096 + 8 * lane);
        ix[4 * h + 0] = ix[4 * h + 1] = (int)c.x;
        ix[4 * h + 2] = ix[4 * h + 3] = (int)c.y;
      }
    }
  };
  auto mma = [&]() {
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      if (dg[h] < 0) continue;
#pragma unroll
      for (int bm = 0; bm < XB; ++bm)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int bn = 4 * h + b4;
          acc[bn][bm] = b4 & 1 ? __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a0[bn], b[bm], acc[bn][bm], ix[bn], 0, 1)
                               : __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a0[bn], b[bm], acc[bn][bm], ix[bn], 0, 0);
        }
      if (dg[h] > 0) {
#pragma unroll
        for (int bm = 0; bm < XB; ++bm)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const int bn = 4 * h + b4;
            acc[bn][bm] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a1[bn], b[bm], acc[bn][bm], 0xEEEE, 0, 0);
          }
      }
    }
  };
  // The two computing waves of a SIMD (wave w and w + 4) run half a step
  // apart: waves 0-3 read step i and multiply it, waves 4-7 multiply step
  // i - 1 (read in the previous step) and then read step i, so that one of
  // them reads LDS while the other keeps the matrix unit busy.  Separate
  // loops keep the compiler from holding both schedules' registers.
  // With KS = 2 the lagging waves multiply all but the last K step of a stage
  // load at once and carry that one over the barrier.
  int stage = 0;
  if (wn == 0) {
    for (int i = 0; i < nstages; ++i) {
      wait_copies_but(0);  // this wave's LDS reads of the previous load are done
      barrier();           // load i is in `stage`
#pragma unroll
      for (int j = 0; j < KS; ++j)
        if (KS * i + j < nsteps) {
          load_ops(KS * i + j, stage);
          mma();
        }
      stage = stage == 2 ? 0 : stage + 1;
    }
  } else if (nsteps > 0) {
    for (int i = 0; i < nstages; ++i) {
      wait_copies_but(0);
      barrier();
      if (i > 0) mma();  // the last K step of load i - 1
#pragma unroll
      for (int j = 0; j < KS; ++j)
        if (KS * i + j < nsteps) {
          if (j > 0) mma();
          load_ops(KS * i + j, stage);
        }
      stage = stage == 2 ? 0 : stage + 1;
    }
    mma();
  }
  // After the last barrier only the stage of load nstages - 1 is still read,
  // and no copy is in flight: the stage load nstages would have used holds
  // the computing waves' Y blocks (8 x RW x 128 bytes).
  static_assert(8 * RW * 128 <= STAGE_BYTES, "Y staging fits one stage");
  uint8_t* region = lds + (nstages % STAGES) * STAGE_BYTES + wave * (RW * 128);
  store_block<F32, RW, XB, GW>(acc, region, P.y, P.ldy, m, m0 + RW * wm, wrow0, hok, lane);
}

// Persistent like k_gemm_tiled.
template <bool F32, int BM, int NG, int KS>
__global__ __launch_bounds__(768, 1) void k_gemm_ws(const gemm_group g) {
  for (int slot = blockIdx.x; slot < g.total; slot += gridDim.x) {
    ws_block<F32, BM, NG, KS>(g, slot);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

gemm_problem make_problem(const patch_weight* w, const uint16_t* x, int64_t m, int64_t ldx, void* y, int64_t ldy) {
  gemm_problem p = {};
  p.tile_desc = w->tile_desc;
  p.dense_vals = w->dense_vals;
  p.sparse_vals = w->sparse_vals;
  p.sparse_meta = w->sparse_meta;
  p.x = x;
  p.y = y;
  p.tiles_k = w->tiles_k;
  p.n = w->n;
  p.k = w->k;
  p.m = m;
  p.ldx = ldx;
  p.ldy = ldy;
  p.tn = w->tn;
  p.tk = w->tk;
  const double tiles = (double)(w->n_dense + w->n_sparse);
  p.w_bytes = tiles > 0 ? (float)((2.0 * w->n_dense + 1.125 * w->n_sparse) / tiles) : 2.0f;
  p.group_n = 4;
  p.n_begin = 0;
  p.bm = 0;
  p.mix = (float)row_cost(w, 0, w->tiles_n);
  p.ksplit = 1;
  p.part = nullptr;
  return p;
}

namespace {
// PATCH_LOG=1 in the environment prints every GEMM launch's plan to stderr:
// block height, grid and the entries with their W-row ranges.
bool log_launches() {
  static const bool on = [] {
    const char* e = getenv("PATCH_LOG");
    return e && *e && *e != '0';
  }();
  return on;
}

}  // namespace

namespace {
template <bool F32, int MB, int NBLK, int WAVES, int BATCH, int SPLIT = 1>
hipError_t launch_stream_mb(gemm_group& g, hipStream_t s) {
  int64_t total = 0;
  for (int i = 0; i < g.count; ++i) {  // each product starts on a multiple of 8 (its XCD order)
    if (g.p[i].ksplit != SPLIT) return hipErrorInvalidValue;
    g.p[i].block0 = (int32_t)total;
    g.p[i].blocks = (int32_t)(g.p[i].n / (16 * NBLK) * SPLIT);
    total += (g.p[i].blocks + 7) / 8 * 8;
  }
  if (total == 0) return hipSuccess;
  if (total > INT32_MAX) return hipErrorInvalidValue;  // block numbers are 32-bit
  hipLaunchKernelGGL((k_gemm_stream<F32, MB, NBLK, WAVES, BATCH, SPLIT>), dim3((unsigned)total), dim3(64 * WAVES), 0,
                     s, g);
  return hipGetLastError();
}
template <bool F32>
hipError_t launch_stream_f(gemm_group& g, int waves, int nblk, int mb, hipStream_t s) {
  // LDS per workgroup: WAVES x BATCH x MB x 2 KiB of X slots.  Decode with one
  // W block (MB = 1, 16 waves) keeps two chunks in flight per wave (64 KiB, two
  // workgroups per CU); the other instances keep one.  Eight waves carry the
  // wider accumulator sets (up to 4 x 8 blocks: 128 registers).
  if (waves == streamk::WAVES && nblk == 1) {
    switch (mb) {
      case 1: return launch_stream_mb<F32, 1, 1, streamk::WAVES, streamk::BATCH>(g, s);
      case 2: return launch_stream_mb<F32, 2, 1, 16, 1>(g, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (waves != 8) return hipErrorInvalidValue;
  switch (nblk * 16 + mb) {
    case 16 + 4: return launch_stream_mb<F32, 4, 1, 8, 1>(g, s);
    case 16 + 8: return launch_stream_mb<F32, 8, 1, 8, 1>(g, s);
    case 32 + 1: return launch_stream_mb<F32, 1, 2, 8, 2>(g, s);
    case 32 + 2: return launch_stream_mb<F32, 2, 2, 8, 1>(g, s);
    case 32 + 4: return launch_stream_mb<F32, 4, 2, 8, 1>(g, s);
    case 32 + 8: return launch_stream_mb<F32, 8, 2, 8, 1>(g, s);
    case 64 + 1: return launch_stream_mb<F32, 1, 4, 8, 1>(g, s);
    case 64 + 2: return launch_stream_mb<F32, 2, 4, 8, 1>(g, s);
    case 64 + 4: return launch_stream_mb<F32, 4, 4, 8, 1>(g, s);
    case 64 + 8: return launch_stream_mb<F32, 8, 4, 8, 1>(g, s);
    default: return hipErrorInvalidValue;
  }
}
// The K-split instances: four workgroups per W block, 8 waves, 2 or 4 W blocks.
template <bool F32>
hipError_t launch_split_f(gemm_group& g, int nblk, int mb, hipStream_t s) {
  switch (nblk * 16 + mb) {
    case 32 + 1: return launch_stream_mb<F32, 1, 2, 8, 2, 4>(g, s);
    case 32 + 2: return launch_stream_mb<F32, 2, 2, 8, 1, 4>(g, s);
    case 32 + 4: return launch_stream_mb<F32, 4, 2, 8, 1, 4>(g, s);
    case 32 + 8: return launch_stream_mb<F32, 8, 2, 8, 1, 4>(g, s);
    case 64 + 1: return launch_stream_mb<F32, 1, 4, 8, 1, 4>(g, s);
    case 64 + 2: return launch_stream_mb<F32, 2, 4, 8, 1, 4>(g, s);
    case 64 + 4: return launch_stream_mb<F32, 4, 4, 8, 1, 4>(g, s);
    case 64 + 8: return launch_stream_mb<F32, 8, 4, 8, 1, 4>(g, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

int stream_x_blocks(int64_t m) { return m <= 16 ? 1 : m <= 32 ? 2 : m <= 64 ? 4 : m <= PATCH_STREAM_MAX_M ? 8 : 0; }

// Measured on MI355X with the weights read from HBM (90% 2:4 tiles, N from
// 2048 to 14336, m from 1 to 128): the fastest W-block count was the largest
// that still leaves 160 workgroups, e.g. 4 for 11008 and 13824 rows (up to 32%
// faster than one block at m = 16, 25% at m = 32), 2 for 5120 to 8192, 1 for
// 4096 and below.
int stream_w_blocks(int64_t n) { return n >= 160 * 64 ? 4 : n >= 160 * 32 ? 2 : 1; }

// 16 waves split K for one W block and at most two X blocks (4-19% faster
// than 8 there on long-K products at m = 17); 8 waves otherwise (up to 40%
// faster than 16 with four W or X blocks: half the reduction, and two
// workgroups per CU).
int stream_waves(int64_t m, int64_t n) { return stream_w_blocks(n) == 1 && stream_x_blocks(m) <= 2 ? 16 : 8; }

// A narrow W (fewer than 5120 rows: one W block per workgroup, at most 319
// workgroups) with a long K (at least 128 chunks) leaves each wave a long
// chain of dependent chunks, and every workgroup copies all of X.  Given a
// workspace, four workgroups share each W block's K range instead, each with
// 4 W blocks (4096 rows and more) or 2: the X copies fall by that factor and
// the grid stays at 256-384 workgroups.  Measured on MI355X with the weights
// read from HBM, the summing launch included: 2048 x 8192 at m = 64 and 128
// in 14.6 and 20.4 us against 21.6 and 36.1; 4096 x 11008 in 23.0 and 33.5
// against 30.5 and 48.5.  At decode sizes (m <= 16) the summing launch costs
// about what the split saves once the unsplit grid already has a workgroup
// per CU (4096 x 11008 at m = 1: 15.1 against 13.2 us), so there only
// narrower weights split (2048 x 8192 at m = 16: 10.5 against 11.8 us).
// Products with 64 chunks (K = 4096) gained at most 6% before the sum.
int stream_k_split(int64_t m, int64_t n, int64_t k) {
  if (stream_w_blocks(n) != 1 || n < 2048 || (k >> 6) < 128) return 1;
  return m <= 16 && n >= 4096 ? 1 : 4;
}
int stream_split_w_blocks(int64_t n) { return n >= 4096 ? 4 : 2; }

namespace {
// Sums the K shares' partials of a split product in share order and writes Y:
// four columns per thread.
template <bool F32>
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ part, int split, int64_t m, int64_t n,
                                                   void* __restrict__ y, int64_t ldy) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x, quads = n >> 2;
  if (q >= m * quads) return;
  const int64_t row = q / quads, col = (q - row * quads) * 4;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + row * n + col);
  for (int s = 1; s < split; ++s) acc += *reinterpret_cast<const f32x4*>(part + (s * m + row) * n + col);
  if (F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + row * ldy + col) = acc;
  } else {
    const uint32_t lo = f32_to_bf16_rne(acc[0]) | (uint32_t)f32_to_bf16_rne(acc[1]) << 16;
    const uint32_t hi = f32_to_bf16_rne(acc[2]) | (uint32_t)f32_to_bf16_rne(acc[3]) << 16;
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + row * ldy + col) = make_uint2(lo, hi);
  }
}
}  // namespace

hipError_t launch_stream_split(const gemm_problem& p, int out_f32, hipStream_t s) {
  if (p.ksplit != 4 || !p.part || p.n % 64 || p.m < 1 || p.m > PATCH_STREAM_MAX_M) return hipErrorInvalidValue;
  gemm_group g = {};
  g.p[g.count++] = p;
  const int nblk = stream_split_w_blocks(p.n), mb = stream_x_blocks(p.m);
  if (log_launches())
    fprintf(stderr, "patch: k_gemm_stream waves 8 w_blocks %d x_blocks %d k_split %d\n", nblk, mb, p.ksplit);
  hipError_t e = out_f32 ? launch_split_f<true>(g, nblk, mb, s) : launch_split_f<false>(g, nblk, mb, s);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((p.m * (p.n >> 2) + 255) / 256);
  if (out_f32) hipLaunchKernelGGL(k_split_sum<true>, dim3(grid), dim3(256), 0, s, p.part, p.ksplit, p.m, p.n, p.y, p.ldy);
  else hipLaunchKernelGGL(k_split_sum<false>, dim3(grid), dim3(256), 0, s, p.part, p.ksplit, p.m, p.n, p.y, p.ldy);
  return hipGetLastError();
}

// A product's Y depends only on how many waves split its K (each wave sums its
// chunks in order, then the waves are summed in order), not on how many X or W
// blocks a workgroup carries, and its wave count depends only on its own m and
// n.  So a launch takes the products of one (waves, W blocks) family and sizes
// its X blocks for their largest m: a product's Y never depends on the others
// in its group.
hipError_t launch_stream_group(gemm_group& g, int out_f32, hipStream_t s) {
  // families: 16 waves x 1 W block, 8 waves x 1, 2 or 4 W blocks
  gemm_group part[4] = {};
  int mb[4] = {1, 1, 1, 1};
  for (int i = 0; i < g.count; ++i) {
    const int xb = stream_x_blocks(g.p[i].m);
    if (xb == 0) return hipErrorInvalidValue;
    const int nblk = stream_w_blocks(g.p[i].n);
    const int j = stream_waves(g.p[i].m, g.p[i].n) == 16 ? 0 : nblk == 1 ? 1 : nblk == 2 ? 2 : 3;
    gemm_group& h = part[j];
    h.p[h.count++] = g.p[i];
    if (xb > mb[j]) mb[j] = xb;
  }
  static const int waves[4] = {16, 8, 8, 8}, nblks[4] = {1, 1, 2, 4};
  for (int j = 0; j < 4; ++j) {
    if (part[j].count == 0) continue;
    if (j == 1 && mb[j] < 4) mb[j] = 4;  // one W block with 8 waves: only for m > 32
    if (log_launches())
      fprintf(stderr, "patch: k_gemm_stream waves %d w_blocks %d x_blocks %d products %d\n", waves[j], nblks[j], mb[j],
              part[j].count);
    const hipError_t e = out_f32 ? launch_stream_f<true>(part[j], waves[j], nblks[j], mb[j], s)
                                 : launch_stream_f<false>(part[j], waves[j], nblks[j], mb[j], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

namespace {
// Opts `kernel` into lds_bytes of dynamic LDS (above the 64 KiB default),
// once per device (done[device]; host threads that race here set the same
// attribute).
hipError_t allow_lds(const void* kernel, int lds_bytes, std::atomic<bool>* done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!done[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    done[dev].store(true, std::memory_order_release);
  }
  return hipSuccess;
}

// Grid of a persistent launch: the workgroups the device holds at once
// (queried once per device into cache[device]), rounded down to a multiple of
// 8, and never more than the launch's slots.  -1 if the device cannot be
// queried.
int persistent_grid(const void* kernel, int threads, int lds_bytes, std::atomic<int>* cache, int64_t slots) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  int held = cache[dev].load(std::memory_order_relaxed);
  if (held == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds_bytes) != hipSuccess)
      return -1;
    const int r = cus * (per_cu > 0 ? per_cu : 1) / 8 * 8;
    held = r > 8 ? r : 8;
    cache[dev].store(held, std::memory_order_relaxed);
  }
  return slots < held ? (int)slots : held;
}

// The workgroups resident on one XCD (per_xcd of them) take consecutive
// block numbers of the walk, so a round of them covers about w block columns
// by per_xcd / w block rows, and that XCD's L2 fetches those blocks' X rows
// and W rows over the whole K once per round: per_xcd / w * (bm K 2 bytes) +
// w * (bn K w_bytes).  Each product gets the power-of-two width (at most its
// block columns) that minimises it; FETCH_SIZE counts on MI355X follow this
// model within a few per cent.  The time does not depend on it (the L2 hides
// these fetches), only the memory traffic does.
void group_width(gemm_group& g, int bm, int bn, int per_xcd) {
  for (int i = 0; i < g.count; ++i) {
    gemm_problem& p = g.p[i];
    const int64_t nbn = (p.n - p.n_begin + bn - 1) / bn;
    const int ebm = p.bm > 0 ? p.bm : bm;
    const double xrow = 2.0 * ebm * (double)p.k, wcol = (double)p.w_bytes * bn * (double)p.k;
    int best = 1;
    double best_b = 0;
    for (int w = 1; w <= 32 && w <= nbn; w *= 2) {
      const double rows = per_xcd / w > 1 ? (double)(per_xcd / w) : 1.0;
      const double b = rows * xrow + w * wcol;
      if (w == 1 || b < best_b) {
        best = w;
        best_b = b;
      }
    }
    p.group_n = best;
  }
}

// Relative cost of one workgroup: block height over its measured efficiency
// (smaller blocks move more LDS bytes per flop), times the K steps.
double block_cost(int bm, int64_t k) {
  // measured in whole rounds on the 8192x2048 and 4096x4096 products at M = 4096
  // (192: from the 8192x2048, 4096x4096 and 5120x5120 products, 0.84-0.96)
  const double eff = bm == 256 ? 1.0 : bm == 192 ? 0.92 : bm == 128 ? 0.96 : 0.68;
  return bm / 256.0 / eff * (double)(k / 64);
}

// Slots s in [0, x) with s % G == w.
inline int64_t slots_below(int64_t x, int w, int G) { return x > w ? (x - 1 - w) / G + 1 : 0; }

// Cost-balanced tail of a launch of 256-row blocks.  Workgroup w of a
// persistent grid of G runs slots w, w + G, ...; when the last entry's blocks
// leave a ragged last round, its first block columns keep 256-row blocks and
// the rest become 192-row blocks (two entries of one launch), if that lowers
// the estimated makespan by 2% or more.  A block's cost is block_cost times the
// mean step cost of its entry's tile rows (row_cost: the dense / 2:4 mix from
// the packed weight's cost prefix).  The split points tried put the end of the
// 256-row blocks on a round boundary.  Example: 11008 x 4096 at M = 4096 is
// 688 blocks of 256 x 256 on 256 workgroups (2.69 rounds); 32 block columns
// (512 blocks, 2 rounds) stay, the other 11 become 242 blocks of 192 rows that
// share the third round.
void plan_tail(gemm_group& g, int G) {
  constexpr int MAXG = 4096;
  if (g.count == 0 || g.count >= PATCH_MAX_GROUP || G <= 0 || G > MAXG) return;
  static thread_local double load[MAXG];
  for (int w = 0; w < G; ++w) load[w] = 0;
  int64_t s0 = 0;
  for (int i = 0; i + 1 < g.count; ++i) {
    const gemm_problem& p = g.p[i];
    const int64_t blocks = ((p.n - p.n_begin + 255) / 256) * ((p.m + 255) / 256);
    const double c = block_cost(256, p.k) * p.mix;
    for (int w = 0; w < G; ++w) load[w] += c * (double)(slots_below(s0 + blocks, w, G) - slots_below(s0, w, G));
    s0 += (blocks + 7) / 8 * 8;
  }
  gemm_problem& last = g.p[g.count - 1];
  const int64_t nbn = (last.n - last.n_begin + 255) / 256, nbm = (last.m + 255) / 256, nbm2 = (last.m + 191) / 192;
  const double c256 = block_cost(256, last.k) * last.mix, c192 = block_cost(192, last.k) * last.mix;
  // makespan with the first ca block columns in 256-row blocks, the rest in 192-row ones
  auto makespan = [&](int64_t ca) {
    const int64_t a = ca * nbm, sb = s0 + (a + 7) / 8 * 8, b = (nbn - ca) * nbm2;
    double worst = 0;
    for (int w = 0; w < G; ++w) {
      const double t = load[w] + c256 * (double)(slots_below(s0 + a, w, G) - slots_below(s0, w, G)) +
                       c192 * (double)(slots_below(sb + b, w, G) - slots_below(sb, w, G));
      worst = t > worst ? t : worst;
    }
    return worst;
  };
  const double base = makespan(nbn);
  int64_t best_ca = nbn;
  double best = base;
  for (int64_t r = 1; r * G <= s0 + nbn * nbm + G; ++r) {
    const int64_t ca = (r * G - s0) / nbm;
    if (ca < 1 || ca >= nbn) continue;
    const double t = makespan(ca);
    if (t < best) {
      best = t;
      best_ca = ca;
    }
  }
  if (best_ca == nbn || best > 0.98 * base) return;
  gemm_problem tail = last;
  tail.n_begin = last.n_begin + best_ca * 256;
  tail.bm = 192;
  last.n = tail.n_begin;
  g.p[g.count++] = tail;
}

void log_plan(const char* kernel, const gemm_group& g, int grid) {
  if (!log_launches()) return;
  fprintf(stderr, "patch: %s grid %d slots %d", kernel, grid, (int)g.total);
  for (int i = 0; i < g.count; ++i)
    fprintf(stderr, " | rows %lld..%lld m %lld k %lld bm %d blocks %d", (long long)g.p[i].n_begin,
            (long long)g.p[i].n, (long long)g.p[i].m, (long long)g.p[i].k, g.p[i].bm, g.p[i].blocks);
  fprintf(stderr, "\n");
}

template <bool F32, int BM>
hipError_t launch_tiled_bm(gemm_group& g, bool plan, hipStream_t s) {
  constexpr int lds_bytes = tiled::STAGES * tiled::stage_bytes<BM>();
  static std::atomic<bool> lds_allowed[64] = {};
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(&k_gemm_tiled<F32, BM>), lds_bytes, lds_allowed);
  if (e != hipSuccess) return e;
  static std::atomic<int> resident[64] = {};
  const int held = persistent_grid(reinterpret_cast<const void*>(&k_gemm_tiled<F32, BM>), 512, lds_bytes, resident,
                                   INT32_MAX);
  if (held < 0) return hipErrorInvalidDevice;
  for (int i = 0; i < g.count; ++i) g.p[i].bm = BM;
  if (BM == 256 && plan) plan_tail(g, held);
  // Each entry's workgroups start at a multiple of 8 (the XCD count), so the
  // block order inside it stays XCD-aware; padding slots are skipped.
  int64_t total = 0;
  for (int i = 0; i < g.count; ++i) {
    g.p[i].block0 = (int32_t)total;
    g.p[i].blocks = (int32_t)(((g.p[i].n - g.p[i].n_begin + tiled::BN - 1) / tiled::BN) *
                              ((g.p[i].m + g.p[i].bm - 1) / g.p[i].bm));
    total += (g.p[i].blocks + 7) / 8 * 8;
  }
  if (total == 0) return hipSuccess;
  if (total > INT32_MAX) return hipErrorInvalidValue;  // block numbers are 32-bit
  const int grid = total < held ? (int)total : held;
  g.total = (int32_t)total;
  group_width(g, BM, tiled::BN, grid / 8);
  log_plan("k_gemm_tiled", g, grid);
  hipLaunchKernelGGL((k_gemm_tiled<F32, BM>), dim3((unsigned)grid), dim3(512), lds_bytes, s, g);
  return hipGetLastError();
}

template <bool F32, int BM, int NG, int KS>
hipError_t launch_ws(gemm_group& g, hipStream_t s) {
  constexpr int BN = 64 * NG;
  constexpr int lds_bytes = wsk::STAGES * KS * wsk::step_bytes<BM, NG>();  // 144 KiB at 128 x 256
  static_assert(lds_bytes <= 160 * 1024, "LDS of one workgroup");
  static std::atomic<bool> lds_allowed[64] = {};
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(&k_gemm_ws<F32, BM, NG, KS>), lds_bytes, lds_allowed);
  if (e != hipSuccess) return e;
  int64_t total = 0;
  for (int i = 0; i < g.count; ++i) {
    g.p[i].block0 = (int32_t)total;
    g.p[i].blocks = (int32_t)(((g.p[i].n + BN - 1) / BN) * ((g.p[i].m + BM - 1) / BM));
    total += (g.p[i].blocks + 7) / 8 * 8;
  }
  if (total == 0) return hipSuccess;
  if (total > INT32_MAX) return hipErrorInvalidValue;  // block numbers are 32-bit
  static std::atomic<int> resident[64] = {};
  const int grid =
      persistent_grid(reinterpret_cast<const void*>(&k_gemm_ws<F32, BM, NG, KS>), 64 * wsk::WAVES, lds_bytes, resident, total);
  if (grid < 0) return hipErrorInvalidDevice;
  g.total = (int32_t)total;
  for (int i = 0; i < g.count; ++i) g.p[i].bm = BM;
  group_width(g, BM, BN, grid / 8);
  log_plan("k_gemm_ws", g, grid);
  hipLaunchKernelGGL((k_gemm_ws<F32, BM, NG, KS>), dim3((unsigned)grid), dim3(64 * wsk::WAVES), lds_bytes, s, g);
  return hipGetLastError();
}

// Workgroups of a launch of bn x bm blocks, each product padded to a multiple of 8.
int64_t padded_blocks(const gemm_group& g, int bm, int bn) {
  int64_t total = 0;
  for (int i = 0; i < g.count; ++i) total += (((g.p[i].n + bn - 1) / bn) * ((g.p[i].m + bm - 1) / bm) + 7) / 8 * 8;
  return total;
}

}  // namespace

int tiled_block_m(const gemm_group& g) {
  // Estimated time of each block height: rounds of 256 workgroups when every
  // product has the same K, else total cost spread over the CUs but never less
  // than the longest workgroup.  Block costs carry each product's dense / 2:4
  // mix (gemm_problem.mix).
  const int bms[4] = {256, 192, 128, 64};
  bool same_k = true;
  for (int i = 1; i < g.count; ++i) same_k = same_k && g.p[i].k == g.p[0].k;
  int best = 256;
  double best_t = 0;
  for (int j = 0; j < 4; ++j) {
    int64_t blocks = 0;
    double cost = 0, longest = 0;
    for (int i = 0; i < g.count; ++i) {
      const int64_t b = ((g.p[i].n + tiled::BN - 1) / tiled::BN) * ((g.p[i].m + bms[j] - 1) / bms[j]);
      const double c = block_cost(bms[j], g.p[i].k) * g.p[i].mix;
      blocks += b;
      cost += b * c;
      longest = longest > c ? longest : c;
    }
    const double t = same_k ? (double)((blocks + 255) / 256) * longest : (cost / 256 > longest ? cost / 256 : longest);
    if (j == 0 || t < best_t - 1e-9) {
      best = bms[j];
      best_t = t;
    }
  }
  return best;
}

hipError_t launch_tiled_group(gemm_group& g, int out_f32, int block_m, hipStream_t s) {
  // most expensive blocks first (K steps times the dense / 2:4 mix), so that
  // the cheaper ones fill the last round
  auto key = [](const gemm_problem& p) { return (double)p.k * p.mix; };
  for (int i = 1; i < g.count; ++i)
    for (int j = i; j > 0 && key(g.p[j]) > key(g.p[j - 1]); --j) {
      const gemm_problem t = g.p[j];
      g.p[j] = g.p[j - 1];
      g.p[j - 1] = t;
    }
  const int bm = block_m > 0 ? block_m : tiled_block_m(g);
  switch (bm) {
    case 64:
      // Two 64-row k_gemm_tiled workgroups share a CU and overlap each other;
      // when the grid gives each CU at most one, the warp-specialised kernel
      // (copies two steps ahead) is 15-20% faster (512 x 2048 at M = 4096),
      // and when it would leave half the CUs idle, blocks of 128 W rows
      // (twice the workgroups) are faster still.
      if (padded_blocks(g, 64, 256) <= 128)
        return out_f32 ? launch_ws<true, 64, 2, 2>(g, s) : launch_ws<false, 64, 2, 2>(g, s);
      if (padded_blocks(g, 64, 256) <= 256)
        return out_f32 ? launch_ws<true, 64, 4, 1>(g, s) : launch_ws<false, 64, 4, 1>(g, s);
      return out_f32 ? launch_tiled_bm<true, 64>(g, false, s) : launch_tiled_bm<false, 64>(g, false, s);
    case 128:
      return out_f32 ? launch_ws<true, 128, 4, 1>(g, s) : launch_ws<false, 128, 4, 1>(g, s);
    case 192:
      return out_f32 ? launch_tiled_bm<true, 192>(g, false, s) : launch_tiled_bm<false, 192>(g, false, s);
    default:
      return out_f32 ? launch_tiled_bm<true, 256>(g, block_m <= 0, s) : launch_tiled_bm<false, 256>(g, block_m <= 0, s);
  }
}

hipError_t launch_fill_zero_y(void* y, int64_t m, int64_t n, int64_t ldy, int out_f32, hipStream_t s) {
  const int64_t total = m * n;
  if (total <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (out_f32) hipLaunchKernelGGL(k_fill_zero_y<true>, dim3(grid), dim3(256), 0, s, y, m, n, ldy);
  else hipLaunchKernelGGL(k_fill_zero_y<false>, dim3(grid), dim3(256), 0, s, y, m, n, ldy);
  return hipGetLastError();
}
