// Operand-order layout of the packed pools on the device.
//
// The GEMM feeds W to smfmac 16x16x64 as the A operand, one 16-row block and
// one 64-wide K step at a time: unit u = step * (TN / 16) + block,
// for step < TK / 64 and block < TN / 16.  Lane l = 16 q + r of a wave holds
// row r of the block.  Each unit of a tile is stored as exactly the 64 lane
// operands, in lane order, so that one 16-byte load per lane fetches a whole
// operand (1 KiB contiguous per wave):
//
//   2:4 values  [slot][u][lane] 8 bf16: the 8 kept values of dense k = 16 q ..
//               16 q + 15 of the step (two per group of four, ascending k), the
//               A operand of v_smfmac_f32_16x16x64_bf16.
//   2:4 codes   [slot][u / 4][lane][u % 4] u16: the 4-bit code i0 | i1 << 2 of
//               group g of those 16 k at bits 4 g .. 4 g + 3 (the smfmac index
//               operand); the codes of the four blocks of a 64-row group sit
//               together, 8 bytes per lane.
//   dense       [slot][u][half][lane] 8 bf16: of the lane's 16 k (16 q .. 16 q
//               + 15), half 0 holds positions 0 and 1 of each group of four
//               and half 1 positions 2 and 3, so that a dense step runs as two
//               smfmacs with the constant codes 0x4444 and 0xEEEE.
//
// Pool sizes equal those of the row-major format (2 TN TK, TN TK and TN TK / 8
// bytes per tile).  These functions map a row-major position inside one tile
// to its element index inside the tile's slot of the device pool (the pack and
// unpack kernels write and read this layout); the host-side import and export
// convert with them.  Plain constexpr arithmetic, usable from host and device
// code alike.
#pragma once

#include <stdint.h>

namespace patch_layout {

// dense tile, bf16 element (row, col) -> index in uint16 units
constexpr int64_t dense_index(int64_t row, int64_t col, int64_t tn) {
  const int64_t step = col >> 6, cc = col & 63;
  const int64_t q = cc >> 4, within = cc & 15, pair = within >> 1;  // pair p: positions 2(p&1), +1 of group p>>1
  const int64_t u = step * (tn >> 4) + (row >> 4);
  return u * 1024 + (pair & 1) * 512 + (q * 16 + (row & 15)) * 8 + (pair >> 1) * 2 + (within & 1);
}

// 2:4 tile, kept value c (0 .. TK/2 - 1, two per group) of row `row` -> index in uint16 units
constexpr int64_t sparse_value_index(int64_t row, int64_t c, int64_t tn) {
  const int64_t step = c >> 5, q = (c & 31) >> 3, j = c & 7;
  const int64_t u = step * (tn >> 4) + (row >> 4);
  return u * 512 + (q * 16 + (row & 15)) * 8 + j;
}

// 2:4 tile, code byte b (0 .. TK/8 - 1, groups 2b and 2b + 1) of row `row` -> byte index
constexpr int64_t sparse_code_index(int64_t row, int64_t b, int64_t tn) {
  const int64_t step = b >> 3, bb = b & 7, q = bb >> 1;
  const int64_t u = step * (tn >> 4) + (row >> 4);
  return (u >> 2) * 512 + (q * 16 + (row & 15)) * 8 + (u & 3) * 2 + (bb & 1);
}

}  // namespace patch_layout

// Host conversions between the device pools (operand order) and the row-major
// exported format, `tiles` tile slots each.  Source and destination hold
// exactly the pool sizes above; every destination element is written once.
namespace patch_layout {

inline void dense_to_row_major(const uint16_t* dev, uint16_t* rm, int64_t tiles, int64_t tn, int64_t tk) {
  for (int64_t s = 0; s < tiles; ++s)
    for (int64_t row = 0; row < tn; ++row)
      for (int64_t col = 0; col < tk; ++col)
        rm[(s * tn + row) * tk + col] = dev[s * tn * tk + dense_index(row, col, tn)];
}

inline void dense_from_row_major(const uint16_t* rm, uint16_t* dev, int64_t tiles, int64_t tn, int64_t tk) {
  for (int64_t s = 0; s < tiles; ++s)
    for (int64_t row = 0; row < tn; ++row)
      for (int64_t col = 0; col < tk; ++col)
        dev[s * tn * tk + dense_index(row, col, tn)] = rm[(s * tn + row) * tk + col];
}

inline void sparse_values_to_row_major(const uint16_t* dev, uint16_t* rm, int64_t tiles, int64_t tn, int64_t tk) {
  for (int64_t s = 0; s < tiles; ++s)
    for (int64_t row = 0; row < tn; ++row)
      for (int64_t c = 0; c < tk / 2; ++c)
        rm[(s * tn + row) * (tk / 2) + c] = dev[s * tn * tk / 2 + sparse_value_index(row, c, tn)];
}

inline void sparse_values_from_row_major(const uint16_t* rm, uint16_t* dev, int64_t tiles, int64_t tn, int64_t tk) {
  for (int64_t s = 0; s < tiles; ++s)
    for (int64_t row = 0; row < tn; ++row)
      for (int64_t c = 0; c < tk / 2; ++c)
        dev[s * tn * tk / 2 + sparse_value_index(row, c, tn)] = rm[(s * tn + row) * (tk / 2) + c];
}

inline void sparse_codes_to_row_major(const uint8_t* dev, uint8_t* rm, int64_t tiles, int64_t tn, int64_t tk) {
  for (int64_t s = 0; s < tiles; ++s)
    for (int64_t row = 0; row < tn; ++row)
      for (int64_t b = 0; b < tk / 8; ++b)
        rm[(s * tn + row) * (tk / 8) + b] = dev[s * tn * tk / 8 + sparse_code_index(row, b, tn)];
}

inline void sparse_codes_from_row_major(const uint8_t* rm, uint8_t* dev, int64_t tiles, int64_t tn, int64_t tk) {
  for (int64_t s = 0; s < tiles; ++s)
    for (int64_t row = 0; row < tn; ++row)
      for (int64_t b = 0; b < tk / 8; ++b)
        dev[s * tn * tk / 8 + sparse_code_index(row, b, tn)] = rm[(s * tn + row) * (tk / 8) + b];
}

}  // namespace patch_layout
