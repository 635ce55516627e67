// Index arithmetic of the LDS-staged chunk operands (bf16).  Pure functions,
// used by the kernels and also compiled for the host, where a check walks
// every copy, lane and chunk length and confirms that each global byte a
// staging copy reads lies inside the chunk's rows and that the LDS tiles are
// covered exactly once.
//
// Row tile: 64 token rows x 128 bf16 (256 B per row) in 16 copies of 1 KiB.
// Copy i moves rows 4 i .. 4 i + 3; lane l moves row 4 i + l / 16 and writes
// physical 16-byte block l mod 16 of that row, which holds source block
// (l mod 16) ^ (row mod 16) -- the XOR swizzle that spreads an MFMA
// fragment's 16 rows over distinct banks.
//
// v block: 64 token rows x 32 bf16 (64 B per row) in 4 copies of 1 KiB; copy
// j moves rows 16 j .. 16 j + 15, lane l moves row 16 j + l / 4, physical
// block l mod 4, source block (l mod 4) ^ ((row / 4) mod 4).
//
// Rows at or past a partial chunk's length repeat row len - 1 (finite,
// in-bounds filler that the chunk algebra multiplies by exact zeros).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gdn {

__host__ __device__ constexpr int clamp_row(int row, int len) { return row < len ? row : len - 1; }

// ---- row tile ----
// Element offset of logical (row, col) in a swizzled row tile.
__host__ __device__ constexpr int rowtile_off(int row, int col) {
  return row * 128 + 8 * ((col >> 3) ^ (row & 15)) + (col & 7);
}
__host__ __device__ constexpr int rowtile_copy_row(int i, int lane) { return 4 * i + (lane >> 4); }
__host__ __device__ constexpr int rowtile_copy_block(int i, int lane) {
  return (lane & 15) ^ (rowtile_copy_row(i, lane) & 15);
}
// Source byte offset (from the chunk's first row) that lane `lane` of copy
// `i` reads, rows clamped to `len`; `stride` is the row stride in elements.
__host__ __device__ constexpr int64_t rowtile_copy_src(int i, int lane, int len, int64_t stride) {
  return 2 * (int64_t(clamp_row(rowtile_copy_row(i, lane), len)) * stride +
              8 * rowtile_copy_block(i, lane));
}
// A full chunk's offset split into a wave-uniform part for copy i ...
__host__ __device__ constexpr int64_t rowtile_copy_uniform(int i, int64_t stride) {
  return int64_t(8) * i * stride;  // 4 i rows of 2-byte elements
}
// ... and a lane part that depends on the copy only through i mod 4.
__host__ __device__ constexpr uint32_t rowtile_copy_lane(int i, int lane, int64_t stride) {
  return uint32_t(2 * (int64_t(lane >> 4) * stride + 8 * rowtile_copy_block(i, lane)));
}

// Bytes of a chunk's row-tile source that are valid when it has `len` rows
// (row stride `row_bytes` >= 256): rows below len lie wholly inside, and every
// copy of a row at or past len starts at or beyond the end.
__host__ __device__ constexpr uint32_t rowtile_valid_bytes(int len, uint32_t row_bytes) {
  return uint32_t(len - 1) * row_bytes + 256;
}

// ---- v block ----
__host__ __device__ constexpr int vblock_copy_row(int j, int lane) { return 16 * j + (lane >> 2); }
__host__ __device__ constexpr int vblock_copy_block(int j, int lane) {
  return (lane & 3) ^ ((vblock_copy_row(j, lane) >> 2) & 3);
}
__host__ __device__ constexpr int64_t vblock_copy_src(int j, int lane, int len, int64_t stride) {
  return 2 * (int64_t(clamp_row(vblock_copy_row(j, lane), len)) * stride +
              8 * vblock_copy_block(j, lane));
}

// Same for a v block source (row stride `row_bytes` >= 64).
__host__ __device__ constexpr uint32_t vblock_valid_bytes(int len, uint32_t row_bytes) {
  return uint32_t(len - 1) * row_bytes + 64;
}

// Byte offset of logical (row, col) in the staged v block.
__host__ __device__ constexpr int vtile_byte(int row, int col) {
  return 2 * (row * 32 + 8 * ((col >> 3) ^ ((row >> 2) & 3)) + (col & 7));
}

// ---- v block, 16 columns (a block of one column group) ----
// 64 token rows x 16 bf16 (32 B per row) in 2 copies of 1 KiB; copy j moves
// rows 32 j .. 32 j + 31, lane l moves row 32 j + l / 2, physical block
// l mod 2, source block (l mod 2) ^ ((row / 4) mod 2).
__host__ __device__ constexpr int vblock16_copy_row(int j, int lane) { return 32 * j + (lane >> 1); }
__host__ __device__ constexpr int vblock16_copy_block(int j, int lane) {
  return (lane & 1) ^ ((vblock16_copy_row(j, lane) >> 2) & 1);
}
__host__ __device__ constexpr int64_t vblock16_copy_src(int j, int lane, int len, int64_t stride) {
  return 2 * (int64_t(clamp_row(vblock16_copy_row(j, lane), len)) * stride + 8 * vblock16_copy_block(j, lane));
}
__host__ __device__ constexpr uint32_t vblock16_valid_bytes(int len, uint32_t row_bytes) {
  return uint32_t(len - 1) * row_bytes + 32;
}
// Byte offset of logical (row, col) in the staged 16-column v block.
__host__ __device__ constexpr int vtile16_byte(int row, int col) {
  return 2 * (row * 16 + 8 * ((col >> 3) ^ ((row >> 2) & 1)) + (col & 7));
}

// ---- outputs as the MFMA leaves them (transposed tiles) ----
// Output tile rt, lane l: token row 16 rt + l mod 16, columns
// 16 cg + 4 (l / 16) .. + 3 of column group cg of the block.
__host__ __device__ constexpr int out_acc_row(int rt, int lane) { return 16 * rt + (lane & 15); }
__host__ __device__ constexpr int out_acc_col(int cg, int lane) { return 16 * cg + 4 * (lane >> 4); }

// ---- T fragments in a stage ----
// LDS slot of T fragment f: fragments 1 and 3 (rows 0-31 x columns 32-63 of
// the lower-triangular T) are zero and not staged; the other six fill slots
// 0-5.
__host__ __device__ constexpr int t_slot(int f) { return f < 4 ? f / 2 : f - 2; }

// ---- T fragments in a staged workspace entry ----
// Fragments 0 and 5 (rows 0-15 x columns 0-31 and rows 32-47 x columns
// 32-63) lie on T's diagonal: their elements 4-7 in every lane (contraction
// indices 16-31 of the fragment, above the diagonal) are zero.  The entry
// keeps only elements 0-3 of those two, 64 lanes x 8 bytes; the other four
// are whole, 64 lanes x 16 bytes.  Byte offset of fragment f in the entry:
__host__ __device__ constexpr bool t_compact(int f) { return f == 0 || f == 5; }
__host__ __device__ constexpr int t_entry_byte(int f) {
  return f == 0 ? 0 : f == 2 ? 512 : f == 4 ? 1536 : f == 5 ? 2560 : f == 6 ? 3072 : 4096;
}

// ---- outputs leaving through the output staging buffer ----
// 64 token rows x 32 bf16 (64 bytes per row), 16-byte pieces XOR-swizzled by
// the row: physical piece = piece ^ ((row / 4) mod 4).
__host__ __device__ constexpr int out_stage_byte(int row, int col) {
  return row * 64 + 16 * (((col >> 3) ^ (row >> 2)) & 3) + 2 * (col & 7);
}
// Read-back piece of lane l in row block rt: row 16 rt + l / 4, columns
// 8 (l mod 4) .. + 7 (one 16-byte piece; 16 rows x 64 bytes per instruction).
__host__ __device__ constexpr int out_piece_row(int rt, int lane) { return 16 * rt + (lane >> 2); }
__host__ __device__ constexpr int out_piece_col(int lane) { return 8 * (lane & 3); }

// The same for a 16-column block (32 bytes per row; physical piece =
// piece ^ ((row / 4) mod 2)).  Read-back: lane l stores row
// 16 rt + (l mod 32) / 2 of row block rt = copy_rows(cw, l / 32), columns
// 8 (l mod 2) .. + 7 -- both row blocks of a copy wave in one instruction.
__host__ __device__ constexpr int out_stage16_byte(int row, int col) {
  return row * 32 + 16 * (((col >> 3) ^ (row >> 2)) & 1) + 2 * (col & 7);
}
__host__ __device__ constexpr int out_piece16_row(int rt, int lane) { return 16 * rt + ((lane & 31) >> 1); }
__host__ __device__ constexpr int out_piece16_col(int lane) { return 8 * (lane & 1); }

// Token row blocks (of P and of the outputs) that copy wave cw = 0, 1 owns:
// {0, 3} and {1, 2}.  Row block rt of the lower-triangular P has rt + 1
// tiles of 16 x 16, so each copy wave forms five.
__host__ __device__ constexpr int copy_rows(int cw, int a) { return cw == 0 ? (a == 0 ? 0 : 3) : (a == 0 ? 1 : 2); }

}  // namespace gdn
