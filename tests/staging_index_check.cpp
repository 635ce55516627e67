// Host check of the LDS-staging index arithmetic in tile_index.hpp (the same
// functions the staged kernels call).  For every copy, lane, chunk length and
// a range of row strides it confirms that
//   * each global byte offset a copy reads lies inside the chunk's rows
//     [0, len) and inside the 128 (row tile) or 32 (v block) columns it owns;
//   * a full chunk's split into wave-uniform and lane parts adds up to the
//     direct offset;
//   * the bytes every lane writes into LDS are where the kernels' readers
//     (rowtile_off, vtile_byte) look for them, and each tile is covered once;
//   * the output pieces leaving the v block cover its 64 x 32 outputs once.
// Prints "OK" and exits 0, or names the first violation and exits 1.
#include <cstdio>
#include <vector>

#include "tile_index.hpp"

using namespace gdn;

static int fails = 0;
#define CHECK(cond, ...)                    \
  do {                                      \
    if (!(cond)) {                          \
      if (fails < 10) {                     \
        std::printf("FAIL %s: ", #cond);    \
        std::printf(__VA_ARGS__);           \
        std::printf("\n");                  \
      }                                     \
      ++fails;                              \
    }                                       \
  } while (0)

int main() {
  const long long strides[] = {128, 256, 384, 2048, 4096, 128 * 64};
  for (long long s : strides) {
    // ---- row tile: 16 copies x 64 lanes ----
    for (int len = 1; len <= 64; ++len) {
      for (int i = 0; i < 16; ++i)
        for (int l = 0; l < 64; ++l) {
          const long long off = rowtile_copy_src(i, l, len, s);
          CHECK(off % 16 == 0, "row tile copy %d lane %d: offset %lld not 16-byte aligned", i, l, off);
          const long long e = off / 2, row = e / s, col = e % s;
          CHECK(row >= 0 && row < len, "row tile copy %d lane %d len %d stride %lld reads row %lld",
                i, l, len, s, row);
          CHECK(col >= 0 && col + 8 <= 128, "row tile copy %d lane %d reads columns %lld..+7", i, l, col);
          if (len == 64) {
            const long long split = rowtile_copy_uniform(i, s) + rowtile_copy_lane(i & 3, l, s);
            CHECK(split == off, "row tile copy %d lane %d stride %lld: uniform + lane = %lld, direct %lld",
                  i, l, s, split, off);
          }
        }
    }
    // ---- bounds-checked copies: full-chunk offsets against the valid size ----
    for (int len = 1; len <= 64; ++len) {
      const uint32_t row_bytes = uint32_t(2 * s);
      const uint32_t valid = rowtile_valid_bytes(len, row_bytes);
      for (int i = 0; i < 16; ++i)
        for (int l = 0; l < 64; ++l) {
          const long long off = rowtile_copy_src(i, l, 64, s);
          const bool in = rowtile_copy_row(i, l) < len;
          CHECK(in ? off + 16 <= valid : off >= valid,
                "row tile copy %d lane %d len %d stride %lld: offset %lld vs valid %u", i, l, len, s, off, valid);
        }
    }
  }
  // v rows can be as narrow as one 32-column block (64 bytes)
  for (long long s : {32LL, 64LL, 96LL, 128LL, 4096LL}) {
    for (int len = 1; len <= 64; ++len) {
      const uint32_t vvalid = vblock_valid_bytes(len, uint32_t(2 * s));
      for (int j = 0; j < 4; ++j)
        for (int l = 0; l < 64; ++l) {
          const long long off = vblock_copy_src(j, l, 64, s);
          const bool in = vblock_copy_row(j, l) < len;
          CHECK(in ? off + 16 <= vvalid : off >= vvalid,
                "v copy %d lane %d len %d stride %lld: offset %lld vs valid %u", j, l, len, s, off, vvalid);
        }
    }
    // ---- v block: 4 copies x 64 lanes ----
    for (int len = 1; len <= 64; ++len)
      for (int j = 0; j < 4; ++j)
        for (int l = 0; l < 64; ++l) {
          const long long off = vblock_copy_src(j, l, len, s);
          CHECK(off % 16 == 0, "v copy %d lane %d: offset %lld not aligned", j, l, off);
          const long long e = off / 2, row = e / s, col = e % s;
          CHECK(row >= 0 && row < len, "v copy %d lane %d len %d reads row %lld", j, l, len, row);
          CHECK(col >= 0 && col + 8 <= 32, "v copy %d lane %d reads columns %lld..+7", j, l, col);
        }
  }

  // ---- LDS placement: copy i, lane l writes bytes [1024 i + 16 l, +16) ----
  {
    std::vector<int> seen(64 * 128, 0);
    for (int i = 0; i < 16; ++i)
      for (int l = 0; l < 64; ++l) {
        const int row = rowtile_copy_row(i, l), col = 8 * rowtile_copy_block(i, l);
        const int at = 2 * rowtile_off(row, col);
        CHECK(at == 1024 * i + 16 * l, "row tile (%d,%d) read at byte %d, written at %d", row, col, at,
              1024 * i + 16 * l);
        for (int c = 0; c < 8; ++c) {
          CHECK(2 * rowtile_off(row, col + c) == at + 2 * c, "row tile (%d,%d) not contiguous", row, col + c);
          seen[row * 128 + col + c]++;
        }
      }
    for (int x = 0; x < 64 * 128; ++x) CHECK(seen[x] == 1, "row tile element %d copied %d times", x, seen[x]);
  }
  {
    std::vector<int> seen(64 * 32, 0);
    for (int j = 0; j < 4; ++j)
      for (int l = 0; l < 64; ++l) {
        const int row = vblock_copy_row(j, l), col = 8 * vblock_copy_block(j, l);
        const int at = vtile_byte(row, col);
        CHECK(at == 1024 * j + 16 * l, "v block (%d,%d) read at byte %d, written at %d", row, col, at,
              1024 * j + 16 * l);
        for (int c = 0; c < 8; ++c) {
          CHECK(vtile_byte(row, col + c) == at + 2 * c, "v block (%d,%d) not contiguous", row, col + c);
          seen[row * 32 + col + c]++;
        }
      }
    for (int x = 0; x < 64 * 32; ++x) CHECK(seen[x] == 1, "v block element %d copied %d times", x, seen[x]);
  }

  // ---- outputs: 2 copy waves x 2 row blocks x 2 column groups x 64 lanes, 4 columns each ----
  {
    std::vector<int> seen(64 * 32, 0), p_tiles(2, 0);
    for (int cw = 0; cw < 2; ++cw)
      for (int a = 0; a < 2; ++a) {
        const int rt = copy_rows(cw, a);
        CHECK(rt >= 0 && rt < 4, "copy wave %d row block %d", cw, rt);
        p_tiles[cw] += rt + 1;
        for (int cg = 0; cg < 2; ++cg)
          for (int l = 0; l < 64; ++l) {
            const int row = out_acc_row(rt, l), col = out_acc_col(cg, l);
            CHECK(row < 64 && col + 4 <= 32 && col % 4 == 0, "output tile %d lane %d at (%d,%d)", rt, l, row, col);
            CHECK(row == out_acc_row(0, l) + 16 * rt && col == out_acc_col(0, l) + 16 * cg,
                  "output tile %d lane %d offset", rt, l);
            for (int c = 0; c < 4; ++c) seen[row * 32 + col + c]++;
          }
      }
    for (int x = 0; x < 64 * 32; ++x) CHECK(seen[x] == 1, "output element %d written %d times", x, seen[x]);
    CHECK(p_tiles[0] == 5 && p_tiles[1] == 5, "P tiles per copy wave %d / %d", p_tiles[0], p_tiles[1]);
  }

  // ---- 16-column v block: 2 copies x 64 lanes cover 64 rows x 16 columns once ----
  for (int len = 1; len <= 64; ++len) {
    const int64_t stride = 32 * 128;  // elements between token rows (32 heads x 128)
    for (int j = 0; j < 2; ++j)
      for (int l = 0; l < 64; ++l) {
        const int64_t src = vblock16_copy_src(j, l, len, stride);
        const int row = vblock16_copy_row(j, l);
        CHECK(src >= 0 && src + 16 <= int64_t(vblock16_valid_bytes(len, uint32_t(2 * stride))),
              "v16 copy %d lane %d len %d reads past the chunk", j, l, len);
        CHECK(src / (2 * stride) == (row < len ? row : len - 1), "v16 copy %d lane %d row", j, l);
      }
  }
  {
    std::vector<int> seen(64 * 16, 0);
    for (int j = 0; j < 2; ++j)
      for (int l = 0; l < 64; ++l) {
        const int row = vblock16_copy_row(j, l), col = 8 * vblock16_copy_block(j, l);
        const int at = vtile16_byte(row, col);
        CHECK(at == 1024 * j + 16 * l, "v16 block (%d,%d) read at byte %d, written at %d", row, col, at, 1024 * j + 16 * l);
        for (int c = 0; c < 8; ++c) {
          CHECK(vtile16_byte(row, col + c) == at + 2 * c, "v16 block (%d,%d) not contiguous", row, col + c);
          seen[row * 16 + col + c]++;
        }
      }
    for (int x = 0; x < 64 * 16; ++x) CHECK(seen[x] == 1, "v16 block element %d copied %d times", x, seen[x]);
  }

  // ---- output staging, 16-column blocks: each copy wave writes its two row
  // blocks as 8-byte tile pieces and reads both back with one 16-byte piece
  // per lane ----
  {
    std::vector<int> wrote(64 * 16, -1), read(64 * 16, 0);
    for (int cw = 0; cw < 2; ++cw) {
      for (int a = 0; a < 2; ++a) {
        const int rt = copy_rows(cw, a);
        for (int l = 0; l < 64; ++l) {
          const int row = out_acc_row(rt, l), col = out_acc_col(0, l);
          const int base = out_stage16_byte(row, col);
          CHECK(base % 8 == 0 && base + 8 <= 2048, "staging16 write (%d,%d) at %d", row, col, base);
          for (int c = 0; c < 4; ++c) {
            CHECK(out_stage16_byte(row, col + c) == base + 2 * c, "staging16 write (%d,%d) not contiguous", row, col + c);
            CHECK(wrote[row * 16 + col + c] == -1, "output16 (%d,%d) staged twice", row, col + c);
            wrote[row * 16 + col + c] = cw;
          }
        }
      }
      for (int l = 0; l < 64; ++l) {
        const int rt = copy_rows(cw, l >> 5);
        const int row = out_piece16_row(rt, l), col = out_piece16_col(l);
        const int base = out_stage16_byte(row, col);
        CHECK(base % 16 == 0 && base + 16 <= 2048, "staging16 read (%d,%d) at %d", row, col, base);
        CHECK(row / 16 == rt, "read-back16 row %d outside row block %d", row, rt);
        for (int c = 0; c < 8; ++c) {
          CHECK(out_stage16_byte(row, col + c) == base + 2 * c, "staging16 read (%d,%d) not contiguous", row, col + c);
          CHECK(wrote[row * 16 + col + c] == cw, "output16 (%d,%d) read back by the other wave", row, col + c);
          read[row * 16 + col + c]++;
        }
      }
    }
    for (int x = 0; x < 64 * 16; ++x) CHECK(wrote[x] >= 0 && read[x] == 1, "output16 element %d", x);
  }

  // ---- T fragments: the six non-zero ones fill six distinct slots ----
  {
    std::vector<int> seen(6, 0);
    for (int f = 0; f < 8; ++f) {
      if (f == 1 || f == 3) continue;
      const int sl = t_slot(f);
      CHECK(sl >= 0 && sl < 6, "T fragment %d slot %d", f, sl);
      if (sl >= 0 && sl < 6) seen[sl]++;
    }
    for (int sl = 0; sl < 6; ++sl) CHECK(seen[sl] == 1, "T slot %d used %d times", sl, seen[sl]);
  }

  // ---- output staging: each copy wave writes its two row blocks as 8-byte
  // tile pieces and reads them back as 16-byte row pieces; every element is
  // written once and read back once, each wave reads only what it wrote, and
  // the staging buffer's 4 KiB hold the whole block ----
  {
    std::vector<int> wrote(64 * 32, -1), read(64 * 32, 0), at(64 * 32, -1);
    for (int cw = 0; cw < 2; ++cw)
      for (int a = 0; a < 2; ++a) {
        const int rt = copy_rows(cw, a);
        for (int cg = 0; cg < 2; ++cg)
          for (int l = 0; l < 64; ++l) {
            const int row = out_acc_row(rt, l), col = out_acc_col(cg, l);
            const int base = out_stage_byte(row, col);
            CHECK(base % 8 == 0 && base + 8 <= 4096, "staging write (%d,%d) at %d", row, col, base);
            for (int c = 0; c < 4; ++c) {
              CHECK(out_stage_byte(row, col + c) == base + 2 * c, "staging write (%d,%d) not contiguous", row, col + c);
              CHECK(wrote[row * 32 + col + c] == -1, "output (%d,%d) staged twice", row, col + c);
              wrote[row * 32 + col + c] = cw;
              at[row * 32 + col + c] = out_stage_byte(row, col + c);
            }
          }
        for (int l = 0; l < 64; ++l) {
          const int row = out_piece_row(rt, l), col = out_piece_col(l);
          const int base = out_stage_byte(row, col);
          CHECK(base % 16 == 0 && base + 16 <= 4096, "staging read (%d,%d) at %d", row, col, base);
          CHECK(row / 16 == rt, "read-back row %d outside row block %d", row, rt);
          for (int c = 0; c < 8; ++c) {
            CHECK(out_stage_byte(row, col + c) == base + 2 * c, "staging read (%d,%d) not contiguous", row, col + c);
            read[row * 32 + col + c]++;
          }
        }
      }
    std::vector<int> bytes(4096, 0);
    for (int x = 0; x < 64 * 32; ++x) {
      CHECK(wrote[x] >= 0 && read[x] == 1, "output element %d staged %d / read %d times", x, wrote[x] >= 0, read[x]);
      if (at[x] >= 0) bytes[at[x]]++;
    }
    for (int b = 0; b < 4096; b += 2) CHECK(bytes[b] == 1, "staging byte %d holds %d elements", b, bytes[b]);
  }

  if (fails) {
    std::printf("%d violations\n", fails);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
