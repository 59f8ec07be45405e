// Host-side check of the LDS tile layout helpers of ra_device.h (swizzle, MFMA
// operand read offsets): every lane's read offsets address the rows and 16-byte
// chunks its MFMA operand needs, and both read patterns are free of bank
// conflicts.  Prints "ok" and exits 0, or prints the first mismatch and exits 1.
#include <cstdio>
#include <set>

#include "../context_long_sequence_amd/csrc/ra_device.h"

using namespace ra;

static int fails = 0;
static void expect(bool c, const char* what, int a, int b, int x) {
  if (!c && fails++ < 10) std::printf("mismatch: %s (%d, %d, %d)\n", what, a, b, x);
}

int main() {
  for (int lane = 0; lane < 64; ++lane) {
    const int half = lane >> 5, col = lane & 31;
    // Row reads (A operand of S = Q K^T): lane reads chunk 2s + half of row
    // key_of_row(col) of a 32-row block.
    const int A = row_read_base(lane);
    for (int s = 0; s < 8; ++s)
      expect((A ^ (s << 5)) == tile_off(key_of_row(col), 2 * s + half), "row read", lane, s, 0);
    // Transposing reads: lane m + 4k of a 16-lane group addresses row r0 + k at
    // columns c0 + 4m .. +3 (8 bytes); rows 16*half + 8m' + k (B0) and + 4 (B1),
    // 32-column block db.
    const TrBases tb = tr_bases(lane);
    const int s16 = lane & 15, mm = s16 & 3, kk = s16 >> 2;
    for (int m = 0; m < 2; ++m)
      for (int db = 0; db < 4; ++db) {
        const int col0 = 32 * db + 16 * ((lane >> 4) & 1) + 4 * mm;  // first of this lane's 4 columns
        const int chunk = col0 / 8, sub = (col0 % 8) * 2;            // 16-byte chunk, byte offset in it
        const int r0 = 16 * half + 8 * m + kk;
        expect(((tb.b0 ^ (db << 6)) + 2048 * m) == tile_off(r0, chunk) + sub, "tr read B0", lane, m, db);
        expect(((tb.b1 ^ (db << 6)) + 2048 * m) == tile_off(r0 + 4, chunk) + sub, "tr read B1", lane, m, db);
      }
  }
  // Bank conflicts (64 banks of 4 bytes).  Row reads: each group of 16 lanes reads
  // 16 x 16 bytes that must cover 64 distinct banks.
  for (int g = 0; g < 4; ++g)
    for (int s = 0; s < 8; ++s) {
      std::set<int> banks;
      for (int lane = 16 * g; lane < 16 * g + 16; ++lane) {
        const int off = row_read_base(lane) ^ (s << 5);
        for (int w = 0; w < 4; ++w) banks.insert((off / 4 + w) % 64);
      }
      expect(banks.size() == 64, "row-read banks", g, s, (int)banks.size());
    }
  // Transposing reads: each group of 32 lanes reads 32 x 8 bytes over 64 distinct banks.
  for (int g = 0; g < 2; ++g)
    for (int m = 0; m < 2; ++m)
      for (int db = 0; db < 4; ++db)
        for (int which = 0; which < 2; ++which) {
          std::set<int> banks;
          for (int lane = 32 * g; lane < 32 * g + 32; ++lane) {
            const TrBases tb = tr_bases(lane);
            const int off = ((which ? tb.b1 : tb.b0) ^ (db << 6)) + 2048 * m;
            for (int w = 0; w < 2; ++w) banks.insert((off / 4 + w) % 64);
          }
          expect(banks.size() == 64, "transposing-read banks", g, m * 4 + db, (int)banks.size());
        }
  if (fails) return 1;
  std::printf("ok\n");
  return 0;
}
