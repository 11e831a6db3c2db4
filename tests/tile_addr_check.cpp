// Host-side check of the K/V tile addressing the bf16 kernels use
// (exact_blockwise_long_amd/csrc/tile_addr.h), built with g++ by
// tests/test_tile_addr_cpu.py.
//
// For every tile configuration the kernels launch, head_dim, key stride and
// key count n up to several tiles (ragged tails included), and every tile
// start k0 < n, it enumerates each lane's 16-byte load and checks:
//   * the tile's (row, chunk) pairs are each loaded exactly once, and each
//     lands where the swizzled operand reads look for it;
//   * a lane whose key is below n has a per-lane offset wholly inside the
//     resource (offset + 16 <= num_records), and its absolute bytes lie inside
//     that key's row;
//   * a lane whose key is at or past n has a per-lane offset at or past
//     num_records, so the range check returns zeros and no memory is touched.
// The scalar offset is always 0 (the range check ignores it), so the per-lane
// offset is the whole offset from the tile's base.
// Prints "ok <cases>" and exits 0, or prints the first failure and exits 1.
#define BA_HD
#include "tile_addr.h"

#include <cstdio>
#include <vector>

namespace {

long long g_cases = 0;

template <int D, int W, int TK>
bool check(uint32_t stride, int n) {
  using G = ba::TileGeom<D, W, TK>;
  for (int k0 = 0; k0 < n; k0 += TK) {
    const uint32_t rec = ba::tile_records<D>(n, k0, stride);
    std::vector<int> seen(TK * G::CPR, 0);
    for (int wave = 0; wave < W; ++wave)
      for (int lane = 0; lane < 64; ++lane)
        for (int j = 0; j < G::LPW; ++j) {
          ++g_cases;
          const int row = ba::tile_lane_row<D, W, TK>(wave, lane, j);
          const uint32_t off = ba::tile_lane_offset<D, W, TK>(stride, wave, lane, j);
          if (row < 0 || row >= TK) {
            std::printf("D=%d W=%d TK=%d: row %d outside the tile\n", D, W, TK, row);
            return false;
          }
          // LDS placement: lane `lane` of load j writes 16 bytes at row
          // (w*LPW + j)*RPI + lane / CPR, chunk position lane % CPR, which must
          // hold global chunk (lane % CPR) ^ swz(row).
          const int p = lane % G::CPR;
          const int chunk = p ^ ba::swz<D>(row);
          if (chunk < 0 || chunk >= G::CPR) {
            std::printf("D=%d: swizzled chunk %d out of the row\n", D, chunk);
            return false;
          }
          if (off != (uint32_t)row * stride + (uint32_t)chunk * 16) {
            std::printf("D=%d W=%d TK=%d stride=%u: lane offset %u does not address row %d chunk %d\n", D, W,
                        TK, stride, off, row, chunk);
            return false;
          }
          ++seen[row * G::CPR + chunk];
          const int key = k0 + row;
          if (key < n) {
            if ((uint64_t)off + 16 > rec) {
              std::printf("D=%d W=%d TK=%d stride=%u n=%d k0=%d: key %d (in range) offset %u + 16 > records %u\n",
                          D, W, TK, stride, n, k0, key, off, rec);
              return false;
            }
            const uint64_t abs = (uint64_t)k0 * stride + off;
            if (abs < (uint64_t)key * stride || abs + 16 > (uint64_t)key * stride + 2 * D) {
              std::printf("D=%d stride=%u: bytes of key %d leave its row\n", D, stride, key);
              return false;
            }
          } else if (off < rec) {
            std::printf("D=%d W=%d TK=%d stride=%u n=%d k0=%d: key %d (past the range) offset %u < records %u\n",
                        D, W, TK, stride, n, k0, key, off, rec);
            return false;
          }
        }
    for (int i = 0; i < TK * G::CPR; ++i)
      if (seen[i] != 1) {
        std::printf("D=%d W=%d TK=%d: row %d chunk %d loaded %d times\n", D, W, TK, i / G::CPR, i % G::CPR,
                    seen[i]);
        return false;
      }
  }
  return true;
}

template <int D, int W, int TK>
bool sweep() {
  // Strides in bytes: one KV head (2D), GQA with 8 KV heads, a row with extra
  // padding, and K/V as views into a fused [tokens, 2, Hkv, D] buffer.
  const uint32_t strides[] = {2 * D, 2 * D + 16, 16 * D, 2 * 2 * 8 * D};
  for (uint32_t st : strides)
    for (int n = 1; n <= 3 * TK + 5; ++n)
      if (!check<D, W, TK>(st, n)) return false;
  return true;
}

}  // namespace

int main() {
  // (waves, keys per tile) of every launch: the walk and the wide split (8, 128),
  // the narrow split and the fan-out (4, 64), the wide fan-out and the dQ walk (8, 64).
  const bool ok = sweep<128, 8, 128>() && sweep<128, 4, 64>() && sweep<128, 8, 64>() && sweep<64, 8, 128>() &&
                  sweep<64, 4, 64>() && sweep<64, 8, 64>();
  if (!ok) return 1;
  std::printf("ok %lld\n", g_cases);
  return 0;
}
