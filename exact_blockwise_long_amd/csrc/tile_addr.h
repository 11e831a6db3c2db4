// Byte addressing of the K/V tile loads (HBM -> LDS) of the bf16 kernels.
//
// Plain integer arithmetic with no HIP builtins, so that the same functions
// serve the device code and a host-side checker that enumerates every lane of
// every tile for ragged key counts.
//
// A tile load is `buffer_load_dwordx4 ... lds` through a buffer resource.  The
// hardware range check of a raw buffer (stride 0) compares only the per-lane
// offset (VGPR offset plus the instruction's immediate offset) with the
// resource's num_records; the scalar offset operand is added to the address
// after the check.  A load whose per-lane offset is at or past num_records
// returns zeros and touches no memory.  So the kernels put everything that
// must be checked into the per-lane offset: each tile gets its own resource
// whose base is the tile's first key and whose num_records ends at the last
// byte of the last key the tile may read, and the scalar offset is always 0.
#pragma once

#include <stdint.h>

#ifndef BA_HD
#define BA_HD __host__ __device__
#endif

namespace ba {

// Chunk swizzle of every LDS tile: global 16-byte chunk c of tile row r sits
// at chunk c ^ swz(r).  Tiles are read two ways: 16-byte row reads (lane l
// reads row l % 16 of a 16-row block, chunk 4*dc + l / 16) and transposing
// 8-byte reads (lane l reads 8 bytes of row 4*(l / 16) + (l % 16) / 4 of a
// 16-row block, chunk pair 2*db + {0, 1}).  LDS has 64 banks of 4 bytes;
// measured with a one-wave probe on the bank-conflict counter, a 16-byte read
// is served in four 16-lane passes, each pairing lanes 8a .. 8a + 7 of one
// quarter-wave with eight lanes of the other half of an odd quarter-wave, and
// a transposing read in two 32-lane passes.  For D = 128 (one row per bank
// line) (r & 7) << 1 keeps both kinds conflict-free, while r & 15 doubles the
// transposing reads' passes; for D = 64 (two rows per bank line) r & 7 does.
template <int D>
BA_HD inline int swz(int row) {
  return D == 128 ? ((row & 7) << 1) : (row & 7);
}

// Geometry of the wave-wide loads of one TK-key tile for head_dim D and W
// waves: each load moves 1 KiB, RPI whole rows of D bf16; wave w issues loads
// j = 0 .. LPW-1 of K (and the same of V), covering rows
// (w * LPW + j) * RPI .. + RPI - 1.
template <int D, int W, int TK>
struct TileGeom {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;       // rows per wave-wide load
  static constexpr int LPW = TK / RPI / W;   // loads per wave per tile (each of K and V)
  static_assert(LPW * RPI * W == TK, "a tile must split evenly over the waves' loads");
};

// Tile row (key index within the tile) that lane `lane` of wave `wave` moves
// in its load j.
template <int D, int W, int TK>
BA_HD inline int tile_lane_row(int wave, int lane, int j) {
  using G = TileGeom<D, W, TK>;
  return (wave * G::LPW + j) * G::RPI + lane / G::CPR;
}

// Per-lane byte offset, from the tile's first key, of the 16-byte chunk that
// lane `lane` of wave `wave` moves in its load j: the lane at chunk position
// p of its row fetches global chunk p ^ swz(row), which is where the operand
// reads look for it.  `stride` is the byte distance between keys.
template <int D, int W, int TK>
BA_HD inline uint32_t tile_lane_offset(uint32_t stride, int wave, int lane, int j) {
  using G = TileGeom<D, W, TK>;
  const int row = tile_lane_row<D, W, TK>(wave, lane, j);
  const int p = lane % G::CPR;
  return (uint32_t)row * stride + (uint32_t)((p ^ swz<D>(row)) * 16);
}

// num_records of the resource of the tile whose first key is key k0 of a
// range whose first n keys may be read (0 <= k0 < n): the bytes from key k0
// to the end of key n - 1.  With stride >= 2 * D (a key's row never overlaps
// the next key's), a lane moving key k0 + r gets an offset wholly inside the
// range when r < n - k0 and at or past num_records when r >= n - k0.
template <int D>
BA_HD inline uint32_t tile_records(int n, int k0, uint32_t stride) {
  return (uint32_t)(n - k0 - 1) * stride + (uint32_t)(2 * D);
}

}  // namespace ba
