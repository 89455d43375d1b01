// Layout of the packed key/value buffer written by bsa_kv_pack and read by
// bsa_sparse_attention.
#pragma once

#include "common.hpp"

namespace bsa {

constexpr int kPackTile = 64;  // keys per packed tile

// Byte offsets of the packed buffer's sections, and its tile counts.  `nl` key layouts: 1 (one
// layout shared by every head) or B*Hkv (one per (batch, K/V head), layout b*Hkv + kvh).
//   hmix      int32 [B*Hkv]            nonzero when some V^T tile of the head is bfloat16
//   flags     uint8 [B*Hkv][tiles]     V^T tile format: 1 = float16 / float32, 0 = bfloat16
//   k         T     [B*Hkv][tiles][64][D]
//   v         [B*Hkv][tiles][D][64]    16-bit for bfloat16 inputs, float32 for float32 inputs;
//                                      within each group of 16 keys the positions hold keys
//                                      0-3, 8-11, 4-7, 12-15
//   tile_off  int32 [nl][C + 1]        first tile of each key cluster in the head's tiles
//   clog2n    float [nl][C]            log2 of the count n_c that weighs centroid column c
//                                      (-inf for n_c = 0: the column vanishes)
// The tile sections do not depend on nl.  Per head, token tiles come first (sum over clusters
// of ceil(n_c / 64) <= ceil(S/64) + C of them), then ceil(C / 64) centroid tiles starting at
// first_centroid_tile.
struct PackLayout {
  size_t tile_off, hmix, flags, k, v, clog2n, total;
  int tiles_per_head, first_centroid_tile, centroid_tiles;
};

inline size_t pack_align(size_t x) { return (x + 255) / 256 * 256; }

inline PackLayout pack_layout(int B, int Hkv, int S, int D, int C, size_t elem, int nl = 1) {
  PackLayout L;
  const int tok_tiles = (S + kPackTile - 1) / kPackTile + C;
  L.centroid_tiles = (C + kPackTile - 1) / kPackTile;
  L.first_centroid_tile = tok_tiles;
  L.tiles_per_head = tok_tiles + L.centroid_tiles;
  const size_t nt = static_cast<size_t>(B) * Hkv * L.tiles_per_head;
  size_t off = 0;
  L.hmix = off;
  off = pack_align(off + static_cast<size_t>(B) * Hkv * 4);
  L.flags = off;
  off = pack_align(off + nt);
  L.k = off;
  off = pack_align(off + nt * kPackTile * D * elem);
  L.v = off;
  off = pack_align(off + nt * kPackTile * D * elem);
  L.tile_off = off;
  off = pack_align(off + static_cast<size_t>(nl) * (static_cast<size_t>(C) + 1) * 4);
  L.clog2n = off;
  off = pack_align(off + static_cast<size_t>(nl) * C * 4);
  L.total = off;
  return L;
}

// Layout of (batch x K/V head) bkv among nl layouts.
__host__ __device__ inline size_t layout_of(int nl, size_t bkv) { return nl == 1 ? 0 : bkv; }

}  // namespace bsa
