// Tile geometry and tile-map entries shared by the kernels and the host side
// of the attention-JVP library.  Not part of the public C ABI.
#pragma once

#include <stdint.h>

namespace aj {

// Tile geometry of the kernels.  Every instantiation (bf16 / fp32, D = 64 / 128)
// uses 128 query rows per workgroup and 64 keys per streamed tile, so one key
// bitmask row is one 64-bit word.
constexpr int kTileM = 128;
constexpr int kTileN = 64;
// Query rows per workgroup of the primal forward at head_dim 128: eight
// 32-row waves (two per SIMD, one workgroup per CU) share one key stream, half
// the key-tile traffic per FLOP of two 128-row workgroups.  It has a tile map
// of its own (aj_mask_desc::rows_w).
constexpr int kTileMWide = 256;

// Which tangents a (query tile, key tile) pair carries, from the caller's
// declaration of tokens whose tangents are zero (Entry::flags).  Only the
// tokens taking part in the tile count: the keys that some query of the tile
// may attend, and the queries attending one of them (a masked pair has P = 0
// and its tS is set to 0, whatever the tangents).
//   kTileJvp       the general case: every product of the JVP
//   kTileKeysFree  tK = tV = 0 on every taking-part key: tS = c tQ K^T and
//                  (A + B) gets only (P.tS) V
//   kTileAllFree   tQ = tK = tV = 0 on every taking-part token: tS = 0, so only
//                  the primal products remain
// A query-tangent-free tile whose keys carry tangents runs as kTileJvp (tQ is
// zero there and simply multiplies in).
constexpr int32_t kTileJvp = 0;
constexpr int32_t kTileKeysFree = 1;
constexpr int32_t kTileAllFree = 3;

// One run of key tiles visited by a query tile.  pidx < 0: every tile in
// [kt0, kt1) is full.  pidx >= 0: the single tile kt0 (kt1 = kt0 + 1) is
// partial and its per-row key bitmask starts at bits[pidx * kTileM].  Every
// tile of a run has the same flags (one of the kTile* variants).
struct Entry {
  int32_t kt0, kt1, pidx, flags;
};

struct DeviceMap {
  const int32_t* qt_off = nullptr;
  const Entry* entries = nullptr;
  const int32_t* tasks = nullptr;
  const int32_t* tasks_split = nullptr;
  const uint64_t* bits = nullptr;
};

}  // namespace aj
