// Internal definitions shared by the host side of the attention-JVP library:
// the mask descriptor (tile map built from admissible rectangles) and the
// kernel launch arguments.  Not part of the public C ABI.
#pragma once

#include <stdint.h>

#include <mutex>
#include <vector>

#include "../../include/attn_jvp.h"

namespace aj {

// Tile geometry of the kernels.  Every instantiation (bf16 / fp32, D = 64 / 128)
// uses 128 query rows per workgroup and 64 keys per streamed tile, so one key
// bitmask row is one 64-bit word.
constexpr int kTileM = 128;
constexpr int kTileN = 64;
constexpr int kMaxDevices = 64;

inline bool supported_head_dim(int d) { return d == 64 || d == 128; }
inline bool supported_dtype(int t) { return t == AJ_F32 || t == AJ_BF16; }

// Which tangents a (query tile, key tile) pair carries, from the caller's
// declaration of tokens whose tangents are zero (Entry::flags):
//   kTileJvp       the general case: every product of the JVP
//   kTileKeysFree  tK = tV = 0 on every key of the tile: tS = c tQ K^T and
//                  (A + B) gets only (P.tS) V
//   kTileAllFree   tQ = tK = tV = 0 for the whole tile: tS = 0, so only the
//                  primal products remain
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

// A tile map over one orientation of the mask: for every tile of kTileM
// rows (the "owner" axis) the runs of kTileN-wide tiles of the other axis it
// must visit, per-row bitmasks of its partial tiles and a longest-first task
// order.  The row map (owner = query tiles) drives the forward kernels and the
// dQ kernel; the column map (owner = key tiles, built from the transposed
// rectangles) drives the dK / dV kernel.
struct TileMap {
  int32_t n_qt = 0, n_kt = 0;       // owner tiles, visited-axis tiles
  int32_t full_tiles = 0, partial_tiles = 0;
  int64_t pairs_by_var[3] = {0, 0, 0};  // allowed pairs in kTileJvp / KeysFree / AllFree tiles
  std::vector<int32_t> qt_off;      // n_qt + 1 offsets into entries
  std::vector<Entry> entries;
  std::vector<int32_t> tasks;       // owner tiles, most work first
  // The same tasks split by class, each part most work first: first the
  // owner tiles whose every span is kTileAllFree (or that have none: nothing
  // of the JVP but the primal remains), n_primal_tasks of them, then the rest.
  std::vector<int32_t> tasks_split;
  int32_t n_primal_tasks = 0;
  std::vector<uint64_t> bits;       // partial_tiles * kTileM words
};

struct DeviceMap {
  const int32_t* qt_off = nullptr;
  const Entry* entries = nullptr;
  const int32_t* tasks = nullptr;
  const int32_t* tasks_split = nullptr;
  const uint64_t* bits = nullptr;
};

struct DeviceTables {
  void* base = nullptr;  // one hipMalloc holding both maps
  DeviceMap rows, cols;
};

}  // namespace aj

struct aj_mask_desc {
  int32_t seq_len = 0, head_dim = 0, dtype = 0;  // seq_len: query length
  int32_t kv_len = 0;                            // key length (= seq_len unless built for a KV cache)
  int32_t tile_m = aj::kTileM, tile_n = aj::kTileN;
  int64_t pairs = 0;
  std::vector<int32_t> rects;       // the admissible rectangles {q0,q1,k0,k1}
  std::vector<int32_t> tfree;       // merged tangent-free token ranges {t0,t1}
  aj::TileMap rows;                 // query tiles -> key-tile runs
  aj::TileMap cols;                 // key tiles -> query-tile runs (transposed mask)
  std::mutex mu;                    // guards dev[]
  aj::DeviceTables dev[aj::kMaxDevices];
};

namespace aj {
// Builds the tile maps from disjoint rectangles {q0,q1,k0,k1} inside
// [0, q_len) x [0, kv_len); tfree holds n_tfree token ranges {t0,t1} whose
// tangents are declared zero (square masks only).
int32_t build_from_rects(int32_t q_len, int32_t kv_len, const int32_t* rects, int32_t n, int32_t head_dim,
                         int32_t dtype, const int32_t* tfree, int32_t n_tfree, aj_mask_desc** out);
// Expands a frame-level layout into disjoint rectangles.
int32_t layout_rects(const aj_mask_spec* spec, int32_t seq_len, std::vector<int32_t>* rects);
}  // namespace aj
