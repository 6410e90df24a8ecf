// Host-side internals of the attention-JVP library: the mask descriptor (tile
// maps built from admissible rectangles) and its device tables.  Not part of
// the public C ABI.
#pragma once

#include <stdint.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/attn_jvp.h"
#include "aj_tiles.h"

namespace aj {

constexpr int kMaxDevices = 64;

inline bool supported_head_dim(int d) { return d == 64 || d == 128; }
inline bool supported_dtype(int t) { return t == AJ_F32 || t == AJ_BF16; }

// A tile map over one orientation of the mask: for every tile of bm (kTileM
// or kTileMWide) rows of the "owner" axis the runs of kTileN-wide tiles of the other axis it
// must visit, per-row bitmasks of its partial tiles and a longest-first task
// order.  The row map (owner = query tiles) drives the forward kernels and the
// dQ kernel; the column map (owner = key tiles, built from the transposed
// rectangles) drives the dK / dV kernel.
struct TileMap {
  int32_t bm = kTileM;              // rows (owner-axis tokens) per owner tile
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
  std::vector<uint64_t> bits;       // partial_tiles * bm words
};

struct DeviceTables {
  void* base = nullptr;  // one hipMalloc holding the three maps
  DeviceMap rows, cols, rows_w;
  // set once base and the maps are valid (attn_jvp_mask_desc_upload); launches
  // read the tables without taking the descriptor's lock
  std::atomic<bool> ready{false};
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
  aj::TileMap rows_w;               // query tiles of kTileMWide rows -> key-tile runs (no variants)
  std::mutex mu;                    // serialises uploads into dev[]
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

// Capacity (floats) of the per-GPU array that holds D for attn_bwd_noalloc:
// B * H * L of a call may not exceed it (16 MiB).
constexpr int64_t kBwdScratchFloats = int64_t(1) << 22;

// Device address of that array on the current device (attn_bwd.hip: looked
// up once per device with hipGetSymbolAddress, then cached); allocates
// nothing.  Returns an aj_status.
int bwd_scratch(float** out);
}  // namespace aj
