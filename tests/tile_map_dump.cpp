// Test helper (not part of the library): builds a mask descriptor from
// rectangles read on stdin with the library's own builder and prints its
// query-tile maps (the 128-row map of the JVP kernels and the 256-row map of
// the primal forward) as text, for tests/test_tile_maps_wide.py to compare with
// the oracle's element predicate.
//
// stdin: "R q_len kv_len n" and n rectangles q0 q1 k0 k1, or
// "L kind num_frames frame_tokens frames_per_chunk" (a frame-level layout,
// expanded by the library into rectangles); then optionally "F n" and n
// tangent-free token ranges t0 t1.
// stdout, per map (query tiles of 128 rows, of 256 rows, then the transposed
// map of 128-key tiles): "M rows n_qt n_kt", then per entry
// "E qt kt0 kt1 pidx flags" followed, for a partial tile, by its per-row
// bitmasks (hex, one per row), then "T" and the task order, and for a map
// with primal-only tiles "S n_primal" and the split task order.
// On a builder error: "ERR status", exit code 1.
#include <cstdio>
#include <vector>

#include "aj_internal.h"

int main() {
  char mode = 0;
  if (std::scanf(" %c", &mode) != 1) return 2;
  std::vector<int32_t> r;
  int lq = 0, lk = 0;
  if (mode == 'L') {
    aj_mask_spec spec{};
    if (std::scanf("%d %d %d %d", &spec.kind, &spec.num_frames, &spec.frame_tokens, &spec.frames_per_chunk) != 4)
      return 2;
    lq = lk = spec.num_frames * spec.frame_tokens * (spec.kind == AJ_MASK_TF_CLEAN_NOISY ? 2 : 1);
    if (aj::layout_rects(&spec, lq, &r) != AJ_OK) return 1;
  } else {
    int n = 0;
    if (std::scanf("%d %d %d", &lq, &lk, &n) != 3) return 2;
    r.resize(4 * size_t(n));
    for (int32_t& x : r)
      if (std::scanf("%d", &x) != 1) return 2;
  }
  std::vector<int32_t> tf;
  char f = 0;
  if (std::scanf(" %c", &f) == 1) {
    int n_tf = 0;
    if (f != 'F' || std::scanf("%d", &n_tf) != 1 || n_tf < 0) return 2;
    tf.resize(2 * size_t(n_tf));
    for (int32_t& x : tf)
      if (std::scanf("%d", &x) != 1) return 2;
  }
  aj_mask_desc* d = nullptr;
  const int32_t st = aj::build_from_rects(lq, lk, r.data(), int32_t(r.size() / 4), 128, AJ_BF16, tf.data(),
                                          int32_t(tf.size() / 2), &d);
  if (st != AJ_OK) {
    std::printf("ERR %d\n", st);
    return 1;
  }
  for (const aj::TileMap* m : {&d->rows, &d->rows_w, &d->cols}) {
    std::printf("M %d %d %d\n", m->bm, m->n_qt, m->n_kt);
    for (int32_t qt = 0; qt < m->n_qt; ++qt)
      for (int32_t e = m->qt_off[qt]; e < m->qt_off[qt + 1]; ++e) {
        const aj::Entry& x = m->entries[e];
        std::printf("E %d %d %d %d %d\n", qt, x.kt0, x.kt1, x.pidx, x.flags);
        if (x.pidx >= 0)
          for (int32_t row = 0; row < m->bm; ++row)
            std::printf("%llx\n", static_cast<unsigned long long>(m->bits[size_t(x.pidx) * m->bm + row]));
      }
    std::printf("T");
    for (int32_t t : m->tasks) std::printf(" %d", t);
    std::printf("\n");
    if (!m->tasks_split.empty()) {
      std::printf("S %d", m->n_primal_tasks);
      for (int32_t t : m->tasks_split) std::printf(" %d", t);
      std::printf("\n");
    }
  }
  delete d;
  return 0;
}
