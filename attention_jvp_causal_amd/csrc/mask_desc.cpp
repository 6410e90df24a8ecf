// Host-side mask descriptor: frame-level layouts -> admissible rectangles ->
// tile-level skip / partial / full maps (by query tile, and by key tile for
// the key-parallel gradient kernel) -> longest-first task lists.
//
// "Causal-rCM", App. B ("Sparse custom-mask representation"): the custom mask
// is a set of query groups, each a contiguous query interval with a list of
// admissible key intervals; each task streams only the key ranges of its group.
// Here a query group is a kernel query tile, and its key ranges are stored as
// runs of full key tiles plus single partial tiles carrying per-row bitmasks,
// so the kernel never evaluates a mask predicate on a full tile.
#include <algorithm>
#include <map>
#include <new>
#include <vector>

#include "aj_internal.h"

namespace aj {

namespace {

int32_t validate_rects(int32_t Lq, int32_t Lk, const int32_t* r, int32_t n) {
  for (int32_t i = 0; i < n; ++i) {
    const int32_t q0 = r[4 * i], q1 = r[4 * i + 1], k0 = r[4 * i + 2], k1 = r[4 * i + 3];
    if (q0 < 0 || q0 >= q1 || q1 > Lq || k0 < 0 || k0 >= k1 || k1 > Lk) return AJ_EMASK;
  }
  // pairwise disjointness: sort by q0, compare only rectangles whose query
  // ranges overlap
  std::vector<int32_t> order(n);
  for (int32_t i = 0; i < n; ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return r[4 * a] < r[4 * b]; });
  for (int32_t x = 0; x < n; ++x) {
    const int32_t* a = r + 4 * order[x];
    for (int32_t y = x + 1; y < n; ++y) {
      const int32_t* b = r + 4 * order[y];
      if (b[0] >= a[1]) break;
      if (b[2] < a[3] && a[2] < b[3]) return AJ_EMASK;
    }
  }
  return AJ_OK;
}

struct RectRef {
  int32_t q0, q1, k0, k1;
};

// Validates token ranges {t0, t1} (half-open, inside [0, L), may overlap) and
// returns their sorted union.
int32_t merge_ranges(int32_t L, const int32_t* t, int32_t n, std::vector<int32_t>* out) {
  std::vector<std::pair<int32_t, int32_t>> v;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t a = t[2 * i], b = t[2 * i + 1];
    if (a < 0 || a >= b || b > L) return AJ_EINVAL;
    v.emplace_back(a, b);
  }
  std::sort(v.begin(), v.end());
  out->clear();
  for (const auto& x : v) {
    if (!out->empty() && x.first <= out->back())
      out->back() = std::max(out->back(), x.second);
    else {
      out->push_back(x.first);
      out->push_back(x.second);
    }
  }
  return AJ_OK;
}

// Whether [a, b) lies inside the union of the merged ranges r.
bool covered(const std::vector<int32_t>& r, int32_t a, int32_t b) {
  // last range starting at or before a
  size_t lo = 0, hi = r.size() / 2;
  while (lo < hi) {
    const size_t mid = (lo + hi) / 2;
    if (r[2 * mid] <= a) lo = mid + 1;
    else hi = mid;
  }
  return lo > 0 && r[2 * (lo - 1) + 1] >= b;
}

// Relative cost of one tile of each variant (units of 4d FLOP per pair).
// Variant of a partial tile from the tokens that take part in it: the keys of
// bitmask `keys` (key `key0 + j` for bit j) and whether every row attending one
// of them is tangent-free.  Masked pairs contribute nothing (P = 0, tS is
// set to 0), so the tangents of keys and rows outside the mask do not matter.
int32_t partial_variant(const std::vector<int32_t>& tfree, uint64_t keys, int32_t key0, bool rows_free) {
  bool keys_free = true;
  for (int j = 0; j < 64 && keys_free; ++j)
    if ((keys >> j) & 1ull) keys_free = covered(tfree, key0 + j, key0 + j + 1);
  return keys_free ? (rows_free ? kTileAllFree : kTileKeysFree) : kTileJvp;
}

int64_t tile_cost(int32_t flags) { return flags == kTileJvp ? 3 : flags == kTileKeysFree ? 2 : 1; }
int var_index(int32_t flags) { return flags == kTileJvp ? 0 : flags == kTileKeysFree ? 1 : 2; }

}  // namespace

int32_t layout_rects(const aj_mask_spec* s, int32_t L, std::vector<int32_t>* out) {
  if (s->num_frames < 1 || s->frame_tokens < 1 || s->frames_per_chunk < 1) return AJ_EMASK;
  const int64_t half = int64_t(s->num_frames) * s->frame_tokens;
  const int64_t want = s->kind == AJ_MASK_TF_CLEAN_NOISY ? 2 * half : half;
  if (s->kind != AJ_MASK_FULL && s->kind != AJ_MASK_BLOCK_CAUSAL && s->kind != AJ_MASK_TF_CLEAN_NOISY)
    return AJ_EMASK;
  if (want != L) return AJ_EMASK;
  const int64_t C = int64_t(s->frames_per_chunk) * s->frame_tokens;  // tokens per chunk
  const int64_t nchunks = (half + C - 1) / C;
  auto push = [&](int64_t q0, int64_t q1, int64_t k0, int64_t k1) {
    if (q0 < q1 && k0 < k1) {
      out->push_back(int32_t(q0));
      out->push_back(int32_t(q1));
      out->push_back(int32_t(k0));
      out->push_back(int32_t(k1));
    }
  };
  out->clear();
  if (s->kind == AJ_MASK_FULL) {
    push(0, L, 0, L);
    return AJ_OK;
  }
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t b = c * C, e = std::min(half, (c + 1) * C);
    // own chunk and all earlier chunks (clean stream for teacher forcing)
    push(b, e, 0, e);
    if (s->kind == AJ_MASK_TF_CLEAN_NOISY) {
      push(half + b, half + e, 0, b);            // strictly earlier clean chunks
      push(half + b, half + e, half + b, half + e);  // own noisy chunk
    }
  }
  return AJ_OK;
}

// Tile map of rectangles r (owner axis first: {o0, o1, v0, v1}) with owner
// tiles of BM rows over [0, Lo) and visited tiles of kTileN over [0, Lv).
// tfree (merged ranges) marks tangent-free tokens (square masks: both axes
// index the same sequence).
static void build_map(int32_t Lo, int32_t Lv, const int32_t* r, int32_t n, const std::vector<int32_t>& tfree,
                      int32_t BM, TileMap* m) {
  const int32_t BN = kTileN;
  m->bm = BM;
  m->n_qt = (Lo + BM - 1) / BM;
  m->n_kt = (Lv + BN - 1) / BN;
  // tangent-free owner and visited tiles of full runs: every token of the
  // tile inside the sequence is declared tangent-free (in a full tile every
  // row attends every key); partial tiles decide from their bitmasks below
  auto q_free = [&](int32_t qt) { return covered(tfree, qt * BM, std::min(Lo, qt * BM + BM)); };
  auto k_free = [&](int32_t kt) { return covered(tfree, kt * BN, std::min(Lv, kt * BN + BN)); };
  auto variant = [&](bool qf, int32_t kt) {
    return k_free(kt) ? (qf ? kTileAllFree : kTileKeysFree) : kTileJvp;
  };

  // bucket rectangles by the owner tiles they touch
  std::vector<std::vector<RectRef>> per_qt(m->n_qt);
  for (int32_t i = 0; i < n; ++i) {
    RectRef x{r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]};
    for (int32_t qt = x.q0 / BM; qt <= (x.q1 - 1) / BM; ++qt) per_qt[qt].push_back(x);
  }

  std::vector<int64_t> work(m->n_qt, 0);
  m->qt_off.assign(m->n_qt + 1, 0);
  for (int32_t qt = 0; qt < m->n_qt; ++qt) {
    m->qt_off[qt] = int32_t(m->entries.size());
    const bool qf = q_free(qt);
    const int32_t a = qt * BM, b = std::min(Lo, a + BM);
    const int64_t full_count = int64_t(b - a) * BN;  // allowed pairs in a full tile
    // allowed-pair count per visited tile: runs of interior tiles go into a
    // difference map, the (at most two) boundary tiles of each rectangle
    // into a point map
    std::map<int32_t, int64_t> run_delta, points;
    for (const RectRef& x : per_qt[qt]) {
      const int64_t rows = std::min(b, x.q1) - std::max(a, x.q0);
      const int32_t kf = x.k0 / BN, kl = (x.k1 - 1) / BN;
      if (kf == kl) {
        points[kf] += rows * (x.k1 - x.k0);
        continue;
      }
      points[kf] += rows * (int64_t(kf + 1) * BN - x.k0);
      points[kl] += rows * (x.k1 - int64_t(kl) * BN);
      if (kl > kf + 1) {
        run_delta[kf + 1] += rows * BN;
        run_delta[kl] -= rows * BN;
      }
    }
    // sweep over breakpoints in visited-tile order
    std::vector<int32_t> cuts;
    for (auto& kv : run_delta) cuts.push_back(kv.first);
    for (auto& kv : points) {
      cuts.push_back(kv.first);
      cuts.push_back(kv.first + 1);
    }
    std::sort(cuts.begin(), cuts.end());
    cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
    int64_t run = 0;
    auto rd = run_delta.begin();
    for (size_t ci = 0; ci + 1 < cuts.size(); ++ci) {
      const int32_t s0 = cuts[ci], s1 = cuts[ci + 1];
      while (rd != run_delta.end() && rd->first <= s0) run += (rd++)->second;
      auto pt = points.find(s0);
      const bool is_point = pt != points.end();
      const int64_t cnt = run + (is_point ? pt->second : 0);
      // cuts include p and p + 1 for every point tile p, so a point segment
      // is exactly one tile wide
      const int32_t e1 = s1;
      if (cnt == 0) continue;
      const bool in_range = int64_t(e1) * BN <= Lv;
      if (cnt == full_count && in_range) {
        for (int32_t kt = s0; kt < e1; ++kt) {
          const int32_t fl = variant(qf, kt);
          if (int32_t(m->entries.size()) > m->qt_off[qt] && m->entries.back().pidx < 0 &&
              m->entries.back().kt1 == kt && m->entries.back().flags == fl)
            m->entries.back().kt1 = kt + 1;  // extend the previous full run
          else
            m->entries.push_back(Entry{kt, kt + 1, -1, fl});
          m->pairs_by_var[var_index(fl)] += full_count;
        }
        m->full_tiles += e1 - s0;
      } else {
        for (int32_t kt = s0; kt < e1; ++kt) {
          const int32_t pidx = m->partial_tiles++;
          m->bits.resize(size_t(m->partial_tiles) * BM, 0);
          uint64_t* rowbits = &m->bits[size_t(pidx) * BM];
          const int32_t key0 = kt * BN;
          for (const RectRef& x : per_qt[qt]) {
            const int32_t kk0 = std::max(x.k0, key0), kk1 = std::min(x.k1, key0 + BN);
            if (kk0 >= kk1) continue;
            const int32_t w = kk1 - kk0;
            const uint64_t msk = (w == 64 ? ~0ull : ((1ull << w) - 1)) << (kk0 - key0);
            for (int32_t q = std::max(a, x.q0); q < std::min(b, x.q1); ++q) rowbits[q - a] |= msk;
          }
          int64_t c = 0;
          uint64_t keys = 0;  // keys that some row of the tile may attend
          bool rows_free = true;  // every row that attends one of them is tangent-free
          for (int32_t row = 0; row < BM; ++row) {
            c += __builtin_popcountll(rowbits[row]);
            keys |= rowbits[row];
            if (rowbits[row] && rows_free) rows_free = covered(tfree, a + row, a + row + 1);
          }
          const int32_t fl = partial_variant(tfree, keys, key0, rows_free);
          m->entries.push_back(Entry{kt, kt + 1, pidx, fl});
          m->pairs_by_var[var_index(fl)] += c;
        }
      }
    }
    for (int32_t e = m->qt_off[qt]; e < int32_t(m->entries.size()); ++e)
      work[qt] += (m->entries[e].kt1 - m->entries[e].kt0) * tile_cost(m->entries[e].flags);
  }
  m->qt_off[m->n_qt] = int32_t(m->entries.size());

  // tasks: every owner tile (tiles with nothing allowed still write zeros),
  // most work first (visited tiles weighted by their variant's cost); ties by
  // larger tile index
  m->tasks.resize(m->n_qt);
  for (int32_t qt = 0; qt < m->n_qt; ++qt) m->tasks[qt] = qt;
  std::stable_sort(m->tasks.begin(), m->tasks.end(), [&](int32_t x, int32_t y) {
    return work[x] != work[y] ? work[x] > work[y] : x > y;
  });
  auto primal_only = [&](int32_t qt) {
    for (int32_t e = m->qt_off[qt]; e < m->qt_off[qt + 1]; ++e)
      if (m->entries[e].flags != kTileAllFree) return false;
    return true;
  };
  m->tasks_split.clear();
  for (int32_t qt : m->tasks)
    if (primal_only(qt)) m->tasks_split.push_back(qt);
  m->n_primal_tasks = int32_t(m->tasks_split.size());
  for (int32_t qt : m->tasks)
    if (!primal_only(qt)) m->tasks_split.push_back(qt);
}

int32_t build_from_rects(int32_t Lq, int32_t Lk, const int32_t* r, int32_t n, int32_t head_dim, int32_t dtype,
                         const int32_t* tf, int32_t n_tf, aj_mask_desc** out) {
  if (!out) return AJ_EINVAL;
  *out = nullptr;
  if (Lq < 1 || Lk < 1 || n < 0 || (n > 0 && !r) || n_tf < 0 || (n_tf > 0 && !tf)) return AJ_EINVAL;
  if (n_tf > 0 && Lq != Lk) return AJ_EINVAL;
  if (!supported_head_dim(head_dim) || !supported_dtype(dtype)) return AJ_ENOTSUP;
  int32_t st = validate_rects(Lq, Lk, r, n);
  if (st != AJ_OK) return st;
  std::vector<int32_t> tfree;
  st = merge_ranges(Lq, tf, n_tf, &tfree);
  if (st != AJ_OK) return st;

  aj_mask_desc* d = new (std::nothrow) aj_mask_desc();
  if (!d) return AJ_ENOMEM;
  try {
    d->seq_len = Lq;
    d->kv_len = Lk;
    d->head_dim = head_dim;
    d->dtype = dtype;
    d->rects.assign(r, r + 4 * size_t(n));
    d->tfree = tfree;
    for (int32_t i = 0; i < n; ++i) d->pairs += int64_t(r[4 * i + 1] - r[4 * i]) * (r[4 * i + 3] - r[4 * i + 2]);
    build_map(Lq, Lk, r, n, tfree, kTileM, &d->rows);
    // the primal forward's wide query tiles (no tangents, so no variants)
    build_map(Lq, Lk, r, n, std::vector<int32_t>(), kTileMWide, &d->rows_w);
    // the transposed mask: key tiles own runs of query tiles (no variants)
    std::vector<int32_t> tr(4 * size_t(n));
    for (int32_t i = 0; i < n; ++i) {
      tr[4 * i] = r[4 * i + 2];
      tr[4 * i + 1] = r[4 * i + 3];
      tr[4 * i + 2] = r[4 * i];
      tr[4 * i + 3] = r[4 * i + 1];
    }
    build_map(Lk, Lq, tr.data(), n, std::vector<int32_t>(), kTileM, &d->cols);
  } catch (const std::bad_alloc&) {
    delete d;
    return AJ_ENOMEM;
  } catch (...) {
    delete d;
    return AJ_EINVAL;
  }
  *out = d;
  return AJ_OK;
}

}  // namespace aj
