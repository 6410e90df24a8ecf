// C ABI of the attention-JVP library: argument validation, mask descriptor
// lifetime and device upload, and kernel dispatch.  See include/attn_jvp.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <new>
#include <utility>
#include <vector>

#include "aj_internal.h"
#include "aj_launch.h"

using aj::DeviceTables;
using aj::Entry;

namespace {

constexpr int32_t kVersion = 1 * 10000 + 0 * 100 + 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A usable softmax scale: finite and > 0.  Tested on the bit pattern (sign
// clear, exponent not all ones, not zero), so the check holds under any
// floating-point model the compiler is given.
bool valid_scale(float scale) {
  uint32_t u = 0;
  std::memcpy(&u, &scale, sizeof u);
  return (u >> 31) == 0 && (u & 0x7f800000u) != 0x7f800000u && (u & 0x7fffffffu) != 0;
}

// The descriptor's tables on the current device, as attn_jvp_mask_desc_upload
// left them.  A lookup only: allocates, copies and synchronises nothing, so a
// launch that calls it may be captured into a HIP graph.
int32_t device_tables(const aj_mask_desc* d, const DeviceTables** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return AJ_EHIP;
  if (dev < 0 || dev >= aj::kMaxDevices) return AJ_ENOTSUP;
  const DeviceTables& t = d->dev[dev];
  if (!t.ready.load(std::memory_order_acquire)) return AJ_ENOTLOADED;
  *out = &t;
  return AJ_OK;
}

// Copies the descriptor's tables to device `dev` (one hipMalloc, one blocking
// hipMemcpy), unless they are there already.  The caller has made `dev`
// current.
int32_t upload_tables(aj_mask_desc* d, int dev) {
  std::lock_guard<std::mutex> lock(d->mu);
  DeviceTables& t = d->dev[dev];
  if (t.ready.load(std::memory_order_acquire)) return AJ_OK;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  // layout: [rows map | cols map | wide rows map], each {qt_off | entries | tasks | tasks_split | bits}
  struct Part {
    const void* src;
    size_t bytes, off;
  };
  std::vector<Part> parts;
  size_t total = 0;
  auto add = [&](const void* src, size_t bytes) {
    parts.push_back(Part{src, bytes, total});
    total += align(std::max<size_t>(bytes, 16));
  };
  for (const aj::TileMap* m : {&d->rows, &d->cols, &d->rows_w}) {
    add(m->qt_off.data(), m->qt_off.size() * sizeof(int32_t));
    add(m->entries.data(), m->entries.size() * sizeof(Entry));
    add(m->tasks.data(), m->tasks.size() * sizeof(int32_t));
    add(m->tasks_split.data(), m->tasks_split.size() * sizeof(int32_t));
    add(m->bits.data(), m->bits.size() * sizeof(uint64_t));
  }
  std::vector<uint8_t> host(total, 0);
  for (const Part& x : parts)
    if (x.bytes) std::memcpy(host.data() + x.off, x.src, x.bytes);
  void* base = nullptr;
  if (hipMalloc(&base, total) != hipSuccess) return AJ_ENOMEM;
  if (hipMemcpy(base, host.data(), total, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(base);
    return AJ_EHIP;
  }
  uint8_t* b = static_cast<uint8_t*>(base);
  aj::DeviceMap* dm[3] = {&t.rows, &t.cols, &t.rows_w};
  for (int i = 0; i < 3; ++i) {
    dm[i]->qt_off = reinterpret_cast<const int32_t*>(b + parts[5 * i].off);
    dm[i]->entries = reinterpret_cast<const Entry*>(b + parts[5 * i + 1].off);
    dm[i]->tasks = reinterpret_cast<const int32_t*>(b + parts[5 * i + 2].off);
    dm[i]->tasks_split = reinterpret_cast<const int32_t*>(b + parts[5 * i + 3].off);
    dm[i]->bits = reinterpret_cast<const uint64_t*>(b + parts[5 * i + 4].off);
  }
  t.base = base;
  t.ready.store(true, std::memory_order_release);
  return AJ_OK;
}

// Sizes and strides of one call: the square entry points take them from
// aj_shape (keys and values share the queries' strides and length), the
// KV-cache forward from aj_kv_shape.
struct Geometry {
  int32_t B, H, Lq, Lk, D, in_dtype, out_dtype;
  int64_t qs[3], ks[3], os[3];  // strides (elements) over b, h, l
};

Geometry from_shape(const aj_shape* s) {
  Geometry g{s->batch, s->heads, s->seq_len, s->seq_len, s->head_dim, s->in_dtype, s->out_dtype,
             {s->in_stride_b, s->in_stride_h, s->in_stride_l}, {s->in_stride_b, s->in_stride_h, s->in_stride_l},
             {s->out_stride_b, s->out_stride_h, s->out_stride_l}};
  return g;
}

// Checks the arguments shared by the forward entry points and fills the
// common launch arguments (q, k, v, o, lse, strides, sizes, scale, tables).
// ins = {q, k, v, ...}, outs = {o, [to,] lse}; every pointer non-null and
// 16-byte aligned.
int32_t prepare_geom(const Geometry& s, const void* const* ins, int n_in, const void* const* outs, int n_out,
                     const aj_mask_desc* mask, float scale, aj::FwdArgs* a) {
  if (!mask) return AJ_EINVAL;
  for (int i = 0; i < n_in; ++i)
    if (!ins[i] || !aligned16(ins[i])) return AJ_EINVAL;
  for (int i = 0; i < n_out; ++i)
    if (!outs[i] || !aligned16(outs[i])) return AJ_EINVAL;
  if (s.B < 1 || s.H < 1 || s.Lq < 1 || s.Lk < 1) return AJ_EINVAL;
  if (!valid_scale(scale)) return AJ_EINVAL;
  if (!aj::supported_head_dim(s.D)) return AJ_ENOTSUP;
  if (!aj::supported_dtype(s.in_dtype) || !aj::supported_dtype(s.out_dtype)) return AJ_ENOTSUP;
  if (s.in_dtype == AJ_F32 && s.out_dtype != AJ_F32) return AJ_ENOTSUP;
  const int64_t esz_in = s.in_dtype == AJ_F32 ? 4 : 2, esz_out = s.out_dtype == AJ_F32 ? 4 : 2;
  const int64_t vin = 16 / esz_in, vout = 16 / esz_out;  // elements per 16 bytes
  const int64_t D = s.D;
  // strides: non-negative, 16-byte multiples, rows at least D apart
  for (int i = 0; i < 3; ++i) {
    if (s.qs[i] < 0 || s.qs[i] % vin != 0 || s.ks[i] < 0 || s.ks[i] % vin != 0) return AJ_EINVAL;
    if (s.os[i] < 0 || s.os[i] % vout != 0) return AJ_EINVAL;
  }
  // key rows are read as whole rows through a 32-bit buffer range per key
  // tile: distinct rows, and 64 rows' bytes must fit in 31 bits
  if (s.qs[2] < D || s.ks[2] < D || s.ks[2] * esz_in * aj::kTileN >= (int64_t(1) << 31)) return AJ_EINVAL;
  // outputs must not overlap themselves: sorted by stride, every stride must
  // clear the extent of the axes below it (rows are D elements long).  Inputs
  // are only read and may alias (a zero stride broadcasts).
  {
    int64_t st3[3][2] = {{s.os[0], s.B}, {s.os[1], s.H}, {s.os[2], s.Lq}};
    for (int i = 0; i < 3; ++i)
      for (int j = i + 1; j < 3; ++j)
        if (st3[j][0] < st3[i][0]) std::swap(st3[i], st3[j]);
    int64_t span = D;
    for (int i = 0; i < 3; ++i) {
      if (st3[i][1] == 1) continue;
      if (st3[i][0] < span) return AJ_EINVAL;
      span = st3[i][0] * st3[i][1];
    }
  }
  if (mask->seq_len != s.Lq || mask->kv_len != s.Lk || mask->head_dim != s.D || mask->dtype != s.in_dtype)
    return AJ_EMASK;
  const int64_t BHL = int64_t(s.B) * s.H * std::max(s.Lq, s.Lk);
  if (BHL > (int64_t(1) << 40)) return AJ_EINVAL;

  const DeviceTables* t = nullptr;
  int32_t st = device_tables(mask, &t);
  if (st != AJ_OK) return st;

  aj::FwdArgs& r = *a;
  r = aj::FwdArgs{};
  r.q = ins[0]; r.k = ins[1]; r.v = ins[2];
  r.o = const_cast<void*>(outs[0]);
  r.lse = static_cast<float*>(const_cast<void*>(outs[n_out - 1]));
  r.isb = s.qs[0]; r.ish = s.qs[1]; r.isl = s.qs[2];
  r.ksb = s.ks[0]; r.ksh = s.ks[1]; r.ksl = s.ks[2];
  r.osb = s.os[0]; r.osh = s.os[1]; r.osl = s.os[2];
  r.B = s.B; r.H = s.H; r.L = s.Lq; r.Lk = s.Lk;
  r.n_tasks = mask->rows.n_qt;
  r.tile_m = aj::kTileM;
  r.scale = scale;
  r.scale_log2 = float(double(scale) * 1.4426950408889634074);
  r.qt_off = t->rows.qt_off; r.entries = t->rows.entries; r.tasks = t->rows.tasks; r.bits = t->rows.bits;
  return AJ_OK;
}

int32_t prepare(const aj_shape* s, const void* const* ins, int n_in, const void* const* outs, int n_out,
                const aj_mask_desc* mask, float scale, aj::FwdArgs* a) {
  if (!s) return AJ_EINVAL;
  return prepare_geom(from_shape(s), ins, n_in, outs, n_out, mask, scale, a);
}

// The primal forward at head_dim 128 runs 256-row tasks: point the launch at
// the descriptor's wide map (after prepare_geom has checked the tables).
int32_t use_wide_map(const aj_mask_desc* mask, int32_t head_dim, aj::FwdArgs* a) {
  if (head_dim != 128) return AJ_OK;
  const DeviceTables* t = nullptr;
  int32_t st = device_tables(mask, &t);
  if (st != AJ_OK) return st;
  a->n_tasks = mask->rows_w.n_qt;
  a->tile_m = aj::kTileMWide;
  a->qt_off = t->rows_w.qt_off; a->entries = t->rows_w.entries; a->tasks = t->rows_w.tasks; a->bits = t->rows_w.bits;
  return AJ_OK;
}

}  // namespace

extern "C" {

const char* attn_jvp_status_str(int32_t status) {
  switch (status) {
    case AJ_OK: return "AJ_OK: success";
    case AJ_EINVAL: return "AJ_EINVAL: invalid argument";
    case AJ_ENOTSUP: return "AJ_ENOTSUP: unsupported head_dim or dtype";
    case AJ_ENOMEM: return "AJ_ENOMEM: allocation failed";
    case AJ_EHIP: return "AJ_EHIP: HIP runtime error";
    case AJ_EMASK: return "AJ_EMASK: invalid mask or descriptor mismatch";
    case AJ_ENOTLOADED: return "AJ_ENOTLOADED: descriptor not uploaded to the current device";
    default: return "unknown status";
  }
}

int32_t attn_jvp_version(void) { return kVersion; }

int32_t attn_jvp_mask_desc_build(const aj_mask_spec* spec, int32_t seq_len, int32_t head_dim,
                                 int32_t dtype, aj_mask_desc** out) {
  if (!out) return AJ_EINVAL;
  *out = nullptr;
  if (!spec || seq_len < 1) return AJ_EINVAL;
  if (!aj::supported_head_dim(head_dim) || !aj::supported_dtype(dtype)) return AJ_ENOTSUP;
  try {
    std::vector<int32_t> rects;
    const int32_t st = aj::layout_rects(spec, seq_len, &rects);
    if (st != AJ_OK) return st;
    return aj::build_from_rects(seq_len, seq_len, rects.data(), int32_t(rects.size() / 4), head_dim, dtype,
                                nullptr, 0, out);
  } catch (const std::bad_alloc&) {
    return AJ_ENOMEM;
  } catch (...) {
    return AJ_EINVAL;
  }
}

int32_t attn_jvp_mask_desc_from_rects(int32_t seq_len, const int32_t* rects, int32_t n_rects,
                                      int32_t head_dim, int32_t dtype, aj_mask_desc** out) {
  return aj::build_from_rects(seq_len, seq_len, rects, n_rects, head_dim, dtype, nullptr, 0, out);
}

int32_t attn_jvp_mask_desc_from_rects_kv(int32_t q_len, int32_t kv_len, const int32_t* rects, int32_t n_rects,
                                         int32_t head_dim, int32_t dtype, aj_mask_desc** out) {
  return aj::build_from_rects(q_len, kv_len, rects, n_rects, head_dim, dtype, nullptr, 0, out);
}

int32_t attn_jvp_mask_desc_tangent_free(const aj_mask_desc* base, const int32_t* ranges, int32_t n_ranges,
                                        aj_mask_desc** out) {
  if (!out) return AJ_EINVAL;
  *out = nullptr;
  if (!base) return AJ_EINVAL;
  try {
    return aj::build_from_rects(base->seq_len, base->kv_len, base->rects.data(), int32_t(base->rects.size() / 4),
                                base->head_dim, base->dtype, ranges, n_ranges, out);
  } catch (const std::bad_alloc&) {
    return AJ_ENOMEM;
  } catch (...) {
    return AJ_EINVAL;
  }
}

int32_t attn_jvp_mask_desc_upload(aj_mask_desc* d, int32_t device) {
  if (!d) return AJ_EINVAL;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess) return AJ_EHIP;
  if (device < 0 || device >= n) return AJ_EINVAL;
  if (device >= aj::kMaxDevices) return AJ_ENOTSUP;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return AJ_EHIP;
  if (cur != device && hipSetDevice(device) != hipSuccess) return AJ_EHIP;
  int32_t st = AJ_OK;
  try {
    st = upload_tables(d, device);
  } catch (const std::bad_alloc&) {
    st = AJ_ENOMEM;
  }
  // set-up of the device for attn_bwd_noalloc: the address of its array
  float* scratch_addr = nullptr;
  if (st == AJ_OK) st = aj::bwd_scratch(&scratch_addr);
  if (cur != device) (void)hipSetDevice(cur);
  return st;
}

int32_t attn_jvp_mask_desc_work(const aj_mask_desc* d, int64_t* pairs_by_variant) {
  if (!d || !pairs_by_variant) return AJ_EINVAL;
  for (int i = 0; i < 3; ++i) pairs_by_variant[i] = d->rows.pairs_by_var[i];
  return AJ_OK;
}

int32_t attn_jvp_mask_desc_stats(const aj_mask_desc* d, aj_mask_stats* s) {
  if (!d || !s) return AJ_EINVAL;
  s->unmasked_pairs = d->pairs;
  s->seq_len = d->seq_len;
  s->tile_m = d->tile_m;
  s->tile_n = d->tile_n;
  s->num_q_tiles = d->rows.n_qt;
  s->num_k_tiles = d->rows.n_kt;
  s->full_tiles = d->rows.full_tiles;
  s->partial_tiles = d->rows.partial_tiles;
  s->num_entries = int32_t(d->rows.entries.size());
  s->kv_len = d->kv_len;
  return AJ_OK;
}

static const Entry* find_entry(const aj::TileMap& m, int32_t qt, int32_t kt) {
  for (int32_t e = m.qt_off[qt]; e < m.qt_off[qt + 1]; ++e)
    if (m.entries[e].kt0 <= kt && kt < m.entries[e].kt1) return &m.entries[e];
  return nullptr;
}

int32_t attn_jvp_mask_desc_tile_kind(const aj_mask_desc* d, int32_t qt, int32_t kt, int32_t* kind) {
  if (!d || !kind || qt < 0 || qt >= d->rows.n_qt || kt < 0 || kt >= d->rows.n_kt) return AJ_EINVAL;
  const Entry* e = find_entry(d->rows, qt, kt);
  *kind = !e ? 0 : (e->pidx >= 0 ? 1 : 2);
  return AJ_OK;
}

int32_t attn_jvp_mask_desc_tile_variant(const aj_mask_desc* d, int32_t qt, int32_t kt, int32_t* variant) {
  if (!d || !variant || qt < 0 || qt >= d->rows.n_qt || kt < 0 || kt >= d->rows.n_kt) return AJ_EINVAL;
  const Entry* e = find_entry(d->rows, qt, kt);
  *variant = !e ? -1 : e->flags;
  return AJ_OK;
}

// Bitmask of one owner row of tile (ot, vt) in map m (see row_bits).
static int32_t map_bits(const aj::TileMap& m, int32_t L, int32_t ot, int32_t vt, int32_t row, uint64_t* bits) {
  if (!bits || ot < 0 || ot >= m.n_qt || vt < 0 || vt >= m.n_kt || row < 0 || row >= aj::kTileM)
    return AJ_EINVAL;
  const Entry* e = find_entry(m, ot, vt);
  if (!e || ot * aj::kTileM + row >= L) *bits = 0;
  else if (e->pidx < 0) *bits = ~0ull;
  else *bits = m.bits[size_t(e->pidx) * aj::kTileM + row];
  return AJ_OK;
}

int32_t attn_jvp_mask_desc_row_bits(const aj_mask_desc* d, int32_t qt, int32_t kt, int32_t row,
                                    uint64_t* bits) {
  if (!d) return AJ_EINVAL;
  return map_bits(d->rows, d->seq_len, qt, kt, row, bits);
}

int32_t attn_jvp_mask_desc_col_bits(const aj_mask_desc* d, int32_t k_tile, int32_t q_tile, int32_t key_row,
                                    uint64_t* bits) {
  if (!d) return AJ_EINVAL;
  return map_bits(d->cols, d->kv_len, k_tile, q_tile, key_row, bits);
}

void attn_jvp_mask_desc_free(aj_mask_desc* d) {
  if (!d) return;
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (int dev = 0; dev < aj::kMaxDevices; ++dev) {
    if (!d->dev[dev].ready.load(std::memory_order_acquire)) continue;
    if (hipSetDevice(dev) == hipSuccess) (void)hipFree(d->dev[dev].base);
  }
  if (have_cur) (void)hipSetDevice(cur);
  delete d;
}

}  // extern "C"

namespace {

// attn_jvp_fwd, and attn_jvp_fwd_v16 when v16 and tv16 are given (checked by
// the caller).
int32_t jvp_fwd(const aj_shape* s, const void* q, const void* k, const void* v, const void* tq, const void* tk,
                const void* tv, const aj_mask_desc* mask, float scale, void* o, void* to, float* lse, void* v16,
                void* tv16, void* stream) {
  const void* ins[6] = {q, k, v, tq, tk, tv};
  const void* outs[3] = {o, to, lse};
  aj::FwdArgs a;
  int32_t st = prepare(s, ins, 6, outs, 3, mask, scale, &a);
  if (st != AJ_OK) return st;
  a.tq = tq; a.tk = tk; a.tv = tv; a.to = to;
  a.v16 = v16; a.tv16 = tv16;
  const bool variants = mask->rows.pairs_by_var[1] + mask->rows.pairs_by_var[2] > 0;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (!variants || s->in_dtype != AJ_BF16)
    return aj::launch_fwd(a, s->in_dtype, s->out_dtype, s->head_dim, true, variants, hs);
  // Tangent-free declarations: the query tiles left with only primal work
  // (every span tangent-free, or none) run the primal kernel, which writes
  // tO = 0 for them; the others run the JVP kernel.  Two launches in stream
  // order over disjoint rows.
  const DeviceTables* t = nullptr;
  st = device_tables(mask, &t);
  if (st != AJ_OK) return st;
  const int32_t np = mask->rows.n_primal_tasks, nq = mask->rows.n_qt;
  if (np > 0) {
    aj::FwdArgs p = a;
    p.tasks = t->rows.tasks_split;
    p.n_tasks = np;
    p.v16 = p.tv16 = nullptr;  // the primal kernel reads V in bf16
    st = aj::launch_fwd(p, s->in_dtype, s->out_dtype, s->head_dim, false, false, hs);
    if (st != AJ_OK) return st;
  }
  if (nq > np) {
    aj::FwdArgs r = a;
    r.tasks = t->rows.tasks_split + np;
    r.n_tasks = nq - np;
    st = aj::launch_fwd(r, s->in_dtype, s->out_dtype, s->head_dim, true, variants, hs);
  }
  return st;
}

}  // namespace

extern "C" {

int32_t attn_jvp_fwd(const aj_shape* s, const void* q, const void* k, const void* v, const void* tq,
                     const void* tk, const void* tv, const aj_mask_desc* mask, float scale, void* o,
                     void* to, float* lse, void* stream) {
  return jvp_fwd(s, q, k, v, tq, tk, tv, mask, scale, o, to, lse, nullptr, nullptr, stream);
}

int32_t attn_jvp_fwd_v16(const aj_shape* s, const void* q, const void* k, const void* v, const void* tq,
                         const void* tk, const void* tv, const aj_mask_desc* mask, float scale, void* o,
                         void* to, float* lse, void* v16, void* tv16, void* stream) {
  if (!v16 || !tv16 || !aligned16(v16) || !aligned16(tv16)) return AJ_EINVAL;
  // the copies are written before the kernels read the inputs: the obvious
  // aliases are rejected (partial overlaps remain the caller's to avoid)
  for (const void* x : {q, k, v, tq, tk, tv, static_cast<const void*>(o), static_cast<const void*>(to),
                        static_cast<const void*>(lse)})
    if (x == v16 || x == tv16) return AJ_EINVAL;
  if (v16 == tv16) return AJ_EINVAL;
  if (s && (s->head_dim != 64 || s->in_dtype != AJ_BF16)) return AJ_ENOTSUP;  // before any device work
  return jvp_fwd(s, q, k, v, tq, tk, tv, mask, scale, o, to, lse, v16, tv16, stream);
}

int32_t attn_fwd(const aj_shape* s, const void* q, const void* k, const void* v, const aj_mask_desc* mask,
                 float scale, void* o, float* lse, void* stream) {
  if (s && s->in_dtype != AJ_BF16) return AJ_ENOTSUP;  // before any device work
  const void* ins[3] = {q, k, v};
  const void* outs[2] = {o, lse};
  aj::FwdArgs a;
  int32_t st = prepare(s, ins, 3, outs, 2, mask, scale, &a);
  if (st == AJ_OK) st = use_wide_map(mask, s->head_dim, &a);
  if (st != AJ_OK) return st;
  a.tq = a.tk = a.tv = nullptr;
  a.to = nullptr;
  return aj::launch_fwd(a, s->in_dtype, s->out_dtype, s->head_dim, false, false,
                        static_cast<hipStream_t>(stream));
}

// The gradient entry points: attn_bwd with the caller's delta, attn_bwd_noalloc
// (delta == nullptr) with the library's per-GPU array.
static int32_t bwd_entry(const aj_shape* s, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, const aj_mask_desc* mask, float scale, void* dq,
                         void* dk, void* dv, float* delta, void* stream) {
  // checks of this entry point first: nothing may reach the device before all pass
  if (!s || !mask) return AJ_EINVAL;
  if (!lse || !aligned16(lse)) return AJ_EINVAL;
  if (s->in_dtype != AJ_BF16) return AJ_ENOTSUP;
  if (mask->kv_len != mask->seq_len) return AJ_EMASK;
  const bool own_delta = delta == nullptr;
  if (own_delta && (s->batch < 1 || s->heads < 1 || s->seq_len < 1 ||
                    int64_t(s->batch) * s->heads * s->seq_len > aj::kBwdScratchFloats))
    return AJ_EINVAL;
  const void* ins[5] = {q, k, v, o, dout};
  const void* outs[4] = {dq, dk, dv, delta};
  aj::FwdArgs f;
  int32_t st = prepare(s, ins, 5, outs, own_delta ? 3 : 4, mask, scale, &f);
  if (st != AJ_OK) return st;
  const DeviceTables* t = nullptr;
  st = device_tables(mask, &t);
  if (st != AJ_OK) return st;
  if (own_delta) {
    st = aj::bwd_scratch(&delta);
    if (st != AJ_OK) return st;
  }
  aj::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout;
  a.lse = lse; a.delta = delta;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.isb = f.isb; a.ish = f.ish; a.isl = f.isl;
  a.osb = f.osb; a.osh = f.osh; a.osl = f.osl;
  a.B = f.B; a.H = f.H; a.L = f.L;
  a.n_row_tasks = mask->rows.n_qt;
  a.n_col_tasks = mask->cols.n_qt;
  a.scale = f.scale;
  a.scale_log2 = f.scale_log2;
  a.rows = t->rows;
  a.cols = t->cols;
  return aj::launch_bwd(a, s->out_dtype, s->head_dim, static_cast<hipStream_t>(stream));
}

int32_t attn_bwd(const aj_shape* s, const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, const aj_mask_desc* mask, float scale, void* dq, void* dk, void* dv,
                 float* delta, void* stream) {
  if (!delta) return AJ_EINVAL;
  return bwd_entry(s, q, k, v, o, dout, lse, mask, scale, dq, dk, dv, delta, stream);
}

int32_t attn_bwd_noalloc(const aj_shape* s, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, const aj_mask_desc* mask, float scale, void* dq,
                         void* dk, void* dv, void* stream) {
  return bwd_entry(s, q, k, v, o, dout, lse, mask, scale, dq, dk, dv, nullptr, stream);
}

int32_t attn_fwd_kv(const aj_kv_shape* s, const void* q, const void* k, const void* v, const aj_mask_desc* mask,
                    float scale, void* o, float* lse, void* stream) {
  if (!s) return AJ_EINVAL;
  const Geometry g{s->batch, s->heads, s->q_len, s->kv_len, s->head_dim, s->in_dtype, s->out_dtype,
                   {s->q_stride_b, s->q_stride_h, s->q_stride_l}, {s->kv_stride_b, s->kv_stride_h, s->kv_stride_l},
                   {s->out_stride_b, s->out_stride_h, s->out_stride_l}};
  if (s->in_dtype != AJ_BF16) return AJ_ENOTSUP;  // before any device work
  const void* ins[3] = {q, k, v};
  const void* outs[2] = {o, lse};
  aj::FwdArgs a;
  int32_t st = prepare_geom(g, ins, 3, outs, 2, mask, scale, &a);
  if (st == AJ_OK) st = use_wide_map(mask, s->head_dim, &a);
  if (st != AJ_OK) return st;
  a.tq = a.tk = a.tv = nullptr;
  a.to = nullptr;
  return aj::launch_fwd(a, s->in_dtype, s->out_dtype, s->head_dim, false, false,
                        static_cast<hipStream_t>(stream));
}

}  // extern "C"
