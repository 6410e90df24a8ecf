/*
 * attn_jvp.h - C ABI of the MI355X (gfx950) custom-mask attention-JVP library.
 *
 * The operation ("Causal-rCM: A Unified Teacher-Forcing and Self-Forcing Open
 * Recipe for Autoregressive Diffusion Distillation", App. B, "FlashAttention-2
 * JVP Kernel with Custom Masks"): for every (batch, head), given primal Q, K, V,
 * tangents tQ, tK, tV and a mask M of admissible (query, key) pairs,
 *
 *   s_ij  = scale * <q_i, k_j>                       masked softmax attention (Eq. 42)
 *   ts_ij = scale * (<tq_i, k_j> + <q_i, tk_j>)       score tangent (Eq. 43)
 *   P_ij  = softmax_j over allowed keys of s_ij;  O_i = sum_j P_ij v_j
 *   tO_i  = sum_j P_ij (ts_ij - sum_k P_ik ts_ik) v_j + sum_j P_ij tv_j   (Eq. 44)
 *   lse_i = log sum_j exp(s_ij)  over allowed keys (natural log)
 *
 * The mask has no tangent: masked-out pairs take part in neither O nor tO.
 * The kernel evaluates Eq. 44 in the online-softmax form of Eq. 45 in a single
 * streaming pass over the admissible rectangles of the mask (App. B,
 * "Sparse custom-mask representation").
 *
 * Tensor layout: [B, H, L, D] with D contiguous (the per-rank layout of the
 * attention in Sec. 3.2.1); lse is [B, H, L] float32, contiguous.
 *
 * Conventions for every entry point:
 *  - Return value is an aj_status; AJ_OK (0) on success.
 *  - All argument checks happen before any device work is enqueued; on error
 *    nothing is written and nothing is launched.
 *  - No C++ exception crosses this boundary.
 *  - Device pointers are owned by the caller; the library never frees or
 *    retains them.  Mask descriptors are owned by the library (create with a
 *    builder, copy to a device with attn_jvp_mask_desc_upload, release with
 *    attn_jvp_mask_desc_free).
 *  - The launch entry points allocate no memory, copy nothing and do not
 *    synchronise: they validate, look up the descriptor's device tables and
 *    enqueue kernels.
 */
#ifndef ATTN_JVP_H_
#define ATTN_JVP_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AJ_OK = 0,
  AJ_EINVAL = 1,   /* bad argument: null/misaligned pointer, bad size or stride, non-finite scale */
  AJ_ENOTSUP = 2,  /* valid but unsupported: head_dim not in {64, 128}, dtype pair not built */
  AJ_ENOMEM = 3,   /* host or device allocation failed */
  AJ_EHIP = 4,     /* a HIP runtime call failed (no device, launch failure, ...) */
  AJ_EMASK = 5,    /* mask specification invalid, or descriptor does not match the call */
  AJ_ENOTLOADED = 6 /* the descriptor's tables are not on the current device:
                       call attn_jvp_mask_desc_upload first */
} aj_status;

/* Element types of Q, K, V, tQ, tK, tV (in) and O, tO (out). */
typedef enum { AJ_F32 = 0, AJ_BF16 = 1 } aj_dtype;

/* Frame-level mask layouts (Sec. 2.3, Sec. 3.1.1 / Eq. 8 and the c1-1 / c3-3
 * chunk patterns of Sec. 5).  Tokens are laid out frame after frame, each frame
 * frame_tokens contiguous tokens; a chunk is frames_per_chunk frames (the last
 * chunk may be shorter).  Attention inside a chunk is always full.
 *  AJ_MASK_FULL            every query sees every key (L = num_frames * frame_tokens)
 *  AJ_MASK_BLOCK_CAUSAL    a query sees keys of its own chunk and all earlier
 *                          chunks; frames_per_chunk = 1 is frame-causal
 *  AJ_MASK_TF_CLEAN_NOISY  packed [clean | noisy] teacher-forcing sequence,
 *                          L = 2 * num_frames * frame_tokens: clean chunk i sees
 *                          clean chunks <= i; noisy chunk i sees clean chunks
 *                          < i and its own noisy chunk */
typedef enum {
  AJ_MASK_FULL = 0,
  AJ_MASK_BLOCK_CAUSAL = 1,
  AJ_MASK_TF_CLEAN_NOISY = 2
} aj_mask_kind;

typedef struct {
  int32_t kind;              /* aj_mask_kind */
  int32_t num_frames;        /* frames (per half for AJ_MASK_TF_CLEAN_NOISY), >= 1 */
  int32_t frame_tokens;      /* tokens per frame, >= 1 */
  int32_t frames_per_chunk;  /* >= 1 */
} aj_mask_spec;

/* Opaque descriptor: the mask as a tile-level skip / partial / full map over
 * the kernel's query and key tiles, per-row key bitmasks for partial tiles and
 * a longest-first task order.  Its mask and tables are immutable after
 * creation; it may be shared by threads and streams.  Device copies of the
 * tables are made by attn_jvp_mask_desc_upload, once per device, and freed by
 * attn_jvp_mask_desc_free. */
typedef struct aj_mask_desc aj_mask_desc;

typedef struct {
  int64_t unmasked_pairs;   /* allowed (query, key) pairs per (batch, head) */
  int32_t seq_len;
  int32_t tile_m;           /* query rows per tile */
  int32_t tile_n;           /* keys per tile */
  int32_t num_q_tiles;
  int32_t num_k_tiles;
  int32_t full_tiles;       /* tiles with every (query < L, key) pair allowed */
  int32_t partial_tiles;    /* tiles with some, not all, pairs allowed */
  int32_t num_entries;      /* span entries over all query tiles */
  int32_t kv_len;           /* key length (= seq_len except for KV-cache descriptors) */
} aj_mask_stats;

/* Human-readable name of a status code (static storage; never NULL). */
const char* attn_jvp_status_str(int32_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t attn_jvp_version(void);

/* Build a descriptor for a frame-level layout.
 * seq_len must equal the layout's length (see aj_mask_kind); head_dim and dtype
 * select the kernel whose tile geometry the map is built for.
 * Host-only: touches no device.  Errors: AJ_EINVAL (null out, bad sizes),
 * AJ_EMASK (unknown kind, seq_len mismatch), AJ_ENOTSUP (head_dim/dtype),
 * AJ_ENOMEM.  On error *out is set to NULL. */
int32_t attn_jvp_mask_desc_build(const aj_mask_spec* spec, int32_t seq_len, int32_t head_dim,
                                 int32_t dtype, aj_mask_desc** out);

/* Build a descriptor from admissible rectangles (App. B: a mask as a list of
 * query-key rectangles).  rects holds n_rects * 4 int32 values
 * {q0, q1, k0, k1} per rectangle, each half-open, inside [0, seq_len), with
 * q0 < q1 and k0 < k1; rectangles must be pairwise disjoint.  n_rects may be 0
 * (nothing allowed).  Host-only.  Errors as for attn_jvp_mask_desc_build; an
 * overlap or out-of-range rectangle gives AJ_EMASK. */
int32_t attn_jvp_mask_desc_from_rects(int32_t seq_len, const int32_t* rects, int32_t n_rects,
                                      int32_t head_dim, int32_t dtype, aj_mask_desc** out);

/* Build a descriptor whose queries and keys are different sequences: the
 * current chunk of an autoregressive rollout (q_len tokens) attending keys
 * held in a KV cache (kv_len tokens; Sec. 3.2.1 "KV Cache": a readonly
 * forward exposes only the committed prefix the current chunk needs).  rects
 * holds n_rects * 4 int32 {q0, q1, k0, k1}, half-open, disjoint, inside
 * [0, q_len) x [0, kv_len).  Only attn_fwd_kv accepts such a descriptor when
 * kv_len != q_len.  Host-only.  Errors as for attn_jvp_mask_desc_from_rects. */
int32_t attn_jvp_mask_desc_from_rects_kv(int32_t q_len, int32_t kv_len, const int32_t* rects, int32_t n_rects,
                                         int32_t head_dim, int32_t dtype, aj_mask_desc** out);

/* Copy a descriptor's tables to GPU `device` (App. B, "Sparse custom-mask
 * representation": the mask reaches the kernel as a precomputed list of
 * admissible ranges; this call puts that list in device memory).  The launch
 * entry points (attn_jvp_fwd, attn_fwd, attn_fwd_kv, attn_bwd) read the tables
 * of the device current at the call and never allocate or copy them: call
 * this once per device before the first launch, outside any HIP-graph
 * capture.  Allocates device memory (hipMalloc) and copies synchronously
 * (hipMemcpy); restores the caller's current device.  A second call for the
 * same device does nothing and returns AJ_OK; calls from several threads are
 * serialised.  Errors: AJ_EINVAL (null desc, device out of range), AJ_ENOTSUP
 * (device index >= 64), AJ_ENOMEM (device or host allocation failed), AJ_EHIP
 * (no device, copy failed). */
int32_t attn_jvp_mask_desc_upload(aj_mask_desc* desc, int32_t device);

/* Derive a descriptor that also knows which tokens carry no tangent.
 * In teacher-forcing sCM / MeanFlow the JVP runs through the packed
 * [clean | noisy] forward and the clean context has zero tangent (Sec. 3.1.2);
 * then most of the JVP's products vanish: for a query whose tangent is zero,
 * attending keys whose tangents are zero, only the primal products remain;
 * for a key whose tangents are zero, tS reduces to scale * <tq, k> and the tV
 * product drops.
 * ranges holds n_ranges half-open token intervals {t0, t1} inside
 * [0, seq_len) (they may overlap); the new descriptor has base's mask, head_dim
 * and dtype.  By passing it to attn_jvp_fwd the caller declares that tq, tk
 * and tv are exactly zero at these tokens (for every batch and head); the
 * kernel then skips the products that are zero, per tile of 128 queries x 64
 * keys, and need not read those tangents.  A tile's keys count as
 * tangent-free when every key that some query of the tile may attend lies
 * inside the ranges, and its queries when every query attending one of those
 * keys does (masked pairs contribute nothing, whatever their tangents).
 * Query tiles left with only primal work (queries and keys tangent-free in
 * every tile they visit) run the primal forward of attn_fwd, which writes
 * tO = 0 for them, in a launch of their own before the JVP kernel's.  The
 * result equals attn_jvp_fwd with the plain descriptor whenever the
 * declaration holds: bit for bit, except that O and lse of the primal-only
 * query tiles agree to rounding (as attn_fwd's do); if the
 * declaration does not hold, the tangent output is unspecified.  Host-only.
 * Errors: AJ_EINVAL (null pointers, bad range), AJ_ENOMEM.  On error *out is
 * set to NULL. */
int32_t attn_jvp_mask_desc_tangent_free(const aj_mask_desc* base, const int32_t* ranges, int32_t n_ranges,
                                        aj_mask_desc** out);

/* Allowed (query, key) pairs per (batch, head) by the work the kernel does on
 * them: pairs_by_variant[0] in tiles with all JVP products (12 D FLOP per
 * pair), [1] in tiles whose keys carry no tangent (8 D), [2] in tiles where
 * neither queries nor keys do (4 D, the primal products only).  Without
 * tangent-free ranges every pair is in [0].  Errors: AJ_EINVAL on null. */
int32_t attn_jvp_mask_desc_work(const aj_mask_desc* desc, int64_t* pairs_by_variant);

/* Summary of a descriptor.  Errors: AJ_EINVAL on null arguments. */
int32_t attn_jvp_mask_desc_stats(const aj_mask_desc* desc, aj_mask_stats* out);

/* Classification of tile (q_tile, k_tile): *kind = 0 skip, 1 partial, 2 full.
 * Errors: AJ_EINVAL on null arguments or out-of-range tile indices. */
int32_t attn_jvp_mask_desc_tile_kind(const aj_mask_desc* desc, int32_t q_tile, int32_t k_tile,
                                     int32_t* kind);

/* Work variant of tile (q_tile, k_tile): -1 skipped, 0 all JVP products,
 * 1 keys carry no tangent, 3 neither queries nor keys carry tangents (see
 * attn_jvp_mask_desc_tangent_free).  Errors: AJ_EINVAL on null arguments or
 * out-of-range tile indices. */
int32_t attn_jvp_mask_desc_tile_variant(const aj_mask_desc* desc, int32_t q_tile, int32_t k_tile,
                                        int32_t* variant);

/* Key bitmask of one query row of a tile: bit j set when key
 * k_tile * tile_n + j is allowed for query q_tile * tile_m + row.  For full
 * tiles all tile_n bits are set, for skipped tiles none.
 * Errors: AJ_EINVAL on null arguments or out-of-range indices. */
int32_t attn_jvp_mask_desc_row_bits(const aj_mask_desc* desc, int32_t q_tile, int32_t k_tile,
                                    int32_t row, uint64_t* bits);

/* The same mask seen from the keys (the map the key-parallel gradient kernel
 * walks): bit j set when query q_tile * 64 + j may attend key
 * k_tile * 128 + key_row.  Key tiles are 128 keys, query tiles 64 queries.
 * Errors: AJ_EINVAL on null arguments or out-of-range indices. */
int32_t attn_jvp_mask_desc_col_bits(const aj_mask_desc* desc, int32_t k_tile, int32_t q_tile, int32_t key_row,
                                    uint64_t* bits);

/* Release a descriptor and its device tables on every device it was uploaded
 * to.  Must not be called while a launch that uses it may still run, nor while
 * a HIP graph that captured such a launch may still be replayed (the graph
 * holds the addresses of the tables).  NULL is a no-op. */
void attn_jvp_mask_desc_free(aj_mask_desc* desc);

/* Shapes and strides of one call.  Strides are in elements.  The six inputs
 * share in_stride_{b,h,l}; O and tO share out_stride_{b,h,l}; the D axis is
 * contiguous for all of them.  lse is a contiguous [B, H, L] float32 array. */
typedef struct {
  int32_t batch;      /* B >= 1 */
  int32_t heads;      /* H >= 1 */
  int32_t seq_len;    /* L >= 1, equal to the descriptor's */
  int32_t head_dim;   /* D in {64, 128} */
  int32_t in_dtype;   /* aj_dtype */
  int32_t out_dtype;  /* aj_dtype: AJ_BF16 needs in_dtype AJ_BF16; AJ_F32 is accepted for both */
  int64_t in_stride_b, in_stride_h, in_stride_l;
  int64_t out_stride_b, out_stride_h, out_stride_l;
} aj_shape;

/* Forward-mode JVP of masked attention: writes O, tO ([B, H, L, D], out_dtype)
 * and lse ([B, H, L] float32) for inputs q, k, v, tq, tk, tv ([B, H, L, D],
 * in_dtype), all device pointers, 16-byte aligned, strides multiples of
 * 16 bytes / element size, in_stride_l >= D and 64 * in_stride_l * element
 * size < 2^31.  scale multiplies the scores and their tangents;
 * pass 1/sqrt(D) for the usual softmax scale.  Rows with no allowed key get
 * O = tO = 0 and lse = -inf.  Input values at masked-out positions must be
 * finite (they are read for partial tiles and multiplied by zero).  At
 * head_dim 64 with bf16 inputs the value products run in fp16: V and tV
 * must lie within fp16's range (|x| <= 65504; larger magnitudes saturate)
 * and |scale * (<tq, k> + <q, tk>)| must stay below 65504.
 * The outputs must not overlap the inputs.
 * Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and runs
 * asynchronously; device faults surface at the caller's next synchronisation.
 * The descriptor must have been uploaded to the current device
 * (attn_jvp_mask_desc_upload).  The call only enqueues kernels: it allocates,
 * copies and synchronises nothing, so it may be captured into a HIP graph.
 * Errors: AJ_EINVAL, AJ_ENOTSUP, AJ_EMASK (desc seq_len / head_dim / dtype
 * differ from the call), AJ_ENOTLOADED (desc not uploaded to the current
 * device), AJ_EHIP. */
int32_t attn_jvp_fwd(const aj_shape* shape, const void* q, const void* k, const void* v,
                     const void* tq, const void* tk, const void* tv, const aj_mask_desc* mask,
                     float scale, void* o, void* to, float* lse, void* stream);

/* attn_jvp_fwd at head_dim 64 with bf16 inputs, for callers that can give it
 * two buffers: v16 and tv16 are device buffers (16-byte aligned, owned by the
 * caller, each covering every element of v at the input strides) that the
 * call first fills with fp16 copies of v and tv, with the conversion the
 * kernel otherwise applies to every key tile in its local memory (exact for
 * magnitudes in [2^-14, 65504]; round toward zero below, saturation above);
 * the JVP kernel then reads the copies.  Same operation as attn_jvp_fwd
 * ("Causal-rCM", App. B, Eqs. 42-45), same results bit for bit, fewer
 * instructions per key tile.  v16 and tv16 must not overlap each other or any
 * other argument; after the call they hold the copies, unless a tangent-free
 * declaration leaves only primal-only query tiles (then no JVP kernel runs and
 * they are not written).  Two kernels in stream order; allocates nothing.
 * Errors: those of attn_jvp_fwd; AJ_EINVAL for a null or misaligned v16 /
 * tv16, or one equal to another pointer argument; AJ_ENOTSUP unless head_dim
 * is 64 and in_dtype AJ_BF16. */
int32_t attn_jvp_fwd_v16(const aj_shape* shape, const void* q, const void* k, const void* v, const void* tq,
                         const void* tk, const void* tv, const aj_mask_desc* mask, float scale, void* o, void* to,
                         float* lse, void* v16, void* tv16, void* stream);

/* Primal masked attention (Eq. 42): O = softmax(scale * Q K^T + M) V and lse,
 * the forward of the student's packed teacher-forcing attention (Sec. 3.1.1,
 * Eq. 8) on the same descriptor as the JVP.  Same shapes, strides and checks
 * as attn_jvp_fwd; O and lse agree with attn_jvp_fwd's to rounding (at
 * head_dim 128 32-row waves instead of the JVP's 16; at 64 the JVP runs its
 * value products in fp16, this kernel in bf16).  in_dtype must be AJ_BF16
 * (AJ_ENOTSUP otherwise).  o is [B, H, L, D] out_dtype, lse [B, H, L] float32.
 * Errors: AJ_EINVAL, AJ_ENOTSUP, AJ_EMASK, AJ_ENOTLOADED, AJ_EHIP. */
int32_t attn_fwd(const aj_shape* shape, const void* q, const void* k, const void* v, const aj_mask_desc* mask,
                 float scale, void* o, float* lse, void* stream);

/* Shapes and strides of a KV-cache forward.  Queries [B, H, q_len, D] with
 * q strides; keys and values [B, H, kv_len, D] inside a cache buffer with
 * their own strides (the post-all-to-all [B, H/P, L, C] cache layout of
 * Sec. 3.2.1, of which the first kv_len positions are used); the output
 * [B, H, q_len, D] with out strides.  Strides in elements, D contiguous. */
typedef struct {
  int32_t batch, heads, q_len, kv_len, head_dim, in_dtype, out_dtype;
  int64_t q_stride_b, q_stride_h, q_stride_l;
  int64_t kv_stride_b, kv_stride_h, kv_stride_l;
  int64_t out_stride_b, out_stride_h, out_stride_l;
} aj_kv_shape;

/* Primal masked attention of a query chunk over a KV cache (readonly mode of
 * Sec. 3.2.1: the chunk being generated attends the committed prefix, and
 * itself once its keys sit in the cache slots after the prefix).  Same
 * operation, kernels, checks, errors and upload requirement as attn_fwd with the key length and
 * strides taken from the shape; the descriptor must have been built for
 * (q_len, kv_len).  lse is [B, H, q_len] float32.  in_dtype must be AJ_BF16. */
int32_t attn_fwd_kv(const aj_kv_shape* shape, const void* q, const void* k, const void* v,
                    const aj_mask_desc* mask, float scale, void* o, float* lse, void* stream);

/* Gradients of masked attention for a cotangent dout: dq, dk, dv of
 * O = softmax(scale * Q K^T + M) V, the backward of attn_fwd on the same
 * descriptor (training differentiates the packed teacher-forcing forward,
 * Sec. 3.1.1, Eq. 8).  With P_ij = exp(scale <q_i, k_j> - lse_i) on allowed
 * pairs, D_i = <dout_i, o_i> and dS_ij = P_ij (<dout_i, v_j> - D_i):
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 *   dv_j = sum_i P_ij dout_i.
 * Inputs q, k, v, o, dout: [B, H, L, D] bf16 sharing the input strides; o
 * and lse as written by attn_fwd (or attn_jvp_fwd) for the same q, k, v,
 * descriptor and scale.  Outputs dq, dk, dv: [B, H, L, D] out_dtype sharing
 * the output strides (fully written; rows no query or key uses get zeros).
 * delta: [B, H, L] float32, written with D (workspace the caller owns; the
 * kernels read it back).  Two kernels run in order on `stream`; no atomics,
 * the result is deterministic.  Same checks as attn_jvp_fwd; in_dtype must be
 * AJ_BF16 (AJ_ENOTSUP otherwise).  Outputs must not overlap the inputs or
 * each other.  Errors: AJ_EINVAL, AJ_ENOTSUP, AJ_EMASK, AJ_ENOTLOADED,
 * AJ_EHIP. */
int32_t attn_bwd(const aj_shape* shape, const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, const aj_mask_desc* mask, float scale, void* dq,
                 void* dk, void* dv, float* delta, void* stream);

/* attn_bwd without the delta workspace, for callers that cannot allocate
 * device memory (code under HIP-graph capture, tight training loops,
 * harnesses that forbid hipMalloc): D lives in an array the library keeps in
 * device memory, one per GPU for the life of the process (16 MiB).  Same
 * operation, kernels, results (bit for bit), checks and errors as attn_bwd,
 * minus the delta argument; in addition B * H * L must not exceed 4,194,304
 * (AJ_EINVAL otherwise, before any device work).  Allocates nothing: the
 * array's address is looked up once per device (at attn_jvp_mask_desc_upload
 * or, failing that, at the first call on the device).  Every call on a GPU
 * shares that GPU's array: calls that may overlap in time on one GPU (other
 * streams, other threads) race and give wrong gradients; calls in one
 * stream's order are safe. */
int32_t attn_bwd_noalloc(const aj_shape* shape, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, const aj_mask_desc* mask, float scale, void* dq,
                         void* dk, void* dv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_JVP_H_ */
