"""MI355X (gfx950) custom-mask attention JVP: Python binding of the C ABI.

The work is done by hand-written HIP kernels in ``libattnjvp.so`` (built
in-tree by ``attention_jvp_causal_amd.build``).  This module only marshals
arguments: it checks tensors, allocates outputs with torch (device memory and
streams are torch's), and calls the C entry points declared in
``include/attn_jvp.h`` through ctypes.  There is no fallback: if the library is
missing, every call raises.

    desc = attn_jvp_mask_desc_build("block_causal", num_frames=21, frame_tokens=1560,
                                    frames_per_chunk=3, head_dim=128, dtype="bf16")
    o, to, lse = attn_jvp_fwd(q, k, v, tq, tk, tv, desc)

The builders copy the descriptor's tables to the current GPU (``device="auto"``)
so that the launches themselves never allocate; pass ``device=None`` to build
on the host only and call ``desc.upload(device)`` later.  A descriptor must
outlive every HIP graph that captured a launch using it.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattnjvp.so")

AJ_OK, AJ_EINVAL, AJ_ENOTSUP, AJ_ENOMEM, AJ_EHIP, AJ_EMASK, AJ_ENOTLOADED = range(7)
AJ_F32, AJ_BF16 = 0, 1
MASK_KINDS = {"full": 0, "block_causal": 1, "frame_causal": 1, "tf_clean_noisy": 2}
DTYPES = {"f32": AJ_F32, "float32": AJ_F32, "bf16": AJ_BF16, "bfloat16": AJ_BF16}


class AttnJvpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


class aj_mask_spec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("num_frames", ctypes.c_int32),
                ("frame_tokens", ctypes.c_int32), ("frames_per_chunk", ctypes.c_int32)]


class aj_mask_stats(ctypes.Structure):
    _fields_ = [("unmasked_pairs", ctypes.c_int64), ("seq_len", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("num_q_tiles", ctypes.c_int32), ("num_k_tiles", ctypes.c_int32),
                ("full_tiles", ctypes.c_int32), ("partial_tiles", ctypes.c_int32),
                ("num_entries", ctypes.c_int32), ("kv_len", ctypes.c_int32)]


class aj_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("in_stride_b", ctypes.c_int64), ("in_stride_h", ctypes.c_int64), ("in_stride_l", ctypes.c_int64),
                ("out_stride_b", ctypes.c_int64), ("out_stride_h", ctypes.c_int64), ("out_stride_l", ctypes.c_int64)]


class aj_kv_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("kv_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32),
                ("q_stride_b", ctypes.c_int64), ("q_stride_h", ctypes.c_int64), ("q_stride_l", ctypes.c_int64),
                ("kv_stride_b", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64), ("kv_stride_l", ctypes.c_int64),
                ("out_stride_b", ctypes.c_int64), ("out_stride_h", ctypes.c_int64), ("out_stride_l", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_jvp_causal_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    pdesc = ctypes.c_void_p
    L.attn_jvp_status_str.argtypes, L.attn_jvp_status_str.restype = [i32], ctypes.c_char_p
    L.attn_jvp_version.argtypes, L.attn_jvp_version.restype = [], i32
    L.attn_jvp_mask_desc_build.argtypes = [ctypes.POINTER(aj_mask_spec), i32, i32, i32, ctypes.POINTER(pdesc)]
    L.attn_jvp_mask_desc_from_rects.argtypes = [i32, P, i32, i32, i32, ctypes.POINTER(pdesc)]
    L.attn_jvp_mask_desc_stats.argtypes = [pdesc, ctypes.POINTER(aj_mask_stats)]
    L.attn_jvp_mask_desc_tile_kind.argtypes = [pdesc, i32, i32, ctypes.POINTER(i32)]
    L.attn_jvp_mask_desc_row_bits.argtypes = [pdesc, i32, i32, i32, ctypes.POINTER(ctypes.c_uint64)]
    L.attn_jvp_mask_desc_free.argtypes, L.attn_jvp_mask_desc_free.restype = [pdesc], None
    L.attn_jvp_mask_desc_tangent_free.argtypes = [pdesc, P, i32, ctypes.POINTER(pdesc)]
    L.attn_jvp_mask_desc_work.argtypes = [pdesc, ctypes.POINTER(i64)]
    L.attn_jvp_mask_desc_tile_variant.argtypes = [pdesc, i32, i32, ctypes.POINTER(i32)]
    L.attn_jvp_fwd.argtypes = [ctypes.POINTER(aj_shape), P, P, P, P, P, P, pdesc, f32, P, P, P, P]
    L.attn_jvp_fwd_v16.argtypes = [ctypes.POINTER(aj_shape), P, P, P, P, P, P, pdesc, f32, P, P, P, P, P, P]
    L.attn_fwd.argtypes = [ctypes.POINTER(aj_shape), P, P, P, pdesc, f32, P, P, P]
    L.attn_bwd.argtypes = [ctypes.POINTER(aj_shape), P, P, P, P, P, P, pdesc, f32, P, P, P, P, P]
    L.attn_fwd_kv.argtypes = [ctypes.POINTER(aj_kv_shape), P, P, P, pdesc, f32, P, P, P]
    L.attn_jvp_mask_desc_from_rects_kv.argtypes = [i32, i32, P, i32, i32, i32, ctypes.POINTER(pdesc)]
    L.attn_jvp_mask_desc_col_bits.argtypes = [pdesc, i32, i32, i32, ctypes.POINTER(ctypes.c_uint64)]
    L.attn_jvp_mask_desc_upload.argtypes = [pdesc, i32]
    L.attn_bwd_noalloc.argtypes = [ctypes.POINTER(aj_shape), P, P, P, P, P, P, pdesc, f32, P, P, P, P]
    for fn in ("attn_jvp_mask_desc_build", "attn_jvp_mask_desc_from_rects", "attn_jvp_mask_desc_stats",
               "attn_jvp_mask_desc_tile_kind", "attn_jvp_mask_desc_row_bits", "attn_jvp_fwd",
               "attn_jvp_mask_desc_tangent_free", "attn_jvp_mask_desc_work", "attn_jvp_mask_desc_tile_variant",
               "attn_fwd", "attn_bwd", "attn_jvp_mask_desc_col_bits", "attn_fwd_kv",
               "attn_jvp_mask_desc_from_rects_kv", "attn_jvp_mask_desc_upload", "attn_bwd_noalloc",
               "attn_jvp_fwd_v16"):
        getattr(L, fn).restype = i32
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().attn_jvp_status_str(int(status)).decode()


def attn_jvp_version() -> int:
    return int(lib().attn_jvp_version())


def _check(st: int, where: str) -> None:
    if st != AJ_OK:
        raise AttnJvpError(st, where)


def _dtype_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    key = str(dtype).replace("torch.", "")
    if key not in DTYPES:
        raise ValueError(f"unsupported dtype {dtype!r}")
    return DTYPES[key]


class MaskDesc:
    """Owner of an ``aj_mask_desc*`` (freed on close / garbage collection)."""

    def __init__(self, handle: int, head_dim: int, dtype: int):
        self._h = ctypes.c_void_p(handle)
        self.head_dim = head_dim
        self.dtype = dtype
        s = self.stats()
        self.seq_len = s["seq_len"]
        self.kv_len = s["kv_len"]
        self.unmasked_pairs = s["unmasked_pairs"]

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ValueError("mask descriptor already freed")
        return self._h

    def stats(self) -> dict:
        st = aj_mask_stats()
        _check(lib().attn_jvp_mask_desc_stats(self.handle, ctypes.byref(st)), "attn_jvp_mask_desc_stats")
        return {f: getattr(st, f) for f, _ in aj_mask_stats._fields_}

    def tile_kind(self, q_tile: int, k_tile: int) -> int:
        k = ctypes.c_int32()
        _check(lib().attn_jvp_mask_desc_tile_kind(self.handle, q_tile, k_tile, ctypes.byref(k)),
               "attn_jvp_mask_desc_tile_kind")
        return k.value

    def tile_variant(self, q_tile: int, k_tile: int) -> int:
        """-1 skipped, 0 all JVP products, 1 keys tangent-free, 3 all tangent-free."""
        k = ctypes.c_int32()
        _check(lib().attn_jvp_mask_desc_tile_variant(self.handle, q_tile, k_tile, ctypes.byref(k)),
               "attn_jvp_mask_desc_tile_variant")
        return k.value

    def work(self) -> Tuple[int, int, int]:
        """Allowed pairs per (batch, head) in tiles doing 12 D, 8 D and 4 D FLOP per pair."""
        w = (ctypes.c_int64 * 3)()
        _check(lib().attn_jvp_mask_desc_work(self.handle, w), "attn_jvp_mask_desc_work")
        return int(w[0]), int(w[1]), int(w[2])

    def row_bits(self, q_tile: int, k_tile: int, row: int) -> int:
        b = ctypes.c_uint64()
        _check(lib().attn_jvp_mask_desc_row_bits(self.handle, q_tile, k_tile, row, ctypes.byref(b)),
               "attn_jvp_mask_desc_row_bits")
        return b.value

    def col_bits(self, k_tile: int, q_tile: int, key_row: int) -> int:
        """Bitmask over the 64 queries of q_tile that may attend key k_tile*128 + key_row."""
        b = ctypes.c_uint64()
        _check(lib().attn_jvp_mask_desc_col_bits(self.handle, k_tile, q_tile, key_row, ctypes.byref(b)),
               "attn_jvp_mask_desc_col_bits")
        return b.value

    def upload(self, device=None) -> "MaskDesc":
        """Copies the tables to a GPU (default: torch's current device); once per
        device, before the first launch there and outside any graph capture."""
        import torch

        if device is None:
            index = torch.cuda.current_device()
        else:
            dv = torch.device(device) if not isinstance(device, int) else torch.device("cuda", device)
            if dv.type != "cuda":
                raise ValueError(f"descriptor tables go to a GPU, not {dv}")
            index = torch.cuda.current_device() if dv.index is None else dv.index
        _check(lib().attn_jvp_mask_desc_upload(self.handle, int(index)), "attn_jvp_mask_desc_upload")
        return self

    def close(self) -> None:
        if self._h:
            attn_jvp_mask_desc_free(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _place(desc: MaskDesc, device) -> MaskDesc:
    """Uploads a new descriptor: device "auto" = torch's current GPU if there is
    one (none: host-only), None = host-only, else that device."""
    if device is None:
        return desc
    if isinstance(device, str) and device == "auto":
        import torch

        if not torch.cuda.is_available():
            return desc
        device = None
    return desc.upload(device)


def _flatten(items, width: int, what: str):
    """Flattens a sequence of width-tuples of ints, rejecting tuples of any other length."""
    flat = []
    for r in items:
        r = [int(x) for x in r]
        if len(r) != width:
            raise ValueError(f"each {what} needs {width} integers, got {len(r)}")
        flat.extend(r)
    return flat


def attn_jvp_mask_desc_build(kind: str, num_frames: int, frame_tokens: int, frames_per_chunk: int = 1,
                             head_dim: int = 128, dtype="bf16", seq_len: Optional[int] = None,
                             device="auto") -> MaskDesc:
    """Descriptor for a frame-level layout (see ``aj_mask_kind`` in the header),
    uploaded to ``device`` (see ``_place``)."""
    k = MASK_KINDS[kind] if isinstance(kind, str) else int(kind)
    spec = aj_mask_spec(k, num_frames, frame_tokens, frames_per_chunk)
    if seq_len is None:
        seq_len = num_frames * frame_tokens * (2 if k == MASK_KINDS["tf_clean_noisy"] else 1)
    out = ctypes.c_void_p()
    dt = _dtype_code(dtype)
    _check(lib().attn_jvp_mask_desc_build(ctypes.byref(spec), seq_len, head_dim, dt, ctypes.byref(out)),
           "attn_jvp_mask_desc_build")
    return _place(MaskDesc(out.value, head_dim, dt), device)


def attn_jvp_mask_desc_from_rects(seq_len: int, rects: Sequence[Sequence[int]], head_dim: int = 128,
                                  dtype="bf16", device="auto") -> MaskDesc:
    """Descriptor from disjoint half-open rectangles (q0, q1, k0, k1)."""
    flat = _flatten(rects, 4, "rectangle")
    arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    out = ctypes.c_void_p()
    dt = _dtype_code(dtype)
    _check(lib().attn_jvp_mask_desc_from_rects(seq_len, ctypes.cast(arr, ctypes.c_void_p), len(flat) // 4,
                                               head_dim, dt, ctypes.byref(out)),
           "attn_jvp_mask_desc_from_rects")
    return _place(MaskDesc(out.value, head_dim, dt), device)


def attn_jvp_mask_desc_from_rects_kv(q_len: int, kv_len: int, rects: Sequence[Sequence[int]], head_dim: int = 128,
                                     dtype="bf16", device="auto") -> MaskDesc:
    """Descriptor for a query chunk of q_len tokens over kv_len cached keys, from
    disjoint half-open rectangles (q0, q1, k0, k1)."""
    flat = _flatten(rects, 4, "rectangle")
    arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    out = ctypes.c_void_p()
    dt = _dtype_code(dtype)
    _check(lib().attn_jvp_mask_desc_from_rects_kv(q_len, kv_len, ctypes.cast(arr, ctypes.c_void_p), len(flat) // 4,
                                                  head_dim, dt, ctypes.byref(out)),
           "attn_jvp_mask_desc_from_rects_kv")
    return _place(MaskDesc(out.value, head_dim, dt), device)


def attn_jvp_mask_desc_tangent_free(base: MaskDesc, ranges: Sequence[Sequence[int]], device="auto") -> MaskDesc:
    """Descriptor with base's mask that declares tq, tk, tv zero on the token
    ranges [t0, t1) (see the header); the JVP then skips the zero products."""
    flat = _flatten(ranges, 2, "range")
    arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    out = ctypes.c_void_p()
    _check(lib().attn_jvp_mask_desc_tangent_free(base.handle, ctypes.cast(arr, ctypes.c_void_p), len(flat) // 2,
                                                 ctypes.byref(out)),
           "attn_jvp_mask_desc_tangent_free")
    return _place(MaskDesc(out.value, base.head_dim, base.dtype), device)


def attn_jvp_mask_desc_free(handle) -> None:
    lib().attn_jvp_mask_desc_free(handle)


def _prepare(ins, out_dtype, scale, out, n_out_tensors):
    """Checks the inputs and builds (shape struct, outputs, scale)."""
    import torch

    x0 = ins[0]
    if any(t.device != x0.device for t in ins) or x0.device.type != "cuda":
        raise ValueError("all inputs must be on the same GPU device")
    if any(t.dtype != x0.dtype for t in ins) or any(t.shape != x0.shape for t in ins):
        raise ValueError("inputs must share dtype and shape")
    if any(t.stride() != x0.stride() for t in ins):
        raise ValueError("inputs must share strides")
    if x0.dim() != 4 or x0.stride(3) != 1:
        raise ValueError("inputs must be [B, H, L, D] with D contiguous")
    B, H, L, D = x0.shape
    in_dt = {torch.bfloat16: AJ_BF16, torch.float32: AJ_F32}.get(x0.dtype)
    if in_dt is None:
        raise ValueError(f"unsupported input dtype {x0.dtype}")
    odt = x0.dtype if out_dtype is None else out_dtype
    out_dt = {torch.bfloat16: AJ_BF16, torch.float32: AJ_F32}.get(odt)
    if out_dt is None:
        raise ValueError(f"unsupported output dtype {odt}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        # outputs in the inputs' layout (e.g. [B, L, H, D] storage viewed as
        # [B, H, L, D]), so that attn_fwd's O can feed attn_bwd, which reads O
        # with the inputs' strides
        outs = [torch.empty_like(x0, dtype=odt) for _ in range(n_out_tensors)]
        if outs[0].stride(3) != 1:
            outs = [torch.empty((B, H, L, D), dtype=odt, device=x0.device) for _ in range(n_out_tensors)]
        lse = torch.empty((B, H, L), dtype=torch.float32, device=x0.device)
    else:
        *outs, lse = out
        if len(outs) != n_out_tensors:
            raise ValueError(f"out must hold {n_out_tensors + 1} tensors")
        if any(t.device != x0.device for t in (*outs, lse)):
            raise ValueError("preallocated outputs must be on the inputs' device")
        for o in outs:
            if o.shape != x0.shape or o.dtype != odt:
                raise ValueError("preallocated outputs have the wrong shape or dtype")
            if o.stride() != outs[0].stride() or o.stride(3) != 1:
                raise ValueError("preallocated outputs must share strides with D contiguous")
        if lse.shape != (B, H, L) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("preallocated lse must be a contiguous float32 [B, H, L] tensor")
    sh = aj_shape(B, H, L, D, in_dt, out_dt, *x0.stride()[:3], *outs[0].stride()[:3])
    return sh, outs, lse, float(scale)


def attn_jvp_fwd(q, k, v, tq, tk, tv, mask: MaskDesc, scale: Optional[float] = None,
                 out_dtype=None, out: Optional[Tuple] = None, stream=None):
    """O, tO, lse of masked attention and its JVP on the GPU (one kernel launch).

    q, k, v, tq, tk, tv: CUDA/HIP tensors [B, H, L, D] (bf16 or fp32) with the
    D axis contiguous and identical strides.  Returns (o, to, lse): o and to
    [B, H, L, D] in ``out_dtype`` (default: the input dtype), lse [B, H, L]
    float32.  ``out`` may pass preallocated (o, to, lse).
    """
    import torch

    ins = (q, k, v, tq, tk, tv)
    sh, (o, to), lse, scale = _prepare(ins, out_dtype, scale, out, 2)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().attn_jvp_fwd(ctypes.byref(sh), *(t.data_ptr() for t in ins), mask.handle, scale,
                                o.data_ptr(), to.data_ptr(), lse.data_ptr(), ctypes.c_void_p(stream))
    _check(st, "attn_jvp_fwd")
    return o, to, lse


def attn_jvp_fwd_v16(q, k, v, tq, tk, tv, mask: MaskDesc, scale: Optional[float] = None,
                     out_dtype=None, out: Optional[Tuple] = None, v16: Optional[Tuple] = None, stream=None):
    """attn_jvp_fwd at head_dim 64 (bf16 inputs) through fp16 copies of v and tv
    that the call writes first into ``v16`` = (v16, tv16): float16 tensors of
    v's shape and strides (allocated here when not given).  Same results as
    attn_jvp_fwd, bit for bit.  Returns (o, to, lse)."""
    import torch

    ins = (q, k, v, tq, tk, tv)
    sh, (o, to), lse, scale = _prepare(ins, out_dtype, scale, out, 2)
    if v16 is None:
        v16 = tuple(torch.empty_like(v, dtype=torch.float16) for _ in range(2))
    if len(v16) != 2 or any(t.dtype != torch.float16 or t.shape != v.shape or t.stride() != v.stride()
                            or t.device != v.device for t in v16):
        raise ValueError("v16 must hold two float16 tensors with v's shape, strides and device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().attn_jvp_fwd_v16(ctypes.byref(sh), *(t.data_ptr() for t in ins), mask.handle, scale,
                                    o.data_ptr(), to.data_ptr(), lse.data_ptr(), v16[0].data_ptr(),
                                    v16[1].data_ptr(), ctypes.c_void_p(stream))
    _check(st, "attn_jvp_fwd_v16")
    return o, to, lse


def attn_fwd(q, k, v, mask: MaskDesc, scale: Optional[float] = None, out_dtype=None,
             out: Optional[Tuple] = None, stream=None):
    """O, lse of masked attention (primal forward, bf16 inputs) on the GPU.

    Same conventions as ``attn_jvp_fwd``; ``out`` may pass preallocated (o, lse).
    """
    import torch

    ins = (q, k, v)
    sh, (o,), lse, scale = _prepare(ins, out_dtype, scale, out, 1)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().attn_fwd(ctypes.byref(sh), *(t.data_ptr() for t in ins), mask.handle, scale,
                            o.data_ptr(), lse.data_ptr(), ctypes.c_void_p(stream))
    _check(st, "attn_fwd")
    return o, lse


def attn_fwd_kv(q, k_cache, v_cache, mask: MaskDesc, scale: Optional[float] = None, out_dtype=None,
                out: Optional[Tuple] = None, stream=None):
    """O, lse of a query chunk q [B, H, Lq, D] over the first ``mask.kv_len``
    positions of the caches k_cache, v_cache [B, H, >= kv_len, D] (bf16, D
    contiguous, own strides).  ``out`` may pass preallocated (o, lse)."""
    import torch

    if q.dim() != 4 or k_cache.dim() != 4 or q.stride(3) != 1 or k_cache.stride(3) != 1:
        raise ValueError("q and the caches must be [B, H, L, D] with D contiguous")
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share shape and strides")
    if any(t.device != q.device for t in (k_cache, v_cache)) or q.device.type != "cuda":
        raise ValueError("all tensors must be on the same GPU device")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share dtype")
    B, H, Lq, D = q.shape
    if k_cache.shape[0] != B or k_cache.shape[1] != H or k_cache.shape[3] != D:
        raise ValueError("cache batch, heads and head_dim must match q")
    kv_len = mask.kv_len
    if k_cache.shape[2] < kv_len:
        raise ValueError(f"cache holds {k_cache.shape[2]} positions, the mask needs {kv_len}")
    in_dt = {torch.bfloat16: AJ_BF16, torch.float32: AJ_F32}.get(q.dtype)
    if in_dt is None:
        raise ValueError(f"unsupported input dtype {q.dtype}")
    odt = q.dtype if out_dtype is None else out_dtype
    out_dt = {torch.bfloat16: AJ_BF16, torch.float32: AJ_F32}.get(odt)
    if out_dt is None:
        raise ValueError(f"unsupported output dtype {odt}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        o = torch.empty((B, H, Lq, D), dtype=odt, device=q.device)
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if o.device != q.device or lse.device != q.device:
            raise ValueError("preallocated outputs must be on the inputs' device")
        if o.shape != q.shape or o.dtype != odt or o.stride(3) != 1:
            raise ValueError("preallocated o has the wrong shape, dtype or layout")
        if lse.shape != (B, H, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("preallocated lse must be a contiguous float32 [B, H, Lq] tensor")
    sh = aj_kv_shape(B, H, Lq, kv_len, D, in_dt, out_dt, *q.stride()[:3], *k_cache.stride()[:3], *o.stride()[:3])
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().attn_fwd_kv(ctypes.byref(sh), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), mask.handle,
                               float(scale), o.data_ptr(), lse.data_ptr(), ctypes.c_void_p(stream))
    _check(st, "attn_fwd_kv")
    return o, lse


def attn_bwd(q, k, v, o, dout, lse, mask: MaskDesc, scale: Optional[float] = None, out_dtype=None,
             out: Optional[Tuple] = None, stream=None):
    """dq, dk, dv of masked attention for the cotangent ``dout`` (bf16 inputs).

    ``o`` and ``lse`` are the forward's outputs for the same inputs, mask and
    scale.  ``o`` and ``dout`` must have q's dtype (bf16) and strides: the C
    entry point reads all five inputs with one set of strides; attn_fwd's
    default output has the inputs' layout.  Returns (dq, dk, dv, delta): the
    gradients [B, H, L, D] in
    ``out_dtype`` (default bf16) and delta = rowsum(dout * o) [B, H, L] float32.
    ``out`` may pass preallocated (dq, dk, dv, delta).
    """
    import torch

    ins = (q, k, v, o, dout)
    x0 = q
    B, H, L, D = x0.shape
    if lse.shape != (B, H, L) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != x0.device:
        raise ValueError("lse must be a contiguous float32 [B, H, L] tensor on the inputs' device")
    if out is None:
        sh, (dq, dk, dv), delta, scale = _prepare(ins, out_dtype, scale, None, 3)
    else:
        sh, (dq, dk, dv), delta, scale = _prepare(ins, out_dtype, scale, tuple(out), 3)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().attn_bwd(ctypes.byref(sh), *(t.data_ptr() for t in ins), lse.data_ptr(), mask.handle, scale,
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), ctypes.c_void_p(stream))
    _check(st, "attn_bwd")
    return dq, dk, dv, delta


def attn_bwd_noalloc(q, k, v, o, dout, lse, mask: MaskDesc, scale: Optional[float] = None, out_dtype=None,
                     out: Optional[Tuple] = None, stream=None):
    """attn_bwd for callers that cannot allocate device memory: D is kept in the
    library's per-GPU array (B * H * L <= 4,194,304; calls that overlap on one
    GPU race).  Returns (dq, dk, dv); ``out`` may pass preallocated (dq, dk, dv)
    so that the call allocates nothing at all."""
    import torch

    ins = (q, k, v, o, dout)
    B, H, L, D = q.shape
    if lse.shape != (B, H, L) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, L] tensor on the inputs' device")
    if out is None:
        sh, (dq, dk, dv), _, scale = _prepare(ins, out_dtype, scale, None, 3)
    else:
        # _prepare's out carries an lse slot; pass the input lse there (only checked)
        sh, (dq, dk, dv), _, scale = _prepare(ins, out_dtype, scale, tuple(out) + (lse,), 3)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().attn_bwd_noalloc(ctypes.byref(sh), *(t.data_ptr() for t in ins), lse.data_ptr(), mask.handle,
                                    scale, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ctypes.c_void_p(stream))
    _check(st, "attn_bwd_noalloc")
    return dq, dk, dv


__all__ = [
    "AJ_OK", "AJ_EINVAL", "AJ_ENOTSUP", "AJ_ENOMEM", "AJ_EHIP", "AJ_EMASK", "AJ_ENOTLOADED", "AJ_F32", "AJ_BF16",
    "AttnJvpError", "MaskDesc", "lib", "status_str", "attn_jvp_version", "attn_jvp_mask_desc_build",
    "attn_jvp_mask_desc_from_rects", "attn_jvp_mask_desc_tangent_free", "attn_jvp_mask_desc_free",
    "attn_jvp_mask_desc_from_rects_kv", "attn_jvp_fwd", "attn_jvp_fwd_v16", "attn_fwd", "attn_fwd_kv", "attn_bwd",
    "attn_bwd_noalloc",
    "LIB_PATH",
]
