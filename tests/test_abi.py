"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any device work (CPU only: every forward call
here carries an invalid argument, so nothing is ever launched)."""
import ctypes
import math
import os
import re

import pytest

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd import aj_shape

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn_jvp.h")
FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails validation first


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 9
    lib = aj.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    for code in range(7):
        s = aj.status_str(code)
        assert s.startswith("AJ_")
    assert aj.status_str(99) == "unknown status"
    assert aj.attn_jvp_version() >= 10000


def _build(kind, T, F, c, L, D=128, dt=aj.AJ_BF16):
    spec = aj.aj_mask_spec(kind, T, F, c)
    out = ctypes.c_void_p(1234)
    st = aj.lib().attn_jvp_mask_desc_build(ctypes.byref(spec), L, D, dt, ctypes.byref(out))
    if st == aj.AJ_OK:
        aj.lib().attn_jvp_mask_desc_free(out)
    else:
        assert out.value is None  # set to NULL on error
    return st


def test_mask_desc_build_errors():
    lib = aj.lib()
    assert lib.attn_jvp_mask_desc_build(None, 10, 128, aj.AJ_BF16, None) == aj.AJ_EINVAL
    out = ctypes.c_void_p()
    assert lib.attn_jvp_mask_desc_build(None, 10, 128, aj.AJ_BF16, ctypes.byref(out)) == aj.AJ_EINVAL
    assert _build(1, 4, 16, 1, 64) == aj.AJ_OK
    assert _build(7, 4, 16, 1, 64) == aj.AJ_EMASK          # unknown kind
    assert _build(1, 4, 16, 1, 65) == aj.AJ_EMASK          # seq_len mismatch
    assert _build(2, 4, 16, 1, 64) == aj.AJ_EMASK          # TF needs 2 * T * F
    assert _build(2, 4, 16, 1, 128) == aj.AJ_OK
    assert _build(1, 0, 16, 1, 0) == aj.AJ_EINVAL          # seq_len < 1
    assert _build(1, 4, 0, 1, 64) == aj.AJ_EMASK           # bad frame size
    assert _build(1, 4, 16, 0, 64) == aj.AJ_EMASK          # bad chunk size
    assert _build(1, 4, 16, 1, 64, D=96) == aj.AJ_ENOTSUP
    assert _build(1, 4, 16, 1, 64, dt=5) == aj.AJ_ENOTSUP


def _rects(L, rects):
    flat = [x for r in rects for x in r]
    arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    out = ctypes.c_void_p()
    st = aj.lib().attn_jvp_mask_desc_from_rects(L, ctypes.cast(arr, ctypes.c_void_p), len(rects), 128,
                                                aj.AJ_BF16, ctypes.byref(out))
    if st == aj.AJ_OK:
        aj.lib().attn_jvp_mask_desc_free(out)
    return st


def test_from_rects_errors():
    assert _rects(100, [(0, 50, 0, 50), (50, 100, 0, 100)]) == aj.AJ_OK
    assert _rects(100, [(0, 50, 0, 50), (40, 100, 40, 60)]) == aj.AJ_EMASK   # overlap
    assert _rects(100, [(0, 101, 0, 50)]) == aj.AJ_EMASK                     # out of range
    assert _rects(100, [(5, 5, 0, 50)]) == aj.AJ_EMASK                       # empty range
    assert _rects(100, [(0, 10, -1, 5)]) == aj.AJ_EMASK
    assert _rects(100, []) == aj.AJ_OK                                       # nothing allowed
    assert aj.lib().attn_jvp_mask_desc_from_rects(100, None, 3, 128, aj.AJ_BF16, ctypes.byref(ctypes.c_void_p())) == aj.AJ_EINVAL


def test_binding_rejects_ragged_rectangles_and_ranges():
    with pytest.raises(ValueError):
        aj.attn_jvp_mask_desc_from_rects(100, [(0, 50, 0)], head_dim=128)
    with pytest.raises(ValueError):
        aj.attn_jvp_mask_desc_from_rects_kv(10, 100, [(0, 10, 0, 100, 7)], head_dim=128)
    base = aj.attn_jvp_mask_desc_build("block_causal", 4, 50, 1, head_dim=128)
    with pytest.raises(ValueError):
        aj.attn_jvp_mask_desc_tangent_free(base, [(0, 50, 60)])
    d = aj.attn_jvp_mask_desc_tangent_free(base, [(0, 50)])
    assert d.seq_len == 200


def test_query_errors():
    lib = aj.lib()
    d = aj.attn_jvp_mask_desc_build("block_causal", 4, 50, 1, head_dim=128)
    k = ctypes.c_int32()
    b = ctypes.c_uint64()
    assert lib.attn_jvp_mask_desc_stats(None, None) == aj.AJ_EINVAL
    assert lib.attn_jvp_mask_desc_tile_kind(d.handle, 2, 0, ctypes.byref(k)) == aj.AJ_EINVAL
    assert lib.attn_jvp_mask_desc_tile_kind(d.handle, 0, 4, ctypes.byref(k)) == aj.AJ_EINVAL
    assert lib.attn_jvp_mask_desc_tile_kind(d.handle, 0, 0, None) == aj.AJ_EINVAL
    assert lib.attn_jvp_mask_desc_row_bits(d.handle, 0, 0, 128, ctypes.byref(b)) == aj.AJ_EINVAL
    assert lib.attn_jvp_mask_desc_row_bits(d.handle, 0, 0, -1, ctypes.byref(b)) == aj.AJ_EINVAL
    lib.attn_jvp_mask_desc_free(None)  # no-op
    d.close()
    d.close()  # idempotent on the Python side
    with pytest.raises(ValueError):
        d.stats()


def _shape(B=1, H=2, L=64, D=128, idt=aj.AJ_BF16, odt=aj.AJ_BF16, ins=None, outs=None):
    ins = ins or (H * L * D, L * D, D)
    outs = outs or (H * L * D, L * D, D)
    return aj_shape(B, H, L, D, idt, odt, *ins, *outs)


def _fwd(shape, desc, ptrs=None, scale=0.125, lse=FAKE):
    ptrs = ptrs or [FAKE] * 8
    p = [ctypes.c_void_p(x) if x is not None else None for x in ptrs]
    return aj.lib().attn_jvp_fwd(ctypes.byref(shape) if shape is not None else None, *p[:6],
                                 desc, ctypes.c_float(scale), p[6], p[7],
                                 ctypes.c_void_p(lse) if lse is not None else None, None)


def test_fwd_rejects_bad_arguments_before_launch():
    d = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=128, dtype="bf16")
    h = d.handle
    d64 = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=64, dtype="bf16")
    df32 = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=128, dtype="f32")
    E = aj
    assert _fwd(None, h) == E.AJ_EINVAL
    assert _fwd(_shape(), None) == E.AJ_EINVAL
    for i in range(8):  # each null pointer (q..tv, o, to)
        ptrs = [FAKE] * 8
        ptrs[i] = None
        assert _fwd(_shape(), h, ptrs) == E.AJ_EINVAL
    assert _fwd(_shape(), h, lse=None) == E.AJ_EINVAL
    ptrs = [FAKE] * 8
    ptrs[2] = FAKE + 8  # misaligned v
    assert _fwd(_shape(), h, ptrs) == E.AJ_EINVAL
    assert _fwd(_shape(), h, lse=FAKE + 4) == E.AJ_EINVAL
    assert _fwd(_shape(B=0), h) == E.AJ_EINVAL
    assert _fwd(_shape(H=0), h) == E.AJ_EINVAL
    assert _fwd(_shape(), h, scale=float("nan")) == E.AJ_EINVAL
    assert _fwd(_shape(), h, scale=float("inf")) == E.AJ_EINVAL
    assert _fwd(_shape(), h, scale=0.0) == E.AJ_EINVAL
    assert _fwd(_shape(), h, scale=-0.1) == E.AJ_EINVAL
    assert _fwd(_shape(), h, scale=-0.0) == E.AJ_EINVAL
    assert _fwd(_shape(), h, scale=float("-inf")) == E.AJ_EINVAL
    assert _fwd(_shape(), h, scale=-float("nan")) == E.AJ_EINVAL
    assert _fwd(_shape(D=96), h) == E.AJ_ENOTSUP
    assert _fwd(_shape(idt=aj.AJ_F32, odt=aj.AJ_BF16), df32.handle) == E.AJ_ENOTSUP
    assert _fwd(_shape(idt=3), h) == E.AJ_ENOTSUP
    assert _fwd(_shape(ins=(2 * 64 * 128, 64 * 128, 132)), h) == E.AJ_EINVAL      # stride not 16-byte multiple
    assert _fwd(_shape(outs=(2 * 64 * 128, 64 * 128, 64)), h) == E.AJ_EINVAL     # overlapping output rows
    assert _fwd(_shape(B=2, outs=(2 * 64 * 128, 100 * 128, 128)), h) == E.AJ_EINVAL  # head 1 overlaps batch 1
    assert _fwd(_shape(outs=(-128, 64 * 128, 128)), h) == E.AJ_EINVAL
    assert _fwd(_shape(L=80), h) == E.AJ_EMASK                                   # descriptor L differs
    assert _fwd(_shape(D=64), h) == E.AJ_EMASK                                   # descriptor D differs
    assert _fwd(_shape(), df32.handle) == E.AJ_EMASK                             # descriptor dtype differs
    assert _fwd(_shape(D=128), d64.handle) == E.AJ_EMASK


def _fwd_v16(shape, desc, ptrs=None, scale=0.125, lse=FAKE, v16=FAKE + 4096, tv16=FAKE + 8192):
    ptrs = ptrs or [FAKE] * 8
    p = [ctypes.c_void_p(x) if x is not None else None for x in ptrs]
    w = [ctypes.c_void_p(x) if x is not None else None for x in (v16, tv16)]
    return aj.lib().attn_jvp_fwd_v16(ctypes.byref(shape) if shape is not None else None, *p[:6],
                                     desc, ctypes.c_float(scale), p[6], p[7],
                                     ctypes.c_void_p(lse) if lse is not None else None, *w, None)


def test_fwd_v16_rejects_bad_arguments_before_launch():
    d64 = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=64, dtype="bf16")
    d128 = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=128, dtype="bf16")
    df32 = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=64, dtype="f32")
    s64 = _shape(D=64, ins=(2 * 64 * 64, 64 * 64, 64), outs=(2 * 64 * 64, 64 * 64, 64))
    assert _fwd_v16(s64, d64.handle, v16=None) == aj.AJ_EINVAL
    assert _fwd_v16(s64, d64.handle, tv16=None) == aj.AJ_EINVAL
    assert _fwd_v16(s64, d64.handle, v16=FAKE + 8) == aj.AJ_EINVAL             # misaligned copy buffer
    assert _fwd_v16(s64, d64.handle, v16=FAKE) == aj.AJ_EINVAL                  # the copy buffer is an input
    assert _fwd_v16(s64, d64.handle, v16=FAKE + 4096, tv16=FAKE + 4096) == aj.AJ_EINVAL  # one buffer for both
    assert _fwd_v16(_shape(), d128.handle) == aj.AJ_ENOTSUP                     # head_dim 128: no fp16 copies
    s64f = _shape(D=64, idt=aj.AJ_F32, odt=aj.AJ_F32, ins=(2 * 64 * 64, 64 * 64, 64), outs=(2 * 64 * 64, 64 * 64, 64))
    assert _fwd_v16(s64f, df32.handle) == aj.AJ_ENOTSUP                         # fp32 inputs
    # the checks of attn_jvp_fwd apply as well
    assert _fwd_v16(None, d64.handle) == aj.AJ_EINVAL
    ptrs = [FAKE] * 8
    ptrs[2] = None
    assert _fwd_v16(s64, d64.handle, ptrs) == aj.AJ_EINVAL
    assert _fwd_v16(s64, d64.handle, scale=float("nan")) == aj.AJ_EINVAL
    assert _fwd_v16(s64, d128.handle) == aj.AJ_EMASK


def test_fwd_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; a valid call would launch")
    d = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=128, dtype="bf16")
    assert _fwd(_shape(), d.handle) == aj.AJ_EHIP


def test_permuted_output_layout_is_accepted_by_validation():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; a valid call would launch")
    # [B, L, H, D] strides are a valid non-overlapping layout (fails later for lack of a GPU)
    d = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=128, dtype="bf16")
    sh = _shape(outs=(64 * 2 * 128, 128, 2 * 128))
    assert _fwd(sh, d.handle) == aj.AJ_EHIP


def _primal(shape, desc, ptrs=None, scale=0.125, lse=FAKE):
    ptrs = ptrs or [FAKE] * 4
    p = [ctypes.c_void_p(x) if x is not None else None for x in ptrs]
    return aj.lib().attn_fwd(ctypes.byref(shape) if shape is not None else None, *p[:3], desc,
                             ctypes.c_float(scale), p[3], ctypes.c_void_p(lse) if lse is not None else None, None)


def _bwd(shape, desc, ptrs=None, scale=0.125, lse=FAKE, delta=FAKE):
    ptrs = ptrs or [FAKE] * 8  # q, k, v, o, dout, dq, dk, dv
    p = [ctypes.c_void_p(x) if x is not None else None for x in ptrs]
    return aj.lib().attn_bwd(ctypes.byref(shape) if shape is not None else None, *p[:5],
                             ctypes.c_void_p(lse) if lse is not None else None, desc, ctypes.c_float(scale),
                             *p[5:8], ctypes.c_void_p(delta) if delta is not None else None, None)


def test_primal_and_gradient_entry_points_reject_bad_arguments():
    d = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=128, dtype="bf16")
    df32 = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=128, dtype="f32")
    kv = aj.attn_jvp_mask_desc_from_rects_kv(64, 100, [(0, 64, 0, 100)], head_dim=128, dtype="bf16")
    h = d.handle
    assert _primal(None, h) == aj.AJ_EINVAL
    assert _primal(_shape(), None) == aj.AJ_EINVAL
    for i in range(4):
        ptrs = [FAKE] * 4
        ptrs[i] = None
        assert _primal(_shape(), h, ptrs) == aj.AJ_EINVAL
    assert _primal(_shape(), h, lse=None) == aj.AJ_EINVAL
    assert _primal(_shape(), h, scale=float("nan")) == aj.AJ_EINVAL
    assert _primal(_shape(idt=aj.AJ_F32, odt=aj.AJ_F32), df32.handle) == aj.AJ_ENOTSUP  # bf16 only
    assert _primal(_shape(), kv.handle) == aj.AJ_EMASK                                   # key length differs
    for i in range(8):
        ptrs = [FAKE] * 8
        ptrs[i] = None
        assert _bwd(_shape(), h, ptrs) == aj.AJ_EINVAL
    assert _bwd(_shape(), h, lse=None) == aj.AJ_EINVAL
    assert _bwd(_shape(), h, lse=FAKE + 4) == aj.AJ_EINVAL
    assert _bwd(_shape(), h, delta=None) == aj.AJ_EINVAL
    assert _bwd(_shape(), h, scale=0.0) == aj.AJ_EINVAL
    assert _bwd(_shape(L=80), h) == aj.AJ_EMASK
    assert _bwd(_shape(idt=aj.AJ_F32, odt=aj.AJ_F32), df32.handle) == aj.AJ_ENOTSUP
    assert _bwd(_shape(outs=(2 * 64 * 128, 64 * 128, 64)), h) == aj.AJ_EINVAL  # overlapping gradient rows


def _kvshape(B=1, H=2, Lq=64, Lk=100, D=128, qs=None, ks=None, os_=None, idt=aj.AJ_BF16, odt=aj.AJ_BF16):
    qs = qs or (H * Lq * D, Lq * D, D)
    ks = ks or (H * 4096 * D, 4096 * D, D)
    os_ = os_ or (H * Lq * D, Lq * D, D)
    return aj.aj_kv_shape(B, H, Lq, Lk, D, idt, odt, *qs, *ks, *os_)


def _fwd_kv(shape, desc, ptrs=None, scale=0.125, lse=FAKE):
    ptrs = ptrs or [FAKE] * 4
    p = [ctypes.c_void_p(x) if x is not None else None for x in ptrs]
    return aj.lib().attn_fwd_kv(ctypes.byref(shape) if shape is not None else None, *p[:3], desc,
                                ctypes.c_float(scale), p[3], ctypes.c_void_p(lse) if lse is not None else None, None)


def test_kv_entry_point_rejects_bad_arguments():
    kv = aj.attn_jvp_mask_desc_from_rects_kv(64, 100, [(0, 64, 0, 100)], head_dim=128, dtype="bf16")
    h = kv.handle
    assert _fwd_kv(None, h) == aj.AJ_EINVAL
    assert _fwd_kv(_kvshape(), None) == aj.AJ_EINVAL
    assert _fwd_kv(_kvshape(Lk=101), h) == aj.AJ_EMASK                      # descriptor key length differs
    assert _fwd_kv(_kvshape(Lq=65), h) == aj.AJ_EMASK
    assert _fwd_kv(_kvshape(ks=(0, 0, 64)), h) == aj.AJ_EINVAL              # key rows closer than D
    assert _fwd_kv(_kvshape(ks=(0, 0, 1 << 24)), h) == aj.AJ_EINVAL         # 64 key rows exceed a 31-bit range
    assert _fwd_kv(_kvshape(qs=(0, 0, 100)), h) == aj.AJ_EINVAL             # not a 16-byte multiple
    assert _fwd_kv(_kvshape(idt=aj.AJ_F32, odt=aj.AJ_F32), h) == aj.AJ_ENOTSUP  # bf16 only


def test_kv_entry_point_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; a valid call would launch")
    kv = aj.attn_jvp_mask_desc_from_rects_kv(64, 100, [(0, 64, 0, 100)], head_dim=128, dtype="bf16")
    assert _fwd_kv(_kvshape(), kv.handle) == aj.AJ_EHIP


def test_upload_rejects_bad_arguments():
    assert aj.lib().attn_jvp_mask_desc_upload(None, 0) == aj.AJ_EINVAL
    d = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=128, dtype="bf16", device=None)
    assert aj.lib().attn_jvp_mask_desc_upload(d.handle, -1) in (aj.AJ_EINVAL, aj.AJ_EHIP)
    import torch
    if torch.cuda.is_available():
        n = torch.cuda.device_count()
        assert aj.lib().attn_jvp_mask_desc_upload(d.handle, n) == aj.AJ_EINVAL
    else:
        # no GPU: the device count is unavailable
        assert aj.lib().attn_jvp_mask_desc_upload(d.handle, 0) == aj.AJ_EHIP
        # and the auto placement of the builders leaves the descriptor host-only
        d2 = aj.attn_jvp_mask_desc_build("block_causal", 4, 16, 1, head_dim=128, dtype="bf16")
        assert d2.stats()["seq_len"] == 64


def test_noalloc_gradients_reject_sizes_beyond_the_array():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; checked on the host only")
    # B * H * L = 1 * 64 * 65600 > 4,194,304: refused before any device work
    d = aj.attn_jvp_mask_desc_build("full", 1, 65600, 1, head_dim=64, dtype="bf16")
    sh = _shape(B=1, H=64, L=65600, D=64)
    p = [ctypes.c_void_p(FAKE)] * 8
    st = aj.lib().attn_bwd_noalloc(ctypes.byref(sh), *p[:5], ctypes.c_void_p(FAKE), d.handle, ctypes.c_float(0.125),
                                   *p[5:8], None)
    assert st == aj.AJ_EINVAL
    # within the limit the same call gets as far as the device (none here)
    d2 = aj.attn_jvp_mask_desc_build("full", 1, 64, 1, head_dim=64, dtype="bf16")
    sh2 = _shape(B=1, H=2, L=64, D=64)
    st = aj.lib().attn_bwd_noalloc(ctypes.byref(sh2), *p[:5], ctypes.c_void_p(FAKE), d2.handle, ctypes.c_float(0.125),
                                   *p[5:8], None)
    assert st == aj.AJ_EHIP
    # attn_bwd itself needs its delta argument
    assert _bwd(sh2, d2.handle, delta=None) == aj.AJ_EINVAL
