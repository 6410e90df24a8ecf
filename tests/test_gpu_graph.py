"""The launch paths under HIP graph capture.

The descriptor builders upload the tables to the GPU; after that attn_jvp_fwd
(also with a tangent-free descriptor: two launches), attn_jvp_fwd_v16 (the fp16
copies, then the JVP), attn_fwd, attn_fwd_kv and attn_bwd enqueue kernels only: no allocation, no memset, no host
synchronisation, from the very first call on.  They are captured into a graph on torch's capture stream and
the graph is replayed several times, with eager work and synchronisation in
between; every replay must reproduce the eager results bit for bit (the
kernels are deterministic).
"""
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "tq", "tk", "tv")


def test_jvp_and_gradients_replay_from_a_graph():
    w = Workload("graph", 1, 2, 128, "bf16", "block_causal", 5, 90, 1, seed=160)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    desc = aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=w.head_dim, dtype=w.dtype)
    B, H, L, D = w.shape
    jvp_out = (torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L), dtype=torch.float32, device="cuda"))
    fwd_out = (torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L), dtype=torch.float32, device="cuda"))
    bwd_out = tuple(torch.empty((B, H, L, D), dtype=torch.float32, device="cuda") for _ in range(3)) + (
        torch.empty((B, H, L), dtype=torch.float32, device="cuda"),)
    g = torch.Generator().manual_seed(3)
    d_out = torch.randn(w.shape, generator=g).to(torch.bfloat16).cuda()

    def run():
        aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc, scale=w.scale, out=jvp_out)
        aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc, scale=w.scale, out=fwd_out)
        aj.attn_bwd(dev["q"], dev["k"], dev["v"], fwd_out[0], d_out, fwd_out[1], desc, scale=w.scale,
                    out_dtype=torch.float32, out=bwd_out)

    run()  # eager reference
    torch.cuda.synchronize()
    want = [t.clone() for t in jvp_out + fwd_out + bwd_out]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for t in jvp_out + fwd_out + bwd_out:
            t.fill_(float("nan"))  # eager, outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in jvp_out + fwd_out + bwd_out:
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(jvp_out + fwd_out + bwd_out, want):
            assert torch.equal(got, ref), f"replay {rep} differs from the eager result"


def test_tangent_free_path_and_kv_forward_replay_from_a_graph():
    # the tangent-free descriptor takes two launches per call (primal-only
    # query tiles, then the rest); the KV-cache forward reads a cache longer
    # than the prefix it uses
    w = Workload("graph_tf", 1, 2, 128, "bf16", "tf_clean_noisy", 4, 90, 1, seed=161, clean_tangent_zero=True)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    base = aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=w.head_dim, dtype=w.dtype)
    fast = aj.attn_jvp_mask_desc_tangent_free(base, [(0, w.seq_len // 2)])
    assert fast.work()[2] > 0
    B, H, L, D = w.shape
    q_len, kv_len = 120, 300
    kv_desc = aj.attn_jvp_mask_desc_from_rects_kv(q_len, kv_len, [(0, q_len, 0, kv_len)], head_dim=D, dtype="bf16")
    q_chunk = dev["q"][:, :, L - q_len:]
    jvp_out = (torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L), dtype=torch.float32, device="cuda"))
    kv_out = (torch.empty((B, H, q_len, D), dtype=torch.bfloat16, device="cuda"),
              torch.empty((B, H, q_len), dtype=torch.float32, device="cuda"))

    def run():
        aj.attn_jvp_fwd(*(dev[n] for n in NAMES), fast, scale=w.scale, out=jvp_out)
        aj.attn_fwd_kv(q_chunk, dev["k"], dev["v"], kv_desc, scale=w.scale, out=kv_out)

    run()  # eager reference
    torch.cuda.synchronize()
    want = [t.clone() for t in jvp_out + kv_out]
    assert bool((want[1][:, :, : L // 2] == 0).all())  # tO on the declared tangent-free rows

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for t in jvp_out + kv_out:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in jvp_out + kv_out:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(jvp_out + kv_out, want):
            assert torch.equal(got, ref), f"replay {rep} differs from the eager result"


def test_first_launch_of_a_fresh_descriptor_is_captured():
    # Fresh descriptors whose first launch ever happens inside the capture:
    # the builders uploaded their tables, so the launches only enqueue kernels.
    # A descriptor built host-only is refused inside the capture with a status
    # code, enqueues nothing, and the capture goes on.
    w = Workload("graph_first", 1, 3, 64, "bf16", "block_causal", 6, 70, 2, seed=162)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    B, H, L, D = w.shape
    mk = lambda device: aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                                    head_dim=D, dtype=w.dtype, device=device)
    desc, desc_f = mk("auto"), mk("auto")
    host_only = mk(None)
    jvp_out = (torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L), dtype=torch.float32, device="cuda"))
    fwd_out = (torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L), dtype=torch.float32, device="cuda"))
    refused = (torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L), dtype=torch.float32, device="cuda"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    print("[case] first launch of fresh descriptors under capture", flush=True)
    with torch.cuda.stream(s):
        for t in jvp_out + fwd_out + refused:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc, scale=w.scale, out=jvp_out)
            with pytest.raises(aj.AttnJvpError) as e:
                aj.attn_fwd(dev["q"], dev["k"], dev["v"], host_only, scale=w.scale, out=refused)
            assert e.value.status == aj.AJ_ENOTLOADED
            aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc_f, scale=w.scale, out=fwd_out)
    torch.cuda.synchronize()
    # eager references, after the capture
    want_jvp = aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc, scale=w.scale)
    want_fwd = aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc_f, scale=w.scale)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in jvp_out + fwd_out:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(jvp_out + fwd_out, want_jvp + want_fwd):
            assert torch.equal(got, ref), f"replay {rep} differs from the eager result"
        assert all(bool(t.isnan().all()) for t in refused), "the refused call must write nothing"
    # once uploaded, the host-only descriptor gives the same result
    host_only.upload()
    o, lse = aj.attn_fwd(dev["q"], dev["k"], dev["v"], host_only, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, want_fwd[0]) and torch.equal(lse, want_fwd[1])


def test_fp16_copy_path_replays_from_a_graph():
    # attn_jvp_fwd_v16: the conversion kernel and the JVP kernel, both captured;
    # the copy buffers are filled with NaN between replays
    w = Workload("graph_v16", 2, 2, 64, "bf16", "block_causal", 6, 70, 3, seed=162)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    desc = aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=w.head_dim, dtype=w.dtype)
    B, H, L, D = w.shape
    out = (torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
           torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
           torch.empty((B, H, L), dtype=torch.float32, device="cuda"))
    v16 = tuple(torch.empty_like(dev[n], dtype=torch.float16) for n in ("v", "tv"))

    def run():
        aj.attn_jvp_fwd_v16(*(dev[n] for n in NAMES), desc, scale=w.scale, out=out, v16=v16)

    run()
    torch.cuda.synchronize()
    want = [t.clone() for t in out + v16]
    plain = aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc, scale=w.scale)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(out, plain)), "attn_jvp_fwd_v16 differs from attn_jvp_fwd"

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for t in out + v16:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out + v16:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(out + v16, want):
            assert torch.equal(got, ref), f"replay {rep} differs from the eager result"
