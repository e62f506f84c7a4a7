"""Split-KV workspace handling of the binding: a graph captured earlier
keeps working after a later call needs a larger workspace (superseded
buffers are never released), growth is refused during capture, and calls on
different streams use different buffers."""

from __future__ import annotations

import pytest
import torch

from attention_forward_amd import fa
from attention_forward_amd.workloads import WORKLOADS, make_custom, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def test_graph_survives_workspace_growth(gpu_device):
    """Capture the small-M shape, then run a causal chunk of 64 positions
    over an 8192-key cache on the same stream (a larger workspace), return
    freed memory to the device, and replay the first graph: bit-identical
    to eager."""
    _say("workspace growth after capture")
    w = WORKLOADS["action_expert_small_m"]
    q, k, v, s = (None if t is None else t.to(gpu_device) for t in make_inputs(w.name))
    o_eager, l_eager = fa.attention(q, k, v, seqused_k=s, scale=w.scale)
    out, lse = torch.empty_like(o_eager), torch.empty_like(l_eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fa.attention(q, k, v, seqused_k=s, scale=w.scale, out=out, lse=lse)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fa.attention(q, k, v, seqused_k=s, scale=w.scale, out=out, lse=lse)
    small = fa.fa_fwd_workspace_bytes(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D, w.causal)
    big = fa.fa_fwd_workspace_bytes(2, 64, 8192, 8, 1, 256, 1)
    held = fa._workspaces[(gpu_device.index or 0, stream.cuda_stream)].numel()
    assert big > held >= small, (small, held, big)
    dq, dk, dv, ds = (t.to(gpu_device) for t in make_custom(2, 64, 8192, 8, 1, 256, seed=9, n_valid=[8000, 8192]))
    with torch.cuda.stream(stream):
        fa.attention(dq, dk, dv, causal=True, seqused_k=ds, scale=0.0625)
    stream.synchronize()
    del dq, dk, dv
    torch.cuda.empty_cache()
    # scribble over whatever memory the allocator hands out now
    junk = torch.full((64 << 20,), 7, dtype=torch.uint8, device=gpu_device)
    for i in range(3):
        out.fill_(3.0)
        lse.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_eager) and torch.equal(lse, l_eager), f"replay {i}"
    del junk


def test_growth_refused_during_capture(gpu_device):
    """A call under capture that needs more workspace than its stream holds
    raises before anything is queued (here a variant that splits the
    prefix shape into 32-key ranges, a workspace of ~270 MB, more than any
    stream can hold from the shapes before it)."""
    _say("workspace growth refused under capture")
    stream = torch.cuda.Stream()
    w = WORKLOADS["prefix_gqa_padded"]
    variant = (1, 4, 4, 32, 1, 32)
    need = fa.fa_fwd_variant_workspace_bytes(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D, w.causal, *variant)
    buf = fa._workspaces.get((gpu_device.index or 0, stream.cuda_stream))
    assert buf is None or buf.numel() < need, (need, buf.numel())
    q, k, v, s = (None if t is None else t.to(gpu_device) for t in make_inputs(w.name))
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device=gpu_device)
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(fa.WorkspaceCaptureError):
        with torch.cuda.graph(graph, stream=stream):
            fa.attention(q, k, v, seqused_k=s, scale=w.scale, out=out, lse=lse, variant=variant)
    torch.cuda.synchronize()


def test_streams_get_their_own_workspace(gpu_device):
    """Split-path calls on two streams at once use two buffers, and both
    results equal the single-stream result."""
    _say("workspace per stream")
    w = WORKLOADS["action_expert_small_m"]
    q, k, v, s = (None if t is None else t.to(gpu_device) for t in make_inputs(w.name))
    o_ref, l_ref = fa.attention(q, k, v, seqused_k=s, scale=w.scale)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            outs.append([fa.attention(q, k, v, seqused_k=s, scale=w.scale) for _ in range(20)])
    torch.cuda.synchronize()
    keys = {(gpu_device.index or 0, st.cuda_stream) for st in streams}
    assert keys <= set(fa._workspaces), "each stream registers a buffer of its own"
    ptrs = {fa._workspaces[key].data_ptr() for key in keys}
    assert len(ptrs) == 2
    for per_stream in outs:
        for o, l in per_stream:
            assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
