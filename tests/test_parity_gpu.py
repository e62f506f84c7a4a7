"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: max|dout| <= 1e-2 and max|dlse| <= 1e-3 (bf16 inputs, fp32
accumulation), exact where the mathematics gives an exact answer (a single
key), and bit-identical where the method must not depend on data it never
reads (padding past seqused_k)."""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

from attention_forward_amd import fa
from attention_forward_amd.workloads import WORKLOADS, make_custom, make_inputs
from tests.gpu_util import assert_parity, run_gpu, run_oracle, to64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_matches_oracle(gpu_device, name):
    w = WORKLOADS[name]
    _say(f"workload {name}")
    q, k, v, s = make_inputs(name)
    got = run_gpu(q, k, v, s, causal=w.causal, scale=w.scale)
    want = run_oracle(q, k, v, s, causal=w.causal, scale=w.scale)
    d_out, d_lse = assert_parity(got, want, name)
    _say(f"  {name}: max|dout|={d_out:.3e} max|dlse|={d_lse:.3e}")


@pytest.mark.parametrize("name", ["prefix_gqa_padded", "action_expert_small_m"])
@pytest.mark.parametrize("poison", [1.0e4, float("inf"), float("nan"), -1.0e4])
def test_padding_is_bit_identical_to_truncated(gpu_device, name, poison):
    """Padded buffer + seqused_k == dense call on the buffer cut to the valid
    length, bit for bit, whatever the padding holds."""
    w = WORKLOADS[name]
    _say(f"padding {name} poison={poison}")
    q, k, v, s = make_inputs(name, pad_value=poison)
    n = w.n_valid
    o1, l1 = run_gpu(q, k, v, s, scale=w.scale)
    o2, l2 = run_gpu(q, k[:, :n].contiguous(), v[:, :n].contiguous(), None, scale=w.scale)
    assert torch.equal(o1, o2), "padding changed out"
    assert torch.equal(l1, l2), "padding changed lse"


CASES = [
    # (B, Sq, Sk, Hq, Hkv, D, causal, n_valid)
    (1, 64, 1, 8, 1, 256, False, None),
    (1, 64, 63, 8, 1, 256, False, None),
    (1, 64, 65, 8, 1, 256, False, None),
    (1, 100, 1025, 8, 1, 256, False, None),
    (1, 37, 2048, 8, 1, 256, False, None),
    (2, 41, 1056, 8, 1, 256, False, [1009, 5]),
    (2, 50, 300, 8, 2, 256, False, [300, 129]),
    (1, 41, 1056, 8, 1, 256, False, [0]),
    (1, 41, 1056, 8, 1, 256, False, [1]),
    (1, 41, 1056, 8, 1, 256, False, [1056]),
    (1, 1, 1, 1, 1, 256, False, None),
    (1, 129, 129, 8, 1, 256, True, None),
    (2, 100, 100, 4, 2, 256, True, None),
    (1, 1, 1, 8, 1, 256, True, None),
    (1, 65, 65, 2, 2, 64, True, None),
    (2, 77, 77, 16, 16, 72, True, None),
    (3, 256, 256, 16, 16, 72, False, [256, 100, 3]),
    (1, 200, 333, 4, 4, 72, False, None),
    (1, 9, 1000, 2, 1, 72, False, None),
    (1, 64, 64, 1, 1, 64, False, None),
    (2, 130, 70, 6, 3, 64, False, [70, 0]),
    (1, 5, 3000, 1, 1, 64, False, None),
    # long contexts (hundreds of split ranges, 32-bit key offsets up to 64 MiB)
    # and a large batch of small problems
    (1, 16, 131072, 8, 1, 256, False, None),
    (1, 7, 65536, 2, 1, 64, False, [60000]),
    (2, 33, 40000, 4, 4, 72, True, None),
    (64, 64, 64, 16, 16, 64, False, None),
    # causal decode into long padded caches (split ranges sized from the buffer)
    (1, 1, 32768, 8, 1, 256, True, [30001]),
    (2, 3, 20000, 8, 1, 256, True, [19999, 5000]),
    # GQA groups larger than a 16-row block: one query position's heads span
    # several row blocks (and split ranges)
    (1, 37, 300, 32, 1, 256, False, None),
    (1, 50, 50, 24, 1, 64, True, None),
    (2, 3, 777, 48, 2, 256, True, [700, 3]),
    (1, 129, 129, 20, 1, 72, False, None),
    (1, 1, 4000, 32, 1, 256, True, [3999]),
    # default plans with two key groups of waves (row-split) and 16-row
    # key-split blocks without a split
    (1, 256, 256, 16, 16, 72, False, None),
    (1, 1024, 1024, 12, 12, 72, False, [1000]),
    (1, 2048, 2048, 5, 5, 64, True, None),
    (1, 512, 512, 8, 1, 256, False, [500]),
    (1, 1024, 1024, 16, 16, 72, True, None),      # causal, two key groups
    (2, 1024, 1024, 16, 16, 64, False, None),     # two rounds of 128-key tiles
    (4, 1024, 1024, 16, 16, 64, False, None),     # 32 rows per wave, 128-row blocks
    (2, 2048, 2048, 16, 16, 72, False, [2048, 1500]),
    (8, 41, 1056, 8, 1, 256, False, [1009, 1, 0, 1056, 500, 41, 1008, 7]),   # batched action expert, no split
    (4, 1024, 1024, 8, 1, 256, False, [968, 1024, 300, 5]),                 # batched prefix: row-split D256
    (2, 768, 768, 8, 1, 256, False, [700, 768]),                            # two rounds D256: key-split ring
    (1, 1024, 1024, 16, 2, 256, False, [1000]),                             # two (batch, kv head) pairs, ring
    (1, 2048, 2048, 8, 1, 256, True, [2000]),                               # causal ring with seqused_k
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[str(c) for c in CASES])
def test_shapes_and_edges(gpu_device, idx):
    case = CASES[idx]
    B, Sq, Sk, Hq, Hkv, D, causal, n_valid = case
    _say(f"case {case}")
    q, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=100 + idx, n_valid=n_valid)
    scale = 1.0 / math.sqrt(D)
    got = run_gpu(q, k, v, s, causal=causal, scale=scale)
    want = run_oracle(q, k, v, s, causal=causal, scale=scale)
    assert_parity(got, want, str(case), strict=False)


@pytest.mark.parametrize("D", [64, 72, 256])
def test_single_key_gives_v0_exactly(gpu_device, D):
    """One attended key: out = v0 bit for bit and lse = scale * q . k0."""
    _say(f"single key D={D}")
    q, k, v, s = make_custom(1, 40, 70, 8, 1, D, seed=5, n_valid=1)
    o, l = run_gpu(q, k, v, s, scale=1.0 / math.sqrt(D))
    assert torch.equal(o, v[:, :1].expand(1, 40, 8, D).contiguous())
    s0 = np.einsum("bihd,bd->bhi", to64(q), to64(k)[:, 0, 0]) * float(np.float32(1.0 / math.sqrt(D)))
    assert np.max(np.abs(to64(l) - s0)) <= 1e-4 * max(1.0, np.abs(s0).max())


@pytest.mark.parametrize("D", [64, 72, 256])
def test_equal_logits_give_mean_and_log_n(gpu_device, D):
    """q = 0: lse = ln n and out = mean of the valid V rows."""
    _say(f"equal logits D={D}")
    q, k, v, s = make_custom(1, 33, 500, 8, 1, D, seed=6, n_valid=477)
    q.zero_()
    o, l = run_gpu(q, k, v, s, scale=0.1)
    assert np.max(np.abs(to64(l) - math.log(477))) <= 1e-5
    mean = to64(v)[0, :477, 0].mean(axis=0)
    assert np.max(np.abs(to64(o)[0] - mean[None, None, :])) <= 2e-3


def test_gqa_equals_replicated_mha_on_gpu(gpu_device):
    _say("gqa vs mha")
    q, k, v, _ = make_custom(2, 70, 130, 8, 2, 256, seed=7)
    o1, l1 = run_gpu(q, k, v)
    o2, l2 = run_gpu(q, k.repeat_interleave(4, dim=2).contiguous(), v.repeat_interleave(4, dim=2).contiguous())
    assert np.max(np.abs(to64(o1) - to64(o2))) <= 1e-2
    assert np.max(np.abs(to64(l1) - to64(l2))) <= 1e-3


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_deterministic_across_calls(gpu_device, name):
    w = WORKLOADS[name]
    _say(f"determinism {name}")
    q, k, v, s = (None if t is None else t.to(gpu_device) for t in make_inputs(name))
    o0, l0 = fa.attention(q, k, v, causal=w.causal, seqused_k=s, scale=w.scale)
    for _ in range(50):
        o, l = fa.attention(q, k, v, causal=w.causal, seqused_k=s, scale=w.scale)
        assert torch.equal(o, o0) and torch.equal(l, l0)


def test_lse_optional_and_preallocated_out(gpu_device):
    _say("lse optional")
    w = WORKLOADS["action_expert_small_m"]
    q, k, v, s = (None if t is None else t.to(gpu_device) for t in make_inputs(w.name))
    o_ref, l_ref = fa.attention(q, k, v, seqused_k=s, scale=w.scale)
    out = torch.full_like(q, 7.0)
    o, l = fa.attention(q, k, v, seqused_k=s, scale=w.scale, out=out, return_lse=False)
    assert l is None and o.data_ptr() == out.data_ptr()
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)


def test_raw_c_entry_point(gpu_device):
    """fa_fwd called with raw device pointers and the current stream."""
    _say("raw fa_fwd")
    w = WORKLOADS["vit_multiview"]
    q, k, v, _ = (None if t is None else t.to(gpu_device) for t in make_inputs(w.name))
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device=gpu_device)
    rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                   w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D, 0, 0, w.scale,
                   torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK
    o2, l2 = fa.attention(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("name", ["vit_multiview", "action_expert_small_m", "causal_gqa_prefill"])
def test_graph_replay_matches_eager(gpu_device, name):
    """fa_fwd captured in a HIP graph: every replay equals the eager call."""
    _say(f"graph {name}")
    w = WORKLOADS[name]
    q, k, v, s = (None if t is None else t.to(gpu_device) for t in make_inputs(name))
    o_eager, l_eager = fa.attention(q, k, v, causal=w.causal, seqused_k=s, scale=w.scale)
    out = torch.empty_like(q)
    lse = torch.empty_like(l_eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fa.attention(q, k, v, causal=w.causal, seqused_k=s, scale=w.scale, out=out, lse=lse)  # warm-up
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):  # the stream whose workspace the warm-up reserved
        fa.attention(q, k, v, causal=w.causal, seqused_k=s, scale=w.scale, out=out, lse=lse)
    for i in range(4):
        out.fill_(3.0)
        lse.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_eager), f"replay {i}: out"
        assert torch.equal(lse, l_eager), f"replay {i}: lse"
