"""fa_fwd_static (the entry point that allocates nothing: split-KV partials
in the library's static device scratch) against fa_fwd with a registered
workspace, through the C ABI: bit-identical results on two calls in a row,
the second with a smaller input, and on a single-pass shape."""

from __future__ import annotations

import pytest
import torch

from attention_forward_amd import fa
from attention_forward_amd.workloads import WORKLOADS, make_custom, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _both(q, k, v, s, causal, scale):
    """(out, lse) of fa_fwd_static and of fa_fwd on the same device tensors."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    stream = torch.cuda.current_stream().cuda_stream
    res = []
    for entry in (fa.fa_fwd_static, fa.fa_fwd):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=q.device)
        if entry is fa.fa_fwd:
            fa.reserve_workspace(q.device, fa.fa_fwd_workspace_bytes(B, Sq, Sk, Hq, Hkv, D, causal))
        rc = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Sq, Sk, Hq, Hkv, D,
                   int(causal), 0 if s is None else s.data_ptr(), float(scale), stream)
        assert rc == fa.FA_OK, fa.fa_status_string(rc)
        res.append((out, lse))
    torch.cuda.synchronize()
    return res


def test_static_matches_registered_workspace(gpu_device):
    w = WORKLOADS["action_expert_small_m"]
    plan = fa.fa_fwd_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D, w.causal)
    assert plan[5] > 0, "the small-M shape takes the split path"
    _say(f"static scratch: {w.name} plan {plan}")
    q, k, v, s = (t.to(gpu_device) for t in make_inputs(w.name))
    (o1, l1), (o2, l2) = _both(q, k, v, s, w.causal, w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # a second call right after, with a smaller input (fewer rows and keys,
    # causal): the scratch keeps the last call's contents, which must not matter
    shape = (1, 16, 600, 8, 1, 256)
    plan2 = fa.fa_fwd_plan(*shape, 1)
    assert plan2[5] > 0
    _say(f"static scratch: second call {shape} causal plan {plan2}")
    q2, k2, v2, s2 = (t.to(gpu_device) for t in make_custom(*shape, seed=11, n_valid=[577]))
    (o1, l1), (o2, l2) = _both(q2, k2, v2, s2, True, 0.0625)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert not torch.isnan(o1).any()
    # and back to the first shape
    (o1, l1), (o2, l2) = _both(q, k, v, s, w.causal, w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_static_single_pass_shape(gpu_device):
    """A shape without split uses no scratch and is fa_fwd exactly."""
    w = WORKLOADS["vit_multiview"]
    assert fa.fa_fwd_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D, w.causal)[5] == 0
    _say("static scratch: single-pass shape")
    q, k, v, _ = (None if t is None else t.to(gpu_device) for t in make_inputs(w.name))
    (o1, l1), (o2, l2) = _both(q, k, v, None, w.causal, w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
