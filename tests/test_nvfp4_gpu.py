"""NVFP4 output (fa_fwd_nvfp4) against the oracle's quantisation of its own
fp64 attention output, through the C ABI.

The kernel quantises its fp32 output; the bf16 entry point runs the same
plan and arithmetic and returns that output rounded to bf16, which bounds
per element how far the kernel's value can be from the oracle's (the
window of tests/nvfp4_check.py).  A code or scale may differ from the
oracle's only at a near-tie inside that window, by one step, and at most
1 % of them may differ.  Exact cases -- one attended key with q = 0, so the
output is that key's V row bit for bit, planted on E2M1 decision points and
UE4M3 ties -- must give the oracle's codes and scales bit for bit."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from attention_forward_amd import fa
from attention_forward_amd.workloads import WORKLOADS, make_custom, make_inputs
from oracle.nvfp4 import attention_nvfp4_ref
from tests.gpu_util import LSE_TOL, run_oracle, to64
from tests.nvfp4_check import CASES, check_nvfp4, check_nvfp4_exact, decision_window, planted_rows

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run(q, k, v, s, causal, scale):
    """NVFP4 codes, scales, lse and the bf16 output of the same call shape."""
    dev = "cuda:0"
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    ds = None if s is None else s.to(dev)
    codes, sf, lse = fa.attention_nvfp4(dq, dk, dv, causal=causal, seqused_k=ds, scale=scale)
    out_b, _ = fa.attention(dq, dk, dv, causal=causal, seqused_k=ds, scale=scale)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sf.cpu().numpy(), lse.cpu(), to64(out_b)


def assert_nvfp4_parity(got, q, k, v, s, causal, scale, what):
    codes_k, sf_k, lse_k, out_bf16 = got
    _, _, lse_o = attention_nvfp4_ref(to64(q), to64(k), to64(v), causal=causal,
                                      seqused_k=None if s is None else s.numpy(), scale=scale)
    out64, _ = run_oracle(q, k, v, s, causal=causal, scale=scale)
    x = out64.astype(np.float32).astype(np.float64)   # the oracle's decision inputs

    # lse as in the bf16 path
    l, lref = to64(lse_k), lse_o
    fin = np.isfinite(lref)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: lse finiteness"
    assert (np.max(np.abs(l[fin] - lref[fin])) if fin.any() else 0.0) <= LSE_TOL, f"{what}: lse"

    win = decision_window(out_bf16, x)
    nc, ns = check_nvfp4(codes_k, sf_k, x, win, what)
    _say(f"{what}: {nc} of {x.size} codes and {ns} of {x.size // 16} scales at a near-tie "
         f"(max window {np.max(win):.2e})")


@pytest.mark.parametrize("name", list(CASES))
def test_nvfp4_matches_oracle(gpu_device, name):
    B, Sq, Sk, Hq, Hkv, D, causal, nv = CASES[name]
    _say(f"nvfp4 {name} plan {fa.fa_fwd_plan(B, Sq, Sk, Hq, Hkv, D, causal)}")
    q, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=31 + len(name), n_valid=nv)
    scale = 1.0 / math.sqrt(D)
    assert_nvfp4_parity(_run(q, k, v, s, causal, scale), q, k, v, s, causal, scale, name)


@pytest.mark.parametrize("name", ["prefix_gqa_padded", "action_expert_small_m"])
def test_nvfp4_workloads(gpu_device, name):
    w = WORKLOADS[name]
    _say(f"nvfp4 workload {name}")
    q, k, v, s = make_inputs(name)
    assert_nvfp4_parity(_run(q, k, v, s, w.causal, w.scale), q, k, v, s, w.causal, w.scale, name)


@pytest.mark.parametrize("name", list(CASES))
def test_nvfp4_exact_ties(gpu_device, name):
    """One valid key and q = 0: every score is 0, the single probability is
    exactly 1, and the fp32 output the kernel quantises is V's first row
    exactly.  That row holds values on E2M1 decision points and blocks whose
    amax/6 is on or halfway between UE4M3 values, so the ties-to-even rules
    decide; codes and scales must be the oracle's bit for bit."""
    B, Sq, Sk, Hq, Hkv, D, causal, _ = CASES[name]
    _say(f"nvfp4 exact {name} plan {fa.fa_fwd_plan(B, Sq, Sk, Hq, Hkv, D, causal)}")
    _, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=77, n_valid=[1] * B)
    rows = planted_rows(B * Hkv, D, seed=len(name)).reshape(B, Hkv, D)
    v[:, 0] = torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(v[:, 0].double(), torch.tensor(rows))
    q = torch.zeros(B, Sq, Hq, D, dtype=torch.bfloat16)
    codes_k, sf_k, lse_k, _ = _run(q, k, v, s, causal, 1.0 / math.sqrt(D))
    out64, lse64 = run_oracle(q, k, v, s, causal=causal, scale=1.0 / math.sqrt(D))
    g = Hq // Hkv
    # the oracle's output is V's first row where a row attends key 0, else 0
    want = np.zeros((B, Sq, Hq, D))
    attends = np.isfinite(lse64.transpose(0, 2, 1))    # [B, Sq, Hq]
    for h in range(Hq):
        want[:, :, h] = np.where(attends[:, :, h, None], rows[:, None, h // g], 0.0)
    assert np.array_equal(out64, want), f"{name}: oracle output is not the planted row"
    assert attends.any(), name
    check_nvfp4_exact(codes_k, sf_k, want, name)
    assert np.array_equal(np.isfinite(to64(lse_k)), np.isfinite(lse64)), f"{name}: lse finiteness"


@pytest.mark.parametrize("name", ["d256_split_small_m", "d64_split_gqa", "d256_causal_single_pass"])
def test_nvfp4_lse_equals_bf16_path(gpu_device, name):
    """Same plan and arithmetic as fa_fwd up to the output: lse bit for bit."""
    B, Sq, Sk, Hq, Hkv, D, causal, nv = CASES[name]
    _say(f"nvfp4 lse {name}")
    q, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=5, n_valid=nv)
    dev = "cuda:0"
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    ds = None if s is None else s.to(dev)
    _, _, lse = fa.attention_nvfp4(dq, dk, dv, causal=causal, seqused_k=ds)
    _, lse_b = fa.attention(dq, dk, dv, causal=causal, seqused_k=ds)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse_b)


def test_nvfp4_padding_is_never_read(gpu_device):
    """Poisoned padding past seqused_k: codes and scales bit-identical to the
    same keys without the padding."""
    _say("nvfp4 padding")
    B, Sq, Sk, Hq, Hkv, D, n = 1, 41, 1056, 8, 1, 256, 1009
    q, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=8, n_valid=n, pad_value=float("nan"))
    a = _run(q, k, v, s, False, 0.0625)
    b = _run(q, k[:, :n].contiguous(), v[:, :n].contiguous(), None, False, 0.0625)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_nvfp4_graph_replay(gpu_device):
    """Captured in a HIP graph (split path): every replay equals the eager call."""
    _say("nvfp4 graph")
    q, k, v, s = (t.to("cuda:0") if t is not None else None for t in make_inputs("action_expert_small_m"))
    c0, f0, l0 = fa.attention_nvfp4(q, k, v, seqused_k=s, scale=0.0625)
    codes, sf, lse = torch.empty_like(c0), torch.empty_like(f0), torch.empty_like(l0)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fa.attention_nvfp4(q, k, v, seqused_k=s, scale=0.0625, out_fp4=codes, out_sf=sf, lse=lse)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):  # the stream whose workspace the warm-up reserved
        fa.attention_nvfp4(q, k, v, seqused_k=s, scale=0.0625, out_fp4=codes, out_sf=sf, lse=lse)
    for i in range(3):
        codes.fill_(0xAB)
        sf.fill_(0xCD)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, c0) and torch.equal(sf, f0) and torch.equal(lse, l0), f"replay {i}"
