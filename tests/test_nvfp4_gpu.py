"""NVFP4 output (fa_fwd_nvfp4) against the oracle's quantisation of its own
fp64 attention output, through the C ABI.

The kernel quantises its fp32 output, which differs from the oracle's (P is
rounded to bf16 before P V, as in the bf16 path: within the 1e-2 output
tolerance).  So a code or a scale may only differ where the oracle's value
lies within that tolerance of a rounding midpoint, and then only by one step;
everywhere else they are equal.  Every dequantised element is also within
half a grid step (plus the tolerance) of the oracle's output."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from attention_forward_amd import fa
from attention_forward_amd.workloads import WORKLOADS, make_custom, make_inputs
from oracle.nvfp4 import attention_nvfp4_ref, nvfp4_dequantize, ue4m3_value
from tests.gpu_util import LSE_TOL, OUT_TOL, run_oracle, to64

pytestmark = pytest.mark.gpu

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
UE4M3 = np.array([ue4m3_value(c) for c in range(0x7F)])


def _say(msg):
    print(msg, flush=True)


def _run(q, k, v, s, causal, scale):
    dev = "cuda:0"
    codes, sf, lse = fa.attention_nvfp4(q.to(dev), k.to(dev), v.to(dev), causal=causal,
                                        seqused_k=None if s is None else s.to(dev), scale=scale)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sf.cpu().numpy(), lse.cpu()


def _nibbles(packed):
    c = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    c[..., 0::2] = packed & 0xF
    c[..., 1::2] = packed >> 4
    return c


def assert_nvfp4_parity(got, q, k, v, s, causal, scale, what):
    codes_k, sf_k, lse_k = got
    codes_o, sf_o, lse_o = attention_nvfp4_ref(to64(q), to64(k), to64(v), causal=causal,
                                               seqused_k=None if s is None else s.numpy(), scale=scale)
    out64, _ = run_oracle(q, k, v, s, causal=causal, scale=scale)
    D = q.shape[-1]
    x = out64.astype(np.float32).astype(np.float64).reshape(-1, D // 16, 16)   # the oracle's decision inputs
    ck = _nibbles(codes_k).reshape(x.shape).astype(np.int64)
    co = _nibbles(codes_o).reshape(x.shape).astype(np.int64)
    sk, so = sf_k.reshape(x.shape[:2]).astype(np.int64), sf_o.reshape(x.shape[:2]).astype(np.int64)
    tol = OUT_TOL

    # lse as in the bf16 path
    l, lref = to64(lse_k), lse_o
    fin = np.isfinite(lref)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: lse finiteness"
    assert (np.max(np.abs(l[fin] - lref[fin])) if fin.any() else 0.0) <= LSE_TOL, f"{what}: lse"

    # scales: equal, or adjacent where amax/6 is within tol/6 of their midpoint
    amax = np.max(np.abs(x), axis=-1)
    diff = sk != so
    if diff.any():
        lo, hi = np.minimum(sk, so)[diff], np.maximum(sk, so)[diff]
        assert np.all(hi - lo == 1), f"{what}: scale codes differ by more than one step"
        mid = (UE4M3[lo] + UE4M3[hi]) / 2
        assert np.all(np.abs(amax[diff] / 6 - mid) <= tol / 6 + 1e-12), f"{what}: a scale differs away from a midpoint"
    # elements of blocks with equal scales: equal, or adjacent magnitudes near
    # their decision point (sign free only where |x| is within the tolerance)
    s_dec = UE4M3[so]
    for blk in zip(*np.nonzero(~diff & np.any(ck != co, axis=-1))):
        a, b = ck[blk], co[blk]
        xs, sd = x[blk], s_dec[blk]
        for e in np.nonzero(a != b)[0]:
            ma, mb = a[e] & 7, b[e] & 7
            sign_ok = (a[e] & 8) == (b[e] & 8) or abs(xs[e]) <= tol
            near = abs(ma - mb) == 1 and abs(abs(xs[e]) / sd - (E2M1_MAG[ma] + E2M1_MAG[mb]) / 2) <= tol / sd + 1e-12
            zero_sign = ma == mb == 0
            assert sign_ok and (near or zero_sign), f"{what}: code {a[e]:#x} vs {b[e]:#x} at x/s = {xs[e] / sd}"
    # every dequantised element within half a grid step (plus tol) of the oracle's output
    deq = nvfp4_dequantize(codes_k, sf_k).reshape(x.shape)
    sc = UE4M3[sk][..., None]
    rel = np.abs(x) / np.where(sc > 0, sc, 1)
    half_step = np.where(rel < 2, 0.25, np.where(rel < 4, 0.5, 1.0)) * sc
    sat = np.maximum(np.abs(x) - 6 * sc, 0)
    assert np.all(np.abs(deq - x) <= half_step + sat + tol + 1e-12), f"{what}: dequantised values"
    mism = int(np.sum(ck != co))
    _say(f"{what}: {mism} of {ck.size} codes and {int(diff.sum())} of {sk.size} scales at a midpoint")


CASES = {
    # name: (B, Sq, Sk, Hq, Hkv, D, causal, n_valid)
    "d256_single_pass": (1, 640, 300, 8, 1, 256, False, None),
    "d256_split_small_m": (1, 41, 1056, 8, 1, 256, False, [1009]),
    "d256_causal_split": (1, 64, 1024, 8, 1, 256, True, None),   # a chunk of new positions over a cache
    "d256_causal_single_pass": (1, 700, 700, 8, 1, 256, True, None),
    "d64_single_pass": (4, 1024, 1024, 8, 8, 64, False, None),
    "d64_split_gqa": (2, 150, 333, 6, 3, 64, False, [333, 71]),
    "d64_causal": (1, 130, 130, 4, 2, 64, True, None),
    "d64_large_group": (1, 40, 200, 24, 1, 64, True, [180]),  # a position's heads span two row blocks
    "d64_key_groups": (1, 1024, 1024, 12, 12, 64, False, None),  # two key groups of four row waves
    "d64_key_groups_32row": (1, 256, 256, 16, 16, 64, False, None),  # two key groups of two row waves
    "d64_32_rows_per_wave": (4, 1024, 1024, 16, 16, 64, False, None),
    "d256_16row_single_pass": (1, 512, 512, 8, 1, 256, False, [480]),
    "d256_row_split_batched": (4, 1024, 1024, 8, 1, 256, False, [968, 1024, 300, 5]),
    "d256_row_split_64_rows": (2, 768, 768, 8, 1, 256, False, [700, 768]),
}


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
    with torch.cuda.graph(graph):
        fa.attention_nvfp4(q, k, v, seqused_k=s, scale=0.0625, out_fp4=codes, out_sf=sf, lse=lse)
    for i in range(3):
        codes.fill_(0xAB)
        sf.fill_(0xCD)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, c0) and torch.equal(sf, f0) and torch.equal(lse, l0), f"replay {i}"
