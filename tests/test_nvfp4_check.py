"""The NVFP4 parity check itself, on the CPU: it accepts the oracle's own
quantiser on outputs perturbed within the measured window, and rejects
planted mistakes in a copy of the oracle's quantiser on every NVFP4 case
shape (a 5 % shift of the decision points) and on the exact-tie rows
(ties rounded away from the even code)."""

from __future__ import annotations

import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle.nvfp4 as nv
from attention_forward_amd.workloads import make_custom
from oracle import attention_ref
from tests.nvfp4_check import CASES, check_nvfp4, check_nvfp4_exact, decision_window, planted_rows

# Query positions kept per case: the output values' distribution does not
# depend on how many positions there are, and the oracle stays fast.
MAX_POS = 48


def _mutant(old, new):
    src = inspect.getsource(nv)
    assert src.count(old) == 1, old
    mod = types.ModuleType("nvfp4_mutant")
    exec(compile(src.replace(old, new), "nvfp4_mutant", "exec"), mod.__dict__)
    return mod


MIDPOINT_SHIFT = ("d_lo, d_hi = v - vals[lo], vals[hi] - v", "d_lo, d_hi = v * 1.05 - vals[lo], vals[hi] - v * 1.05")
TIES_AWAY = ("((d_hi == d_lo) & (codes[hi] % 2 == 0) & (hi != lo))", "((d_hi == d_lo) & (hi != lo))")


def _bf16(x):
    return torch.tensor(np.asarray(x), dtype=torch.float32).to(torch.bfloat16).double().numpy()


def _p_rounded_model(q, k, v, n_valid, causal, scale):
    """The output with each probability rounded to bf16 before it weights
    V (the sum l kept unrounded), the largest rounding the bf16 path adds
    beyond the oracle's: a stand-in for a kernel's fp32 output."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        n = Sk if n_valid is None else int(n_valid[b])
        for h in range(Hq):
            s = scale * q[b, :, h] @ k[b, :n, h // g].T
            if causal:
                s = np.where(np.arange(n)[None, :] <= np.arange(Sq)[:, None] + n - Sq, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            out[b, :, h] = np.where(l > 0, (_bf16(p) @ v[b, :n, h // g]) / np.where(l > 0, l, 1), 0)
    return out


def _case_output(name):
    """(oracle output rounded to fp32, the P-rounded model of it in fp32)."""
    B, Sq, Sk, Hq, Hkv, D, causal, nv_ = CASES[name]
    q, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=31 + len(name), n_valid=nv_)
    f64 = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    # the last MAX_POS positions (causal rows there attend the most keys)
    q, k, v = f64(q[:, -MAX_POS:]), f64(k), f64(v)
    sn = None if s is None else s.numpy()
    out, _ = attention_ref(q, k, v, causal=causal, seqused_k=sn, scale=1.0 / math.sqrt(D))
    model = _p_rounded_model(q, k, v, sn, causal, float(np.float32(1.0 / math.sqrt(D))))
    return out.astype(np.float32).astype(np.float64), model.astype(np.float32)


@pytest.fixture(scope="module")
def outputs():
    return {name: _case_output(name) for name in CASES}


def test_check_accepts_oracle_quantiser_on_rounded_model(outputs):
    """The unmutated quantiser on the P-rounded model of each case's output
    passes the element checks, near-ties included; over all cases together
    (the slices here are smaller than the GPU cases) under 1 % of the codes
    and of the scales differ."""
    tot = [0, 0, 0, 0]
    for name, (x, xk) in outputs.items():
        codes, sf = nv.nvfp4_quantize(xk)
        nc, ns = check_nvfp4(codes, sf, x, decision_window(_bf16(xk), x), name, max_frac=None)
        tot = [tot[0] + nc, tot[1] + x.size, tot[2] + ns, tot[3] + x.size // 16]
    print(f"codes {tot[0]} of {tot[1]}, scales {tot[2]} of {tot[3]}")
    assert tot[0] <= 0.01 * tot[1] and tot[2] <= 0.01 * tot[3]


@pytest.mark.parametrize("name", list(CASES))
def test_check_rejects_midpoint_shift(outputs, name):
    x, _ = outputs[name]
    mod = _mutant(*MIDPOINT_SHIFT)
    codes, sf = mod.nvfp4_quantize(x.astype(np.float32))
    with pytest.raises(AssertionError):
        check_nvfp4(codes, sf, x, decision_window(_bf16(x.astype(np.float32)), x), name)


@pytest.mark.parametrize("mutation", [MIDPOINT_SHIFT, TIES_AWAY], ids=["midpoint_shift", "ties_away"])
@pytest.mark.parametrize("D", [64, 256])
def test_exact_check_rejects_mutants(mutation, D):
    x = planted_rows(12, D, seed=D)
    codes, sf = nv.nvfp4_quantize(x.astype(np.float32))
    check_nvfp4_exact(codes, sf, x, "oracle")
    mod = _mutant(*mutation)
    codes_m, sf_m = mod.nvfp4_quantize(x.astype(np.float32))
    with pytest.raises(AssertionError):
        check_nvfp4_exact(codes_m, sf_m, x, "mutant")


def test_planted_rows_are_bf16_ties():
    """The planted rows are bf16 numbers, and each block's amax/6 is on a
    UE4M3 value or exactly halfway between two; each block holds every E2M1
    midpoint times its scale (or is a zero-scale block)."""
    from tests.nvfp4_check import E2M1_MIDS, TIE_BLOCKS, UE4M3
    x = planted_rows(9, 256, seed=3)
    assert np.array_equal(_bf16(x), x)
    blocks = x.reshape(-1, 16)
    for i, blk in enumerate(blocks):
        amax, scale = TIE_BLOCKS[i % len(TIE_BLOCKS)]
        assert np.max(np.abs(blk)) == amax
        s = amax / 6
        on = np.any(UE4M3 == s)
        between = np.any((UE4M3[:-1] + UE4M3[1:]) / 2 == s)
        assert on or between or s > 448, (i, s)
        if scale > 0:
            mags = set(np.abs(blk).tolist())
            assert all(m * scale in mags for m in E2M1_MIDS if m * scale <= amax), i
