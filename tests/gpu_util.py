"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare."""

from __future__ import annotations

import numpy as np
import torch

from attention_forward_amd import fa
from oracle import attention_ref

OUT_TOL = 1e-2   # max |out_gpu - out_oracle| for bf16 inputs, fp32 accumulation
LSE_TOL = 1e-3   # max |lse_gpu - lse_oracle|
# Shapes other than the five workloads may attend very few keys, so that
# |out| reaches a few units; the bf16 rounding of out alone is then up to
# half an ulp, 2^-8 |out|.  Those cases get OUT_TOL + 2^-8 |out_oracle| per
# element (the 2^-9 max|v| error of rounding P to bf16 stays inside OUT_TOL
# for |v| <= 5).
REL_OUT = 2.0 ** -8


def to64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def run_gpu(q, k, v, seqused=None, *, causal=False, scale=None, device="cuda:0"):
    """HIP path: inputs are CPU tensors, copied to the device first."""
    dq, dk, dv = (t.to(device) for t in (q, k, v))
    ds = None if seqused is None else seqused.to(device)
    out, lse = fa.attention(dq, dk, dv, causal=causal, seqused_k=ds, scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def run_oracle(q, k, v, seqused=None, *, causal=False, scale=None):
    return attention_ref(to64(q), to64(k), to64(v), causal=causal,
                         seqused_k=None if seqused is None else seqused.numpy(), scale=scale)


def assert_parity(got, want, what="", strict=True):
    out, lse = got
    oref, lref = want
    o = to64(out)
    l = to64(lse)
    assert np.all(np.isfinite(o)), f"{what}: non-finite out"
    err = np.abs(o - oref)
    d_out = np.max(err) if o.size else 0.0
    fin = np.isfinite(lref)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: lse finiteness differs"
    assert np.array_equal(l[~fin], lref[~fin]), f"{what}: lse infinities differ"
    d_lse = np.max(np.abs(l[fin] - lref[fin])) if fin.any() else 0.0
    if strict:
        assert d_out <= OUT_TOL, f"{what}: max|dout| = {d_out}"
    else:
        excess = err - (OUT_TOL + REL_OUT * np.abs(oref))
        assert np.all(excess <= 0), f"{what}: max|dout| = {d_out}, worst excess {excess.max()}"
    assert d_lse <= LSE_TOL, f"{what}: max|dlse| = {d_lse}"
    return d_out, d_lse
