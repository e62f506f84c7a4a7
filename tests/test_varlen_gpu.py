"""GPU parity of the packed variable-length forward (fa_fwd_varlen through
the C ABI) against the fp64 oracle's attention_varlen_ref: uneven lengths
(including sequences without queries or without keys), causal within each
sequence, the split-KV path, fp16, offsets that leave the tensors (clamped on
the device), bit-identity with the batched call when all lengths are equal,
and rows outside every sequence left untouched."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from attention_forward_amd import fa
from oracle import attention_varlen_ref, varlen_spans
from tests.gpu_util import LSE_TOL, OUT_TOL, REL_OUT, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(total_q, total_k, Hq, Hkv, D, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(total_q, Hq, D, generator=g).to(dtype)
    k = torch.randn(total_k, Hkv, D, generator=g).to(dtype)
    v = torch.randn(total_k, Hkv, D, generator=g).to(dtype)
    return q, k, v


def _check(q, k, v, cu_q, cu_k, max_q, max_k, causal, what, dtype=torch.bfloat16):
    total_q, Hq, D = q.shape
    dq, dk, dv = (t.to(DEV) for t in (q, k, v))
    out = torch.full(q.shape, 3.0, dtype=dtype, device=DEV)
    lse = torch.full((Hq, total_q), 5.0, dtype=torch.float32, device=DEV)
    fa.attention_varlen(dq, dk, dv, torch.tensor(cu_q, dtype=torch.int32, device=DEV),
                        torch.tensor(cu_k, dtype=torch.int32, device=DEV), max_q, max_k, causal=causal,
                        out=out, lse=lse)
    torch.cuda.synchronize()
    o, l = to64(out.cpu()), to64(lse.cpu())
    oref, lref = attention_varlen_ref(to64(q), to64(k), to64(v), cu_q, cu_k, max_q, max_k, causal=causal)
    covered = np.zeros(total_q, dtype=bool)
    for start, n in varlen_spans(cu_q, total_q, max_q):
        covered[start:start + n] = True
    assert np.all(o[~covered] == 3.0) and np.all(l[:, ~covered] == 5.0), f"{what}: rows outside sequences written"
    o, oref, l, lref = o[covered], oref[covered], l[:, covered], lref[:, covered]
    assert np.all(np.isfinite(o)), f"{what}: non-finite out"
    excess = np.abs(o - oref) - (OUT_TOL + REL_OUT * np.abs(oref))
    assert np.all(excess <= 0), f"{what}: max|dout| = {np.abs(o - oref).max()}"
    fin = np.isfinite(lref)
    assert np.array_equal(np.isfinite(l), fin) and np.array_equal(l[~fin], lref[~fin]), f"{what}: lse -inf rows"
    if fin.any():
        assert np.abs(l[fin] - lref[fin]).max() <= LSE_TOL, f"{what}: max|dlse| = {np.abs(l[fin] - lref[fin]).max()}"
    return out, lse


# (lengths_q, lengths_k, Hq, Hkv, D)
SHAPES = [
    ([37, 0, 150, 64, 5], [37, 20, 150, 0, 90], 4, 4, 64),
    ([256, 256, 256], [256, 256, 256], 16, 16, 72),          # the multi-view ViT batch, packed
    ([130, 17, 300], [200, 17, 64], 8, 1, 256),               # GQA, key-split kernel
    ([41, 20], [1009, 500], 8, 1, 256),                       # few rows, long keys: split-KV path
    ([1, 1, 1, 1], [700, 5, 0, 300], 8, 1, 256),              # decode-like rows
    ([3, 16], [5000, 2500], 8, 1, 256),                       # long keys: ranges sized from the buffer
    ([2, 9], [3000, 4100], 4, 2, 64),
    ([20, 3, 0], [300, 1000, 7], 32, 1, 256),                 # 32 heads per K/V head, a sequence without queries
    ([1024], [1024], 12, 12, 72),                             # two key groups of four row waves
    ([256, 100], [256, 200], 16, 16, 64),                     # two key groups of two row waves
    ([1024, 1024, 1000, 1024], [1024, 1024, 1024, 900], 16, 16, 64),  # 32 rows per wave
    ([1024, 1000, 1024, 1024], [968, 1024, 1024, 1024], 8, 1, 256),   # D256 row-split, 128 rows
    ([768, 700], [768, 600], 8, 1, 256),                      # D256 two rounds: key-split ring
    ([2048], [2048], 8, 1, 256),                              # one sequence of 512 blocks: ring (causal: paired)
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{len(s[0])}seq-D{s[4]}")
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_varlen_matches_oracle(gpu_device, shape, causal, dtype):
    lq, lk, Hq, Hkv, D = shape
    _say(f"varlen {shape} causal={causal} {dtype}")
    cu_q = [0] + list(np.cumsum(lq))
    cu_k = [0] + list(np.cumsum(lk))
    q, k, v = _inputs(sum(lq) + 3, sum(lk) + 2, Hq, Hkv, D, seed=sum(lq) + D, dtype=dtype)  # spare rows at the end
    _check(q, k, v, cu_q, cu_k, max(lq), max(lk), causal, f"varlen {shape} causal={causal}", dtype)


def test_varlen_equal_lengths_match_batched_bitwise(gpu_device):
    # 3 views x 256 tokens, 16 heads, D72: the same kernel variant over the
    # same values, so the packed call reproduces the batched call exactly.
    B, S, H, D = 3, 256, 16, 72
    q, k, v = _inputs(B * S, B * S, H, H, D, seed=5)
    cu = [0, S, 2 * S, 3 * S]
    out, lse = _check(q, k, v, cu, cu, S, S, False, "equal lengths")
    ob, lb = fa.attention(q.view(B, S, H, D).to(DEV), k.view(B, S, H, D).to(DEV), v.view(B, S, H, D).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out.view(B, S, H, D), ob)
    assert torch.equal(lse.view(H, B, S).permute(1, 0, 2), lb)


def test_varlen_offsets_are_clamped(gpu_device):
    # offsets past the end and below zero: spans are clamped into the tensors
    # and cut at max_seqlen (no access outside them), as the oracle defines
    q, k, v = _inputs(120, 150, 4, 2, 64, seed=8)
    _check(q, k, v, [0, 50, 500], [-5, 40, 1000], 64, 100, False, "clamped offsets")
    _check(q, k, v, [0, 50, 500], [-5, 40, 1000], 64, 100, True, "clamped offsets causal")
