"""GPU parity of causal attention with the last query aligned to the last
valid key (query i attends keys j <= i + n_b - Sq) against the fp64 oracle:
chunks of new positions attending a cache (Sq < Sk), decode (Sq = 1),
more queries than keys (leading rows attend nothing), and causal with a
device-side seqused_k over a poisoned padded buffer.  Bar: the per-element
bound of tests/gpu_util.py, exact -inf lse and zero out on empty rows, and
bit-identical results whatever the padding holds."""

from __future__ import annotations

import sys

import pytest
import torch

from attention_forward_amd import fa
from attention_forward_amd.workloads import make_custom
from tests.gpu_util import assert_parity, run_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, Sq, Sk, Hq, Hkv, D, n_valid)
CASES = [
    (1, 64, 300, 8, 1, 256, None),          # prefill chunk into a cache, key-split kernel
    (2, 1, 500, 8, 1, 256, [500, 321]),     # decode with seqused_k (split-KV path)
    (1, 41, 1056, 8, 1, 256, [1009]),       # action-expert rows, causal over the cache
    (2, 100, 60, 4, 4, 72, None),           # more queries than keys: 40 empty rows
    (2, 77, 150, 6, 3, 64, [150, 90]),      # GQA, per-batch valid lengths
    (1, 333, 1000, 16, 16, 72, [700]),      # MHA D72, row-split kernel
    (1, 130, 130, 8, 1, 256, [100]),        # Sq == Sk with seqused_k: offset -30
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(q, k, v, s, variant=None):
    out, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=True,
                            seqused_k=None if s is None else s.to(DEV), variant=variant)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(str(x) for x in c[:6]))
def test_bottom_right_causal_matches_oracle(gpu_device, case):
    B, Sq, Sk, Hq, Hkv, D, nv = case
    _say(f"causal {case} plan {fa.fa_fwd_plan(B, Sq, Sk, Hq, Hkv, D, 1)}")
    q, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=21, n_valid=nv)
    got = _run(q, k, v, s)
    want = run_oracle(q, k, v, s, causal=True)
    assert_parity(got, want, f"causal {case}", strict=False)
    # rows with no attended key: out exactly 0, lse -inf
    n = [Sk] * B if nv is None else nv
    for b in range(B):
        empty = max(0, Sq - n[b])
        if empty:
            assert torch.all(got[0][b, :empty] == 0)
            assert torch.all(torch.isneginf(got[1][b, :, :empty]))


@pytest.mark.parametrize("case", [c for c in CASES if c[6] is not None], ids=lambda c: "x".join(str(x) for x in c[:6]))
def test_causal_padding_never_read(gpu_device, case):
    B, Sq, Sk, Hq, Hkv, D, nv = case
    base = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=22, n_valid=nv)
    ref = _run(*base)
    for pad in (float("inf"), float("nan"), -1e4):
        got = _run(*make_custom(B, Sq, Sk, Hq, Hkv, D, seed=22, n_valid=nv, pad_value=pad))
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), pad


VARIANTS = {64: [(1, 4, 1, 64, 2), (1, 4, 1, 64, 3), (2, 4, 4, 64, 1)],
            72: [(1, 4, 1, 64, 2), (1, 4, 1, 64, 3), (2, 2, 1, 64, 2), (2, 4, 4, 64, 1)],
            256: [(1, 4, 1, 32, 2), (2, 4, 1, 32, 4), (2, 4, 4, 32, 1), (2, 4, 4, 32, 2), (1, 4, 4, 32, 2), (2, 2, 2, 32, 1)]}


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[3], CASES[4], CASES[6]],
                         ids=lambda c: "x".join(str(x) for x in c[:6]))
@pytest.mark.parametrize("split", [0, 1, 3])
def test_bottom_right_causal_variants(gpu_device, case, split):
    B, Sq, Sk, Hq, Hkv, D, nv = case
    q, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=23, n_valid=nv)
    want = run_oracle(q, k, v, s, causal=True)
    for var in VARIANTS[D]:
        kps = split * var[3]
        _say(f"causal variant {case} {var} kps={kps}")
        got = _run(q, k, v, s, variant=var + (kps,))
        assert_parity(got, want, f"causal {case} {var} kps={kps}", strict=False)
