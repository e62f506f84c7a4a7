"""Every compiled kernel variant (rows per wave, waves, key tile) with and
without causal masking and key splitting, against the fp64 oracle, through
the fa_fwd_variant entry point."""

from __future__ import annotations

import math
import sys

import pytest
import torch

from attention_forward_amd.workloads import make_custom
from tests.gpu_util import assert_parity, run_oracle

pytestmark = pytest.mark.gpu

# (D, qt, nw, kw, bn, nst): the variants compiled into the library.  kw = 1:
# waves own different rows and share K/V tiles; kw = nw: waves share rows and
# split the keys (each streams its own tiles; nst = 1: whole-tile buffers, 2:
# piecewise refill, 3: piecewise refill through one ring buffer per wave, two
# workgroups per compute unit); kw = 2 < nw: two key
# groups of nw/2 waves, each group sharing its own tiles, merged at the end.
VARIANTS = [(64, 1, 4, 1, 64, 2), (64, 1, 4, 1, 128, 2), (72, 1, 4, 1, 128, 2), (64, 1, 4, 1, 64, 3), (64, 2, 2, 1, 64, 2), (64, 2, 4, 1, 64, 2),
            (72, 1, 4, 1, 64, 2), (72, 1, 4, 1, 64, 3), (72, 1, 4, 1, 64, 4), (72, 2, 2, 1, 64, 2), (72, 2, 2, 1, 64, 3), (72, 2, 4, 1, 64, 2), (256, 1, 4, 1, 32, 2), (256, 1, 4, 1, 32, 4), (256, 1, 4, 1, 64, 2),
            (256, 2, 4, 1, 32, 2), (256, 2, 4, 1, 32, 4), (256, 2, 4, 1, 64, 2),
            (64, 2, 4, 4, 64, 1), (72, 2, 4, 4, 64, 1), (256, 2, 4, 4, 32, 1), (256, 1, 4, 4, 32, 1), (256, 2, 2, 2, 32, 1),
            (256, 2, 4, 4, 32, 2), (256, 2, 4, 4, 32, 3), (256, 1, 4, 4, 32, 2),
            (64, 1, 8, 2, 64, 2), (72, 1, 8, 2, 64, 2), (72, 1, 4, 2, 64, 2), (64, 1, 4, 2, 64, 2)]

SHAPES = {
    # D: (non-causal: B, Sq, Sk, Hq, Hkv, n_valid), (causal: B, S, Hq, Hkv)
    64: ((2, 150, 333, 6, 3, [333, 71]), (2, 130, 6, 3)),
    72: ((2, 150, 333, 4, 4, [333, 71]), (1, 130, 4, 2)),
    256: ((2, 100, 300, 8, 2, [300, 77]), (1, 150, 8, 1)),
}


def _run(q, k, v, s, causal, variant, scale):
    from attention_forward_amd import fa
    dev = "cuda:0"
    out, lse = fa.attention(q.to(dev), k.to(dev), v.to(dev), causal=causal,
                            seqused_k=None if s is None else s.to(dev), scale=scale, variant=variant)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("var", VARIANTS, ids=[str(v) for v in VARIANTS])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("split", [0, 1, 3])
def test_variant_matches_oracle(gpu_device, var, causal, split):
    D, qt, nw, kw, bn, nst = var
    kps = split * bn
    print(f"variant {var} causal={causal} kps={kps}", flush=True)
    if causal:
        B, S, Hq, Hkv = SHAPES[D][1]
        q, k, v, s = make_custom(B, S, S, Hq, Hkv, D, seed=7 + split)
    else:
        B, Sq, Sk, Hq, Hkv, nv = SHAPES[D][0]
        q, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, D, seed=9 + split, n_valid=nv)
    scale = 1.0 / math.sqrt(D)
    got = _run(q, k, v, s, causal, (qt, nw, kw, bn, nst, kps), scale)
    want = run_oracle(q, k, v, s, causal=causal, scale=scale)
    assert_parity(got, want, f"{var} causal={causal} kps={kps}", strict=False)


@pytest.mark.parametrize("var", VARIANTS, ids=[str(v) for v in VARIANTS])
@pytest.mark.parametrize("split", [0, 2])
def test_variant_padding_bit_identical(gpu_device, var, split):
    """Same variant, padded buffer + seqused_k vs buffer cut to the valid
    length: bit-identical for every variant, split or not."""
    D, qt, nw, kw, bn, nst = var
    kps = split * bn
    print(f"padding variant {var} kps={kps}", flush=True)
    q, k, v, s = make_custom(1, 37, 200, 8, 1, D, seed=3, n_valid=131, pad_value=float("nan"))
    a = _run(q, k, v, s, False, (qt, nw, kw, bn, nst, kps), 0.1)
    b = _run(q, k[:, :131].contiguous(), v[:, :131].contiguous(), None, False, (qt, nw, kw, bn, nst, kps), 0.1)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_unknown_variant_is_rejected(gpu_device):
    from attention_forward_amd import fa
    q, k, v, _ = make_custom(1, 8, 8, 1, 1, 64, seed=1)
    with pytest.raises(fa.FAError) as e:
        _run(q, k, v, None, False, (3, 4, 1, 64, 2, 0), 0.125)
    assert e.value.code == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(fa.FAError) as e:
        _run(q, k, v, None, False, (1, 4, 1, 64, 2, 32), 0.125)  # kps not a multiple of bn
    assert e.value.code == fa.FA_ERR_UNSUPPORTED


# The ring buffer scheme (nst 3) changes only where and when the key-split
# kernel stages K and V; every wave computes the same tiles and the merge
# runs in the same order, so its results equal the two-buffer scheme's
# (nst 2) bit for bit.
RING_CASES = [
    (1, 2048, 2048, 8, 1, True, None),          # the causal prefill: paired row blocks
    (1, 2048, 2048, 8, 1, True, [1900]),        # causal with fewer valid keys
    (2, 768, 768, 8, 1, False, [700, 768]),     # two rounds, non-causal
    (1, 200, 1000, 8, 1, False, [1000]),        # one round (unpaired)
]


@pytest.mark.parametrize("case", RING_CASES, ids=[str(c) for c in RING_CASES])
def test_ring_equals_two_buffer_bitwise(gpu_device, case):
    B, Sq, Sk, Hq, Hkv, causal, nv = case
    print(f"ring vs two-buffer {case}", flush=True)
    q, k, v, s = make_custom(B, Sq, Sk, Hq, Hkv, 256, seed=21, n_valid=nv)
    o2, l2 = _run(q, k, v, s, causal, (2, 4, 4, 32, 2, 0), 1.0 / 16)
    o3, l3 = _run(q, k, v, s, causal, (2, 4, 4, 32, 3, 0), 1.0 / 16)
    assert torch.equal(o2, o3) and torch.equal(l2, l3)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("split", [0, 1])
def test_ring_edge_lengths(gpu_device, causal, split):
    """The ring scheme with batch entries of no valid key, one valid key and
    a full buffer (waves without tiles, a wave whose only tile is masked),
    against the oracle."""
    var = (2, 4, 4, 32, 3, 32 * split)
    print(f"ring edge lengths causal={causal} {var}", flush=True)
    q, k, v, s = make_custom(3, 100, 300, 8, 1, 256, seed=31, n_valid=[0, 1, 300], pad_value=float("nan"))
    got = _run(q, k, v, s, causal, var, 1.0 / 16)
    want = run_oracle(q, k, v, s, causal=causal, scale=1.0 / 16)
    assert_parity(got, want, f"ring edge lengths causal={causal} {var}", strict=False)
