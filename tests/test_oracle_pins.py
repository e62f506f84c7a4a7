"""The fp64 oracle against closed forms, invariants and brute force, and a
mutation check: every planted mistake in a copy of the oracle must be caught
by at least one pin."""

from __future__ import annotations

import inspect
import types

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle.reference as ref
from oracle import attention_ref
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(attention_ref)


@pytest.mark.parametrize("pin", pins.VARLEN_PINS, ids=lambda p: p.__name__)
def test_oracle_varlen_pin(pin):
    from oracle import attention_varlen_ref
    pin(attention_varlen_ref)


@settings(max_examples=25, deadline=None)
@given(
    B=st.integers(1, 2),
    Sq=st.integers(1, 4),
    Sk=st.integers(1, 5),
    Hkv=st.integers(1, 2),
    g=st.integers(1, 3),
    D=st.integers(1, 4),
    causal=st.booleans(),
    seq_frac=st.lists(st.floats(0, 1.2), min_size=2, max_size=2),
    use_seq=st.booleans(),
)
def test_oracle_matches_brute_force_random_shapes(B, Sq, Sk, Hkv, g, D, causal, seq_frac, use_seq):
    seq = None
    if use_seq:
        seq = np.array([int(round(f * Sk)) for f in seq_frac[:B]])
    pins.pin_brute_force(attention_ref, cases=[dict(B=B, Sq=Sq, Sk=Sk, Hq=Hkv * g, Hkv=Hkv, D=D,
                                                    causal=causal, seq=None if seq is None else list(seq))])


# Planted mistakes: (description, original text, replacement).  Each is
# applied to the oracle's own source; the mutant must fail some pin.
MUTATIONS = [
    ("GQA head index h % Hkv", "hk = h // group", "hk = h % Hkv"),
    ("no max subtraction", "m = np.max(s, axis=1, keepdims=True)", "m = np.zeros_like(s[:, :1])"),
    ("lse drops the max term", "lse[b, h, rows] = (m + np.log(l))[:, 0]", "lse[b, h, rows] = np.log(l)[:, 0]"),
    ("lse in log2", "lse[b, h, rows] = (m + np.log(l))[:, 0]", "lse[b, h, rows] = (m + np.log2(l))[:, 0]"),
    ("scale dropped", "s = sigma * np.matmul", "s = np.matmul"),
    ("scale divides", "s = sigma * np.matmul(q[b, :, h, :], kb[:, hk, :].T)",
     "s = np.matmul(q[b, :, h, :], kb[:, hk, :].T) / sigma"),
    ("causal j < i", "keep = (j <= i + (nb - Sq))", "keep = (j < i + (nb - Sq))"),
    ("causal mask transposed", "keep = (j <= i + (nb - Sq))", "keep = (j >= i + (nb - Sq))"),
    ("causal aligned top-left", "keep = (j <= i + (nb - Sq))", "keep = (j <= i)"),
    ("causal offset from the buffer length", "keep = (j <= i + (nb - Sq))", "keep = (j <= i + (Sk - Sq))"),
    ("rows without keys computed", "rows = np.any(keep, axis=1)", "rows = np.ones(Sq, dtype=bool)"),
    ("padding read", "kb = k[b, :nb]", "kb = k[b, :]"),
    ("V replaced by K", "out[b, rows, h, :] = np.matmul(w, vb[:, hk, :]) / l",
     "out[b, rows, h, :] = np.matmul(w, kb[:, hk, :]) / l"),
    ("no normalisation", "out[b, rows, h, :] = np.matmul(w, vb[:, hk, :]) / l",
     "out[b, rows, h, :] = np.matmul(w, vb[:, hk, :])"),
    ("exp sign flipped", "w = np.exp(s - m)", "w = np.exp(m - s)"),
    ("exp base 2", "w = np.exp(s - m)", "w = np.exp2(s - m)"),
    ("empty row lse 0", "lse = np.full((B, Hq, Sq), -np.inf, dtype=np.float64)",
     "lse = np.zeros((B, Hq, Sq), dtype=np.float64)"),
    ("default scale 1/D", "scale = 1.0 / math.sqrt(head_dim)", "scale = 1.0 / head_dim"),
    ("scale kept in float64", "return float(np.float32(scale))", "return float(scale)"),
    ("q and k swapped heads", "s = sigma * np.matmul(q[b, :, h, :], kb[:, hk, :].T)",
     "s = sigma * np.matmul(q[b, :, hk, :], kb[:, hk, :].T)"),
    ("wrong batch for K", "kb = k[b, :nb]", "kb = k[0, :nb]"),
    ("seqused ignored", "nb = int(n[b])", "nb = k.shape[1]"),
    ("varlen keys sliced by query offsets", "k[None, k0:k0 + lk], v[None, k0:k0 + lk]",
     "k[None, q0:q0 + lk], v[None, q0:q0 + lk]"),
    ("varlen sequences not cut at max_seqlen", "spans.append((start, min(end - start, max_seqlen)))",
     "spans.append((start, end - start))"),
    ("varlen negative start kept", "start = min(max(int(cu[b]), 0), total)", "start = min(int(cu[b]), total)"),
    ("varlen lse laid out per row", "lse[:, q0:q0 + lq] = l[0]", "lse[:, q0:q0 + lq] = l[0][::-1]"),
    ("varlen scale dropped", "causal=causal,\n                             scale=scale)",
     "causal=causal,\n                             scale=None)"),
]


def _mutant(src_old, src_new):
    src = inspect.getsource(ref)
    assert src.count(src_old) >= 1, f"mutation anchor not found: {src_old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(src_old, src_new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _caught(mod):
    runs = [(pin, mod.attention_ref) for pin in pins.ALL_PINS]
    runs += [(pin, mod.attention_varlen_ref) for pin in pins.VARLEN_PINS]
    for pin, impl in runs:
        try:
            with np.errstate(all="ignore"):
                if pin is pins.pin_varlen_equal_lengths:
                    pin(impl, batched=mod.attention_ref)
                else:
                    pin(impl)
        except Exception:  # AssertionError, or the mutant crashing
            return pin.__name__
    return None


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(desc, old, new):
    assert _caught(_mutant(old, new)) is not None, f"no pin catches: {desc}"


def test_attended_pairs_counts():
    # non-causal: Sq * n per head; causal: S(S+1)/2 per head
    assert ref.attended_pairs(1, 1024, 1024, 8, False, [968]) == 8 * 1024 * 968
    assert ref.attended_pairs(1, 2048, 2048, 8, True, None) == 8 * 2048 * 2049 // 2
    assert ref.attended_pairs(3, 256, 256, 16, False, None) == 3 * 16 * 256 * 256
    assert ref.attended_pairs(1, 41, 1056, 8, False, [1009]) == 8 * 41 * 1009
    assert ref.attended_pairs(2, 4, 6, 1, False, [0, 9]) == 4 * 6
    # causal, bottom-right: query i attends min(i + 1 + n - Sq, n) keys (>= 0)
    assert ref.attended_pairs(1, 41, 1056, 8, True, [1009]) == 8 * sum(969 + i for i in range(41))
    assert ref.attended_pairs(1, 1, 10, 2, True, None) == 2 * 10
    assert ref.attended_pairs(1, 6, 4, 1, True, None) == 0 + 0 + 1 + 2 + 3 + 4
