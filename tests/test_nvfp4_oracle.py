"""The NVFP4 quantiser of the oracle against the formats' definitions
(landmark values, round trips, ties, saturation, the scale rule, packing)
and a mutation check: every planted mistake in a copy of it must be caught."""

from __future__ import annotations

import inspect
import json
import math
import os
import types

import numpy as np
import pytest

import oracle.nvfp4 as nv

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_formats.json")))


def pin_e2m1_table(m):
    mags = GOLDEN["e2m1_magnitudes_by_code"]
    for c in range(8):
        assert m.e2m1_value(c) == mags[c]
        assert m.e2m1_value(c | 8) == -mags[c]


def pin_ue4m3_landmarks(m):
    for code, val in GOLDEN["ue4m3_landmarks"].items():
        assert m.ue4m3_value(int(code, 16)) == val, code
    for code in GOLDEN["ue4m3_nan_codes"]:
        assert math.isnan(m.ue4m3_value(int(code, 16)))
    # every finite code is 2^(e-7) (1 + m/8), or m/8 * 2^-6 below the normals
    for c in range(0x7F):
        e, mt = c >> 3, c & 7
        want = mt / 8 * 2.0 ** -6 if e == 0 else (1 + mt / 8) * 2.0 ** (e - 7)
        assert m.ue4m3_value(c) == want


def pin_round_trip(m):
    for c in range(16):
        if c == 8:
            continue  # negative zero encodes as +0 only from +0; checked below
        assert int(m.e2m1_encode(m.e2m1_value(c))) == c, c
    assert int(m.e2m1_encode(-0.1)) == 8 and int(m.e2m1_encode(0.0)) == 0
    for c in range(0x7F):
        assert int(m.ue4m3_encode(m.ue4m3_value(c))) == c, hex(c)


def pin_ties_to_even(m):
    # E2M1 midpoints: the even code wins
    for x, code in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]:
        assert int(m.e2m1_encode(x)) == code, x
        assert int(m.e2m1_encode(-x)) == code | 8, -x
    # just off the midpoints: the nearer value wins
    for x, code in [(0.2500001, 1), (0.7499999, 1), (1.2500001, 3), (4.9999, 6), (5.0001, 7)]:
        assert int(m.e2m1_encode(x)) == code, x
    # UE4M3: 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39)
    assert int(m.ue4m3_encode(1.0625)) == 0x38
    assert int(m.ue4m3_encode(1.1875)) == 0x3A   # between 0x39 and 0x3A
    assert int(m.ue4m3_encode(1.06251)) == 0x39
    assert int(m.ue4m3_encode(2.0 ** -10)) == 0x00   # halfway between 0 and the smallest subnormal


def pin_saturation(m):
    assert int(m.e2m1_encode(7.0)) == 7 and int(m.e2m1_encode(-1e9)) == 15
    assert int(m.ue4m3_encode(500.0)) == 0x7E and int(m.ue4m3_encode(1e30)) == 0x7E
    assert int(m.ue4m3_encode(460.0)) == 0x7E      # nearer 448 than the NaN slot's 480


def pin_scale_rule(m):
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 0] = 6.0
    codes, sf = m.nvfp4_quantize(x)
    assert sf.tolist() == [[0x38]]                 # 6 / 6 = 1.0
    assert codes[0, 0] & 0xF == 7 and (codes[0, 0] >> 4) == 0
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :4] = [-3.0, 1.5, 0.75, -0.25]
    codes, sf = m.nvfp4_quantize(x)
    assert sf.tolist() == [[0x30]]                 # 3 / 6 = 0.5
    # -3/0.5 = -6 -> 0xF, 1.5/0.5 = 3 -> 5, 0.75/0.5 = 1.5 -> 3, -0.25/0.5 = -0.5 -> 0x9
    assert codes[0, 0] == (0xF | (5 << 4)) and codes[0, 1] == (3 | (0x9 << 4))
    # amax 0.7: 0.7/6 = 0.1167 rounds to 0.1171875 (0x1F: exponent field 3, 1.875 * 2^-4);
    # 0.7 / 0.1171875 = 5.97 -> 6
    x = np.full((1, 16), 0.7, dtype=np.float32)
    codes, sf = m.nvfp4_quantize(x)
    assert sf.tolist() == [[0x1F]] and set((codes[0] & 0xF).tolist()) == {7}
    # a block of zeros, and a block too small for any non-zero scale
    for val in (0.0, 1e-5):
        codes, sf = m.nvfp4_quantize(np.full((1, 16), val, dtype=np.float32))
        assert sf.tolist() == [[0]] and not codes.any()
    # blocks are independent: 16 elements each
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0], x[0, 16] = 6.0, 12.0
    codes, sf = m.nvfp4_quantize(x)
    assert sf.tolist() == [[0x38, 0x40]]


def pin_dequant_error(m):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 256)) * rng.uniform(0.01, 20, (64, 1))).astype(np.float32)
    codes, sf = m.nvfp4_quantize(x)
    deq = m.nvfp4_dequantize(codes, sf)
    s = np.repeat(np.vectorize(m.ue4m3_value)(sf), 16, axis=-1)
    # inside the grid the error is at most half a step: 0.25 s below 2, 0.5 s below 4, 1 s above;
    # the block maximum maps near 6 (within the scale's rounding, 1/16) and may saturate
    step = np.where(np.abs(x) / s < 2, 0.5, np.where(np.abs(x) / s < 4, 1.0, 2.0)) * s
    over = np.abs(x) / s > 6
    assert np.all((np.abs(deq - x) <= step / 2 + 1e-12) | over)
    assert np.all(np.abs(deq - x)[over] <= (np.abs(x) - 6 * s)[over] + 1e-12)
    assert np.all(np.max(np.abs(x.reshape(64, 16, 16)), -1) / np.vectorize(m.ue4m3_value)(sf) <= 6 * 17 / 16)


def pin_packing_and_shapes(m):
    x = np.zeros((2, 3, 32), dtype=np.float32)
    x[1, 2, 0], x[1, 2, 1], x[1, 2, 3] = 6.0, 0.5, -1.0
    codes, sf = m.nvfp4_quantize(x)
    assert codes.shape == (2, 3, 16) and sf.shape == (2, 3, 2) and codes.dtype == np.uint8
    assert codes[1, 2, 0] == (7 | (1 << 4)) and codes[1, 2, 1] == (0 | (0xA << 4))
    assert not codes[0].any() and not codes[1, :2].any()
    with pytest.raises(ValueError):
        m.nvfp4_quantize(np.zeros((1, 72), dtype=np.float32))


def pin_attention_composition(m):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 3, 2, 32))
    k = rng.standard_normal((1, 5, 1, 32))
    v = rng.standard_normal((1, 5, 1, 32))
    codes, sf, lse = m.attention_nvfp4_ref(q, k, v, causal=True, scale=0.25)
    out, lse2 = m.attention_ref(q, k, v, causal=True, scale=0.25)
    c2, s2 = m.nvfp4_quantize(out.astype(np.float32))
    assert np.array_equal(codes, c2) and np.array_equal(sf, s2) and np.array_equal(lse, lse2)
    # a single attended key: out = v exactly, so the codes are those of v
    c1, s1, _ = m.attention_nvfp4_ref(q[:, :1], k[:, :1], v[:, :1])
    cv, sv = m.nvfp4_quantize(np.broadcast_to(v[:, :1], (1, 1, 2, 32)).astype(np.float32))
    assert np.array_equal(c1, cv) and np.array_equal(s1, sv)


PINS = [pin_e2m1_table, pin_ue4m3_landmarks, pin_round_trip, pin_ties_to_even, pin_saturation, pin_scale_rule,
        pin_dequant_error, pin_packing_and_shapes, pin_attention_composition]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_nvfp4_pin(pin):
    pin(nv)


MUTATIONS = [
    ("ties away from zero", "((d_hi == d_lo) & (codes[hi] % 2 == 0) & (hi != lo))", "((d_hi == d_lo) & (hi != lo))"),
    ("ties toward zero", "pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0) & (hi != lo))",
     "pick_hi = (d_hi < d_lo)"),
    ("UE4M3 NaN slot used as 480", "_UE4M3_VALS, _UE4M3_CODES = _table(ue4m3_value, range(0x7F))",
     "_UE4M3_VALS, _UE4M3_CODES = _table(lambda c: 480.0 if c == 0x7F else ue4m3_value(c), range(0x80))"),
    ("E2M1 grid without 6", "_E2M1_VALS, _E2M1_CODES = _table(e2m1_value, range(8))",
     "_E2M1_VALS, _E2M1_CODES = _table(e2m1_value, range(7))"),
    ("scale amax/7", "s = amax / np.float32(6.0)", "s = amax / np.float32(7.0)"),
    ("undecoded scale", "qv = blocks / s_dec[..., None]", "qv = blocks / s[..., None]"),
    ("nibbles swapped", "(codes[..., 0::2] | (codes[..., 1::2] << 4))", "(codes[..., 1::2] | (codes[..., 0::2] << 4))"),
    ("sign on x <= 0", "np.where(x < 0, 0x8, 0)", "np.where(x <= 0, 0x8, 0)"),
    ("E2M1 bias 0", "(1.0 + m * 0.5) * 2.0 ** (e - 1)", "(1.0 + m * 0.5) * 2.0 ** e"),
    ("E2M1 no subnormal", "mag = m * 0.5 if e == 0 else", "mag = (1.0 + m * 0.5) * 0.5 if e == 0 else"),
    ("UE4M3 bias 8", "(1.0 + m / 8.0) * 2.0 ** (e - 7)", "(1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    ("UE4M3 subnormal scale", "return m / 8.0 * 2.0 ** -6", "return m / 8.0 * 2.0 ** -7"),
    ("block of 32", "BLOCK = 16", "BLOCK = 32"),
    ("zero scale keeps codes", "codes = np.where(s_dec[..., None] > 0, e2m1_encode(qv), 0)",
     "codes = e2m1_encode(np.nan_to_num(qv, posinf=6.0, neginf=-6.0))"),
    ("amax without abs", "amax = np.max(np.abs(blocks), axis=-1)", "amax = np.max(blocks, axis=-1)"),
]


def _mutant(old, new):
    src = inspect.getsource(nv)
    assert src.count(old) == 1, old
    mod = types.ModuleType("nvfp4_mutant")
    exec(compile(src.replace(old, new), "nvfp4_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(desc, old, new):
    mod = _mutant(old, new)
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:
            return
    pytest.fail(f"no pin catches: {desc}")
