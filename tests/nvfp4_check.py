"""Comparison of NVFP4 codes and scales from the HIP path with the oracle's.

Pure CPU logic (numpy), shared by the GPU parity tests and by the CPU tests
that plant mistakes in a copy of the oracle's quantiser and require this
check to reject them.

The kernel quantises its fp32 output x_k; the oracle quantises its fp64
output rounded to fp32, x_o.  The bf16 entry point runs the same plan and
the same arithmetic up to the last rounding and returns bf16(x_k), so per
element

    |x_k - x_o| <= |bf16(x_k) - x_o| + 2^-8 |bf16(x_k)|  =: w

(bf16 keeps 8 significant bits, so rounding moves a value by at most
2^-8 of its magnitude).  A code or scale of the kernel may therefore differ
from the oracle's only by one step, and only where the oracle's value lies
within w of the decision point between the two.  Such near-ties are rare:
at most MAX_MISMATCH_FRAC of the codes and of the scales may differ.

Exact cases (the output equals an input row bit for bit) need no window:
there codes and scales must be identical.
"""

from __future__ import annotations

import numpy as np

from oracle.nvfp4 import nvfp4_dequantize, nvfp4_quantize, ue4m3_value

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
UE4M3 = np.array([ue4m3_value(c) for c in range(0x7F)])
MAX_MISMATCH_FRAC = 0.01
BF16_HALF_ULP = 2.0 ** -8
# fp32 evaluation of amax / 6 adds one rounding of at most 2^-24 relative
FP32_REL = 2.0 ** -23


def nibbles(packed):
    """[..., D/2] packed bytes -> [..., D] codes (element 2i in the low nibble)."""
    packed = np.asarray(packed, dtype=np.uint8)
    c = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    c[..., 0::2] = packed & 0xF
    c[..., 1::2] = packed >> 4
    return c


def decision_window(out_bf16, x_oracle):
    """Per-element bound w on |x_kernel - x_oracle| (see the module docstring)."""
    ob = np.asarray(out_bf16, dtype=np.float64)
    return np.abs(ob - x_oracle) + BF16_HALF_ULP * np.abs(ob)


def check_nvfp4(codes_k, sf_k, x_oracle, window, what="", max_frac=MAX_MISMATCH_FRAC):
    """Raise AssertionError unless the kernel's NVFP4 codes / scales agree
    with the oracle's quantisation of ``x_oracle`` (fp32 values as float64,
    [..., D]) up to near-ties inside ``window`` (same shape), and at most
    ``max_frac`` of them differ (None: no count bound).  Returns (code
    mismatches, scale mismatches)."""
    x = np.asarray(x_oracle, dtype=np.float64)
    D = x.shape[-1]
    codes_o, sf_o = nvfp4_quantize(x.astype(np.float32))
    x = x.reshape(-1, D // 16, 16)
    win = np.asarray(window, dtype=np.float64).reshape(x.shape)
    ck = nibbles(codes_k).reshape(x.shape).astype(np.int64)
    co = nibbles(codes_o).reshape(x.shape).astype(np.int64)
    sk = np.asarray(sf_k).reshape(x.shape[:2]).astype(np.int64)
    so = np.asarray(sf_o).reshape(x.shape[:2]).astype(np.int64)
    assert np.all(sk < 0x7F), f"{what}: a scale byte is the NaN code or has the top bit set"

    # scales: equal, or adjacent where amax/6 is within the block's window
    # (over 6) of the midpoint between them
    amax = np.max(np.abs(x), axis=-1)
    bwin = np.max(win, axis=-1)
    sdiff = sk != so
    n_sdiff = int(sdiff.sum())
    assert max_frac is None or n_sdiff <= max_frac * sk.size, f"{what}: {n_sdiff} of {sk.size} scales differ"
    if n_sdiff:
        lo, hi = np.minimum(sk, so)[sdiff], np.maximum(sk, so)[sdiff]
        assert np.all(hi - lo == 1), f"{what}: scale codes differ by more than one step"
        mid = (UE4M3[lo] + UE4M3[hi]) / 2
        assert np.all(np.abs(amax[sdiff] / 6 - mid) <= bwin[sdiff] / 6 + FP32_REL * mid), \
            f"{what}: a scale differs away from a midpoint"

    # elements of blocks with equal scales: equal, or adjacent magnitudes
    # whose decision point lies within the element's window of x; the sign
    # may differ only where both magnitudes are zero and |x| is within it
    s_dec = UE4M3[so]
    cdiff = (ck != co) & ~sdiff[..., None]
    n_cdiff = int(cdiff.sum())
    assert max_frac is None or n_cdiff <= max_frac * ck.size, f"{what}: {n_cdiff} of {ck.size} codes differ"
    if n_cdiff:
        a, b = ck[cdiff], co[cdiff]
        xs, ws = x[cdiff], win[cdiff]
        sd = np.broadcast_to(s_dec[..., None], x.shape)[cdiff]
        ma, mb = a & 7, b & 7
        same_sign = (a & 8) == (b & 8)
        zero_pair = (ma == 0) & (mb == 0) & (np.abs(xs) <= ws)
        edge = (E2M1_MAG[ma] + E2M1_MAG[mb]) / 2 * sd
        near = (np.abs(ma - mb) == 1) & same_sign & (np.abs(np.abs(xs) - edge) <= ws)
        bad = ~(near | zero_pair)
        if bad.any():
            i = int(np.argmax(bad))
            raise AssertionError(f"{what}: code {a[i]:#x} vs {b[i]:#x} at x = {xs[i]!r}, scale {sd[i]!r}, "
                                 f"window {ws[i]!r}")

    # every dequantised element within half a grid step of its own scale
    # (plus any saturation and the window) of the oracle's value
    deq = nvfp4_dequantize(codes_k, sf_k).reshape(x.shape)
    sc = UE4M3[sk][..., None]
    rel = np.abs(x) / np.where(sc > 0, sc, 1)
    half_step = np.where(rel < 2, 0.25, np.where(rel < 4, 0.5, 1.0)) * sc
    sat = np.maximum(np.abs(x) - 6 * sc, 0)
    # a scale rounded down to zero codes the whole block as zero
    zero_blk = np.broadcast_to((sc == 0), x.shape)
    ok = (np.abs(deq - x) <= half_step + sat + win) | (zero_blk & (deq == 0))
    assert np.all(ok), f"{what}: dequantised values"
    return int(np.sum(ck != co)), n_sdiff


def check_nvfp4_exact(codes_k, sf_k, x_exact, what=""):
    """Exact case: the fp32 output the kernel quantises equals ``x_exact``,
    so codes and scales must be the oracle's bit for bit."""
    codes_o, sf_o = nvfp4_quantize(np.asarray(x_exact, dtype=np.float32))
    ck, co = nibbles(codes_k), nibbles(codes_o)
    if not np.array_equal(np.asarray(sf_k), sf_o):
        i = np.argwhere(np.asarray(sf_k) != sf_o)[0]
        raise AssertionError(f"{what}: scale {int(np.asarray(sf_k)[tuple(i)]):#x} vs {int(sf_o[tuple(i)]):#x} at {i}")
    if not np.array_equal(ck, co):
        i = np.argwhere(ck != co)[0]
        raise AssertionError(f"{what}: code {int(ck[tuple(i)]):#x} vs {int(co[tuple(i)]):#x} at {i}, "
                             f"x = {float(np.asarray(x_exact)[tuple(i)])!r}")


# ------------------------------------------------------------ planted values
# Blocks of 16 whose values sit exactly on E2M1 decision points (the
# midpoints between neighbouring magnitudes) times a block scale, some of
# whose amax / 6 is exactly halfway between two UE4M3 values.  Every value
# is a bf16 number, so a single attended key reproduces it exactly.
E2M1_MIDS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def _block(amax, scale, rng):
    """16 values: amax, then E2M1 midpoints and grid points times ``scale``
    with random signs, shuffled."""
    mids = [m for m in E2M1_MIDS if m * scale <= amax]  # a scale rounded up may put 5s above amax
    vals = [amax] + [m * scale for m in mids] + [g * scale for g in (0.5, 1.0, 1.5, 3.0, 4.0)]
    vals += [m * scale for m in rng.choice(mids, 16 - len(vals))]
    vals = np.array(vals, dtype=np.float64) * rng.choice([-1.0, 1.0], 16)
    return vals[rng.permutation(16)]


# (amax, decoded scale the block gets): amax / 6 exactly on a UE4M3 value, or
# exactly halfway between two (ties go to the even code)
TIE_BLOCKS = [
    (6.0, 1.0),                     # amax/6 = 1.0 (0x38)
    (6.375, 1.0),                   # 1.0625: halfway 0x38 / 0x39 -> 0x38
    (7.125, 1.25),                  # 1.1875: halfway 0x39 / 0x3A -> 0x3A
    (6.0 * 3 * 2.0 ** -10, 2.0 ** -8),   # 1.5 * 2^-9: halfway subnormals 0x01 / 0x02 -> 0x02
    (6.0 * 2.0 ** -10, 0.0),        # halfway 0 / 0x01 -> 0: the whole block codes as zero
    (6.0 * 448.0, 448.0),           # largest finite scale (0x7E)
    (6.0 * 464.0, 448.0),           # past 448: saturates to 0x7E
    (6.0 * 0.1875, 0.1875),         # 0x24 = 1.5 * 2^-3
    (6.0 * 1.125 * 2.0 ** -7, 2.0 ** -7),    # halfway subnormals 0x04 / 0x05 -> 0x04
]


def planted_rows(n_rows, D, seed):
    """[n_rows, D] float64 rows of planted blocks (bf16-exact values)."""
    rng = np.random.default_rng(seed)
    rows = np.empty((n_rows, D), dtype=np.float64)
    for r in range(n_rows):
        for j in range(D // 16):
            amax, scale = TIE_BLOCKS[(r * (D // 16) + j) % len(TIE_BLOCKS)]
            if scale == 0.0:
                blk = np.full(16, amax) * rng.choice([-1.0, 1.0], 16) * rng.choice([0.25, 0.5, 1.0], 16)
                blk[0] = amax
            else:
                blk = _block(amax, scale, rng)
            rows[r, 16 * j:16 * j + 16] = blk
    return rows


# NVFP4 parity cases: (B, Sq, Sk, Hq, Hkv, D, causal, n_valid), covering
# every plan the NVFP4 entry point has (row-split and key-split, split and
# single pass, causal, GQA groups spanning row blocks, two key groups).
# Each has at least 5000 blocks of 16, so that the near-tie mismatches
# (about 0.6 % of codes and scales with the bf16 rounding of P) stay
# clear of the 1 % bound.
CASES = {
    "d256_single_pass": (1, 640, 300, 8, 1, 256, False, None),
    "d256_split_small_m": (1, 41, 1056, 8, 1, 256, False, [1009]),
    "d256_causal_split": (1, 64, 1024, 8, 1, 256, True, None),   # a chunk of new positions over a cache
    "d256_causal_single_pass": (1, 700, 700, 8, 1, 256, True, None),
    "d256_causal_ring": (1, 1984, 1984, 8, 1, 256, True, None),  # 496 blocks: two workgroups per compute unit
    "d64_single_pass": (4, 1024, 1024, 8, 8, 64, False, None),
    "d64_split_gqa": (2, 150, 333, 6, 3, 64, False, [333, 71]),
    "d64_causal": (3, 130, 130, 4, 2, 64, True, None),
    "d64_large_group": (2, 40, 200, 24, 1, 64, True, [180, 200]),  # a position's heads span two row blocks
    "d64_key_groups": (1, 1024, 1024, 12, 12, 64, False, None),  # two key groups of four row waves
    "d64_key_groups_32row": (1, 256, 256, 16, 16, 64, False, None),  # two key groups of two row waves
    "d64_32_rows_per_wave": (4, 1024, 1024, 16, 16, 64, False, None),
    "d256_16row_single_pass": (1, 512, 512, 8, 1, 256, False, [480]),
    "d256_row_split_batched": (4, 1024, 1024, 8, 1, 256, False, [968, 1024, 300, 5]),
    "d256_two_rounds": (2, 768, 768, 8, 1, 256, False, [700, 768]),  # 384 blocks: key-split ring
}
