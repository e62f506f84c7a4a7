"""NVFP4 quantisation of the attention output: plain CPU reference.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from ``attention_forward_amd``.

What the pages fix:

* The attention output is quantised to NVFP4 before the output projection,
  dynamically (from the values themselves): "pi05_thor_decoder_fp4_e2e.md",
  section "Implemented Path".
* Activation quantisation is per 16 elements, with no calibration pass:
  "GROOT N1.7 update: Thor NVFP4 + FA4 performance tier", section "What is
  in the tier".
* The elements are E2M1 and each block of 16 has a UE4M3 scale equal to the
  block's largest magnitude over the grid's largest value (amax/7 for the
  0..7 grid): "pi05_thor_decoder_fp4_e2e.md", section "E0M3 Uniform-INT4
  Decoder Weights".  UE4M3 bytes 0x7F and 0xFF are NaN: same page, section
  "Encoder Attention QKV NVFP4 + Scale-Factor Zero-Init".

The two formats, by their standard bit-level definitions:

* E2M1 (4 bits): sign, 2-bit exponent with bias 1, 1-bit mantissa; exponent
  0 is subnormal.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* UE4M3 (one byte, sign bit ignored): 4-bit exponent with bias 7, 3-bit
  mantissa; exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa
  7 is NaN; the largest finite value is 448.

Readings taken where the pages are silent:

* A block is 16 consecutive head-dim elements of one (token, head) row, so
  the head dim must be a multiple of 16.
* The values quantised are the attention output in float32 (the precision
  the kernels hold it in before any rounding).
* Scale: amax / 6 evaluated in float32 (E2M1's largest value is 6, as 7 is
  the 0..7 grid's), rounded to the nearest UE4M3 value with ties to the
  even code; values above 448 become 448.
* Element: the float32 quotient x / decoded scale rounded to the nearest E2M1
  magnitude with ties to the even code; above 6 it becomes 6; the sign bit
  is set when x < 0.  A block whose scale rounds to zero gets zero codes.
* Packing: element 2i in the low nibble of byte i, element 2i+1 in the high
  nibble, (token, head) rows as in the bf16 output; scales row-major,
  D/16 bytes per (token, head).  No per-tensor scale (none is mentioned).
"""

from __future__ import annotations

import numpy as np

from oracle.reference import attention_ref

__all__ = ["e2m1_value", "ue4m3_value", "e2m1_encode", "ue4m3_encode", "nvfp4_quantize", "nvfp4_dequantize",
           "attention_nvfp4_ref", "BLOCK"]

BLOCK = 16


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code."""
    sign = -1.0 if code & 0x8 else 1.0
    e, m = (code >> 1) & 0x3, code & 0x1
    mag = m * 0.5 if e == 0 else (1.0 + m * 0.5) * 2.0 ** (e - 1)
    return sign * mag


def ue4m3_value(code: int) -> float:
    """Value of a UE4M3 scale byte (the top bit is not part of the value)."""
    c = code & 0x7F
    if c == 0x7F:
        return float("nan")
    e, m = c >> 3, c & 0x7
    if e == 0:
        return m / 8.0 * 2.0 ** -6
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _table(values_of, codes):
    """(sorted finite non-negative values, their codes)."""
    pairs = sorted((values_of(c), c) for c in codes)
    return np.array([v for v, _ in pairs], dtype=np.float64), np.array([c for _, c in pairs], dtype=np.int64)


_E2M1_VALS, _E2M1_CODES = _table(e2m1_value, range(8))
_UE4M3_VALS, _UE4M3_CODES = _table(ue4m3_value, range(0x7F))


def _nearest(v, vals, codes):
    """Code of the value in ``vals`` nearest to each v >= 0; a tie goes to
    the even code; beyond the largest value, the largest code."""
    v = np.asarray(v, dtype=np.float64)
    lo = np.clip(np.searchsorted(vals, v, side="right") - 1, 0, len(vals) - 1)
    hi = np.minimum(lo + 1, len(vals) - 1)
    d_lo, d_hi = v - vals[lo], vals[hi] - v
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0) & (hi != lo))
    out = np.where(pick_hi, codes[hi], codes[lo])
    return np.where(v >= vals[-1], codes[-1], out)


def e2m1_encode(x):
    """E2M1 codes of float values (nearest, ties to even, saturating)."""
    x = np.asarray(x, dtype=np.float64)
    mag = _nearest(np.abs(x), _E2M1_VALS, _E2M1_CODES)
    return (mag | np.where(x < 0, 0x8, 0)).astype(np.uint8)


def ue4m3_encode(v):
    """UE4M3 codes of values >= 0 (nearest, ties to even, saturating)."""
    return _nearest(v, _UE4M3_VALS, _UE4M3_CODES).astype(np.uint8)


def nvfp4_quantize(x):
    """x [..., D] (taken as float32) -> (codes uint8 [..., D/2], scales uint8 [..., D/16])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    if D % BLOCK != 0:
        raise ValueError("the head dim must be a multiple of 16")
    blocks = x.reshape(x.shape[:-1] + (D // BLOCK, BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)                        # exact in float32
    s = amax / np.float32(6.0)                                     # float32 division
    sf = ue4m3_encode(s.astype(np.float64))
    s_dec = np.vectorize(ue4m3_value, otypes=[np.float64])(sf).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qv = blocks / s_dec[..., None]                             # float32 division
    codes = np.where(s_dec[..., None] > 0, e2m1_encode(qv), 0).astype(np.uint8)
    codes = codes.reshape(x.shape[:-1] + (D,))
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, sf


def nvfp4_dequantize(packed, sf):
    """Values (float64) of packed NVFP4 codes with their block scales."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    vals = np.vectorize(e2m1_value, otypes=[np.float64])(codes)
    scales = np.vectorize(ue4m3_value, otypes=[np.float64])(np.asarray(sf, dtype=np.uint8))
    return vals * np.repeat(scales, BLOCK, axis=-1)


def attention_nvfp4_ref(q, k, v, *, causal=False, seqused_k=None, scale=None):
    """(codes [B, Sq, Hq, D/2], scales [B, Sq, Hq, D/16], lse [B, Hq, Sq]):
    attention_ref's output rounded to float32, then nvfp4_quantize."""
    out, lse = attention_ref(q, k, v, causal=causal, seqused_k=seqused_k, scale=scale)
    codes, sf = nvfp4_quantize(out.astype(np.float32))
    return codes, sf, lse
