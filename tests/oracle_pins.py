"""Pins that tie the fp64 oracle to facts other than itself.

Each pin takes an attention implementation ``impl(q, k, v, causal=,
seqused_k=, scale=) -> (out, lse)`` (numpy in, numpy out) and raises
AssertionError when the implementation disagrees with:

* closed forms (single key, equal logits, two keys),
* a pure-Python brute force in 50-digit mpmath on tiny inputs,
* invariants the definition implies (padding is never read, key
  permutation, shift of all keys, linearity in V, GQA equals MHA with
  replicated K/V, causal row i equals non-causal attention over keys
  0..i + n_b - Sq),
* numerical stability at logits of size 1e4 (against mpmath).

VARLEN_PINS do the same for the packed variable-length form
``vimpl(q, k, v, cu_q, cu_k, max_q, max_k, causal=, scale=)``: equal
lengths reduce to the batched form, uneven lengths agree with the brute
force per sequence, sequences are independent, and the span rule is pinned
by closed form.

The same pins run against the oracle and against mutants of it with a
planted mistake (tests/test_oracle_pins.py), which shows that each kind of
plausible mistake is caught by at least one pin.
"""

from __future__ import annotations

import math

import mpmath
import numpy as np

mpmath.mp.dps = 50


def _rng(seed):
    return np.random.default_rng(seed)


def _randn(rng, *shape):
    # Values with few mantissa bits, as bf16 inputs have.
    return np.round(rng.standard_normal(shape) * 64.0) / 64.0


def brute_force(q, k, v, *, causal=False, seqused_k=None, scale=None):
    """Attention by nested loops in 50-digit mpmath (tiny inputs only).

    Written without numpy arithmetic: every dot product, exponential and sum
    is an mpmath operation, so it shares no rounding or library routine with
    the oracle.
    """
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    sigma = mpmath.mpf(float(np.float32(1.0 / math.sqrt(D) if scale is None else scale)))
    g = Hq // Hkv
    out = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        nb = Sk if seqused_k is None else max(0, min(int(seqused_k[b]), Sk))
        for h in range(Hq):
            hk = h // g
            for i in range(Sq):
                # causal: the last query lines up with the last valid key
                keys = [j for j in range(nb) if (not causal or j - i <= nb - Sq)]
                if not keys:
                    lse[b, h, i] = -math.inf
                    continue
                s = {j: sigma * mpmath.fsum(mpmath.mpf(float(q[b, i, h, d])) * mpmath.mpf(float(k[b, j, hk, d]))
                                            for d in range(D)) for j in keys}
                total = mpmath.fsum(mpmath.exp(s[j]) for j in keys)
                lse[b, h, i] = float(mpmath.log(total))
                for d in range(D):
                    num = mpmath.fsum(mpmath.exp(s[j]) * mpmath.mpf(float(v[b, j, hk, d])) for j in keys)
                    out[b, i, h, d] = float(num / total)
    return out, lse


def _close(a, b, atol, rtol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: non-finite pattern differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: infinities differ"
    err = np.abs(a[fin] - b[fin])
    lim = atol + rtol * np.abs(b[fin])
    assert np.all(err <= lim), f"{what}: max err {err.max() if err.size else 0}"


# ---------------------------------------------------------------- closed forms

def pin_single_key(impl):
    """One key: out = v0 exactly, lse = sigma * q . k0."""
    rng = _rng(11)
    for (Hq, Hkv, D) in [(1, 1, 8), (4, 2, 16), (3, 1, 5)]:
        q = _randn(rng, 2, 3, Hq, D)
        k = _randn(rng, 2, 1, Hkv, D)
        v = _randn(rng, 2, 1, Hkv, D)
        out, lse = impl(q, k, v, scale=0.25)
        g = Hq // Hkv
        for b in range(2):
            for i in range(3):
                for h in range(Hq):
                    assert np.array_equal(out[b, i, h], v[b, 0, h // g]), "single key: out != v0"
                    s0 = 0.25 * math.fsum(q[b, i, h, d] * k[b, 0, h // g, d] for d in range(D))
                    assert abs(lse[b, h, i] - s0) <= 1e-12 * max(1.0, abs(s0)), "single key: lse != s0"


def pin_equal_logits(impl):
    """q = 0: every logit is 0, so lse = ln n and out = mean of the valid v."""
    rng = _rng(12)
    B, S, Sk, H, D = 2, 5, 9, 2, 6
    q = np.zeros((B, S, H, D))
    k = _randn(rng, B, Sk, H, D)
    v = _randn(rng, B, Sk, H, D)
    seq = np.array([9, 4])
    out, lse = impl(q, k, v, seqused_k=seq)
    for b in range(B):
        n = int(seq[b])
        for h in range(H):
            for i in range(S):
                assert abs(lse[b, h, i] - math.log(n)) <= 1e-13, "equal logits: lse != ln n"
                for d in range(D):
                    mean = math.fsum(v[b, j, h, d] for j in range(n)) / n
                    assert abs(out[b, i, h, d] - mean) <= 1e-13, "equal logits: out != mean(v)"
    # Equal keys instead of zero queries: lse = ln n + sigma * q . k
    kk = np.broadcast_to(_randn(rng, 1, 1, H, D), (B, Sk, H, D)).copy()
    q2 = _randn(rng, B, S, H, D)
    out2, lse2 = impl(q2, kk, v, scale=0.5)
    for b in range(B):
        for h in range(H):
            for i in range(S):
                s = 0.5 * math.fsum(q2[b, i, h, d] * kk[0, 0, h, d] for d in range(D))
                assert abs(lse2[b, h, i] - (math.log(Sk) + s)) <= 1e-12 * max(1, abs(s)), "equal keys: lse"


def pin_two_keys(impl):
    """Two keys: lse = log(e^s0 + e^s1); out = sig(s0-s1) v0 + sig(s1-s0) v1."""
    rng = _rng(13)
    D = 4
    q = _randn(rng, 1, 2, 1, D) * 3
    k = _randn(rng, 1, 2, 1, D)
    v = _randn(rng, 1, 2, 1, D)
    out, lse = impl(q, k, v, scale=1.0)
    for i in range(2):
        s0 = mpmath.fsum(mpmath.mpf(q[0, i, 0, d]) * mpmath.mpf(k[0, 0, 0, d]) for d in range(D))
        s1 = mpmath.fsum(mpmath.mpf(q[0, i, 0, d]) * mpmath.mpf(k[0, 1, 0, d]) for d in range(D))
        assert abs(lse[0, 0, i] - float(mpmath.log(mpmath.exp(s0) + mpmath.exp(s1)))) <= 1e-13
        w0 = 1 / (1 + mpmath.exp(s1 - s0))
        w1 = 1 / (1 + mpmath.exp(s0 - s1))
        for d in range(D):
            want = float(w0 * mpmath.mpf(v[0, 0, 0, d]) + w1 * mpmath.mpf(v[0, 1, 0, d]))
            assert abs(out[0, i, 0, d] - want) <= 1e-13, "two keys: out"


def pin_empty(impl):
    """No attended key (seqused_k = 0): out = 0 and lse = -inf."""
    rng = _rng(14)
    q = _randn(rng, 2, 3, 2, 4)
    k = _randn(rng, 2, 5, 1, 4)
    v = _randn(rng, 2, 5, 1, 4)
    out, lse = impl(q, k, v, seqused_k=np.array([0, 2]))
    assert np.all(out[0] == 0.0), "empty: out != 0"
    assert np.all(np.isneginf(lse[0])), "empty: lse != -inf"
    assert np.all(np.isfinite(lse[1])), "non-empty row must be finite"


# ------------------------------------------------------------------ brute force

def pin_brute_force(impl, cases=None):
    """Agreement with the mpmath brute force on tiny shapes, 1e-12."""
    rng = _rng(15)
    if cases is None:
        cases = [
            dict(B=1, Sq=3, Sk=4, Hq=1, Hkv=1, D=3, causal=False, seq=None),
            dict(B=2, Sq=4, Sk=4, Hq=4, Hkv=2, D=5, causal=True, seq=None),
            dict(B=2, Sq=3, Sk=6, Hq=2, Hkv=1, D=4, causal=False, seq=[6, 2]),
            dict(B=1, Sq=5, Sk=5, Hq=3, Hkv=3, D=2, causal=True, seq=None),
            dict(B=1, Sq=2, Sk=5, Hq=2, Hkv=1, D=3, causal=True, seq=None),
            dict(B=2, Sq=4, Sk=6, Hq=2, Hkv=2, D=2, causal=True, seq=[5, 2]),
            dict(B=1, Sq=5, Sk=3, Hq=1, Hkv=1, D=3, causal=True, seq=None),
        ]
    for c in cases:
        q = _randn(rng, c["B"], c["Sq"], c["Hq"], c["D"])
        k = _randn(rng, c["B"], c["Sk"], c["Hkv"], c["D"])
        v = _randn(rng, c["B"], c["Sk"], c["Hkv"], c["D"])
        seq = None if c["seq"] is None else np.array(c["seq"])
        if seq is not None:
            for b in range(c["B"]):
                k[b, seq[b]:] = 1e4
                v[b, seq[b]:] = 1e4
        got = impl(q, k, v, causal=c["causal"], seqused_k=seq, scale=0.7)
        want = brute_force(q, k, v, causal=c["causal"], seqused_k=seq, scale=0.7)
        _close(got[0], want[0], 1e-12, what=f"brute out {c}")
        _close(got[1], want[1], 1e-12, what=f"brute lse {c}")


# ------------------------------------------------------------------- invariants

def pin_padding_never_read(impl):
    """Garbage (1e4, +inf, nan) past seqused_k changes nothing: the result is
    exactly that of the buffer truncated to the valid length."""
    rng = _rng(16)
    B, Sq, Sk, Hq, Hkv, D = 2, 4, 9, 4, 1, 6
    q = _randn(rng, B, Sq, Hq, D)
    k = _randn(rng, B, Sk, Hkv, D)
    v = _randn(rng, B, Sk, Hkv, D)
    seq = np.array([7, 3])
    for poison in (1e4, np.inf, np.nan, -1e4):
        kp, vp = k.copy(), v.copy()
        for b in range(B):
            kp[b, seq[b]:] = poison
            vp[b, seq[b]:] = poison
        out, lse = impl(q, kp, vp, seqused_k=seq)
        for b in range(B):
            n = int(seq[b])
            ob, lb = impl(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n])
            assert np.array_equal(out[b:b + 1], ob), f"padding {poison} leaked into out"
            assert np.array_equal(lse[b:b + 1], lb), f"padding {poison} leaked into lse"


def pin_key_permutation(impl):
    """Non-causal: permuting K and V rows together leaves the result unchanged."""
    rng = _rng(17)
    q = _randn(rng, 1, 5, 2, 7)
    k = _randn(rng, 1, 11, 2, 7)
    v = _randn(rng, 1, 11, 2, 7)
    p = rng.permutation(11)
    o1, l1 = impl(q, k, v)
    o2, l2 = impl(q, k[:, p], v[:, p])
    _close(o2, o1, 1e-13, what="permutation out")
    _close(l2, l1, 1e-13, what="permutation lse")


def pin_key_shift(impl):
    """k_j -> k_j + u for all j: out unchanged, lse_i + sigma * q_i . u."""
    rng = _rng(18)
    q = _randn(rng, 1, 4, 2, 5)
    k = _randn(rng, 1, 6, 2, 5)
    v = _randn(rng, 1, 6, 2, 5)
    u = _randn(rng, 5)
    o1, l1 = impl(q, k, v, scale=0.5)
    o2, l2 = impl(q, k + u, v, scale=0.5)
    _close(o2, o1, 1e-12, what="shift out")
    shift = 0.5 * np.einsum("bihd,d->bhi", q, u)
    _close(l2, l1 + shift, 1e-12, what="shift lse")


def pin_v_linearity(impl):
    """out is linear in V; lse does not depend on V."""
    rng = _rng(19)
    q = _randn(rng, 1, 4, 2, 5)
    k = _randn(rng, 1, 6, 1, 5)
    v1 = _randn(rng, 1, 6, 1, 5)
    v2 = _randn(rng, 1, 6, 1, 5)
    o1, l1 = impl(q, k, v1)
    o2, l2 = impl(q, k, v2)
    o3, l3 = impl(q, k, 2.0 * v1 - 3.0 * v2)
    _close(o3, 2.0 * o1 - 3.0 * o2, 1e-12, what="linearity")
    assert np.array_equal(l1, l2) and np.array_equal(l1, l3), "lse depends on V"


def pin_gqa_is_replicated_mha(impl):
    """GQA(Hq, Hkv) equals MHA(Hq, Hq) with each K/V head repeated Hq/Hkv
    times in place (heads h = hk*g .. hk*g+g-1 read K/V head hk)."""
    rng = _rng(20)
    for (Hq, Hkv) in [(4, 2), (8, 1), (6, 3)]:
        g = Hq // Hkv
        q = _randn(rng, 2, 3, Hq, 4)
        k = _randn(rng, 2, 5, Hkv, 4)
        v = _randn(rng, 2, 5, Hkv, 4)
        o1, l1 = impl(q, k, v)
        o2, l2 = impl(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2))
        _close(o1, o2, 1e-13, what=f"gqa out {Hq}/{Hkv}")
        _close(l1, l2, 1e-13, what=f"gqa lse {Hq}/{Hkv}")


def pin_causal_prefix(impl):
    """Causal row 0 equals v0; causal row i equals non-causal attention over
    keys 0..i."""
    rng = _rng(21)
    S = 6
    q = _randn(rng, 1, S, 2, 4)
    k = _randn(rng, 1, S, 1, 4)
    v = _randn(rng, 1, S, 1, 4)
    out, lse = impl(q, k, v, causal=True)
    for h in range(2):
        assert np.array_equal(out[0, 0, h], v[0, 0, 0]), "causal row 0 != v0"
    for i in range(S):
        oi, li = impl(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1])
        _close(out[:, i:i + 1], oi, 1e-13, what=f"causal row {i} out")
        _close(lse[:, :, i:i + 1], li, 1e-13, what=f"causal row {i} lse")


def pin_causal_bottom_right(impl):
    """Causal with Sq != n_b (n_b valid keys): query i attends keys
    0..i + n_b - Sq.  Row i equals non-causal attention over that key
    prefix; a single query (decode) attends every valid key; with more
    queries than keys the first Sq - n_b rows attend nothing (out 0,
    lse -inf); padding past seqused_k is never read."""
    rng = _rng(24)
    D = 4
    for Sq, Sk, seq in ((3, 7, None), (1, 6, None), (6, 4, None), (4, 9, [6]), (5, 9, [3])):
        q = _randn(rng, 1, Sq, 2, D)
        k = _randn(rng, 1, Sk, 1, D)
        v = _randn(rng, 1, Sk, 1, D)
        n = Sk if seq is None else seq[0]
        if seq is not None:
            k[0, n:] = np.nan
            v[0, n:] = np.nan
        sq = None if seq is None else np.array(seq)
        out, lse = impl(q, k, v, causal=True, seqused_k=sq)
        for i in range(Sq):
            last = i + n - Sq  # last attended key
            if last < 0:
                assert np.all(out[0, i] == 0.0) and np.all(np.isneginf(lse[0, :, i])), f"empty row {i}"
                continue
            oi, li = impl(q[:, i:i + 1], k[:, :last + 1], v[:, :last + 1])
            _close(out[:, i:i + 1], oi, 1e-13, what=f"bottom-right row {i} out ({Sq},{Sk},{seq})")
            _close(lse[:, :, i:i + 1], li, 1e-13, what=f"bottom-right row {i} lse ({Sq},{Sk},{seq})")


def pin_scale(impl):
    """The logits are sigma * q.k with sigma = float32(scale); the default
    scale is 1/sqrt(D)."""
    rng = _rng(22)
    q = _randn(rng, 1, 3, 1, 16)
    k = _randn(rng, 1, 5, 1, 16)
    v = _randn(rng, 1, 5, 1, 16)
    o1, l1 = impl(q, k, v)
    o2, l2 = impl(q, k, v, scale=0.25)  # 1/sqrt(16), exact
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "default scale != 1/sqrt(D)"
    o3, l3 = impl(q * 0.25, k, v, scale=1.0)  # power-of-two scale is exact
    _close(o3, o2, 1e-14, what="scale multiplies logits (out)")
    _close(l3, l2, 1e-14, what="scale multiplies logits (lse)")
    o4, l4 = impl(q, k, v, scale=0.1)
    o5, l5 = impl(q, k, v, scale=float(np.float32(0.1)))
    assert np.array_equal(o4, o5) and np.array_equal(l4, l5), "scale is not rounded to float32"


def pin_large_logits(impl):
    """Logits of magnitude ~1e4 (exp overflows without the max shift):
    agreement with 50-digit mpmath."""
    rng = _rng(23)
    q = _randn(rng, 1, 3, 1, 4) * 100
    k = _randn(rng, 1, 5, 1, 4) * 100
    v = _randn(rng, 1, 5, 1, 4)
    out, lse = impl(q, k, v, scale=1.0)
    want = brute_force(q, k, v, scale=1.0)
    assert np.all(np.abs(lse) > 100), "test needs large logits"
    _close(out, want[0], 1e-12, what="large logits out")
    _close(lse, want[1], 0.0, rtol=1e-14, what="large logits lse")


ALL_PINS = [
    pin_single_key,
    pin_equal_logits,
    pin_two_keys,
    pin_empty,
    pin_brute_force,
    pin_padding_never_read,
    pin_key_permutation,
    pin_key_shift,
    pin_v_linearity,
    pin_gqa_is_replicated_mha,
    pin_causal_prefix,
    pin_causal_bottom_right,
    pin_scale,
    pin_large_logits,
]


# ------------------------------------------------------------------- varlen

def _pack(rng, lens, H, D):
    return _randn(rng, int(sum(lens)), H, D)


def pin_varlen_equal_lengths(vimpl, batched=None):
    """B sequences of equal lengths packed back to back: the batched
    attention of the same tensors, causal or not."""
    from oracle import attention_ref as batched_ref  # pinned on its own above
    batched = batched or batched_ref
    rng = _rng(30)
    B, Lq, Lk, Hq, Hkv, D = 3, 4, 6, 4, 2, 5
    for causal in (False, True):
        q = _randn(rng, B, Lq, Hq, D)
        k = _randn(rng, B, Lk, Hkv, D)
        v = _randn(rng, B, Lk, Hkv, D)
        cu_q = np.arange(B + 1) * Lq
        cu_k = np.arange(B + 1) * Lk
        out, lse = vimpl(q.reshape(B * Lq, Hq, D), k.reshape(B * Lk, Hkv, D), v.reshape(B * Lk, Hkv, D),
                         cu_q, cu_k, Lq, Lk, causal=causal, scale=0.6)
        ob, lb = batched(q, k, v, causal=causal, scale=0.6)
        _close(out, ob.reshape(B * Lq, Hq, D), 1e-14, what=f"varlen equal lengths out causal={causal}")
        _close(lse, lb.transpose(1, 0, 2).reshape(Hq, B * Lq), 1e-14, what=f"varlen equal lengths lse {causal}")


def pin_varlen_brute_force(vimpl):
    """Uneven lengths, including a sequence without queries and one without
    keys: each sequence agrees with the mpmath brute force; rows of a
    sequence without keys are out 0, lse -inf."""
    rng = _rng(31)
    lq, lk = [3, 0, 2, 4], [5, 3, 0, 2]
    Hq, Hkv, D = 2, 1, 3
    q, k, v = _pack(rng, lq, Hq, D), _pack(rng, lk, Hkv, D), _pack(rng, lk, Hkv, D)
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    for causal in (False, True):
        out, lse = vimpl(q, k, v, cu_q, cu_k, max(lq), max(lk), causal=causal, scale=0.9)
        for b in range(len(lq)):
            qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
            if lq[b] == 0:
                continue
            if lk[b] == 0:
                assert np.all(out[qs] == 0) and np.all(np.isneginf(lse[:, qs])), "varlen: no keys"
                continue
            want = brute_force(q[None, qs], k[None, ks], v[None, ks], causal=causal, scale=0.9)
            _close(out[None, qs], want[0], 1e-12, what=f"varlen brute out seq {b} causal={causal}")
            _close(lse[None, :, qs], want[1], 1e-12, what=f"varlen brute lse seq {b} causal={causal}")


def pin_varlen_independence(vimpl):
    """Changing the queries and keys of one sequence leaves the others'
    results bit for bit."""
    rng = _rng(32)
    lq, lk = [3, 4, 2], [4, 5, 3]
    q, k, v = _pack(rng, lq, 2, 4), _pack(rng, lk, 2, 4), _pack(rng, lk, 2, 4)
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    o1, l1 = vimpl(q, k, v, cu_q, cu_k, 4, 5)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[3:7] += 1.0
    k2[4:9] -= 0.5
    v2[4:9] *= 3.0
    o2, l2 = vimpl(q2, k2, v2, cu_q, cu_k, 4, 5)
    for sl in (slice(0, 3), slice(7, 9)):
        assert np.array_equal(o1[sl], o2[sl]) and np.array_equal(l1[:, sl], l2[:, sl]), "varlen: sequences interact"
    assert not np.allclose(o1[3:7], o2[3:7]), "varlen: changed sequence unchanged"


def pin_varlen_spans(vimpl):
    """Offsets that leave the packed tensor are clamped:
    start = clamp(cu[b], 0, total), end = clamp(cu[b+1], start, total),
    length = min(end - start, max_seqlen).  Checked on the result: rows in
    no span stay out 0 / lse -inf, a sequence cut at max_seqlen equals the
    same sequence given exactly."""
    rng = _rng(33)
    total_q, total_k = 9, 8
    q, k, v = _randn(rng, total_q, 1, 3), _randn(rng, total_k, 1, 3), _randn(rng, total_k, 1, 3)
    cu_q = np.array([-4, 2, 2, 20])   # spans: [0, 2), [2, 2) empty, [2, 9) cut to 4 rows
    cu_k = np.array([0, 3, 5, 99])    # spans: [0, 3), [3, 5), [5, 8)
    out, lse = vimpl(q, k, v, cu_q, cu_k, 4, 4)
    assert np.all(out[6:] == 0) and np.all(np.isneginf(lse[:, 6:])), "varlen: rows past the cut written"
    o_a, l_a = vimpl(q[0:2], k[0:3], v[0:3], np.array([0, 2]), np.array([0, 3]), 2, 3)
    assert np.array_equal(out[0:2], o_a) and np.array_equal(lse[:, 0:2], l_a), "varlen: clamped first span"
    o_c, l_c = vimpl(q[2:6], k[5:8], v[5:8], np.array([0, 4]), np.array([0, 3]), 4, 3)
    assert np.array_equal(out[2:6], o_c) and np.array_equal(lse[:, 2:6], l_c), "varlen: span cut at max_seqlen"


VARLEN_PINS = [pin_varlen_equal_lengths, pin_varlen_brute_force, pin_varlen_independence, pin_varlen_spans]
