"""Plain fp64 CPU oracle for fused attention forward with log-sum-exp.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from ``attention_forward_amd``.

What it computes (the plain definition, evaluated directly in float64):

    out[b, i, h, :] = sum_{j in J} softmax_j(sigma * q_i . k_j) * v_j
    lse[b, h, i]    = log sum_{j in J} exp(sigma * q_i . k_j)

Sources for each part of the definition:

* The operation itself, forward only, returning the pair ``(out, lse)``:
  "flashrt/fa4-cute-runtime" model card, section "Functions" (the vendored
  forward wrapper returns the output together with the log-sum-exp).
* Tensor layout (batch, sequence, heads, head_dim): same card, closing
  paragraph on the FlashAttention input contract.
* ``seqused_k``: same card, the padded fixed-shape graph example -- keys at
  positions ``>= seqused_k[b]`` of a padded K/V buffer are not attended.
  "pi05_thor_decoder_fp4_e2e.md", section "Fused GeGLU FFN in the Decoder"
  (the seqused attention passage): out-of-range columns contribute exactly
  zero probability, so the result equals attention over the valid prefix.
* Grouped-query heads (several Q heads share one K/V head, ``pack_gqa``):
  model card, padded-graph example; "GROOT N1.7 update: Thor NVFP4 + FA4
  performance tier", section "What is in the tier" (LLM causal GQA).
* Causal masking for the prefill, bidirectional attention for the action
  expert: "Model Demo: PI0.5 End-to-End VLA Inference", section "Model
  stages".

Readings taken where the pages are silent:

* lse is the natural logarithm of the sum of exp(sigma * q . k) over the
  attended keys (scale included), laid out [B, Hq, Sq].
* The Q head h reads K/V head floor(h / (Hq / Hkv)).
* seqused_k[b] is clamped to [0, Sk]; an empty key set gives out = 0 and
  lse = -inf.
* Causal means key j is attended by query i iff j <= i + (n_b - Sq): the
  last query row lines up with the last valid key (the bottom-right
  alignment of FlashAttention, whose input contract the model card's
  runtime follows).  With Sq == Sk and no seqused_k this is j <= i, the
  causal prefill of the PI0.5 demo; with fewer queries than keys it is a
  chunk of new positions attending a cache, and with more queries than keys
  the first Sq - n_b rows attend nothing.
* sigma is float64(float32(scale)): the value the device receives.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["attention_ref", "attention_varlen_ref", "varlen_spans", "effective_scale", "valid_lengths",
           "attended_pairs"]


def effective_scale(scale, head_dim: int) -> float:
    """sigma = float32(scale) widened to float64; default 1/sqrt(head_dim).

    The default mirrors the usual softmax temperature of scaled dot-product
    attention; the model card's examples pass no scale, so the conventional
    1/sqrt(D) is the plain reading.
    """
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return float(np.float32(scale))


def valid_lengths(batch: int, sk: int, seqused_k) -> np.ndarray:
    """n_b = clamp(seqused_k[b], 0, Sk), or Sk for every b when absent.

    Model card "flashrt/fa4-cute-runtime", padded fixed-shape graph example.
    """
    if seqused_k is None:
        return np.full(batch, sk, dtype=np.int64)
    n = np.asarray(seqused_k, dtype=np.int64).reshape(-1)
    if n.shape[0] != batch:
        raise ValueError("seqused_k must hold one length per batch entry")
    return np.clip(n, 0, sk)


def attended_pairs(batch, sq, sk, hq, causal, seqused_k) -> int:
    """Number of (query, key) pairs that take part, over all heads.

    Used for the effective-FLOP count 4 * D * pairs (two multiply-adds per
    pair and head-dim element: one for q.k, one for p*v).
    """
    n = valid_lengths(batch, sk, seqused_k)
    total = 0
    for b in range(batch):
        if causal:
            # query i attends keys 0..min(i + n_b - Sq, n_b - 1)
            i = np.arange(sq, dtype=np.int64)
            total += int(np.minimum(i + 1 + (n[b] - sq), n[b]).clip(min=0).sum())
        else:
            total += sq * int(n[b])
    return total * hq


def attention_ref(q, k, v, *, causal=False, seqused_k=None, scale=None):
    """Reference attention forward in float64.

    Args:
      q: array [B, Sq, Hq, D] (any float dtype; widened exactly to float64).
      k, v: arrays [B, Sk, Hkv, D]; Hq must be a multiple of Hkv.
      causal: key j is attended by query i only when j <= i + (n_b - Sq),
        n_b the number of valid keys of batch entry b.
      seqused_k: None, or B integers: keys j >= seqused_k[b] are not read.
      scale: softmax temperature; None means 1/sqrt(D).

    Returns:
      (out [B, Sq, Hq, D] float64, lse [B, Hq, Sq] float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D (batch, seq, heads, head_dim)")
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape:
        raise ValueError("k and v must be [B, Sk, Hkv, D] matching q")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    sigma = effective_scale(scale, D)
    group = Hq // Hkv
    n = valid_lengths(B, Sk, seqused_k)

    out = np.zeros((B, Sq, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq, Sq), -np.inf, dtype=np.float64)

    for b in range(B):
        nb = int(n[b])
        if nb == 0:
            continue  # no key attended: out stays 0, lse stays -inf
        # Padding rows j >= n_b are never read: slice them off first.
        kb = k[b, :nb]  # [nb, Hkv, D]
        vb = v[b, :nb]
        i = np.arange(Sq)[:, None]
        j = np.arange(nb)[None, :]
        keep = (j <= i + (nb - Sq)) if causal else np.ones((Sq, nb), dtype=bool)
        rows = np.any(keep, axis=1)  # queries that attend at least one key
        for h in range(Hq):
            hk = h // group
            s = sigma * np.matmul(q[b, :, h, :], kb[:, hk, :].T)  # [Sq, nb]
            s = np.where(keep, s, -np.inf)[rows]
            m = np.max(s, axis=1, keepdims=True)  # finite: every kept row attends a key
            w = np.exp(s - m)
            l = np.sum(w, axis=1, keepdims=True)
            out[b, rows, h, :] = np.matmul(w, vb[:, hk, :]) / l
            lse[b, h, rows] = (m + np.log(l))[:, 0]
    return out, lse


def varlen_spans(cu_seqlens, total: int, max_seqlen: int):
    """(start, length) of each packed sequence: sequence b covers rows
    [start_b, start_b + length_b) with start_b = clamp(cu[b], 0, total),
    end_b = clamp(cu[b + 1], start_b, total), length_b = min(end_b - start_b,
    max_seqlen).  The offsets live on the device and cannot be checked by the
    host, so any values give rows inside the packed tensor (reading taken
    where the pages are silent); offsets that run backwards make spans
    overlap, and rows shared by two sequences are then not specified."""
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    spans = []
    for b in range(cu.shape[0] - 1):
        start = min(max(int(cu[b]), 0), total)
        end = min(max(int(cu[b + 1]), start), total)
        spans.append((start, min(end - start, max_seqlen)))
    return spans


def attention_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
                         scale=None):
    """Reference attention over packed variable-length sequences.

    "flashrt/fa4-cute-runtime" model card, section "Functions": besides the
    fixed-shape forward the runtime exposes FlashAttention's varlen forward,
    in which B sequences of different lengths are packed along one token
    dimension and delimited by cumulative offsets.  Each sequence is an
    independent attention problem; causal is aligned bottom-right within a
    sequence (as in attention_ref).

    Args:
      q: [total_q, Hq, D]; k, v: [total_k, Hkv, D].
      cu_seqlens_q, cu_seqlens_k: B + 1 offsets each (spans: varlen_spans).
      max_seqlen_q, max_seqlen_k: longest sequence; longer ones are cut.

    Returns:
      (out [total_q, Hq, D] float64, lse [Hq, total_q] float64); rows that
      belong to no sequence are out 0 and lse -inf here (the device leaves
      them untouched).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    total_q, Hq, D = q.shape
    total_k = k.shape[0]
    sq = varlen_spans(cu_seqlens_q, total_q, max_seqlen_q)
    sk = varlen_spans(cu_seqlens_k, total_k, max_seqlen_k)
    if len(sq) != len(sk):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    lse = np.full((Hq, total_q), -np.inf, dtype=np.float64)
    for (q0, lq), (k0, lk) in zip(sq, sk):
        if lq == 0:
            continue
        if lk == 0:
            continue  # no key: out 0, lse -inf
        o, l = attention_ref(q[None, q0:q0 + lq], k[None, k0:k0 + lk], v[None, k0:k0 + lk], causal=causal,
                             scale=scale)
        out[q0:q0 + lq] = o[0]
        lse[:, q0:q0 + lq] = l[0]
    return out, lse
