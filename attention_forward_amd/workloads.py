"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic: it only draws random tensors of
the shapes the workloads use, so that the HIP path and the fp64 oracle are
fed the very same bytes.  It imports torch for the generator and bf16
rounding only and never touches a GPU.

Workload shapes (each from the pages, see the citations per entry):

* ``single_head``: a one-head 64x64 sanity case (no page shape; the
  smallest case with a full 64-key tile).
* ``vit_multiview``: 3 camera views of 256 SigLIP tokens ("Model Demo:
  PI0.5 End-to-End VLA Inference", section "Model stages": pixel_values for
  three cameras give image embeddings of 3 x 256 tokens); D72 MHA from the
  "flashrt/fa4-cute-runtime" card's qualified profiles; 16 heads.
* ``prefix_gqa_padded``: the 968-token prefix (768 image + 200 language
  tokens, "Model Demo: PI0.5", section "Model stages") in a 1024-key padded
  buffer with ``seqused_k`` on the device; 8 Q heads / 1 KV head at D256
  (model card introduction and padded-graph example).
* ``causal_gqa_prefill``: causal 8Q/1KV D256 prefill over 2048 tokens
  ("GROOT N1.7 update", section "What is in the tier": LLM causal GQA).
* ``action_expert_small_m``: 41 action rows ("GROOT N1.7 update", section
  "What is in the tier": the DiT runs at M=41) attending a 1056-key padded
  buffer with 1009 = 968 + 41 valid keys (prefix plus self, "Model Demo:
  PI0.5", section "Model stages").

Recipe: ``torch.Generator().manual_seed(seed)``; ``torch.randn`` in float32
on the CPU for q [B,Sq,Hq,D], then k and v [B,Sk,Hkv,D] in that order; each
rounded to bfloat16 (round-to-nearest-even).  For padded buffers, K and V
rows ``[n_valid, Sk)`` are then overwritten with a poison value (1e4 by
default, which bf16 stores as 9984) so that any leak from padding shows.
"""

from __future__ import annotations

import dataclasses
import math

import torch

__all__ = ["Workload", "WORKLOADS", "WORKLOAD_ORDER", "make_inputs", "make_custom"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Sq: int
    Sk: int  # K/V buffer length
    n_valid: int | None  # None: no seqused_k, every key valid
    Hq: int
    Hkv: int
    D: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def valid_keys(self) -> int:
        return self.Sk if self.n_valid is None else self.n_valid


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head", 1, 64, 64, None, 1, 1, 64, False, 1),
        Workload("vit_multiview", 3, 256, 256, None, 16, 16, 72, False, 2),
        Workload("prefix_gqa_padded", 1, 1024, 1024, 968, 8, 1, 256, False, 3),
        Workload("causal_gqa_prefill", 1, 2048, 2048, None, 8, 1, 256, True, 4),
        Workload("action_expert_small_m", 1, 41, 1056, 1009, 8, 1, 256, False, 5),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)


def make_custom(B, Sq, Sk, Hq, Hkv, D, *, seed, n_valid=None, pad_value=1.0e4,
                q_scale=1.0, k_scale=1.0, v_scale=1.0, dtype=torch.bfloat16):
    """Seeded CPU tensors q [B,Sq,Hq,D], k and v [B,Sk,Hkv,D] of ``dtype``
    (bfloat16 by default, or float16), drawn N(0,1) in fp32 and rounded.

    ``n_valid`` may be an int (same for all batch entries) or a sequence of
    B ints; rows ``[n_valid[b], Sk)`` of K and V are set to ``pad_value``
    (which may be ``float('nan')`` or ``float('inf')``).  Returns
    (q, k, v, seqused_k) with seqused_k an int32 CPU tensor or None.
    """
    g = torch.Generator().manual_seed(int(seed))
    q = torch.randn(B, Sq, Hq, D, generator=g, dtype=torch.float32) * q_scale
    k = torch.randn(B, Sk, Hkv, D, generator=g, dtype=torch.float32) * k_scale
    v = torch.randn(B, Sk, Hkv, D, generator=g, dtype=torch.float32) * v_scale
    q, k, v = (t.to(dtype) for t in (q, k, v))
    seqused = None
    if n_valid is not None:
        lens = [int(n_valid)] * B if isinstance(n_valid, int) else [int(x) for x in n_valid]
        if len(lens) != B:
            raise ValueError("n_valid needs one entry per batch element")
        for b, n in enumerate(lens):
            lo = max(0, min(n, Sk))
            k[b, lo:] = pad_value
            v[b, lo:] = pad_value
        seqused = torch.tensor(lens, dtype=torch.int32)
    return q, k, v, seqused


def make_inputs(name_or_workload, *, seed=None, pad_value=1.0e4, dtype=torch.bfloat16):
    """Inputs for one named workload (CPU tensors, seqused_k or None)."""
    w = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    return make_custom(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D,
                       seed=w.seed if seed is None else seed,
                       n_valid=w.n_valid, pad_value=pad_value, dtype=dtype)
