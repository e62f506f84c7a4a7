"""The synthetic workloads use the shapes the pages state (tests/golden)."""

import json
import os

import torch

from attention_forward_amd.workloads import WORKLOADS, make_custom, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload_facts.json")


def _facts():
    with open(GOLDEN) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


def test_shapes_follow_the_pages():
    f = _facts()
    vit = WORKLOADS["vit_multiview"]
    assert (vit.B, vit.Sq, vit.D) == (f["camera_views"], f["tokens_per_view"], f["vit_head_dim"])
    assert f["image_tokens"] == f["camera_views"] * f["tokens_per_view"]
    assert f["prefill_sequence"] == f["image_tokens"] + f["language_tail_tokens"]
    pre = WORKLOADS["prefix_gqa_padded"]
    assert pre.n_valid == f["prefill_sequence"] and pre.Sk >= pre.n_valid
    ae = WORKLOADS["action_expert_small_m"]
    assert ae.Sq == f["dit_rows"] and ae.n_valid == f["prefill_sequence"] + f["dit_rows"]
    for w in (pre, ae, WORKLOADS["causal_gqa_prefill"]):
        assert (w.Hq, w.Hkv, w.D) == (f["gqa_q_heads"], f["gqa_kv_heads"], f["gqa_head_dim"])
    # q, k, v projections of 8 + 1 + 1 heads at D256; o projection reads 8 heads
    assert (f["gqa_q_heads"] + 2 * f["gqa_kv_heads"]) * f["gqa_head_dim"] == f["decoder_qkv_n"]
    assert f["gqa_q_heads"] * f["gqa_head_dim"] == f["decoder_o_k"]


def test_inputs_are_seeded_and_poisoned():
    q1, k1, v1, s1 = make_inputs("prefix_gqa_padded")
    q2, k2, v2, s2 = make_inputs("prefix_gqa_padded")
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    assert q1.dtype == torch.bfloat16 and q1.shape == (1, 1024, 8, 256)
    assert k1.shape == (1, 1024, 1, 256) and s1.tolist() == [968]
    assert torch.all(k1[0, 968:] == 9984.0) and torch.all(v1[0, 968:] == 9984.0)
    assert torch.all(k1[0, :968].abs() < 100)
    _, k3, _, s3 = make_custom(2, 3, 5, 2, 1, 8, seed=7, n_valid=[5, 2], pad_value=float("nan"))
    assert s3.tolist() == [5, 2] and torch.isnan(k3[1, 2:]).all() and not torch.isnan(k3[0]).any()
