"""GPU parity of the strided / fp16 entry point (fa_fwd_strided through the
C ABI) against the fp64 oracle.

Strided views are how the attention reads a fused QKV GEMM output in place
("GROOT N1.7 update: Thor NVFP4 + FA4 performance tier", section "What is in
the tier"); fp16 is the other element type of the pages' attention kernels.
The oracle takes the exact element values, so the bar is the one of the
contiguous path: max|dout| <= 1e-2, max|dlse| <= 1e-3 on the workloads
(fp16 rounds out and P more finely than bf16), the per-element bound of
tests/gpu_util.py elsewhere; a strided bf16 call is bit-identical to the
contiguous call on the same values (same kernel, same arithmetic), and no
byte outside the output view is written."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from attention_forward_amd import fa
from attention_forward_amd.workloads import WORKLOADS, make_custom, make_inputs
from tests.gpu_util import assert_parity, run_oracle, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fused(q, k, v):
    """q, k, v as slices of one [B, S, Hq + 2 Hkv, D] buffer on the device
    (the layout of a fused QKV projection); requires Sq == Sk."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    buf = torch.empty(B, S, Hq + 2 * Hkv, D, dtype=q.dtype, device=DEV)
    buf[:, :, :Hq] = q.to(DEV)
    buf[:, :, Hq:Hq + Hkv] = k.to(DEV)
    buf[:, :, Hq + Hkv:] = v.to(DEV)
    return buf[:, :, :Hq], buf[:, :, Hq:Hq + Hkv], buf[:, :, Hq + Hkv:]


def _run(q, k, v, s=None, **kw):
    out, lse = fa.attention(q, k, v, seqused_k=None if s is None else s.to(DEV), **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


# (B, S, Hq, Hkv, D, causal, n_valid): self-attention shapes read from a fused buffer
FUSED = [
    (2, 150, 4, 4, 64, False, None),
    (3, 256, 16, 16, 72, False, None),      # the multi-view ViT shape
    (1, 300, 8, 1, 256, False, [260]),      # GQA with seqused_k
    (2, 130, 6, 3, 64, True, None),         # causal GQA
    (1, 520, 8, 1, 256, True, None),        # causal, key-split kernel
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "x".join(str(x) for x in c[:5]) + ("c" if c[5] else ""))
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_fused_qkv_views_match_oracle(gpu_device, case, dtype):
    B, S, Hq, Hkv, D, causal, nv = case
    _say(f"fused {case} {dtype}")
    q, k, v, s = make_custom(B, S, S, Hq, Hkv, D, seed=11, n_valid=nv, dtype=dtype)
    qv, kv, vv = _fused(q, k, v)
    assert not qv.is_contiguous()
    got = _run(qv, kv, vv, s, causal=causal)
    want = run_oracle(q, k, v, s, causal=causal)
    assert_parity(got, want, f"fused {case} {dtype}", strict=False)
    if dtype == torch.bfloat16:
        # same values through the contiguous entry point: bit-identical
        ref = _run(q.to(DEV), k.to(DEV), v.to(DEV), s, causal=causal)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_fp16_workloads_match_oracle(gpu_device, name):
    w = WORKLOADS[name]
    _say(f"fp16 workload {name}")
    q, k, v, s = make_inputs(name, dtype=torch.float16)
    got = _run(q.to(DEV), k.to(DEV), v.to(DEV), s, causal=w.causal, scale=w.scale)
    assert got[0].dtype == torch.float16
    want = run_oracle(q, k, v, s, causal=w.causal, scale=w.scale)
    d_out, d_lse = assert_parity(got, want, f"fp16 {name}")
    _say(f"  fp16 {name}: max|dout|={d_out:.3e} max|dlse|={d_lse:.3e}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_fp16_and_bf16_padding_never_read(gpu_device, dtype):
    # keys past seqused_k filled with inf/nan leave the result bit-identical
    base = make_custom(1, 41, 1056, 8, 1, 256, seed=5, n_valid=1009, dtype=dtype)
    ref = _run(*(t.to(DEV) for t in base[:3]), base[3])
    for pad in (float("inf"), float("nan"), -1e4):
        q, k, v, s = make_custom(1, 41, 1056, 8, 1, 256, seed=5, n_valid=1009, pad_value=pad, dtype=dtype)
        got = _run(q.to(DEV), k.to(DEV), v.to(DEV), s)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), pad


@pytest.mark.parametrize("D", [64, 72, 256])
def test_output_view_writes_only_its_rows(gpu_device, D):
    # out is a [B, S, H, D] view of a wider buffer; the columns around it keep
    # their sentinel bytes.  q and k/v also come in transposed (batch, head,
    # seq, dim) storage.
    B, S, H = 2, 97, 4
    q, k, v, _ = make_custom(B, S, S, H, H, D, seed=3)
    qt = q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)   # strides (H S D, D, S D)
    kt = k.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    vt = v.to(DEV)
    wide = torch.full((B, S, H, D + 16), 7.0, dtype=torch.bfloat16, device=DEV)
    out = wide[:, :, :, 8:8 + D]
    lse = torch.empty(B, H, S, dtype=torch.float32, device=DEV)
    fa.attention(qt, kt, vt, out=out, lse=lse)
    torch.cuda.synchronize()
    w = wide.cpu()
    assert torch.all(w[..., :8] == 7.0) and torch.all(w[..., 8 + D:] == 7.0)
    assert_parity((out.cpu(), lse.cpu()), run_oracle(q, k, v), f"out view D={D}", strict=False)


def test_small_m_split_path_from_fused_buffer(gpu_device):
    # action-expert shape whose queries come from a strided buffer: the
    # split-KV partials and the merge kernel write through the output view
    q, k, v, s = make_custom(1, 41, 1056, 8, 1, 256, seed=9, n_valid=1009)
    qbuf = torch.zeros(1, 41, 24, 256, dtype=torch.bfloat16, device=DEV)
    qbuf[:, :, 8:16] = q.to(DEV)
    got = _run(qbuf[:, :, 8:16], k.to(DEV), v.to(DEV), s)
    assert_parity(got, run_oracle(q, k, v, s), "split from view")
    ref = _run(q.to(DEV), k.to(DEV), v.to(DEV), s)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_strided_rejections_raise(gpu_device):
    q, k, v, _ = make_custom(1, 64, 64, 2, 2, 64, seed=1)
    buf = torch.zeros(1, 64, 2, 68, dtype=torch.bfloat16, device=DEV)   # row stride 68: not 8-aligned heads
    with pytest.raises(fa.FAError) as e:
        fa.attention(buf[..., :64], k.to(DEV), v.to(DEV))
    assert e.value.code == fa.FA_ERR_ALIGN
    with pytest.raises(ValueError):
        fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), variant=(1, 4, 1, 64, 2, 0), out=torch.empty(
            1, 64, 2, 64, dtype=torch.bfloat16, device=DEV).transpose(1, 2).contiguous().transpose(1, 2))
    with pytest.raises(TypeError):
        fa.attention(q.to(DEV), k.to(DEV).half(), v.to(DEV))
