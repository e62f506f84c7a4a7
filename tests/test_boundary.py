"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/fa.h declares, and rejects every invalid argument with its
documented code before any HIP call is made (pointers here are never
dereferenced: the library checks them only as numbers)."""

from __future__ import annotations

import ast
import os
import re

import pytest

from attention_forward_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# Aligned fake device addresses, far apart (never dereferenced on the host).
Q, K, V, O, L, S = (0x10000000 * (i + 1) for i in range(6))


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("library not built: run `python -m attention_forward_amd.build` (or __graft_entry__.build())")
    return fa.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(fa.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"


def test_abi_version_and_status_strings(lib):
    assert fa.fa_abi_version() == 5
    for code in range(10):
        assert fa.fa_status_string(code).startswith("FA_")
    assert "UNKNOWN" in fa.fa_status_string(99)


def _call(**over):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=1, Sq=64, Sk=64, Hq=8, Hkv=1, D=256, causal=0,
             seqused_k=0, scale=0.0625, stream=0)
    a.update(over)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Sq"], a["Sk"], a["Hq"],
                     a["Hkv"], a["D"], a["causal"], a["seqused_k"], a["scale"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=0), fa.FA_ERR_NULL),
    (dict(k=0), fa.FA_ERR_NULL),
    (dict(v=0), fa.FA_ERR_NULL),
    (dict(out=0), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(Sq=0), fa.FA_ERR_SHAPE),
    (dict(Sk=-1), fa.FA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_SHAPE),
    (dict(Hkv=0), fa.FA_ERR_SHAPE),
    (dict(causal=2), fa.FA_ERR_SHAPE),
    (dict(B=70000, Sq=1, Sk=1, Hq=1, Hkv=1, D=64), fa.FA_ERR_SHAPE),
    (dict(B=1, Sq=1 << 20, Sk=64, Hq=8, Hkv=1, D=256), fa.FA_ERR_SHAPE),
    (dict(D=128), fa.FA_ERR_UNSUPPORTED),
    (dict(D=80), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_SCALE),
    (dict(scale=-1.0), fa.FA_ERR_SCALE),
    (dict(scale=float("inf")), fa.FA_ERR_SCALE),
    (dict(scale=float("nan")), fa.FA_ERR_SCALE),
    (dict(q=Q + 8), fa.FA_ERR_ALIGN),
    (dict(out=O + 2), fa.FA_ERR_ALIGN),
    (dict(lse=L + 2), fa.FA_ERR_ALIGN),
    (dict(seqused_k=S + 1), fa.FA_ERR_ALIGN),
    (dict(out=Q), fa.FA_ERR_ALIAS),
    (dict(out=K + 4096), fa.FA_ERR_ALIAS),
    (dict(lse=V), fa.FA_ERR_ALIAS),
    (dict(lse=O + 1024), fa.FA_ERR_ALIAS),
    (dict(seqused_k=O + 4096), fa.FA_ERR_ALIAS),      # inside out
    (dict(seqused_k=L + 16), fa.FA_ERR_ALIAS),        # inside lse
    (dict(seqused_k=L - 4, B=2), fa.FA_ERR_ALIAS),    # its second entry is lse's first
])
def test_invalid_arguments_return_their_code(lib, over, code):
    assert _call(**over) == code


def _call_strided(qs=None, ks=None, vs=None, os_=None, dtype=fa.FA_BF16, **over):
    """fa_fwd_strided with contiguous strides unless overridden."""
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=1, Sq=64, Sk=64, Hq=8, Hkv=1, D=256, causal=0,
             seqused_k=0, scale=0.0625, stream=0)
    a.update(over)
    B, Sq, Sk, Hq, Hkv, D = (a[x] for x in ("B", "Sq", "Sk", "Hq", "Hkv", "D"))
    qs = qs or (Sq * Hq * D, Hq * D, D)
    ks = ks or (Sk * Hkv * D, Hkv * D, D)
    vs = vs or ks
    os_ = os_ or (Sq * Hq * D, Hq * D, D)
    return fa.fa_fwd_strided(a["q"], a["k"], a["v"], a["out"], a["lse"], B, Sq, Sk, Hq, Hkv, D,
                             qs, ks, vs, os_, dtype, a["causal"], a["seqused_k"], a["scale"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=0), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_SHAPE),
    (dict(D=128), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_SCALE),
    (dict(q=Q + 8), fa.FA_ERR_ALIGN),
    (dict(out=Q), fa.FA_ERR_ALIAS),
    (dict(lse=K + 64), fa.FA_ERR_ALIAS),
    (dict(seqused_k=O + 64), fa.FA_ERR_ALIAS),
    (dict(seqused_k=L), fa.FA_ERR_ALIAS),
    # element type
    (dict(dtype=2), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=-1), fa.FA_ERR_UNSUPPORTED),
    # strides: multiples of 8 elements (16-byte rows)
    (dict(qs=(64 * 8 * 256, 8 * 256 + 4, 256)), fa.FA_ERR_ALIGN),
    (dict(ks=(64 * 256, 260, 256)), fa.FA_ERR_ALIGN),
    (dict(os_=(64 * 8 * 264, 8 * 264, 260)), fa.FA_ERR_ALIGN),
    # negative strides, overlapping key rows, overlapping output rows
    (dict(qs=(-8, 8 * 256, 256)), fa.FA_ERR_SHAPE),
    (dict(ks=(64 * 256, 128, 256)), fa.FA_ERR_SHAPE),
    (dict(vs=(64 * 256, 0, 256)), fa.FA_ERR_SHAPE),
    (dict(os_=(64 * 8 * 256, 0, 256)), fa.FA_ERR_SHAPE),
    (dict(os_=(64 * 8 * 256, 8 * 256, 128)), fa.FA_ERR_SHAPE),
    # 32-bit key offsets of one (batch, kv head)
    (dict(ks=(0, 1 << 24, 256)), fa.FA_ERR_SHAPE),
    # head strides below 2^31 elements (32x32-bit index products); with one
    # kv head nothing else about these views is wrong
    (dict(ks=(64 * 256, 256, 1 << 31)), fa.FA_ERR_SHAPE),
    (dict(vs=(64 * 256, 256, 1 << 32)), fa.FA_ERR_SHAPE),
    # out inside the span of a strided q (one buffer)
    (dict(out=Q + 512, os_=(64 * 8 * 3 * 256, 8 * 3 * 256, 256), qs=(64 * 8 * 3 * 256, 8 * 3 * 256, 256)),
     fa.FA_ERR_ALIAS),
])
def test_strided_invalid_arguments_return_their_code(lib, over, code):
    assert _call_strided(**over) == code


def _call_varlen(**over):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, cu_q=S, cu_k=S + 64, B=2, max_q=64, max_k=64, total_q=100,
             total_k=100, Hq=8, Hkv=1, D=256, dtype=fa.FA_BF16, causal=0, scale=0.0625, stream=0)
    a.update(over)
    return fa.fa_fwd_varlen(a["q"], a["k"], a["v"], a["out"], a["lse"], a["cu_q"], a["cu_k"], a["B"], a["max_q"],
                            a["max_k"], a["total_q"], a["total_k"], a["Hq"], a["Hkv"], a["D"], a["dtype"],
                            a["causal"], a["scale"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=0), fa.FA_ERR_NULL),
    (dict(cu_q=0), fa.FA_ERR_NULL),
    (dict(cu_k=0), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(max_q=0), fa.FA_ERR_SHAPE),
    (dict(max_k=0), fa.FA_ERR_SHAPE),
    (dict(total_q=0), fa.FA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_SHAPE),
    (dict(causal=3), fa.FA_ERR_SHAPE),
    (dict(B=70000, Hkv=1), fa.FA_ERR_SHAPE),
    (dict(total_q=1 << 24), fa.FA_ERR_SHAPE),
    (dict(max_k=1 << 22), fa.FA_ERR_SHAPE),
    (dict(D=128), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=-1.0), fa.FA_ERR_SCALE),
    (dict(k=K + 8), fa.FA_ERR_ALIGN),
    (dict(cu_q=S + 2), fa.FA_ERR_ALIGN),
    (dict(lse=L + 1), fa.FA_ERR_ALIGN),
    (dict(out=Q + 1024), fa.FA_ERR_ALIAS),
    (dict(lse=O + 4096), fa.FA_ERR_ALIAS),
    (dict(cu_q=O + 64), fa.FA_ERR_ALIAS),
    (dict(cu_k=L + 8), fa.FA_ERR_ALIAS),
])
def test_varlen_invalid_arguments_return_their_code(lib, over, code):
    assert _call_varlen(**over) == code


def test_check_order_is_null_then_shape(lib):
    # A NULL pointer is reported even when the shape is also wrong.
    assert _call(q=0, B=0) == fa.FA_ERR_NULL
    assert _call(B=0, D=128) == fa.FA_ERR_SHAPE


def test_workspace_sizes(lib):
    # Long K/V buffers with few packed rows take the split-KV path ...
    n = fa.fa_fwd_workspace_bytes(1, 41, 1056, 8, 1, 256, 0)
    assert n > 0
    # ... and the size depends on the shape only, never on seqused_k values
    assert n == fa.fa_fwd_workspace_bytes(1, 41, 1056, 8, 1, 256, 0)
    # a single-pass plan needs none; a split plan needs some
    for shape in [(1, 1024, 1024, 8, 1, 256, 0), (1, 2048, 2048, 8, 1, 256, 1), (1, 64, 64, 1, 1, 64, 0),
                  (3, 256, 256, 16, 16, 72, 0)]:
        assert (fa.fa_fwd_workspace_bytes(*shape) > 0) == (fa.fa_fwd_plan(*shape)[5] > 0)
    assert fa.fa_fwd_workspace_bytes(1, 64, 64, 1, 1, 64, 0) == 0
    assert fa.fa_fwd_workspace_bytes(0, 64, 64, 1, 1, 64, 0) == 0


def test_plan_and_variant_sizes(lib):
    assert fa.fa_fwd_plan(1, 41, 1056, 8, 1, 256, 0)[5] > 0      # small M: split keys
    assert fa.fa_fwd_plan(3, 256, 256, 16, 16, 72, 0)[5] == 0    # enough rows: single pass
    plan = fa.fa_fwd_plan(1, 41, 1056, 8, 1, 256, 0)
    assert fa.fa_fwd_variant_workspace_bytes(1, 41, 1056, 8, 1, 256, 0, *plan) == \
        fa.fa_fwd_workspace_bytes(1, 41, 1056, 8, 1, 256, 0)
    assert fa.fa_fwd_variant_workspace_bytes(1, 41, 1056, 8, 1, 256, 0, 3, 4, 1, 64, 2, 0) == 0
    assert fa.fa_fwd_variant_workspace_bytes(1, 41, 1056, 8, 1, 256, 0, 1, 4, 1, 32, 2, 0) == 0


def test_plan_kernel_choice(lib):
    # Head dim 256: key-split workgroups (four waves over the keys of the same
    # 32 rows, piecewise refill of their tile buffers); with a row block per
    # compute unit there is no split-KV ...
    assert fa.fa_fwd_plan(1, 1024, 1024, 8, 1, 256, 0) == (2, 4, 4, 32, 2, 0)
    assert fa.fa_fwd_plan(1, 2048, 2048, 8, 1, 256, 1) == (2, 4, 4, 32, 3, 0)  # 512 blocks: two per CU
    assert fa.fa_fwd_plan(1, 1984, 1984, 8, 1, 256, 1) == (2, 4, 4, 32, 3, 0)  # 496 blocks
    assert fa.fa_fwd_plan(1, 1536, 1536, 8, 1, 256, 1) == (2, 4, 4, 32, 2, 0)  # 384 blocks: the heaviest run alone
    # ... a padded K/V buffer runs the same plan as the unpadded keys
    assert fa.fa_fwd_plan(1, 1024, 968, 8, 1, 256, 0) == fa.fa_fwd_plan(1, 1024, 1024, 8, 1, 256, 0)
    assert fa.fa_fwd_plan(1, 41, 1009, 8, 1, 256, 0) == fa.fa_fwd_plan(1, 41, 1056, 8, 1, 256, 0)
    # ... few rows: the keys are split into fixed ranges as well, over
    # 16-row workgroups (range size from the 16-row grid: 21 blocks -> 256)
    assert fa.fa_fwd_plan(1, 41, 1056, 8, 1, 256, 0) == (1, 4, 4, 32, 2, 256)
    assert fa.fa_fwd_plan(1, 1, 1056, 8, 1, 256, 1) == (1, 4, 4, 32, 2, 128)    # decode: 1 block
    assert fa.fa_fwd_plan(1, 256, 1024, 8, 1, 256, 1) == (1, 4, 4, 32, 2, 512)  # 128 blocks
    assert fa.fa_fwd_plan(1, 512, 512, 8, 1, 256, 0) == (1, 4, 4, 32, 2, 0)   # 128 blocks: 16-row blocks, no split
    assert fa.fa_fwd_plan(8, 41, 1056, 8, 1, 256, 0) == (1, 4, 4, 32, 2, 0)   # 168 16-row blocks: no split
    assert fa.fa_fwd_plan(4, 1024, 1024, 8, 1, 256, 0) == (2, 4, 1, 32, 2, 0)  # 1024 blocks: row-split, 128 rows
    assert fa.fa_fwd_plan(2, 1024, 1024, 8, 1, 256, 0) == (2, 4, 4, 32, 3, 0)  # 512 blocks: key-split ring
    assert fa.fa_fwd_plan(3, 700, 700, 8, 1, 256, 0) == (2, 4, 4, 32, 3, 0)    # 525 blocks: key-split ring
    assert fa.fa_fwd_plan(3, 1024, 1024, 8, 1, 256, 0) == (2, 4, 4, 32, 3, 0)  # 768 blocks: ring
    assert fa.fa_fwd_plan(4, 896, 896, 8, 1, 256, 0) == (2, 4, 1, 32, 2, 0)    # 896 blocks: row-split, 128 rows
    assert fa.fa_fwd_plan(2, 2048, 2048, 8, 1, 256, 1) == (2, 4, 4, 32, 2, 0)  # causal keeps key-split
    # ... long key buffers (over 2048 keys): about 32 power-of-two ranges per
    # row block, 32-row workgroups unless the rows fit in 16
    assert fa.fa_fwd_plan(1, 16, 131072, 8, 1, 256, 0) == (2, 4, 4, 32, 2, 4096)
    assert fa.fa_fwd_plan(1, 1, 32768, 8, 1, 256, 1) == (1, 4, 4, 32, 2, 1024)
    assert fa.fa_fwd_plan(1, 7, 65536, 2, 1, 64, 0) == (1, 4, 1, 128, 2, 2048)
    assert fa.fa_fwd_plan(1, 256, 8192, 8, 1, 256, 1) == (2, 4, 4, 32, 2, 2048)  # 64 blocks: 4 ranges
    assert fa.fa_fwd_plan(1, 1, 4096, 8, 8, 64, 1) == (1, 4, 1, 128, 2, 256)     # ranges of at least 256 keys
    # Smaller head dims: row-split workgroups, 16 rows per wave
    assert fa.fa_fwd_plan(3, 256, 256, 16, 16, 72, 0) == (1, 4, 1, 128, 2, 0)   # 192 blocks: 128-key tiles
    assert fa.fa_fwd_plan(6, 256, 256, 16, 16, 72, 0) == (1, 4, 1, 64, 2, 0)    # 384 blocks: 64-key tiles
    assert fa.fa_fwd_plan(2, 77, 77, 16, 16, 72, 1) == (1, 4, 1, 64, 2, 0)      # fewer than 128 keys
    # ... two key groups on the same rows once a row sees enough keys
    assert fa.fa_fwd_plan(1, 256, 256, 16, 16, 72, 0) == (1, 4, 2, 64, 2, 0)    # 64 blocks: 32-row blocks
    assert fa.fa_fwd_plan(1, 1024, 1024, 16, 16, 72, 0) == (1, 8, 2, 64, 2, 0)  # 1024 keys per row
    assert fa.fa_fwd_plan(1, 2048, 2048, 8, 8, 64, 1) == (1, 8, 2, 64, 2, 0)    # causal: 1024 on average
    assert fa.fa_fwd_plan(4, 512, 512, 8, 8, 64, 0) == (1, 4, 1, 128, 2, 0)     # 512 keys, 256 blocks: one group
    assert fa.fa_fwd_plan(1, 1024, 1024, 16, 16, 72, 1) == (1, 8, 2, 64, 2, 0)  # causal over 1024 keys
    assert fa.fa_fwd_plan(2, 1024, 1024, 16, 16, 64, 0) == (1, 4, 1, 128, 2, 0) # 512 blocks, 1024 keys: 128-key tiles
    assert fa.fa_fwd_plan(4, 1024, 1024, 8, 8, 72, 0) == (1, 4, 1, 64, 2, 0)    # ... not at D72
    assert fa.fa_fwd_plan(8, 1024, 1024, 16, 16, 64, 0) == (2, 4, 1, 64, 2, 0)  # 2048 blocks: 32 rows per wave
    assert fa.fa_fwd_plan(1, 2048, 2048, 32, 4, 64, 1) == (1, 4, 1, 64, 2, 0)   # causal: 16 rows per wave
    assert fa.fa_fwd_plan(1, 64, 64, 1, 1, 64, 0) == (1, 4, 1, 64, 2, 0)


def test_variant_rejections(lib):
    args = [Q, K, V, O, L, 1, 64, 64, 8, 1, 256, 0, 0, 0.0625]
    assert fa.fa_fwd_variant(*args, 3, 4, 1, 64, 2, 0, 0) == fa.FA_ERR_UNSUPPORTED   # not compiled
    assert fa.fa_fwd_variant(*args, 1, 4, 1, 32, 3, 0, 0) == fa.FA_ERR_UNSUPPORTED   # no 3-stage build
    assert fa.fa_fwd_variant(*args, 1, 4, 4, 32, 3, 0, 0) == fa.FA_ERR_UNSUPPORTED   # key-split ring: 32 rows only
    assert fa.fa_fwd_variant(*args, 2, 4, 4, 32, 4, 0, 0) == fa.FA_ERR_UNSUPPORTED   # key-split: nst 1 to 3
    assert fa.fa_fwd_variant(*args, 2, 4, 4, 64, 2, 0, 0) == fa.FA_ERR_UNSUPPORTED   # piecewise: 32-key tiles only
    assert fa.fa_fwd_variant(*args, 2, 4, 2, 32, 1, 0, 0) == fa.FA_ERR_UNSUPPORTED   # key groups: nst 2, not D256
    assert fa.fa_fwd_variant(*args, 1, 8, 2, 32, 2, 0, 0) == fa.FA_ERR_UNSUPPORTED   # key groups: not D256
    assert fa.fa_fwd_variant(*args, 1, 4, 3, 32, 2, 0, 0) == fa.FA_ERR_UNSUPPORTED   # nw not a multiple of kw
    assert fa.fa_fwd_variant(*args, 1, 4, 0, 32, 2, 0, 0) == fa.FA_ERR_UNSUPPORTED   # kw < 1
    assert fa.fa_fwd_variant_workspace_bytes(1, 64, 64, 8, 1, 256, 0, 1, 4, 0, 32, 2, 0) == 0
    assert fa.fa_fwd_variant(*args, 1, 4, 1, 32, 2, 48, 0) == fa.FA_ERR_UNSUPPORTED  # kps % bn
    assert fa.fa_fwd_variant(*args, 1, 4, 1, 32, 2, -32, 0) == fa.FA_ERR_UNSUPPORTED
    bad = list(args)
    bad[0] = 0
    assert fa.fa_fwd_variant(*bad, 1, 4, 1, 32, 2, 0, 0) == fa.FA_ERR_NULL


def _call_nvfp4(**over):
    """fa_fwd_nvfp4 with valid defaults (fake device addresses: nothing is
    launched, every case fails a host check first)."""
    a = dict(q=Q, k=K, v=V, fp4=O, sf=O + (1 << 24), lse=L, B=1, Sq=64, Sk=64, Hq=8, Hkv=1, D=256, causal=0,
             seqused_k=0, scale=0.0625, stream=0)
    a.update(over)
    return fa.fa_fwd_nvfp4(a["q"], a["k"], a["v"], a["fp4"], a["sf"], a["lse"], a["B"], a["Sq"], a["Sk"], a["Hq"],
                           a["Hkv"], a["D"], a["causal"], a["seqused_k"], a["scale"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=0), fa.FA_ERR_NULL),
    (dict(fp4=0), fa.FA_ERR_NULL),
    (dict(sf=0), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_SHAPE),
    (dict(D=72, Hq=16, Hkv=16), fa.FA_ERR_UNSUPPORTED),   # blocks of 16 would straddle heads
    (dict(D=128), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_SCALE),
    (dict(fp4=O + 2), fa.FA_ERR_ALIGN),
    (dict(q=Q + 8), fa.FA_ERR_ALIGN),
    (dict(lse=L + 2), fa.FA_ERR_ALIGN),
    (dict(fp4=Q), fa.FA_ERR_ALIAS),
    (dict(sf=K + 64), fa.FA_ERR_ALIAS),
    (dict(sf=O + 1024), fa.FA_ERR_ALIAS),            # inside the codes (64 rows x 128 bytes)
    (dict(lse=O + 4096), fa.FA_ERR_ALIAS),
    (dict(seqused_k=O + 64), fa.FA_ERR_ALIAS),       # inside the codes
    (dict(seqused_k=O + (1 << 24) + 8), fa.FA_ERR_ALIAS),   # inside the scales
    (dict(seqused_k=L + 4), fa.FA_ERR_ALIAS),
])
def test_nvfp4_invalid_arguments_return_their_code(lib, over, code):
    assert _call_nvfp4(**over) == code


def test_static_entry_point_host_checks(lib):
    """fa_fwd_static: the argument checks of fa_fwd, and a shape whose
    split-KV partials exceed the static scratch is refused before any
    device work (both hold without a GPU)."""
    def call(**over):
        a = dict(q=Q, k=K, v=V, out=O, lse=L, B=1, Sq=64, Sk=64, Hq=8, Hkv=1, D=256, causal=0,
                 seqused_k=0, scale=0.0625, stream=0)
        a.update(over)
        return fa.fa_fwd_static(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Sq"], a["Sk"], a["Hq"],
                                a["Hkv"], a["D"], a["causal"], a["seqused_k"], a["scale"], a["stream"])
    assert call(q=0) == fa.FA_ERR_NULL
    assert call(D=128) == fa.FA_ERR_UNSUPPORTED
    assert call(scale=-1.0) == fa.FA_ERR_SCALE
    assert call(out=Q) == fa.FA_ERR_ALIAS
    # 8 views of 16 heads at D72, 64 rows over 2048 keys: split partials of 9.25 MiB
    big = dict(B=8, Sq=64, Sk=2048, Hq=16, Hkv=16, D=72)
    need = fa.fa_fwd_workspace_bytes(8, 64, 2048, 16, 16, 72, 0)
    assert need > fa.FA_STATIC_SCRATCH_BYTES
    assert call(**big) == fa.FA_ERR_SCRATCH
    assert "static scratch" in fa.fa_status_string(fa.FA_ERR_SCRATCH)
    # every workload fits (the split ones need well under the maximum)
    from attention_forward_amd.workloads import WORKLOADS
    for w in WORKLOADS.values():
        assert fa.fa_fwd_workspace_bytes(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D, w.causal) <= fa.FA_STATIC_SCRATCH_BYTES


def test_set_workspace_null_with_size(lib):
    assert fa.fa_set_workspace(0, 1024) == fa.FA_ERR_NULL


def test_tensor_interface_rejects_cpu_tensors():
    import torch

    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        fa.attention(q, q, q)


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "attention_forward_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            path = os.path.join(dirpath, f)
            if f.endswith(".py"):
                tree = ast.parse(open(path).read())
                for node in ast.walk(tree):
                    if isinstance(node, ast.Import):
                        names = [a.name for a in node.names]
                    elif isinstance(node, ast.ImportFrom):
                        names = [node.module or ""]
                    else:
                        continue
                    assert not any(n.split(".")[0] == "oracle" for n in names), path
            elif f.endswith((".hip", ".cpp", ".h")):
                assert "oracle" not in open(path).read().lower(), path
