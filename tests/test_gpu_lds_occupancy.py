"""LDS race check: the fused forward and backward kernels launched with extra dynamic LDS
(SAGE_DEBUG_LDS_PAD), so that fewer workgroups share a CU and the waves interleave differently,
must give the same bits as the default launch -- for every kernel family (one- and two-buffer
forward, every format pair, packed sequences, both backward kernels, d = 64 and 128)."""
import os

import pytest
import torch

from gpu_util import banner, device

pytestmark = pytest.mark.gpu

PAD = str(96 * 1024)


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_smooth_amd as S
    S.lib()
    return S


def _twice(fn):
    """fn() with the default launch, then with the padded one (the variable is read per launch)."""
    os.environ.pop("SAGE_DEBUG_LDS_PAD", None)
    a = fn()
    torch.cuda.synchronize()
    os.environ["SAGE_DEBUG_LDS_PAD"] = PAD
    try:
        b = fn()
        torch.cuda.synchronize()
    finally:
        os.environ.pop("SAGE_DEBUG_LDS_PAD", None)
    return a, b


def _inputs(B, H, N, d, seed):
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(seed)
    x = {n: torch.randn(B, H, N, d, device=dev, generator=gen).to(torch.bfloat16) for n in ("q", "k", "v", "do")}
    x["k"] += 3.0 * torch.randn(B, H, 1, d, device=dev, generator=gen).to(torch.bfloat16)
    return x


CASES = [("int8", "fp8", 128, True), ("int8", "fp8", 64, False), ("int8", "f16", 128, False),
         ("int8_token", "fp8", 128, True), ("mxfp4", "fp8", 128, False), ("mxfp4", "mxfp4", 128, True),
         ("mxfp4", "mxfp8", 64, False), ("mxfp4_qblock", "fp8", 128, True)]


@pytest.mark.parametrize("qk,pv,d,causal", CASES, ids=[f"{a}_{b}_d{c}_{'causal' if e else 'full'}" for a, b, c, e in CASES])
def test_forward_bits_do_not_depend_on_occupancy(sage, qk, pv, d, causal):
    banner(f"LDS pad forward {qk}/{pv} d={d} causal={causal}")
    x = _inputs(2, 8, 1000, d, seed=11)
    a, b = _twice(lambda: sage.sageattn(x["q"], x["k"], x["v"], causal=causal, qk_fmt=qk, pv_fmt=pv, return_lse=True))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_packed_forward_bits_do_not_depend_on_occupancy(sage):
    banner("LDS pad packed forward")
    dev = device()
    x = _inputs(1, 8, 900, 128, seed=12)
    pk = {n: x[n][0].permute(1, 0, 2).contiguous() for n in "qkv"}
    cu = torch.tensor([0, 130, 131, 600, 900], dtype=torch.int32, device=dev)
    kv = {n: pk[n][:, :2].contiguous() for n in "kv"}
    a, b = _twice(lambda: sage.sageattn_varlen(pk["q"], kv["k"], kv["v"], cu, cu, 469, 469, causal=True,
                                               qk_fmt="mxfp4", pv_fmt="fp8", return_lse=True))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("d", [64, 128])
def test_backward_bits_do_not_depend_on_occupancy(sage, d):
    banner(f"LDS pad backward d={d}")
    x = _inputs(2, 4, 700, d, seed=13)
    o, lse = sage.sageattn(x["q"], x["k"], x["v"], causal=True, return_lse=True)
    a, b = _twice(lambda: sage.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, causal=True))
    for ga, gb in zip(a, b):
        assert torch.equal(ga, gb)
