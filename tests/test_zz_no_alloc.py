"""The no-allocation forward (sage_attn_fwd_noalloc) against the one-call forward it varies
(sage_attn_fwd): the same kernels on the same inputs, so the outputs must be bit-identical.  Two
calls in a row share the library's per-GPU scratch array, the second on a smaller problem (and
another format pair), so stale contents of the larger call must not leak into the smaller one."""
import ctypes
import math

import pytest
import torch

from gpu_util import banner, device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_smooth_amd as S
    S.lib()
    return S


def _inputs(B, H, N, d, seed):
    from bit_quantized_attention_smooth_amd.workloads import make_inputs
    x = make_inputs(B, H, N, d, dtype="bf16", seed=seed, k_off_std=3.0)
    return [x[n].to(device()) for n in "qkv"]


def _call(S, entry, q, k, v, causal, qk, pv):
    B, H, N, d = q.shape
    o = torch.full_like(q, float("nan"))
    st = getattr(S.lib(), entry)(S._ptr(q), S._ptr(k), S._ptr(v), S._ptr(o), B, H, N, d, int(causal),
                                 ctypes.c_float(1 / math.sqrt(d)), S.FMT[qk], S.FMT[pv], S._stream())
    assert st == S.OK, S.lib().sage_last_error()
    return o


def test_noalloc_matches_one_call_entry_twice(sage):
    # large then small: (shape, causal, qk, pv)
    for (B, H, N, d), causal, qk, pv, seed in (((1, 16, 2048, 128), True, "int8", "fp8", 5),
                                                ((2, 2, 333, 64), False, "mxfp4", "mxfp4", 6)):
        banner(f"no-alloc forward B={B} H={H} N={N} d={d} causal={causal} {qk}/{pv}")
        q, k, v = _inputs(B, H, N, d, seed)
        got = _call(sage, "sage_attn_fwd_noalloc", q, k, v, causal, qk, pv)
        want = _call(sage, "sage_attn_fwd", q, k, v, causal, qk, pv)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        assert torch.equal(got, want)


def test_noalloc_binding_and_scratch_reuse_on_one_stream(sage):
    """Back-to-back calls on one stream without a host synchronization between them (the stream
    orders them), through the Python binding with a caller-provided output."""
    banner("no-alloc forward back to back")
    a = _inputs(1, 4, 700, 128, 11)
    b = _inputs(1, 3, 200, 64, 12)
    oa, ob = torch.empty_like(a[0]), torch.empty_like(b[0])
    sage.attn_fwd_noalloc(*a, causal=True, out=oa)
    sage.attn_fwd_noalloc(*b, causal=False, qk_fmt="int8", pv_fmt="fp8", out=ob)
    wa = sage.attn_fwd_oneshot(*a, causal=True)
    wb = sage.attn_fwd_oneshot(*b, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(oa, wa) and torch.equal(ob, wb)
