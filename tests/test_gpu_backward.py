"""GPU 8-bit backward (dQ, dK, dV) against exact fp64 gradients of softmax attention:
cosine >= 0.99 per gradient, on small ragged cases at d = 64 and 128, on the training
workload (B=8 H=16 N=2048 d=64, causal; every head, with its forward O and LSE) and on a
d = 128 causal case (every head)."""
import math

import numpy as np
import pytest
import torch

from gpu_util import banner, cos, device, to_np64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_smooth_amd as S
    S.lib()
    return S


def _run(S, x, causal, sm):
    g = {n: x[n].to(device()) for n in ("q", "k", "v", "do")}
    o, lse = S.sageattn(g["q"], g["k"], g["v"], causal=causal, sm_scale=sm, return_lse=True)
    dq, dk, dv = S.attn_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal, sm_scale=sm)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,dtype", [(300, "bf16"), (64, "bf16"), (129, "f16")])
def test_backward_matches_fp64(sage, causal, N, dtype, d):
    import oracle
    from bit_quantized_attention_smooth_amd.workloads import make_inputs, as_u16
    banner(f"backward N={N} causal={causal} {dtype} d={d}")
    B, H, sm = 1, 2, 1 / math.sqrt(d)
    x = make_inputs(B, H, N, d, dtype=dtype, seed=40 + N, k_off_std=2.0, with_do=True)
    _, _, dq, dk, dv = _run(sage, x, causal, sm)
    f = {n: oracle.widen(as_u16(x[n]), dtype).reshape(B * H, N, d) for n in ("q", "k", "v", "do")}
    rq, rk, rv = oracle.attn_bwd_ref(f["q"], f["k"], f["v"], f["do"], causal, sm)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = to_np64(got).reshape(B * H, N, d)
        assert np.isfinite(g).all(), name
        assert cos(g, ref) >= 0.99, (name, cos(g, ref))


@pytest.mark.parametrize("d", [64, 128])
def test_backward_dv_column_sum(sage, d):
    """Rows of P sum to one, so sum_j dV_j = sum_i dO_i per head and channel, up to the FP8
    rounding of dO and P~.  Each E4M3 code of dO is off by at most half an ulp, 2^-4 of the value,
    and round-to-nearest makes these errors independent and uniform: a column's error has a
    standard deviation of at most 2^-4 sqrt(sum_i dO_i^2 / 3).  Allowed: 6 of those plus 3 % of
    the column sum (the rows of 448 P quantized to E4M3 sum to 448 within that)."""
    from bit_quantized_attention_smooth_amd.workloads import make_inputs
    banner(f"backward dV column sum d={d}")
    x = make_inputs(1, 2, 512, d, dtype="bf16", seed=77, with_do=True)
    _, _, _, _, dv = _run(sage, x, False, 1 / math.sqrt(d))
    got = dv.float().sum(dim=2).cpu().numpy().astype(np.float64)
    dof = x["do"].float().numpy().astype(np.float64)
    want = dof.sum(axis=2)
    sigma = 2.0 ** -4 * np.sqrt((dof * dof).sum(axis=2) / 3.0)
    err = np.abs(got - want)
    assert (err <= 6.0 * sigma + 0.03 * np.abs(want)).all(), (err.max(), sigma.max())
    # and the errors look like rounding noise, not a bias: their RMS stays near one sigma
    assert np.sqrt((err * err).mean()) <= 1.5 * np.sqrt((sigma * sigma).mean()), (np.sqrt((err * err).mean()), sigma.max())


def _per_head_cos(got, ref):
    return [cos(got[i], ref[i]) for i in range(got.shape[0])]


def test_backward_training_workload_all_heads(sage):
    """The training workload (B=8 H=16 N=2048 d=64, causal) in full: the forward's O and LSE on
    every row of every head against the oracle's simulation (element-wise with the admissible-
    code slack, cosine >= 0.9999) and against exact fp64 attention (cosine >= 0.99 per head), and
    dQ, dK, dV of every head against the exact fp64 gradients at cosine >= 0.99 per head."""
    import oracle
    from bit_quantized_attention_smooth_amd.workloads import workload_inputs, as_u16
    from gpu_util import excess, within
    banner("backward training workload b8h16n2048d64 causal, all heads")
    x, w = workload_inputs("train_causal_b8h16n2048d64")
    B, H, N, d, sm = w["B"], w["H"], w["N"], w["d"], w["sm_scale"]
    BH = B * H
    o, lse, dq, dk, dv = _run(sage, x, True, sm)
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
    f = {n: oracle.widen(as_u16(x[n]), "bf16").reshape(BH, N, d) for n in ("q", "k", "v", "do")}
    qz = oracle.quant_int8_fp8(f["q"], f["k"], f["v"], sm)
    o_sim, lse_sim, sl = oracle.attn_int8_fp8(qz, N, d, True, sm, 64, slack=True)
    o_ref, lse_ref = oracle.attn_ref(f["q"], f["k"], f["v"], True, sm)
    og = to_np64(o).reshape(BH, N, d)
    assert within(og, o_sim, sl), excess(og, o_sim, sl)
    assert cos(og, o_sim) >= 0.9999
    assert np.allclose(lse.cpu().numpy().reshape(BH, N), lse_sim, rtol=1e-4, atol=2e-3)
    assert min(_per_head_cos(og, o_ref)) >= 0.99
    rq, rk, rv = oracle.attn_bwd_ref(f["q"], f["k"], f["v"], f["do"], True, sm)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        ph = _per_head_cos(to_np64(got).reshape(BH, N, d), ref)
        print(f"  {name}: per-head cosine min {min(ph):.5f} (head {int(np.argmin(ph))}), mean {np.mean(ph):.5f}",
              flush=True)
        assert min(ph) >= 0.99, (name, min(ph), int(np.argmin(ph)))


def test_backward_d128_causal_all_heads(sage):
    """Head dimension 128 at a prefill-like size (B=2 H=8 N=2048, causal): every head's
    gradients at cosine >= 0.99 of the exact fp64 gradients."""
    import oracle
    from bit_quantized_attention_smooth_amd.workloads import make_inputs, as_u16
    banner("backward b2h8n2048d128 causal, all heads")
    B, H, N, d = 2, 8, 2048, 128
    sm = 1 / math.sqrt(d)
    x = make_inputs(B, H, N, d, dtype="bf16", seed=79, k_off_std=2.0, with_do=True)
    o, lse, dq, dk, dv = _run(sage, x, True, sm)
    f = {n: oracle.widen(as_u16(x[n]), "bf16").reshape(B * H, N, d) for n in ("q", "k", "v", "do")}
    rq, rk, rv = oracle.attn_bwd_ref(f["q"], f["k"], f["v"], f["do"], True, sm)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        ph = _per_head_cos(to_np64(got).reshape(B * H, N, d), ref)
        assert min(ph) >= 0.99, (name, min(ph), int(np.argmin(ph)))
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()


@pytest.mark.parametrize("d", [64, 128])
def test_backward_tiny_output_gradient(sage, d):
    """dO with magnitudes near 1e-36: 448 / max|dO| exceeds binary32, so the FP8 codes of dO must
    be formed in a scaled frame; every gradient stays finite and at cosine >= 0.99 of the exact
    fp64 gradients (which are of the same tiny magnitude, still normal in bf16)."""
    import oracle
    from bit_quantized_attention_smooth_amd.workloads import make_inputs, as_u16
    banner(f"backward tiny dO d={d}")
    B, H, N = 1, 2, 200
    sm = 1 / math.sqrt(d)
    x = make_inputs(B, H, N, d, dtype="bf16", seed=91, k_off_std=2.0, with_do=True)
    x["do"] = (x["do"].float() * 2.5e-37).to(torch.bfloat16)
    assert 1e-37 < float(x["do"].float().abs().max()) < 1.3e-36
    _, _, dq, dk, dv = _run(sage, x, True, sm)
    f = {n: oracle.widen(as_u16(x[n]), "bf16").reshape(B * H, N, d) for n in ("q", "k", "v", "do")}
    rq, rk, rv = oracle.attn_bwd_ref(f["q"], f["k"], f["v"], f["do"], True, sm)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = to_np64(got).reshape(B * H, N, d)
        assert np.isfinite(g).all(), name
        assert cos(g, ref) >= 0.99, (name, cos(g, ref))


def test_autograd_function(sage):
    from bit_quantized_attention_smooth_amd.workloads import make_inputs
    banner("autograd SageAttnFn")
    x = make_inputs(1, 2, 256, 64, dtype="bf16", seed=78, with_do=True)
    g = {n: x[n].to(device()) for n in ("q", "k", "v", "do")}
    q, k, v = (g[n].clone().requires_grad_(True) for n in "qkv")
    out = sage.SageAttnFn.apply(q, k, v, True, 1 / 8)
    out.backward(g["do"])
    _, _, dq, dk, dv = _run(sage, x, True, 1 / 8)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)


@pytest.mark.parametrize("d,causal,dtype", [(64, True, "bf16"), (128, False, "f16"), (128, True, "bf16")])
def test_backward_after_forward_reuses_the_forward_quantization(sage, d, causal, dtype):
    """sage_attn_bwd_after_fwd on the workspace the forward wrote gives the bits of the
    standalone backward (which quantizes Q and K again: the same kernels on the same data)."""
    from bit_quantized_attention_smooth_amd.workloads import make_inputs
    banner(f"backward after forward d={d} causal={causal} {dtype}")
    x = make_inputs(2, 3, 333, d, dtype=dtype, seed=79, k_off_std=2.0, with_do=True)
    g = {n: x[n].to(device()) for n in ("q", "k", "v", "do")}
    sm = 1 / math.sqrt(d)
    ws = sage.bwd_workspace(g["q"], causal=causal, sm_scale=sm)
    o, lse = sage.sageattn(g["q"], g["k"], g["v"], causal=causal, sm_scale=sm, return_lse=True, workspace=ws)
    a = sage.attn_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal, sm_scale=sm, fwd_workspace=ws)
    b = sage.attn_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal, sm_scale=sm)
    torch.cuda.synchronize()
    for ga, gb in zip(a, b):
        assert torch.isfinite(ga).all() and torch.equal(ga, gb)


def test_backward_beyond_2e31_elements_matches_heads_alone(sage):
    """Each tensor holds more than 2^31 elements (B=1, H=128, N=131149 ragged, d=128, causal).
    Heads are independent problems (their own statistics, steps and tiles), so the first and
    the last head must come out bit-identical to the same two heads run alone: every offset
    into the inputs, the workspace and the gradients must be 64-bit."""
    B, H, N, d = 1, 128, 131149, 128
    assert B * H * N * d > 2 ** 31
    banner("backward beyond 2^31 elements")
    sm = 1 / math.sqrt(d)
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(78)
    x = {}
    for n in ("q", "k", "v", "do"):
        t = torch.randn(B, H, N, d, device=dev, generator=gen, dtype=torch.float32)
        if n == "k":
            t += 2.0 * torch.randn(B, H, 1, d, device=dev, generator=gen, dtype=torch.float32)
        x[n] = t.to(torch.bfloat16)
        del t
    heads = [0, H - 1]
    small = {n: x[n][:, heads].contiguous() for n in x}
    big = _run(sage, x, True, sm)
    got = [t[:, heads].contiguous() for t in big]
    del big, x
    torch.cuda.empty_cache()
    want = _run(sage, small, True, sm)
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, want):
        assert torch.isfinite(a).all(), name
        assert torch.equal(a, b), name


@pytest.mark.parametrize("i", range(24))
def test_backward_random_sweep(sage, i):
    """Seeded random configurations (B <= 2, H <= 3, N in [64, 400], d 64 or 128, bf16 or fp16,
    causal or not, K channel offsets or not): every gradient within the backward band of the
    exact fp64 gradients."""
    import oracle
    from bit_quantized_attention_smooth_amd.workloads import make_inputs, as_u16
    rng = np.random.default_rng(3000 + i)
    B, H, N = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(64, 401))
    d, dtype = int(rng.choice([64, 128])), str(rng.choice(["bf16", "f16"]))
    causal, koff = bool(rng.integers(0, 2)), float(rng.choice([0.0, 2.0]))
    sm = 1 / math.sqrt(d)
    banner(f"backward sweep {i}: B={B} H={H} N={N} d={d} {dtype} causal={causal} koff={koff}")
    x = make_inputs(B, H, N, d, dtype=dtype, seed=4000 + i, k_off_std=koff, with_do=True)
    _, _, dq, dk, dv = _run(sage, x, causal, sm)
    f = {n: oracle.widen(as_u16(x[n]), dtype).reshape(B * H, N, d) for n in ("q", "k", "v", "do")}
    rq, rk, rv = oracle.attn_bwd_ref(f["q"], f["k"], f["v"], f["do"], causal, sm)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = to_np64(got).reshape(B * H, N, d)
        assert np.isfinite(g).all(), name
        assert cos(g, ref) >= 0.99, (name, cos(g, ref))
