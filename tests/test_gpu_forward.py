"""GPU parity of the smoothing/quantization prologue and the fused forward
against the CPU oracle: codes and scales bit-exact; O within 2e-2 element-wise
(plus the oracle's slack where a P~ weight has two admissible codes) and cosine
>= 0.9999 of the oracle's simulation of the same quantization; cosine
against exact fp64 attention >= 0.99 (INT8 QK), 0.98 (MXFP4 QK with FP8 P~ and
FP8 or MXFP8 V) or 0.965 (MXFP4 QK and P~V: the oracle's own simulation reaches
about 0.972 on these inputs)."""
import math

import numpy as np
import pytest
import torch

from gpu_util import banner, cos, device, excess, sample_rows, to_np64, unpack_int8_fp8, unpack_mxfp4, within

pytestmark = pytest.mark.gpu

TILE = 64          # the fused kernel's K tile (the simulation must use the same tiling)


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_smooth_amd as S
    S.lib()
    return S


def _inputs(B, H, N, d, dtype, seed, k_off=0.0, outliers=0.0, causal=False):
    from bit_quantized_attention_smooth_amd.workloads import make_inputs, as_u16
    import oracle
    x = make_inputs(B, H, N, d, dtype=dtype, seed=seed, k_off_std=k_off, outlier_frac=outliers)
    f = {n: oracle.widen(as_u16(x[n]), dtype).reshape(B * H, N, d) for n in "qkv"}
    g = {n: x[n].to(device()) for n in "qkv"}
    return f, g


CASES = [
    # name, B, H, N, d, dtype, causal, qk, pv, seed, k_off, outliers, sm
    ("int8_b1h2n256d64_f16", 1, 2, 256, 64, "f16", False, "int8", "fp8", 0, 4.0, 0.0, 1 / 8),
    ("int8_causal_ragged_d128", 1, 3, 1000, 128, "bf16", True, "int8", "fp8", 1, 5.0, 0.01, 1 / math.sqrt(128)),
    ("int8_ragged_d64", 2, 2, 777, 64, "bf16", False, "int8", "fp8", 2, 3.0, 0.0, 1 / 8),
    ("int8_causal_d64_f16", 1, 2, 300, 64, "f16", True, "int8", "fp8", 5, 2.0, 0.0, 1 / 8),
    ("mxfp4_fp8_d128", 1, 3, 600, 128, "bf16", False, "mxfp4", "fp8", 3, 5.0, 0.0, 1 / math.sqrt(128)),
    ("mxfp4_fp8_causal_d64", 1, 2, 333, 64, "bf16", True, "mxfp4", "fp8", 6, 5.0, 0.0, 1 / 8),
    ("mxfp4_mxfp4_d128", 1, 3, 600, 128, "bf16", False, "mxfp4", "mxfp4", 3, 5.0, 0.0, 1 / math.sqrt(128)),
    ("mxfp4_mxfp4_causal_d64", 1, 2, 333, 64, "bf16", True, "mxfp4", "mxfp4", 6, 5.0, 0.0, 1 / 8),
    ("mxfp4_mxfp4_d64_f16", 1, 2, 200, 64, "f16", False, "mxfp4", "mxfp4", 8, 2.0, 0.0, 1 / 8),
    ("mxfp4_mxfp8_d128", 1, 3, 600, 128, "bf16", False, "mxfp4", "mxfp8", 3, 5.0, 0.0, 1 / math.sqrt(128)),
    ("mxfp4_mxfp8_causal_d64", 1, 2, 333, 64, "bf16", True, "mxfp4", "mxfp8", 6, 5.0, 0.0, 1 / 8),
    ("mxfp4_mxfp8_causal_d128_f16", 1, 2, 700, 128, "f16", True, "mxfp4", "mxfp8", 10, 3.0, 0.01,
     1 / math.sqrt(128)),
    ("int8_f16pv_causal_ragged_d128", 1, 3, 1000, 128, "bf16", True, "int8", "f16", 1, 5.0, 0.01,
     1 / math.sqrt(128)),
    ("int8_f16pv_ragged_d64_f16", 2, 2, 777, 64, "f16", False, "int8", "f16", 2, 3.0, 0.0, 1 / 8),
    ("int8tok_causal_ragged_d128", 1, 3, 1000, 128, "bf16", True, "int8_token", "fp8", 1, 5.0, 0.01,
     1 / math.sqrt(128)),
    ("int8tok_f16pv_ragged_d64", 2, 2, 777, 64, "bf16", False, "int8_token", "f16", 2, 3.0, 0.01, 1 / 8),
    ("int8tok_d64_f16", 1, 2, 256, 64, "f16", False, "int8_token", "fp8", 0, 4.0, 0.0, 1 / 8),
    ("mxfp4qb_fp8_d128", 1, 3, 600, 128, "bf16", False, "mxfp4_qblock", "fp8", 3, 5.0, 0.0, 1 / math.sqrt(128)),
    ("mxfp4qb_mxfp4_causal_d64", 1, 2, 333, 64, "bf16", True, "mxfp4_qblock", "mxfp4", 6, 5.0, 0.0, 1 / 8),
    ("mxfp4qb_mxfp8_causal_d128_f16", 1, 2, 700, 128, "f16", True, "mxfp4_qblock", "mxfp8", 10, 3.0, 0.01,
     1 / math.sqrt(128)),
]


def _ref_band(qk, pv):
    """Cosine floor against exact fp64 attention for a format pair."""
    if qk.startswith("int8"):
        return 0.99
    return 0.965 if pv == "mxfp4" else 0.98


def _oracle_quant(f, qk, pv, sm):
    """The oracle's prologue for a format pair (INT8 steps per 64 tokens, or per query token and
    per 32 keys for int8_token)."""
    import oracle
    if qk.startswith("int8"):
        fine = qk == "int8_token"
        return oracle.quant_int8_fp8(f["q"], f["k"], f["v"], sm, pv_fmt=pv, qblk=1 if fine else 64,
                                     kblk=32 if fine else 64)
    return oracle.quant_mxfp4(f["q"], f["k"], f["v"], sm, pv_fmt=pv, qsb=128 if qk == "mxfp4_qblock" else 0)


def _unpack(buf, p, lay, qk, pv):
    if qk.startswith("int8"):
        return unpack_int8_fp8(buf, p, lay, pv, fine=qk == "int8_token")
    return unpack_mxfp4(buf, p, lay, pv, qblock=qk == "mxfp4_qblock")


def _oracle_sim(f, qz_or, qk, pv, N, d, causal, sm, rows=None):
    """The oracle's simulation: (O, LSE, slack), slack bounding the effect of admissible P~ codes."""
    import oracle
    if qk.startswith("int8"):
        return oracle.attn_int8_fp8(qz_or, N, d, causal, sm, TILE, rows=rows, slack=True)
    return oracle.attn_mxfp4(qz_or, N, d, causal, sm, TILE, rows=rows, slack=True)


def _check_codes(r, qz, qk, pv):
    if qk.startswith("int8"):
        assert np.array_equal(r["mu_k"], qz["mu_k"])
        if pv == "f16":
            assert np.array_equal(r["vh"], qz["vh"]) and not r["vh_all"][:, qz["vh"].shape[1]:].any()
        assert np.array_equal(r["qs"], qz["qs"]) and np.array_equal(r["ks"], qz["ks"])
        assert np.array_equal(r["qc"], qz["qc"]) and np.array_equal(r["kc"], qz["kc"])
        assert not r["qc_all"][:, qz["qc"].shape[1]:].any() and not r["kc_all"][:, qz["kc"].shape[1]:].any()
    else:
        assert np.array_equal(r["mu_k"], qz["mu_k"]) and np.array_equal(r["mu_q"], qz["mu_q"])
        assert np.array_equal(r["qe"], qz["qe"]) and np.array_equal(r["ke"], qz["ke"])
        assert np.array_equal(r["qc"], qz["qc"]) and np.array_equal(r["kc"], qz["kc"])
        if qk == "mxfp4_qblock":
            # summed in channel order by chained fp64 MFMAs, as the oracle sums: the same bits
            assert np.array_equal(r["dS"], qz["dS"])
        else:
            # one fp64 sum per key, reduced across lanes in tree order: equal up to the last bit
            assert np.allclose(r["dS"], qz["dS"], rtol=1e-6, atol=1e-6 * np.abs(qz["dS"]).max())
    if pv == "f16":
        pass
    elif pv == "fp8":
        assert np.array_equal(r["vs"], qz["vs"])
        assert np.array_equal(r["vc"], qz["vc"])
    else:
        assert np.array_equal(r["ve"], qz["ve"]) and np.array_equal(r["vc"], qz["vc"])
    if pv == "mxfp8":
        assert not r["vc_all"][:, qz["vc"].shape[1]:].any()      # padding tokens carry zero codes
    assert np.allclose(r["corr"], qz["corr"], rtol=1e-5, atol=1e-5 * (np.abs(qz["corr"]).max() + 1))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prologue_codes_bit_exact(sage, case):
    import oracle
    name, B, H, N, d, dt, causal, qk, pv, seed, koff, outl, sm = case
    banner(f"prologue {name}")
    f, g = _inputs(B, H, N, d, dt, seed, koff, outl)
    buf, p, lay = sage.quantize(g["q"], g["k"], g["v"], causal=causal, sm_scale=sm, qk_fmt=qk, pv_fmt=pv)
    torch.cuda.synchronize()
    r = _unpack(buf, p, lay, qk, pv)
    qz = _oracle_quant(f, qk, pv, sm)
    _check_codes(r, qz, qk, pv)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_matches_oracle(sage, case):
    import oracle
    name, B, H, N, d, dt, causal, qk, pv, seed, koff, outl, sm = case
    banner(f"forward {name}")
    f, g = _inputs(B, H, N, d, dt, seed, koff, outl)
    o, lse = sage.sageattn(g["q"], g["k"], g["v"], causal=causal, sm_scale=sm, qk_fmt=qk, pv_fmt=pv, return_lse=True)
    torch.cuda.synchronize()
    o = to_np64(o).reshape(B * H, N, d)
    lse = lse.cpu().numpy().reshape(B * H, N).astype(np.float64)
    qz = _oracle_quant(f, qk, pv, sm)
    o_sim, lse_sim, sl = _oracle_sim(f, qz, qk, pv, N, d, causal, sm)
    o_ref, lse_ref = oracle.attn_ref(f["q"], f["k"], f["v"], causal, sm)
    assert within(o, o_sim, sl), excess(o, o_sim, sl)
    assert cos(o, o_sim) >= 0.9999
    assert cos(o, o_ref) >= _ref_band(qk, pv)
    assert np.allclose(lse, lse_sim, rtol=1e-4, atol=2e-3)


SWEEP_PAIRS = [("int8", "fp8"), ("int8", "f16"), ("int8_token", "fp8"), ("int8_token", "f16"), ("mxfp4", "fp8"),
               ("mxfp4", "mxfp4"), ("mxfp4", "mxfp8"), ("mxfp4_qblock", "fp8"), ("mxfp4_qblock", "mxfp4"),
               ("mxfp4_qblock", "mxfp8")]


def _sweep_case(i):
    """Configuration i of a seeded random sweep over shapes, dtypes, masks and format pairs."""
    rng = np.random.default_rng(1000 + i)
    qk, pv = SWEEP_PAIRS[i % len(SWEEP_PAIRS)]
    return dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 5)), N=int(rng.integers(1, 701)),
                d=int(rng.choice([64, 128])), dt=str(rng.choice(["bf16", "f16"])), causal=bool(rng.integers(0, 2)),
                qk=qk, pv=pv, koff=float(rng.choice([0.0, 3.0])), sm=float(rng.uniform(0.05, 0.2)))


@pytest.mark.parametrize("i", range(120))
def test_forward_random_sweep(sage, i):
    """Seeded random configurations: codes bit-exact and outputs within the forward tolerances of
    the oracle's simulation."""
    c = _sweep_case(i)
    banner(f"sweep {i}: {c}")
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    f, g = _inputs(B, H, N, d, c["dt"], 2000 + i, c["koff"])
    buf, p, lay = sage.quantize(g["q"], g["k"], g["v"], causal=c["causal"], sm_scale=c["sm"], qk_fmt=c["qk"],
                                pv_fmt=c["pv"])
    o, lse = sage.attn_fwd_quantized(buf, p, dtype=g["q"].dtype, return_lse=True)
    torch.cuda.synchronize()
    qz = _oracle_quant(f, c["qk"], c["pv"], c["sm"])
    _check_codes(_unpack(buf, p, lay, c["qk"], c["pv"]), qz, c["qk"], c["pv"])
    o = to_np64(o).reshape(B * H, N, d)
    o_sim, lse_sim, sl = _oracle_sim(f, qz, c["qk"], c["pv"], N, d, c["causal"], c["sm"])
    assert within(o, o_sim, sl), excess(o, o_sim, sl)
    assert cos(o, o_sim) >= 0.9999
    assert np.allclose(lse.cpu().numpy().reshape(B * H, N), lse_sim, rtol=1e-4, atol=2e-3)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 192])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_edge_lengths(sage, N, causal):
    import oracle
    banner(f"edge N={N} causal={causal}")
    for qk, d, pv in (("int8", 64, "fp8"), ("int8", 128, "fp8"), ("mxfp4", 128, "fp8"), ("mxfp4", 64, "mxfp4"),
                      ("mxfp4", 128, "mxfp8"), ("int8", 128, "f16"), ("int8_token", 128, "fp8"),
                      ("int8_token", 64, "f16"), ("mxfp4_qblock", 128, "fp8")):
        f, g = _inputs(1, 2, N, d, "bf16", 100 + N, 2.0)
        sm = 1 / math.sqrt(d)
        o, lse = sage.sageattn(g["q"], g["k"], g["v"], causal=causal, sm_scale=sm, qk_fmt=qk, pv_fmt=pv,
                               return_lse=True)
        torch.cuda.synchronize()
        o = to_np64(o).reshape(2, N, d)
        qz = _oracle_quant(f, qk, pv, sm)
        o_sim, lse_sim, sl = _oracle_sim(f, qz, qk, pv, N, d, causal, sm)
        assert within(o, o_sim, sl), (qk, d, pv, excess(o, o_sim, sl))
        if N > 1:
            assert cos(o, o_sim) >= 0.9999, (qk, d, pv)
        else:
            # one key: O is the dequantized V row
            assert within(o, o_sim, sl)
        assert np.allclose(lse.cpu().numpy().reshape(2, N), lse_sim, rtol=1e-4, atol=2e-3)


ZERO_PAIRS = [("int8", "fp8"), ("int8", "f16"), ("int8_token", "fp8"), ("mxfp4", "fp8"), ("mxfp4", "mxfp4"),
              ("mxfp4", "mxfp8"), ("mxfp4_qblock", "fp8")]


@pytest.mark.parametrize("qk,pv", ZERO_PAIRS, ids=[f"{a}_{b}" for a, b in ZERO_PAIRS])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_zero_inputs(sage, qk, pv, causal):
    """Degenerate inputs: an all-zero Q or K has zero quantization steps, so every score is 0
    and the weights are uniform (O is the (prefix) mean of the dequantized V); an all-zero V
    gives O = 0.  Everything stays finite and matches the oracle's simulation."""
    banner(f"zero inputs {qk}/{pv} causal={causal}")
    B, H, N, d = 1, 2, 200, 64
    sm = 1 / 8
    for zero in "qkv":
        f, g = _inputs(B, H, N, d, "bf16", 31, 2.0)
        g[zero] = torch.zeros_like(g[zero])
        f[zero] = np.zeros_like(f[zero])
        o, lse = sage.sageattn(g["q"], g["k"], g["v"], causal=causal, sm_scale=sm, qk_fmt=qk, pv_fmt=pv,
                               return_lse=True)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all(), zero
        o = to_np64(o).reshape(B * H, N, d)
        qz = _oracle_quant(f, qk, pv, sm)
        o_sim, lse_sim, sl = _oracle_sim(f, qz, qk, pv, N, d, causal, sm)
        assert within(o, o_sim, sl), (zero, excess(o, o_sim, sl))
        assert np.allclose(lse.cpu().numpy().reshape(B * H, N), lse_sim, rtol=1e-4, atol=2e-3), zero
        if zero == "v":
            assert not o.any()


@pytest.mark.parametrize("qk,pv", SWEEP_PAIRS, ids=[f"{a}_{b}" for a, b in SWEEP_PAIRS])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_tiny_magnitude_inputs(sage, qk, pv, causal):
    """Q and K with block maxima near 1e-21 (bf16 holds them; their codes are ordinary).  The
    scores are below 1e-40, so exact attention is uniform: O is the (prefix) mean of V.  The
    product of the two steps underflows binary32, which must not turn the integer code dot
    products into log2-domain scores (that gives one-hot weights): every format pair must stay
    within the forward tolerances of the oracle and at cosine >= 0.99 of exact attention."""
    import oracle
    banner(f"tiny-magnitude inputs {qk}/{pv} causal={causal}")
    B, H, N, d = 1, 2, 300, 128
    sm = 1 / math.sqrt(d)
    f, g = _inputs(B, H, N, d, "bf16", 51, 2.0)
    for n in "qk":
        g[n] = (g[n].float() * 1e-21).to(torch.bfloat16)
        f[n] = g[n].float().cpu().numpy().reshape(B * H, N, d)
    assert 1e-22 < float(np.abs(f["q"]).max()) < 1e-19 and 1e-22 < float(np.abs(f["k"]).max()) < 1e-19
    o, lse = sage.sageattn(g["q"], g["k"], g["v"], causal=causal, sm_scale=sm, qk_fmt=qk, pv_fmt=pv,
                           return_lse=True)
    torch.cuda.synchronize()
    o = to_np64(o).reshape(B * H, N, d)
    qz = _oracle_quant(f, qk, pv, sm)
    o_sim, lse_sim, sl = _oracle_sim(f, qz, qk, pv, N, d, causal, sm)
    o_ref, lse_ref = oracle.attn_ref(f["q"], f["k"], f["v"], causal, sm)
    assert within(o, o_sim, sl), excess(o, o_sim, sl)
    assert cos(o, o_sim) >= 0.9999
    assert cos(o, o_ref) >= 0.99, cos(o, o_ref)
    assert np.allclose(lse.cpu().numpy().reshape(B * H, N), lse_ref, rtol=1e-4, atol=2e-3)


# (tensor, head, row, channel, value): a NaN in Q, a NaN in K (it reaches the K mean, so the
# whole head), an Inf in V (it reaches the channel's step or MX scale)
NONFINITE = [("q", 0, 70, 5, float("nan")), ("k", 1, 10, 3, float("nan")), ("v", 0, 33, 7, float("inf")),
             ("q", 1, 150, 60, float("inf"))]


@pytest.mark.parametrize("qk,pv", ZERO_PAIRS, ids=[f"{a}_{b}" for a, b in ZERO_PAIRS])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_nonfinite_inputs(sage, qk, pv, causal):
    """NaN or Inf inputs are not errors: they propagate into the scales and rows they reach.
    The GPU and the oracle's simulation must agree on which outputs (O and LSE) are not finite,
    the injected element must reach its own output row, and the finite outputs must match."""
    banner(f"non-finite inputs {qk}/{pv} causal={causal}")
    B, H, N, d = 1, 2, 200, 64
    sm = 1 / 8
    for t, h, row, ch, val in NONFINITE:
        f, g = _inputs(B, H, N, d, "bf16", 41, 2.0)
        g[t][0, h, row, ch] = val
        f[t][h, row, ch] = val
        o, lse = sage.sageattn(g["q"], g["k"], g["v"], causal=causal, sm_scale=sm, qk_fmt=qk, pv_fmt=pv,
                               return_lse=True)
        torch.cuda.synchronize()
        o = to_np64(o).reshape(B * H, N, d)
        lse = lse.cpu().numpy().reshape(B * H, N).astype(np.float64)
        with np.errstate(invalid="ignore", over="ignore"):
            qz = _oracle_quant(f, qk, pv, sm)
            o_sim, lse_sim, sl = _oracle_sim(f, qz, qk, pv, N, d, causal, sm)
        bad, bad_sim = ~np.isfinite(o), ~np.isfinite(o_sim)
        assert np.array_equal(bad, bad_sim), (t, int(bad.sum()), int(bad_sim.sum()))
        assert np.array_equal(~np.isfinite(lse), ~np.isfinite(np.asarray(lse_sim, np.float64))), t
        assert bad[h, row].any() if t != "v" else bad[h, row:, ch].all(), t
        ok = ~bad
        assert within(o[ok], o_sim[ok], sl[ok]), t
        okl = np.isfinite(lse)
        assert np.allclose(lse[okl], np.asarray(lse_sim)[okl], rtol=1e-4, atol=2e-3), t


@pytest.mark.parametrize("qk", ["int8", "mxfp4"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_constant_keys_closed_form(sage, qk, causal):
    """K constant along tokens: every score is 0, so O_i is the mean (prefix mean if
    causal) of the FP8-dequantized V rows -- exact up to the output rounding."""
    import oracle
    banner(f"constant keys {qk} causal={causal}")
    B, H, N, d = 1, 2, 200, 128
    f, g = _inputs(B, H, N, d, "bf16", 7)
    g["k"] = g["k"][:, :, :1].expand(-1, -1, N, -1).contiguous()
    f["k"] = np.repeat(f["k"][:, :1], N, axis=1)
    o = sage.sageattn(g["q"], g["k"], g["v"], causal=causal, qk_fmt=qk)
    torch.cuda.synchronize()
    o = to_np64(o).reshape(B * H, N, d)
    qz = oracle.quant_int8_fp8(f["q"], f["k"], f["v"], 0.1)
    vdq = oracle.e4m3_decode(qz["vc"]) * qz["vs"][:, None, :].astype(np.float64)
    want = np.cumsum(vdq, axis=1) / np.arange(1, N + 1)[None, :, None] if causal else \
        np.broadcast_to(vdq.mean(axis=1, keepdims=True), vdq.shape)
    # bf16 output rounding: half an ulp of |O| <= 2^-9 relative
    assert np.all(np.abs(o - want) <= np.abs(want) * 2.0 ** -8 + 1e-6)


@pytest.mark.parametrize("pv", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_constant_keys_mx_pv(sage, causal, pv):
    """MXFP4 QK with MX V and K constant along tokens: every p is 1.  MXFP4 P~: sigma = 6/max p
    = 6 and each P~ element is exactly E2M1 6 with block scale 2^0.  MXFP8 V: each P~ element
    is exactly E4M3 448.  O_i is then the (prefix) mean of the MX-dequantized V rows, exact up
    to fp32 accumulation and the output rounding."""
    import oracle
    banner(f"constant keys {pv} V causal={causal}")
    B, H, N, d = 1, 2, 200, 128
    f, g = _inputs(B, H, N, d, "bf16", 9)
    g["k"] = g["k"][:, :, :1].expand(-1, -1, N, -1).contiguous()
    f["k"] = np.repeat(f["k"][:, :1], N, axis=1)
    o = sage.sageattn(g["q"], g["k"], g["v"], causal=causal, qk_fmt="mxfp4", pv_fmt=pv)
    torch.cuda.synchronize()
    o = to_np64(o).reshape(B * H, N, d)
    qz = oracle.quant_mxfp4(f["q"], f["k"], f["v"], 0.1, pv_fmt=pv)
    ve = np.repeat(qz["ve"].astype(np.int64), 32, axis=1)[:, :N]            # [BH, N, d] E8M0 bytes
    dec = oracle.e2m1_decode if pv == "mxfp4" else oracle.e4m3_decode
    vdq = dec(qz["vc"]) * np.ldexp(1.0, ve - 127)
    want = np.cumsum(vdq, axis=1) / np.arange(1, N + 1)[None, :, None] if causal else \
        np.broadcast_to(vdq.mean(axis=1, keepdims=True), vdq.shape)
    assert np.all(np.abs(o - want) <= np.abs(want) * 2.0 ** -8 + 1e-5 * np.abs(vdq).max())


def test_forward_constant_keys_f16_pv(sage):
    """INT8 QK with the 16-bit P~V fallback and K constant along tokens: every p is 1 and
    P~ = fp16(1) = 1 exactly, so O_i is the (prefix) mean of the fp16-rounded V rows."""
    import oracle
    for causal in (False, True):
        banner(f"constant keys f16 P~V causal={causal}")
        B, H, N, d = 1, 2, 200, 128
        f, g = _inputs(B, H, N, d, "bf16", 13)
        g["k"] = g["k"][:, :, :1].expand(-1, -1, N, -1).contiguous()
        f["k"] = np.repeat(f["k"][:, :1], N, axis=1)
        o = sage.sageattn(g["q"], g["k"], g["v"], causal=causal, qk_fmt="int8", pv_fmt="f16")
        torch.cuda.synchronize()
        o = to_np64(o).reshape(B * H, N, d)
        vdq = f["v"].astype(np.float16).astype(np.float64)
        want = np.cumsum(vdq, axis=1) / np.arange(1, N + 1)[None, :, None] if causal else \
            np.broadcast_to(vdq.mean(axis=1, keepdims=True), vdq.shape)
        assert np.all(np.abs(o - want) <= np.abs(want) * 2.0 ** -8 + 1e-5 * np.abs(vdq).max())


@pytest.mark.parametrize("pv", ["fp8", "mxfp4"])
def test_forward_block_q_smoothing_under_drift(sage, pv):
    """Q with channel offsets that drift along the sequence: the per-block smoothing path matches
    the oracle and is closer to exact attention than smoothing over the whole sequence."""
    import oracle
    banner(f"block Q smoothing drift {pv}")
    B, H, N, d = 1, 2, 1000, 128
    g0 = torch.Generator().manual_seed(31)
    q = torch.randn(B, H, N, d, generator=g0) + torch.linspace(-1, 1, N)[None, None, :, None] * \
        6 * torch.randn(B, H, 1, d, generator=g0)
    k = torch.randn(B, H, N, d, generator=g0) + 4 * torch.randn(B, H, 1, d, generator=g0)
    v = torch.randn(B, H, N, d, generator=g0)
    x = {n: t.to(torch.bfloat16) for n, t in zip("qkv", (q, k, v))}
    f = {n: x[n].float().numpy().reshape(B * H, N, d) for n in "qkv"}
    sm = 1 / math.sqrt(d)
    o_ref, _ = oracle.attn_ref(f["q"], f["k"], f["v"], False, sm)
    cs = {}
    for qk in ("mxfp4", "mxfp4_qblock"):
        o = sage.sageattn(*(x[n].to(device()) for n in "qkv"), sm_scale=sm, qk_fmt=qk, pv_fmt=pv)
        torch.cuda.synchronize()
        o = to_np64(o).reshape(B * H, N, d)
        o_sim, _, sl = _oracle_sim(f, _oracle_quant(f, qk, pv, sm), qk, pv, N, d, False, sm)
        assert within(o, o_sim, sl) and cos(o, o_sim) >= 0.9999, qk
        cs[qk] = cos(o, o_ref)
    assert cs["mxfp4_qblock"] > cs["mxfp4"]


# (workload, P~V format, QK format or None for the workload's own, heads compared): "all" compares
# every row of every head; an integer n compares every row of n heads spread over the batch; "rows"
# compares sampled rows of three heads.
FULL = [("int8_fp8_b1h2n256d64", "fp8", None, "all"),
        ("int8_fp8_causal_b1h32n4096d128", "fp8", None, "all"),
        ("train_causal_b8h16n2048d64", "fp8", None, "all"),
        ("int8_fp8_b2h24n16384d64", "fp8", None, 4),
        ("mxfp4_b4h32n8192d128", "fp8", None, 4),
        ("mxfp4_b4h32n8192d128", "mxfp4", None, 4),
        ("mxfp4_b4h32n8192d128", "mxfp8", None, "rows"),
        ("mxfp4_b4h32n8192d128", "fp8", "mxfp4_qblock", "rows"),
        ("int8_fp8_causal_b1h32n4096d128", "fp8", "int8_token", "all"),
        ("int8_fp8_b1h32n8192d128", "f16", None, "rows"),
        ("int8_fp8_b1h32n8192d128", "fp8", None, 4),
        ("int8_fp8_causal_b1h32n16384d128", "fp8", None, "rows")]


def _full_id(c):
    return "-".join(str(t) for t in (c[0], c[2] or "", c[1], c[3]) if t != "")


@pytest.mark.parametrize("spec", FULL, ids=[_full_id(c) for c in FULL])
def test_full_size_parity(sage, spec):
    """The named workloads at full size in the benchmark's launch configuration.  The oracle
    recomputes every row of every head (the small and training workloads and the causal
    prefill), every row of four heads spread over the batch (the long workloads), or sampled
    rows of three heads (the remaining format variants); codes, O and LSE are compared on all
    of them, O per element with the admissible-code slack and by cosine, and the cosine against
    exact attention per head."""
    import oracle
    from bit_quantized_attention_smooth_amd.workloads import workload_inputs, as_u16
    name, pv, qk_over, which = spec
    banner(f"full size {spec}")
    x, w = workload_inputs(name)
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    qk, sm, causal = (qk_over or w["qk_fmt"]), w["sm_scale"], w["causal"]
    g = {n: x[n].to(device()) for n in "qkv"}
    buf, p, lay = sage.quantize(g["q"], g["k"], g["v"], causal=causal, sm_scale=sm, qk_fmt=qk, pv_fmt=pv)
    o, lse = sage.attn_fwd_quantized(buf, p, dtype=g["q"].dtype, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()                # every output finite at full size
    BH = B * H
    if which == "all":
        heads = list(range(BH))
    elif which == "rows":
        heads = sorted({0, BH // 2, BH - 1})
    else:
        heads = sorted({round(i * (BH - 1) / (which - 1)) for i in range(which)})
    rows = sample_rows(N) if which == "rows" else None
    sel = lambda t: t.reshape(BH, N, d)[heads]
    f = {n: oracle.widen(as_u16(sel(x[n])), w["dtype"]).reshape(len(heads), N, d) for n in "qkv"}
    qz = _oracle_quant(f, qk, pv, sm)
    r = _unpack(buf, p, lay, qk, pv)
    if qk.startswith("int8"):
        for key in ("qc", "kc", "qs", "ks", "mu_k") + (("vh",) if pv == "f16" else ("vc", "vs")):
            assert np.array_equal(r[key][heads], qz[key]), key
    else:
        for key in ("qc", "kc", "qe", "ke", "vc", "vs" if pv == "fp8" else "ve", "mu_k", "mu_q"):
            assert np.array_equal(r[key][heads], qz[key]), key
    o_sim, lse_sim, sl = _oracle_sim(f, qz, qk, pv, N, d, causal, sm, rows=rows)
    o_ref, _ = oracle.attn_ref(f["q"], f["k"], f["v"], causal, sm, rows=rows)
    og = to_np64(o).reshape(BH, N, d)[heads]
    lg = lse.cpu().numpy().reshape(BH, N)[heads]
    if rows is not None:
        og, lg = og[:, rows], lg[:, rows]
    assert within(og, o_sim, sl), excess(og, o_sim, sl)
    assert cos(og, o_sim) >= 0.9999
    assert np.allclose(lg, lse_sim, rtol=1e-4, atol=2e-3)
    band = _ref_band(qk, pv)
    per_head = [cos(og[i], o_ref[i]) for i in range(len(heads))]
    assert min(per_head) >= band, (min(per_head), int(np.argmin(per_head)))


@pytest.mark.parametrize("qk", ["int8", "mxfp4"])
def test_forward_beyond_2e31_elements(sage, qk):
    """Each input holds more than 2^31 elements (B=1, H=128, N=131149 ragged, d=128, causal):
    every offset into the inputs, the quantized buffer and the output must be 64-bit.  The
    oracle recomputes sampled rows of the first and the last head."""
    import oracle
    B, H, N, d = 1, 128, 131149, 128
    assert B * H * N * d > 2 ** 31
    banner(f"beyond 2^31 elements {qk}")
    sm = 1 / math.sqrt(d)
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(77)
    q = torch.randn(B, H, N, d, device=dev, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    k = (torch.randn(B, H, N, d, device=dev, generator=gen, dtype=torch.float32) +
         3.0 * torch.randn(B, H, 1, d, device=dev, generator=gen, dtype=torch.float32)).to(torch.bfloat16)
    v = torch.randn(B, H, N, d, device=dev, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    o, lse = sage.sageattn(q, k, v, causal=True, sm_scale=sm, qk_fmt=qk, pv_fmt="fp8", return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    heads = [0, H - 1]
    f = {n: t[0, heads].float().cpu().numpy() for n, t in (("q", q), ("k", k), ("v", v))}
    del q, k, v
    rows = sample_rows(N, k=12, seed=3)
    qz = _oracle_quant(f, qk, "fp8", sm)
    o_sim, lse_sim, sl = _oracle_sim(f, qz, qk, "fp8", N, d, True, sm, rows=rows)
    ri = torch.as_tensor(rows, dtype=torch.long, device=dev)
    og = to_np64(o[0, heads][:, ri])
    lg = lse[0, heads][:, ri].cpu().numpy()
    assert within(og, o_sim, sl), excess(og, o_sim, sl)
    assert cos(og, o_sim) >= 0.9999
    assert np.allclose(lg, lse_sim, rtol=1e-4, atol=2e-3)


def test_oneshot_entry_matches_ex(sage):
    banner("one-call entry vs workspace entry")
    f, g = _inputs(1, 4, 512, 128, "bf16", 11, 5.0)
    a = sage.attn_fwd_oneshot(g["q"], g["k"], g["v"], causal=True)
    b = sage.sageattn(g["q"], g["k"], g["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_caller_workspace_is_used_as_given_or_refused(sage):
    """sageattn(..., workspace=) writes the quantization into the caller's buffer (a training step
    reads it back); a buffer of the wrong dtype, on the host, or too small raises instead of being
    replaced by a fresh one, and a large enough one gives the same output as a fresh buffer."""
    banner("caller workspace")
    _, g = _inputs(1, 2, 256, 64, "bf16", 12, 3.0)
    want = sage.sageattn(g["q"], g["k"], g["v"], causal=True)
    ws = sage.bwd_workspace(g["q"], causal=True)
    got = sage.sageattn(g["q"], g["k"], g["v"], causal=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    for bad in (ws[:64], ws.view(torch.int32) if ws.numel() % 4 == 0 else ws.float(), ws.cpu()):
        with pytest.raises(ValueError, match="workspace"):
            sage.sageattn(g["q"], g["k"], g["v"], causal=True, workspace=bad)


def test_named_fp16_pv_entry_is_the_f16_format(sage):
    """sageattn_qk_int8_pv_fp16 (the entry name the code-link page lists) is the INT8 QK / fp16
    P~V pair, bit for bit."""
    banner("named fp16 P~V entry")
    _, g = _inputs(1, 2, 300, 128, "bf16", seed=77, k_off=2.0)
    a = sage.sageattn_qk_int8_pv_fp16(g["q"], g["k"], g["v"], causal=True, return_lse=True)
    b = sage.sageattn(g["q"], g["k"], g["v"], causal=True, qk_fmt="int8", pv_fmt="f16", return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("qk,pv", [("int8", "fp8"), ("mxfp4", "fp8"), ("int8", "f16")])
def test_sageattn_layouts_grouped_heads_and_cross_lengths(sage, qk, pv):
    """sageattn with tensor_layout "NHD" gives the "HND" bits (same rows, permuted); grouped KV
    heads give the bits of the same call with each KV head repeated; N_q != N_k matches the
    oracle's per-sequence simulation (causal top-left aligned)."""
    import oracle
    banner(f"sageattn layouts / GQA / cross lengths {qk}/{pv}")
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(81)
    B, H, Hkv, d = 2, 6, 2, 128
    q = torch.randn(B, H, 300, d, device=dev, generator=gen).to(torch.bfloat16)
    k = (torch.randn(B, Hkv, 300, d, device=dev, generator=gen) + 2.0).to(torch.bfloat16)
    v = torch.randn(B, Hkv, 300, d, device=dev, generator=gen).to(torch.bfloat16)
    kr, vr = (t.repeat_interleave(H // Hkv, dim=1).contiguous() for t in (k, v))
    for causal in (False, True):
        a = sage.sageattn(q, kr, vr, causal=causal, qk_fmt=qk, pv_fmt=pv, return_lse=True)   # plain entry
        b = sage.sageattn(q, k, v, causal=causal, qk_fmt=qk, pv_fmt=pv, return_lse=True)     # grouped heads
        nhd = [t.permute(0, 2, 1, 3).contiguous() for t in (q, kr, vr)]
        c = sage.sageattn(*nhd, causal=causal, qk_fmt=qk, pv_fmt=pv, return_lse=True, tensor_layout="NHD")
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        assert torch.equal(c[0].permute(0, 2, 1, 3), a[0]) and torch.equal(c[1], a[1])
    # cross lengths: 300 queries against 450 keys
    k2 = (torch.randn(B, Hkv, 450, d, device=dev, generator=gen) + 2.0).to(torch.bfloat16)
    v2 = torch.randn(B, Hkv, 450, d, device=dev, generator=gen).to(torch.bfloat16)
    sm = 1 / math.sqrt(d)
    for causal in (False, True):
        o, lse = sage.sageattn(q, k2, v2, causal=causal, sm_scale=sm, qk_fmt=qk, pv_fmt=pv, return_lse=True)
        torch.cuda.synchronize()
        rows = [t.permute(0, 2, 1, 3).reshape(-1, t.shape[1], d).float().cpu().numpy() for t in (q, k2, v2)]
        cq, ck = np.array([0, 300, 600], np.int32), np.array([0, 450, 900], np.int32)
        o_sim, lse_sim, _, sl = oracle.attn_varlen(*rows, cq, ck, causal, sm, qk_fmt=qk, pv_fmt=pv, tile=TILE,
                                                   slack=True)
        og = to_np64(o.permute(0, 2, 1, 3).reshape(-1, H, d))
        assert within(og, o_sim, sl), excess(og, o_sim, sl)
        assert cos(og, o_sim) >= 0.9999
        assert np.allclose(lse.permute(1, 0, 2).reshape(H, -1).cpu().numpy(), lse_sim, rtol=1e-4, atol=2e-3)
