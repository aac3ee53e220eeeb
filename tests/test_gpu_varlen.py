"""GPU parity of the packed-sequence entry (cu_seqlens, grouped KV heads) against the CPU
oracle's per-sequence simulation, plus two properties that hold bit for bit at any size:
equal-length packed sequences reproduce the fixed-length path, and grouped KV heads reproduce
the same call with every KV head repeated for its query heads."""
import math

import numpy as np
import pytest
import torch

from gpu_util import banner, cos, device, excess, to_np64, within

pytestmark = pytest.mark.gpu

TILE = 64


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_smooth_amd as S
    S.lib()
    return S


def _packed(lens_q, lens_k, H, Hkv, d, seed, dtype=torch.bfloat16, k_off=3.0):
    g = torch.Generator().manual_seed(seed)
    cu_q = torch.tensor([0] + list(np.cumsum(lens_q)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(lens_k)), dtype=torch.int32)
    q = torch.randn(int(cu_q[-1]), H, d, generator=g).to(dtype)
    k = (torch.randn(int(cu_k[-1]), Hkv, d, generator=g) + k_off * torch.randn(1, Hkv, d, generator=g)).to(dtype)
    v = torch.randn(int(cu_k[-1]), Hkv, d, generator=g).to(dtype)
    return q, k, v, cu_q, cu_k


def _run(sage, q, k, v, cu_q, cu_k, causal, sm, qk, pv, max_q=None, max_k=None):
    dev = device()
    lq = (cu_q[1:] - cu_q[:-1]).tolist()
    lk = (cu_k[1:] - cu_k[:-1]).tolist()
    o, lse = sage.sageattn_varlen(q.to(dev), k.to(dev), v.to(dev), cu_q.to(dev), cu_k.to(dev),
                                  max(lq) if max_q is None else max_q, max(lk) if max_k is None else max_k,
                                  causal=causal, sm_scale=sm, qk_fmt=qk, pv_fmt=pv, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def _f32(t):
    return t.float().numpy()


PAIRS = [("int8", "fp8"), ("int8", "f16"), ("int8_token", "fp8"), ("int8_token", "f16"), ("mxfp4", "fp8"),
         ("mxfp4", "mxfp4"), ("mxfp4", "mxfp8"), ("mxfp4_qblock", "fp8"), ("mxfp4_qblock", "mxfp4"),
         ("mxfp4_qblock", "mxfp8")]


@pytest.mark.parametrize("qk,pv", PAIRS, ids=[f"{a}_{b}" for a, b in PAIRS])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_gqa_matches_oracle(sage, qk, pv, causal, d):
    import oracle
    banner(f"varlen {qk}/{pv} causal={causal} d={d}")
    # ragged lengths: a 1-token sequence, lengths across tile and block edges, unequal q / k
    lens_q = [1, 129, 300, 64, 77]
    lens_k = [1, 129, 300, 200, 33] if not causal else lens_q
    H, Hkv = 6, 2
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, H, Hkv, d, seed=10 + d + 2 * causal)
    sm = 1 / math.sqrt(d)
    o, lse = _run(sage, q, k, v, cu_q, cu_k, causal, sm, qk, pv)
    o_sim, lse_sim, _, sl = oracle.attn_varlen(_f32(q), _f32(k), _f32(v), cu_q.numpy(), cu_k.numpy(), causal, sm,
                                               qk_fmt=qk, pv_fmt=pv, tile=TILE, slack=True)
    o_ref, _, _ = oracle.attn_varlen(_f32(q), _f32(k), _f32(v), cu_q.numpy(), cu_k.numpy(), causal, sm, exact=True)
    og = to_np64(o)
    assert within(og, o_sim, sl), excess(og, o_sim, sl)
    assert cos(og, o_sim) >= 0.9999
    assert cos(og, o_ref) >= (0.99 if qk.startswith("int8") else 0.965 if pv == "mxfp4" else 0.98)
    assert np.allclose(lse.cpu().numpy(), lse_sim, rtol=1e-4, atol=2e-3)


@pytest.mark.parametrize("qk,pv", PAIRS, ids=[f"{a}_{b}" for a, b in PAIRS])
def test_varlen_f16_io_matches_oracle(sage, qk, pv):
    """fp16 inputs and outputs on the packed path (ragged lengths, grouped KV heads, causal)."""
    import oracle
    banner(f"varlen f16 I/O {qk}/{pv}")
    lens = [200, 1, 130, 64]
    H, Hkv, d = 4, 2, 64
    q, k, v, cu_q, cu_k = _packed(lens, lens, H, Hkv, d, seed=33, dtype=torch.float16)
    o, lse = _run(sage, q, k, v, cu_q, cu_k, True, 0.125, qk, pv)
    assert o.dtype == torch.float16
    o_sim, lse_sim, _, sl = oracle.attn_varlen(_f32(q), _f32(k), _f32(v), cu_q.numpy(), cu_k.numpy(), True, 0.125,
                                               qk_fmt=qk, pv_fmt=pv, tile=TILE, slack=True)
    og = to_np64(o)
    assert within(og, o_sim, sl), excess(og, o_sim, sl)
    assert cos(og, o_sim) >= 0.9999
    assert np.allclose(lse.cpu().numpy(), lse_sim, rtol=1e-4, atol=2e-3)


@pytest.mark.parametrize("pv", ["fp8", "mxfp4", "mxfp8"])
def test_varlen_mxfp4_keys_longer_than_queries(sage, pv):
    """MXFP4 QK without grouped heads, key sequences longer than their query sequences by more
    than a 128-token tile: the dS of keys past the last query block must still use mu_q."""
    import oracle
    banner(f"varlen mxfp4/{pv} long keys")
    lens_q, lens_k = [40, 130, 1], [400, 300, 260]
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, 4, 4, 128, seed=21)
    q = (q.float() + 2.0 * torch.randn(1, 4, 128, generator=torch.Generator().manual_seed(22))).to(q.dtype)
    o, lse = _run(sage, q, k, v, cu_q, cu_k, False, 0.09, "mxfp4", pv)
    o_sim, lse_sim, _, sl = oracle.attn_varlen(_f32(q), _f32(k), _f32(v), cu_q.numpy(), cu_k.numpy(), False, 0.09,
                                               qk_fmt="mxfp4", pv_fmt=pv, tile=TILE, slack=True)
    og = to_np64(o)
    assert within(og, o_sim, sl), excess(og, o_sim, sl)
    assert cos(og, o_sim) >= 0.9999
    assert np.allclose(lse.cpu().numpy(), lse_sim, rtol=1e-4, atol=2e-3)


@pytest.mark.parametrize("pv", ["fp8", "mxfp4", "mxfp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_qblock_drifting_queries(sage, pv, causal):
    """Per-block Q smoothing on packed sequences: queries whose mean drifts along each sequence
    (so the 128-query block means differ), sequences that start off the 128-row grid and span
    several blocks, a partial last block, a 1-token sequence, keys longer and shorter than the
    queries (non-causal), grouped KV heads; against the oracle's per-sequence simulation with
    blocks counted from each sequence's first query, and against fp64 attention."""
    import oracle
    banner(f"varlen qblock drift {pv} causal={causal}")
    lens_q = [300, 1, 129, 513, 77]
    lens_k = lens_q if causal else [700, 40, 129, 200, 300]
    H, Hkv, d = 6, 2, 128
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, H, Hkv, d, seed=41)
    g = torch.Generator().manual_seed(42)
    direction = torch.randn(1, H, d, generator=g)
    t = torch.cat([torch.arange(n, dtype=torch.float32) for n in lens_q])
    q = (q.float() + 2.5 * torch.sin(t / 90.0)[:, None, None] * direction).to(q.dtype)
    sm = 1 / math.sqrt(d)
    o, lse = _run(sage, q, k, v, cu_q, cu_k, causal, sm, "mxfp4_qblock", pv)
    o_sim, lse_sim, _, sl = oracle.attn_varlen(_f32(q), _f32(k), _f32(v), cu_q.numpy(), cu_k.numpy(), causal, sm,
                                               qk_fmt="mxfp4_qblock", pv_fmt=pv, tile=TILE, slack=True)
    o_ref, _, _ = oracle.attn_varlen(_f32(q), _f32(k), _f32(v), cu_q.numpy(), cu_k.numpy(), causal, sm, exact=True)
    og = to_np64(o)
    assert within(og, o_sim, sl), excess(og, o_sim, sl)
    assert cos(og, o_sim) >= 0.9999
    assert cos(og, o_ref) >= (0.965 if pv == "mxfp4" else 0.98)
    assert np.allclose(lse.cpu().numpy(), lse_sim, rtol=1e-4, atol=2e-3)


def test_varlen_empty_sequences(sage):
    """Empty query sequences write nothing; a query sequence with no keys gets zero output
    and LSE -inf; the neighbours are unaffected."""
    import oracle
    banner("varlen empty sequences")
    lens_q, lens_k = [3, 0, 70, 5], [40, 8, 0, 66]
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, 4, 4, 64, seed=3)
    for qk, pv in PAIRS:
        o, lse = _run(sage, q, k, v, cu_q, cu_k, False, 0.125, qk, pv)
        og, lg = to_np64(o), lse.cpu().numpy()
        assert np.all(og[3:73] == 0.0) and np.all(np.isneginf(lg[:, 3:73])), (qk, pv)
        o_sim, lse_sim, _, sl = oracle.attn_varlen(_f32(q), _f32(k), _f32(v), cu_q.numpy(), cu_k.numpy(), False, 0.125,
                                                   qk_fmt=qk, pv_fmt=pv, slack=True)
        keep = np.r_[0:3, 73:78]
        assert within(og[keep], o_sim[keep], sl[keep])
        assert np.allclose(lg[:, keep], lse_sim[:, keep], rtol=1e-4, atol=2e-3)


@pytest.mark.parametrize("qk,pv", PAIRS, ids=[f"{a}_{b}" for a, b in PAIRS])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_equal_length_packed_equals_fixed_length(sage, qk, pv, dtype):
    """B sequences of one length N, H_kv = H: the packed entry computes exactly what the
    [B,H,N,d] entry does (same per-instance quantization and kernels), bit for bit."""
    banner(f"packed == fixed {qk}/{pv} {dtype}")
    B, H, N, d = 3, 4, 333, 128
    dev = device()
    g = torch.Generator().manual_seed(5)
    x = {n: torch.randn(B, H, N, d, generator=g).to(dtype).to(dev) for n in "qkv"}
    for causal in (False, True):
        of, lf = sage.sageattn(x["q"], x["k"], x["v"], causal=causal, qk_fmt=qk, pv_fmt=pv, return_lse=True)
        pk = {n: x[n].permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous() for n in "qkv"}
        cu = torch.arange(0, B * N + 1, N, dtype=torch.int32, device=dev)
        ov, lv = sage.sageattn_varlen(pk["q"], pk["k"], pk["v"], cu, cu, N, N, causal=causal, qk_fmt=qk, pv_fmt=pv,
                                      return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(ov.reshape(B, N, H, d).permute(0, 2, 1, 3), of)
        assert torch.equal(lv.reshape(H, B, N).permute(1, 0, 2), lf)


@pytest.mark.parametrize("qk,pv", PAIRS, ids=[f"{a}_{b}" for a, b in PAIRS])
def test_gqa_equals_repeated_kv_heads(sage, qk, pv):
    """Grouped KV heads give the same bits as the same call with each KV head repeated for
    its query heads (the per-instance prologue sees identical data either way)."""
    banner(f"gqa == repeated kv {qk}/{pv}")
    lens = [500, 3, 129, 1024]
    H, Hkv, d = 8, 2, 128
    q, k, v, cu_q, cu_k = _packed(lens, lens, H, Hkv, d, seed=9)
    kr, vr = (t.repeat_interleave(H // Hkv, dim=1).contiguous() for t in (k, v))
    for causal in (False, True):
        a = _run(sage, q, k, v, cu_q, cu_k, causal, 0.09, qk, pv)
        b = _run(sage, q, kr, vr, cu_q, cu_k, causal, 0.09, qk, pv)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_loose_max_seqlen_bounds(sage):
    """max_seqlen larger than every sequence only adds idle workgroups."""
    banner("varlen loose bounds")
    q, k, v, cu_q, cu_k = _packed([100, 250], [100, 250], 4, 1, 64, seed=12)
    a = _run(sage, q, k, v, cu_q, cu_k, True, 0.125, "int8", "fp8")
    b = _run(sage, q, k, v, cu_q, cu_k, True, 0.125, "int8", "fp8", max_q=1000, max_k=777)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_full_size_llm_prefill_sampled(sage):
    """A packed prefill batch at full size (8 sequences, 16384 tokens, 32 query / 8 KV heads,
    d = 128, causal) in the benchmark's configuration; the oracle recomputes two sequences."""
    import oracle
    from bit_quantized_attention_smooth_amd.workloads import varlen_workload
    banner("varlen full size")
    x, w = varlen_workload("varlen_gqa_causal_b8h32kv8t16384d128")
    dev = device()
    o = sage.sageattn_varlen(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), x["cu_q"].to(dev), x["cu_k"].to(dev),
                             w["max_seqlen"], w["max_seqlen"], causal=True, sm_scale=w["sm_scale"])
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    cu = x["cu_q"].numpy()
    for b in (0, len(cu) - 2):
        rows = slice(cu[b], cu[b + 1])
        sub = {n: _f32(x[n][rows]) for n in "qkv"}
        n = cu[b + 1] - cu[b]
        c = np.array([0, n], np.int32)
        o_sim, _, _, sl = oracle.attn_varlen(sub["q"], sub["k"], sub["v"], c, c, True, w["sm_scale"], tile=TILE,
                                             slack=True)
        og = to_np64(o[rows])
        assert within(og, o_sim, sl), excess(og, o_sim, sl)
        assert cos(og, o_sim) >= 0.9999


def test_varlen_full_size_qblock_sampled(sage):
    """Per-block Q smoothing on the full-size packed prefill batch (8 sequences from 256 to 4096
    tokens at starts off the 128-row grid, 32 query / 8 KV heads, d = 128, causal): the oracle
    recomputes the shortest and the last sequence."""
    import oracle
    from bit_quantized_attention_smooth_amd.workloads import varlen_workload
    banner("varlen full size mxfp4_qblock")
    x, w = varlen_workload("varlen_gqa_causal_b8h32kv8t16384d128")
    dev = device()
    o = sage.sageattn_varlen(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), x["cu_q"].to(dev), x["cu_k"].to(dev),
                             w["max_seqlen"], w["max_seqlen"], causal=True, sm_scale=w["sm_scale"],
                             qk_fmt="mxfp4_qblock", pv_fmt="fp8")
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    cu = x["cu_q"].numpy()
    lens = cu[1:] - cu[:-1]
    for b in (int(np.argmin(lens)), len(cu) - 2):
        rows = slice(cu[b], cu[b + 1])
        sub = {n: _f32(x[n][rows]) for n in "qkv"}
        c = np.array([0, cu[b + 1] - cu[b]], np.int32)
        o_sim, _, _, sl = oracle.attn_varlen(sub["q"], sub["k"], sub["v"], c, c, True, w["sm_scale"],
                                             qk_fmt="mxfp4_qblock", pv_fmt="fp8", tile=TILE, slack=True)
        og = to_np64(o[rows])
        assert within(og, o_sim, sl), excess(og, o_sim, sl)
        assert cos(og, o_sim) >= 0.9999


@pytest.mark.parametrize("qk,pv", [("int8", "fp8"), ("mxfp4", "fp8")])
def test_varlen_beyond_2e31_elements_equals_fixed_length(sage, qk, pv):
    """Packed tensors of more than 2^31 elements (2 sequences of 65575 tokens, 128 heads,
    d = 128, causal): bit-identical to the fixed-length entry on the same data, so every
    packed offset is 64-bit."""
    B, H, N, d = 2, 128, 65575, 128
    assert B * N * H * d > 2 ** 31
    banner(f"varlen beyond 2^31 elements {qk}/{pv}")
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(79)
    x = {n: torch.randn(B, H, N, d, device=dev, generator=gen, dtype=torch.float32).to(torch.bfloat16) for n in "qkv"}
    of, lf = sage.sageattn(x["q"], x["k"], x["v"], causal=True, qk_fmt=qk, pv_fmt=pv, return_lse=True)
    torch.cuda.synchronize()
    pk = {}
    for n in "qkv":
        pk[n] = x[n].permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous()
        del x[n]
    cu = torch.arange(0, B * N + 1, N, dtype=torch.int32, device=dev)
    ov, lv = sage.sageattn_varlen(pk["q"], pk["k"], pk["v"], cu, cu, N, N, causal=True, qk_fmt=qk, pv_fmt=pv,
                                  return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(of).all()
    assert torch.equal(ov.reshape(B, N, H, d).permute(0, 2, 1, 3), of)
    assert torch.equal(lv.reshape(H, B, N).permute(1, 0, 2), lf)


@pytest.mark.parametrize("i", range(40))
def test_varlen_random_sweep(sage, i):
    """Seeded random packed batches: up to 4 sequences of 0..300 tokens (query and key lengths
    equal when causal), grouped KV heads, d 64 or 128, bf16 or fp16, every format pair; within
    the forward tolerances of the oracle's per-sequence simulation."""
    import oracle
    rng = np.random.default_rng(5000 + i)
    qk, pv = PAIRS[i % len(PAIRS)]
    nb = int(rng.integers(1, 5))
    causal = bool(rng.integers(0, 2))
    lens_q = [int(v) for v in rng.integers(0, 301, nb)]
    lens_k = lens_q if causal else [int(v) for v in rng.integers(0, 301, nb)]
    Hkv = int(rng.choice([1, 2]))
    H = Hkv * int(rng.choice([1, 2, 3]))
    d = int(rng.choice([64, 128]))
    dtype = torch.float16 if rng.integers(0, 2) else torch.bfloat16
    sm = float(rng.uniform(0.05, 0.2))
    banner(f"varlen sweep {i}: {qk}/{pv} lens_q={lens_q} lens_k={lens_k} H={H}/{Hkv} d={d} {dtype} causal={causal}")
    if sum(lens_q) == 0:   # the entry needs non-empty q, k and v tensors
        lens_q = lens_q[:-1] + [1]
        if causal:
            lens_k = lens_q
    if sum(lens_k) == 0:
        lens_k = lens_k[:-1] + [1]
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, H, Hkv, d, seed=6000 + i, dtype=dtype)
    o, lse = _run(sage, q, k, v, cu_q, cu_k, causal, sm, qk, pv, max_q=max(lens_q), max_k=max(max(lens_k), 1))
    o_sim, lse_sim, _, sl = oracle.attn_varlen(_f32(q), _f32(k), _f32(v), cu_q.numpy(), cu_k.numpy(), causal, sm,
                                               qk_fmt=qk, pv_fmt=pv, tile=TILE, slack=True)
    og = to_np64(o)
    assert within(og, o_sim, sl), excess(og, o_sim, sl)
    if np.abs(o_sim).max() > 0:
        assert cos(og, o_sim) >= 0.9999
    assert np.allclose(lse.cpu().numpy(), lse_sim, rtol=1e-4, atol=2e-3)
