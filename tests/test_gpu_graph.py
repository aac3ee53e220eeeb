"""HIP graph capture and concurrent streams.  The workspace entry points (fixed-length forward
with LSE, 8-bit backward, packed-sequence forward) launch kernels only (no allocation, no
memset), so a captured graph replayed on new inputs must reproduce the eager calls bit for bit;
each replay is followed by eager work and a synchronization, and every replay is checked.
Calls on two streams at once must give the bits of the same calls run one after another."""
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


def test_graph_capture_replays_match_eager(sage):
    banner("graph capture: forward, backward, packed forward")
    dev = device()
    B, H, N, d = 1, 4, 1000, 128
    gen = torch.Generator(device=dev).manual_seed(5)
    cu = torch.tensor([0, 300, 301, N], dtype=torch.int32, device=dev)

    def fresh():
        x = {n: torch.randn(B, H, N, d, device=dev, generator=gen).to(torch.bfloat16) for n in ("q", "k", "v", "do")}
        x["k"] += 2.0 * torch.randn(B, H, 1, d, device=dev, generator=gen).to(torch.bfloat16)
        return x

    def run(x):
        o, lse = sage.sageattn(x["q"], x["k"], x["v"], causal=True, return_lse=True)
        dq, dk, dv = sage.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, causal=True)
        pk = {n: x[n][0].permute(1, 0, 2).contiguous() for n in "qkv"}   # [N, H, d]: 3 packed sequences
        ov, lv = sage.sageattn_varlen(pk["q"], pk["k"][:, :2].contiguous(), pk["v"][:, :2].contiguous(), cu, cu,
                                      699, 699, causal=True, qk_fmt="mxfp4", pv_fmt="mxfp8", return_lse=True)
        return [o, lse, dq, dk, dv, ov, lv]

    static = fresh()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run(static)
    torch.cuda.synchronize()
    names = ("o", "lse", "dq", "dk", "dv", "o_packed", "lse_packed")
    for rep in range(3):
        x = fresh()
        for n in x:
            static[n].copy_(x[n])
        graph.replay()
        torch.cuda.synchronize()
        want = run(x)
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, want):
            assert torch.isfinite(a).all(), (rep, name)
            assert torch.equal(a, b), (rep, name)


def test_concurrent_streams_match_sequential(sage):
    """Calls on two streams at once (each with its own workspace, and the one-call entry with its
    stream-ordered scratch) give the same bits as the same calls run one after another."""
    banner("two streams at once")
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(6)
    a = {n: torch.randn(1, 8, 2048, 128, device=dev, generator=gen).to(torch.bfloat16) for n in "qkv"}
    b = {n: torch.randn(2, 4, 777, 64, device=dev, generator=gen).to(torch.bfloat16) for n in "qkv"}
    want_a = sage.sageattn(a["q"], a["k"], a["v"], causal=True)
    want_b = sage.attn_fwd_oneshot(b["q"], b["k"], b["v"])
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        outs_a, outs_b = [], []
        for _ in range(4):
            with torch.cuda.stream(s1):
                outs_a.append(sage.sageattn(a["q"], a["k"], a["v"], causal=True))
            with torch.cuda.stream(s2):
                outs_b.append(sage.attn_fwd_oneshot(b["q"], b["k"], b["v"]))
        torch.cuda.synchronize()
        assert all(torch.equal(o, want_a) for o in outs_a)
        assert all(torch.equal(o, want_b) for o in outs_b)


def test_graph_capture_packed_qblock_replays_match_eager(sage):
    """The packed per-block Q smoothing path (table, block means, codes, dS on the fp64 MFMA,
    fused kernel) under graph capture: replays on new inputs match eager calls bit for bit."""
    banner("graph capture: packed per-block Q smoothing")
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(8)
    cu = torch.tensor([0, 130, 131, 500, 900], dtype=torch.int32, device=dev)

    def fresh():
        return {"q": torch.randn(900, 6, 128, device=dev, generator=gen).to(torch.bfloat16),
                "k": torch.randn(900, 2, 128, device=dev, generator=gen).to(torch.bfloat16),
                "v": torch.randn(900, 2, 128, device=dev, generator=gen).to(torch.bfloat16)}

    def run(x):
        return list(sage.sageattn_varlen(x["q"], x["k"], x["v"], cu, cu, 400, 400, causal=False,
                                         qk_fmt="mxfp4_qblock", pv_fmt="fp8", return_lse=True))

    static = fresh()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run(static)
    torch.cuda.synchronize()
    for rep in range(3):
        x = fresh()
        for n in x:
            static[n].copy_(x[n])
        graph.replay()
        torch.cuda.synchronize()
        want = run(x)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse"), outs, want):
            assert torch.isfinite(a).all(), (rep, name)
            assert torch.equal(a, b), (rep, name)
