"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import bit_quantized_attention_smooth_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)        # aligned, never dereferenced: validation fails or injects first


def _declared():
    src = open(os.path.join(ROOT, "include", "sage_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = S.lib()
    declared = _declared()
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(S.EXPORTS) == declared
    assert L.sage_abi_version() == 2


def _p(**kw):
    base = dict(B=1, H=2, N=100, d=128, causal=0, sm_scale=0.125, io_dtype=0, qk_fmt=1, pv_fmt=2)
    base.update(kw)
    return S.Problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), S.ERR_INVALID_ARG), (dict(N=0), S.ERR_INVALID_ARG), (dict(H=-1), S.ERR_INVALID_ARG),
    (dict(B=1, H=1, d=64, N=2 ** 31 - 1), S.ERR_INVALID_ARG), (dict(B=1, H=1, d=64, N=2 ** 30 + 1), S.ERR_INVALID_ARG),
    (dict(d=96), S.ERR_UNSUPPORTED), (dict(d=256), S.ERR_UNSUPPORTED),
    (dict(sm_scale=0.0), S.ERR_INVALID_ARG), (dict(sm_scale=float("nan")), S.ERR_INVALID_ARG),
    (dict(sm_scale=float("inf")), S.ERR_INVALID_ARG), (dict(causal=2), S.ERR_INVALID_ARG),
    (dict(io_dtype=7), S.ERR_INVALID_ARG), (dict(qk_fmt=9), S.ERR_INVALID_ARG),
    (dict(qk_fmt=2, pv_fmt=2), S.ERR_UNSUPPORTED), (dict(qk_fmt=1, pv_fmt=3), S.ERR_UNSUPPORTED),
    (dict(qk_fmt=1, pv_fmt=4), S.ERR_UNSUPPORTED), (dict(pv_fmt=8), S.ERR_INVALID_ARG),
    (dict(qk_fmt=7, pv_fmt=5), S.ERR_UNSUPPORTED), (dict(qk_fmt=1, pv_fmt=7), S.ERR_UNSUPPORTED),
    (dict(qk_fmt=6, pv_fmt=3), S.ERR_UNSUPPORTED), (dict(qk_fmt=2, pv_fmt=6), S.ERR_UNSUPPORTED),
    (dict(qk_fmt=3, pv_fmt=5), S.ERR_UNSUPPORTED),
])
def test_problem_validation(kw, status):
    L = S.lib()
    n = ctypes.c_size_t(12345)
    assert L.sage_quant_size(ctypes.byref(_p(**kw)), ctypes.byref(n), None) == status
    assert n.value == 12345                       # output untouched on error
    assert L.sage_last_error()                    # message set
    st = L.sage_quantize(FAKE, FAKE, FAKE, ctypes.byref(_p(**kw)), FAKE, 1 << 40, None)
    assert st == status


def test_null_and_misaligned_pointers_rejected():
    L = S.lib()
    p = _p()
    assert L.sage_quantize(None, FAKE, FAKE, ctypes.byref(p), FAKE, 1 << 40, None) == S.ERR_INVALID_ARG
    assert L.sage_quantize(FAKE, FAKE, ctypes.c_void_p(0x100004), ctypes.byref(p), FAKE, 1 << 40, None) == S.ERR_INVALID_ARG
    assert L.sage_attn_fwd_quantized(FAKE, 1 << 40, ctypes.byref(p), None, None, None) == S.ERR_INVALID_ARG
    assert L.sage_attn_fwd(FAKE, FAKE, FAKE, None, 1, 2, 64, 128, 0, 0.1, 1, 2, None) == S.ERR_INVALID_ARG
    assert L.sage_quant_size(None, None, None) == S.ERR_INVALID_ARG


def test_workspace_too_small_rejected():
    L = S.lib()
    p = _p()
    need, _ = S.quant_size(p)
    assert L.sage_quantize(FAKE, FAKE, FAKE, ctypes.byref(p), FAKE, need - 1, None) == S.ERR_WORKSPACE
    assert L.sage_attn_fwd_ex(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1, None) == S.ERR_WORKSPACE
    assert L.sage_attn_fwd_quantized(FAKE, need - 1, ctypes.byref(p), FAKE, None, None) == S.ERR_WORKSPACE
    assert b"needs" in L.sage_last_error()


def test_quant_layout_sizes():
    """Offsets are 256-byte aligned, ordered, and each part has the documented size."""
    for qk, pv in ((1, 2), (1, 5), (6, 2), (6, 5), (3, 2), (3, 3), (3, 4), (7, 2), (7, 3)):
        for N in (1, 100, 4096):
            p = _p(N=N, qk_fmt=qk, pv_fmt=pv)
            total, lay = S.quant_size(p)
            BH, d, Np = 2, 128, (N + 127) // 128 * 128
            offs = [lay[k] for k in ("mu_k", "mu_q", "q_codes", "q_scales", "k_codes", "k_scales",
                                     "v_codes", "v_scales", "delta_s", "lse_corr", "stats")]
            assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
            codes = BH * Np * d // (2 if qk in (3, 7) else 1)
            assert lay["q_scales"] - lay["q_codes"] >= codes
            if qk == 7:      # a Q mean per 128-query block (fp32, then fp64 over whole 16-block
                nb = Np // 128   # groups), a dS row per block
                assert lay["q_codes"] - lay["mu_q"] >= BH * nb * d * 4 + BH * ((nb + 15) // 16 * 16) * d * 8
                assert lay["lse_corr"] - lay["delta_s"] >= BH * (Np // 128) * Np * 4
            if qk == 6:      # a step per query token and per 32 keys
                assert lay["k_codes"] - lay["q_scales"] >= BH * Np * 4
                assert lay["v_codes"] - lay["k_scales"] >= BH * Np // 32 * 4
            assert lay["v_scales"] - lay["v_codes"] >= BH * Np * d * {3: 1, 5: 4}.get(pv, 2) // 2
            if pv in (3, 4):    # E8M0 byte per channel per 32 tokens
                assert lay["delta_s"] - lay["v_scales"] >= BH * (Np // 32) * d
            assert total >= lay["stats"] + 8 * BH * d * 20


def test_injected_allocation_failure(monkeypatch):
    L = S.lib()
    monkeypatch.setenv("SAGE_FAULT_INJECT", "alloc")
    st = L.sage_attn_fwd(FAKE, FAKE, FAKE, FAKE, 1, 2, 64, 128, 0, 0.1, 1, 2, None)
    assert st == S.ERR_OUT_OF_MEMORY
    assert b"injected" in L.sage_last_error()


def test_status_strings():
    L = S.lib()
    for s in range(6):
        assert L.sage_status_string(s)
    assert L.sage_status_string(99) == b"unknown status"


def test_backward_rejects_unsupported_problems():
    L = S.lib()
    n = ctypes.c_size_t()
    assert L.sage_attn_bwd_ws_size(ctypes.byref(_p(qk_fmt=3, pv_fmt=2)), ctypes.byref(n)) == S.ERR_UNSUPPORTED
    assert L.sage_attn_bwd_ws_size(ctypes.byref(_p(d=96)), ctypes.byref(n)) == S.ERR_UNSUPPORTED
    assert L.sage_attn_bwd_ws_size(ctypes.byref(_p(d=128)), ctypes.byref(n)) == S.OK
    # the forward's quantized buffer, then five 8-bit operand tensors (dO, V token-major; dO^T,
    # Q^T, K_s^T) of BH x Np x d bytes each, plus steps, D and the log2-domain LSE
    quant128, _ = S.quant_size(_p(d=128))
    BH, Np = 2, 128
    assert n.value >= quant128 + 5 * BH * Np * 128 + 2 * BH * Np * 4
    assert L.sage_attn_bwd_ws_size(ctypes.byref(_p(d=64)), ctypes.byref(n)) == S.OK
    quant, _ = S.quant_size(_p(d=64))
    assert n.value > quant
    p = _p(d=64)
    assert L.sage_attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n.value - 1,
                           None) == S.ERR_WORKSPACE
    assert L.sage_attn_bwd(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n.value,
                           None) == S.ERR_INVALID_ARG
    # the after-forward entry checks the same things
    fn = L.sage_attn_bwd_after_fwd
    assert fn(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n.value - 1,
              None) == S.ERR_WORKSPACE
    assert fn(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n.value,
              None) == S.ERR_INVALID_ARG
    assert fn(ctypes.byref(_p(qk_fmt=3, pv_fmt=2)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
              n.value, None) == S.ERR_UNSUPPORTED


def _vp(**kw):
    base = dict(B=2, H=4, H_kv=2, d=128, causal=0, sm_scale=0.125, io_dtype=0, qk_fmt=1, pv_fmt=2,
                total_q=100, total_k=90, max_seqlen_q=60, max_seqlen_k=50)
    base.update(kw)
    return S.VarlenProblem(*[base[n] for n, _ in S.VarlenProblem._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), S.ERR_INVALID_ARG), (dict(H_kv=0), S.ERR_INVALID_ARG), (dict(H=6, H_kv=4), S.ERR_INVALID_ARG),
    (dict(total_q=-1), S.ERR_INVALID_ARG), (dict(max_seqlen_k=-5), S.ERR_INVALID_ARG),
    (dict(d=96), S.ERR_UNSUPPORTED), (dict(qk_fmt=1, pv_fmt=3), S.ERR_UNSUPPORTED),
    (dict(sm_scale=float("nan")), S.ERR_INVALID_ARG), (dict(total_q=2 ** 31 - 1), S.ERR_INVALID_ARG),
    (dict(qk_fmt=7, pv_fmt=5), S.ERR_UNSUPPORTED),
    (dict(qk_fmt=7, pv_fmt=2, total_q=2 ** 28, total_k=2 ** 28, max_seqlen_k=2 ** 28), S.ERR_INVALID_ARG),
])
def test_varlen_validation(kw, status):
    L = S.lib()
    n = ctypes.c_size_t(777)
    assert L.sage_varlen_ws_size(ctypes.byref(_vp(**kw)), ctypes.byref(n)) == status
    assert n.value == 777 and L.sage_last_error()
    assert L.sage_attn_varlen_fwd(ctypes.byref(_vp(**kw)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                  1 << 40, None) == status


def test_varlen_pointer_and_workspace_checks():
    L = S.lib()
    p = _vp()
    n = ctypes.c_size_t()
    assert L.sage_varlen_ws_size(ctypes.byref(p), ctypes.byref(n)) == S.OK
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE]
    assert L.sage_attn_varlen_fwd(ctypes.byref(p), *args[:3], None, FAKE, *args[5:], n.value, None) == S.ERR_INVALID_ARG
    assert L.sage_attn_varlen_fwd(ctypes.byref(p), *args[:3], ctypes.c_void_p(0x100002), FAKE, *args[5:], n.value,
                                  None) == S.ERR_INVALID_ARG
    assert L.sage_attn_varlen_fwd(ctypes.byref(p), *args, n.value - 1, None) == S.ERR_WORKSPACE
    # no query rows: nothing to launch, every other pointer may be NULL
    assert L.sage_attn_varlen_fwd(ctypes.byref(_vp(total_q=0)), None, None, None, FAKE, FAKE, None, None, None, 0,
                                  None) == S.OK


def test_varlen_bounds_beyond_the_totals_are_clamped():
    """max_seqlen_q / max_seqlen_k up to INT32_MAX: no sequence can be longer than its tensor, so
    the bounds are clamped to total_q / total_k (no integer overflow in the checks, the same
    workspace as exact bounds, for every format pair)."""
    L = S.lib()
    for qk, pv in ((1, 2), (3, 2), (7, 3), (6, 5)):
        a, b = ctypes.c_size_t(), ctypes.c_size_t()
        assert L.sage_varlen_ws_size(ctypes.byref(_vp(qk_fmt=qk, pv_fmt=pv)), ctypes.byref(a)) == S.OK
        loose = _vp(qk_fmt=qk, pv_fmt=pv, max_seqlen_q=2 ** 31 - 1, max_seqlen_k=2 ** 31 - 1)
        assert L.sage_varlen_ws_size(ctypes.byref(loose), ctypes.byref(b)) == S.OK
        assert b.value == a.value   # (per-block strips: 50 and 90 keys both round up to 128)


def test_varlen_workspace_covers_every_sequence_padding():
    """Per head, each sequence gets a 64-aligned start and room for its length rounded up to 128
    before the next one begins; the workspace grows with the batch size accordingly."""
    L = S.lib()
    sizes = []
    for B in (1, 8, 64):
        n = ctypes.c_size_t()
        assert L.sage_varlen_ws_size(ctypes.byref(_vp(B=B, total_q=4096, total_k=4096, max_seqlen_q=4096,
                                                      max_seqlen_k=4096)), ctypes.byref(n)) == S.OK
        sizes.append(n.value)
    # INT8 / FP8: per key token 2 B of K and V codes per KV head, per query token 1 B of Q codes
    # per query head; 256 extra tokens per sequence
    per_seq = 256 * (2 * 128 + 4 * 128)
    assert sizes[1] - sizes[0] >= 7 * per_seq and sizes[2] - sizes[1] >= 56 * per_seq


def test_varlen_qblock_workspace_holds_every_block_strip():
    """Per-block Q smoothing on packed sequences: per head, total_q / 128 + B + 1 block slots,
    each with a mean (fp32, then fp64 with 16 rows of padding) and a dS strip of max_seqlen_k
    keys rounded up to 128; the workspace is the plain MXFP4 one plus those."""
    L = S.lib()
    n_mx, n_qb = ctypes.c_size_t(), ctypes.c_size_t()
    kw = dict(B=3, H=4, H_kv=2, d=128, total_q=1000, total_k=700, max_seqlen_q=500, max_seqlen_k=300)
    assert L.sage_varlen_ws_size(ctypes.byref(_vp(qk_fmt=3, pv_fmt=2, **kw)), ctypes.byref(n_mx)) == S.OK
    assert L.sage_varlen_ws_size(ctypes.byref(_vp(qk_fmt=7, pv_fmt=2, **kw)), ctypes.byref(n_qb)) == S.OK
    slots = 4 * (1000 // 128 + 3 + 1)
    # replaced: a mean per query instance (B H of them) and a dS row per query head over the
    # packed key tokens (700 rounded up to 64, plus 256 per sequence)
    plain = 12 * 128 * 4 + 4 * (704 + 3 * 256) * 4
    extra = slots * 128 * 4 + (slots + 16) * 128 * 8 + slots * 384 * 4 - plain
    assert abs(n_qb.value - n_mx.value - extra) <= 2 * 256
    # the strip never exceeds total_k: a loose max_seqlen_k bound changes nothing
    n_loose = ctypes.c_size_t()
    loose = dict(kw, max_seqlen_k=2 ** 30)
    assert L.sage_varlen_ws_size(ctypes.byref(_vp(qk_fmt=7, pv_fmt=2, **loose)), ctypes.byref(n_loose)) == S.OK
    assert n_loose.value == n_qb.value + 4 * (1000 // 128 + 4) * (768 - 384) * 4
    # the size guard is the per-block one: the same sizes without it are accepted
    big = dict(total_q=2 ** 28, total_k=2 ** 28, max_seqlen_k=2 ** 28)
    assert L.sage_varlen_ws_size(ctypes.byref(_vp(qk_fmt=3, pv_fmt=2, **big)), ctypes.byref(n_mx)) == S.OK


def test_backward_binding_rejects_mismatched_o_do_lse():
    """The Python binding is the only guard of the backward's raw-pointer arguments: O and dO
    must match Q, and LSE must be float32 [B, H, N] (a bf16 LSE, the packed path's [H, total]
    LSE or a shorter dO would be read past their ends on the device)."""
    import torch
    import bit_quantized_attention_smooth_amd as S
    B, H, N, d = 1, 2, 96, 64
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    good = dict(o=torch.zeros_like(q), do=torch.zeros_like(q), lse=torch.zeros(B, H, N))
    S.check_bwd_inputs(q, **good)
    bad = [("o", torch.zeros(B, H, N - 1, d, dtype=torch.bfloat16)),
           ("o", torch.zeros(B, H, N, d, dtype=torch.float16)),
           ("do", torch.zeros(B, H, N // 2, d, dtype=torch.bfloat16)),
           ("do", torch.zeros(B, H, N, d)),
           ("lse", torch.zeros(B, H, N, dtype=torch.bfloat16)),
           ("lse", torch.zeros(H, B * N)),
           ("lse", torch.zeros(B, H, N - 1)),
           ("lse", None)]
    for name, t in bad:
        kw = dict(good, **{name: t})
        with pytest.raises(ValueError):
            S.check_bwd_inputs(q, **kw)


def test_one_call_entries_reject_float16_in_the_binding():
    """The one-call C entries (sage_attn_fwd, sage_attn_fwd_noalloc) take no dtype argument and
    read bfloat16: the binding refuses float16 tensors before any pointer reaches them."""
    import torch
    import bit_quantized_attention_smooth_amd as S
    q = torch.zeros(1, 2, 64, 64, dtype=torch.float16)
    for fn in (S.attn_fwd_oneshot, S.attn_fwd_noalloc):
        with pytest.raises(ValueError, match="bfloat16"):
            fn(q, q, q)
        with pytest.raises(ValueError, match="bfloat16"):
            fn(q.bfloat16(), q, q.bfloat16())


def test_noalloc_entry_rejects_problems_beyond_its_scratch():
    """The no-allocation forward holds a 64 MiB quantized buffer per GPU: a problem that needs more
    (B=1 H=32 N=8192 d=128, INT8 / FP8: about 99 MiB) is refused on the host, before any device
    call, and a null pointer is still refused first."""
    L = S.lib()
    n = ctypes.c_size_t()
    assert L.sage_quant_size(ctypes.byref(_p(B=1, H=32, N=8192, d=128)), ctypes.byref(n), None) == S.OK
    assert n.value > 64 << 20
    st = L.sage_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, 1, 32, 8192, 128, 0, 0.088, 1, 2, None)
    assert st == S.ERR_WORKSPACE, L.sage_last_error()
    assert b"64" in L.sage_last_error() or b"67108864" in L.sage_last_error()
    assert L.sage_attn_fwd_noalloc(None, FAKE, FAKE, FAKE, 1, 2, 100, 64, 0, 0.125, 1, 2, None) == S.ERR_INVALID_ARG
    assert L.sage_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, 1, 2, 100, 96, 0, 0.125, 1, 2, None) == S.ERR_UNSUPPORTED


def test_sage_log_prints_one_line_per_outermost_call():
    """SAGE_LOG=1: each entry-point call prints one line on stderr (name, problem, status and
    the error text); without it the library prints nothing.  A host-only call in a child
    process, so the variable is read as a user would set it."""
    import subprocess
    import sys
    code = ("import ctypes, bit_quantized_attention_smooth_amd as S\n"
            "L = S.lib(); n = ctypes.c_size_t()\n"
            "p = S.Problem(1, 2, 256, 64, 0, 0.125, 0, 1, 2)\n"
            "assert L.sage_quant_size(ctypes.byref(p), ctypes.byref(n), None) == S.OK\n"
            "p.d = 96\n"
            "assert L.sage_quant_size(ctypes.byref(p), ctypes.byref(n), None) == S.ERR_UNSUPPORTED\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=root)
    env.pop("SAGE_LOG", None)
    quiet = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert quiet.returncode == 0, quiet.stderr
    assert "sage:" not in quiet.stderr
    env["SAGE_LOG"] = "1"
    loud = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert loud.returncode == 0, loud.stderr
    lines = [l for l in loud.stderr.splitlines() if l.startswith("sage:")]
    assert len(lines) == 2, loud.stderr
    assert lines[0].startswith("sage: sage_quant_size(B=1 H=2 N=256 d=64") and lines[0].endswith("-> ok")
    assert "d=96" in lines[1] and "-> unsupported: head dim d=96" in lines[1]
