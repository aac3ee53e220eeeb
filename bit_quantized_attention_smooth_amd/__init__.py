"""MI355X-native SageAttention-style quantized attention.

A thin ctypes binding over ``libsage_attn.so`` (C ABI in ``include/sage_attn.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensor shapes, allocates outputs / workspaces with torch and
passes raw device pointers and the current HIP stream.  If the library is not
built, every entry point raises; there is no CPU fallback.

Entry points follow the pages' names: ``sageattn`` (alias ``attn``) computes
softmax(sm_scale Q K^T) V with INT8 or MXFP4 QK^T and FP8 P~V; ``quantize``
and ``attn_fwd_quantized`` expose the two stages; ``sageattn_varlen`` takes packed
sequences (cu_seqlens) with grouped KV heads; ``attn_bwd`` and ``SageAttnFn`` give
the 8-bit backward.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SAGE_ATTN_LIBRARY selects another build of the same library (the host-sanitized build the
# ABI tests run under); there is no fallback: a missing library raises in lib().
LIB_PATH = os.environ.get("SAGE_ATTN_LIBRARY") or os.path.join(_HERE, "libsage_attn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_OUT_OF_MEMORY, ERR_HIP = range(6)
FMT = {"int8": 1, "fp8": 2, "mxfp4": 3, "mxfp8": 4, "f16": 5, "int8_token": 6, "mxfp4_qblock": 7}
DT = {torch.bfloat16: 0, torch.float16: 1}

# Every symbol the header declares (kept in sync by a CPU test that parses the header).
EXPORTS = ["sage_attn_fwd", "sage_attn_fwd_noalloc", "sage_quant_size", "sage_quantize", "sage_attn_fwd_quantized",
           "sage_attn_fwd_ws_size", "sage_attn_fwd_ex", "sage_attn_bwd_ws_size", "sage_attn_bwd",
           "sage_attn_bwd_after_fwd",
           "sage_varlen_ws_size", "sage_attn_varlen_fwd",
           "sage_status_string", "sage_last_error", "sage_abi_version"]


class SageError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"sage status {status}: {msg}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("d", ctypes.c_int),
                ("causal", ctypes.c_int), ("sm_scale", ctypes.c_float), ("io_dtype", ctypes.c_int),
                ("qk_fmt", ctypes.c_int), ("pv_fmt", ctypes.c_int)]


class VarlenProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("H_kv", ctypes.c_int), ("d", ctypes.c_int),
                ("causal", ctypes.c_int), ("sm_scale", ctypes.c_float), ("io_dtype", ctypes.c_int),
                ("qk_fmt", ctypes.c_int), ("pv_fmt", ctypes.c_int), ("total_q", ctypes.c_int),
                ("total_k", ctypes.c_int), ("max_seqlen_q", ctypes.c_int), ("max_seqlen_k", ctypes.c_int)]


class QuantLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("mu_k", "mu_q", "q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales",
                 "delta_s", "lse_corr", "stats", "total")]


_lib = None


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run bit_quantized_attention_smooth_amd/build.py "
                               "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i, f = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
        P = ctypes.POINTER(Problem)
        sigs = {
            "sage_attn_fwd": [vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp],
            "sage_attn_fwd_noalloc": [vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp],
            "sage_quant_size": [P, ctypes.POINTER(sz), ctypes.POINTER(QuantLayout)],
            "sage_quantize": [vp, vp, vp, P, vp, sz, vp],
            "sage_attn_fwd_quantized": [vp, sz, P, vp, vp, vp],
            "sage_attn_fwd_ws_size": [P, ctypes.POINTER(sz)],
            "sage_attn_fwd_ex": [P, vp, vp, vp, vp, vp, vp, sz, vp],
            "sage_attn_bwd_ws_size": [P, ctypes.POINTER(sz)],
            "sage_attn_bwd": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "sage_attn_bwd_after_fwd": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "sage_varlen_ws_size": [ctypes.POINTER(VarlenProblem), ctypes.POINTER(sz)],
            "sage_attn_varlen_fwd": [ctypes.POINTER(VarlenProblem), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.sage_status_string.argtypes = [ctypes.c_int]
        L.sage_status_string.restype = ctypes.c_char_p
        L.sage_last_error.restype = ctypes.c_char_p
        L.sage_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status != OK:
        raise SageError(status, lib().sage_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def problem(B, H, N, d, *, causal=False, sm_scale=None, dtype=torch.bfloat16, qk_fmt="int8", pv_fmt="fp8"):
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    return Problem(B, H, N, d, int(bool(causal)), sm, DT[dtype], FMT[qk_fmt], FMT[pv_fmt])


def quant_size(p):
    """(bytes, {part: byte offset}) of the quantized buffer for problem ``p``."""
    n = ctypes.c_size_t()
    lay = QuantLayout()
    _check(lib().sage_quant_size(ctypes.byref(p), ctypes.byref(n), ctypes.byref(lay)))
    return n.value, {name: getattr(lay, name) for name, _ in QuantLayout._fields_}


def _qkv(q, k, v):
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share a [B,H,N,d] shape, got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if q.dtype not in DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be bfloat16 or all float16")
    return q.contiguous(), k.contiguous(), v.contiguous()


def quantize(q, k, v, *, causal=False, sm_scale=None, qk_fmt="int8", pv_fmt="fp8"):
    """Smoothing + quantization prologue; returns (buffer uint8 tensor, problem, layout)."""
    q, k, v = _qkv(q, k, v)
    B, H, N, d = q.shape
    p = problem(B, H, N, d, causal=causal, sm_scale=sm_scale, dtype=q.dtype, qk_fmt=qk_fmt, pv_fmt=pv_fmt)
    nbytes, lay = quant_size(p)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check(lib().sage_quantize(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(p), _ptr(buf), nbytes, _stream()))
    return buf, p, lay


def attn_fwd_quantized(buf, p, *, dtype=torch.bfloat16, return_lse=False):
    """Fused attention on a quantized buffer; returns O (and the fp32 LSE)."""
    o = torch.empty((p.B, p.H, p.N, p.d), dtype=dtype, device=buf.device)
    lse = torch.empty((p.B, p.H, p.N), dtype=torch.float32, device=buf.device) if return_lse else None
    _check(lib().sage_attn_fwd_quantized(_ptr(buf), buf.numel(), ctypes.byref(p), _ptr(o), _ptr(lse), _stream()))
    return (o, lse) if return_lse else o


def _via_packed(q, k, v, layout, causal, sm_scale, qk_fmt, pv_fmt, return_lse):
    """B equal-length sequences through the packed-sequence entry (each sequence and head gets
    the fixed-length entry's quantization and kernels): grouped KV heads, query and key lengths
    that differ, or [B,N,H,d] tensors, which are already the packed [B*N,H,d] rows."""
    if layout == "HND":
        (B, H, Nq, d), (Hkv, Nk) = q.shape, k.shape[1:3]
        rows = [t.permute(0, 2, 1, 3).reshape(B * n, h, d) for t, n, h in ((q, Nq, H), (k, Nk, Hkv), (v, Nk, Hkv))]
    else:
        (B, Nq, H, d), (Nk, Hkv) = q.shape, k.shape[1:3]
        rows = [t.reshape(B * n, h, d) for t, n, h in ((q, Nq, H), (k, Nk, Hkv), (v, Nk, Hkv))]
    cu_q = torch.arange(0, B * Nq + 1, Nq, dtype=torch.int32, device=q.device)
    cu_k = torch.arange(0, B * Nk + 1, Nk, dtype=torch.int32, device=q.device)
    o, lse = sageattn_varlen(*rows, cu_q, cu_k, Nq, Nk, causal=causal, sm_scale=sm_scale, qk_fmt=qk_fmt,
                             pv_fmt=pv_fmt, return_lse=True)
    o = o.reshape(B, Nq, H, d)
    if layout == "HND":
        o = o.permute(0, 2, 1, 3).contiguous()
    lse = lse.reshape(H, B, Nq).permute(1, 0, 2).contiguous()
    return (o, lse) if return_lse else o


def sageattn(q, k, v, *, causal=False, sm_scale=None, qk_fmt="int8", pv_fmt="fp8", return_lse=False, workspace=None,
             tensor_layout="HND"):
    """Quantized attention forward on bf16/fp16 device tensors: q [B,H,N_q,d], k and v
    [B,H_kv,N_k,d] (tensor_layout "HND"), or q [B,N_q,H,d], k and v [B,N_k,H_kv,d] ("NHD").
    Query head h reads KV head h / (H / H_kv).  Returns O in q's layout (and LSE [B,H,N_q]).
    Grouped KV heads, N_q != N_k (causal masking then top-left aligned) and "NHD" run through the
    packed-sequence entry with B equal-length sequences; workspace applies to the plain case."""
    if tensor_layout not in ("HND", "NHD"):
        raise ValueError(f"tensor_layout must be 'HND' or 'NHD', got {tensor_layout!r}")
    if q.dim() == 4 and k.dim() == 4 and k.shape == v.shape:
        hq, hk = (1, 1) if tensor_layout == "HND" else (2, 2)
        nq, nk = (2, 2) if tensor_layout == "HND" else (1, 1)
        same_bd = q.shape[0] == k.shape[0] and q.shape[3] == k.shape[3]
        grouped_ok = k.shape[hk] >= 1 and q.shape[hq] % k.shape[hk] == 0
        if same_bd and grouped_ok and (tensor_layout == "NHD" or q.shape[hq] != k.shape[hk]
                                       or q.shape[nq] != k.shape[nk]):
            if not (q.is_cuda and k.is_cuda and v.is_cuda):
                raise ValueError("q, k, v must be device tensors")
            return _via_packed(q, k, v, tensor_layout, causal, sm_scale, qk_fmt, pv_fmt, return_lse)
    q, k, v = _qkv(q, k, v)
    B, H, N, d = q.shape
    p = problem(B, H, N, d, causal=causal, sm_scale=sm_scale, dtype=q.dtype, qk_fmt=qk_fmt, pv_fmt=pv_fmt)
    nbytes = ctypes.c_size_t()
    _check(lib().sage_attn_fwd_ws_size(ctypes.byref(p), ctypes.byref(nbytes)))
    if workspace is not None:
        # a caller's workspace is used as given (a training step reads the quantization back from
        # it), so one that cannot hold it is an error rather than silently replaced
        if (not torch.is_tensor(workspace) or workspace.dtype != torch.uint8 or workspace.device != q.device
                or not workspace.is_contiguous() or workspace.numel() < nbytes.value):
            raise ValueError(f"workspace must be a contiguous uint8 tensor on {q.device} of at least "
                             f"{nbytes.value} bytes")
        ws = workspace
    else:
        ws = torch.empty(nbytes.value, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib().sage_attn_fwd_ex(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws),
                                  ws.numel(), _stream()))
    return (o, lse) if return_lse else o


attn = sageattn


def sageattn_qk_int8_pv_fp16(q, k, v, *, causal=False, sm_scale=None, return_lse=False, workspace=None):
    """The 16-bit P~V fallback under the entry name the SageAttention3 code-link page lists
    (INT8 QK^T with IEEE fp16 P~ and V, fp32 accumulation on the matrix cores)."""
    return sageattn(q, k, v, causal=causal, sm_scale=sm_scale, qk_fmt="int8", pv_fmt="f16", return_lse=return_lse,
                    workspace=workspace)


def varlen_problem(B, H, H_kv, d, total_q, total_k, max_seqlen_q, max_seqlen_k, *, causal=False, sm_scale=None,
                   dtype=torch.bfloat16, qk_fmt="int8", pv_fmt="fp8"):
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    return VarlenProblem(B, H, H_kv, d, int(bool(causal)), sm, DT[dtype], FMT[qk_fmt], FMT[pv_fmt],
                         total_q, total_k, max_seqlen_q, max_seqlen_k)


def sageattn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
                    sm_scale=None, qk_fmt="int8", pv_fmt="fp8", return_lse=False):
    """Packed sequences: q [total_q,H,d], k and v [total_k,H_kv,d] bf16/fp16 device tensors,
    cu_seqlens_* int32 device tensors [B+1].  Returns O [total_q,H,d] (and LSE [H,total_q])."""
    if not (q.is_cuda and k.is_cuda and v.is_cuda and cu_seqlens_q.is_cuda and cu_seqlens_k.is_cuda):
        raise ValueError("q, k, v and the cu_seqlens must be device tensors")
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError(f"expected q [total_q,H,d] and k, v [total_k,H_kv,d], got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if q.dtype not in DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be bfloat16 or all float16")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 or \
            cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q / cu_seqlens_k must be int32 tensors of the same length B+1 >= 2")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    cu_q, cu_k = cu_seqlens_q.contiguous(), cu_seqlens_k.contiguous()
    (total_q, H, d), (total_k, H_kv) = q.shape, k.shape[:2]
    p = varlen_problem(cu_q.numel() - 1, H, H_kv, d, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k),
                       causal=causal, sm_scale=sm_scale, dtype=q.dtype, qk_fmt=qk_fmt, pv_fmt=pv_fmt)
    nbytes = ctypes.c_size_t()
    _check(lib().sage_varlen_ws_size(ctypes.byref(p), ctypes.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 16), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib().sage_attn_varlen_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_q), _ptr(cu_k), _ptr(o),
                                      _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return (o, lse) if return_lse else o


def _bf16_only(q, k, v):
    # the one-call C entries take no dtype argument: their inputs and output are bfloat16
    if not all(torch.is_tensor(t) and t.dtype == torch.bfloat16 for t in (q, k, v)):
        raise ValueError("this entry takes bfloat16 q, k, v only (use sageattn for float16)")


def attn_fwd_oneshot(q, k, v, *, causal=False, sm_scale=None, qk_fmt="int8", pv_fmt="fp8"):
    """The one-call C entry (bf16 only; the library allocates its scratch stream-ordered)."""
    _bf16_only(q, k, v)
    q, k, v = _qkv(q, k, v)
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    _check(lib().sage_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, int(bool(causal)), sm,
                               FMT[qk_fmt], FMT[pv_fmt], _stream()))
    return o


def attn_fwd_noalloc(q, k, v, *, causal=False, sm_scale=None, qk_fmt="int8", pv_fmt="fp8", out=None):
    """The no-allocation C entry (bf16 only): its scratch is a fixed 64 MiB array the library
    holds per GPU, shared by every call on that GPU.  `out` (bf16, q's shape) may be given so the
    call allocates nothing here either."""
    _bf16_only(q, k, v)
    q, k, v = _qkv(q, k, v)
    B, H, N, d = q.shape
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or o.device != q.device or not o.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    _check(lib().sage_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, int(bool(causal)), sm,
                                       FMT[qk_fmt], FMT[pv_fmt], _stream()))
    return o


def check_bwd_inputs(q, o, do, lse):
    """The backward's C entry takes raw pointers: it reads O and dO with Q's offsets and dtype and
    LSE as fp32 [B, H, N], so anything else would be read past its end.  Raises ValueError unless
    o and do match q (shape, dtype, device) and lse is a float32 [B, H, N] tensor on q's device."""
    B, H, N, _ = q.shape
    for name, t in (("o", o), ("do", do)):
        if not (torch.is_tensor(t) and t.device == q.device and t.shape == q.shape and t.dtype == q.dtype):
            raise ValueError(f"{name} must be a {q.dtype} tensor of shape {tuple(q.shape)} on {q.device}")
    if not (torch.is_tensor(lse) and lse.device == q.device and lse.dtype == torch.float32 and
            tuple(lse.shape) == (B, H, N)):
        raise ValueError(f"lse must be a float32 tensor of shape {(B, H, N)} on {q.device} "
                         f"(the forward's LSE of fixed-length inputs)")


def bwd_workspace(q, *, causal=False, sm_scale=None):
    """A workspace for a training step: pass it to sageattn(..., workspace=) and then to
    attn_bwd(..., fwd_workspace=), so the backward reuses the forward's quantization."""
    B, H, N, d = q.shape
    p = problem(B, H, N, d, causal=causal, sm_scale=sm_scale, dtype=q.dtype)
    nbytes = ctypes.c_size_t()
    _check(lib().sage_attn_bwd_ws_size(ctypes.byref(p), ctypes.byref(nbytes)))
    return torch.empty(max(nbytes.value, 16), dtype=torch.uint8, device=q.device)


def attn_bwd(q, k, v, o, do, lse, *, causal=False, sm_scale=None, fwd_workspace=None):
    """8-bit backward: returns dQ, dK, dV in the input dtype.  fwd_workspace: the workspace the
    forward of these q, k, v wrote (bwd_workspace); its quantization of Q and K is then reused
    (sage_attn_bwd_after_fwd) instead of recomputed."""
    q, k, v = _qkv(q, k, v)
    B, H, N, d = q.shape
    check_bwd_inputs(q, o, do, lse)
    p = problem(B, H, N, d, causal=causal, sm_scale=sm_scale, dtype=q.dtype)
    nbytes = ctypes.c_size_t()
    _check(lib().sage_attn_bwd_ws_size(ctypes.byref(p), ctypes.byref(nbytes)))
    if fwd_workspace is not None:
        if (fwd_workspace.dtype != torch.uint8 or fwd_workspace.device != q.device or
                fwd_workspace.numel() < nbytes.value or not fwd_workspace.is_contiguous()):
            raise ValueError("fwd_workspace must be a contiguous uint8 tensor on q's device of at least "
                             f"{nbytes.value} bytes (bwd_workspace)")
        ws, fn = fwd_workspace, lib().sage_attn_bwd_after_fwd
    else:
        ws, fn = torch.empty(max(nbytes.value, 16), dtype=torch.uint8, device=q.device), lib().sage_attn_bwd
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    o, do, lse = o.contiguous(), do.contiguous(), lse.contiguous()
    _check(fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream()))
    return dq, dk, dv


class SageAttnFn(torch.autograd.Function):
    """Training attention: 8-bit forward (INT8 QK, FP8 P~V) and 8-bit backward."""

    @staticmethod
    def forward(ctx, q, k, v, causal=False, sm_scale=None):
        # the forward quantizes into a backward-sized workspace that the backward then reuses
        ws = bwd_workspace(q, causal=causal, sm_scale=sm_scale)
        o, lse = sageattn(q, k, v, causal=causal, sm_scale=sm_scale, return_lse=True, workspace=ws)
        ctx.save_for_backward(q, k, v, o, lse, ws)
        ctx.causal, ctx.sm_scale = causal, sm_scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, ws = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q, k, v, o, do, lse, causal=ctx.causal, sm_scale=ctx.sm_scale, fwd_workspace=ws)
        return dq, dk, dv, None, None
