"""CPU oracle for SageAttention-style quantized attention (test infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
use this package; the library's product path never imports it.  The numeric
work is plain C in ``sage_oracle.c`` (fp64 unless the format fixes fp32),
loaded here through ctypes.  This file marshals numpy arrays to it and, for
packed sequences, slices each sequence out of the packed arrays and repeats KV
heads for grouped-query attention (attn_varlen); it holds no other arithmetic.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build():
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.or_e4m3_decode.restype = ctypes.c_double
        L.or_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.or_e4m3_encode.restype = ctypes.c_uint8
        L.or_e4m3_encode.argtypes = [ctypes.c_double]
        L.or_e2m1_decode.restype = ctypes.c_double
        L.or_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.or_e2m1_encode.restype = ctypes.c_uint8
        L.or_e2m1_encode.argtypes = [ctypes.c_double]
        L.or_mx_scale_byte.restype = ctypes.c_uint8
        L.or_mx_scale_byte.argtypes = [ctypes.c_double, ctypes.c_int]
        L.or_f16_decode.restype = ctypes.c_double
        L.or_f16_decode.argtypes = [ctypes.c_uint16]
        L.or_f16_encode.restype = ctypes.c_uint16
        L.or_f16_encode.argtypes = [ctypes.c_double]
        L.or_int8_encode.restype = ctypes.c_int8
        L.or_int8_encode.argtypes = [ctypes.c_float, ctypes.c_float]
        _lib = L
    return _lib


def set_threads(n):
    """Host threads of the oracle's parallel loops (n <= 0 leaves them as they are); returns the
    count in effect.  Results do not depend on it."""
    return int(lib().or_set_threads(int(n)))


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def widen(u16, dtype):
    """bf16 ('bf16') or fp16 ('f16') bit patterns -> float32, exactly."""
    u16 = np.ascontiguousarray(u16, dtype=np.uint16)
    out = np.empty(u16.shape, np.float32)
    lib().or_widen(_p(u16), ctypes.c_int(0 if dtype == "bf16" else 1), _p(out), ctypes.c_int64(u16.size))
    return out


def e4m3_encode(x):
    f = lib().or_e4m3_encode
    return np.array([f(float(v)) for v in np.ravel(x)], np.uint8).reshape(np.shape(x))


def e4m3_decode(c):
    f = lib().or_e4m3_decode
    return np.array([f(int(v)) for v in np.ravel(c)], np.float64).reshape(np.shape(c))


def e2m1_encode(x):
    f = lib().or_e2m1_encode
    return np.array([f(float(v)) for v in np.ravel(x)], np.uint8).reshape(np.shape(x))


def e2m1_decode(c):
    f = lib().or_e2m1_decode
    return np.array([f(int(v)) for v in np.ravel(c)], np.float64).reshape(np.shape(c))


def mx_scale_byte(amax, emax):
    return int(lib().or_mx_scale_byte(float(amax), int(emax)))


def f16_encode(x):
    f = lib().or_f16_encode
    return np.array([f(float(v)) for v in np.ravel(x)], np.uint16).reshape(np.shape(x))


def f16_decode(c):
    f = lib().or_f16_decode
    return np.array([f(int(v)) for v in np.ravel(c)], np.float64).reshape(np.shape(c))


def int8_encode(x, delta):
    return int(lib().or_int8_encode(float(x), float(delta)))


def quant_int8_fp8(q, k, v, sm, blk=64, pv_fmt="fp8", qblk=None, kblk=None):
    """Prologue of the INT8 path: q [BH,Nq,d], k and v [BH,Nk,d] float32.  One step per qblk
    query tokens and per kblk key tokens (both blk unless given).  pv_fmt "fp8": FP8 V codes with
    per-channel steps; "f16": V as fp16 codes (vh) for the 16-bit P~V fallback."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    BH, Nq, d = q.shape
    Nk = k.shape[1]
    qblk = blk if qblk is None else qblk
    kblk = blk if kblk is None else kblk
    nbq, nbk = (Nq + qblk - 1) // qblk, (Nk + kblk - 1) // kblk
    r = dict(mu_k=np.empty((BH, d), np.float32), qc=np.empty((BH, Nq, d), np.int8),
             qs=np.empty((BH, nbq), np.float32), kc=np.empty((BH, Nk, d), np.int8),
             ks=np.empty((BH, nbk), np.float32), vc=np.empty((BH, Nk, d), np.uint8),
             vs=np.empty((BH, d), np.float32), corr=np.empty((BH, Nq), np.float64))
    lib().or_quant_int8_fp8_x(_p(q), _p(k), _p(v), BH, Nq, Nk, d, qblk, kblk, ctypes.c_double(sm),
                              _p(r["mu_k"]), _p(r["qc"]), _p(r["qs"]), _p(r["kc"]), _p(r["ks"]),
                              _p(r["vc"]), _p(r["vs"]), _p(r["corr"]))
    r["pv_fmt"] = pv_fmt
    r["qblk"], r["kblk"] = qblk, kblk
    if pv_fmt == "f16":
        r["vh"] = np.empty((BH, Nk, d), np.uint16)
        lib().or_quant_v_f16(_p(v), ctypes.c_int64(v.size), _p(r["vh"]))
    return r


_PV = {"fp8": 2, "mxfp4": 3, "mxfp8": 4}


def quant_mxfp4(q, k, v, sm, pv_fmt="mxfp4", qsb=0):
    """Prologue of the MXFP4 path: q [BH,Nq,d], k and v [BH,Nk,d] float32 (codes one per byte).
    qsb > 0 smooths Q per block of qsb query tokens: mu_q [BH,nqb,d] and dS [BH,nqb,Nk]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    BH, Nq, d = q.shape
    Nk = k.shape[1]
    ng, nvg = d // 32, (Nk + 31) // 32
    pv = _PV[pv_fmt]
    nqb = max(1, (Nq + qsb - 1) // qsb) if qsb else 1
    r = dict(mu_q=np.empty((BH, nqb, d), np.float32), mu_k=np.empty((BH, d), np.float32),
             qc=np.empty((BH, Nq, d), np.uint8), qe=np.empty((BH, Nq, ng), np.uint8),
             kc=np.empty((BH, Nk, d), np.uint8), ke=np.empty((BH, Nk, ng), np.uint8),
             dS=np.empty((BH, nqb, Nk), np.float32), corr=np.empty((BH, Nq), np.float64),
             vc=np.empty((BH, Nk, d), np.uint8), ve=np.zeros((BH, nvg, d), np.uint8),
             vs=np.zeros((BH, d), np.float32))
    lib().or_quant_mxfp4_x(_p(q), _p(k), _p(v), BH, Nq, Nk, d, pv, int(qsb), ctypes.c_double(sm),
                         _p(r["mu_q"]), _p(r["mu_k"]), _p(r["qc"]), _p(r["qe"]), _p(r["kc"]), _p(r["ke"]),
                         _p(r["dS"]), _p(r["corr"]), _p(r["vc"]), _p(r["ve"]), _p(r["vs"]))
    r["pv_fmt"] = pv_fmt
    r["qsb"] = int(qsb)
    if not qsb:                          # one block: the per-head shapes
        r["mu_q"], r["dS"] = r["mu_q"][:, 0], r["dS"][:, 0]
    return r


def _rows(rows, N):
    rows = np.arange(N, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    assert len(rows) == 0 or (rows.min() >= 0 and rows.max() < N)
    return rows


def attn_int8_fp8(qz, N, d, causal, sm, tile, rows=None, blk=64, slack=False):
    """Tiled quantized forward (INT8 QK; FP8 or fp16 P~V) on a quant_int8_fp8 result (N = query rows).
    Returns (out, lse), or (out, lse, slack) with slack: per output element, how far a different
    choice among the admissible P~ codes could move it (zero for almost every element)."""
    BH, Nq, Nk = qz["qc"].shape[0], qz["qc"].shape[1], qz["kc"].shape[1]
    assert N == Nq
    rows = _rows(rows, N)
    out = np.empty((BH, len(rows), d), np.float64)
    lse = np.empty((BH, len(rows)), np.float64)
    sl = np.empty((BH, len(rows), d), np.float64)
    qblk, kblk = qz.get("qblk", blk), qz.get("kblk", blk)
    if qz.get("pv_fmt", "fp8") == "f16":
        lib().or_attn_int8_f16_x(_p(qz["qc"]), _p(qz["qs"]), _p(qz["kc"]), _p(qz["ks"]), _p(qz["vh"]),
                                 _p(qz["corr"]), BH, Nq, Nk, d, qblk, kblk, tile, int(causal),
                                 ctypes.c_double(sm), _p(rows), len(rows), _p(out), _p(lse), _p(sl))
    else:
        lib().or_attn_int8_fp8_x(_p(qz["qc"]), _p(qz["qs"]), _p(qz["kc"]), _p(qz["ks"]), _p(qz["vc"]),
                                 _p(qz["vs"]), _p(qz["corr"]), BH, Nq, Nk, d, qblk, kblk, tile, int(causal),
                                 ctypes.c_double(sm), _p(rows), len(rows), _p(out), _p(lse), _p(sl))
    return (out, lse, sl) if slack else (out, lse)


def attn_mxfp4(qz, N, d, causal, sm, tile, rows=None, slack=False):
    """Tiled quantized forward (MXFP4 QK; P~V as MXFP4, FP8, or FP8 P~ with MXFP8 V); N = query rows.
    Returns (out, lse), or (out, lse, slack) as attn_int8_fp8."""
    BH, Nq, Nk = qz["qc"].shape[0], qz["qc"].shape[1], qz["kc"].shape[1]
    assert N == Nq
    rows = _rows(rows, N)
    out = np.empty((BH, len(rows), d), np.float64)
    lse = np.empty((BH, len(rows)), np.float64)
    sl = np.empty((BH, len(rows), d), np.float64)
    pv = _PV[qz["pv_fmt"]]
    dS = np.ascontiguousarray(qz["dS"])
    lib().or_attn_mxfp4_x(_p(qz["qc"]), _p(qz["qe"]), _p(qz["kc"]), _p(qz["ke"]), _p(dS), _p(qz["corr"]),
                          _p(qz["vc"]), _p(qz["ve"]), _p(qz["vs"]), pv, qz.get("qsb", 0), BH, Nq, Nk, d, tile, int(causal),
                          ctypes.c_double(sm), _p(rows), len(rows), _p(out), _p(lse), _p(sl))
    return (out, lse, sl) if slack else (out, lse)


def attn_tiled_exact(q, k, v, causal, sm, tile, smooth_q=False, rows=None):
    """The tiled forward with identity codecs (smoothing and its corrections kept, in fp64)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    BH, N, d = q.shape
    rows = _rows(rows, N)
    out = np.empty((BH, len(rows), d), np.float64)
    lse = np.empty((BH, len(rows)), np.float64)
    lib().or_attn_tiled_exact(_p(q), _p(k), _p(v), BH, N, d, tile, int(causal), ctypes.c_double(sm),
                              int(smooth_q), _p(rows), len(rows), _p(out), _p(lse))
    return out, lse


def attn_ref(q, k, v, causal, sm, rows=None):
    """Exact fp64 two-pass attention and LSE for the listed query rows (q [BH,Nq,d], k, v [BH,Nk,d])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    BH, Nq, d = q.shape
    Nk = k.shape[1]
    rows = _rows(rows, Nq)
    out = np.empty((BH, len(rows), d), np.float64)
    lse = np.empty((BH, len(rows)), np.float64)
    lib().or_attn_ref_x(_p(q), _p(k), _p(v), BH, Nq, Nk, d, int(causal), ctypes.c_double(sm),
                        _p(rows), len(rows), _p(out), _p(lse))
    return out, lse


def attn_bwd_ref(q, k, v, do, causal, sm):
    """Exact fp64 gradients dQ, dK, dV of softmax attention."""
    q, k, v, do = _f32(q), _f32(k), _f32(v), _f32(do)
    BH, N, d = q.shape
    dq, dk, dv = (np.empty((BH, N, d), np.float64) for _ in range(3))
    lib().or_attn_bwd_ref(_p(q), _p(k), _p(v), _p(do), BH, N, d, int(causal), ctypes.c_double(sm),
                          _p(dq), _p(dk), _p(dv))
    return dq, dk, dv


# ---------------------------------------------------------------- packed sequences

def _seq_heads(x, c0, c1, Hx, H):
    """Rows [c0, c1) of a packed [total, Hx, d] array as [H, n, d]; with Hx < H each of the
    Hx heads serves H / Hx consecutive query heads (grouped-query attention)."""
    seg = np.ascontiguousarray(np.transpose(x[c0:c1], (1, 0, 2)))
    return np.repeat(seg, H // Hx, axis=0) if Hx != H else seg


def attn_varlen(q, k, v, cu_q, cu_k, causal, sm, qk_fmt="int8", pv_fmt="fp8", tile=64, exact=False, slack=False):
    """Packed sequences: q [total_q,H,d], k and v [total_k,Hkv,d], cu_q / cu_k [B+1].  Sequence b
    is attention of q rows [cu_q[b], cu_q[b+1]) against k, v rows [cu_k[b], cu_k[b+1]), query head
    h reading KV head h // (H / Hkv).  Returns o [total_q,H,d], lse [H,total_q] and the per-sequence
    prologue results (None when exact: the exact fp64 reference); with slack, also the admissible
    P~ slack of every output element ([total_q,H,d], zero for exact).

    Beyond marshalling, this function does the packed-sequence bookkeeping in numpy: it slices each
    sequence out of the packed arrays and repeats each KV head for the query heads that share it,
    then runs the per-sequence prologue and simulation above on the slices."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    total_q, H, d = q.shape
    Hkv = k.shape[1]
    assert H % Hkv == 0
    o = np.zeros((total_q, H, d), np.float64)
    sl = np.zeros((total_q, H, d), np.float64)
    lse = np.full((H, total_q), -np.inf)
    quants = []
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            quants.append(None)
            continue
        qs, ks, vs = _seq_heads(q, q0, q1, H, H), _seq_heads(k, k0, k1, Hkv, H), _seq_heads(v, k0, k1, Hkv, H)
        sb = None
        if exact:
            ob, lb = attn_ref(qs, ks, vs, causal, sm)
            qz = None
        elif qk_fmt in ("int8", "int8_token"):
            fine = qk_fmt == "int8_token"
            qz = quant_int8_fp8(qs, ks, vs, sm, pv_fmt=pv_fmt, qblk=1 if fine else 64, kblk=32 if fine else 64)
            ob, lb, sb = attn_int8_fp8(qz, q1 - q0, d, causal, sm, tile, slack=True)
        else:
            # mxfp4_qblock: Q smoothed per 128-query block counted from the sequence's first query
            qz = quant_mxfp4(qs, ks, vs, sm, pv_fmt=pv_fmt, qsb=128 if qk_fmt == "mxfp4_qblock" else 0)
            ob, lb, sb = attn_mxfp4(qz, q1 - q0, d, causal, sm, tile, slack=True)
        o[q0:q1] = np.transpose(ob, (1, 0, 2))
        if sb is not None:
            sl[q0:q1] = np.transpose(sb, (1, 0, 2))
        lse[:, q0:q1] = lb
        quants.append(qz)
    return (o, lse, quants, sl) if slack else (o, lse, quants)
