"""Helpers for the GPU parity tests: unpacking the device buffer layouts into the
oracle's plain [BH, N, d] arrays, metrics, and a case banner.  No attention or
quantization arithmetic lives here."""
import math
import sys

import numpy as np
import torch


def banner(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def part(buf_np, lay, name, dtype, count):
    off = lay[name]
    return np.frombuffer(buf_np, dtype=dtype, count=count, offset=off)


def unpack_nibbles(packed, n):
    """Bytes with element 2i in the low nibble of byte i -> one code per byte (last axis n)."""
    lo = packed & 0x0F
    hi = packed >> 4
    out = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (2 * packed.shape[-1],))
    return out[..., :n]


def unpack_int8_fp8(buf, p, lay, pv="fp8", fine=False):
    """Device quant buffer (INT8 QK; FP8 or fp16 V) -> dict of oracle-shaped arrays.  fine: a step
    per query token and per 32 keys instead of per 64 tokens."""
    b = buf.cpu().numpy()
    BH, N, d = p.B * p.H, p.N, p.d
    Np = (N + 127) // 128 * 128
    nb = Np // 64
    r = {"mu_k": part(b, lay, "mu_k", np.float32, BH * d).reshape(BH, d)}
    r["qc_all"] = part(b, lay, "q_codes", np.int8, BH * Np * d).reshape(BH, Np, d)
    r["kc_all"] = part(b, lay, "k_codes", np.int8, BH * Np * d).reshape(BH, Np, d)
    r["qc"], r["kc"] = r["qc_all"][:, :N], r["kc_all"][:, :N]
    nq, nk = (Np, Np // 32) if fine else (nb, nb)
    r["qs_all"] = part(b, lay, "q_scales", np.float32, BH * nq).reshape(BH, nq)
    r["ks_all"] = part(b, lay, "k_scales", np.float32, BH * nk).reshape(BH, nk)
    r["qs"] = r["qs_all"][:, :N] if fine else r["qs_all"][:, :(N + 63) // 64]
    r["ks"] = r["ks_all"][:, :(N + 31) // 32] if fine else r["ks_all"][:, :(N + 63) // 64]
    if pv == "f16":
        vt = part(b, lay, "v_codes", np.uint16, BH * Np * d).reshape(BH, Np // 64, d, 64)
        r["vh_all"] = vt.transpose(0, 1, 3, 2).reshape(BH, Np, d)
        r["vh"] = r["vh_all"][:, :N]
    else:
        vt = part(b, lay, "v_codes", np.uint8, BH * Np * d).reshape(BH, Np // 64, d, 64)
        r["vc_all"] = vt.transpose(0, 1, 3, 2).reshape(BH, Np, d)
        r["vc"] = r["vc_all"][:, :N]
        r["vs"] = part(b, lay, "v_scales", np.float32, BH * d).reshape(BH, d)
    r["corr"] = part(b, lay, "lse_corr", np.float32, BH * N).reshape(BH, N)
    return r


def unpack_mxfp4(buf, p, lay, pv_fmt, qblock=False):
    """qblock: Q smoothed per 128-query block (mu_q [BH, NB, d], dS [BH, NB, N])."""
    b = buf.cpu().numpy()
    BH, N, d = p.B * p.H, p.N, p.d
    Np = (N + 127) // 128 * 128
    nb = Np // 128 if qblock else 1
    r = {"mu_k": part(b, lay, "mu_k", np.float32, BH * d).reshape(BH, d),
         "mu_q": part(b, lay, "mu_q", np.float32, BH * nb * d).reshape((BH, nb, d) if qblock else (BH, d))}
    for t in ("q", "k"):
        pk = part(b, lay, f"{t}_codes", np.uint8, BH * Np * d // 2).reshape(BH, Np, d // 2)
        r[f"{t}c_all"] = unpack_nibbles(pk, d)
        r[f"{t}c"] = r[f"{t}c_all"][:, :N]
        r[f"{t}e_all"] = part(b, lay, f"{t}_scales", np.uint8, BH * Np * d // 32).reshape(BH, Np, d // 32)
        r[f"{t}e"] = r[f"{t}e_all"][:, :N]
    if qblock:
        r["dS_all"] = part(b, lay, "delta_s", np.float32, BH * nb * Np).reshape(BH, nb, Np)
        r["dS"] = r["dS_all"][:, :, :N]
    else:
        r["dS_all"] = part(b, lay, "delta_s", np.float32, BH * Np).reshape(BH, Np)
        r["dS"] = r["dS_all"][:, :N]
    r["corr"] = part(b, lay, "lse_corr", np.float32, BH * N).reshape(BH, N)
    if pv_fmt in ("fp8", "mxfp8"):
        vt = part(b, lay, "v_codes", np.uint8, BH * Np * d).reshape(BH, Np // 64, d, 64)
        r["vc_all"] = vt.transpose(0, 1, 3, 2).reshape(BH, Np, d)
        r["vc"] = r["vc_all"][:, :N]
        if pv_fmt == "fp8":
            r["vs"] = part(b, lay, "v_scales", np.float32, BH * d).reshape(BH, d)
        else:
            ve = part(b, lay, "v_scales", np.uint8, BH * (Np // 32) * d).reshape(BH, Np // 32, d)
            r["ve"] = ve[:, :(N + 31) // 32]
    else:
        vt = part(b, lay, "v_codes", np.uint8, BH * Np * d // 2).reshape(BH, Np // 64, d, 32)
        codes = unpack_nibbles(vt, 64)                       # [BH, Np/64, d, 64 tokens]
        r["vc"] = codes.transpose(0, 1, 3, 2).reshape(BH, Np, d)[:, :N]
        ve = part(b, lay, "v_scales", np.uint8, BH * (Np // 32) * d).reshape(BH, Np // 32, d)
        r["ve"] = ve[:, :(N + 31) // 32]
    return r


def cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / math.sqrt((a @ a) * (b @ b)))


def to_np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def sample_rows(N, k=24, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 127, 128, N // 2, N - 65, N - 64, N - 2, N - 1]
    rows = sorted({r for r in fixed if 0 <= r < N} | set(rng.integers(0, N, size=k).tolist()))
    return np.array(rows, np.int32)


def device():
    return torch.device("cuda:0")


ATOL = 2e-2     # the forward's max-abs tolerance against the oracle's simulation


def within(o, o_sim, slack, atol=ATOL):
    """Element-wise |o - o_sim| <= atol + slack, where slack is the oracle's per-element bound on
    what a different choice among the admissible P~ codes can change (zero almost everywhere)."""
    o = np.asarray(o, np.float64)
    return bool(np.all(np.abs(o - o_sim) <= atol + slack))


def excess(o, o_sim, slack, atol=ATOL):
    """The largest amount by which |o - o_sim| exceeds atol + slack (<= 0 when within)."""
    return float((np.abs(np.asarray(o, np.float64) - o_sim) - atol - slack).max())
