"""Inputs that drive every 16-bit input pattern through the device quantizers.

Each builder returns float32 arrays [H, N, d] whose values are exactly representable in the
input dtype (bf16 or fp16).  They only place values: no quantization arithmetic lives here.
The designs fix the quantization steps so that the quantizer sees each pattern directly:
  - int8_fp8(): V's per-channel maximum and Q's per-64-token-block maximum are set to A per
    head (row 0 of V, row 64 b of Q), so the FP8 step A / 448 and the INT8 step A / 127 are
    fixed, and every pattern of magnitude <= A passes through the division and the rounding;
  - mx(): V's 32-token groups (per channel) and the 32-channel groups of Q and K (per row)
    have their maximum G per head, and Q and K are built as rows R followed by -R with values
    in [G 2^-24, G], so every channel sum is exactly 0 in binary64 in any order: the channel
    means are 0 and the smoothed Q and K equal the inputs.
"""
import numpy as np
import torch

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}

# per head: the INT8 block and FP8 channel maximum A (steps A / 127 and A / 448), each a value of
# the dtype: a step of 1 for FP8 (448) or INT8 (127), inexact steps (1), the largest magnitudes
AMAX = {"bf16": [448.0, 127.0, 1.0, 2.0 ** 100], "f16": [448.0, 127.0, 1.0, 30000.0]}
# per head: the MX group maximum G (E2M1: scale 2^(floor(log2 G) - 2); E4M3: 2^(floor(log2 G) - 8))
GMAX = [4.0, 7.5, 0.5, 448.0]


def to_bits(x, dtype):
    """float32 values that the 16-bit dtype holds exactly -> their uint16 patterns (bf16: the top
    half of the binary32 bits; fp16: numpy's conversion, exact for representable values)."""
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32)
        bad = np.flatnonzero(u & 0xFFFF)
        assert bad.size == 0, f"not a bf16 value: {x.ravel()[bad[:4]]} ({bad.size} elements)"
        return (u >> 16).astype(np.uint16)
    h = x.astype(np.float16)
    bad = np.flatnonzero(h.astype(np.float32) != x)
    assert bad.size == 0, f"not an fp16 value: {x.ravel()[bad[:4]]} ({bad.size} elements)"
    return h.view(np.uint16)


def from_bits(u, dtype):
    """uint16 patterns -> their float32 values, by bit manipulation only (bf16: the top half of a
    binary32; fp16: numpy's half-precision widening, exact for every pattern)."""
    u = np.asarray(u, np.uint16)
    if dtype == "bf16":
        return (u.astype(np.uint32) << 16).view(np.float32)
    return u.view(np.float16).astype(np.float32)


def patterns(dtype, hi, lo=0.0):
    """Every finite pattern of the 16-bit dtype with magnitude in [lo, hi], both signs, and 0.
    The patterns are non-negative bit strings below the sign bit, so they ascend with magnitude."""
    u = np.arange(1, 0x8000, dtype=np.uint16)
    f = from_bits(u, dtype)
    keep = np.isfinite(f) & (f >= lo) & (f <= hi)
    u = u[keep]
    return from_bits(np.concatenate([np.zeros(1, np.uint16), u, u | np.uint16(0x8000)]), dtype)


def _fill(rows, d, vals, skip):
    """rows x d array holding vals in row-major order, skipping the rows in `skip` (set later)."""
    out = np.zeros((rows, d), np.float32)
    free = [r for r in range(rows) if r not in skip]
    flat = np.zeros(len(free) * d, np.float32)
    assert len(vals) <= flat.size
    flat[:len(vals)] = vals
    out[free] = flat.reshape(len(free), d)
    return out


def int8_fp8(dtype, amaxes, d=64, seed=0):
    """(q, k, v) [H, N, d] for INT8 Q and FP8 V codecs: head h has Q block maxima and V channel
    maxima A = amaxes[h]; K is random."""
    lists = [patterns(dtype, a) for a in amaxes]
    need = max(len(v) for v in lists)
    N = 64 * int(np.ceil((need / d + 1) / 63 + 1))
    H = len(amaxes)
    q = np.zeros((H, N, d), np.float32)
    v = np.zeros((H, N, d), np.float32)
    for h, (a, vals) in enumerate(zip(amaxes, lists)):
        qb = set(range(0, N, 64))
        q[h] = _fill(N, d, vals, qb)
        q[h, sorted(qb), :] = a
        v[h] = _fill(N, d, vals, {0})
        v[h, 0, :] = a
    k = np.random.default_rng(seed).standard_normal((H, N, d)).astype(np.float32)
    if dtype == "bf16":
        k = from_bits((k.view(np.uint32) >> 16).astype(np.uint16), dtype)   # truncated to bf16
    else:
        k = k.astype(np.float16).astype(np.float32)
    return q, k, v


def mx(dtype, gmaxes, d=64):
    """(q, k, v) [H, N, d] for MX codecs: head h has group maxima G = gmaxes[h] in V (32 tokens
    per channel) and in Q and K (32 channels per row); Q and K have channel sums exactly 0."""
    H = len(gmaxes)
    vlists = [patterns(dtype, g) for g in gmaxes]
    qlists = [patterns(dtype, g, lo=g * 2.0 ** -24) for g in gmaxes]
    nv = max(len(x) for x in vlists)
    nq = max(len(x) for x in qlists)
    half = int(np.ceil(nq / (d - d // 32)))
    N = 64 * int(np.ceil(max(2 * half, nv / (d * 31 / 32) + 32) / 64))
    half = N // 2
    q = np.zeros((H, N, d), np.float32)
    v = np.zeros((H, N, d), np.float32)
    for h, g in enumerate(gmaxes):
        gm = set(range(0, N, 32))
        v[h] = _fill(N, d, vlists[h], gm)
        v[h, sorted(gm), :] = g
        r = _fill(half, d - d // 32, qlists[h], set())
        rr = np.zeros((half, d), np.float32)
        keep = [c for c in range(d) if c % 32]
        rr[:, keep] = r
        rr[:, ::32] = g
        q[h] = np.concatenate([rr, -rr])
    k = np.ascontiguousarray(q[:, ::-1])
    return q, k, v
