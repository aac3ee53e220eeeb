"""Pins of the oracle's element codecs against brute force, library routines and
closed forms (OCP E4M3FN, OCP MX E2M1 + E8M0, symmetric INT8)."""
import math

import numpy as np
import torch


def _all_finite_16bit():
    u = np.arange(65536, dtype=np.uint16)
    f16 = u.view(np.float16).astype(np.float64)
    bf = (u.astype(np.uint32) << 16).view(np.float32)
    bf = bf[np.isfinite(bf)].astype(np.float64)
    xs = np.concatenate([f16, bf])
    return xs[np.isfinite(xs)]


def _nearest_even(table_vals, table_codes, xs):
    """Brute-force nearest magnitude in a decode table; ties go to the even code."""
    a = np.abs(xs)[:, None]
    dist = np.abs(a - table_vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates prefer an even code, then the smaller code
    pref = np.where(cand, (table_codes[None, :] & 1) * 1000 + table_codes[None, :], 10**9)
    pick = table_codes[np.argmin(pref, axis=1)]
    return pick


def test_e4m3_decode_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.all(both_nan | (mine == ref))


def test_e4m3_encode_exhaustive_16bit_brute_force(orc):
    xs = _all_finite_16bit()
    big = xs[np.abs(xs) > 1024]          # beyond: saturation (distances below are exact in fp64)
    assert np.all((orc.e4m3_encode(big) & 0x7F) == 0x7E)
    xs = xs[np.abs(xs) <= 1024]
    codes = np.arange(0x7F, dtype=np.int64)             # finite non-negative codes 0x00..0x7E
    vals = orc.e4m3_decode(codes.astype(np.uint8))
    want = _nearest_even(vals, codes, xs) | np.where(np.signbit(xs), 0x80, 0)
    got = orc.e4m3_encode(xs)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs[i], got[i], want[i]) for i in bad[:10]]


def test_e4m3_encode_matches_torch_in_range(orc):
    xs = _all_finite_16bit()
    xs = xs[np.abs(xs) <= 448.0]
    got = orc.e4m3_encode(xs)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_saturates_and_keeps_sign(orc):
    assert orc.e4m3_encode(np.array([500.0, 1e30, -1e30, 448.0, -0.0])).tolist() == [0x7E, 0x7E, 0xFE, 0x7E, 0x80]


def test_e2m1_table_and_ties(orc):
    assert orc.e2m1_decode(np.arange(8, dtype=np.uint8)).tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert orc.e2m1_decode(np.arange(8, 16, dtype=np.uint8)).tolist() == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    # midpoints between neighbours round to the even mantissa
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert orc.e2m1_decode(orc.e2m1_encode(mids)).tolist() == [0, 1, 1, 2, 2, 4, 4]


def test_e2m1_encode_exhaustive_brute_force(orc):
    xs = _all_finite_16bit()
    xs = xs[np.abs(xs) < 64]
    codes = np.arange(8, dtype=np.int64)
    vals = orc.e2m1_decode(codes.astype(np.uint8))
    want = _nearest_even(vals, codes, xs) | np.where(np.signbit(xs), 8, 0)
    got = orc.e2m1_encode(xs)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs[i], got[i], want[i]) for i in bad[:10]]


def test_mx_scale_byte_against_frexp(orc):
    rng = np.random.default_rng(0)
    vals = np.concatenate([np.exp2(rng.uniform(-140, 120, 2000)).astype(np.float32).astype(np.float64),
                           [1.0, 6.0, 4.0, 7.99, 8.0, 448.0, 2.0 ** -149]])
    for a in vals:
        for emax in (2, 8):
            e = math.frexp(a)[1] - 1 - emax
            e = max(-127, min(127, e))
            assert orc.mx_scale_byte(a, emax) == e + 127
    assert orc.mx_scale_byte(0.0, 2) == 0


def test_mx_block_max_lands_in_top_binade(orc):
    """With e = floor(log2 amax) - 2 the block max scales into [4, 8): it maps to 4 or 6
    (or saturates to 6), never above the E2M1 range."""
    rng = np.random.default_rng(1)
    for a in np.exp2(rng.uniform(-20, 20, 500)):
        e = orc.mx_scale_byte(a, 2) - 127
        y = a * 2.0 ** -e
        assert 4.0 <= y < 8.0
        assert orc.e2m1_decode(orc.e2m1_encode(np.array([y])))[0] in (4.0, 6.0)


def test_int8_encode_properties(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(4000).astype(np.float32) * np.float32(3.0)
    a = np.float32(np.max(np.abs(x)))
    delta = np.float32(a / np.float32(127.0))
    codes = np.array([orc.int8_encode(v, delta) for v in x])
    assert codes.min() >= -127 and codes.max() <= 127
    assert abs(codes[np.argmax(np.abs(x))]) == 127
    # reconstruction error at most half a step (plus fp32 rounding of x/delta)
    err = np.abs(codes * np.float64(delta) - x.astype(np.float64))
    assert np.all(err <= 0.5 * float(delta) * (1 + 1e-6))
    # odd symmetry and zero step
    assert all(orc.int8_encode(-v, delta) == -orc.int8_encode(v, delta) for v in x[:200])
    assert orc.int8_encode(1.5, 0.0) == 0
    # exact halves round to even
    assert orc.int8_encode(2.5, 1.0) == 2 and orc.int8_encode(3.5, 1.0) == 4 and orc.int8_encode(-2.5, 1.0) == -2


def test_int8_encode_nonfinite(orc):
    """Non-finite quotients: the clamp is fmax / fmin (IEEE maxNum / minNum return the non-NaN
    operand), so NaN clamps to -127 and +-Inf to +-127; a finite x over an infinite step is 0."""
    nan, inf = float("nan"), float("inf")
    assert orc.int8_encode(nan, 0.5) == -127
    assert orc.int8_encode(inf, 0.5) == 127 and orc.int8_encode(-inf, 0.5) == -127
    assert orc.int8_encode(1.0, inf) == 0 and orc.int8_encode(-3.0, inf) == 0
    assert orc.int8_encode(inf, inf) == -127          # inf / inf = NaN
    assert orc.mx_scale_byte(nan, 2) == 0xFF and orc.mx_scale_byte(inf, 2) == 0xFF


def test_widen_matches_numpy_and_torch(orc):
    u = np.arange(65536, dtype=np.uint16)
    f = orc.widen(u, "f16")
    ref = u.view(np.float16).astype(np.float32)
    assert np.array_equal(np.isnan(f), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(f[ok].view(np.uint32), ref[ok].view(np.uint32))
    b = orc.widen(u, "bf16")
    refb = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    okb = ~np.isnan(refb)
    assert np.array_equal(b[okb].view(np.uint32), refb[okb].view(np.uint32))


def test_mx_e4m3_v_groups_against_frexp_and_torch(orc):
    """MXFP8 V: per channel per 32-token group, E8M0 = floor(log2 amax) - 8 (from frexp) and
    E4M3 codes of v * 2^-e, saturated at 448 (torch's float8_e4m3fn cast after clamping);
    the last group is ragged."""
    import torch
    rng = np.random.default_rng(7)
    BH, N, d = 2, 100, 64
    v = (rng.standard_normal((BH, N, d)) * 2.0 ** rng.integers(-6, 6, size=(BH, 1, d))).astype(np.float32)
    v[0, 40:64, 3] = 0.0
    v[0, 32:40, 3] = 0.0                                       # one all-zero group
    z = np.zeros_like(v)
    r = orc.quant_mxfp4(z, z, v, 0.1, pv_fmt="mxfp8")
    for h in range(BH):
        for g0 in range(0, N, 32):
            blk = v[h, g0:g0 + 32].astype(np.float64)            # [n, d]
            for c in range(d):
                a = np.abs(blk[:, c]).max()
                if a == 0.0:
                    assert r["ve"][h, g0 // 32, c] == 0
                    assert not (r["vc"][h, g0:g0 + 32, c] & 0x7f).any()
                    continue
                e = math.frexp(a)[1] - 1 - 8
                assert r["ve"][h, g0 // 32, c] == e + 127
                y = np.clip(blk[:, c] * 2.0 ** -e, -448.0, 448.0)
                want = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                assert np.array_equal(r["vc"][h, g0:g0 + 32, c], want)


def test_f16_decode_all_codes_against_numpy(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = codes.view(np.float16).astype(np.float64)
    got = orc.f16_decode(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_f16_encode_against_numpy_rounding(orc):
    """Round to nearest even with subnormals and overflow to infinity, checked against
    numpy's float64 -> float16 conversion on random values, exact ties and the edges."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(20000) * 2.0 ** rng.integers(-30, 18, size=20000)
    grid = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    grid = grid[np.isfinite(grid)]
    g = np.sort(np.unique(np.abs(grid)))
    ties = (g[:-1] + g[1:]) / 2                              # exact midpoints (ties)
    edges = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e6, 2.0 ** -24, 2.0 ** -25, 2.0 ** -26, 0.0, -0.0])
    x = np.concatenate([x, ties[::7], -ties[::11], edges, -edges])
    with np.errstate(over="ignore"):                          # the overflow cases are intended
        want = x.astype(np.float16).view(np.uint16)
    got = orc.f16_encode(x)
    assert np.array_equal(got, want)
