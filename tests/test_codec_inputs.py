"""CPU checks of the exhaustive codec designs (codec_inputs.py): they hold every pattern they
claim, their values are exact in the 16-bit dtype, and their maxima and channel sums are what
fixes the quantization steps."""
import math

import numpy as np
import pytest
import torch

import codec_inputs as ci


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_patterns_are_every_finite_value(dtype):
    p = ci.patterns(dtype, float("inf"))
    u = np.arange(0, 0x10000, dtype=np.uint16)
    f = torch.from_numpy(u.view(np.int16)).view(ci.TDT[dtype]).float().numpy()
    assert np.array_equal(np.unique(p), np.unique(f[np.isfinite(f)]))
    # the bit-level widening agrees with torch's for every pattern (NaNs aside)
    g = ci.from_bits(u, dtype)
    fin = np.isfinite(f)
    assert np.array_equal(g[fin], f[fin]) and np.array_equal(ci.to_bits(g[fin], dtype), u[fin])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_int8_fp8_design(dtype):
    amax = ci.AMAX[dtype]
    q, k, v = ci.int8_fp8(dtype, amax)
    H, N, d = q.shape
    for h, a in enumerate(amax):
        want = set(ci.patterns(dtype, a).tolist())
        assert want <= set(q[h].ravel().tolist()) and want <= set(v[h].ravel().tolist())
        assert np.all(np.abs(v[h]).max(axis=0) == a)                       # every channel's maximum
        blk = np.abs(q[h]).reshape(N // 64, 64 * d).max(axis=1)
        assert np.all(blk == a)                                             # every 64-token block's
    for x in (q, k, v):
        u = ci.to_bits(x, dtype)                                            # exact 16-bit values
        assert np.array_equal(torch.from_numpy(u.view(np.int16)).view(ci.TDT[dtype]).float().numpy(), x)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mx_design(dtype):
    g = ci.GMAX
    q, k, v = ci.mx(dtype, g)
    H, N, d = q.shape
    for h, gm in enumerate(g):
        assert set(ci.patterns(dtype, gm).tolist()) <= set(v[h].ravel().tolist())
        assert set(ci.patterns(dtype, gm, lo=gm * 2.0 ** -24).tolist()) <= set(q[h].ravel().tolist())
        assert np.all(np.abs(v[h]).reshape(N // 32, 32, d).max(axis=1) == gm)
        for x in (q[h], k[h]):
            assert np.all(np.abs(x).reshape(N, d // 32, 32).max(axis=2) == gm)
            for c in range(d):
                col = x[:, c].astype(np.float64)
                assert math.fsum(col) == 0.0
                s = 0.0
                for t in col:                                               # any order is exact:
                    s += t                                                  # token order
                assert s == 0.0 and col.reshape(8, -1).sum(axis=1).sum() == 0.0   # and chunked
    for x in (q, k, v):
        u = ci.to_bits(x, dtype)                                            # exact 16-bit values
        assert np.array_equal(torch.from_numpy(u.view(np.int16)).view(ci.TDT[dtype]).float().numpy(), x)
