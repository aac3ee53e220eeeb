"""Exhaustive on-device codec parity: every finite 16-bit input pattern (bf16 and fp16) in
range passes through the device quantizers -- the correctly rounded division and round-to-
nearest-even of the INT8 codes, the FP8 (E4M3) conversion of V, the scaled FP4 (E2M1)
conversion of Q, K and V, and the MXFP8 V conversion -- and every code and step must equal
the oracle's encoders bit for bit (those encoders are pinned exhaustively against brute-force
nearest search on the CPU).  The input designs fix the quantization steps so that each
pattern, including every rounding midpoint the 16-bit formats hold, reaches the converter
(codec_inputs.py)."""
import numpy as np
import pytest
import torch

import codec_inputs as ci
from gpu_util import banner, device, unpack_int8_fp8, unpack_mxfp4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_smooth_amd as S
    S.lib()
    return S


def _to_dev(x, dtype):
    """The exact 16-bit patterns of x as a device tensor [1, H, N, d], built from the bits (a
    float conversion on the host may flush subnormals)."""
    t = torch.from_numpy(ci.to_bits(x, dtype).view(np.int16)).view(ci.TDT[dtype])
    return t.unsqueeze(0).to(device())


AMAX, GMAX = ci.AMAX, ci.GMAX


@pytest.mark.parametrize("qk", ["int8", "int8_token"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_int8_and_fp8_codecs_every_pattern(sage, dtype, qk):
    """qk int8: a step per 64 tokens (A / 127 by design); int8_token: a step per query token and
    per 32 keys, so the same patterns also meet the steps of each row's own maximum."""
    import oracle
    banner(f"exhaustive INT8 / FP8 codecs {dtype} {qk}")
    q, k, v = ci.int8_fp8(dtype, AMAX[dtype])
    H, N, d = q.shape
    sm = 0.125
    buf, p, lay = sage.quantize(_to_dev(q, dtype), _to_dev(k, dtype), _to_dev(v, dtype), sm_scale=sm,
                                qk_fmt=qk, pv_fmt="fp8")
    torch.cuda.synchronize()
    fine = qk == "int8_token"
    r = unpack_int8_fp8(buf, p, lay, "fp8", fine=fine)
    qz = oracle.quant_int8_fp8(q, k, v, sm, qblk=1 if fine else 64, kblk=32 if fine else 64)
    for key in ("qs", "qc", "vs", "vc", "mu_k", "ks", "kc"):
        assert np.array_equal(r[key], qz[key]), (key, int((r[key] != qz[key]).sum()))
    # the designs really put the patterns through fixed steps
    assert np.array_equal(qz["vs"], np.repeat(np.float32(AMAX[dtype])[:, None] / np.float32(448), d, 1))




@pytest.mark.parametrize("pv", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mx_codecs_every_pattern(sage, dtype, pv):
    import oracle
    banner(f"exhaustive MX codecs {dtype} V {pv}")
    q, k, v = ci.mx(dtype, GMAX)
    H, N, d = q.shape
    sm = 0.125
    buf, p, lay = sage.quantize(_to_dev(q, dtype), _to_dev(k, dtype), _to_dev(v, dtype), sm_scale=sm,
                                qk_fmt="mxfp4", pv_fmt=pv)
    torch.cuda.synchronize()
    r = unpack_mxfp4(buf, p, lay, pv)
    qz = oracle.quant_mxfp4(q, k, v, sm, pv_fmt=pv)
    assert not qz["mu_q"].any() and not qz["mu_k"].any()          # smoothing is the identity here
    for key in ("mu_q", "mu_k", "qe", "qc", "ke", "kc", "ve", "vc"):
        assert np.array_equal(r[key], qz[key]), (key, int((r[key] != qz[key]).sum()))
