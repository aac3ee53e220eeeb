"""Seeded synthetic inputs for the quantized-attention workloads.

This module only draws random numbers and casts them to the I/O dtype; it
holds none of the attention or quantization arithmetic, so both the HIP path
and the CPU oracle can take their inputs from it.

Draw order (PCG64 via ``numpy.random.default_rng(seed)``, float32, C order):
Q, K, V, [dO], then the per-channel K offsets (shape [B,H,1,d], shared by
every token), then the outlier channel picks (first for Q, then for K).  With
``stress=True`` the three tensors are drawn as the SageAttention kernel
accuracy protocol describes them (SageAttention paper, reviewer tyTT reply,
accuracy table): standard normal with 1 % of the entries replaced by draws
from N(1, 10); the replacement masks and values are drawn after the offsets.
N(a, b) means mean a and standard deviation b.  Values are cast to bf16/fp16
with round-to-nearest-even (torch CPU ``.to``).

The named workloads stand in for the LLM-prefill and video-diffusion attention
shapes the pages evaluate on; no weights or datasets are involved.
"""
import math

import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}

# Workloads by name: shape, mask, formats and the generator recipe.
WORKLOADS = {
    # INT8-QK / FP8-PV, smoothing exercised by a per-channel K offset.
    "int8_fp8_b1h2n256d64": dict(B=1, H=2, N=256, d=64, causal=False, dtype="f16",
                                 qk_fmt="int8", pv_fmt="fp8", seed=0, k_off_std=4.0,
                                 outlier_frac=0.0, sm_scale=1.0 / 8),
    # LLM-prefill shape, causal, with 1 % outlier channels in Q and K.
    "int8_fp8_causal_b1h32n4096d128": dict(B=1, H=32, N=4096, d=128, causal=True, dtype="bf16",
                                           qk_fmt="int8", pv_fmt="fp8", seed=1, k_off_std=5.0,
                                           outlier_frac=0.01, sm_scale=1.0 / math.sqrt(128)),
    # Video-diffusion shape.
    "int8_fp8_b2h24n16384d64": dict(B=2, H=24, N=16384, d=64, causal=False, dtype="bf16",
                                    qk_fmt="int8", pv_fmt="fp8", seed=2, k_off_std=3.0,
                                    outlier_frac=0.0, sm_scale=1.0 / 8),
    # Microscaled FP4 forward.
    "mxfp4_b4h32n8192d128": dict(B=4, H=32, N=8192, d=128, causal=False, dtype="bf16",
                                 qk_fmt="mxfp4", pv_fmt="mxfp4", seed=3, k_off_std=5.0,
                                 outlier_frac=0.0, sm_scale=1.0 / math.sqrt(128)),
    # 8-bit training forward + backward.
    "train_causal_b8h16n2048d64": dict(B=8, H=16, N=2048, d=64, causal=True, dtype="bf16",
                                       qk_fmt="int8", pv_fmt="fp8", seed=4, k_off_std=0.0,
                                       outlier_frac=0.0, sm_scale=1.0 / 8, with_do=True),
    # The same training shape at head dimension 128.
    "train_causal_b8h16n2048d128": dict(B=8, H=16, N=2048, d=128, causal=True, dtype="bf16",
                                        qk_fmt="int8", pv_fmt="fp8", seed=7, k_off_std=0.0,
                                        outlier_frac=0.0, sm_scale=1.0 / math.sqrt(128), with_do=True),
    # Long-sequence d=128 INT8/FP8 sweep points (LLM-prefill generator).
    "int8_fp8_b1h32n8192d128": dict(B=1, H=32, N=8192, d=128, causal=False, dtype="bf16",
                                    qk_fmt="int8", pv_fmt="fp8", seed=5, k_off_std=5.0,
                                    outlier_frac=0.01, sm_scale=1.0 / math.sqrt(128)),
    "int8_fp8_causal_b1h32n16384d128": dict(B=1, H=32, N=16384, d=128, causal=True, dtype="bf16",
                                            qk_fmt="int8", pv_fmt="fp8", seed=5, k_off_std=5.0,
                                            outlier_frac=0.01, sm_scale=1.0 / math.sqrt(128)),
}


def make_inputs(B, H, N, d, *, dtype="bf16", seed=0, k_off_std=0.0, q_off_std=0.0,
                outlier_frac=0.0, with_do=False, stress=False):
    """Return a dict of CPU tensors q, k, v (and do) of shape [B,H,N,d] in ``dtype``."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32) if with_do else None
    if k_off_std > 0:
        k += rng.normal(0.0, k_off_std, size=(B, H, 1, d)).astype(np.float32)
    if q_off_std > 0:
        q += rng.normal(0.0, q_off_std, size=(B, H, 1, d)).astype(np.float32)
    n_out = int(round(outlier_frac * B * H * d))
    if n_out > 0:
        for x in (q, k):
            pick = rng.choice(B * H * d, size=n_out, replace=False)
            xv = x.transpose(0, 1, 3, 2).reshape(B * H * d, N)  # view: one row per (b,h,c)
            xv[pick, :] *= 10.0
    if stress:
        for x in (q, k, v):
            mask = rng.random(shape) < 0.01
            x[mask] = rng.normal(1.0, 10.0, size=int(mask.sum())).astype(np.float32)
    tdt = DTYPES[dtype]
    out = {"q": torch.from_numpy(q).to(tdt), "k": torch.from_numpy(k).to(tdt),
           "v": torch.from_numpy(v).to(tdt)}
    if do is not None:
        out["do"] = torch.from_numpy(do).to(tdt)
    return out


def workload_inputs(name, **override):
    """Inputs of a named workload (sizes may be overridden for small parity cases)."""
    w = dict(WORKLOADS[name])
    w.update(override)
    return make_inputs(w["B"], w["H"], w["N"], w["d"], dtype=w["dtype"], seed=w["seed"],
                       k_off_std=w.get("k_off_std", 0.0), outlier_frac=w.get("outlier_frac", 0.0),
                       with_do=w.get("with_do", False)), w


def as_u16(t):
    """Raw 16-bit patterns of a bf16/fp16 CPU tensor as a numpy uint16 array (no copy of values)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# Packed (cu_seqlens) workloads: a batch of prefill sequences of mixed lengths with grouped KV
# heads, as an LLM serving step packs them.
VARLEN_WORKLOADS = {
    "varlen_gqa_causal_b8h32kv8t16384d128": dict(lens=[3072, 256, 4096, 1000, 2048, 777, 3135, 2000],
                                                 H=32, Hkv=8, d=128, causal=True, dtype="bf16", seed=6,
                                                 k_off_std=5.0, outlier_frac=0.01, sm_scale=1.0 / math.sqrt(128)),
}


def varlen_workload(name):
    """Packed inputs: q [T,H,d], k and v [T,Hkv,d] CPU tensors, int32 cu_q = cu_k [B+1].
    Draw order: Q, K, V, the per-(KV head, channel) K offsets, the outlier picks (Q, then K)."""
    w = dict(VARLEN_WORKLOADS[name])
    lens, H, Hkv, d = w["lens"], w["H"], w["Hkv"], w["d"]
    T = int(sum(lens))
    rng = np.random.default_rng(w["seed"])
    q = rng.standard_normal((T, H, d), dtype=np.float32)
    k = rng.standard_normal((T, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((T, Hkv, d), dtype=np.float32)
    k += rng.normal(0.0, w["k_off_std"], size=(1, Hkv, d)).astype(np.float32)
    for x in (q, k):
        hc = x.shape[1] * d
        n_out = int(round(w["outlier_frac"] * hc))
        pick = rng.choice(hc, size=n_out, replace=False)
        xv = x.reshape(T, hc)
        xv[:, pick] *= 10.0
    tdt = DTYPES[w["dtype"]]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    x = {"q": torch.from_numpy(q).to(tdt), "k": torch.from_numpy(k).to(tdt), "v": torch.from_numpy(v).to(tdt),
         "cu_q": cu, "cu_k": cu.clone()}
    w.update(B=len(lens), T=T, max_seqlen=int(max(lens)))
    return x, w
