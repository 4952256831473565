"""Seeded synthetic inputs for the quantized linear layer.

This module only draws random numbers; it holds none of the method's
arithmetic (no quantisation, packing, smoothing or normalisation).  Both the
HIP path and the CPU oracle receive the arrays it returns, so the two sides
see identical inputs.

Shapes and value distributions follow the LLaMA-7B / LLaMA-13B layers the
pages discuss (q_proj [4096, 4096] in the LMDeploy walkthrough, section 2;
fused QKV and RMSNorm-before-Linear in the FastLLM architecture page, section
5.1; the SmoothQuant W8A8 flow in the LMDeploy W8A8 guide).  No dataset or
trained checkpoint is involved: every tensor is drawn from NumPy's
``default_rng`` with a fixed draw order, so a seed fully determines it.

Weights are float32 [N out, K in] (torch ``Linear`` convention); activations
are float16 [M, K] produced by round-to-nearest-even from float32 draws.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "weight", "activations", "smoothquant_inputs", "config_weight",
    "DECODE_M", "C1", "C2_GATEUP", "C2_DOWN", "C3", "C4", "C5_SHAPES", "C5_M",
]

# (N, K, group) of the configurations
C1 = (4096, 4096, 128)            # LLaMA-7B q_proj, decode GEMV
C2_GATEUP = (22016, 4096, 128)    # LLaMA-7B fused gate/up
C2_DOWN = (4096, 11008, 128)      # LLaMA-7B down_proj
DECODE_M = (1, 4, 8, 16, 32)
C3 = (12288, 4096, 64)            # LLaMA-7B fused QKV, prefill M=512
C4 = dict(m=2048, k=4096, n=11008)
C5_SHAPES = ((13824, 5120), (5120, 13824))   # (N, K) LLaMA-13B MLP up / down
C5_M = (1, 8, 64, 256, 1024)


def weight(rng: np.random.Generator, n: int, k: int, *, base_std: float = 0.02,
           outliers: str | None = "pm0.3", outlier_frac: float = 1e-3) -> np.ndarray:
    """float32 [n, k] ~ N(0, base_std) with a fraction of entries replaced by outliers.

    outliers:
      None       -- no outliers
      "pm0.3"    -- round(frac*n*k) entries, chosen without replacement, set to
                    +0.3 or -0.3 (sign drawn uniformly)
      "normal0.3"-- the same entries replaced by N(0, 0.3) draws
    Draw order: base normals, outlier indices, outlier values.
    """
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(base_std)
    if outliers is None:
        return w
    cnt = int(round(outlier_frac * n * k))
    idx = rng.choice(n * k, size=cnt, replace=False)
    flat = w.reshape(-1)
    if outliers == "pm0.3":
        sign = rng.integers(0, 2, size=cnt).astype(np.float32) * 2 - 1
        flat[idx] = np.float32(0.3) * sign
    elif outliers == "normal0.3":
        flat[idx] = rng.standard_normal(cnt, dtype=np.float32) * np.float32(0.3)
    else:
        raise ValueError(outliers)
    return w


def activations(rng: np.random.Generator, m: int, k: int, *, outlier_channel_frac: float = 0.0,
                outlier_scale: float = 20.0) -> np.ndarray:
    """float16 [m, k] ~ N(0, 1); optionally round(frac*k) channels (columns),
    chosen without replacement, multiplied by outlier_scale before the fp16 cast."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    if outlier_channel_frac > 0:
        cnt = int(round(outlier_channel_frac * k))
        ch = rng.choice(k, size=cnt, replace=False)
        x[:, ch] *= np.float32(outlier_scale)
    return x.astype(np.float16)


def config_weight(name: str, seed: int = 0, **kw) -> np.ndarray:
    """Weight tensor of a named configuration, one generator per tensor."""
    table = {
        "q_proj": (C1[0], C1[1], "pm0.3"),
        "gate_up": (C2_GATEUP[0], C2_GATEUP[1], "pm0.3"),
        "down": (C2_DOWN[0], C2_DOWN[1], "pm0.3"),
        "qkv": (C3[0], C3[1], None),
        "13b_up": (C5_SHAPES[0][0], C5_SHAPES[0][1], "normal0.3"),
        "13b_down": (C5_SHAPES[1][0], C5_SHAPES[1][1], "normal0.3"),
    }
    n, k, outl = table[name]
    tag = sorted(table).index(name)
    rng = np.random.default_rng([seed, 1, tag])
    return weight(rng, n, k, outliers=outl, **kw)


def config_activations(name: str, m: int, k: int, seed: int = 0) -> np.ndarray:
    """Activations for a named configuration (fp16 [m, k])."""
    frac = 0.01 if name == "qkv" else 0.0
    rng = np.random.default_rng([seed, 2, m, k, int(frac * 1000)])
    return activations(rng, m, k, outlier_channel_frac=frac)


def smoothquant_inputs(m: int = C4["m"], k: int = C4["k"], n: int = C4["n"], seed: int = 0):
    """Inputs of the W8A8 SmoothQuant workload.

    X fp16 [m, k]: per-channel magnitudes c ~ lognormal(0, 1), round(0.5% k)
    channels (without replacement) multiplied by 50, X = N(0,1) * c.
    gamma fp16 [k] ~ U(0.5, 1.5) (RMSNorm weight).
    W float32 [n, k] ~ N(0, 0.02).
    Draw order: c, outlier channels, X normals, gamma, W.
    """
    rng = np.random.default_rng([seed, 4])
    c = rng.lognormal(0.0, 1.0, size=k).astype(np.float32)
    cnt = int(round(0.005 * k))
    ch = rng.choice(k, size=cnt, replace=False)
    c[ch] *= np.float32(50.0)
    x = (rng.standard_normal((m, k), dtype=np.float32) * c[None, :]).astype(np.float16)
    gamma = rng.uniform(0.5, 1.5, size=k).astype(np.float16)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    return x, gamma, w
