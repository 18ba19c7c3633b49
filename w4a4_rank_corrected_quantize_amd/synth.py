"""Seeded synthetic inputs for the SVDQuant W4A4 linear layer.

This module only draws random numbers and rounds them to the storage dtypes
(bf16 activations / weights / bias).  It holds none of the method's
arithmetic, so both the HIP path (through the binding) and the CPU oracle
consume exactly the same inputs.

The pages ("Bringing Nunchaku 4-bit Diffusion Inference to Diffusers",
section "Quantizing your own model") measure on diffusion transformers whose
weights, prompts and calibration data are not available here; these
generators stand in for them with the shapes of a FLUX-like DiT block:
4608 tokens (a 64x64 patch grid = 4096 image tokens plus 512 text tokens),
hidden size 3072, a fused QKV projection 3072 -> 9216 (the three projections
concatenated along the output dimension, section "Quantizing models with
structural rewrites") and an MLP 3072 -> 12288 -> 3072.

Recipe (every draw in float64 with numpy's PCG64, then rounded
float64 -> float32 -> bf16, each step round-to-nearest-even):
  * seed = 1000 * config_id + stream; stream 0 = X, 1 = W, 2 = bias,
    3 = choice of outlier channels; the second MLP linear uses config 3,
    streams 4 (W) and 5 (bias).
  * "small":  X ~ N(0, 1) with 4 outlier channels scaled x30,
              W ~ N(0, 0.02^2), no bias.
  * DiT layers: X ~ Student-t(nu=4) with 16 outlier channels scaled x50,
              W ~ N(0, 0.02^2), bias ~ N(0, 0.01^2).
  * NF4 weight-only layers (config 5, QKV and fc1 shapes): X ~ N(0, 1), no
              outlier channels, W ~ N(0, 0.02^2), no bias.
The calibration statistic that the packing step consumes (per-channel max
|X|) is taken over the very X of the run: the pages' calibration pass needs
a dataset, and this stands in for it.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


# ---------------------------------------------------------------- dtype helpers

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def f64_to_bf16_bits(a) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 (RNE)."""
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float64).astype(np.float32))


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- layer specs

@dataclass(frozen=True)
class LayerSpec:
    name: str
    config_id: int
    M: int
    K: int
    N: int
    x_dist: str            # "normal" | "student_t4" | "external" (fed by a previous layer)
    n_outliers: int
    outlier_scale: float
    w_std: float = 0.02
    bias_std: Optional[float] = 0.01
    gelu: bool = False
    w_stream: int = 1
    bias_stream: int = 2
    mx: bool = False       # MXFP4 variant of the layer


SPECS = {
    "small": LayerSpec("small", 1, 128, 256, 256, "normal", 4, 30.0, bias_std=None),
    "qkv": LayerSpec("qkv", 2, 4608, 3072, 9216, "student_t4", 16, 50.0),
    "fc1": LayerSpec("fc1", 3, 4608, 3072, 12288, "student_t4", 16, 50.0, gelu=True),
    "fc2": LayerSpec("fc2", 3, 4608, 12288, 3072, "external", 0, 1.0,
                     w_stream=4, bias_stream=5),
    "mx_qkv": LayerSpec("mx_qkv", 4, 4608, 3072, 9216, "student_t4", 16, 50.0, mx=True),
    "mx_fc1": LayerSpec("mx_fc1", 4, 4608, 3072, 12288, "student_t4", 16, 50.0,
                        gelu=True, mx=True, w_stream=5, bias_stream=6),
    "mx_fc2": LayerSpec("mx_fc2", 4, 4608, 12288, 3072, "external", 0, 1.0,
                        mx=True, w_stream=7, bias_stream=8),
    # the same three MXFP4 linears for a 512 x 512 image: 1024 image tokens,
    # text tokens left out
    "mx1k_qkv": LayerSpec("mx1k_qkv", 7, 1024, 3072, 9216, "student_t4", 16, 50.0, mx=True),
    "mx1k_fc1": LayerSpec("mx1k_fc1", 7, 1024, 3072, 12288, "student_t4", 16, 50.0,
                          gelu=True, mx=True, w_stream=5, bias_stream=6),
    "mx1k_fc2": LayerSpec("mx1k_fc2", 7, 1024, 12288, 3072, "external", 0, 1.0,
                          mx=True, w_stream=7, bias_stream=8),
    # weight-only AWQ W4A16 modulation layer: one conditioning vector per
    # image, 3072 -> 6 x 3072 (shift, scale and gate of two norms)
    "awq_mod": LayerSpec("awq_mod", 6, 1, 3072, 18432, "normal", 0, 1.0),
    # weight-only NF4 W4A16 comparison path on the QKV and fc1 shapes:
    # activations N(0, 1) without outlier channels, no bias
    "nf4_qkv": LayerSpec("nf4_qkv", 5, 4608, 3072, 9216, "normal", 0, 1.0, bias_std=None),
    "nf4_fc1": LayerSpec("nf4_fc1", 5, 4608, 3072, 12288, "normal", 0, 1.0, bias_std=None, w_stream=3),
}


def rng_for(config_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(1000 * config_id + stream)


def gen_activation(config_id: int, M: int, K: int, dist: str, n_outliers: int,
                   outlier_scale: float) -> tuple[np.ndarray, np.ndarray]:
    """bf16 activation [M][K] (uint16 bits) and the chosen outlier channels."""
    rng = rng_for(config_id, 0)
    if dist == "normal":
        x = rng.standard_normal((M, K))
    elif dist == "student_t4":
        x = rng.standard_t(4.0, size=(M, K))
    else:
        raise ValueError(f"unknown activation distribution {dist!r}")
    n_out = min(n_outliers, K)
    ch = np.sort(rng_for(config_id, 3).choice(K, n_out, replace=False)) if n_out else \
        np.zeros(0, dtype=np.int64)
    if n_out:
        x[:, ch] *= outlier_scale
    return f64_to_bf16_bits(x), ch


def gen_weight(config_id: int, stream: int, N: int, K: int, std: float) -> np.ndarray:
    """bf16 weight [N][K] (nn.Linear layout: out_features x in_features)."""
    return f64_to_bf16_bits(rng_for(config_id, stream).normal(0.0, std, size=(N, K)))


def gen_bias(config_id: int, stream: int, N: int, std: Optional[float]) -> Optional[np.ndarray]:
    if std is None:
        return None
    return f64_to_bf16_bits(rng_for(config_id, stream).normal(0.0, std, size=(N,)))


def calibration_absmax(X_bits: np.ndarray) -> np.ndarray:
    """Per-channel max |X| over the rows of a bf16 activation (float32, exact)."""
    x = bf16_bits_to_f32(X_bits)
    return np.abs(x).max(axis=0).astype(np.float32) if x.shape[0] else \
        np.zeros(x.shape[1], np.float32)


def make_layer(spec: LayerSpec, M: Optional[int] = None, K: Optional[int] = None,
               N: Optional[int] = None, X_bits: Optional[np.ndarray] = None) -> dict:
    """Inputs of one linear: X (unless external), W, bias, calibration absmax.

    M/K/N override the spec's sizes (for parity cases at reduced size); the
    distributions and seeds stay those of the spec.
    """
    M = spec.M if M is None else M
    K = spec.K if K is None else K
    N = spec.N if N is None else N
    out = {"spec": spec, "M": M, "K": K, "N": N}
    if X_bits is None:
        if spec.x_dist == "external":
            raise ValueError(f"layer {spec.name} takes its activation from the previous layer")
        X_bits, ch = gen_activation(spec.config_id, M, K, spec.x_dist, spec.n_outliers,
                                    spec.outlier_scale)
        out["outlier_channels"] = ch
    else:
        assert X_bits.shape == (M, K) and X_bits.dtype == np.uint16
    out["X"] = np.ascontiguousarray(X_bits)
    out["W"] = gen_weight(spec.config_id, spec.w_stream, N, K, spec.w_std)
    out["bias"] = gen_bias(spec.config_id, spec.bias_stream, N, spec.bias_std)
    out["act_absmax"] = calibration_absmax(out["X"])
    return out


# ------------------------------------------- Q/K norm weights and rotary angles

def gen_qk_norm(config_id: int, stream: int) -> np.ndarray:
    """bf16 RMS-norm weight of a 128-channel head, N(1, 0.1^2)."""
    return f64_to_bf16_bits(rng_for(config_id, stream).normal(1.0, 0.1, size=(128,)))


def gen_rope(M: int, text_tokens: Optional[int] = None, grid_w: int = 64,
             axes_dim=(16, 56, 56), theta: float = 10000.0) -> tuple[np.ndarray, np.ndarray]:
    """cos and sin [M][64] (fp32) of a FLUX-like 3-axis rotary embedding: the
    first `text_tokens` tokens sit at position (0, 0, 0), the rest on a
    grid_w-wide patch grid at (0, row, col); pair j of an axis of d channels
    turns by position * theta^(-2j/d)."""
    if text_tokens is None:
        text_tokens = 512 if M == 4608 else M // 9
    ids = np.zeros((M, 3), np.float64)
    i = np.arange(M) - text_tokens
    img = i >= 0
    ids[img, 1] = i[img] // grid_w
    ids[img, 2] = i[img] % grid_w
    ang = []
    for a, d in enumerate(axes_dim):
        w = theta ** (-np.arange(0, d, 2, dtype=np.float64) / d)
        ang.append(ids[:, a:a + 1] * w[None, :])
    th = np.concatenate(ang, axis=1)
    assert th.shape == (M, 64)
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
