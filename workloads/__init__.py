"""Seeded synthetic inputs for PaTH attention, shared by the tests and the bench.

This module holds no arithmetic of the method itself: it only draws random
numbers, normalises the direction vectors w_t to unit length, and rounds to the
storage dtypes.  Both the HIP path and the fp64 oracle consume exactly the
arrays produced here.

Recipe (the same for every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64), all draws in float64, in the
    order q, k, v, w, beta, [near-2 mask, near-2 values], [forget gate];
  * q, k, v ~ N(0, 1) elementwise (optionally q is multiplied by ``q_scale``);
  * w: N(0, 1) elementwise, divided by its L2 norm per (b, h, t), so each w_t
    is a unit vector before rounding (the pages' producer ends in an L2 norm);
  * beta = 2 * sigmoid(N(0, beta_sigma)), with beta_sigma the standard
    deviation; with ``near2_frac`` > 0 a Bernoulli(near2_frac) mask over all
    (b, h, t) replaces beta by 1.9 + 0.1 * U[0, 1);
  * log f = logsigmoid(N(3, 1)) (PaTH-FoX only), computed stably;
  * rounding: float64 -> float32 (round to nearest even), then for bf16 inputs
    float32 -> bf16 (round to nearest even).  beta and log f stay float32.
    beta is clamped to the largest float32 below 2 so that it stays in (0, 2).

Shapes: q, k, v, w are [B, H, T, d]; beta and log f are [B, H, T].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": storage dtype of q, k, v, w and out
    B: int
    H: int
    T: int
    d: int
    seed: int
    beta_sigma: float = 1.0
    near2_frac: float = 0.0
    fox: bool = False
    q_scale: float = 1.0
    beta_const: Optional[float] = None   # diagnostic: every beta set to this

    @property
    def n_tokens(self) -> int:
        return self.B * self.T

    def flops_path(self) -> float:
        """Algorithmic flops B*H*T^2*(2d + d^2/64): causal QK^T and PV
        (4d per pair over T^2/2 pairs) plus one 2d^2 chunk transform per
        query row and earlier 64-token chunk."""
        return float(self.B * self.H) * self.T * self.T * (2 * self.d + self.d * self.d / 64.0)

    def flops_attn(self) -> float:
        """Ordinary causal attention flops 2*B*H*d*T^2."""
        return 2.0 * self.B * self.H * self.d * self.T * self.T

    def hbm_bytes(self) -> int:
        """Algorithmic HBM bytes: read q, k, v, w, beta (and log f), write
        out and lse."""
        e = 2 if self.dtype == "bf16" else 4
        per_token = 4 * self.d * e + 4 + self.d * e + 4 + (4 if self.fox else 0)
        return self.B * self.H * self.T * per_token


# The five synthetic workloads.  Shapes follow the (batch, length, head dim)
# rows of the authors' kernel latency table (author-response page, "Efficiency
# Evaluation"), plus a tiny fp32 case the oracle finishes in about a second.
TINY_F32 = Workload("tiny_f32_b1h2t256d64", "f32", 1, 2, 256, 64, seed=0,
                    beta_sigma=1.0)
MID_D64 = Workload("bf16_b16h16t2048d64", "bf16", 16, 16, 2048, 64, seed=1,
                   beta_sigma=1.5)
MID_D128_NEAR2 = Workload("bf16_b16h8t2048d128_near2", "bf16", 16, 8, 2048, 128,
                          seed=2, beta_sigma=1.5, near2_frac=0.1)
LONG_D64 = Workload("bf16_b2h16t16384d64", "bf16", 2, 16, 16384, 64, seed=3,
                    beta_sigma=1.0)
FOX_D128 = Workload("bf16_fox_b4h8t8192d128", "bf16", 4, 8, 8192, 128, seed=4,
                    beta_sigma=1.0, fox=True)

WORKLOADS = [TINY_F32, MID_D64, MID_D128_NEAR2, LONG_D64, FOX_D128]
BY_NAME = {w.name: w for w in WORKLOADS}

# Diagnostic inputs (reported, not graded).
REFLECT_F32 = Workload("diag_reflect_f32_b1h2t2048d64", "f32", 1, 2, 2048, 64,
                       seed=11, beta_const=2.0)
REFLECT_BF16 = Workload("diag_reflect_bf16_b1h2t2048d64", "bf16", 1, 2, 2048, 64,
                        seed=11, beta_const=2.0)
SHARP_D64 = dataclasses.replace(MID_D64, name="diag_sharp_bf16_b16h16t2048d64",
                                q_scale=3.0)
BETA0_D64 = dataclasses.replace(MID_D64, name="diag_beta0_bf16_b16h16t2048d64",
                                beta_const=0.0)


def bf16_round(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even); returned as float32."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x32.shape)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    return np.where(x > 0, -np.log1p(np.exp(-np.abs(x))), x - np.log1p(np.exp(-np.abs(x))))


_BETA_MAX = np.nextafter(np.float32(2.0), np.float32(0.0))


def generate(wl: Workload, B: Optional[int] = None, H: Optional[int] = None,
             T: Optional[int] = None) -> dict:
    """Draw the inputs of a workload.

    Returns a dict of numpy arrays: q, k, v, w (float32 holding the exact
    storage values, i.e. bf16-representable for bf16 workloads), beta
    (float32) and logf (float32 or None).  B, H, T may override the
    workload's sizes (used by small parity cases).
    """
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    T = wl.T if T is None else T
    d = wl.d
    rng = np.random.default_rng(wl.seed)
    shape = (B, H, T, d)
    q = rng.standard_normal(shape) * wl.q_scale
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    w = rng.standard_normal(shape)
    w /= np.linalg.norm(w, axis=-1, keepdims=True)
    beta = 2.0 / (1.0 + np.exp(-rng.normal(0.0, wl.beta_sigma, size=(B, H, T))))
    if wl.near2_frac > 0:
        mask = rng.random((B, H, T)) < wl.near2_frac
        near = 1.9 + 0.1 * rng.random((B, H, T))
        beta = np.where(mask, near, beta)
    if wl.beta_const is not None:
        beta = np.full((B, H, T), wl.beta_const)
    logf = None
    if wl.fox:
        logf = _logsigmoid(rng.normal(3.0, 1.0, size=(B, H, T))).astype(np.float32)

    def store(x):
        x32 = x.astype(np.float32)
        return bf16_round(x32) if wl.dtype == "bf16" else x32

    beta32 = beta.astype(np.float32)
    if wl.beta_const is None:
        beta32 = np.minimum(beta32, _BETA_MAX)
    return dict(q=store(q), k=store(k), v=store(v), w=store(w), beta=beta32,
                logf=logf)


def small(dtype: str, B: int, H: int, T: int, d: int, seed: int, *,
          beta_sigma: float = 1.0, near2_frac: float = 0.0, fox: bool = False,
          q_scale: float = 1.0, beta_const: Optional[float] = None) -> dict:
    """Inputs for an ad-hoc small case with the same recipe."""
    wl = Workload(f"small_{dtype}_b{B}h{H}t{T}d{d}_s{seed}", dtype, B, H, T, d,
                  seed=seed, beta_sigma=beta_sigma, near2_frac=near2_frac,
                  fox=fox, q_scale=q_scale, beta_const=beta_const)
    return generate(wl)


def cotangents(dtype: str, B: int, H: int, T: int, d: int, seed: int,
               with_dlse: bool = True) -> dict:
    """Seeded output gradients for the backward pass: dout ~ N(0, 1) of shape
    [B, H, T, d] (stored like q: bf16-representable for bf16) and, if asked,
    dlse ~ N(0, 1) of shape [B, H, T] in float32 (else None).  Drawn with
    ``numpy.random.default_rng(seed)`` in the order dout, dlse."""
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((B, H, T, d)).astype(np.float32)
    if dtype == "bf16":
        dout = bf16_round(dout)
    dlse = rng.standard_normal((B, H, T)).astype(np.float32) if with_dlse else None
    return dict(dout=dout, dlse=dlse)
