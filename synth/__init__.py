"""Seeded synthetic inputs for the packed LM-head forward.

This module only draws random numbers and stores them in the storage types the
packed head uses (bf16 bit patterns, fp16, int8/uint8 codes).  It holds none of
the method's arithmetic: no dequantisation, no packing, no products.  Both the
CPU oracle and the GPU path are fed from here, and nothing else is shared
between them.

Workloads (the five shapes used throughout, "ARCHead: Activation-Metric Residual
Correction for Large Language Model Output Heads", Sec. 3 and Alg. 1 define the
components; the shapes stand in for the Qwen3-8B-Base head of its Tables 4-8
and a 70B-class head):

  tiny      V=1024   D=256  N=4    r_c=16 r_r=8  g=64   4 outlier ch. x20, fp32 Y
  decode    V=151936 D=4096 N=1    r_c=32 r_r=32 g=128 16 outlier ch. x20, fp32 Y
  batched   V=151936 D=4096 N=64   r_c=32 r_r=32 g=128 16 outlier ch. x20, fp32 Y
  prefill   V=151936 D=4096 N=4096 r_c=64 r_r=64 g=128 16 outlier ch. x20, bf16 Y
  head70b   V=128256 D=8192 N=256  r_c=64 r_r=64 g=128 32 outlier ch. x25, fp32 Y

Value distributions (same for every workload):
  H      bf16, N(0,1) drawn in fp32, outlier channels multiplied by the factor
         in fp32, then rounded once to bf16 (round to nearest even).
  q4     signed INT4 residual codes, uniform on [-8, 7].
  c8     uint8 group-scale codes, uniform on [1, 255].
  s_R    per-row fp16 residual scale, |N(0, 1e-3)| drawn in fp64, rounded to fp16.
  A_c/A_w  INT8 codes uniform on [-127, 127]; fp16 row scales |N(0, 1e-2)|.
  B_c/B_w  INT8 codes uniform on [-127, 127]; fp16 group scales |N(0, 1e-2)|.

Draw order from one numpy PCG64 stream (``numpy.random.default_rng(seed)``):
H, outlier channel indices, q4, c8, s_R, A_c, A_w, s_Ac, s_Aw, B_c, B_w, s_Bc,
s_Bw.  The default seed of a workload is its index in ``CONFIGS``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

CONFIGS = [
    dict(name="tiny", V=1024, D=256, N=4, r_c=16, r_r=8, g=64,
         n_outlier=4, outlier_scale=20.0, y_dtype="f32"),
    dict(name="decode", V=151936, D=4096, N=1, r_c=32, r_r=32, g=128,
         n_outlier=16, outlier_scale=20.0, y_dtype="f32"),
    dict(name="batched", V=151936, D=4096, N=64, r_c=32, r_r=32, g=128,
         n_outlier=16, outlier_scale=20.0, y_dtype="f32"),
    dict(name="prefill", V=151936, D=4096, N=4096, r_c=64, r_r=64, g=128,
         n_outlier=16, outlier_scale=20.0, y_dtype="bf16"),
    dict(name="head70b", V=128256, D=8192, N=256, r_c=64, r_r=64, g=128,
         n_outlier=32, outlier_scale=25.0, y_dtype="f32"),
]


def config(name_or_index) -> dict:
    if isinstance(name_or_index, int):
        return dict(CONFIGS[name_or_index])
    for c in CONFIGS:
        if c["name"] == name_or_index:
            return dict(c)
    raise KeyError(name_or_index)


@dataclass
class Head:
    """Quantised components of one packed head, unpacked (one code per element).

    Shapes: q4 [V, D] int8 in [-8, 7]; c8 [V, D/g] uint8; s_R [V] float16;
    A_c [V, r_c] int8; A_w [V, r_r] int8; s_Ac, s_Aw [V] float16;
    B_c [r_c, D] int8; B_w [r_r, D] int8; s_Bc [r_c, D/g], s_Bw [r_r, D/g] float16.
    """
    V: int
    D: int
    r_c: int
    r_r: int
    g: int
    q4: np.ndarray
    c8: np.ndarray
    s_R: np.ndarray
    A_c: np.ndarray
    A_w: np.ndarray
    s_Ac: np.ndarray
    s_Aw: np.ndarray
    B_c: np.ndarray
    B_w: np.ndarray
    s_Bc: np.ndarray
    s_Bw: np.ndarray

    @property
    def dims(self):
        return dict(V=self.V, D=self.D, r_c=self.r_c, r_r=self.r_r, g=self.g)


@dataclass
class Inputs:
    H_bits: np.ndarray          # [N, D] uint16, bf16 bit patterns
    head: Head
    outlier_channels: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    seed: Optional[int] = None


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def _abs_normal_f16(rng, sigma, size):
    return np.abs(rng.normal(0.0, sigma, size=size)).astype(np.float16)


def draw_hidden(rng, N, D, n_outlier, outlier_scale):
    h = rng.standard_normal((N, D), dtype=np.float32)
    n_outlier = min(n_outlier, D)
    idx = np.sort(rng.choice(D, size=n_outlier, replace=False)) if n_outlier else np.zeros(0, np.int64)
    if n_outlier:
        h[:, idx] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(h), idx


def draw_head(rng, V, D, r_c, r_r, g) -> Head:
    ng = D // g
    q4 = rng.integers(-8, 8, size=(V, D), dtype=np.int8)
    c8 = rng.integers(1, 256, size=(V, ng), dtype=np.uint8)
    s_R = _abs_normal_f16(rng, 1e-3, V)
    A_c = rng.integers(-127, 128, size=(V, r_c), dtype=np.int8)
    A_w = rng.integers(-127, 128, size=(V, r_r), dtype=np.int8)
    s_Ac = _abs_normal_f16(rng, 1e-2, V)
    s_Aw = _abs_normal_f16(rng, 1e-2, V)
    B_c = rng.integers(-127, 128, size=(r_c, D), dtype=np.int8)
    B_w = rng.integers(-127, 128, size=(r_r, D), dtype=np.int8)
    s_Bc = _abs_normal_f16(rng, 1e-2, (r_c, ng))
    s_Bw = _abs_normal_f16(rng, 1e-2, (r_r, ng))
    return Head(V, D, r_c, r_r, g, q4, c8, s_R, A_c, A_w, s_Ac, s_Aw, B_c, B_w, s_Bc, s_Bw)


@dataclass
class AltHead:
    """A storage-matched comparison head, unpacked.  fmt 1 (group INT4 with
    fp16 group scales): codes [V, D] int8 in [-8, 7], scales [V, D/g] float16.
    fmt 2 (row INT8): codes [V, D] int8 in [-127, 127], scales [V] float16."""
    fmt: int
    V: int
    D: int
    g: int
    codes: np.ndarray
    scales: np.ndarray


def draw_alt_head(rng, fmt, V, D, g) -> AltHead:
    """Codes uniform over their range; fp16 scales |N(0, 1e-2)| per group
    (fmt 1) or |N(0, 1e-3)| per row (fmt 2).  Draw order: codes, scales."""
    if fmt == 1:
        codes = rng.integers(-8, 8, size=(V, D), dtype=np.int8)
        scales = _abs_normal_f16(rng, 1e-2, (V, D // g))
    elif fmt == 2:
        codes = rng.integers(-127, 128, size=(V, D), dtype=np.int8)
        scales = _abs_normal_f16(rng, 1e-3, V)
    else:
        raise ValueError(fmt)
    return AltHead(fmt, V, D, g, codes, scales)


def make_alt(fmt, seed, V, D, N, g, n_outlier=4, outlier_scale=20.0):
    """Hidden states (drawn first, as in ``make``) and a comparison head of
    format ``fmt`` from one seeded stream.  Returns (H_bits, head)."""
    rng = np.random.default_rng(seed)
    H_bits, _ = draw_hidden(rng, N, D, n_outlier, outlier_scale)
    return H_bits, draw_alt_head(rng, fmt, V, D, g)


@dataclass
class Dense:
    """Dense inputs of the packing step: the head W and the factor matrices."""
    W: np.ndarray      # [V, D] bf16 bit patterns (uint16) or float32
    A_c: np.ndarray    # [V, r_c] float32
    B_c: np.ndarray    # [r_c, D] float32
    A_w: np.ndarray    # [V, r_r] float32
    B_w: np.ndarray    # [r_r, D] float32


def draw_dense(rng, V, D, r_c, r_r, w_dtype="bf16", n_heavy_rows=4) -> Dense:
    """Dense head and factors, drawn independently.

    W      N(0, 0.02) in fp32; n_heavy_rows rows (chosen uniformly) x 30, so that
           row scales differ by orders of magnitude; bf16 (rounded once) or fp32.
    A_c    N(0, 0.1) fp32;  B_c N(0, 0.1) fp32.
    A_w    N(0, 0.05) fp32; B_w N(0, 0.05) fp32.
    Draw order: W, heavy rows, A_c, B_c, A_w, B_w."""
    W = rng.normal(0.0, 0.02, size=(V, D)).astype(np.float32)
    heavy = rng.choice(V, size=min(n_heavy_rows, V), replace=False)
    W[heavy] *= np.float32(30.0)
    A_c = rng.normal(0.0, 0.1, size=(V, r_c)).astype(np.float32)
    B_c = rng.normal(0.0, 0.1, size=(r_c, D)).astype(np.float32)
    A_w = rng.normal(0.0, 0.05, size=(V, r_r)).astype(np.float32)
    B_w = rng.normal(0.0, 0.05, size=(r_r, D)).astype(np.float32)
    return Dense(f32_to_bf16_bits(W) if w_dtype == "bf16" else W, A_c, B_c, A_w, B_w)


@dataclass
class FitInputs:
    """Inputs of the whole construction: dense head, calibration states and the
    randomized SVDs' Gaussian test matrices."""
    W: np.ndarray        # [V, D] bf16 bit patterns (uint16)
    H: np.ndarray        # [N, D] bf16 bit patterns
    omega_c: np.ndarray  # [D, r_c + oversample] float32
    omega_r: np.ndarray  # [D, r_r + oversample] float32


def draw_fit(rng, V, D, r_c, r_r, N, oversample=8, n_outlier=4, outlier_scale=20.0) -> FitInputs:
    """A head with a rank-r_c part plus noise, and calibration hidden states.

    W      L R * 0.02 / sqrt(r_c) + N(0, 0.004), L [V, r_c] and R [r_c, D]
           N(0, 1), computed in fp32 and rounded once to bf16 (the product
           only shapes the synthetic spectrum);
    H      as the forward's hidden states: N(0, 1) with n_outlier channels
           x outlier_scale, bf16;
    omega  N(0, 1) fp32.
    Draw order: L, R, noise, H (with its outlier channels), omega_c, omega_r."""
    L = rng.standard_normal((V, r_c), dtype=np.float32)
    R = rng.standard_normal((r_c, D), dtype=np.float32)
    W = (L @ R) * np.float32(0.02 / np.sqrt(max(r_c, 1))) + rng.normal(0.0, 0.004, size=(V, D)).astype(np.float32)
    H, _ = draw_hidden(rng, N, D, n_outlier, outlier_scale)
    om_c = rng.standard_normal((D, r_c + oversample), dtype=np.float32)
    om_r = rng.standard_normal((D, r_r + oversample), dtype=np.float32)
    return FitInputs(f32_to_bf16_bits(W), H, om_c, om_r)


def make(cfg, seed: Optional[int] = None, N: Optional[int] = None, **overrides) -> Inputs:
    """Draw one workload.  ``cfg`` is a CONFIGS entry, its name or its index.

    ``N`` and keyword overrides (V, D, r_c, r_r, g, n_outlier, outlier_scale)
    change the shape while keeping the distributions and the draw order.
    """
    if not isinstance(cfg, dict):
        if seed is None and isinstance(cfg, int):
            seed = cfg
        cfg = config(cfg)
    c = dict(cfg)
    c.update(overrides)
    if N is not None:
        c["N"] = N
    if seed is None:
        seed = next((i for i, k in enumerate(CONFIGS) if k["name"] == c["name"]), 0)
    rng = np.random.default_rng(seed)
    H_bits, idx = draw_hidden(rng, c["N"], c["D"], c["n_outlier"], c["outlier_scale"])
    head = draw_head(rng, c["V"], c["D"], c["r_c"], c["r_r"], c["g"])
    return Inputs(H_bits=H_bits, head=head, outlier_channels=idx, seed=seed)


def zero_head(V, D, r_c, r_r, g) -> Head:
    """All-zero codes with unit scales; tests overwrite parts of it."""
    ng = D // g
    one = np.float16(1.0)
    return Head(V, D, r_c, r_r, g,
                np.zeros((V, D), np.int8), np.ones((V, ng), np.uint8),
                np.full(V, one, np.float16),
                np.zeros((V, r_c), np.int8), np.zeros((V, r_r), np.int8),
                np.full(V, one, np.float16), np.full(V, one, np.float16),
                np.zeros((r_c, D), np.int8), np.zeros((r_r, D), np.int8),
                np.full((r_c, ng), one, np.float16), np.full((r_r, ng), one, np.float16))
