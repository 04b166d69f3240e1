"""Seeded synthetic inputs for the block-dequant GEMV (shared by tests and bench).

This module only draws random numbers and writes them out as canonical block
bytes. It holds none of the product's arithmetic: no dequantisation, no dot
product, no re-tiling. Both the HIP path and the fp64 oracle read its output.

Canonical formats (GGUF-style, little-endian):
  Q8_0 block, 34 B: fp16 scale d, then 32 int8 quants q; weight = d * q.
  Q4_0 block, 18 B: fp16 scale d, then 16 bytes of nibbles; byte j holds
                    element j (low nibble) and element j+16 (high nibble);
                    weight = d * (nibble - 8).
  Q4_K super-block, 144 B per 256 weights: fp16 d, fp16 dmin, 12 bytes of
                    6-bit sub-block scales and mins, 128 bytes of nibbles.
  Q6_K super-block, 210 B per 256 weights: 128 bytes of low 4-bit parts, 64
                    bytes of high 2-bit parts, 16 int8 scales, fp16 d last.
  F16 matrix: row-major [N][K] IEEE binary16.
A row of a quantised matrix is K/32 consecutive blocks (K/256 for Q4_K, Q6_K).

Value laws (the decode workloads the pages measure on are trained checkpoints;
these seeded draws stand in for them, with the same shapes):
  Q8_0: q uniform integers in [-127, 127]; d = fp16(|N(0, 0.02)| / 127).
  Q4_0: each nibble uniform in 0..15 (a uniform byte carries two independent
        uniform nibbles); d = fp16(|N(0, 0.02)| / 8).
  Q4_K: d = fp16(|N(0, 0.02)| / 480), dmin = fp16(|N(0, 0.02)| / 64); the 12
        scale/min bytes and the 128 quant bytes uniform (so every 6-bit scale
        and min and every nibble is uniform).
  Q6_K: the 192 quant bytes uniform (every 6-bit quant uniform in 0..63), the
        16 scales uniform int8 in [-128, 127], d = fp16(|N(0, 0.02)| / 512)
        (about half of the d are fp16 subnormals).
  F16 : w = fp16(N(0, 0.02)).
  x   : fp32(N(0, 1)) drawn in float64 and rounded to nearest.
fp16 rounding is numpy's float64 -> float16 cast (round to nearest even).
"""
from __future__ import annotations

import numpy as np

Q8_0_BLOCK_BYTES = 34
Q4_0_BLOCK_BYTES = 18
Q4_K_BLOCK_BYTES = 144
Q6_K_BLOCK_BYTES = 210


def _rng(seed):
    if isinstance(seed, np.random.Generator):
        return seed
    return np.random.default_rng(seed)


def fp16_bits(values: np.ndarray) -> np.ndarray:
    """Round float64 values to fp16 (RNE) and return their uint16 bit patterns."""
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def q8_0_matrix(N: int, K: int, seed, scale_sigma: float = 0.02) -> np.ndarray:
    """Random Q8_0 weight matrix as canonical bytes, shape (N * K/32 * 34,) uint8."""
    if K % 32:
        raise ValueError("Q8_0 needs K % 32 == 0")
    rng = _rng(seed)
    nb = N * (K // 32)
    d = fp16_bits(np.abs(rng.normal(0.0, scale_sigma, nb)) / 127.0)
    q = rng.integers(-127, 128, size=(nb, 32), dtype=np.int8)
    out = np.empty((nb, Q8_0_BLOCK_BYTES), np.uint8)
    out[:, 0:2] = d.astype("<u2").view(np.uint8).reshape(nb, 2)
    out[:, 2:] = q.view(np.uint8)
    return out.reshape(-1)


def q4_0_matrix(N: int, K: int, seed, scale_sigma: float = 0.02) -> np.ndarray:
    """Random Q4_0 weight matrix as canonical bytes, shape (N * K/32 * 18,) uint8."""
    if K % 32:
        raise ValueError("Q4_0 needs K % 32 == 0")
    rng = _rng(seed)
    nb = N * (K // 32)
    d = fp16_bits(np.abs(rng.normal(0.0, scale_sigma, nb)) / 8.0)
    qs = rng.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    out = np.empty((nb, Q4_0_BLOCK_BYTES), np.uint8)
    out[:, 0:2] = d.astype("<u2").view(np.uint8).reshape(nb, 2)
    out[:, 2:] = qs
    return out.reshape(-1)


def q4_k_matrix(N: int, K: int, seed, scale_sigma: float = 0.02) -> np.ndarray:
    """Random Q4_K weight matrix as canonical bytes, shape (N * K/256 * 144,) uint8."""
    if K % 256:
        raise ValueError("Q4_K needs K % 256 == 0")
    rng = _rng(seed)
    nb = N * (K // 256)
    d = fp16_bits(np.abs(rng.normal(0.0, scale_sigma, nb)) / 480.0)
    dmin = fp16_bits(np.abs(rng.normal(0.0, scale_sigma, nb)) / 64.0)
    rest = rng.integers(0, 256, size=(nb, 140), dtype=np.uint8)
    out = np.empty((nb, Q4_K_BLOCK_BYTES), np.uint8)
    out[:, 0:2] = d.astype("<u2").view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = dmin.astype("<u2").view(np.uint8).reshape(nb, 2)
    out[:, 4:] = rest
    return out.reshape(-1)


def q6_k_matrix(N: int, K: int, seed, scale_sigma: float = 0.02) -> np.ndarray:
    """Random Q6_K weight matrix as canonical bytes, shape (N * K/256 * 210,) uint8."""
    if K % 256:
        raise ValueError("Q6_K needs K % 256 == 0")
    rng = _rng(seed)
    nb = N * (K // 256)
    d = fp16_bits(np.abs(rng.normal(0.0, scale_sigma, nb)) / 512.0)
    out = np.empty((nb, Q6_K_BLOCK_BYTES), np.uint8)
    out[:, 0:208] = rng.integers(0, 256, size=(nb, 208), dtype=np.uint8)
    out[:, 208:210] = d.astype("<u2").view(np.uint8).reshape(nb, 2)
    return out.reshape(-1)


def f16_matrix(N: int, K: int, seed, sigma: float = 0.02) -> np.ndarray:
    """Random fp16 row-major matrix as uint16 bit patterns, shape (N*K,)."""
    rng = _rng(seed)
    return fp16_bits(rng.normal(0.0, sigma, N * K))


def activation(K: int, seed, M: int | None = None) -> np.ndarray:
    """fp32 N(0,1) activations: shape (K,) or (M, K)."""
    rng = _rng(seed)
    shape = (K,) if M is None else (M, K)
    return rng.standard_normal(shape).astype(np.float32)


def matrix(kind: str, N: int, K: int, seed) -> np.ndarray:
    if kind == "q8_0":
        return q8_0_matrix(N, K, seed)
    if kind == "q4_0":
        return q4_0_matrix(N, K, seed)
    if kind == "q4_k":
        return q4_k_matrix(N, K, seed)
    if kind == "q6_k":
        return q6_k_matrix(N, K, seed)
    if kind == "f16":
        return f16_matrix(N, K, seed)
    raise ValueError(kind)


def matrix_bytes(kind: str, N: int, K: int) -> int:
    """Bytes of the canonical weights (quants + scales, or fp16 values)."""
    if kind == "q8_0":
        return N * (K // 32) * Q8_0_BLOCK_BYTES
    if kind == "q4_0":
        return N * (K // 32) * Q4_0_BLOCK_BYTES
    if kind == "q4_k":
        return N * (K // 256) * Q4_K_BLOCK_BYTES
    if kind == "q6_k":
        return N * (K // 256) * Q6_K_BLOCK_BYTES
    return N * K * 2


# ---- the five workload configurations -------------------------------------
#
# Each entry: (name, kind, N, K, role). Role "gemv" is a plain product,
# "qkv_q"/"qkv_k"/"qkv_v" are the parts packed into one concatenated weight,
# "gate"/"up" are the two halves of a fused gate|up matrix (SiLU epilogue),
# "verify" is a weight used with M = 2..6 activation rows.
# Seeds: config 0 uses seed 0; config i uses seed i. Per-matrix streams come
# from SeedSequence(seed).spawn(len(entries) + activations), in table order.

CONFIGS = {
    0: {
        "name": "q8_0 gemv 1024x1024",
        "matrices": [("w", "q8_0", 1024, 1024, "gemv")],
    },
    1: {
        "name": "qwen3-0.6b-shaped q8_0 decode weight set",
        "matrices": [
            ("q_proj", "q8_0", 2048, 1024, "qkv_q"),
            ("k_proj", "q8_0", 1024, 1024, "qkv_k"),
            ("v_proj", "q8_0", 1024, 1024, "qkv_v"),
            ("o_proj", "q8_0", 1024, 2048, "gemv"),
            ("gate", "q8_0", 3072, 1024, "gate"),
            ("up", "q8_0", 3072, 1024, "up"),
            ("down", "q8_0", 1024, 3072, "gemv"),
            ("lm_head", "q8_0", 151936, 1024, "gemv"),
        ],
    },
    2: {
        "name": "27b-class q4_0 shapes",
        "matrices": [
            ("gate", "q4_0", 17408, 5120, "gate"),
            ("up", "q4_0", 17408, 5120, "up"),
            ("down", "q4_0", 5120, 17408, "gemv"),
            ("lm_head", "q4_0", 248320, 5120, "gemv"),
        ],
    },
    3: {
        "name": "fp16 split-k gemv",
        "matrices": [
            ("square", "f16", 5120, 5120, "gemv"),
            ("thin", "f16", 256, 5120, "gemv"),
            ("small", "f16", 48, 5120, "gemv"),
        ],
    },
    4: {
        "name": "multi-row verify gemv",
        "matrices": [
            ("q4_0_w", "q4_0", 17408, 5120, "verify"),
            ("q8_0_w", "q8_0", 4096, 1024, "verify"),
        ],
    },
}


class Workload:
    """Lazily generated, seeded inputs of one configuration."""

    def __init__(self, cfg: int, seed: int | None = None):
        self.cfg = cfg
        self.spec = CONFIGS[cfg]
        self.seed = cfg if seed is None else seed
        mats = self.spec["matrices"]
        # one stream per matrix, one per matrix activation, in table order
        self._children = np.random.SeedSequence(self.seed).spawn(2 * len(mats))
        self._index = {m[0]: i for i, m in enumerate(mats)}
        self._cache: dict = {}

    def entry(self, name: str):
        return self.spec["matrices"][self._index[name]]

    def weight(self, name: str) -> np.ndarray:
        key = ("w", name)
        if key not in self._cache:
            _, kind, N, K, _ = self.entry(name)
            self._cache[key] = matrix(kind, N, K, np.random.default_rng(self._children[self._index[name]]))
        return self._cache[key]

    def x(self, name: str, M: int | None = None) -> np.ndarray:
        """Activation for matrix `name` (M rows for verify; the M=1 draw is row 0
        of the same stream, so the first row is shared across M)."""
        key = ("x", name, M)
        if key not in self._cache:
            _, _, _, K, _ = self.entry(name)
            rng = np.random.default_rng(self._children[len(self.spec["matrices"]) + self._index[name]])
            self._cache[key] = activation(K, rng, M)
        return self._cache[key]

    def drop(self, name: str):
        for key in [k for k in self._cache if k[1] == name]:
            del self._cache[key]
