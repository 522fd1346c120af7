"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no part of the masking / compression / product arithmetic:
it only produces weight and activation matrices, bit-for-bit reproducibly, so
that the GPU library and the CPU oracle are fed identical inputs.

Recipe (published methods, written from their definitions):

* Random bits: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014).  Draw ``i`` of a stream seeded with ``s`` is
  the ``i``-th output of the generator started at state ``s``, i.e.
  ``mix(s + (i + 1) * 0x9E3779B97F4A7C15)``, so any element can be produced
  independently (counter-based use).
* Uniforms: the top 53 bits of a draw, scaled by 2^-53.
* Normals: Box & Muller (1958), cosine branch; element ``i`` uses draws
  ``2i`` (u1 in (0, 1]) and ``2i + 1`` (u2 in [0, 1)).
* Laplace(0, b): inverse CDF of a uniform in the open interval (0, 1).
* Outliers: element ``i`` is scaled by a factor when draw ``i`` of a separate
  stream, as a uniform in [0, 1), falls below the outlier probability.
* Values are produced in float64, rounded to fp32 (round-to-nearest-even),
  then to bf16 or fp16 (round-to-nearest-even on the fp32 bits).  int8 values
  are the float64 draws rounded to the nearest integer (ties to even) and
  clipped to [-128, 127], i.e. a symmetric quantiser with step 1 (the scale is
  part of the distribution).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 20

DTYPES = ("f32", "f16", "bf16")


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of the SplitMix64 stream seeded with ``seed``."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _top53(z: np.ndarray) -> np.ndarray:
    return (z >> np.uint64(11)).astype(np.float64)


def _normal_chunk(seed: int, start: int, count: int) -> np.ndarray:
    z = splitmix64(seed, 2 * start, 2 * count)
    u1 = (_top53(z[0::2]) + 1.0) * 2.0**-53  # (0, 1]
    u2 = _top53(z[1::2]) * 2.0**-53  # [0, 1)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def _laplace_chunk(seed: int, start: int, count: int, b: float) -> np.ndarray:
    u = (_top53(splitmix64(seed, start, count)) + 0.5) * 2.0**-53  # (0, 1)
    v = u - 0.5
    return -b * np.sign(v) * np.log1p(-2.0 * np.abs(v))


def _uniform_chunk(seed: int, start: int, count: int) -> np.ndarray:
    return _top53(splitmix64(seed, start, count)) * 2.0**-53  # [0, 1)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


# The 127 non-negative finite OCP FP8 E4M3 values, by code (bias 7, 3 fraction bits).
_E4M3_CODES = np.arange(127)
_E4M3_VALUES = np.where(_E4M3_CODES >> 3 == 0, (_E4M3_CODES & 7) * 2.0 ** -9,
                        (8 + (_E4M3_CODES & 7)) * np.exp2((_E4M3_CODES >> 3) - 10.0))


def f32_to_e4m3_bits(x32: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value (ties to the even code), magnitudes clipped to 448 first."""
    x = np.asarray(x32, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_VALUES, a), 1, 126)
    lo = hi - 1
    dlo, dhi = a - _E4M3_VALUES[lo], _E4M3_VALUES[hi] - a
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= _E4M3_VALUES[126], 126, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def round_to(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> fp32 (RNE) -> dtype.  Returns float32 for f32, raw uint16 bits for the
    16-bit types, int8 for i8 (nearest integer, clipped)."""
    if dtype == "i8":
        return np.clip(np.rint(x64), -128, 127).astype(np.int8)
    x32 = x64.astype(np.float32)
    if dtype == "fp8":
        return f32_to_e4m3_bits(x32)
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def bits_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Decode the generator's output format back to float64 (exact)."""
    a = np.asarray(a)
    if dtype == "f32":
        if a.dtype == np.uint32:
            a = a.view(np.float32)
        return a.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "i8":
        return np.asarray(a).view(np.int8).astype(np.float64)
    if dtype == "fp8":
        b = np.asarray(a).view(np.uint8).astype(np.int64)
        v = _E4M3_VALUES[np.minimum(b & 0x7F, 126)]
        v = np.where((b & 0x7F) == 0x7F, np.nan, v)
        return np.where(b & 0x80, -v, v)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


@dataclass(frozen=True)
class Dist:
    """A seeded matrix distribution."""

    kind: str  # "normal" | "laplace"
    seed: int
    scale: float = 1.0  # std for normal, b for laplace
    relu: bool = False
    outlier_seed: int | None = None
    outlier_p: float = 0.0
    outlier_mult: float = 1.0

    def sample_f64(self, start: int, count: int) -> np.ndarray:
        if self.kind == "normal":
            x = self.scale * _normal_chunk(self.seed, start, count)
        elif self.kind == "laplace":
            x = _laplace_chunk(self.seed, start, count, self.scale)
        else:
            raise ValueError(self.kind)
        if self.outlier_seed is not None and self.outlier_p > 0:
            hit = _uniform_chunk(self.outlier_seed, start, count) < self.outlier_p
            x = np.where(hit, x * self.outlier_mult, x)
        if self.relu:
            x = np.where(x > 0.0, x, 0.0)
        return x


def generate(dist: Dist, shape: tuple[int, int], dtype: str) -> np.ndarray:
    """Row-major matrix of ``shape``; element (r, c) is draw r*cols + c of ``dist``."""
    n = int(shape[0]) * int(shape[1])
    out = np.empty(n, dtype={"f32": np.float32, "i8": np.int8, "fp8": np.uint8}.get(dtype, np.uint16))

    def fill(s: int) -> None:
        c = min(_CHUNK, n - s)
        out[s : s + c] = round_to(dist.sample_f64(s, c), dtype)

    starts = range(0, n, _CHUNK)
    if n <= _CHUNK:
        for s in starts:
            fill(s)
    else:  # numpy releases the GIL inside its array kernels
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, starts))
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Workloads: the shapes and value distributions of the pages' model layers.
# W is R x K (groups of M along K), X is K x T.
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    R: int
    K: int
    T: int
    dtype: str
    w: Dist
    x: Dist
    patterns: tuple = ((2, 4),)
    note: str = ""
    extra: dict = field(default_factory=dict)

    def W(self) -> np.ndarray:
        return generate(self.w, (self.R, self.K), self.dtype)

    def X(self) -> np.ndarray:
        return generate(self.x, (self.K, self.T), self.dtype)

    def G(self) -> np.ndarray:
        """A weight gradient of W's shape: N(0, 1e-3^2), seed 3 (the SR-STE backward's input)."""
        return generate(GRAD_DIST, (self.R, self.K), self.dtype)


# Weight gradients for the SR-STE backward: i.i.d. normal, small next to the weights.
GRAD_DIST = Dist("normal", seed=3, scale=1e-3)


def _llama(R, K, name):
    return Workload(
        name=name, R=R, K=K, T=2048, dtype="bf16",
        w=Dist("normal", seed=0, scale=0.02, outlier_seed=2, outlier_p=0.01, outlier_mult=10.0),
        x=Dist("normal", seed=1, scale=1.0),
        note="LLaMA-7B MLP projection, 2048 tokens",
    )


WORKLOADS = {
    # fp32 toy: 64 x 128 weights ~N(0,1) seed 0, 32 activation columns ~N(0,1)
    "toy_f32": Workload("toy_f32", 64, 128, 32, "f32", Dist("normal", 0), Dist("normal", 1)),
    # BERT-base FFN: 3072 x 768 ~N(0, 0.02^2), activations 768 x (8 x 512)
    "bert_ffn": Workload("bert_ffn", 3072, 768, 4096, "bf16", Dist("normal", 0, 0.02),
                         Dist("normal", 1)),
    # ResNet-50 3x3 conv as im2col GEMM: 256 x 2304 Kaiming-normal, ReLU'd activations
    "resnet_conv3x3": Workload("resnet_conv3x3", 256, 2304, 32 * 14 * 14, "bf16",
                               Dist("normal", 0, math.sqrt(2.0 / 2304)),
                               Dist("normal", 1, relu=True)),
    "llama_up": _llama(11008, 4096, "llama_up"),
    "llama_down": _llama(4096, 11008, "llama_down"),
    # the LLaMA-7B MLP pair quantised to int8: weights and activations ~N(0, 24^2)
    # rounded to integers (about 1 in 25,000 draws clipped at +-127.5)
    "llama_up_i8": Workload("llama_up_i8", 11008, 4096, 2048, "i8", Dist("normal", 0, 24.0),
                            Dist("normal", 1, 24.0), note="LLaMA-7B MLP up-projection, int8"),
    "llama_down_i8": Workload("llama_down_i8", 4096, 11008, 2048, "i8", Dist("normal", 0, 24.0),
                              Dist("normal", 1, 24.0), note="LLaMA-7B MLP down-projection, int8"),
    # ... and to OCP FP8 E4M3: weights and activations ~N(0, 1) rounded to E4M3
    "llama_up_fp8": Workload("llama_up_fp8", 11008, 4096, 2048, "fp8", Dist("normal", 0, 1.0),
                             Dist("normal", 1, 1.0), note="LLaMA-7B MLP up-projection, fp8"),
    "llama_down_fp8": Workload("llama_down_fp8", 4096, 11008, 2048, "fp8", Dist("normal", 0, 1.0),
                               Dist("normal", 1, 1.0), note="LLaMA-7B MLP down-projection, fp8"),
    # N:M sweep: fp16 4096 x 4096 ~Laplace(0, 0.05), activations 4096 x 8192 ~N(0,1)
    "sweep_f16": Workload("sweep_f16", 4096, 4096, 8192, "f16", Dist("laplace", 0, 0.05),
                          Dist("normal", 1), patterns=((1, 2), (2, 4), (4, 8))),
    # the same sweep in fp32 (the fp32 product path at a size that fills the device)
    "sweep_f32": Workload("sweep_f32", 4096, 4096, 8192, "f32", Dist("laplace", 0, 0.05),
                          Dist("normal", 1), patterns=((1, 2), (2, 4), (4, 8))),
}
