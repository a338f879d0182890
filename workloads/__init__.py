"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and rounds them to the storage dtype;
it contains none of the quantizer's arithmetic.  Both the HIP path and the
CPU oracle are fed the *rounded* values it returns.

The pages quantize trained OPT/BLOOM/LLaMA-class models calibrated on a few
hundred text samples (Wiki "GPTQ", "Performance and Accuracy"); neither the
weights nor the text are available here, so layers are random Gaussian
weights and calibration activations are per-channel-scaled Gaussians whose
channel scales reproduce the heavy-tailed, outlier-channel structure of LLM
activations.  Each workload is named by what it is.

Generator: numpy PCG64.  seed = 20261203 + 1000 * config + layer.
Stream 0 (SeedSequence([seed, 0])) draws the channel scales, then W.
Calibration tokens are drawn in chunks of 2048 tokens; chunk c uses stream
SeedSequence([seed, 1, c]), so chunks can be generated independently.
X[t, ch] = a_ch * zeta[t, ch], zeta ~ N(0, 1).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BASE_SEED = 20261203
CHUNK_TOKENS = 2048

# ---------------------------------------------------------------------------
# dtype rounding (round to nearest even), numpy only.
# ---------------------------------------------------------------------------


def round_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b16: np.ndarray) -> np.ndarray:
    return (np.asarray(b16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Stored:
    """An array as stored on the device: ``raw`` (bytes-compatible numpy
    array in the storage dtype; bf16 kept as uint16 bit patterns) plus its
    exact float32 value ``f32``."""

    def __init__(self, raw: np.ndarray, dtype: str):
        self.raw = raw
        self.dtype = dtype

    @property
    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.raw)
        return self.raw.astype(np.float32)

    @property
    def shape(self):
        return self.raw.shape


def to_storage(x32: np.ndarray, dtype: str) -> Stored:
    if dtype == "bf16":
        return Stored(round_to_bf16_bits(x32), "bf16")
    if dtype == "f16":
        return Stored(np.asarray(x32, dtype=np.float32).astype(np.float16), "f16")
    if dtype == "f32":
        return Stored(np.asarray(x32, dtype=np.float32), "f32")
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Workload descriptions.
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    m: int
    n: int


@dataclasses.dataclass(frozen=True)
class Workload:
    config: int            # 1-based workload id (seed offset)
    name: str
    layers: tuple
    dtype: str
    w_std: float
    tokens: int
    channels: str          # channel-scale law, see channel_scales()
    levels: int
    group_size: int
    act_order: bool
    block_size: int = 128
    damp_rel: float = 0.01


WORKLOADS = {
    1: Workload(1, "single linear 256x256 fp32, 2048 tokens, 4 outlier channels x20, "
                   "4-bit per-row", (Layer("linear", 256, 256),), "f32", 0.02, 2048,
                "outlier4x20", 16, 0, False),
    2: Workload(2, "Llama-7B attention projection 4096x4096 bf16, 262144 tokens, "
                   "Student-t(4) channel scales, 4-bit g128",
                (Layer("attn_proj", 4096, 4096),), "bf16", 0.02, 262144,
                "student_t4", 16, 128, False),
    3: Workload(3, "Llama-7B MLP up 11008x4096 / down 4096x11008 bf16, 262144 tokens, "
                   "lognormal(1) channel scales, 3-bit g128 act-order",
                (Layer("mlp_up", 11008, 4096), Layer("mlp_down", 4096, 11008)),
                "bf16", 0.02, 262144, "lognormal1", 8, 128, True),
    4: Workload(4, "175B-class 12288x12288 / fc1 49152x12288 fp16, 262144 tokens, "
                   "0.5% outlier channels x50, 4-bit per-row",
                (Layer("attn_proj", 12288, 12288), Layer("fc1", 49152, 12288)),
                "f16", 0.01, 262144, "outlier0.5%x50", 16, 0, False),
}


def seed_for(config: int, layer: int = 0) -> int:
    return BASE_SEED + 1000 * int(config) + int(layer)


def channel_scales(law: str, n: int, rng: np.random.Generator) -> np.ndarray:
    if law == "outlier4x20":
        a = np.ones(n, dtype=np.float64)
        a[rng.choice(n, size=min(4, n), replace=False)] = 20.0
    elif law == "student_t4":
        a = np.abs(rng.standard_t(4.0, size=n))
    elif law == "lognormal1":
        a = np.exp(rng.standard_normal(n))
    elif law == "outlier0.5%x50":
        a = np.ones(n, dtype=np.float64)
        k = int(round(0.005 * n))
        a[rng.choice(n, size=k, replace=False)] = 50.0
    elif law == "unit":
        a = np.ones(n, dtype=np.float64)
    else:
        raise ValueError(law)
    return a.astype(np.float32)


@dataclasses.dataclass
class LayerInputs:
    W: Stored              # m x n
    a: np.ndarray          # channel scales (n,) float32
    seed: int
    dtype: str
    tokens: int
    n: int

    def x_chunk(self, c: int, tokens: int | None = None) -> Stored:
        """Calibration chunk c (CHUNK_TOKENS x n, last chunk may be shorter)."""
        t0 = c * CHUNK_TOKENS
        total = self.tokens if tokens is None else tokens
        rows = min(CHUNK_TOKENS, total - t0)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([self.seed, 1, c])))
        z = rng.standard_normal((rows, self.n), dtype=np.float32)
        z *= self.a[None, :]
        return to_storage(z, self.dtype)

    def x_all(self, tokens: int | None = None, threads: int | None = None) -> Stored:
        """All calibration tokens (or the first ``tokens``) as one array."""
        total = self.tokens if tokens is None else int(tokens)
        nchunks = -(-total // CHUNK_TOKENS)
        item = {"bf16": np.uint16, "f16": np.float16, "f32": np.float32}[self.dtype]
        raw = np.empty((total, self.n), dtype=item)

        def fill(c):
            t0 = c * CHUNK_TOKENS
            raw[t0:t0 + CHUNK_TOKENS] = self.x_chunk(c, total).raw

        threads = threads or min(16, os.cpu_count() or 1)
        if nchunks > 1 and threads > 1:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(fill, range(nchunks)))
        else:
            for c in range(nchunks):
                fill(c)
        return Stored(raw, self.dtype)


def make_layer(m: int, n: int, dtype: str, w_std: float, tokens: int, channels: str,
               seed: int) -> LayerInputs:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0])))
    a = channel_scales(channels, n, rng)
    w = rng.standard_normal((m, n), dtype=np.float32) * np.float32(w_std)
    return LayerInputs(to_storage(w, dtype), a, seed, dtype, tokens, n)


def workload_layer(config: int, layer: int = 0, m: int | None = None, n: int | None = None,
                   tokens: int | None = None) -> LayerInputs:
    """Inputs of a named workload; m/n/tokens may be overridden for a
    scaled-down case of the same distribution."""
    wl = WORKLOADS[config]
    L = wl.layers[layer]
    return make_layer(m or L.m, n or L.n, wl.dtype, wl.w_std,
                      tokens or wl.tokens, wl.channels, seed_for(config, layer))


def correlated_x(tokens: int, n: int, seed: int, dtype: str = "f32") -> Stored:
    """Calibration inputs with correlated channels, X = zeta (I + G / sqrt(n))^T
    with G Gaussian: makes H far from diagonal so that error propagation
    matters (not one of the named workloads; a harder parity input)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2])))
    G = rng.standard_normal((n, n)).astype(np.float32) / np.float32(np.sqrt(n))
    M = np.eye(n, dtype=np.float32) + G
    a = np.exp(0.5 * rng.standard_normal(n)).astype(np.float32)
    z = rng.standard_normal((tokens, n), dtype=np.float32) * a[None, :]
    return to_storage(z @ M.T, dtype)


def gaussian_w(m: int, n: int, seed: int, std: float = 0.02, dtype: str = "f32") -> Stored:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    return to_storage(rng.standard_normal((m, n), dtype=np.float32) * np.float32(std), dtype)
