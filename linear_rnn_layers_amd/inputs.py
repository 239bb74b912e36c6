"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the attention method: it only draws
Gaussian numbers from a named seed and rounds them to the storage type.  Both
the float64 oracle and the HIP library receive exactly the values produced
here (the oracle reads the rounded values, widened exactly to float64).

Recipe (every array):
  numpy ``Generator(PCG64(seed)).standard_normal(shape)`` in float64,
  multiplied by ``sigma``, rounded to float32 (round to nearest even), and for
  bf16 storage rounded once more from float32 to bfloat16 (round to nearest
  even on the upper 16 bits).  Arrays are returned as float32 numpy arrays
  whose values are exactly representable in the storage type.

The workloads mirror the shapes of the experiments on the pages (MNIST-sized
sequences of 784 pixels with 8 heads of 32 dimensions, CIFAR-10-sized
sequences of 3072 pixels, a 2**16-long synthetic sequence, a bidirectional
speech encoder over 800-frame utterances, batched RNN decoding); the datasets themselves are not used, Gaussian inputs stand in.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F32 = "f32"
BF16 = "bf16"
DTYPES = (F32, BF16)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounding = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    out = ((bits + rounding) >> np.uint64(16)) << np.uint64(16)
    return out.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even); returns the uint16 bit patterns (the
    same values as round_to_bf16, without the widening back to float32)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def gaussian_bf16_bits(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    """gaussian(shape, seed, sigma, BF16) as uint16 bfloat16 bit patterns (for uploading large pools)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits((g.standard_normal(size=tuple(int(s) for s in shape)) * sigma).astype(np.float32))


def gaussian(shape, seed: int, sigma: float = 1.0, dtype: str = F32) -> np.ndarray:
    """N(0, sigma^2) samples from PCG64(seed), rounded to ``dtype`` storage."""
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")
    g = np.random.Generator(np.random.PCG64(seed))
    x = (g.standard_normal(size=tuple(int(s) for s in shape)) * sigma).astype(np.float32)
    if dtype == BF16:
        x = round_to_bf16(x)
    return x


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, storage type, input scale and seeds."""

    name: str
    B: int
    H: int
    N: int
    D: int
    M: int
    dtype: str
    sigma: float
    seeds: tuple  # seeds for Q, K, V, dO (and extra as the workload needs)
    layers: int = 1
    steps: int = 0  # decode steps (decode workload only)
    gate_seed: int = 0  # decayed workloads: seed of the per-token gates
    gate_bias: float = 3.0
    features: int = 0  # feature-map workloads: number of features C (random: projection seed seeds[0] + 50)
    fmap: str = "random"  # feature map of the feature-map workloads: "random" or "poly2" (degree 2)

    def projection(self):
        """Random projection W [H, C, D] ~ N(0, 1) float32 for the random-feature workloads."""
        return gaussian((self.H, self.features, self.D), self.seeds[0] + 50, 1.0, F32)

    def qkv(self, layer: int = 0, n: int | None = None):
        """Q [B,H,N,D], K [B,H,N,D], V [B,H,N,M] for one layer (float32 arrays)."""
        n = self.N if n is None else n
        sq, sk, sv = self.layer_seeds(layer)[:3]
        q = gaussian((self.B, self.H, n, self.D), sq, self.sigma, self.dtype)
        k = gaussian((self.B, self.H, n, self.D), sk, self.sigma, self.dtype)
        v = gaussian((self.B, self.H, n, self.M), sv, self.sigma, self.dtype)
        return q, k, v

    def grad_out(self, layer: int = 0, n: int | None = None):
        """Upstream gradient dO [B,H,N,M] ~ N(0,1) in the storage type."""
        n = self.N if n is None else n
        sd = self.layer_seeds(layer)[3]
        return gaussian((self.B, self.H, n, self.M), sd, 1.0, self.dtype)

    def layer_seeds(self, layer: int):
        if self.layers == 1:
            return self.seeds
        base = self.seeds[0]
        return tuple(base + 10 * layer + i for i in range(4))

    def decode_step_inputs(self, step: int):
        """Per-step q [B,H,D], k [B,H,D], v [B,H,M] ~ N(0,1) in the storage type."""
        base = 5_000_000 + 3 * step
        q = gaussian((self.B, self.H, self.D), base + 0, 1.0, self.dtype)
        k = gaussian((self.B, self.H, self.D), base + 1, 1.0, self.dtype)
        v = gaussian((self.B, self.H, self.M), base + 2, 1.0, self.dtype)
        return q, k, v

    def decode_step_bits(self, step: int, base: int = 5_000_000):
        """decode_step_inputs(step) as uint16 bfloat16 bit patterns (bf16 workloads; seeds base + 3 step + i)."""
        b = base + 3 * step
        return (gaussian_bf16_bits((self.B, self.H, self.D), b + 0), gaussian_bf16_bits((self.B, self.H, self.D), b + 1),
                gaussian_bf16_bits((self.B, self.H, self.M), b + 2))

    def log_a(self, n: int | None = None):
        """Per-token, per-head log-decay [B,H,N] float32 for the decayed workloads: the log of a gate
        a = 1 / (1 + exp(-x)), x ~ N(gate_bias, 1) (seed gate_seed); None for the others."""
        if not self.gate_seed:
            return None
        n = self.N if n is None else n
        x = gaussian((self.B, self.H, n), self.gate_seed).astype(np.float64) + self.gate_bias
        return (-np.log1p(np.exp(-x))).astype(np.float32)

    @property
    def tokens(self) -> int:
        return self.B * self.N


# The workloads.  Seeds follow one fixed scheme so every run of every
# test or benchmark sees the same numbers.
SMALL = Workload("causal-fwd-b1h1n64d32-f32", 1, 1, 64, 32, 32, F32, 1.0, (101, 102, 103, 104))
MNIST = Workload("mnist-layer-b16h8n784d32-f32", 16, 8, 784, 32, 32, F32, 1.0, (201, 202, 203, 204))
CIFAR = Workload("cifar-16layers-b4h8n3072d32-bf16", 4, 8, 3072, 32, 32, BF16, 0.5, (3000, 3001, 3002, 3003),
                 layers=16)
LONG = Workload("long-b1h16n65536d64-bf16", 1, 16, 65536, 64, 64, BF16, 1.0 / 8.0, (401, 402, 403, 404))
# Bidirectional speech encoder: 9 layers of 6 heads x 32 over the average utterance length of 800 frames
# (the pages give no batch size; 16 as in the MNIST workload).
SPEECH = Workload("speech-encoder-9layers-b16h6n800d32-f32", 16, 6, 800, 32, 32, F32, 1.0, (6000, 6001, 6002, 6003),
                  layers=9)
# The long sequence with a data-dependent decay on the state (gated variant of the recurrence): per-token gates
# 1 / (1 + exp(-x)), x ~ N(3, 1), i.e. about 0.95 on average.
LONG_DECAY = Workload("long-decay-b1h16n65536d64-bf16", 1, 16, 65536, 64, 64, BF16, 1.0 / 8.0, (421, 422, 423, 424),
                      gate_seed=425)
# The MNIST-shaped layer with positive random features of size 64 in place of elu + 1; queries and keys scaled
# by 32^(-1/4) (the temperature of the softmax kernel exp(q.k / sqrt(d)) that the features estimate).
MNIST_RF = Workload("mnist-random-features-b16h8n784d32c64-f32", 16, 8, 784, 32, 32, F32, 32 ** -0.25,
                    (241, 242, 243, 244), features=64)
# The same layer with 256 positive random features: four 64-feature slices per head.
MNIST_RF256 = Workload("mnist-random-features-b16h8n784d32c256-f32", 16, 8, 784, 32, 32, F32, 32 ** -0.25,
                       (251, 252, 253, 254), features=256)
# One layer of the CIFAR-shaped stack with the degree-2 polynomial map of its 32-wide heads in place of elu + 1:
# C = 1 + 32 + 32^2 = 1057 features, zero-padded to 1088 (17 slices of 64); the quadratic cost in D pays off once
# N exceeds D^2 = 1024 ("Transformers are RNNs -- part 2/3", section 3.2.1).  Queries and keys scaled by
# 32^(-1/4), as for the random features.
CIFAR_POLY2 = Workload("cifar-poly2-b4h8n3072d32c1088-bf16", 4, 8, 3072, 32, 32, BF16, 32 ** -0.25,
                       (3100, 3101, 3102, 3103), features=1088, fmap="poly2")
DECODE = Workload("decode-b256h16d64-4096steps-bf16", 256, 16, 512, 64, 64, BF16, 1.0, (501, 502, 503, 504),
                  steps=4096)

WORKLOADS = {w.name: w for w in (SMALL, MNIST, CIFAR, LONG, SPEECH, LONG_DECAY, MNIST_RF, MNIST_RF256, CIFAR_POLY2,
                                  DECODE)}
