"""Seeded synthetic FNO-shaped gradients and weights.

The TensorGRaD pages train Fourier-neural-operator layers whose spectral weights are
order-4/5 tensors (in-channels, out-channels, Fourier modes...); the datasets behind
their numbers (Navier-Stokes 1024x1024, Darcy, Burgers, EM waves) are not available
here, so every input is drawn by this module instead:

* a Tucker low-rank signal: a core of the given signal ranks, N(0, 1) at step 0 and
  drifting by 0.1 * N(0, 1) per step, expanded by fixed random orthonormal factors
  (QR of a Gaussian matrix, drawn from the base seed);
* Gaussian noise with standard deviation 0.01, fresh every step;
* heavy-tailed outliers: floor(1% N) positions fixed by the base seed, plus (for some
  workloads) floor(0.2% N) positions drawn per step; each outlier *replaces* the entry
  with a Laplace(0, b=5) draw, fresh every step;
* weights drawn N(0, 0.02) in fp32 and rounded to the storage dtype.

Complex workloads draw their real and imaginary parts from two independent real
streams. Step t of a stream with base seed s uses numpy's generator seeded with s + t.

Storage convention (numpy): f32 -> float32, f16 -> float16, bf16 -> uint16 holding the
bf16 bit pattern, c64 -> complex64 (interleaved real, imag). Half-precision arrays are
drawn in fp32 and rounded to nearest-even by torch's CPU cast.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

LR = 1e-3
BETAS = (0.9, 0.999)
EPS = 1e-8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Tuple[int, ...]
    dtype: str                    # "f32" | "f16" | "bf16" | "c64"
    ranks: Tuple[int, ...]        # Tucker ranks of the optimizer
    signal_ranks: Tuple[int, ...]  # ranks of the synthetic signal
    sparse_ratio: float
    T: int
    steps: int
    layers: int = 1
    outlier_fixed: float = 0.01
    outlier_random: float = 0.0
    lr: float = LR
    betas: Tuple[float, float] = BETAS
    eps: float = EPS

    @property
    def numel(self) -> int:
        return int(np.prod(self.shape, dtype=np.int64))

    @property
    def k(self) -> int:
        return int(math.floor(self.sparse_ratio * self.numel))


TINY_F32 = Workload("tiny-fp32-(8,8,6,6)", (8, 8, 6, 6), "f32", (4, 4, 3, 3), (3, 3, 2, 2),
                    0.05, T=5, steps=10)
F32_32x32x16x16 = Workload("fp32-(32,32,16,16)", (32, 32, 16, 16), "f32", (16, 16, 8, 8), (8, 8, 4, 4),
                           0.05, T=10, steps=50, outlier_random=0.002)
F16_4x64x64x64x64 = Workload("fp16-4x(64,64,64,64)", (64, 64, 64, 64), "f16", (32, 32, 32, 32),
                             (16, 16, 16, 16), 0.05, T=100, steps=200, layers=4)
C64_64x64x64x33 = Workload("c64-(64,64,64,33)", (64, 64, 64, 33), "c64", (32, 32, 32, 16), (16, 16, 16, 8),
                           0.05, T=100, steps=100, outlier_random=0.002)
BF16_64x64x48x48x25 = Workload("bf16-(64,64,48,48,25)", (64, 64, 48, 48, 25), "bf16", (32, 32, 24, 24, 13),
                               (16, 16, 12, 12, 6), 0.05, T=200, steps=400)

# every workload by its own name
WORKLOADS = {w.name: w for w in (TINY_F32, F32_32x32x16x16, F16_4x64x64x64x64,
                                  C64_64x64x64x33, BF16_64x64x48x48x25)}

# Seed offsets for independent streams of one workload.
LAYER_SEED_STRIDE = 1000
IMAG_SEED_OFFSET = 100_000


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round an fp32 (or complex64) array to the storage dtype (nearest-even)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float32).astype(np.float16))
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if dtype == "c64":
        return np.ascontiguousarray(x, dtype=np.complex64)
    raise ValueError(dtype)


def storage_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decode a storage array to float32 (complex64 stays complex64). Exact."""
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32)
    if dtype == "c64":
        return x.astype(np.complex64)
    return x.astype(np.float32)


def _orthonormal(rng: np.random.Generator, n: int, r: int) -> np.ndarray:
    q, _ = np.linalg.qr(rng.standard_normal((n, r)))
    return q.astype(np.float32)


class _RealStream:
    """One real-valued stream of synthetic gradients (see module docstring)."""

    def __init__(self, shape, signal_ranks, seed, n_fixed, n_random,
                 noise_std=0.01, drift_std=0.1, laplace_b=5.0):
        self.shape = tuple(int(s) for s in shape)
        self.seed = int(seed)
        self.n = int(np.prod(self.shape, dtype=np.int64))
        base = np.random.default_rng(self.seed)
        self.factors = [_orthonormal(base, i, r) for i, r in zip(self.shape, signal_ranks)]
        self.core = base.standard_normal(tuple(signal_ranks))
        self.fixed_pos = (np.sort(base.choice(self.n, size=n_fixed, replace=False))
                          if n_fixed > 0 else np.zeros(0, np.int64))
        self.n_random = int(n_random)
        self.noise_std = noise_std
        self.drift_std = drift_std
        self.laplace_b = laplace_b
        self.t = 0

    def next(self) -> np.ndarray:
        self.t += 1
        rng = np.random.default_rng(self.seed + self.t)
        self.core = self.core + self.drift_std * rng.standard_normal(self.core.shape)
        sig = self.core.astype(np.float32)
        for n, f in enumerate(self.factors):
            sig = np.moveaxis(np.tensordot(f, sig, axes=([1], [n])), 0, n)
        g = np.ascontiguousarray(sig, dtype=np.float32).reshape(-1)
        g += self.noise_std * rng.standard_normal(self.n, dtype=np.float32)
        if self.fixed_pos.size:
            g[self.fixed_pos] = rng.laplace(0.0, self.laplace_b, self.fixed_pos.size)
        if self.n_random:
            pos = rng.choice(self.n, size=self.n_random, replace=False)
            g[pos] = rng.laplace(0.0, self.laplace_b, self.n_random)
        return g.reshape(self.shape)


class GradStream:
    """Gradient stream of one tensor of a workload: .next() returns step t's gradient in
    storage dtype (see module docstring), starting at t = 1."""

    def __init__(self, wl: Workload, seed: int = 0, layer: int = 0,
                 shape: Optional[Sequence[int]] = None,
                 signal_ranks: Optional[Sequence[int]] = None):
        shape = tuple(shape) if shape is not None else wl.shape
        sr = tuple(signal_ranks) if signal_ranks is not None else wl.signal_ranks
        n = int(np.prod(shape, dtype=np.int64))
        nf = int(math.floor(wl.outlier_fixed * n))
        nr = int(math.floor(wl.outlier_random * n))
        s = seed + LAYER_SEED_STRIDE * layer
        self.dtype = wl.dtype
        self.re = _RealStream(shape, sr, s, nf, nr)
        self.im = _RealStream(shape, sr, s + IMAG_SEED_OFFSET, nf, nr) if wl.dtype == "c64" else None

    def next(self) -> np.ndarray:
        g = self.re.next()
        if self.im is not None:
            g = g.astype(np.complex64)
            g.imag = self.im.next()
        return to_storage(g, self.dtype)


def init_weights(wl: Workload, seed: int = 0, layer: int = 0,
                 shape: Optional[Sequence[int]] = None) -> np.ndarray:
    """Weights N(0, 0.02) drawn in fp32 (complex: independent real/imag), then rounded."""
    shape = tuple(shape) if shape is not None else wl.shape
    rng = np.random.default_rng(seed + LAYER_SEED_STRIDE * layer + 777_777)
    w = 0.02 * rng.standard_normal(shape, dtype=np.float32)
    if wl.dtype == "c64":
        w = w.astype(np.complex64)
        w.imag = 0.02 * rng.standard_normal(shape, dtype=np.float32)
    return to_storage(w, wl.dtype)


def custom(shape, dtype, ranks, sparse_ratio, T=5, steps=3, signal_ranks=None,
           outlier_fixed=0.01, outlier_random=0.0, lr=LR, betas=BETAS, eps=EPS) -> Workload:
    """A workload with arbitrary sizes, for edge-case tests."""
    if signal_ranks is None:
        signal_ranks = tuple(max(1, r // 2) for r in ranks)
    return Workload(f"custom-{dtype}-{tuple(shape)}", tuple(shape), dtype, tuple(ranks),
                    tuple(signal_ranks), float(sparse_ratio), T=T, steps=steps,
                    outlier_fixed=outlier_fixed, outlier_random=outlier_random,
                    lr=lr, betas=betas, eps=eps)
