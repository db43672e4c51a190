"""Seeded synthetic inputs for the LLSA hot path.

This module is shared by the oracle side and the HIP side of the test suite and
by the benchmark.  It holds none of the attention method's arithmetic: it only
draws random fields, smooths them, rescales them and rounds them to the storage
dtype.  Tokens are returned in raster order (row-major over the 2-D grid); each
side applies its own Z-order permutation.

Recipe (stand-in for the pixel-space DiT activations of the LLSA README, page 1
"experiments", whose FFHQ data and checkpoints are not available here):
  1. rng = numpy.random.default_rng(seed)
  2. float64 standard normals [B, H, rows, side, d] for Q, then K, then V
     ([B, H, frames, rows, side, d] for video), then dO with shape [B, H, N, d]
     (dO is not smoothed); rows = side unless the grid is a rectangle
  3. Q, K, V: separable normalised Gaussian blur over the grid axes (frames
     too, for video), sigma cells, radius ceil(4 sigma), periodic boundary;
     sigma 0 leaves them white
  4. each of Q, K, V divided by its own standard deviation
  5. rounding to the storage dtype (fp32, or bf16 round-to-nearest-even)
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "gaussian_kernel_1d", "blur_periodic",
           "round_bf16", "bf16_bits_to_f64", "make_inputs"]


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload: shapes, dtype and method parameters."""
    name: str
    B: int
    H: int
    side: int
    d: int
    dtype: str          # "f32" or "bf16"
    levels: int
    topk: int
    sigma: float
    seed: int = 0
    block_size: int = 16
    frames: int = 1     # > 1: video of `frames` frames
    height: int = 0     # rows of the grid; 0: square (rows = side)

    @property
    def rows(self) -> int:
        return self.height or self.side

    @property
    def N(self) -> int:
        return self.frames * self.rows * self.side

    @property
    def G(self) -> int:
        return self.B * self.H


# The workloads of the LLSA hot path: a small fp32 correctness case, bf16 pixel
# grids of 64^2, 128^2, 256^2 (headline) and 512^2 tokens, two grids the
# README's power-of-two limits exclude (video, a rectangle), and d = 128.
WORKLOADS = {
    w.name: w for w in [
        Workload("grid32_f32_l1_k8", 1, 1, 32, 64, "f32", 1, 8, 2.0),
        Workload("grid64_bf16_l1_k16", 2, 6, 64, 64, "bf16", 1, 16, 2.0),
        Workload("grid128_bf16_l2_k16", 2, 6, 128, 64, "bf16", 2, 16, 2.0),
        Workload("grid256_bf16_l2_k16", 1, 6, 256, 64, "bf16", 2, 16, 4.0),
        Workload("grid512_bf16_l3_k16", 1, 6, 512, 64, "bf16", 3, 16, 2.0),
        # the same token budget as 256^2 as 16 frames of 64^2 (octree order),
        # and a 192 x 320 image (N = 61440, not a power of two)
        Workload("video16x64x64_bf16_l2_k16", 1, 6, 64, 64, "bf16", 2, 16, 2.0, frames=16),
        Workload("rect192x320_bf16_l2_k16", 1, 6, 320, 64, "bf16", 2, 16, 4.0, height=192),
        # head dimension 128 at the headline grid
        Workload("grid256_d128_bf16_l2_k16", 1, 6, 256, 128, "bf16", 2, 16, 4.0),
    ]
}


def gaussian_kernel_1d(sigma: float) -> np.ndarray:
    """Normalised 1-D Gaussian taps for offsets -r..r, r = ceil(4 sigma)."""
    r = int(math.ceil(4.0 * sigma))
    x = np.arange(-r, r + 1, dtype=np.float64)
    w = np.exp(-0.5 * (x / sigma) ** 2)
    return w / w.sum()


def blur_periodic(x: np.ndarray, sigma: float, axes=(-3, -2)) -> np.ndarray:
    """Separable periodic Gaussian blur over the given grid axes (via FFT).

    The taps are wrapped onto the periodic grid, so this is an exact circular
    convolution (up to FFT rounding) even when the grid is smaller than the
    kernel support.
    """
    w = gaussian_kernel_1d(sigma)
    r = (len(w) - 1) // 2
    out = x
    for ax in axes:
        n = x.shape[ax]
        ker = np.zeros(n, dtype=np.float64)
        for o, wt in zip(range(-r, r + 1), w):
            ker[o % n] += wt
        kf = np.fft.rfft(ker)
        shape = [1] * x.ndim
        shape[ax] = kf.shape[0]
        xf = np.fft.rfft(out, axis=ax)
        out = np.fft.irfft(xf * kf.reshape(shape), n=n, axis=ax)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (via fp32, nearest-even); returns uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns."""
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _cast(x: np.ndarray, dtype: str):
    """Return (storage array, exact float64 values of the storage array)."""
    if dtype == "f32":
        s = x.astype(np.float32)
        return s, s.astype(np.float64)
    if dtype == "bf16":
        s = round_bf16(x)
        return s, bf16_bits_to_f64(s)
    raise ValueError(dtype)


def make_inputs(w: Workload, want_grad: bool = True) -> dict:
    """Draw the seeded inputs of workload `w`.

    Returns a dict with, for each of "q", "k", "v" (raster token order) and
    "do" (attention token order), the storage array ("q" etc., np.float32 or
    uint16 bf16 bits, shape [B, H, N, d]) and its exact float64 values
    ("q64" etc.).
    """
    rng = np.random.default_rng(w.seed)
    if w.frames > 1:
        shape, axes = (w.B, w.H, w.frames, w.rows, w.side, w.d), (-4, -3, -2)
    else:
        shape, axes = (w.B, w.H, w.rows, w.side, w.d), (-3, -2)
    out = {}
    for name in ("q", "k", "v"):
        x = rng.standard_normal(shape)
        if w.sigma > 0:  # sigma 0: white noise (the largest shapes, where a blur is costly)
            x = blur_periodic(x, w.sigma, axes)
        x = x / x.std()
        x = x.reshape(w.B, w.H, w.N, w.d)
        out[name], out[name + "64"] = _cast(x, w.dtype)
    if want_grad:
        g = rng.standard_normal((w.B, w.H, w.N, w.d))
        out["do"], out["do64"] = _cast(g, w.dtype)
    return out


def random_tensor(shape, seed: int, dtype: str = "f32", scale: float = 1.0):
    """Plain seeded normal noise (for small unit tests); returns (storage, f64)."""
    rng = np.random.default_rng(seed)
    return _cast(rng.standard_normal(shape) * scale, dtype)
