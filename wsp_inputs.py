"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no part of the windowed-attention arithmetic: it only draws
normal samples, rounds them to bfloat16 and names the workload shapes.  Both
the CPU oracle and the HIP library consume the arrays it returns.

Recipe: tensor ``i`` of workload ``name`` is ``std * standard_normal`` in
float32 drawn in canonical token order from numpy's PCG64 generator, in
chunks of 2**24 values; chunk ``c`` is drawn from
``default_rng([seed, workload_index, i, c])`` so large tensors can be filled
by several threads and stay identical.  bfloat16 inputs are the float32
samples rounded to nearest-even.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 1 << 24


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    T: int
    H: int
    W: int
    nt: int
    nh: int
    nw: int
    heads: int
    head_dim: int
    text_len: int
    dtype: str          # "f32" or "bf16"
    std: float          # standard deviation of q/k/v samples
    layouts: tuple      # window methods run in one pass ("regular", "shifted")

    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W


WORKLOADS = {
    # tiny fp32 grid, 2x2x2 ragged windows, one regular + one shifted layer
    "tiny_f32": Workload("tiny_f32", 0, 5, 20, 36, 2, 3, 3, 4, 64, 16, "f32", 1.0,
                         ("regular", "shifted")),
    # 720p-shaped latent grid, regular layout only
    "720p_bf16": Workload("720p_bf16", 1, 21, 45, 80, 4, 3, 3, 20, 128, 128, "bf16",
                          1.0 / math.sqrt(128), ("regular",)),
    # 1080p-shaped latent grid, regular + shifted layers
    "1080p_bf16": Workload("1080p_bf16", 2, 21, 68, 120, 4, 3, 3, 20, 128, 256, "bf16",
                           1.0 / math.sqrt(128), ("regular", "shifted")),
    # 32-layer alternating stack on the 1080p grid, hidden 2560 = 20 x 128
    "stack32_1080p_bf16": Workload("stack32_1080p_bf16", 3, 21, 68, 120, 4, 3, 3, 20, 128,
                                   256, "bf16", 1.0, ("regular", "shifted")),
    # 4K-shaped latent grid (T=31 exercises the 30-frame cap), shifted layout
    "4k_bf16": Workload("4k_bf16", 4, 31, 135, 240, 4, 3, 3, 20, 128, 512, "bf16",
                        1.0 / math.sqrt(128), ("shifted",)),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(shape, key, std=1.0, threads=None) -> np.ndarray:
    """float32 samples of N(0, std^2), drawn chunk by chunk from ``key``."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    key = [int(x) for x in key]

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.default_rng(key + [c])
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    for lo in range(0, u.size, CHUNK):
        uu = u[lo:lo + CHUNK]
        out[lo:lo + CHUNK] = ((uu + np.uint32(0x7FFF) + ((uu >> np.uint32(16)) & np.uint32(1)))
                              >> np.uint32(16)).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def tensor(w: Workload, i: int, shape, seed=0, std=None, bits_only=False):
    """Tensor ``i`` of workload ``w``.

    Returns (values_f32, bits) where bits is the uint16 bfloat16 pattern (or
    None for float32 workloads) and values_f32 holds exactly the values the
    device will see.  With ``bits_only`` (bf16 workloads) values_f32 is None;
    widen rows on demand with bf16_bits_to_f32.
    """
    x = normal_f32(shape, [seed, w.index, i], w.std if std is None else std)
    if w.dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        del x
        return (None if bits_only else bf16_bits_to_f32(bits)), bits
    return x, None


QKV_NAMES = ("q", "k", "v", "txt_q", "txt_k", "txt_v")


def qkv(w: Workload, seed=0, n_tokens=None, bits_only=False):
    """Canonical-order q, k, v [N, heads, D] and txt_q/k/v [Lt, heads, D].

    Returns a dict name -> (values_f32 or None, bits or None)."""
    n = w.n_tokens if n_tokens is None else n_tokens
    shp = (n, w.heads, w.head_dim)
    tshp = (w.text_len, w.heads, w.head_dim)
    shapes = (shp, shp, shp, tshp, tshp, tshp)
    return {nm: tensor(w, i, s, seed, bits_only=bits_only)
            for i, (nm, s) in enumerate(zip(QKV_NAMES, shapes))}


def custom(name, T, H, W, nt, nh, nw, heads, head_dim, text_len, dtype, std=None, index=100):
    """A workload of any shape (parity cases between the named ones)."""
    if std is None:
        std = 1.0 if dtype == "f32" else 1.0 / math.sqrt(head_dim)
    return Workload(name, index, T, H, W, nt, nh, nw, heads, head_dim, text_len, dtype, std,
                    ("regular", "shifted"))
