"""Seeded synthetic inputs shared by the tests, the bench and the smoke run.

This module holds no attention arithmetic.  It draws i.i.d. N(0, 1) values
with ``numpy.random.default_rng(seed)`` as float32, in the order Q, K, V and
then dO, and rounds them to the storage type with round-to-nearest-even.
The results are float32 numpy arrays whose values are exactly representable
in fp16 or bf16, so the GPU side (which casts them to the storage type) and
the float64 oracle (which upcasts them) see identical numbers.

The long-sequence spiky-key recipe scales every 64th key row (rows 0, 64,
128, ...) by 8 after rounding; 8 is a power of two, so the scaled values are
still exact in bf16.
"""

from __future__ import annotations

import numpy as np

FP16 = "fp16"
BF16 = "bf16"


def round_fp16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest fp16 (ties to even) -> float32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even) -> float32, by bit arithmetic.

    Finite inputs only (the generators never produce inf or nan).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == FP16:
        return round_fp16(x)
    if dtype == BF16:
        return round_bf16(x)
    raise ValueError("dtype must be 'fp16' or 'bf16'")


def make_inputs(B, H, N, D, dtype=FP16, seed=0, spiky_keys=False, with_dout=False,
                heads=None):
    """Draw Q, K, V (and dO) of shape [B, H, N, D] from ``default_rng(seed)``.

    ``heads``: optional list of (b, h) pairs; when given, only those heads are
    returned (shape [len(heads), N, D] each), drawn as if the full tensor had
    been drawn -- used to sample a few heads of a large workload without
    materialising it.  Returns a dict with float32 arrays "q", "k", "v" and,
    with ``with_dout``, "do".
    """
    rng = np.random.default_rng(seed)
    names = ["q", "k", "v"] + (["do"] if with_dout else [])
    out = {}
    per_head = N * D
    for name in names:
        if heads is None:
            x = rng.standard_normal((B, H, N, D), dtype=np.float32)
        else:
            # default_rng draws standard normals sequentially, so drawing the
            # whole tensor head by head reproduces the same stream.
            want = {bh: i for i, bh in enumerate(heads)}
            x = np.empty((len(heads), N, D), dtype=np.float32)
            for b in range(B):
                for h in range(H):
                    blk = rng.standard_normal(per_head, dtype=np.float32)
                    if (b, h) in want:
                        x[want[(b, h)]] = blk.reshape(N, D)
        x = round_to(x, dtype)
        if name == "k" and spiky_keys:
            x[..., ::64, :] *= np.float32(8.0)
        out[name] = x
    return out


def make_key_mask(B, N, kind="lengths", seed=0, p=0.5, lengths=None):
    """Seeded key-padding mask [B, N] (uint8, 1 = visible).

    kinds:
      "lengths" -- a right-padded variable-length batch: element b has
                   ``lengths[b]`` real tokens (drawn uniformly in 1..N when
                   not given), key j visible iff j < L_b;
      "random"  -- every key visible with probability ``p`` (random mask
                   patterns, which may leave rows with no visible key);
      "blocks"  -- each 64-key tile is, with equal odds, wholly hidden,
                   wholly visible or random with probability ``p``, so the
                   block-level flags see every kind of tile;
      "all"     -- every key visible.
    """
    rng = np.random.default_rng(seed)
    if kind == "lengths":
        lens = np.asarray(lengths if lengths is not None else rng.integers(1, N + 1, size=B))
        return (np.arange(N)[None, :] < lens[:, None]).astype(np.uint8)
    if kind == "random":
        return (rng.random((B, N)) < p).astype(np.uint8)
    if kind == "blocks":
        m = np.empty((B, N), dtype=np.uint8)
        for b in range(B):
            for t0 in range(0, N, 64):
                c = rng.integers(0, 3)
                n = min(64, N - t0)
                m[b, t0:t0 + n] = 0 if c == 0 else (1 if c == 1 else (rng.random(n) < p))
        return m
    if kind == "all":
        return np.ones((B, N), dtype=np.uint8)
    raise ValueError("unknown mask kind %r" % kind)
