"""Shared helpers of the GPU parity tests (inputs, guard bands, metrics)."""
from __future__ import annotations

import functools
import sys

import numpy as np

import synth

GUARD = 256
NAN32 = 0x7FC0DEAD
NAN16 = 0x7E01

# GEMM acceptance: normwise relative error and per-token-row cosine against
# the binary64 oracle.
NORMWISE_TOL = 1e-3
COSINE_MIN = 0.9999


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def normwise(y: np.ndarray, ref: np.ndarray) -> float:
    ref = ref.astype(np.float64)
    return float(np.linalg.norm(y.astype(np.float64) - ref) / np.linalg.norm(ref))


def min_row_cos(y: np.ndarray, ref: np.ndarray) -> float:
    y = y.astype(np.float64)
    ref = ref.astype(np.float64)
    num = (y * ref).sum(axis=1)
    den = np.linalg.norm(y, axis=1) * np.linalg.norm(ref, axis=1)
    return float((num / den).min())


def assert_close(y: np.ndarray, ref: np.ndarray, what: str) -> None:
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    nw = normwise(y, ref)
    cs = min_row_cos(y, ref)
    say(f"  {what}: normwise {nw:.3e}  min row cos {cs:.8f}")
    assert nw <= NORMWISE_TOL, f"{what}: normwise {nw:.3e} > {NORMWISE_TOL}"
    assert cs >= COSINE_MIN, f"{what}: min row cosine {cs:.8f} < {COSINE_MIN}"


def sample_tokens(t: int, n: int, seed: int) -> np.ndarray:
    """n token indices spread over [0, t): first, last, and seeded others."""
    rng = np.random.default_rng(seed)
    idx = set([0, t - 1, t // 2])
    while len(idx) < min(n, t):
        idx.add(int(rng.integers(0, t)))
    return np.array(sorted(idx), dtype=np.int64)


def tile_rows(t: int, tile: int, extra: int, seed: int) -> np.ndarray:
    """The first and last token row of every `tile`-row tile of a launch,
    plus `extra` seeded others."""
    idx = set()
    for b in range(0, t, tile):
        idx.add(b)
        idx.add(min(b + tile - 1, t - 1))
    rng = np.random.default_rng(seed)
    target = len(idx) + extra
    while len(idx) < min(target, t):
        idx.add(int(rng.integers(0, t)))
    return np.array(sorted(idx), dtype=np.int64)


@functools.lru_cache(maxsize=None)
def weights(qtype: int, rows: int, cols: int, seed: int) -> np.ndarray:
    return synth.quant_weights(qtype, rows, cols, seed)


@functools.lru_cache(maxsize=None)
def act_f16(rows: int, cols: int, seed: int) -> np.ndarray:
    return synth.activations_f16(rows, cols, seed)
