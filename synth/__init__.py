"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws numbers and lays bytes out in the GGUF block formats; it
holds none of the method's arithmetic (no dequantisation, no product, no norm,
no routing).  Every random draw comes from one counter-based generator,
SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; the finaliser constants are Stafford's "Mix13"):

    z_i   = seed + (i + 1) * 0x9E3779B97F4A7C15      (mod 2^64)
    z     = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
    z     = (z ^ (z >> 27)) * 0x94D049BB133111EB
    out_i = z ^ (z >> 31)

Uniform doubles are (out >> 11) * 2^-53 in [0, 1).  Normals use Box-Muller on
consecutive pairs (u1 = 1 - u_even in (0, 1], u2 = u_odd).

Value recipes (one per workload; the pages name the block types and say the
quants are random, the scale ranges are the workloads' stated ones):
  * fp16 scales d, dmin      : binary16(RNE) of U(1e-3, 1e-2)
  * Q8_0 quants              : integers uniform in [-127, 127]
  * Q4_K 12 scale bytes, qs  : uniform random bytes
  * Q5_K 12 scale bytes, qh, qs : uniform random bytes
  * Q6_K ql, qh              : uniform random bytes; scales int8 uniform over [-128, 127]
  * Q2_K scales, qs          : uniform random bytes
  * F16 weights              : binary16 (RNE) of N(0, 1) * 2^-6
  * activations X            : N(0, 1), as f32 or rounded to binary16 (RNE)
  * QK-norm gains            : f32 U(0.5, 1.5)
  * router logits            : f32 N(0, 1)

Block byte maps (GGUF / ggml on-disk convention; offsets in bytes):
  F16    2 B / 1 weight   : the weight as little-endian binary16
  Q8_0  34 B / 32 weights : d f16 @0, qs int8[32] @2
  Q4_K 144 B / 256        : d f16 @0, dmin f16 @2, scales u8[12] @4, qs u8[128] @16
  Q5_K 176 B / 256        : d f16 @0, dmin f16 @2, scales u8[12] @4, qh u8[32] @16, qs u8[128] @48
  Q6_K 210 B / 256        : ql u8[128] @0, qh u8[64] @128, scales i8[16] @192, d f16 @208
  Q2_K  84 B / 256        : scales u8[16] @0, qs u8[64] @16, d f16 @80, dmin f16 @82
A row of `cols` weights is ceil(cols / QK) whole blocks; a tensor is `rows`
such rows back to back.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
MASK64 = (1 << 64) - 1

# ggml type ids
F16W, Q8_0, Q2_K, Q4_K, Q5_K, Q6_K = 1, 8, 10, 12, 13, 14
Q4_0 = 2  # a KV cache format here, not a weight type
BLOCK = {F16W: (1, 2), Q4_0: (32, 18), Q8_0: (32, 34), Q4_K: (256, 144), Q5_K: (256, 176), Q6_K: (256, 210), Q2_K: (256, 84)}
NAMES = {F16W: "F16", Q4_0: "Q4_0", Q8_0: "Q8_0", Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K", Q2_K: "Q2_K"}
BY_NAME = {v: k for k, v in NAMES.items()}

BASE_SEED = 0x9E3779B9
_CHUNK = 1 << 22


def seed_for(config: int, tensor: int) -> int:
    """Seed of tensor `tensor` of workload `config` (0-based workload index)."""
    return (BASE_SEED + 1000 * config + tensor) & MASK64


def substream(seed: int, tag: int) -> int:
    """Independent sub-stream of `seed` for one field of a tensor."""
    return (seed ^ ((tag + 1) * 0xD1B54A32D192ED03)) & MASK64


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Outputs offset .. offset+n-1 of the SplitMix64 stream with this seed."""
    out = np.empty(n, dtype=np.uint64)
    s = np.uint64(seed & MASK64)
    with np.errstate(over="ignore"):
        for a in range(0, n, _CHUNK):
            b = min(n, a + _CHUNK)
            z = np.arange(offset + a + 1, offset + b + 1, dtype=np.uint64)
            z *= GAMMA
            z += s
            z ^= z >> np.uint64(30)
            z *= M1
            z ^= z >> np.uint64(27)
            z *= M2
            z ^= z >> np.uint64(31)
            out[a:b] = z
    return out


def uniform(seed: int, n: int) -> np.ndarray:
    """n doubles uniform in [0, 1)."""
    return (splitmix64(seed, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform_range(seed: int, n: int, lo: float, hi: float) -> np.ndarray:
    return lo + (hi - lo) * uniform(seed, n)


def normal(seed: int, n: int) -> np.ndarray:
    """n standard normals (float64), Box-Muller over consecutive uniform pairs."""
    m = (n + 1) // 2
    u = uniform(seed, 2 * m)
    u1 = 1.0 - u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * m, dtype=np.float64)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out[:n]


def random_bytes(seed: int, n: int) -> np.ndarray:
    words = splitmix64(seed, (n + 7) // 8)
    return words.view(np.uint8)[:n].copy()


def f16_bits(values: np.ndarray) -> np.ndarray:
    """binary16 bit patterns (numpy's float64 -> float16 conversion is RNE)."""
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def nblocks(qtype: int, cols: int) -> int:
    qk, _ = BLOCK[qtype]
    return (cols + qk - 1) // qk


def row_bytes(qtype: int, cols: int) -> int:
    return nblocks(qtype, cols) * BLOCK[qtype][1]


def _put_f16(blocks: np.ndarray, off: int, bits: np.ndarray) -> None:
    blocks[:, off] = (bits & 0xFF).astype(np.uint8)
    blocks[:, off + 1] = (bits >> 8).astype(np.uint8)


def quant_weights(qtype: int, rows: int, cols: int, seed: int,
                  scale_lo: float = 1e-3, scale_hi: float = 1e-2) -> np.ndarray:
    """A rows x cols weight tensor in `qtype` blocks, as a flat uint8 array."""
    qk, ts = BLOCK[qtype]
    if qtype == F16W:
        return f16_bits(normal(seed, rows * cols) * 2.0 ** -6).view(np.uint8).reshape(-1)
    nb = rows * nblocks(qtype, cols)
    blocks = random_bytes(substream(seed, 0), nb * ts).reshape(nb, ts)
    d = f16_bits(uniform_range(substream(seed, 1), nb, scale_lo, scale_hi))
    if qtype == Q8_0:
        q = np.floor(uniform(substream(seed, 2), nb * 32) * 255.0).astype(np.int64) - 127
        blocks[:, 2:34] = q.astype(np.int8).view(np.uint8).reshape(nb, 32)
        _put_f16(blocks, 0, d)
    elif qtype == Q4_0:
        _put_f16(blocks, 0, d)
    elif qtype in (Q4_K, Q5_K):
        dmin = f16_bits(uniform_range(substream(seed, 3), nb, scale_lo, scale_hi))
        _put_f16(blocks, 0, d)
        _put_f16(blocks, 2, dmin)
    elif qtype == Q6_K:
        _put_f16(blocks, 208, d)
    elif qtype == Q2_K:
        dmin = f16_bits(uniform_range(substream(seed, 3), nb, scale_lo, scale_hi))
        _put_f16(blocks, 80, d)
        _put_f16(blocks, 82, dmin)
    else:
        raise ValueError(f"unsupported qtype {qtype}")
    return blocks.reshape(-1)


def activations_f16(rows: int, cols: int, seed: int) -> np.ndarray:
    """rows x cols binary16 bit patterns of N(0, 1) draws."""
    return f16_bits(normal(seed, rows * cols)).reshape(rows, cols)


def activations_f32(rows: int, cols: int, seed: int) -> np.ndarray:
    return normal(seed, rows * cols).astype(np.float32).reshape(rows, cols)


def gains(n: int, seed: int) -> np.ndarray:
    return uniform_range(seed, n, 0.5, 1.5).astype(np.float32)


def router_logits(tokens: int, experts: int, seed: int) -> np.ndarray:
    return normal(seed, tokens * experts).astype(np.float32).reshape(tokens, experts)


def kv_cache(kvtype: int, tokens: int, n_kv: int, head_dim: int, seed: int) -> np.ndarray:
    """A KV cache of tokens x n_kv rows of head_dim values, flat uint8:
    binary16 N(0, 1) draws; Q8_0 blocks with scales in [1/64, 1/32] and
    quants uniform in [-127, 127] (values within about +-4); or Q4_0 blocks
    with scales in [1/4, 1/2] and uniform 4-bit quants (values within +-4)."""
    if kvtype == F16W:
        return f16_bits(normal(seed, tokens * n_kv * head_dim)).view(np.uint8).reshape(-1)
    if kvtype == Q8_0:
        return quant_weights(Q8_0, tokens * n_kv, head_dim, seed, 1.0 / 64, 1.0 / 32)
    if kvtype == Q4_0:
        return quant_weights(Q4_0, tokens * n_kv, head_dim, seed, 0.25, 0.5)
    raise ValueError(f"no KV cache recipe for type {kvtype}")


# ---------------------------------------------------------------------------
# Workloads.  Shapes are (out_features N, in_features K) per projection.

def qwen3_projections(hidden: int, inter: int, q_out: int, kv_out: int):
    return [("q", q_out, hidden), ("k", kv_out, hidden), ("v", kv_out, hidden),
            ("o", hidden, q_out), ("gate", inter, hidden), ("up", inter, hidden),
            ("down", hidden, inter)]


# Qwen3-1.7B: hidden 2048, intermediate 6144, 16 q heads / 8 kv heads x 128
PROJ_1_7B = qwen3_projections(2048, 6144, 2048, 1024)
# Qwen3-8B: hidden 4096, intermediate 12288, 32 q heads / 8 kv heads x 128
PROJ_8B = qwen3_projections(4096, 12288, 4096, 1024)

WORKLOADS = {
    "q8_0_1024": dict(index=0, qtypes=[Q8_0], proj=[("w", 1024, 1024)], t=64, x="f32"),
    "q4_k_qwen3_1p7b_t512": dict(index=1, qtypes=[Q4_K], proj=PROJ_1_7B, t=512, x="f16"),
    "q6_k_q2_k_qwen3_8b_t2048": dict(index=2, qtypes=[Q6_K, Q2_K], proj=PROJ_8B, t=2048, x="f16"),
    "qknorm_qwen3_8b_t8192": dict(index=3, t=8192, hidden=4096, head_dim=128,
                                  q=(Q4_K, 4096), k=(Q6_K, 1024), eps=1e-6),
    "moe_e128_top8_t4096": dict(index=4, t=4096, hidden=2048, inter=768, experts=128,
                                top_k=8, qtype=Q4_K),
}
