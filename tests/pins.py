"""Pins: checks of the CPU oracle against facts that do not come from the oracle.

Each pin takes an `oracle.Oracle` (the default build, or one compiled with a
planted mistake) and raises AssertionError when the oracle disagrees with:
  * hand-worked single blocks (tests/golden/hand_blocks.json, derivations inline);
  * closed-form values of every (scale, min, quant) combination, with blocks
    built by an encoder written here (the inverse of the byte maps), never by
    the oracle's decoder;
  * invariants (a partial row is the prefix of the full row; rows are
    independent of the row stride; nothing outside rows x cols is written);
  * library routines (numpy's binary16 conversions and float64 matmul, Python's
    sort) and closed forms of the norm, router and SiLU.

The planted-fault test runs this whole battery on every planted build and
requires at least one pin to fail for each.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import synth
from synth import F16W, Q4_0, Q8_0, Q4_K, Q5_K, Q6_K, Q2_K

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "hand_blocks.json")


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def h16(v: float) -> int:
    """binary16 bits of a float via numpy (RNE)."""
    return int(np.array([v], dtype=np.float64).astype(np.float16).view(np.uint16)[0])


def h16_value(bits: int) -> float:
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


# ---------------------------------------------------------------------------
# Block encoders (inverse of the byte maps), independent of the oracle.

def _put16(b: np.ndarray, off: int, bits: int) -> None:
    b[off] = bits & 0xFF
    b[off + 1] = bits >> 8


def enc_q8_0(d_bits: int, q: np.ndarray) -> np.ndarray:
    b = np.zeros(34, np.uint8)
    _put16(b, 0, d_bits)
    b[2:] = np.asarray(q, dtype=np.int64).astype(np.int8).view(np.uint8)
    return b


def enc_q4_0(d_bits: int, q: np.ndarray) -> np.ndarray:
    """Q4_0 block from 32 quants in [0, 15]: quant j < 16 is the low nibble of
    byte 2 + j, quant j >= 16 the high nibble of byte 2 + j - 16."""
    q = np.asarray(q, dtype=np.int64)
    b = np.zeros(18, np.uint8)
    _put16(b, 0, d_bits)
    b[2:] = (q[:16] | (q[16:] << 4)).astype(np.uint8)
    return b


def enc_q4_k(d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    """sc, m: 8 six-bit values; q: 256 four-bit values (weight order)."""
    b = np.zeros(144, np.uint8)
    _put16(b, 0, d_bits)
    _put16(b, 2, dmin_bits)
    s = b[4:16]
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
    for j in range(4, 8):
        s[j + 4] = (sc[j] & 15) | ((m[j] & 15) << 4)
    qs = b[16:]
    for i in range(256):
        idx = 32 * (i // 64) + i % 32
        if (i % 64) < 32:
            qs[idx] |= q[i] & 15
        else:
            qs[idx] |= (q[i] & 15) << 4
    return b


def enc_q5_k(d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    """sc, m: 8 six-bit values; q: 256 five-bit values (weight order).  The
    scales and the low four bits are placed as for Q4_K (qs at byte 48); the
    fifth bit of weight i is bit i // 32 of qh[i % 32] (qh at byte 16)."""
    q = np.asarray(q, dtype=np.int64)
    lo = enc_q4_k(d_bits, dmin_bits, sc, m, q & 15)
    b = np.zeros(176, np.uint8)
    b[0:16] = lo[0:16]
    b[48:176] = lo[16:144]
    qh = b[16:48]
    for i in range(256):
        qh[i % 32] |= ((int(q[i]) >> 4) & 1) << (i // 32)
    return b


def enc_q6_k(d_bits: int, sc, q) -> np.ndarray:
    """sc: 16 signed scales; q: 256 values in [-32, 31]."""
    b = np.zeros(210, np.uint8)
    ql, qh = b[0:128], b[128:192]
    b[192:208] = np.asarray(sc, dtype=np.int64).astype(np.int8).view(np.uint8)
    _put16(b, 208, d_bits)
    for i in range(256):
        u = int(q[i]) + 32
        h, r = divmod(i, 128)
        c, l = divmod(r, 32)
        ql[64 * h + 32 * (c % 2) + l] |= (u & 15) << (4 * (c // 2))
        qh[32 * h + l] |= (u >> 4) << (2 * c)
    return b


def enc_q2_k(d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    """sc, m: 16 four-bit values; q: 256 two-bit values."""
    b = np.zeros(84, np.uint8)
    for g in range(16):
        b[g] = (sc[g] & 15) | ((m[g] & 15) << 4)
    qs = b[16:80]
    for i in range(256):
        h, r = divmod(i, 128)
        j, l = divmod(r, 32)
        qs[32 * h + l] |= (q[i] & 3) << (2 * j)
    _put16(b, 80, d_bits)
    _put16(b, 82, dmin_bits)
    return b


# scale pairs (d, dmin) for the sweeps: a draw from U(1e-3, 1e-2), negative
# values, binary16 subnormals, signed zeros, and the large-d pair of H2a
SCALE_PAIRS = [
    (h16(0.0043), h16(0.0071)),
    (h16(-0.0059), h16(-0.0023)),
    (0x0003, 0x0201),
    (0x0000, 0x8000),
    (0x8000, 0x0000),
    (0x6800, 0x2C00),
]


def _closed_form_f32(d_bits, dmin_bits, sc, q, m) -> np.ndarray:
    """(d*sc)*q - dmin*m evaluated in float64, then rounded once to f32.

    Products are exact in float64 and, for the pairs above, so is the
    difference, so this is the correctly rounded value of the definition."""
    d = h16_value(d_bits)
    v = (np.float64(d) * np.asarray(sc, np.float64)) * np.asarray(q, np.float64)
    if dmin_bits is not None:
        v = v - np.float64(h16_value(dmin_bits)) * np.asarray(m, np.float64)
    return v.astype(np.float32)


# ---------------------------------------------------------------------------
# Pins

def pin_hand_blocks(o):
    fx = json.load(open(GOLDEN))
    for blk in fx["blocks"]:
        qt = synth.BY_NAME[blk["qtype"]]
        raw = np.frombuffer(bytes.fromhex(blk["bytes"]), dtype=np.uint8)
        out = o.dequant_f32(qt, raw, 1, blk["cols"]).view(np.uint32)[0]
        for i, want in blk["expect_f32"].items():
            got = int(out[int(i)])
            assert got == int(want, 16), f"{blk['name']} f32[{i}] = {got:#010x}, want {want}"
        if "expect_f16" in blk:
            out16 = o.dequant_f16_bits(qt, raw, 1, blk["cols"])[0]
            for i, want in blk["expect_f16"].items():
                got = int(out16[int(i)])
                assert got == int(want, 16), f"{blk['name']} f16[{i}] = {got:#06x}, want {want}"


def pin_sweep_q8_0(o):
    q = np.arange(-128, 128)
    for d_bits, _ in SCALE_PAIRS:
        raw = np.concatenate([enc_q8_0(d_bits, q[32 * k:32 * k + 32]) for k in range(8)])
        got = o.dequant_f32(Q8_0, raw, 1, 256)[0]
        want = _closed_form_f32(d_bits, None, np.ones(256), q, None)
        assert np.array_equal(f32_bits(got), f32_bits(want)), f"Q8_0 sweep d={d_bits:#06x}"


def pin_sweep_q4_0(o):
    """Every quant 0..15 at every position (a cyclic shift per block, so a
    position's low and high nibble partners differ), for several scales:
    value = d * (q - 8), exact in binary32."""
    ds = [0x3400, 0x2E66, 0x0001, 0x8400, 0x7BFF, 0x0000, 0x8000, 0x3C00]
    blocks, want = [], []
    for d in ds:
        for shift in range(16):
            q = (np.arange(32) * 5 + shift + (np.arange(32) >= 16) * 3) % 16
            blocks.append(enc_q4_0(d, q))
            want.append(h16_value(d) * (q - 8.0))
    raw = np.concatenate(blocks)
    got = o.dequant_f32(Q4_0, raw, len(blocks), 32)
    assert np.array_equal(f32_bits(got), f32_bits(np.array(want, dtype=np.float64))), "Q4_0 sweep"


def pin_sweep_q4_k(o):
    # every (sc, m) pair once per sub-block; each sub-block holds q = 0..15 twice
    pairs = [(sc, m) for sc in range(64) for m in range(64)]
    qsub = np.tile(np.arange(16), 2)
    for d_bits, dmin_bits in SCALE_PAIRS:
        raws, want = [], []
        for bi in range(0, len(pairs), 8):
            grp = pairs[bi:bi + 8]
            sc = [p[0] for p in grp]
            m = [p[1] for p in grp]
            q = np.concatenate([qsub] * 8)
            raws.append(enc_q4_k(d_bits, dmin_bits, sc, m, q))
            want.append(_closed_form_f32(d_bits, dmin_bits, np.repeat(sc, 32), q, np.repeat(m, 32)))
        raw = np.concatenate(raws)
        nb = len(raws)
        got = o.dequant_f32(Q4_K, raw, nb, 256).reshape(-1)
        assert np.array_equal(f32_bits(got), f32_bits(np.concatenate(want))), \
            f"Q4_K sweep d={d_bits:#06x} dmin={dmin_bits:#06x}"


def pin_sweep_q5_k(o):
    # every (sc, m) pair once per sub-block; each sub-block holds q = 0..31 once
    pairs = [(sc, m) for sc in range(64) for m in range(64)]
    qsub = np.arange(32)
    for d_bits, dmin_bits in SCALE_PAIRS:
        raws, want = [], []
        for bi in range(0, len(pairs), 8):
            grp = pairs[bi:bi + 8]
            sc = [p[0] for p in grp]
            m = [p[1] for p in grp]
            # rotate the quants per sub-block so every qh bit position meets both values
            q = np.concatenate([np.roll(qsub, 5 * j + bi // 8) for j in range(8)])
            raws.append(enc_q5_k(d_bits, dmin_bits, sc, m, q))
            want.append(_closed_form_f32(d_bits, dmin_bits, np.repeat(sc, 32), q, np.repeat(m, 32)))
        raw = np.concatenate(raws)
        got = o.dequant_f32(Q5_K, raw, len(raws), 256).reshape(-1)
        assert np.array_equal(f32_bits(got), f32_bits(np.concatenate(want))), \
            f"Q5_K sweep d={d_bits:#06x} dmin={dmin_bits:#06x}"


def pin_sweep_q6_k(o):
    # every signed scale with every quant in [-32, 31]
    qgrp = np.arange(-32, 32)
    for d_bits, _ in SCALE_PAIRS:
        raws, want = [], []
        scales = np.arange(-128, 128)
        for bi in range(0, 256, 4):
            sc = np.repeat(scales[bi:bi + 4], 4)  # 16 groups of 16 weights
            q = np.tile(qgrp, 4)
            raws.append(enc_q6_k(d_bits, sc, q))
            want.append(_closed_form_f32(d_bits, None, np.repeat(sc, 16), q, None))
        got = o.dequant_f32(Q6_K, np.concatenate(raws), len(raws), 256).reshape(-1)
        assert np.array_equal(f32_bits(got), f32_bits(np.concatenate(want))), f"Q6_K sweep d={d_bits:#06x}"


def pin_sweep_q2_k(o):
    pairs = [(sc, m) for sc in range(16) for m in range(16)]
    qgrp = np.tile(np.arange(4), 4)
    for d_bits, dmin_bits in SCALE_PAIRS:
        raws, want = [], []
        for bi in range(0, 256, 16):
            grp = pairs[bi:bi + 16]
            sc = [p[0] for p in grp]
            m = [p[1] for p in grp]
            q = np.tile(qgrp, 16)
            raws.append(enc_q2_k(d_bits, dmin_bits, sc, m, q))
            want.append(_closed_form_f32(d_bits, dmin_bits, np.repeat(sc, 16), q, np.repeat(m, 16)))
        got = o.dequant_f32(Q2_K, np.concatenate(raws), len(raws), 256).reshape(-1)
        assert np.array_equal(f32_bits(got), f32_bits(np.concatenate(want))), \
            f"Q2_K sweep d={d_bits:#06x} dmin={dmin_bits:#06x}"


def pin_positions(o):
    """Every weight index of a block gets its own (scale, quant) pair."""
    rng = np.random.default_rng(7)
    d_bits, dmin_bits = h16(0.0037), h16(0.0061)
    # Q4_K
    sc = rng.integers(0, 64, 8)
    m = rng.integers(0, 64, 8)
    q = rng.integers(0, 16, 256)
    got = o.dequant_f32(Q4_K, enc_q4_k(d_bits, dmin_bits, sc, m, q), 1, 256)[0]
    want = _closed_form_f32(d_bits, dmin_bits, np.repeat(sc, 32), q, np.repeat(m, 32))
    assert np.array_equal(f32_bits(got), f32_bits(want)), "Q4_K positions"
    # Q5_K
    sc = rng.integers(0, 64, 8)
    m = rng.integers(0, 64, 8)
    q = rng.integers(0, 32, 256)
    got = o.dequant_f32(Q5_K, enc_q5_k(d_bits, dmin_bits, sc, m, q), 1, 256)[0]
    want = _closed_form_f32(d_bits, dmin_bits, np.repeat(sc, 32), q, np.repeat(m, 32))
    assert np.array_equal(f32_bits(got), f32_bits(want)), "Q5_K positions"
    # Q6_K
    sc = rng.integers(-128, 128, 16)
    q = rng.integers(-32, 32, 256)
    got = o.dequant_f32(Q6_K, enc_q6_k(d_bits, sc, q), 1, 256)[0]
    want = _closed_form_f32(d_bits, None, np.repeat(sc, 16), q, None)
    assert np.array_equal(f32_bits(got), f32_bits(want)), "Q6_K positions"
    # Q2_K
    sc = rng.integers(0, 16, 16)
    m = rng.integers(0, 16, 16)
    q = rng.integers(0, 4, 256)
    got = o.dequant_f32(Q2_K, enc_q2_k(d_bits, dmin_bits, sc, m, q), 1, 256)[0]
    want = _closed_form_f32(d_bits, dmin_bits, np.repeat(sc, 16), q, np.repeat(m, 16))
    assert np.array_equal(f32_bits(got), f32_bits(want)), "Q2_K positions"
    # Q8_0
    q = rng.integers(-128, 128, 32)
    got = o.dequant_f32(Q8_0, enc_q8_0(d_bits, q), 1, 32)[0]
    assert np.array_equal(f32_bits(got), f32_bits(_closed_form_f32(d_bits, None, np.ones(32), q, None)))


def pin_f16_from_f32(o):
    """The f16 copy is numpy's RNE binary16 of the f32 dequant (random blocks)."""
    for qt in (F16W, Q8_0, Q4_K, Q5_K, Q6_K, Q2_K):
        cols = 512
        raw = synth.quant_weights(qt, 3, cols, synth.seed_for(90, qt))
        f32 = o.dequant_f32(qt, raw, 3, cols)
        f16 = o.dequant_f16_bits(qt, raw, 3, cols)
        assert np.array_equal(f16, f32.astype(np.float16).view(np.uint16)), f"f16 copy {qt}"


def pin_f16_weights(o):
    """F16 weights: every binary16 pattern, laid out little-endian, widens to
    numpy's float32 of it (NaN stays NaN), in one row and as a 256 x 256
    tensor; the f16 copy gives back the same bits for every non-NaN pattern."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    raw = bits.astype("<u2").view(np.uint8)
    want = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    for rows, cols in ((1, 1 << 16), (256, 256)):
        got = o.dequant_f32(F16W, raw, rows, cols).reshape(-1)
        assert np.array_equal(np.isnan(got), nan), "F16 weights: NaN patterns"
        assert np.array_equal(f32_bits(got[~nan]), f32_bits(want[~nan])), f"F16 weights {rows}x{cols}"
        g16 = o.dequant_f16_bits(F16W, raw, rows, cols).reshape(-1)
        assert np.array_equal(g16[~nan], bits[~nan]), "F16 weights: f16 copy"


def pin_f16_convert_edges(o):
    """binary16 rounding at its edges, against numpy's conversion."""
    vals = [65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14,
            2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1087.5, 1088.5, -0.0, 0.0,
            5.960464477539063e-08, 6.097555160522461e-05, 0.1, 1 / 3.0]
    vals = np.array(vals + [-v for v in vals], dtype=np.float32)
    got = o.float_to_half_array(vals)
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), f"f16 edges {got} vs {want}"


def pin_partial_rows(o):
    """Rows of a tensor with a partial last block: each row is the prefix of
    its own blocks decoded as a full row; no write lands outside rows x cols."""
    for qt in (Q8_0, Q4_K, Q5_K, Q6_K, Q2_K):
        qk, ts = synth.BLOCK[qt]
        tails = [1, 3, 5, 17, 31] if qt == Q8_0 else [1, 16, 77, 129, 255]
        for tail in tails:
            cols = 4 * qk + tail if qt != Q8_0 else 2 * qk + tail
            rows = 3
            raw = synth.quant_weights(qt, rows, cols, synth.seed_for(91, tail))
            nb = (cols + qk - 1) // qk
            got32 = o.dequant_f32(qt, raw, rows, cols)
            got16 = o.dequant_f16_bits(qt, raw, rows, cols)
            for r in range(rows):
                own = raw[r * nb * ts:(r + 1) * nb * ts]
                full = o.dequant_f32(qt, own, 1, nb * qk)[0]
                assert np.array_equal(f32_bits(got32[r]), f32_bits(full[:cols])), f"partial row {qt} {tail} r{r}"
                full16 = o.dequant_f16_bits(qt, own, 1, nb * qk)[0]
                assert np.array_equal(got16[r], full16[:cols]), f"partial row f16 {qt} {tail} r{r}"


def pin_tail_bytes_ignored(o):
    """Bytes of the last block beyond `cols` do not change any output."""
    qt = Q6_K
    cols = 256 + 40
    raw = synth.quant_weights(qt, 1, cols, 1234)
    a = o.dequant_f32(qt, raw, 1, cols)
    raw2 = raw.copy()
    # weights 40..255 of the second block: all their ql/qh bytes are shared
    # with weights < 40 only through whole bytes, so flip the scale bytes of
    # groups 3..15 (weights 48..255), which no kept weight reads
    raw2[210 + 192 + 3:210 + 208] ^= 0x5A
    b = o.dequant_f32(qt, raw2, 1, cols)
    assert np.array_equal(f32_bits(a), f32_bits(b))


def pin_dmin_invariant(o):
    """Q4_K / Q2_K with dmin = 0 are (d*sc)*q; changing dmin shifts each weight by -dmin*m."""
    rng = np.random.default_rng(11)
    d_bits = h16(0.0047)
    sc = rng.integers(0, 64, 8)
    m = rng.integers(0, 64, 8)
    q = rng.integers(0, 16, 256)
    a = o.dequant_f32(Q4_K, enc_q4_k(d_bits, 0, sc, m, q), 1, 256)[0]
    want = (np.float64(h16_value(d_bits)) * np.repeat(sc, 32) * q).astype(np.float32)
    assert np.array_equal(f32_bits(a), f32_bits(want))


def pin_gemm_identity(o):
    """X = I (binary16 ones on the diagonal): Y[t, n] = W[n, t] exactly.  W is
    Q8_0 with d = 1, so W[n, k] is the integer quant placed by the encoder."""
    k = n = 64
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, (n, k))
    raw = np.concatenate([enc_q8_0(0x3C00, q[r, 32 * b:32 * b + 32]) for r in range(n) for b in range(2)])
    x = np.zeros((k, k), np.uint16)
    x[np.arange(k), np.arange(k)] = 0x3C00
    y = o.prefill_gemm(Q8_0, raw, n, k, x)
    assert np.array_equal(y, q.T.astype(np.float64)), "identity X must select W^T"
    # a one-hot row scaled by 2 picks one column of W, doubled
    x1 = np.zeros((1, k), np.uint16)
    x1[0, 5] = 0x4000
    y1 = o.prefill_gemm(Q8_0, raw, n, k, x1)
    assert np.array_equal(y1[0], 2.0 * q[:, 5]), "one-hot row"


def pin_gemm_matmul(o):
    """Against numpy's float64 matmul of the (separately pinned) f32 dequant."""
    for qt, n, k, t in ((F16W, 9, 256, 3), (Q4_K, 48, 512, 5), (Q5_K, 21, 512, 6), (Q6_K, 33, 256, 3), (Q2_K, 17, 768, 4),
                        (Q8_0, 40, 96, 7)):
        raw = synth.quant_weights(qt, n, k, synth.seed_for(92, qt))
        x = synth.activations_f16(t, k, synth.seed_for(93, qt))
        w = o.dequant_f32(qt, raw, n, k).astype(np.float64)
        xf = x.view(np.float16).astype(np.float64)
        want = xf @ w.T
        got = o.prefill_gemm(qt, raw, n, k, x)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max()), f"gemm vs matmul {qt}"
        # f32 activations, and a token subset
        x32 = synth.activations_f32(t, k, synth.seed_for(94, qt))
        sub = np.array([t - 1, 0])
        got = o.prefill_gemm(qt, raw, n, k, x32, tokens=sub)
        want = x32.astype(np.float64)[sub] @ w.T
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max()), f"gemm f32 x {qt}"


def pin_qknorm_closed_forms(o):
    hd = 128
    g = np.linspace(0.5, 1.5, hd).astype(np.float32)
    # constant head c: out_j = c / sqrt(c^2 + eps) * g_j
    y = np.full((1, 2 * hd), 3.0)
    out = o.qknorm(y, hd, g, 0, 1e-6)
    want = 3.0 / math.sqrt(9.0 + 1e-6) * np.tile(g.astype(np.float64), 2)
    assert np.allclose(out[0], want, rtol=1e-14), "constant head"
    # alternating 3, -4: mean square 12.5
    y = np.tile([3.0, -4.0], hd // 2)[None, :]
    out = o.qknorm(y, hd, g, 0, 0.0)
    want = y[0] / math.sqrt(12.5) * g
    assert np.allclose(out[0], want, rtol=1e-14), "alternating head"
    # tiny values: mean square equals eps, so the scale is 1/sqrt(2 eps)
    y = np.full((1, hd), 1e-3)
    out = o.qknorm(y, hd, np.ones(hd, np.float32), 0, 1e-6)
    assert np.allclose(out[0], 1e-3 / math.sqrt(2e-6), rtol=1e-12), "epsilon inside the root"
    # per-head gains (stride = head_dim): head h uses its own vector
    gh = (np.arange(2 * hd, dtype=np.float32) / 100.0 + 0.25)
    y = np.full((1, 2 * hd), -2.0)
    out = o.qknorm(y, hd, gh, hd, 0.0)
    assert np.allclose(out[0], -gh.astype(np.float64), rtol=1e-14), "per-head gains"


def pin_qknorm_invariants(o):
    rng = np.random.default_rng(5)
    y = rng.normal(size=(4, 256)) * 50
    g1 = np.ones(128, np.float32)
    out = o.qknorm(y, 128, g1, 0, 1e-6)
    ms = (out.reshape(4, 2, 128) ** 2).mean(axis=2)
    yms = (y.reshape(4, 2, 128) ** 2).mean(axis=2)
    assert np.allclose(ms, yms / (yms + 1e-6), rtol=1e-12), "unit-gain mean square"
    out2 = o.qknorm(7.0 * y, 128, g1, 0, 0.0)
    out3 = o.qknorm(y, 128, g1, 0, 0.0)
    assert np.allclose(out2, out3, rtol=1e-12), "scale invariance"


def pin_router(o):
    lg = np.log(np.array([[1.0, 2.0, 3.0, 4.0]], np.float32)).astype(np.float32)
    ids, w = o.route_topk(lg, 2)
    assert ids.tolist() == [[3, 2]], ids
    assert np.allclose(w, [[0.4, 0.3]], rtol=1e-6), w
    ids, w = o.route_topk(lg, 2, renorm=True)
    assert np.allclose(w, [[4 / 7, 3 / 7]], rtol=1e-6), w
    # ties: the lower expert index first
    lg = np.array([[1.0, 2.0, 2.0, 0.0, 2.0]], np.float32)
    ids, _ = o.route_topk(lg, 2)
    assert ids.tolist() == [[1, 2]], ids
    # brute force against Python's sort by (-logit, index)
    rng = np.random.default_rng(9)
    lg = rng.normal(size=(50, 16)).astype(np.float32)
    lg[::7, 3] = lg[::7, 9]  # plant some ties
    ids, w = o.route_topk(lg, 4)
    for t in range(50):
        order = sorted(range(16), key=lambda j: (-float(lg[t, j]), j))[:4]
        assert ids[t].tolist() == order, (t, ids[t], order)
        p = np.exp(lg[t].astype(np.float64) - lg[t].max())
        p /= p.sum()
        assert np.allclose(w[t], p[order], rtol=1e-12)


def _identity_experts(n_exp: int, dim: int, scale_of_expert) -> np.ndarray:
    """Q8_0 experts, each scale_of_expert(e) * I_dim (d = 1, quant on the diagonal)."""
    blocks = []
    for e in range(n_exp):
        for r in range(dim):
            q = np.zeros(dim, np.int64)
            q[r] = scale_of_expert(e)
            for b in range(dim // 32):
                blocks.append(enc_q8_0(0x3C00, q[32 * b:32 * b + 32]))
    return np.concatenate(blocks)


def pin_moe_identity(o):
    """Gate = up = I, down = (e+1) I:  out = sum_s w_s (e_s + 1) * SiLU(x) x.
    With h(x) = SiLU(x) x:  h(x) + h(-x) = x^2 and h(x) - h(-x) = x^2 tanh(x/2)."""
    dim, n_exp = 32, 3
    wg = _identity_experts(n_exp, dim, lambda e: 1)
    wu = wg.copy()
    wd = _identity_experts(n_exp, dim, lambda e: e + 1)
    xs = np.linspace(-6.0, 6.0, dim)
    x = np.stack([xs, -xs]).astype(np.float16)
    xb = x.view(np.uint16)
    xv = x.astype(np.float64)[0]
    ids = np.array([[0, 2], [0, 2]], np.int32)
    wts = np.array([[0.25, 0.5], [0.25, 0.5]])
    out = o.moe(Q8_0, wg, wu, wd, n_exp, dim, dim, xb, ids, wts)
    c = 0.25 * 1 + 0.5 * 3
    assert np.allclose(out[0] + out[1], c * xv * xv, rtol=1e-12, atol=1e-12), "h(x) + h(-x)"
    assert np.allclose(out[0] - out[1], c * xv * xv * np.tanh(xv / 2), rtol=1e-12, atol=1e-12), "h(x) - h(-x)"


def pin_moe_dense(o):
    """All tokens on expert 0 with weight 1 is one dense FFN: numpy float64
    matmuls of the (pinned) dequant, SiLU(g) = g * sigmoid(g)."""
    hidden, inter, n_exp, t = 256, 256, 2, 3
    wg = synth.quant_weights(Q4_K, n_exp * inter, hidden, 501)
    wu = synth.quant_weights(Q4_K, n_exp * inter, hidden, 502)
    wd = synth.quant_weights(Q4_K, n_exp * hidden, inter, 503)
    x = synth.activations_f16(t, hidden, 504)
    ids = np.zeros((t, 1), np.int32)
    wts = np.ones((t, 1))
    out = o.moe(Q4_K, wg, wu, wd, n_exp, hidden, inter, x, ids, wts)
    G = o.dequant_f32(Q4_K, wg, n_exp * inter, hidden)[:inter].astype(np.float64)
    U = o.dequant_f32(Q4_K, wu, n_exp * inter, hidden)[:inter].astype(np.float64)
    D = o.dequant_f32(Q4_K, wd, n_exp * hidden, inter)[:hidden].astype(np.float64)
    xf = x.view(np.float16).astype(np.float64)
    g = xf @ G.T
    u = xf @ U.T
    sig = 0.5 * (1.0 + np.tanh(0.5 * g))
    want = ((g * sig) * u) @ D.T
    assert np.allclose(out, want, rtol=1e-9, atol=1e-9 * np.abs(want).max()), "dense FFN"
    # permuting tokens permutes the output
    perm = np.array([2, 0, 1])
    out_p = o.moe(Q4_K, wg, wu, wd, n_exp, hidden, inter, x[perm], ids, wts)
    assert np.array_equal(out_p, out[perm]), "token permutation"


# ---------------------------------------------------------------------------
# Prompt attention.  Caches are [token][kv head][head_dim] rows; the binary16
# cache is built with numpy's conversion, the Q8_0 cache with enc_q8_0, so
# every cache value is known exactly here.

def _f16_cache(vals: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(vals, dtype=np.float16).view(np.uint8).reshape(-1)


def _q8_cache(d_bits: int, q: np.ndarray) -> np.ndarray:
    """Q8_0 cache of rows of 32 weights: one block per row, scale d_bits."""
    q = np.asarray(q).reshape(-1, 32)
    return np.concatenate([enc_q8_0(d_bits, row) for row in q])


def pin_attention_zero_query_prefix_mean(o):
    """q = 0 gives equal weights, so query i returns the mean of value rows
    0 .. n_past + i (later rows must not count)."""
    n_past, t, n_head, hd = 3, 5, 2, 32
    kv = n_past + t
    rng = np.random.default_rng(601)
    v16 = rng.integers(-64, 64, size=(kv, 1, hd)) / 8.0
    k16 = rng.standard_normal((kv, 1, hd))
    q = np.zeros((t, n_head * hd), np.float32)
    out = o.attention(F16W, q, _f16_cache(k16), _f16_cache(v16), n_past, n_head, 1, hd)
    for i in range(t):
        want = v16[:n_past + i + 1, 0].mean(axis=0)
        for h in range(n_head):
            assert np.allclose(out[i, h * hd:(h + 1) * hd], want, rtol=0, atol=1e-12), f"prefix mean q{i} h{h}"
    # the same through a Q8_0 cache: values d * q with d = 1/4
    qv = rng.integers(-127, 128, size=(kv, 32))
    out = o.attention(Q8_0, q[:, :32], _q8_cache(h16(0.25), np.zeros((kv, 32))), _q8_cache(h16(0.25), qv),
                      n_past, 1, 1, 32)
    for i in range(t):
        want = 0.25 * qv[:n_past + i + 1].mean(axis=0)
        assert np.allclose(out[i], want, rtol=0, atol=1e-12), f"Q8_0 prefix mean q{i}"
    # and through a Q4_0 cache: values d * (q - 8) with d = 1/2
    q4 = rng.integers(0, 16, size=(kv, 32))
    kc4 = np.concatenate([enc_q4_0(h16(0.5), row) for row in rng.integers(0, 16, size=(kv, 32))])
    vc4 = np.concatenate([enc_q4_0(h16(0.5), row) for row in q4])
    out = o.attention(Q4_0, q[:, :32], kc4, vc4, n_past, 1, 1, 32)
    for i in range(t):
        want = 0.5 * (q4[:n_past + i + 1] - 8.0).mean(axis=0)
        assert np.allclose(out[i], want, rtol=0, atol=1e-12), f"Q4_0 prefix mean q{i}"


def pin_attention_gqa_constant_values(o):
    """Values constant over tokens, c_g for kv head g: every query of head h
    returns c_{h // (n_head / n_kv)} whatever the scores are."""
    n_past, t, n_head, n_kv, hd = 2, 4, 6, 3, 32
    kv = n_past + t
    rng = np.random.default_rng(602)
    c = rng.integers(-50, 50, size=(n_kv, hd)) / 4.0
    v16 = np.broadcast_to(c, (kv, n_kv, hd))
    k16 = rng.standard_normal((kv, n_kv, hd))
    q = rng.standard_normal((t, n_head * hd)).astype(np.float32)
    out = o.attention(F16W, q, _f16_cache(k16), _f16_cache(v16), n_past, n_head, n_kv, hd)
    for h in range(n_head):
        want = c[h // (n_head // n_kv)]
        assert np.allclose(out[:, h * hd:(h + 1) * hd], want[None, :], rtol=0, atol=1e-12), f"GQA head {h}"


def pin_attention_two_keys_logistic(o):
    """One query over two keys: k0 = 0 and k1 = a*u with q = u gives scores 0
    and scale*a*|u|^2, so the output is v0 + sigmoid(scale*a*|u|^2) (v1 - v0);
    a single visible key returns its value row exactly."""
    hd, a, scale = 32, 0.5, 0.375
    u = np.zeros(hd)
    u[[1, 5, 9, 30]] = [1.0, -2.0, 0.5, 1.5]
    k16 = np.stack([np.zeros(hd), a * u])[:, None, :]
    rng = np.random.default_rng(603)
    v16 = (rng.integers(-32, 32, size=(2, 1, hd)) / 4.0)
    q = u[None, :].astype(np.float32)
    out = o.attention(F16W, q, _f16_cache(k16), _f16_cache(v16), 1, 1, 1, hd, scale=scale)
    z = scale * a * float(u @ u)
    sig = 0.5 * (1.0 + math.tanh(0.5 * z))
    want = v16[0, 0] + sig * (v16[1, 0] - v16[0, 0])
    assert np.allclose(out[0], want, rtol=1e-12, atol=1e-12), "two-key logistic"
    one = o.attention(F16W, q, _f16_cache(k16), _f16_cache(v16), 0, 1, 1, hd, scale=scale)
    assert np.array_equal(one[0], v16[0, 0]), "single key"


def pin_attention_huge_negative_scores(o):
    """Every key equal and every scaled score about -1e31: the softmax is still
    uniform, so query i returns the mean of value rows 0 .. n_past + i (a
    running maximum started at a finite floor above the scores would lose
    every weight)."""
    n_past, t, hd = 2, 4, 32
    kv = n_past + t
    rng = np.random.default_rng(604)
    v16 = rng.integers(-64, 64, size=(kv, 1, hd)) / 8.0
    k16 = np.full((kv, 1, hd), -1.0)
    q = np.full((t, hd), 100.0, np.float32)
    scale = 1e31 / (100.0 * hd)
    out = o.attention(F16W, q, _f16_cache(k16), _f16_cache(v16), n_past, 1, 1, hd, scale=scale)
    for i in range(t):
        want = v16[:n_past + i + 1, 0].mean(axis=0)
        assert np.allclose(out[i], want, rtol=0, atol=1e-12), f"huge negative scores q{i}"


# Rotary step.  Values of cos and sin below are constants of the functions
# (to 16 digits), not calls of a library.
def pin_rope_identity_norms_compose(o):
    """Position 0 is the identity (bit for bit); every half-split pair keeps
    its length; turning by a then by b equals turning by a + b."""
    rng = np.random.default_rng(701)
    n_head, hd = 3, 64
    x = rng.standard_normal((5, n_head * hd + 4)).astype(np.float32)  # 4 spare columns: stride > heads
    y = o.rope(x, n_head, hd, 0, 1e6)
    assert np.array_equal(y[0], x[0]), "position 0 moved"
    assert np.array_equal(y[:, -4:], x[:, -4:]), "columns past the heads changed"
    y = o.rope(x, n_head, hd, 1000, 1e6)
    xa, ya = x[:, :n_head * hd].reshape(5, n_head, 2, hd // 2), y[:, :n_head * hd].reshape(5, n_head, 2, hd // 2)
    nx = np.hypot(xa[:, :, 0].astype(np.float64), xa[:, :, 1])
    ny = np.hypot(ya[:, :, 0].astype(np.float64), ya[:, :, 1])
    assert np.allclose(ny, nx, rtol=1e-6, atol=1e-7), "pair lengths changed"
    a = o.rope(o.rope(x[:1], n_head, hd, 37, 1e6), n_head, hd, 1200, 1e6)
    b = o.rope(x[:1], n_head, hd, 1237, 1e6)
    assert np.allclose(a, b, rtol=1e-5, atol=1e-5), "rotations do not compose"


def pin_rope_closed_form(o):
    """head_dim 4, base 10^4: pair 0 (values 0 and 2) turns by 1 rad per
    position, pair 1 (values 1 and 3) by 10^4^(-1/2) = 0.01 rad.  At position
    50 the unit vectors go to (cos 50, sin 50) and (cos 0.5, sin 0.5)."""
    cos50, sin50 = 0.9649660284921133, -0.26237485370392877
    cos05, sin05 = 0.8775825618903728, 0.479425538604203
    x = np.zeros((1, 4), np.float32)
    x[0, 0] = 1.0
    y = o.rope(x, 1, 4, 50, 1e4)[0]
    assert np.allclose(y, [cos50, 0.0, sin50, 0.0], rtol=0, atol=1e-7), f"pair 0 {y}"
    x = np.zeros((1, 4), np.float32)
    x[0, 1] = 1.0
    y = o.rope(x, 1, 4, 50, 1e4)[0]
    assert np.allclose(y, [0.0, cos05, 0.0, sin05], rtol=0, atol=1e-7), f"pair 1 {y}"
    # the second token of a chunk sits one position further
    x = np.zeros((2, 4), np.float32)
    x[:, 1] = 1.0
    y = o.rope(x, 1, 4, 49, 1e4)
    assert np.allclose(y[1], [0.0, cos05, 0.0, sin05], rtol=0, atol=1e-7), "row 1 not at pos0 + 1"


# KV cache rows: hand-worked blocks and exact round trips.
def pin_kv_q8_0_hand_rows(o):
    """amax 63.5 gives d = 0.5 and codes x * 2 rounded half away from zero;
    amax 1 gives d = 1/127 (binary16 0x2008 stored) and 0.79131 * 127 =
    100.496 -> 100 from the f32 d (the binary16 d would give 100.50 -> 101)."""
    x = np.zeros(32, np.float32)
    x[:8] = [63.5, -63.5, 1.25, -1.25, 0.75, -0.75, 0.24, 0.26]
    b = o.kv_quantize(Q8_0, x[None, :], 1, 32)
    want = np.zeros(34, np.uint8)
    want[0], want[1] = 0x00, 0x38
    want[2:10] = np.array([127, -127, 3, -3, 2, -2, 0, 1], np.int8).view(np.uint8)
    assert np.array_equal(b, want), f"Q8_0 row {b[:10]}"
    x = np.zeros(32, np.float32)
    x[:2] = [1.0, 0.79131]
    b = o.kv_quantize(Q8_0, x[None, :], 1, 32)
    assert (b[0], b[1]) == (0x08, 0x20), "d of amax 1"
    assert list(b[2:4].view(np.int8)) == [127, 100], f"codes {b[2:4].view(np.int8)}"


def pin_kv_q4_0_hand_rows(o):
    """First value of largest magnitude -8: d = 1, code = int(x + 8.5), at most
    15; first such value +8: d = -1, code = int(8.5 - x).  Values 0..15 in
    the low nibbles, 16..31 in the high nibbles."""
    x = np.zeros(32, np.float32)
    x[:9] = [-8.0, 8.0, 7.0, 7.9, 0.5, -0.5, 0.49, 3.2, -2.6]
    x[16:18] = [-3.0, 6.5]
    b = o.kv_quantize(Q4_0, x[None, :], 1, 32)
    assert (b[0], b[1]) == (0x00, 0x3C), "d = 1"
    low = [0, 15, 15, 15, 9, 8, 8, 11, 5] + [8] * 7
    high = [5, 15] + [8] * 14
    assert list(b[2:18] & 0x0F) == low, f"low nibbles {list(b[2:18] & 0x0F)}"
    assert list(b[2:18] >> 4) == high, f"high nibbles {list(b[2:18] >> 4)}"
    x = np.zeros(32, np.float32)
    x[:4] = [8.0, -8.0, 7.0, 0.25]
    b = o.kv_quantize(Q4_0, x[None, :], 1, 32)
    assert (b[0], b[1]) == (0x00, 0xBC), "d = -1"
    assert list(b[2:6] & 0x0F) == [0, 15, 1, 8], f"low nibbles {list(b[2:6] & 0x0F)}"


def pin_kv_round_trips(o):
    """Values the formats hold exactly come back exactly through the cache:
    Q8_0 multiples of 1/8 with a largest |code| of 127; Q4_0 values d (c - 8)
    whose first largest magnitude is -8 d; binary16 values through F16."""
    rng = np.random.default_rng(702)
    t, n_kv, hd = 3, 2, 64
    k = rng.integers(-127, 128, size=(t, n_kv * hd))
    k[:, ::32] = 127
    x = (k / 8.0).astype(np.float32)
    back = o.dequant_f32(Q8_0, o.kv_quantize(Q8_0, x, n_kv, hd), t * n_kv, hd).reshape(t, n_kv * hd)
    assert np.array_equal(back, x), "Q8_0 round trip"
    c = rng.integers(0, 16, size=(t, n_kv * hd))
    c[:, ::32] = 0
    x = ((c - 8) * 0.375).astype(np.float32)
    back = o.dequant_f32(Q4_0, o.kv_quantize(Q4_0, x, n_kv, hd), t * n_kv, hd).reshape(t, n_kv * hd)
    assert np.array_equal(back, x), "Q4_0 round trip"
    x = rng.standard_normal((t, n_kv * hd)).astype(np.float16).astype(np.float32)
    back = o.dequant_f32(F16W, o.kv_quantize(F16W, x, n_kv, hd), t * n_kv, hd).reshape(t, n_kv * hd)
    assert np.array_equal(back, x), "F16 round trip"
    # rows are token-major, then kv head: head 1 of token 2 is cache row 5
    rows = o.kv_quantize(Q8_0, (k / 8.0).astype(np.float32), n_kv, hd).reshape(t * n_kv, -1)
    one = o.kv_quantize(Q8_0, (k[2:3, hd:] / 8.0).astype(np.float32), 1, hd)
    assert np.array_equal(rows[5], one), "row order"


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
