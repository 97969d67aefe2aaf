"""Dequant on the GPU against the oracle, bit for bit (to_bits), with NaN
guard bands on both sides of the output to catch out-of-bounds writes."""
import numpy as np
import pytest

import oracle
import pins
import synth
import quantized_prefill_amd as qp
from gpu_helpers import GUARD, NAN16, NAN32, say, to_dev, weights
from synth import F16W, Q8_0, Q4_K, Q5_K, Q6_K, Q2_K

pytestmark = pytest.mark.gpu

QTYPES = [Q8_0, Q4_K, Q5_K, Q6_K, Q2_K]


def gpu_dequant(qtype, raw: np.ndarray, rows: int, cols: int, f16: bool, dst_off: int = 0):
    """Dequant through the C ABI into a guarded buffer; returns (values, guards_intact).
    dst_off elements before the output move it off 16-byte alignment (the
    kernels' fallback paths)."""
    import torch
    assert raw.size == rows * synth.row_bytes(qtype, cols), "weight buffer does not match rows x row_bytes"
    w = to_dev(raw)
    n = rows * cols
    g0 = GUARD + dst_off
    if f16:
        buf = torch.full((n + 2 * g0,), NAN16, dtype=torch.int16, device="cuda")
        esz = 2
    else:
        buf = torch.full((n + 2 * g0,), NAN32, dtype=torch.int32, device="cuda")
        esz = 4
    before = buf.cpu().numpy().copy()
    fn = qp.lib().qp_dequant_f16 if f16 else qp.lib().qp_dequant_f32
    qp.check(fn(qtype, w.data_ptr(), rows, cols, buf.data_ptr() + g0 * esz,
                torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    after = buf.cpu().numpy()
    intact = np.array_equal(after[:g0], before[:g0]) and np.array_equal(after[g0 + n:], before[g0 + n:])
    vals = after[g0:g0 + n]
    return (vals.view(np.uint16) if f16 else vals.view(np.uint32)).reshape(rows, cols), intact


def check_bits(orc, qtype, raw, rows, cols, what, dst_off=0):
    want32 = orc.dequant_f32(qtype, raw, rows, cols).view(np.uint32)
    got32, ok32 = gpu_dequant(qtype, raw, rows, cols, False, dst_off)
    assert ok32, f"{what}: f32 dequant wrote outside rows x cols"
    bad = np.flatnonzero(got32.reshape(-1) != want32.reshape(-1))
    assert bad.size == 0, f"{what}: f32 mismatch at {bad[:5]} got {got32.reshape(-1)[bad[:5]]} want {want32.reshape(-1)[bad[:5]]}"
    want16 = orc.dequant_f16_bits(qtype, raw, rows, cols)
    got16, ok16 = gpu_dequant(qtype, raw, rows, cols, True, dst_off)
    assert ok16, f"{what}: f16 dequant wrote outside rows x cols"
    bad = np.flatnonzero(got16.reshape(-1) != want16.reshape(-1))
    assert bad.size == 0, f"{what}: f16 mismatch at {bad[:5]}"


@pytest.mark.parametrize("qtype", QTYPES, ids=[synth.NAMES[q] for q in QTYPES])
def test_hand_blocks_and_sweeps(orc, qtype):
    """Every (scale, min, quant) combination, every scale pair of the pins
    (negative, subnormal, signed-zero and large scales), bit for bit."""
    say(f"dequant sweep {synth.NAMES[qtype]}")
    rng = np.random.default_rng(qtype)
    blocks = []
    for d_bits, dmin_bits in pins.SCALE_PAIRS:
        for _ in range(16):
            if qtype == Q8_0:
                blocks.append(pins.enc_q8_0(d_bits, rng.integers(-128, 128, 32)))
            elif qtype == Q4_K:
                blocks.append(pins.enc_q4_k(d_bits, dmin_bits, rng.integers(0, 64, 8), rng.integers(0, 64, 8),
                                            rng.integers(0, 16, 256)))
            elif qtype == Q5_K:
                blocks.append(pins.enc_q5_k(d_bits, dmin_bits, rng.integers(0, 64, 8), rng.integers(0, 64, 8),
                                            rng.integers(0, 32, 256)))
            elif qtype == Q6_K:
                blocks.append(pins.enc_q6_k(d_bits, rng.integers(-128, 128, 16), rng.integers(-32, 32, 256)))
            else:
                blocks.append(pins.enc_q2_k(d_bits, dmin_bits, rng.integers(0, 16, 16), rng.integers(0, 16, 16),
                                            rng.integers(0, 4, 256)))
    raw = np.concatenate(blocks)
    qk = synth.BLOCK[qtype][0]
    check_bits(orc, qtype, raw, len(blocks), qk, "encoded blocks")
    # the same bytes as one long row, and as rows of 4 blocks
    check_bits(orc, qtype, raw, 1, qk * len(blocks), "one row")
    check_bits(orc, qtype, raw, len(blocks) // 4, 4 * qk, "rows of 4 blocks")


@pytest.mark.parametrize("qtype", QTYPES, ids=[synth.NAMES[q] for q in QTYPES])
def test_partial_tails(orc, qtype):
    """Rows whose last block is partial, at every tail length class."""
    qk = synth.BLOCK[qtype][0]
    tails = [1, 3, 4, 5, 15, 16, 17, 31] if qtype == Q8_0 else [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128,
                                                                 129, 255]
    for tail in tails:
        for rows, nfull in ((1, 0), (3, 2), (5, 16)):
            cols = nfull * qk + tail
            raw = weights(qtype, rows, cols, 7000 + tail)
            say(f"dequant tail {synth.NAMES[qtype]} rows={rows} cols={cols}")
            check_bits(orc, qtype, raw, rows, cols, f"tail {tail} rows {rows}")


@pytest.mark.parametrize("qtype", [Q6_K, Q2_K], ids=["Q6_K", "Q2_K"])
def test_extra_partial_row_8b(orc, qtype):
    """The one-row and three-row tensors of 4096 + 77 weights (17 blocks, the
    last holding 77) next to the Qwen3-8B-shaped projections."""
    for rows in (1, 3):
        raw = weights(qtype, rows, 4096 + 77, 7100 + rows)
        check_bits(orc, qtype, raw, rows, 4096 + 77, f"4173-wide rows={rows}")


@pytest.mark.parametrize("qtype", QTYPES, ids=[synth.NAMES[q] for q in QTYPES])
def test_dense_boundaries(orc, qtype):
    """Dense tensors whose weight count ends inside a wave's or a workgroup's
    share of the flat kernel (1, 4096 / QK - 1, 4096 / QK, 4096 / QK + 1 and
    3 (4096 / QK) + 5 blocks), as one row and as one block per row; and
    outputs off 16-byte alignment (the per-unit kernel)."""
    qk = synth.BLOCK[qtype][0]
    nbg = 4096 // qk
    for nb in (1, nbg - 1, nbg, nbg + 1, 3 * nbg + 5):
        for rows in sorted({1, nb}):
            cols = nb * qk // rows
            raw = weights(qtype, rows, cols, 7500 + nb + rows)
            say(f"dequant groups {synth.NAMES[qtype]} rows={rows} cols={cols}")
            check_bits(orc, qtype, raw, rows, cols, f"{nb} blocks as {rows} rows")
    raw = weights(qtype, 3, 5 * qk, 7600)
    for dst_off in (1, 3):
        say(f"dequant output offset {synth.NAMES[qtype]} +{dst_off}")
        check_bits(orc, qtype, raw, 3, 5 * qk, f"dst +{dst_off} elements", dst_off)


def test_edge_sizes(orc):
    """Empty tensor (no-op), one weight, one block, and a single huge row."""
    import torch
    w = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = torch.full((4,), 7.0, device="cuda")
    qp.check(qp.lib().qp_dequant_f32(Q4_K, w.data_ptr(), 0, 256, out.data_ptr(), None))
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [7.0] * 4
    for qtype in QTYPES:
        check_bits(orc, qtype, weights(qtype, 1, 1, 7200 + qtype), 1, 1, "one weight")
        qk = synth.BLOCK[qtype][0]
        check_bits(orc, qtype, weights(qtype, 1, qk, 7300 + qtype), 1, qk, "one block")
        check_bits(orc, qtype, weights(qtype, 1, qk * 999 + 5, 7400 + qtype), 1, qk * 999 + 5, "long row")


def _config_tensors():
    out = []
    out.append(("q8_0_1024", Q8_0, 1024, 1024, synth.seed_for(0, 0)))
    for i, (name, n, k) in enumerate(synth.PROJ_1_7B):
        out.append((f"1.7b_{name}", Q4_K, n, k, synth.seed_for(1, i)))
    for qt in (Q6_K, Q2_K):
        for i, (name, n, k) in enumerate(synth.PROJ_8B):
            out.append((f"8b_{name}_{synth.NAMES[qt]}", qt, n, k, synth.seed_for(2, 10 * qt + i)))
    for i, (name, n, k) in enumerate(synth.PROJ_8B):
        if name in ("q", "gate"):
            out.append((f"8b_{name}_Q5_K", Q5_K, n, k, synth.seed_for(2, 10 * Q5_K + i)))
    out.append(("qknorm_wq", Q4_K, 4096, 4096, synth.seed_for(3, 1)))
    out.append(("qknorm_wk", Q6_K, 1024, 4096, synth.seed_for(3, 2)))
    return out


@pytest.mark.parametrize("name,qtype,n,k,seed", _config_tensors(), ids=[c[0] for c in _config_tensors()])
def test_workload_tensors(orc, name, qtype, n, k, seed):
    """Every projection tensor of the workloads, whole, bit for bit."""
    say(f"dequant workload tensor {name} {n}x{k}")
    raw = weights(qtype, n, k, seed)
    check_bits(orc, qtype, raw, n, k, name)
    weights.cache_clear()


def test_moe_expert_tensors(orc):
    """A sample of the 128 routed experts' gate/up/down tensors (Q4_K)."""
    hidden, inter, ne = 2048, 768, 128
    for which, (rows, cols) in (("gate", (inter, hidden)), ("down", (hidden, inter))):
        raw = synth.quant_weights(Q4_K, 8 * rows, cols, synth.seed_for(4, 77))
        say(f"dequant expert {which} 8 x {rows}x{cols}")
        check_bits(orc, Q4_K, raw, 8 * rows, cols, f"experts {which}")


def test_determinism():
    raw = weights(Q6_K, 64, 4096, 7500)
    a, _ = gpu_dequant(Q6_K, raw, 64, 4096, False)
    b, _ = gpu_dequant(Q6_K, raw, 64, 4096, False)
    assert np.array_equal(a, b)


def test_f16_weights_every_pattern(orc):
    """F16 weights: all 65,536 binary16 patterns (a 256 x 256 tensor and one
    row) widen exactly to f32 and come back unchanged as f16; NaN stays NaN
    (payloads are not part of the definition)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    raw = bits.astype("<u2").view(np.uint8)
    nan = np.isnan(bits.view(np.float16))
    want32 = orc.dequant_f32(F16W, raw, 256, 256).view(np.uint32).reshape(-1)
    for rows, cols in ((256, 256), (1, 1 << 16)):
        say(f"dequant F16 weights every pattern {rows}x{cols}")
        got32, ok32 = gpu_dequant(F16W, raw, rows, cols, False)
        got16, ok16 = gpu_dequant(F16W, raw, rows, cols, True)
        assert ok32 and ok16, "wrote outside rows x cols"
        g32, g16 = got32.reshape(-1), got16.reshape(-1)
        assert np.array_equal(g32[~nan], want32[~nan])
        assert np.all(np.isnan(g32[nan].view(np.float32)))
        assert np.array_equal(g16[~nan], bits[~nan])
        assert np.all(np.isnan(g16[nan].view(np.float16)))


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 7), (5, 1001), (33, 4096)])
def test_f16_weights_ragged(orc, rows, cols):
    """Tensors whose size is not a multiple of the 8-weight vector step."""
    raw = weights(F16W, rows, cols, 7600 + cols)
    check_bits(orc, F16W, raw, rows, cols, f"F16 {rows}x{cols}")


def test_f16_weights_8b_gate(orc):
    raw = weights(F16W, 12288, 4096, synth.seed_for(2, 10 * F16W + 4))
    check_bits(orc, F16W, raw, 12288, 4096, "F16 8B gate")
    weights.cache_clear()
