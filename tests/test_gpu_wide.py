"""The feed-forward input projections in one call (qp_prefill_gemm_gate_up)
and the 256 x 256-tile kernel with weights decoded in registers, which that
call and large plain projections run on, against the binary64 oracle
(normwise relative error <= 1e-3, per-token-row cosine >= 0.9999), plus a
bit-exact check of the in-register decode."""
import numpy as np
import pytest

import synth
import quantized_prefill_amd as qp
from gpu_helpers import assert_close, act_f16, say, tile_rows, to_dev, weights
from synth import Q4_K, Q5_K, Q6_K, Q2_K, F16W, Q8_0

pytestmark = pytest.mark.gpu

WIDE_TYPES = [Q4_K, Q5_K, Q6_K, Q2_K]


def run_gate_up(qtype, wg, wu, n, k, x):
    import torch
    xt = to_dev(x).view(torch.float16)
    yg, yu = qp.prefill_gemm_gate_up(qtype, to_dev(wg), to_dev(wu), n, k, xt)
    torch.cuda.synchronize()
    return yg.cpu().numpy(), yu.cpu().numpy()


@pytest.mark.parametrize("qtype", [Q6_K, Q2_K], ids=["Q6_K", "Q2_K"])
def test_gate_up_workload(orc, qtype):
    """Qwen3-8B gate and up at T = 2048 (one launch of 768 tiles of 256 x 256):
    the first and last token row of every 256-token tile and others, and two
    calls give the same bits."""
    t, n, k = 2048, 12288, 4096
    say(f"gate_up workload {synth.NAMES[qtype]}")
    wg = synth.quant_weights(qtype, n, k, synth.seed_for(2, 10 * qtype + 4))
    wu = synth.quant_weights(qtype, n, k, synth.seed_for(2, 10 * qtype + 5))
    x = act_f16(t, k, synth.seed_for(2, 500 + k // 256))
    yg, yu = run_gate_up(qtype, wg, wu, n, k, x)
    yg2, yu2 = run_gate_up(qtype, wg, wu, n, k, x)
    assert np.array_equal(yg, yg2) and np.array_equal(yu, yu2), "two calls differ"
    tok = tile_rows(t, 256, 24, 9600)
    assert_close(yg[tok], orc.prefill_gemm(qtype, wg, n, k, x, tokens=tok), f"gate {synth.NAMES[qtype]}")
    assert_close(yu[tok], orc.prefill_gemm(qtype, wu, n, k, x, tokens=tok), f"up {synth.NAMES[qtype]}")


@pytest.mark.parametrize("qtype", WIDE_TYPES, ids=[synth.NAMES[q] for q in WIDE_TYPES])
def test_gate_up_ragged(orc, qtype):
    """T off the token tile (1000) and n off the column tile (16384 + 100: the
    last column tile is partial), every output row against the oracle."""
    t, n, k = 1000, 16484, 512
    say(f"gate_up ragged {synth.NAMES[qtype]}")
    wg = weights(qtype, n, k, 9700 + qtype)
    wu = weights(qtype, n, k, 9710 + qtype)
    x = act_f16(t, k, 9701)
    yg, yu = run_gate_up(qtype, wg, wu, n, k, x)
    assert_close(yg, orc.prefill_gemm(qtype, wg, n, k, x), f"gate ragged {synth.NAMES[qtype]}")
    assert_close(yu, orc.prefill_gemm(qtype, wu, n, k, x), f"up ragged {synth.NAMES[qtype]}")
    weights.cache_clear()


@pytest.mark.parametrize("qtype", [F16W, Q8_0, Q6_K], ids=["F16", "Q8_0", "Q6_K-small"])
def test_gate_up_two_calls(orc, qtype):
    """Types the wide kernel does not take, and a launch too small to fill
    the GPU: the two projections run as separate calls."""
    t, n, k = 300, 1024, 512
    wg = weights(qtype, n, k, 9800 + qtype)
    wu = weights(qtype, n, k, 9810 + qtype)
    x = act_f16(t, k, 9801)
    yg, yu = run_gate_up(qtype, wg, wu, n, k, x)
    assert_close(yg, orc.prefill_gemm(qtype, wg, n, k, x), "gate two calls")
    assert_close(yu, orc.prefill_gemm(qtype, wu, n, k, x), "up two calls")


@pytest.mark.parametrize("qtype", WIDE_TYPES, ids=[synth.NAMES[q] for q in WIDE_TYPES])
def test_wide_weights_exact(orc, qtype):
    """One-hot rows (token t selects input column t % K) through the wide
    kernel: every output is one binary16 weight times 1, so the in-register
    decode must equal the oracle's f16 dequant bit for bit."""
    t, n, k = 512, 16384, 512
    wg = weights(qtype, n, k, 9900 + qtype)
    wu = weights(qtype, n, k, 9910 + qtype)
    x = np.zeros((t, k), np.uint16)
    x[np.arange(t), np.arange(t) % k] = 0x3C00
    yg, yu = run_gate_up(qtype, wg, wu, n, k, x)
    for name, raw, y in (("gate", wg, yg), ("up", wu, yu)):
        w16 = orc.dequant_f16_bits(qtype, raw, n, k).view(np.float16).astype(np.float32)
        want = w16[:, np.arange(t) % k].T
        bad = np.argwhere(y != want)
        assert bad.size == 0, f"{name}: {len(bad)} outputs differ, first at {bad[:3].tolist()}"
    weights.cache_clear()


@pytest.mark.parametrize("qtype,t", [(Q6_K, 4096), (Q4_K, 4096), (Q5_K, 4024), (Q2_K, 3950)],
                         ids=["Q6_K", "Q4_K", "Q5_K-last-tile-184-rows", "Q2_K-last-tile-110-rows"])
def test_plain_wide_dispatch(orc, qtype, t):
    """A plain projection large enough for whole rounds of 256 x 256 tiles
    (T = 4096, n = 8192: 512 tiles), with an odd number of blocks per row
    (k = 1280: rows start 2 bytes into a dword for Q6_K on odd rows); with a
    ragged last token tile, that tile runs over 6 M blocks (129-192 rows)
    or 4 (at most 128)."""
    import torch
    n, k = 8192, 1280
    raw = weights(qtype, n, k, 9950 + qtype)
    x = act_f16(t, k, 9951)
    y = qp.prefill_gemm(qtype, to_dev(raw), n, k, to_dev(x).view(torch.float16))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    tok = tile_rows(t, 256, 16, 9952)
    assert_close(y[tok], orc.prefill_gemm(qtype, raw, n, k, x, tokens=tok), f"plain wide {synth.NAMES[qtype]}")
    weights.cache_clear()


@pytest.mark.parametrize("t,n,k", [(2048, 4096, 12288), (2000, 4000, 8192), (2048, 4096, 4096), (2000, 4000, 4096)],
                         ids=["down-halves", "ragged-halves", "o-128-token-tiles", "ragged-128-token-tiles"])
def test_wide_half_round_q2_k(orc, t, n, k):
    """Q2_K launches of half a round of 256 x 256 tiles: with K >= 8192 and a
    workspace, two K halves in one launch plus an in-order add; otherwise the
    wide kernel with 128-token tiles.  Against the oracle on every 256-token
    tile's first and last row, against the call without workspace within the
    tolerance, the same bits on two calls, and the allocation-free call bit
    for bit equal to the workspace call."""
    import torch
    qtype = Q2_K
    say(f"Q2_K half round t={t} n={n} k={k}")
    raw = weights(qtype, n, k, 9700 + k // 256)
    x = act_f16(t, k, 9701)
    w, xt = to_dev(raw), to_dev(x).view(torch.float16)
    if k >= 8192:
        assert qp.lib().qp_prefill_gemm_workspace_bytes(n, k, t) >= 4 * t * n
    a = qp.prefill_gemm(qtype, w, n, k, xt).cpu().numpy()
    b = qp.prefill_gemm(qtype, w, n, k, xt).cpu().numpy()
    assert np.array_equal(a, b), "two calls differ"
    tok = tile_rows(t, 256, 8, 9702)
    assert_close(a[tok], orc.prefill_gemm(qtype, raw, n, k, x, tokens=tok), f"Q2_K half round k={k}")
    whole = qp.prefill_gemm(qtype, w, n, k, xt, workspace=False).cpu().numpy()
    assert_close(a, whole.astype(np.float64), "against the call without workspace")
    out = torch.empty((t, n), dtype=torch.float32, device="cuda")
    qp.prefill_gemm_noalloc(qtype, w, n, k, xt, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), a), "allocation-free call differs from the workspace call"


KSLICE = [(200, 1000, 2048), (500, 4000, 1024), (500, 6000, 1024)]


@pytest.mark.parametrize("qtype", [Q4_K, Q5_K, Q6_K, Q2_K], ids=["Q4_K", "Q5_K", "Q6_K", "Q2_K"])
@pytest.mark.parametrize("t,n,k", KSLICE, ids=["64x64-4-slices", "64x128-2-slices", "128x128-2-slices"])
def test_wide_k_slices(orc, qtype, t, n, k):
    """Short chunks on the wide kernel in K slices (on a 256-CU GPU the three
    shapes take the 64 x 64 tiling with four slices, 64 x 128 and 128 x 128
    with two): ragged token and feature tails, against the oracle on the
    first and last row of every 64-token tile; two calls give the same bits,
    and the allocation-free call matches them."""
    import torch
    say(f"K slices {synth.NAMES[qtype]} t={t} n={n} k={k}")
    raw = weights(qtype, n, k, 9800 + n)
    x = act_f16(t, k, 9801 + t)
    w, xt = to_dev(raw), to_dev(x).view(torch.float16)
    a = qp.prefill_gemm(qtype, w, n, k, xt).cpu().numpy()
    b = qp.prefill_gemm(qtype, w, n, k, xt).cpu().numpy()
    assert np.array_equal(a, b), "two calls differ"
    tok = tile_rows(t, 64, 6, 9802)
    assert_close(a[tok], orc.prefill_gemm(qtype, raw, n, k, x, tokens=tok), f"K slices {synth.NAMES[qtype]} {t}x{n}x{k}")
    out = torch.empty((t, n), dtype=torch.float32, device="cuda")
    qp.prefill_gemm_noalloc(qtype, w, n, k, xt, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), a), "allocation-free call differs"
    weights.cache_clear()
