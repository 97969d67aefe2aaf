"""Prefill projection and its QK-norm epilogue on the GPU against the binary64
oracle: normwise relative error <= 1e-3 and per-token-row cosine >= 0.9999."""
import numpy as np
import pytest

import synth
import quantized_prefill_amd as qp
from gpu_helpers import assert_close, act_f16, sample_tokens, say, tile_rows, to_dev, weights
from synth import F16W, Q8_0, Q4_K, Q5_K, Q6_K, Q2_K

pytestmark = pytest.mark.gpu

QTYPES = [F16W, Q8_0, Q4_K, Q5_K, Q6_K, Q2_K]


def run_gemm(qtype, raw, n, k, x: np.ndarray):
    import torch
    assert raw.size == n * synth.row_bytes(qtype, k)
    assert x.shape[1] == k
    w = to_dev(raw)
    if x.dtype == np.uint16:
        xt = to_dev(x).view(torch.float16)
    else:
        xt = to_dev(x)
    y = qp.prefill_gemm(qtype, w, n, k, xt)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# small and ragged: T and N not multiples of the 128 x 128 tile, one token,
# one output row, several K chunks
SMALL = [(1, 1, 256), (1, 130, 512), (7, 64, 256), (129, 129, 768), (200, 300, 1024), (64, 257, 256),
         (300, 96, 512)]


@pytest.mark.parametrize("qtype", QTYPES, ids=[synth.NAMES[q] for q in QTYPES])
@pytest.mark.parametrize("t,n,k", SMALL)
def test_small_shapes(orc, qtype, t, n, k):
    say(f"gemm {synth.NAMES[qtype]} t={t} n={n} k={k}")
    raw = weights(qtype, n, k, 8000 + n + k)
    x = act_f16(t, k, 8100 + t + k)
    y = run_gemm(qtype, raw, n, k, x)
    ref = orc.prefill_gemm(qtype, raw, n, k, x)
    assert_close(y, ref, f"{synth.NAMES[qtype]} {t}x{n}x{k}")


# launches with fewer 128-token tiles than the GPU has CUs: with a workspace
# K is split into parts whose sums one pass adds in order
KSPLIT = [(Q4_K, 512, 2048, 2048), (Q6_K, 64, 1024, 4096), (Q2_K, 300, 96, 2048), (F16W, 40, 256, 1024),
          (Q5_K, 1, 128, 6144)]


@pytest.mark.parametrize("qtype,t,n,k", KSPLIT, ids=[f"{synth.NAMES[c[0]]}-{c[1]}x{c[2]}x{c[3]}" for c in KSPLIT])
def test_ksplit_against_whole(orc, qtype, t, n, k):
    import torch
    say(f"gemm ksplit {synth.NAMES[qtype]} t={t} n={n} k={k}")
    raw = weights(qtype, n, k, 8050 + n)
    x = act_f16(t, k, 8051 + t)
    w, xt = to_dev(raw), to_dev(x).view(torch.float16)
    assert qp.gemm_workspace(n, k, t, "cuda") is not None, "this shape should split"
    ys = qp.prefill_gemm(qtype, w, n, k, xt)
    ys2 = qp.prefill_gemm(qtype, w, n, k, xt)
    yw = qp.prefill_gemm(qtype, w, n, k, xt, workspace=False)
    torch.cuda.synchronize()
    ys, ys2, yw = ys.cpu().numpy(), ys2.cpu().numpy(), yw.cpu().numpy()
    tok = sample_tokens(t, 12, 8052) if t > 64 else np.arange(t)
    ref = orc.prefill_gemm(qtype, raw, n, k, x, tokens=tok)
    assert_close(ys[tok], ref, f"split {synth.NAMES[qtype]} {t}x{n}x{k}")
    assert_close(yw[tok], ref, f"whole {synth.NAMES[qtype]} {t}x{n}x{k}")
    assert np.array_equal(ys, ys2), "split results differ between two calls"


def test_f32_activations(orc):
    """f32 X (rounded to binary16 on load), the 64 x 1024 x 1024 Q8_0 projection."""
    raw = weights(Q8_0, 1024, 1024, synth.seed_for(0, 0))
    x = synth.activations_f32(64, 1024, synth.seed_for(0, 1))
    y = run_gemm(Q8_0, raw, 1024, 1024, x)
    ref = orc.prefill_gemm(Q8_0, raw, 1024, 1024, x)
    assert_close(y, ref, "q8_0 64x1024x1024 f32 x")


def test_strided_io(orc):
    """X and Y with row strides larger than K and N."""
    import torch
    t, n, k = 100, 192, 512
    raw = weights(Q4_K, n, k, 8200)
    x = act_f16(t, k, 8201)
    xpad = np.zeros((t, k + 64), np.uint16)
    xpad[:, :k] = x
    xt = to_dev(xpad).view(torch.float16)[:, :k]
    ybig = torch.full((t, n + 32), float("nan"), device="cuda")
    yv = ybig[:, :n]
    qp.check(qp.lib().qp_prefill_gemm(Q4_K, to_dev(raw).data_ptr(), n, k, xt.data_ptr(), qp.F16, t, k + 64,
                                      yv.data_ptr(), n + 32, None))
    torch.cuda.synchronize()
    yb = ybig.cpu().numpy()
    assert np.all(np.isnan(yb[:, n:])), "wrote outside the n output columns"
    assert_close(yb[:, :n], orc.prefill_gemm(Q4_K, raw, n, k, x), "strided")


def test_identity_and_determinism(orc):
    """X = I selects W^T; two runs give identical bits."""
    k = n = 256
    raw = weights(Q6_K, n, k, 8300)
    x = np.zeros((k, k), np.uint16)
    x[np.arange(k), np.arange(k)] = 0x3C00
    y = run_gemm(Q6_K, raw, n, k, x)
    w16 = orc.dequant_f16_bits(Q6_K, raw, n, k).view(np.float16).astype(np.float32)
    assert np.array_equal(y, w16.T), "identity X must return the binary16 weights exactly"
    y2 = run_gemm(Q6_K, raw, n, k, x)
    assert np.array_equal(y, y2)


def _projection_cases():
    cases = []
    for i, (name, n, k) in enumerate(synth.PROJ_1_7B):
        cases.append((f"1.7b_{name}_Q4_K", Q4_K, n, k, 512, synth.seed_for(1, i), synth.seed_for(1, 500 + k // 256)))
    for qt in (Q6_K, Q2_K):
        for i, (name, n, k) in enumerate(synth.PROJ_8B):
            cases.append((f"8b_{name}_{synth.NAMES[qt]}", qt, n, k, 2048, synth.seed_for(2, 10 * qt + i),
                          synth.seed_for(2, 500 + k // 256)))
    # Q5_K and F16 weights at two of the 8B shapes
    for qt in (Q5_K, F16W):
        for i, (name, n, k) in enumerate(synth.PROJ_8B):
            if name in ("gate", "down"):
                cases.append((f"8b_{name}_{synth.NAMES[qt]}", qt, n, k, 2048, synth.seed_for(2, 10 * qt + i),
                              synth.seed_for(2, 500 + k // 256)))
    return cases


@pytest.mark.parametrize("name,qtype,n,k,t,wseed,xseed", _projection_cases(), ids=[c[0] for c in _projection_cases()])
def test_workload_projections(orc, name, qtype, n, k, t, wseed, xseed):
    """Full-size projections in the launch configuration the bench times;
    the oracle computes a spread of token rows."""
    say(f"gemm workload {name} t={t} n={n} k={k}")
    raw = weights(qtype, n, k, wseed)
    x = act_f16(t, k, xseed)
    y = run_gemm(qtype, raw, n, k, x)
    tok = tile_rows(t, 256, 8, 9000 + n)  # first and last row of every 256-token tile, and others
    ref = orc.prefill_gemm(qtype, raw, n, k, x, tokens=tok)
    assert_close(y[tok], ref, name)
    weights.cache_clear()


def run_qknorm(qtype, raw, n, k, x, hd, gain, gstride, eps):
    import torch
    w = to_dev(raw)
    xt = to_dev(x).view(torch.float16)
    y = qp.prefill_gemm_qknorm(qtype, w, n, k, xt, hd, to_dev(gain), gstride, eps)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("qtype", QTYPES, ids=[synth.NAMES[q] for q in QTYPES])
def test_qknorm_small(orc, qtype, hd):
    t, n, k = 77, (512 if hd == 256 else 384), 512
    raw = weights(qtype, n, k, 8400 + hd)
    x = act_f16(t, k, 8401)
    for gstride, gn in ((0, hd), (hd, n)):
        gain = synth.gains(gn, 8402 + gstride)
        y = run_qknorm(qtype, raw, n, k, x, hd, gain, gstride, 1e-6)
        ref = orc.prefill_gemm_qknorm(qtype, raw, n, k, x, hd, gain, gstride, 1e-6)
        assert_close(y, ref, f"qknorm {synth.NAMES[qtype]} hd={hd} stride={gstride}")


def test_qknorm_workload(orc):
    """Qwen3-8B attention shapes at T = 8192: Q (Q4_K 4096 -> 32 heads) and
    K (Q6_K 4096 -> 8 heads), per-head RMSNorm with eps 1e-6."""
    t, hidden, hd = 8192, 4096, 128
    x = act_f16(t, hidden, synth.seed_for(3, 0))
    tok = tile_rows(t, 256, 8, 9100)
    for name, qtype, n, wseed, gseed in (("q", Q4_K, 4096, synth.seed_for(3, 1), synth.seed_for(3, 3)),
                                         ("k", Q6_K, 1024, synth.seed_for(3, 2), synth.seed_for(3, 4))):
        say(f"qknorm workload {name} n={n}")
        raw = weights(qtype, n, hidden, wseed)
        gain = synth.gains(hd, gseed)
        y = run_qknorm(qtype, raw, n, hidden, x, hd, gain, 0, 1e-6)
        ref = orc.prefill_gemm_qknorm(qtype, raw, n, hidden, x, hd, gain, 0, 1e-6, tokens=tok)
        assert_close(y[tok], ref, f"qknorm {name}")
        # every head of every token is unit-RMS up to the gains (property at full size)
        hn = (y / np.tile(gain, n // hd)).reshape(t, n // hd, hd)
        ms = (hn.astype(np.float64) ** 2).mean(axis=2)
        assert np.allclose(ms, 1.0, atol=2e-3), f"head mean squares off: {ms.min()} {ms.max()}"


# Shapes that take the 256-token tile (at least 512 tokens and at least 256
# output tiles) with T and N not multiples of the tile, in padded strides.
# (the last case's output stride is not a multiple of 4 floats: the tall tile
# stores 16-byte rows, so that shape goes to the 128 x 128 kernel)
TALL = [(777, 8269, 512, 0), (513, 11009, 256, 0), (640, 8192, 256, 1)]


@pytest.mark.parametrize("qtype", QTYPES, ids=[synth.NAMES[q] for q in QTYPES])
@pytest.mark.parametrize("t,n,k,odd", TALL)
def test_tall_tile_ragged(orc, qtype, t, n, k, odd):
    import torch
    say(f"gemm tall {synth.NAMES[qtype]} t={t} n={n} k={k} odd ldy={odd}")
    raw = weights(qtype, n, k, 8500 + t)
    x = act_f16(t, k, 8501 + t)
    ldx, ldy = k + 64, ((n + 7) // 4 * 4 + 4) + odd
    xpad = np.zeros((t, ldx), np.uint16)
    xpad[:, :k] = x
    xt = to_dev(xpad).view(torch.float16)
    ybig = torch.full((t, ldy), float("nan"), device="cuda")
    qp.check(qp.lib().qp_prefill_gemm(qtype, to_dev(raw).data_ptr(), n, k, xt.data_ptr(), qp.F16, t, ldx,
                                      ybig.data_ptr(), ldy, None))
    torch.cuda.synchronize()
    yb = ybig.cpu().numpy()
    assert np.all(np.isnan(yb[:, n:])), "wrote outside the n output columns"
    assert_close(yb[:, :n], orc.prefill_gemm(qtype, raw, n, k, x), f"tall {synth.NAMES[qtype]} {t}x{n}x{k}")


@pytest.mark.parametrize("hd,n", [(128, 8192), (64, 8256)])
@pytest.mark.parametrize("qtype", [Q4_K, Q6_K], ids=["Q4_K", "Q6_K"])
def test_qknorm_tall_tile_ragged(orc, qtype, hd, n):
    """QK-norm epilogue on the 256-token tile: ragged T; for head_dim 64 the
    last column tile holds a single head."""
    t, k = 777, 512
    say(f"qknorm tall {synth.NAMES[qtype]} t={t} n={n} hd={hd}")
    raw = weights(qtype, n, k, 8600 + hd)
    x = act_f16(t, k, 8601)
    for gstride, gn in ((0, hd), (hd, n)):
        gain = synth.gains(gn, 8602 + gstride)
        y = run_qknorm(qtype, raw, n, k, x, hd, gain, gstride, 1e-6)
        ref = orc.prefill_gemm_qknorm(qtype, raw, n, k, x, hd, gain, gstride, 1e-6)
        assert_close(y, ref, f"qknorm tall {synth.NAMES[qtype]} hd={hd} stride={gstride}")


def run_qkv(qtype, ws, ns, k, x, hd, gains, gstrides, eps=1e-6, workspace=None):
    import torch
    xt = to_dev(x).view(torch.float16)
    wv = to_dev(ws[2]) if ns[2] else None
    yq, yk, yv = qp.prefill_gemm_qkv(qtype, to_dev(ws[0]), ns[0], to_dev(ws[1]), ns[1], wv, ns[2], k, xt, hd,
                                     to_dev(gains[0]), to_dev(gains[1]), gstrides[0], gstrides[1], eps,
                                     workspace=workspace)
    torch.cuda.synchronize()
    return yq.cpu().numpy(), yk.cpu().numpy(), (yv.cpu().numpy() if ns[2] else None)


def check_qkv(orc, qtype, ws, ns, k, x, hd, gains, gstrides, tok, what, workspace=None):
    yq, yk, yv = run_qkv(qtype, ws, ns, k, x, hd, gains, gstrides, workspace=workspace)
    xs = x if tok is None else x[tok]
    sel = (lambda a: a) if tok is None else (lambda a: a[tok])
    for name, y, i in (("q", yq, 0), ("k", yk, 1)):
        ref = orc.prefill_gemm_qknorm(qtype, ws[i], ns[i], k, x, hd, gains[i], gstrides[i], 1e-6, tokens=tok)
        assert_close(sel(y), ref, f"{what} {name}")
    if ns[2]:
        assert_close(sel(yv), orc.prefill_gemm(qtype, ws[2], ns[2], k, x, tokens=tok), f"{what} v")
    return yq, yk, yv


@pytest.mark.parametrize("qtype", [Q6_K, Q2_K], ids=["Q6_K", "Q2_K"])
def test_qkv_workload(orc, qtype):
    """Qwen3-8B attention inputs at T = 2048 in one call (one fused launch:
    384 tall tiles); q also matches the separate QK-norm call bit for bit."""
    t, k, hd = 2048, 4096, 128
    x = act_f16(t, k, synth.seed_for(2, 500 + k // 256))
    names = [p for p in synth.PROJ_8B if p[0] in ("q", "k", "v")]
    ws = [weights(qtype, n, k, synth.seed_for(2, 10 * qtype + synth.PROJ_8B.index(p))) for p in names for n in [p[1]]]
    ns = [p[1] for p in names]
    gains = [synth.gains(hd, synth.seed_for(2, 600 + j)) for j in range(2)]
    say(f"qkv workload {synth.NAMES[qtype]} t={t} n={ns}")
    tok = tile_rows(t, 256, 8, 9200)
    yq, _, _ = check_qkv(orc, qtype, ws, ns, k, x, hd, gains, [0, 0], tok, f"qkv {synth.NAMES[qtype]}")
    y_sep = run_qknorm(qtype, ws[0], ns[0], k, x, hd, gains[0], 0, 1e-6)
    assert np.array_equal(yq, y_sep), "fused q differs from the separate QK-norm launch"
    weights.cache_clear()


@pytest.mark.parametrize("qtype", QTYPES, ids=[synth.NAMES[q] for q in QTYPES])
def test_qkv_ragged(orc, qtype):
    """Fused launch with T off the tile (777), per-head gains, strided gains
    for k; then head_dim 64 with a half-filled last q tile and no v."""
    t, k = 777, 512
    x = act_f16(t, k, 8701)
    ns = [4096, 2048, 2048]
    ws = [weights(qtype, n, k, 8710 + i) for i, n in enumerate(ns)]
    gains = [synth.gains(ns[0], 8720), synth.gains(128, 8721)]
    say(f"qkv ragged {synth.NAMES[qtype]} hd=128")
    check_qkv(orc, qtype, ws, ns, k, x, 128, gains, [128, 0], None, f"qkv ragged {synth.NAMES[qtype]}")
    ns = [6208, 2048, 0]
    ws = [weights(qtype, ns[0], k, 8730), ws[1], None]
    gains = [synth.gains(64, 8731), synth.gains(64, 8732)]
    say(f"qkv ragged {synth.NAMES[qtype]} hd=64 no v")
    check_qkv(orc, qtype, ws, ns, k, x, 64, gains, [0, 0], None, f"qkv ragged hd64 {synth.NAMES[qtype]}")
    # 256 q tiles + 64 k + 64 v tiles (one and a half rounds of the GPU) with
    # per-head k gains: with the workspace k and v run as K halves plus a
    # combine pass, without it as whole tiles; both against the oracle, the
    # split one twice for identical bits, q identical in both
    ns = [8192, 2048, 2048]
    ws = [weights(qtype, ns[0], k, 8740), ws[1], weights(qtype, ns[2], k, 8741)]
    gains = [synth.gains(128, 8742), synth.gains(ns[1], 8743)]
    say(f"qkv ragged {synth.NAMES[qtype]} 384 tiles, K halves")
    a = check_qkv(orc, qtype, ws, ns, k, x, 128, gains, [0, 128], None, f"qkv split {synth.NAMES[qtype]}")
    b = run_qkv(qtype, ws, ns, k, x, 128, gains, [0, 128])
    for u, v in zip(a, b):
        assert np.array_equal(u, v), "q/k/v results differ between two calls"
    say(f"qkv ragged {synth.NAMES[qtype]} 384 tiles, whole")
    c = check_qkv(orc, qtype, ws, ns, k, x, 128, gains, [0, 128], None, f"qkv whole {synth.NAMES[qtype]}",
                  workspace=False)
    assert np.array_equal(a[0], c[0]), "q differs between the split and the whole launch"


@pytest.mark.parametrize("qtype", [Q4_K, Q6_K], ids=["Q4_K", "Q6_K"])
def test_qknorm_head_dim_256(orc, qtype):
    """Heads of 256 columns (the projection, then the norm over each stored
    head): a ragged T on the 256-token tiles with per-head gains, every row
    against the oracle and every head unit-RMS up to its gains; then q/k/v in
    one call with head_dim 256 (three separate launches)."""
    t, n, k, hd = 777, 8192, 512, 256
    raw = weights(qtype, n, k, 8900)
    x = act_f16(t, k, 8901)
    gain = synth.gains(n, 8902)
    say(f"qknorm hd=256 {synth.NAMES[qtype]} t={t} n={n}")
    y = run_qknorm(qtype, raw, n, k, x, hd, gain, hd, 1e-6)
    ref = orc.prefill_gemm_qknorm(qtype, raw, n, k, x, hd, gain, hd, 1e-6)
    assert_close(y, ref, f"qknorm hd=256 {synth.NAMES[qtype]}")
    hn = (y / gain[None, :]).reshape(t, n // hd, hd)
    ms = (hn.astype(np.float64) ** 2).mean(axis=2)
    assert np.allclose(ms, 1.0, atol=2e-3), f"head mean squares off: {ms.min()} {ms.max()}"
    ns = [2048, 512, 512]
    ws = [weights(qtype, nn, k, 8910 + i) for i, nn in enumerate(ns)]
    gains = [synth.gains(hd, 8920), synth.gains(ns[1], 8921)]
    say(f"qkv hd=256 {synth.NAMES[qtype]}")
    check_qkv(orc, qtype, ws, ns, k, x, hd, gains, [0, hd], None, f"qkv hd=256 {synth.NAMES[qtype]}")


def test_qkv_small_falls_back(orc):
    """Too few tiles for one fused launch: the three separate launches."""
    t, k = 50, 256
    x = act_f16(t, k, 8801)
    ns = [256, 128, 128]
    ws = [weights(Q4_K, n, k, 8810 + i) for i, n in enumerate(ns)]
    gains = [synth.gains(128, 8820), synth.gains(128, 8821)]
    check_qkv(orc, Q4_K, ws, ns, k, x, 128, gains, [0, 0], None, "qkv small")


@pytest.mark.parametrize("qtype", QTYPES, ids=[synth.NAMES[q] for q in QTYPES])
def test_tall_tile_weights_exact(orc, qtype):
    """One-hot rows (token t selects input column t % K) on the 256-token
    tile: every output is one binary16 weight times 1, so the tall kernel's
    in-LDS decode must equal the oracle's f16 dequant bit for bit."""
    t, n, k = 512, 16384, 512
    raw = weights(qtype, n, k, 8900)
    x = np.zeros((t, k), np.uint16)
    x[np.arange(t), np.arange(t) % k] = 0x3C00
    y = run_gemm(qtype, raw, n, k, x)
    w16 = orc.dequant_f16_bits(qtype, raw, n, k).view(np.float16).astype(np.float32)
    want = w16[:, np.arange(t) % k].T
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:3].tolist()}"
