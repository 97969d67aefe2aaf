"""The rotary step and the KV cache writes on the GPU against the oracle, and
the chain from the attention-input projections to the prompt attention over
binary16, Q8_0 and Q4_0 caches."""
import numpy as np
import pytest

import synth
import quantized_prefill_amd as qp
from gpu_helpers import assert_close, min_row_cos, normwise, say, to_dev
from synth import F16W, Q4_0, Q8_0, Q4_K, Q6_K

pytestmark = pytest.mark.gpu

KV_TYPES = [F16W, Q8_0, Q4_0]

# The whole chain from X against the oracle's chain.  The projections agree
# to the GEMM tolerance e = 1e-3 (normwise), but a cache code is a rounding
# decision: an input moved by delta flips a code of step s with probability
# about delta / s, and a flip moves the value by s, so the cached K and V
# differ by about sqrt(e * s) in normwise terms, with s the code step over the
# values' RMS: binary16 2^-11, Q8_0 about 3.5 / 127 (amax over 127, amax about
# 3.5 RMS over 32 normal draws), Q4_0 about 3.5 / 8.  The bound is that
# estimate, and never below the GEMM tolerance.
CHAIN_TOL = {F16W: 1e-3, Q8_0: (1e-3 * 3.5 / 127) ** 0.5, Q4_0: (1e-3 * 3.5 / 8) ** 0.5}


def gpu_rope(x, n_head, hd, pos0, base):
    import torch
    xd = to_dev(x)
    qp.rope(xd, n_head, hd, pos0, base)
    torch.cuda.synchronize()
    return xd.cpu().numpy()


def rope_close(y: np.ndarray, ref: np.ndarray, x: np.ndarray, n_head: int, hd: int, pos_max: int, what: str):
    """Both sides compute angle, cosine and sine in binary64 and round once to
    f32, but two math libraries may differ in the last bits of those binary64
    values: an angle error of a few units in 2^-52 of the angle moves a pair
    of length r by that much times r.  Allowed per value: one f32 ulp of the
    result plus 2^-48 * pos_max * r (the pair's length r from x)."""
    t = x.shape[0]
    xh = x[:, :n_head * hd].astype(np.float64).reshape(t, n_head, 2, hd // 2)
    r = np.hypot(xh[:, :, 0], xh[:, :, 1])
    r = np.repeat(r[:, :, None, :], 2, axis=2).reshape(t, n_head * hd)
    yh, rh = y[:, :n_head * hd].astype(np.float64), ref[:, :n_head * hd].astype(np.float64)
    allowed = np.spacing(np.abs(rh).astype(np.float32)).astype(np.float64) + 2.0 ** -48 * max(pos_max, 1) * r
    err = np.abs(yh - rh)
    worst = np.unravel_index(np.argmax(err - allowed), err.shape)
    assert np.all(err <= allowed), f"{what}: error {err[worst]:.3e} above {allowed[worst]:.3e} at {worst}"


@pytest.mark.parametrize("pos0", [0, 1000, 1 << 20])
def test_rope_against_oracle(orc, pos0):
    """Qwen3-8B q heads (32 x 128) at T = 300 in rows wider than the heads:
    every value within the bound of rope_close of the oracle, columns past
    the heads untouched, position 0 unchanged bit for bit."""
    t, n_head, hd = 300, 32, 128
    x = synth.activations_f32(t, n_head * hd + 8, 9950 + pos0 % 97)
    say(f"rope pos0={pos0}")
    y = gpu_rope(x, n_head, hd, pos0, 1e6)
    ref = orc.rope(x, n_head, hd, pos0, 1e6)
    assert np.array_equal(y[:, -8:], x[:, -8:]), "columns past the heads changed"
    rope_close(y, ref, x, n_head, hd, pos0 + t, f"rope pos0={pos0}")
    if pos0 == 0:
        assert np.array_equal(y[0], x[0]), "position 0 moved"


def special_rows(hd: int, n_kv: int, rng) -> np.ndarray:
    """Rows whose blocks hit the quantizers' edge cases: all zeros (d = 0),
    a first largest magnitude negative then positive, exact ties of
    magnitude, values on the rounding boundaries of the codes."""
    rows = []
    z = np.zeros(n_kv * hd, np.float32)
    rows.append(z)
    a = rng.standard_normal(n_kv * hd).astype(np.float32)
    a[0::32] = -7.0
    a[1::32] = 7.0
    rows.append(a)
    b = rng.standard_normal(n_kv * hd).astype(np.float32)
    b[0::32] = 7.0
    b[5::32] = -7.0
    rows.append(b)
    c = (rng.integers(-254, 255, n_kv * hd) / 2.0).astype(np.float32)  # halves: Q8_0 ties at d = 1
    c[0::32] = 127.0
    rows.append(c)
    return np.stack(rows)


@pytest.mark.parametrize("kvtype", KV_TYPES, ids=[synth.NAMES[k] for k in KV_TYPES])
def test_kv_write_bit_exact(orc, kvtype):
    """The chunk's rows land at cache rows row0 * n_kv ...: bytes equal the
    oracle's writer on the same f32 rows (the codes are decided in binary32
    on both sides), rows before and after stay as they were."""
    import torch
    t, n_kv, hd, row0, after = 200, 8, 128, 37, 5
    rng = np.random.default_rng(9960 + kvtype)
    src = np.concatenate([special_rows(hd, n_kv, rng), synth.activations_f32(t - 4, n_kv * hd, 9961)])
    src[4:] *= rng.uniform(0.01, 20.0, size=(t - 4, 1)).astype(np.float32)
    rb = qp.row_bytes(kvtype, hd)
    cache = torch.full(((row0 + t + after) * n_kv * rb,), 0xA5, dtype=torch.uint8, device="cuda")
    say(f"kv write {synth.NAMES[kvtype]} t={t} row0={row0}")
    qp.kv_cache_write(kvtype, to_dev(src), n_kv, hd, cache, row0)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    want = orc.kv_quantize(kvtype, src, n_kv, hd)
    lo, hi = row0 * n_kv * rb, (row0 + t) * n_kv * rb
    assert np.all(got[:lo] == 0xA5) and np.all(got[hi:] == 0xA5), "bytes outside the chunk's rows written"
    bad = np.flatnonzero(got[lo:hi] != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at row {bad[0] // rb} byte {bad[0] % rb}"


def test_kv_write_strided_source(orc):
    """Source rows wider than the kv heads (the k columns of a fused q/k/v
    output), binary16 cache, one token."""
    import torch
    n_kv, hd = 4, 64
    src = synth.activations_f32(3, n_kv * hd + 64, 9970)
    cache = torch.zeros(3 * n_kv * hd * 2, dtype=torch.uint8, device="cuda")
    qp.kv_cache_write(F16W, to_dev(src), n_kv, hd, cache, 0)
    torch.cuda.synchronize()
    assert np.array_equal(cache.cpu().numpy(), orc.kv_quantize(F16W, src[:, :n_kv * hd], n_kv, hd))


@pytest.mark.parametrize("kvtype", KV_TYPES, ids=[synth.NAMES[k] for k in KV_TYPES])
def test_attention_chain(orc, kvtype):
    """Qwen3-8B attention at T = 512 after n_past = 256 cached tokens: q, k and
    v from one q/k/v call (Q6_K, per-head RMSNorm), the rotary step on q and k
    at positions 256 .., k and v written into the cache, then the prompt
    attention.  Each step is checked against the oracle on the GPU's own
    input (rope within the bound of rope_close, cache bytes exact, attention
    within the GEMM tolerance); the whole chain from X against the oracle's
    chain within CHAIN_TOL."""
    import torch
    t, n_past, hidden, n_head, n_kv, hd = 512, 256, 4096, 32, 8, 128
    rng_seed = 9980 + kvtype
    x = synth.activations_f16(t, hidden, rng_seed)
    ws = [synth.quant_weights(Q6_K, n, hidden, rng_seed + 1 + i) for i, n in enumerate((n_head * hd, n_kv * hd,
                                                                                         n_kv * hd))]
    gq, gk = synth.gains(hd, rng_seed + 5), synth.gains(hd, rng_seed + 6)
    say(f"chain {synth.NAMES[kvtype]}: projections")
    xt = to_dev(x).view(torch.float16)
    yq, yk, yv = qp.prefill_gemm_qkv(Q6_K, to_dev(ws[0]), n_head * hd, to_dev(ws[1]), n_kv * hd, to_dev(ws[2]),
                                     n_kv * hd, hidden, xt, hd, to_dev(gq), to_dev(gk))
    torch.cuda.synchronize()
    q_in, k_in, v_in = yq.cpu().numpy(), yk.cpu().numpy(), yv.cpu().numpy()
    say(f"chain {synth.NAMES[kvtype]}: rope and cache")
    qp.rope(yq, n_head, hd, n_past, 1e6)
    qp.rope(yk, n_kv, hd, n_past, 1e6)
    rb = qp.row_bytes(kvtype, hd)
    past_k = synth.kv_cache(kvtype, n_past, n_kv, hd, rng_seed + 7)
    past_v = synth.kv_cache(kvtype, n_past, n_kv, hd, rng_seed + 8)
    kc = torch.zeros((n_past + t) * n_kv * rb, dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:past_k.size] = to_dev(past_k)
    vc[:past_v.size] = to_dev(past_v)
    qp.kv_cache_write(kvtype, yk, n_kv, hd, kc, n_past)
    qp.kv_cache_write(kvtype, yv, n_kv, hd, vc, n_past)
    say(f"chain {synth.NAMES[kvtype]}: attention")
    out = qp.prompt_attention(kvtype, yq, kc, vc, n_past, n_head, n_kv, hd)
    torch.cuda.synchronize()
    q_r, k_r = yq.cpu().numpy(), yk.cpu().numpy()
    kcn, vcn, y = kc.cpu().numpy(), vc.cpu().numpy(), out.cpu().numpy()
    # step by step on the GPU's own inputs
    rope_close(q_r, orc.rope(q_in, n_head, hd, n_past, 1e6), q_in, n_head, hd, n_past + t, "rope q")
    rope_close(k_r, orc.rope(k_in, n_kv, hd, n_past, 1e6), k_in, n_kv, hd, n_past + t, "rope k")
    assert np.array_equal(kcn[:past_k.size], past_k) and np.array_equal(vcn[:past_v.size], past_v), "past rows"
    assert np.array_equal(kcn[past_k.size:], orc.kv_quantize(kvtype, k_r, n_kv, hd)), "k cache rows"
    assert np.array_equal(vcn[past_v.size:], orc.kv_quantize(kvtype, v_in, n_kv, hd)), "v cache rows"
    ref = orc.attention(kvtype, q_r, kcn, vcn, n_past, n_head, n_kv, hd)
    assert_close(y, ref, f"chain {synth.NAMES[kvtype]} attention")
    # the whole chain from X through the oracle
    oq = orc.prefill_gemm_qknorm(Q6_K, ws[0], n_head * hd, hidden, x, hd, gq, 0, 1e-6).astype(np.float32)
    ok_ = orc.prefill_gemm_qknorm(Q6_K, ws[1], n_kv * hd, hidden, x, hd, gk, 0, 1e-6).astype(np.float32)
    ov = orc.prefill_gemm(Q6_K, ws[2], n_kv * hd, hidden, x).astype(np.float32)
    oq, ok_ = orc.rope(oq, n_head, hd, n_past, 1e6), orc.rope(ok_, n_kv, hd, n_past, 1e6)
    okc = np.concatenate([past_k, orc.kv_quantize(kvtype, ok_, n_kv, hd)])
    ovc = np.concatenate([past_v, orc.kv_quantize(kvtype, ov, n_kv, hd)])
    ref2 = orc.attention(kvtype, oq, okc, ovc, n_past, n_head, n_kv, hd)
    nw, cs = normwise(y, ref2), min_row_cos(y, ref2)
    say(f"  chain {synth.NAMES[kvtype]} from X: normwise {nw:.3e}  min row cos {cs:.8f}  bound {CHAIN_TOL[kvtype]:.1e}")
    assert nw <= CHAIN_TOL[kvtype] and cs >= 0.999, f"chain {synth.NAMES[kvtype]} from X: {nw:.3e} {cs:.8f}"
