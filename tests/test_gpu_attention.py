"""Prompt attention over a binary16, Q8_0 or Q4_0 KV cache on the GPU against the oracle."""
import numpy as np
import pytest

import synth
import quantized_prefill_amd as qp
from gpu_helpers import assert_close, sample_tokens, say, to_dev
from synth import F16W, Q4_0, Q8_0

pytestmark = pytest.mark.gpu

HD = 128


def queries(t: int, n_head: int, seed: int, ldq: int | None = None) -> np.ndarray:
    """Query rows as the q projection leaves them after its head norm: N(0, 1)
    values (RMS 1 per head), f32, optionally inside wider rows."""
    q = synth.activations_f32(t, ldq or n_head * HD, seed)
    return q


def run_attention(kvtype, q, kc, vc, n_past, n_head, n_kv, scale=None, ldo=None, workspace=None):
    import torch
    qd = to_dev(q)
    t = q.shape[0]
    out = None
    if ldo is not None:
        out = torch.full((t, ldo), float("nan"), dtype=torch.float32, device="cuda")
    y = qp.prompt_attention(kvtype, qd, to_dev(kc), to_dev(vc), n_past, n_head, n_kv, HD, scale, out=out,
                            workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy()


CASES = [
    # t, n_past, n_head, n_kv : one tile, ragged tails, a prefix of earlier chunks, MHA and GQA
    (1, 0, 4, 4),
    (37, 0, 8, 2),
    (128, 0, 4, 1),
    (300, 0, 8, 2),
    (200, 77, 8, 4),
    (129, 1000, 2, 1),
    (513, 64, 32, 8),
    (1, 4095, 32, 8),     # one query after a long prefix: 64 key blocks, one tile
    (64, 8000, 8, 8),     # a short chunk at the end of a long context
]


@pytest.mark.parametrize("kvtype", [F16W, Q8_0, Q4_0], ids=["F16", "Q8_0", "Q4_0"])
@pytest.mark.parametrize("t,n_past,n_head,n_kv", CASES)
def test_attention_small(orc, kvtype, t, n_past, n_head, n_kv):
    seed = 12000 + 7 * t + n_past + n_head
    q = queries(t, n_head, seed)
    kc = synth.kv_cache(kvtype, n_past + t, n_kv, HD, seed + 1)
    vc = synth.kv_cache(kvtype, n_past + t, n_kv, HD, seed + 2)
    y = run_attention(kvtype, q, kc, vc, n_past, n_head, n_kv)
    ref = orc.attention(kvtype, q, kc, vc, n_past, n_head, n_kv, HD)
    assert_close(y, ref, f"attention {synth.NAMES[kvtype]} t={t} past={n_past} heads={n_head}/{n_kv}")


def test_attention_strides_scale_and_bounds(orc):
    """Wider q and out rows, a non-default scale; columns past the heads stay untouched."""
    t, n_head, n_kv, ldq, ldo = 150, 4, 2, 4 * HD + 64, 4 * HD + 32
    q = queries(t, n_head, 12500, ldq)
    kc = synth.kv_cache(Q8_0, t, n_kv, HD, 12501)
    vc = synth.kv_cache(Q8_0, t, n_kv, HD, 12502)
    y = run_attention(Q8_0, q, kc, vc, 0, n_head, n_kv, scale=0.05, ldo=ldo)
    ref = orc.attention(Q8_0, q, kc, vc, 0, n_head, n_kv, HD, scale=0.05)
    assert_close(y[:, :n_head * HD], ref, "attention strided")
    assert np.all(np.isnan(y[:, n_head * HD:])), "wrote past the heads"


def test_attention_sharp_scores(orc):
    """A large scale makes the softmax nearly one-hot: the masking and the running
    maximum decide the result."""
    t, n_head, n_kv = 256, 4, 4
    q = queries(t, n_head, 12600)
    kc = synth.kv_cache(F16W, t, n_kv, HD, 12601)
    vc = synth.kv_cache(F16W, t, n_kv, HD, 12602)
    y = run_attention(F16W, q, kc, vc, 0, n_head, n_kv, scale=1.0)
    ref = orc.attention(F16W, q, kc, vc, 0, n_head, n_kv, HD, scale=1.0)
    assert_close(y, ref, "attention sharp")


@pytest.mark.parametrize("scale", [-0.09, 1e-44], ids=["negative", "subnormal"])
def test_attention_unusual_scales(orc, scale):
    """A negative scale (the kernel negates Q, exact in binary16) and a
    subnormal one (the softmax is uniform over the visible keys, and masked
    keys still get none of it)."""
    t, n_head, n_kv = 200, 4, 2
    q = queries(t, n_head, 12650)
    kc = synth.kv_cache(F16W, t, n_kv, HD, 12651)
    vc = synth.kv_cache(F16W, t, n_kv, HD, 12652)
    y = run_attention(F16W, q, kc, vc, 0, n_head, n_kv, scale=scale)
    ref = orc.attention(F16W, q, kc, vc, 0, n_head, n_kv, HD, scale=scale)
    assert_close(y, ref, f"attention scale {scale}")


@pytest.mark.parametrize("kvtype", [Q8_0, Q4_0], ids=["Q8_0", "Q4_0"])
@pytest.mark.parametrize("t,n_past,n_head,n_kv", [(200, 77, 8, 4), (2048, 0, 32, 8), (2200, 0, 32, 8)],
                         ids=["prefix", "one-round-halves", "single-halves"])
def test_attention_decoded_cache_bitwise(orc, kvtype, t, n_past, n_head, n_kv):
    """The workspace call decodes the quantized caches to binary16 rows first
    and attends over those; its output equals the call that decodes while
    staging, bit for bit (the binding's default is the workspace call, which
    every other test here checks against the oracle)."""
    seed = 13000 + t + n_past
    q = queries(t, n_head, seed)
    kc = synth.kv_cache(kvtype, n_past + t, n_kv, HD, seed + 1)
    vc = synth.kv_cache(kvtype, n_past + t, n_kv, HD, seed + 2)
    say(f"attention decoded cache {synth.NAMES[kvtype]} t={t} past={n_past}")
    a = run_attention(kvtype, q, kc, vc, n_past, n_head, n_kv)
    b = run_attention(kvtype, q, kc, vc, n_past, n_head, n_kv, workspace=False)
    assert np.array_equal(a, b), "decoded-cache attention differs from the in-kernel decode"


def test_attention_deterministic():
    t, n_head, n_kv = 333, 8, 2
    q = queries(t, n_head, 12700)
    kc = synth.kv_cache(Q8_0, t, n_kv, HD, 12701)
    vc = synth.kv_cache(Q8_0, t, n_kv, HD, 12702)
    a = run_attention(Q8_0, q, kc, vc, 0, n_head, n_kv)
    b = run_attention(Q8_0, q, kc, vc, 0, n_head, n_kv)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kvtype", [F16W, Q8_0, Q4_0], ids=["F16", "Q8_0", "Q4_0"])
def test_attention_qwen3_8b_t2048(orc, kvtype):
    """Qwen3-8B attention shape (32 query heads, 8 kv heads, head_dim 128) at
    T = 2048, the launch the bench times; sampled queries against the oracle."""
    t, n_head, n_kv = 2048, 32, 8
    q = queries(t, n_head, 12800)
    kc = synth.kv_cache(kvtype, t, n_kv, HD, 12801)
    vc = synth.kv_cache(kvtype, t, n_kv, HD, 12802)
    say(f"attention 8B t=2048 {synth.NAMES[kvtype]}")
    y = run_attention(kvtype, q, kc, vc, 0, n_head, n_kv)
    tok = sample_tokens(t, 24, 12803)
    ref = orc.attention(kvtype, q, kc, vc, 0, n_head, n_kv, HD, tokens=tok)
    assert_close(y[tok], ref, f"attention 8B {synth.NAMES[kvtype]}")


@pytest.mark.parametrize("kvtype,t", [(Q8_0, 8192), (Q4_0, 8192), (F16W, 2200)], ids=["Q8_0-8192", "Q4_0-8192",
                                                                                   "F16-2200"])
def test_attention_several_rounds(orc, kvtype, t):
    """Launches of more than one round of workgroups (32 heads: T = 2200, 18
    query tiles with a ragged last one, and the T = 8192 launch the bench
    times) take the single-half workgroups; sampled queries, the last
    included, against the oracle."""
    n_head, n_kv = 32, 8
    q = queries(t, n_head, 12900 + t)
    kc = synth.kv_cache(kvtype, t, n_kv, HD, 12901 + t)
    vc = synth.kv_cache(kvtype, t, n_kv, HD, 12902 + t)
    say(f"attention 8B t={t} {synth.NAMES[kvtype]}")
    y = run_attention(kvtype, q, kc, vc, 0, n_head, n_kv)
    tok = np.unique(np.concatenate([sample_tokens(t, 12, 12903 + t), [0, 127, 128, t - 1]]))
    ref = orc.attention(kvtype, q, kc, vc, 0, n_head, n_kv, HD, tokens=tok)
    assert_close(y[tok], ref, f"attention 8B t={t} {synth.NAMES[kvtype]}")


def test_attention_default_scale_and_huge_negative_scores(orc):
    """scale None takes the library's 1 / sqrt(head_dim), bit for bit the same
    as passing that f32 value; with every key equal and scaled scores near
    -1e31 the output is still the prefix mean of V (the running maximum
    starts at -inf)."""
    t, n_head, n_kv = 96, 4, 2
    q = queries(t, n_head, 9900)
    kc = synth.kv_cache(F16W, t, n_kv, HD, 9901)
    vc = synth.kv_cache(F16W, t, n_kv, HD, 9902)
    say("attention default scale")
    a = run_attention(F16W, q, kc, vc, 0, n_head, n_kv)
    b = run_attention(F16W, q, kc, vc, 0, n_head, n_kv, scale=float(np.float32(1.0 / np.sqrt(HD))))
    assert np.array_equal(a, b), "default scale differs from 1/sqrt(head_dim)"
    say("attention huge negative scores")
    qn = np.full((t, n_head * HD), 100.0, np.float32)
    kneg = np.full((t, n_kv, HD), -1.0, np.float16).view(np.uint8).reshape(-1)
    scale = 1e31 / (100.0 * HD)
    y = run_attention(F16W, qn, kneg, vc, 0, n_head, n_kv, scale=scale)
    assert np.isfinite(y).all(), "non-finite outputs"
    ref = orc.attention(F16W, qn, kneg, vc, 0, n_head, n_kv, HD, scale=scale)
    assert_close(y, ref, "huge negative scores")
