"""Router and routed grouped-expert FFN on the GPU against the oracle."""
import numpy as np
import pytest

import synth
import quantized_prefill_amd as qp
from gpu_helpers import assert_close, act_f16, sample_tokens, say, to_dev
from synth import F16W, Q8_0, Q4_K, Q5_K, Q6_K, Q2_K

pytestmark = pytest.mark.gpu


def gpu_route(logits: np.ndarray, top_k: int, renorm=False):
    import torch
    ids, w = qp.moe_route_topk(to_dev(logits), top_k, renorm)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("t,e,k", [(1, 4, 1), (50, 16, 4), (333, 128, 8), (64, 1024, 8), (17, 64, 64)])
def test_router(orc, t, e, k):
    lg = synth.router_logits(t, e, 9500 + e)
    lg[::5, 1] = lg[::5, 3]  # ties between experts
    ids, w = gpu_route(lg, k)
    rid, rw = orc.route_topk(lg, k)
    assert np.array_equal(ids, rid), "expert selection differs"
    assert np.allclose(w, rw, rtol=2e-6, atol=1e-9), "route weights differ"
    ids, w = gpu_route(lg, k, renorm=True)
    rid, rw = orc.route_topk(lg, k, renorm=True)
    assert np.array_equal(ids, rid)
    assert np.allclose(w, rw, rtol=2e-6, atol=1e-9)


def run_moe(qtype, wg, wu, wd, ne, hidden, inter, x, ids, wts, dropped=None):
    """The routed FFN's output; with dropped=<expected count>, also checks the
    workspace header's count of pairs dropped for an out-of-range id."""
    import torch
    t, top_k = ids.shape
    ws = torch.empty(qp.grouped_expert_workspace_bytes(t, top_k, ne, hidden, inter), dtype=torch.uint8, device="cuda")
    out = qp.grouped_expert_gemm(qtype, to_dev(wg), to_dev(wu), to_dev(wd), ne, hidden, inter,
                                 to_dev(x).view(torch.float16), to_dev(ids.astype(np.int32)),
                                 to_dev(wts.astype(np.float32)), workspace=ws)
    torch.cuda.synchronize()
    if dropped is not None:
        got = qp.grouped_expert_dropped_pairs(ws)
        assert got == dropped, f"dropped-pair count {got}, want {dropped}"
    return out.cpu().numpy()


@pytest.mark.parametrize("qtype", [Q4_K, Q5_K, Q8_0, Q6_K, Q2_K, F16W], ids=["Q4_K", "Q5_K", "Q8_0", "Q6_K", "Q2_K",
                                                                          "F16"])
def test_moe_small(orc, qtype):
    """8 experts, top-2, ragged per-expert counts (some experts empty)."""
    t, ne, k, hidden, inter = 157, 8, 2, 256, 512
    wg = synth.quant_weights(qtype, ne * inter, hidden, 9600)
    wu = synth.quant_weights(qtype, ne * inter, hidden, 9601)
    wd = synth.quant_weights(qtype, ne * hidden, inter, 9602)
    x = act_f16(t, hidden, 9603)
    lg = synth.router_logits(t, ne, 9604)
    lg[:, 5] -= 100.0  # expert 5 never chosen
    ids, wts = orc.route_topk(lg, k)
    y = run_moe(qtype, wg, wu, wd, ne, hidden, inter, x, ids, wts, dropped=0)
    ref = orc.moe(qtype, wg, wu, wd, ne, hidden, inter, x, ids, wts)
    assert_close(y, ref, f"moe small {synth.NAMES[qtype]}")


@pytest.mark.parametrize("qtype", [Q4_K, Q5_K, Q8_0, Q6_K, Q2_K, F16W], ids=["Q4_K", "Q5_K", "Q8_0", "Q6_K", "Q2_K",
                                                                          "F16"])
def test_moe_long_skewed_lists(orc, qtype):
    """Long per-expert lists from skewed routing: one list of several tiles
    (the last ragged), one empty expert; two calls give identical bits."""
    t, ne, k, hidden, inter = 1024, 5, 2, 256, 512
    wg = synth.quant_weights(qtype, ne * inter, hidden, 9650)
    wu = synth.quant_weights(qtype, ne * inter, hidden, 9651)
    wd = synth.quant_weights(qtype, ne * hidden, inter, 9652)
    x = act_f16(t, hidden, 9653)
    lg = synth.router_logits(t, ne, 9654)
    lg[:, 0] += 1.5    # expert 0 takes most tokens
    lg[:, 3] -= 100.0  # expert 3 never chosen
    ids, wts = orc.route_topk(lg, k)
    say(f"moe long lists {synth.NAMES[qtype]} counts {np.bincount(ids.reshape(-1), minlength=ne).tolist()}")
    y = run_moe(qtype, wg, wu, wd, ne, hidden, inter, x, ids, wts)
    tok = sample_tokens(t, 64, 9655)
    ref = orc.moe(qtype, wg, wu, wd, ne, hidden, inter, x, ids, wts, tokens=tok)
    assert_close(y[tok], ref, f"moe long lists {synth.NAMES[qtype]}")
    y2 = run_moe(qtype, wg, wu, wd, ne, hidden, inter, x, ids, wts)
    assert np.array_equal(y, y2), "routed FFN differs between two calls"


def test_moe_invalid_ids_and_determinism(orc):
    """Pairs whose expert id is out of range add nothing; results repeat bit for bit."""
    t, ne, k, hidden, inter = 64, 4, 2, 256, 256
    wg = synth.quant_weights(Q4_K, ne * inter, hidden, 9700)
    wu = synth.quant_weights(Q4_K, ne * inter, hidden, 9701)
    wd = synth.quant_weights(Q4_K, ne * hidden, inter, 9702)
    x = act_f16(t, hidden, 9703)
    ids, wts = orc.route_topk(synth.router_logits(t, ne, 9704), k)
    bad = ids.copy()
    bad[::3, 1] = ne + 5
    bad[1::7, 0] = -1
    keep = (bad >= 0) & (bad < ne)
    y = run_moe(Q4_K, wg, wu, wd, ne, hidden, inter, x, bad, wts, dropped=int((~keep).sum()))
    ref = orc.moe(Q4_K, wg, wu, wd, ne, hidden, inter, x, np.where(keep, bad, 0), np.where(keep, wts, 0.0))
    rows = np.flatnonzero(np.abs(ref).sum(axis=1) > 0)
    assert_close(y[rows], ref[rows], "moe with dropped pairs")
    dead = np.flatnonzero(~keep.any(axis=1))
    assert np.all(y[dead] == 0.0)
    y2 = run_moe(Q4_K, wg, wu, wd, ne, hidden, inter, x, bad, wts)
    assert np.array_equal(y, y2)


def test_moe_workload(orc):
    """128 experts (Q4_K gate/up 2048 -> 768, down 768 -> 2048), T = 4096,
    top-8 of a softmax over N(0, 1) router logits; the router runs on the GPU
    and must pick the oracle's experts."""
    t, ne, k, hidden, inter = 4096, 128, 8, 2048, 768
    say("moe workload: generating experts")
    wg = synth.quant_weights(Q4_K, ne * inter, hidden, synth.seed_for(4, 2))
    wu = synth.quant_weights(Q4_K, ne * inter, hidden, synth.seed_for(4, 3))
    wd = synth.quant_weights(Q4_K, ne * hidden, inter, synth.seed_for(4, 4))
    x = act_f16(t, hidden, synth.seed_for(4, 0))
    lg = synth.router_logits(t, ne, synth.seed_for(4, 1))
    ids, w = gpu_route(lg, k)
    rid, rw = orc.route_topk(lg, k)
    assert np.array_equal(ids, rid)
    assert np.allclose(w, rw, rtol=2e-6)
    say("moe workload: grouped expert GEMM")
    y = run_moe(Q4_K, wg, wu, wd, ne, hidden, inter, x, ids, w)
    tok = sample_tokens(t, 64, 9800)
    ref = orc.moe(Q4_K, wg, wu, wd, ne, hidden, inter, x, rid, rw, tokens=tok)
    assert_close(y[tok], ref, "moe workload")
