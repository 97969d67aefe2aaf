"""Benchmark of the quantized prefill path on one MI355X.

One step is one pass of the path over one Qwen3-8B-shaped layer at T = 2048
prompt tokens, in both Q6_K and Q2_K: the f32 and f16 dequant of every
projection weight (q, k, v, o, gate, up, down), then every projection
Y = X . W^T with W dequantized on load: q, k (through the per-head QK-norm
epilogue) and v in one call over their shared X, then o, gate, up and down.
Inputs are seeded synthetic tensors resident in HBM before timing starts.
`value` is the projection TFLOP/s (sum of algorithmic flops over the
sum of the projection launches' HIP-event durations); the dequant GB/s is
reported beside it, per (type, output dtype) and in total, from a timed
region of the 28 dequants alone, and as measured inside the layer step.
Every dequant writes its own destination (2.3 GB of outputs per pass, far
past the 256 MB last-level cache), so no output is rewritten inside the
cache.  After the timed region the remaining workloads -- the
Q8_0 1024 x 1024 projection, the Q4_K Qwen3-1.7B layer at T = 512, the Q5_K
Qwen3-8B layer at T = 2048 (projections one by one), the fused
QK-norm projections at T = 8192, the routed 128-expert FFN and causal prompt
attention with Qwen3-8B heads over a binary16, Q8_0 or Q4_0 KV cache -- are timed
and reported under "rows".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill projection TFLOP/s (FP16 MFMA %peak) + dequant GB/s, 8B shapes T=2048"
PEAK_F16_TFLOPS = 2500.0   # MI355X dense FP16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
WORKLOAD = "q6_k_q2_k_qwen3_8b_t2048"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_wide_q6k_gate_up_qwen3_8b_t2048.txt")
# The kernel the roofline object describes: the 256 x 256-tile projection
# kernel with weights decoded in registers, for Q6_K weights, running the
# gate and up projections of the 8B layer at T = 2048 in one launch (768
# tiles): the layer's largest share of flops.
DOMINANT = "gemm_wide_kernel<14, 5, 8, 1> (Q6_K gate and up in one launch, f16 X, 256 x 256 tiles)"
DOMINANT_PROJS = ("gate", "up")
KERNEL_SOURCES = ("gemm_wide.hip", "gemm_common.h", "qp_device.h", "qp_internal.h")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantized_prefill_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary ("key: value" lines), if its counters were taken on the current
    kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = dict(l.split(":", 1) for l in fh.read().splitlines() if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    rec = {k.strip(): v.strip() for k, v in rec.items()}
    if rec.get("source_digest") != kernel_source_digest():
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device-to-device copy of 256 MiB, three times: the byte
    counters read on it give the scale from counter units to bytes."""
    import torch
    n = 256 * 1024 * 1024 // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "bytes_written": 4 * n, "launches": 3}), flush=True)


class Timer:
    """HIP-event pairs around launches on torch's current stream."""

    def __init__(self):
        self.pending = []   # (category, start, end)
        self.total = {}
        self.count = {}

    def run(self, cat, fn):
        import torch
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pending.append((cat, s, e))

    def collect(self):
        for cat, s, e in self.pending:
            self.total[cat] = self.total.get(cat, 0.0) + s.elapsed_time(e)
            self.count[cat] = self.count.get(cat, 0) + 1
        self.pending = []

    def reset(self):
        self.pending, self.total, self.count = [], {}, {}


def build_8b(torch, synth, qp):
    """Weights (both types), activations and outputs of the 8B layer."""
    t, hidden = 2048, 4096
    dev = torch.device("cuda")
    xs = {}
    for k in sorted({k for _, _, k in synth.PROJ_8B}):
        xs[k] = torch.from_numpy(synth.activations_f16(t, k, synth.seed_for(2, 500 + k // 256))).to(dev).view(
            torch.float16)
    projs = []
    for qt in (synth.Q6_K, synth.Q2_K):
        for i, (name, n, k) in enumerate(synth.PROJ_8B):
            raw = synth.quant_weights(qt, n, k, synth.seed_for(2, 10 * qt + i))
            projs.append(dict(name=name, qtype=qt, n=n, k=k, w=torch.from_numpy(raw).to(dev),
                              dom=qt == synth.Q6_K and name in DOMINANT_PROJS,
                              y=torch.empty((t, n), dtype=torch.float32, device=dev)))
    gains = {name: torch.from_numpy(synth.gains(128, synth.seed_for(2, 600 + j))).to(dev)
             for j, name in enumerate(("q", "k"))}
    # one f32 and one f16 destination per projection and type
    for p in projs:
        p["d32"] = torch.empty((p["n"], p["k"]), dtype=torch.float32, device=dev)
        p["d16"] = torch.empty((p["n"], p["k"]), dtype=torch.float16, device=dev)
    return dict(t=t, hidden=hidden, xs=xs, projs=projs, gains=gains, qtypes=(synth.Q6_K, synth.Q2_K))


def dequant_group(qp, L, qt, f16):
    """The f32 (or f16) dequant of the seven projections of one type, back to back."""
    for p in L["projs"]:
        if p["qtype"] == qt:
            if f16:
                qp.dequant_f16(qt, p["w"], p["n"], p["k"], out=p["d16"])
            else:
                qp.dequant_f32(qt, p["w"], p["n"], p["k"], out=p["d32"])


def dequant_pass(L, qp, synth, timer):
    """The 28 dequants of the layer, one event pair per (type, dtype) group of 7."""
    for qt in L["qtypes"]:
        for f16 in (False, True):
            timer.run(f"dequant:{synth.NAMES[qt]}:{'f16' if f16 else 'f32'}",
                      lambda qt=qt, f16=f16: dequant_group(qp, L, qt, f16))


def step_8b(L, qp, synth, timer):
    dequant_pass(L, qp, synth, timer)
    for qt in L["qtypes"]:
        pr = {p["name"]: p for p in L["projs"] if p["qtype"] == qt}
        q, k, v = pr["q"], pr["k"], pr["v"]
        x = L["xs"][q["k"]]
        # q and k with the per-head RMSNorm and v, one call over the shared X
        timer.run("gemm", lambda q=q, k=k, v=v, x=x: qp.prefill_gemm_qkv(
            qt, q["w"], q["n"], k["w"], k["n"], v["w"], v["n"], q["k"], x, 128, L["gains"]["q"], L["gains"]["k"],
            out_q=q["y"], out_k=k["y"], out_v=v["y"]))
        o, g, u, dn = pr["o"], pr["gate"], pr["up"], pr["down"]
        timer.run("gemm", lambda p=o: qp.prefill_gemm(p["qtype"], p["w"], p["n"], p["k"], L["xs"][p["k"]], out=p["y"]))
        # gate and up, one call over the shared X
        timer.run("gemm_dom" if g["dom"] else "gemm", lambda g=g, u=u: qp.prefill_gemm_gate_up(
            qt, g["w"], u["w"], g["n"], g["k"], L["xs"][g["k"]], out_gate=g["y"], out_up=u["y"]))
        timer.run("gemm", lambda p=dn: qp.prefill_gemm(p["qtype"], p["w"], p["n"], p["k"], L["xs"][p["k"]], out=p["y"]))


def gemm_flops_8b(L):
    return sum(2.0 * L["t"] * p["n"] * p["k"] for p in L["projs"])


def dequant_bytes_8b(L, synth, qt=None, f16=None):
    """Algorithmic bytes of the layer's dequants (the weights read once per
    launch, every output written once), optionally of one type or dtype."""
    tot = 0.0
    for p in L["projs"]:
        if qt is not None and p["qtype"] != qt:
            continue
        read = p["n"] * synth.row_bytes(p["qtype"], p["k"])
        for is16 in (False, True):
            if f16 is None or f16 == is16:
                tot += read + p["n"] * p["k"] * (2 if is16 else 4)
    return tot


def dequant_graph_gbps(torch, qp, L, synth, replays=10):
    """The layer's 28 dequant launches (f32 and f16 of every weight), captured
    once into a HIP graph and replayed back to back: the kernels' rate without
    the per-launch event pairs and host dispatch between them.  Reported beside
    the per-launch figure, never instead of it."""
    def deq():
        for qt in L["qtypes"]:
            for f16 in (False, True):
                dequant_group(qp, L, qt, f16)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        deq()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        deq()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / replays
    del g
    return dequant_bytes_8b(L, synth) / ms / 1e6


def time_fn(torch, fn, iters):
    fn()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters  # ms


def raw_gemm(torch, qp, qtype, w, n, k, x, y):
    """qp_prefill_gemm_ws with its arguments prepared once (the binding's
    cached workspace): a row of launches of ten microseconds then times the
    library's launches, not the binding's per-call argument checks."""
    t = x.shape[0]
    xd = qp.F16 if x.dtype == torch.float16 else qp.F32
    ws = qp.gemm_workspace(n, k, t, x.device)
    args = (qtype, w.data_ptr(), n, k, x.data_ptr(), xd, t, x.stride(0), y.data_ptr(), y.stride(0),
            ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
            torch.cuda.current_stream().cuda_stream)
    fn = qp.lib().qp_prefill_gemm_ws

    def call():
        if fn(*args) != 0:
            raise RuntimeError("qp_prefill_gemm_ws failed")
    return call


def raw_dequant_f32(torch, qp, qtype, w, rows, cols, out):
    """qp_dequant_f32 with its arguments prepared once (as raw_gemm)."""
    args = (qtype, w.data_ptr(), rows, cols, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    fn = qp.lib().qp_dequant_f32

    def call():
        if fn(*args) != 0:
            raise RuntimeError("qp_dequant_f32 failed")
    return call


def raw_attention(torch, qp, kv_type, q, kc, vc, t, out, n_head=32, n_kv=8, head_dim=128):
    """qp_prompt_attention_ws with its arguments prepared once (the binding's
    cached workspace for a quantized cache; as raw_gemm)."""
    ws = qp.attention_workspace(kv_type, t, n_kv, head_dim, q.device)
    args = (kv_type, q.data_ptr(), q.stride(0), kc.data_ptr(), vc.data_ptr(), 0, t, n_head, n_kv, head_dim, 0.0,
            out.data_ptr(), out.stride(0), ws.data_ptr() if ws is not None else None,
            ws.numel() if ws is not None else 0, torch.cuda.current_stream().cuda_stream)
    fn = qp.lib().qp_prompt_attention_ws

    def call():
        if fn(*args) != 0:
            raise RuntimeError("qp_prompt_attention_ws failed")
    return call


ROW_GROUPS = ("q8_0", "q4_k_1p7b", "q5_k_8b", "qknorm", "moe", "attention")


def other_rows(torch, synth, qp, iters, which=ROW_GROUPS):
    """The other workloads, each timed on its own after the main region
    (`which`: the groups of ROW_GROUPS to run)."""
    dev = torch.device("cuda")
    rows = {}
    if "q8_0" in which:
        rows.update(_rows_q8_0(torch, synth, qp, iters, dev))
    if "q4_k_1p7b" in which:
        rows.update(_rows_q4_k_1p7b(torch, synth, qp, iters, dev))
    if "q5_k_8b" in which:
        rows.update(_rows_q5_k_8b(torch, synth, qp, iters, dev))
    if "qknorm" in which:
        rows.update(_rows_qknorm(torch, synth, qp, iters, dev))
    if "moe" in which:
        rows.update(_rows_moe(torch, synth, qp, iters, dev))
    if "attention" in which:
        rows.update(attention_rows(torch, synth, qp, iters))
    return rows


def _dev(torch, dev, a):
    return torch.from_numpy(a).to(dev)


def _rows_q8_0(torch, synth, qp, iters, dev):
    rows = {}

    def d(a):
        return _dev(torch, dev, a)

    # Q8_0 1024 x 1024, T = 64, f32 activations
    w = d(synth.quant_weights(synth.Q8_0, 1024, 1024, synth.seed_for(0, 0)))
    x = d(synth.activations_f32(64, 1024, synth.seed_for(0, 1)))
    y = torch.empty((64, 1024), device=dev)
    ms = time_fn(torch, raw_gemm(torch, qp, synth.Q8_0, w, 1024, 1024, x, y), iters)
    o32 = torch.empty((1024, 1024), device=dev)
    msd = time_fn(torch, raw_dequant_f32(torch, qp, synth.Q8_0, w, 1024, 1024, o32), iters)
    rows["q8_0_1024_t64"] = dict(gemm_tflops=2 * 64 * 1024 * 1024 / ms / 1e9, gemm_us=ms * 1e3,
                                 dequant_f32_gbps=(1024 * 1088 + 1024 * 1024 * 4) / msd / 1e6)
    return rows


def _rows_q4_k_1p7b(torch, synth, qp, iters, dev):
    rows = {}

    def d(a):
        return _dev(torch, dev, a)

    # Q4_K, Qwen3-1.7B layer at T = 512
    flops, tms, dbytes, dms = 0.0, 0.0, 0.0, 0.0
    for i, (name, n, k) in enumerate(synth.PROJ_1_7B):
        w = d(synth.quant_weights(synth.Q4_K, n, k, synth.seed_for(1, i)))
        x = d(synth.activations_f16(512, k, synth.seed_for(1, 500 + k // 256))).view(torch.float16)
        y = torch.empty((512, n), device=dev)
        tms += time_fn(torch, raw_gemm(torch, qp, synth.Q4_K, w, n, k, x, y), iters)
        flops += 2.0 * 512 * n * k
        o32 = torch.empty((n, k), device=dev)
        dms += time_fn(torch, raw_dequant_f32(torch, qp, synth.Q4_K, w, n, k, o32), iters)
        dbytes += n * synth.row_bytes(synth.Q4_K, k) + 4.0 * n * k
    rows["q4_k_qwen3_1p7b_t512"] = dict(gemm_tflops=flops / tms / 1e9, gemm_us=tms * 1e3,
                                        dequant_f32_gbps=dbytes / dms / 1e6)
    return rows


def _rows_q5_k_8b(torch, synth, qp, iters, dev):
    rows = {}

    def d(a):
        return _dev(torch, dev, a)

    # Q5_K, Qwen3-8B layer at T = 2048 (the seven projections, each on its own)
    flops, tms, dbytes, dms = 0.0, 0.0, 0.0, 0.0
    x8 = {}
    for i, (name, n, k) in enumerate(synth.PROJ_8B):
        if k not in x8:
            x8[k] = d(synth.activations_f16(2048, k, synth.seed_for(2, 500 + k // 256))).view(torch.float16)
        w = d(synth.quant_weights(synth.Q5_K, n, k, synth.seed_for(2, 10 * synth.Q5_K + i)))
        y = torch.empty((2048, n), device=dev)
        tms += time_fn(torch, raw_gemm(torch, qp, synth.Q5_K, w, n, k, x8[k], y), iters)
        flops += 2.0 * 2048 * n * k
        o32 = torch.empty((n, k), device=dev)
        dms += time_fn(torch, raw_dequant_f32(torch, qp, synth.Q5_K, w, n, k, o32), iters)
        dbytes += n * synth.row_bytes(synth.Q5_K, k) + 4.0 * n * k
        del w, y, o32
    rows["q5_k_qwen3_8b_t2048"] = dict(gemm_tflops=flops / tms / 1e9, gemm_us=tms * 1e3,
                                       dequant_f32_gbps=dbytes / dms / 1e6)
    del x8
    return rows


def _rows_qknorm(torch, synth, qp, iters, dev):
    rows = {}

    def d(a):
        return _dev(torch, dev, a)

    # fused QK norm, T = 8192
    t = 8192
    x = d(synth.activations_f16(t, 4096, synth.seed_for(3, 0))).view(torch.float16)
    flops, tms = 0.0, 0.0
    for qt, n, ws, gs in ((synth.Q4_K, 4096, synth.seed_for(3, 1), synth.seed_for(3, 3)),
                          (synth.Q6_K, 1024, synth.seed_for(3, 2), synth.seed_for(3, 4))):
        w = d(synth.quant_weights(qt, n, 4096, ws))
        g = d(synth.gains(128, gs))
        y = torch.empty((t, n), device=dev)
        tms += time_fn(torch, lambda: qp.prefill_gemm_qknorm(qt, w, n, 4096, x, 128, g, 0, 1e-6, out=y), iters)
        flops += 2.0 * t * n * 4096
    rows["qknorm_qwen3_8b_t8192"] = dict(tflops=flops / tms / 1e9, us=tms * 1e3)
    del x, y
    return rows


def _rows_moe(torch, synth, qp, iters, dev):
    rows = {}

    def d(a):
        return _dev(torch, dev, a)

    # routed experts: 128 experts, top-8, T = 4096, router included
    t, ne, k, hidden, inter = 4096, 128, 8, 2048, 768
    wg = d(synth.quant_weights(synth.Q4_K, ne * inter, hidden, synth.seed_for(4, 2)))
    wu = d(synth.quant_weights(synth.Q4_K, ne * inter, hidden, synth.seed_for(4, 3)))
    wd = d(synth.quant_weights(synth.Q4_K, ne * hidden, inter, synth.seed_for(4, 4)))
    x = d(synth.activations_f16(t, hidden, synth.seed_for(4, 0))).view(torch.float16)
    lg = d(synth.router_logits(t, ne, synth.seed_for(4, 1)))
    ids = torch.empty((t, k), dtype=torch.int32, device=dev)
    wts = torch.empty((t, k), dtype=torch.float32, device=dev)
    out = torch.empty((t, hidden), device=dev)
    ws = torch.empty(qp.grouped_expert_workspace_bytes(t, k, ne, hidden, inter), dtype=torch.uint8, device=dev)

    def moe():
        qp.moe_route_topk(lg, k, False, ids=ids, weights=wts)
        qp.grouped_expert_gemm(synth.Q4_K, wg, wu, wd, ne, hidden, inter, x, ids, wts, out=out, workspace=ws)

    ms = time_fn(torch, moe, iters)
    flops = 2.0 * t * k * 3 * hidden * inter
    rows["moe_e128_top8_t4096"] = dict(tflops=flops / ms / 1e9, us=ms * 1e3)
    del wg, wu, wd, x, lg, ids, wts, out, ws
    return rows


def attention_flops(t: int, n_past: int, n_head: int, head_dim: int) -> float:
    """Algorithmic flops of causal prompt attention: query i sees n_past + i + 1
    keys, each costing a head_dim dot product and a head_dim multiply-add of V."""
    keys = t * n_past + t * (t + 1) / 2
    return 4.0 * head_dim * n_head * keys


def attention_rows(torch, synth, qp, iters):
    """Causal prompt attention, Qwen3-8B heads (32 query, 8 kv, head_dim 128),
    over a binary16, Q8_0 or Q4_0 KV cache."""
    dev = torch.device("cuda")
    rows = {}
    for kvtype, t in ((synth.F16W, 2048), (synth.Q8_0, 2048), (synth.Q4_0, 2048), (synth.Q8_0, 8192),
                      (synth.Q4_0, 8192)):
        q = torch.from_numpy(synth.activations_f32(t, 32 * 128, synth.seed_for(5, t))).to(dev)
        kc = torch.from_numpy(synth.kv_cache(kvtype, t, 8, 128, synth.seed_for(5, t + 1))).to(dev)
        vc = torch.from_numpy(synth.kv_cache(kvtype, t, 8, 128, synth.seed_for(5, t + 2))).to(dev)
        out = torch.empty((t, 32 * 128), device=dev)
        qp.prompt_attention(kvtype, q, kc, vc, 0, 32, 8, 128, out=out)  # checks the arguments once
        ms = time_fn(torch, raw_attention(torch, qp, kvtype, q, kc, vc, t, out), iters)
        name = f"attention_{synth.NAMES[kvtype].lower()}_kv_qwen3_8b_t{t}"
        rows[name] = dict(tflops=attention_flops(t, 0, 32, 128) / ms / 1e9, us=ms * 1e3)
        del q, kc, vc, out
    return rows


def cpu_info():
    """(CPU model name, logical CPUs) of the host."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model or "unknown", os.cpu_count()


def cpu_baseline(synth, budget_s: float):
    """The oracle (binary64 GEMM over its own exact dequant, and its f32
    dequant) on the host cores, all threads and one thread, each on a bounded
    sample of the same workload sized to a share of budget_s seconds."""
    import numpy as np
    import oracle
    orc = oracle.get()
    model, nproc = cpu_info()
    threads_all = orc.num_threads()
    projs = []
    for qt in (synth.Q6_K, synth.Q2_K):
        for i, (name, n, k) in enumerate(synth.PROJ_8B):
            projs.append((qt, name, n, k, synth.quant_weights(qt, n, k, synth.seed_for(2, 10 * qt + i))))

    def gemm_rate(sel, share):
        """Grow the token count until the sample takes about `share` seconds
        (the per-token cost falls as the dequant of each weight is shared)."""
        xs = {}

        def run(ntok):
            for k in {p[3] for p in sel}:
                xs[k] = synth.activations_f16(ntok, k, synth.seed_for(2, 500 + k // 256))
            flops = 0.0
            t0 = time.perf_counter()
            for qt, _, n, k, raw in sel:
                orc.prefill_gemm(qt, raw, n, k, xs[k])
                flops += 2.0 * ntok * n * k
            return flops, time.perf_counter() - t0

        ntok = 1
        flops, dt = run(ntok)
        while dt < 0.5 * share and ntok < 512:
            ntok = int(max(ntok + 1, min(512, ntok * share / max(dt, 1e-3))))
            flops, dt = run(ntok)
        return flops / dt / 1e9, ntok, dt

    def dequant_rate(sel):
        nbytes, dt = 0.0, 0.0
        for qt, _, n, k, raw in sel:
            t0 = time.perf_counter()
            out = orc.dequant_f32(qt, raw, n, k)
            dt += time.perf_counter() - t0
            nbytes += raw.size + out.nbytes
            del out
        return nbytes / dt / 1e9, dt

    gate = [p for p in projs if p[1] == "gate"]            # 12288 x 4096, Q6_K and Q2_K
    small = [p for p in projs if p[1] in ("k", "v")]      # 1024 x 4096, both types
    orc.set_num_threads(threads_all)
    g_all, n_all, t_all = gemm_rate(projs, 0.45 * budget_s)
    d_all, td_all = dequant_rate(gate)
    orc.set_num_threads(1)
    g_one, n_one, t_one = gemm_rate(small, 0.25 * budget_s)
    d_one, td_one = dequant_rate(small)
    orc.set_num_threads(threads_all)
    return dict(value=g_all / 1e3, unit="TFLOP/s", cores=threads_all, kind="oracle",
                sample=(f"GEMM: first {n_all} token rows of each of the 14 Qwen3-8B projections (Q6_K and Q2_K) on "
                        f"{threads_all} threads ({t_all:.1f} s), first {n_one} rows of the k and v projections "
                        f"on 1 thread ({t_one:.1f} s), binary64 dot products over the oracle's f32 dequant; "
                        f"dequant to f32: the two 12288 x 4096 gate tensors on {threads_all} threads "
                        f"({td_all:.1f} s), the four 1024 x 4096 k/v tensors on 1 thread ({td_one:.1f} s)"),
                cpu_model=model, nproc=nproc, threads_all=threads_all,
                gemm_gflops_all_threads=round(g_all, 3), gemm_gflops_1_thread=round(g_one, 3),
                dequant_f32_gbps_all_threads=round(d_all, 3), dequant_f32_gbps_1_thread=round(d_one, 3))


def two_pass_row(torch, synth, qp, L, iters):
    """The f16-cache mode as a comparator: the Q6_K layer's weights are
    dequantized once to binary16 (qp.dequant_f16), then the same projections
    run as plain F16-weight products.  Reported beside the dequant-on-load
    time of the same calls: the products alone on the cached weights, the
    whole two passes, and the memory each form of the weights takes."""
    qt = synth.Q6_K
    pr = {p["name"]: p for p in L["projs"] if p["qtype"] == qt}
    cache = {nm: torch.empty((p["n"], p["k"]), dtype=torch.float16, device="cuda") for nm, p in pr.items()}

    def deq():
        for nm, p in pr.items():
            qp.dequant_f16(qt, p["w"], p["n"], p["k"], out=cache[nm])

    def gemms(wt, ws):
        q, k, v = pr["q"], pr["k"], pr["v"]
        qp.prefill_gemm_qkv(wt, ws["q"], q["n"], ws["k"], k["n"], ws["v"], v["n"], q["k"], L["xs"][q["k"]], 128,
                            L["gains"]["q"], L["gains"]["k"], out_q=q["y"], out_k=k["y"], out_v=v["y"])
        for nm in ("o", "gate", "up", "down"):
            p = pr[nm]
            qp.prefill_gemm(wt, ws[nm], p["n"], p["k"], L["xs"][p["k"]], out=p["y"])

    quant = {nm: p["w"] for nm, p in pr.items()}
    flops = sum(2.0 * L["t"] * p["n"] * p["k"] for p in pr.values())
    ms_load = time_fn(torch, lambda: gemms(qt, quant), iters)
    deq()
    ms_cached = time_fn(torch, lambda: gemms(qp.F16W, cache), iters)
    ms_deq = time_fn(torch, deq, iters)
    row = dict(dequant_on_load_tflops=flops / ms_load / 1e9, dequant_on_load_us=ms_load * 1e3,
               f16_cache_gemm_tflops=flops / ms_cached / 1e9, f16_cache_gemm_us=ms_cached * 1e3,
               f16_cache_dequant_us=ms_deq * 1e3, two_pass_us=(ms_deq + ms_cached) * 1e3,
               weights_mb_quantized=sum(p["w"].numel() for p in pr.values()) / 1e6,
               weights_mb_f16_cache=sum(c.numel() * 2 for c in cache.values()) / 1e6)
    del cache
    return row


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-rows", action="store_true", help="skip the other workloads")
    ap.add_argument("--rows", default=",".join(ROW_GROUPS),
                    help="comma-separated groups of the other workloads to run: " + ", ".join(ROW_GROUPS))
    ap.add_argument("--no-two-pass", action="store_true", help="skip the f16-cache comparator")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 256 MiB copy that calibrates the byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import quantized_prefill_amd as qp

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    qp.lib()
    print("bench: generating the 8B-layer inputs", file=sys.stderr, flush=True)
    L = build_8b(torch, synth, qp)
    torch.cuda.synchronize()
    timer = Timer()
    for _ in range(args.warmup):
        step_8b(L, qp, synth, timer)
    torch.cuda.synchronize()
    timer.reset()
    print("bench: timed steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_8b(L, qp, synth, timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.collect()

    dom_ms = timer.total["gemm_dom"] / timer.count["gemm_dom"]   # average launch
    dom_flops = sum(2.0 * L["t"] * p["n"] * p["k"] for p in L["projs"] if p["dom"])  # one launch covers them
    gemm_ms = (timer.total["gemm"] + timer.total["gemm_dom"]) / args.steps
    deq_cats = [c for c in timer.total if c.startswith("dequant:")]
    deq_layer_ms = sum(timer.total[c] for c in deq_cats) / args.steps
    # the dequants again in a timed region of their own: inside the layer step
    # each follows the previous step's projections, whose outputs (up to
    # 200 MB of Y) are still dirty in the last-level cache and get written
    # back while the dequant streams its own outputs
    print("bench: dequant region", file=sys.stderr, flush=True)
    dtimer = Timer()
    for _ in range(2):
        dequant_pass(L, qp, synth, dtimer)
    torch.cuda.synchronize()
    dtimer.reset()
    for _ in range(args.steps):
        dequant_pass(L, qp, synth, dtimer)
    torch.cuda.synchronize()
    dtimer.collect()
    deq_ms = sum(dtimer.total.values()) / args.steps
    deq_rows = {}
    for c in sorted(dtimer.total):
        _, tname, dt = c.split(":")
        qt = synth.BY_NAME[tname]
        ms = dtimer.total[c] / dtimer.count[c]
        nbytes = dequant_bytes_8b(L, synth, qt, dt == "f16")
        deq_rows[f"{tname}_{dt}"] = {"gbps": round(nbytes / ms / 1e6, 1), "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBPS, 4),
                                     "us": round(ms * 1e3, 2), "mbytes": round(nbytes / 1e6, 1), "launches": 7}
    flops = gemm_flops_8b(L)
    tflops = flops / gemm_ms / 1e9
    dq_gbps = dequant_bytes_8b(L, synth) / deq_ms / 1e6
    dq_layer_gbps = dequant_bytes_8b(L, synth) / deq_layer_ms / 1e6
    traffic = recorded_traffic()
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "t": L["t"], "hidden": 4096, "intermediate": 12288, "qtypes": ["Q6_K", "Q2_K"],
                   "projections": 14},
        "mfma_frac": round(tflops / PEAK_F16_TFLOPS, 4),
        "gemm_ms_per_step": round(gemm_ms, 4),
        "dequant_gbps": round(dq_gbps, 1),
        "dequant_hbm_frac": round(dq_gbps / PEAK_HBM_GBPS, 4),
        "dequant_ms_per_step": round(deq_ms, 4),
        "dequant_by_type": deq_rows,
        "dequant_in_layer_gbps": round(dq_layer_gbps, 1),
        "roofline": {
            "kernel": DOMINANT,
            "bound": "mfma",
            "achieved": round(dom_flops / dom_ms / 1e9, 2),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dom_flops / dom_ms / 1e9 / PEAK_F16_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_launch": dom_flops,
            "avg_launch_us": round(dom_ms * 1e3, 2),
        },
    }
    print("bench: dequant as one graph", file=sys.stderr, flush=True)
    dq_graph = dequant_graph_gbps(torch, qp, L, synth)
    res["dequant_graph_gbps"] = round(dq_graph, 1)
    res["dequant_graph_hbm_frac"] = round(dq_graph / PEAK_HBM_GBPS, 4)
    two_pass = None
    if not args.no_rows and not args.no_two_pass:
        print("bench: f16-cache comparator", file=sys.stderr, flush=True)
        two_pass = two_pass_row(torch, synth, qp, L, 10)
    del L
    torch.cuda.empty_cache()
    if not args.no_rows:
        print("bench: other workloads", file=sys.stderr, flush=True)
        which = [g for g in args.rows.split(",") if g]
        unknown = set(which) - set(ROW_GROUPS)
        if unknown:
            print(f"bench.py: unknown row groups {sorted(unknown)}", file=sys.stderr)
            sys.exit(2)
        rows = other_rows(torch, synth, qp, 10, which)
        if two_pass is not None:
            rows["two_pass_f16_cache_q6_k_qwen3_8b_t2048"] = two_pass
        res["rows"] = {k: {kk: round(vv, 2) for kk, vv in v.items()} for k, v in rows.items()}
    if not args.no_cpu:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(synth, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
