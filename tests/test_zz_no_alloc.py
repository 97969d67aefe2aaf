"""qp_prefill_gemm_noalloc (the allocation-free K split) against
qp_prefill_gemm_ws with a caller workspace: identical bits, and within the
GEMM tolerance of the binary64 oracle, on two calls in a row, the second one
smaller.  Run alone and after the other GPU tests."""
import numpy as np
import pytest

import synth
import quantized_prefill_amd as qp
from gpu_helpers import assert_close, act_f16, say, to_dev, weights
from synth import Q4_K, Q6_K, Q8_0

pytestmark = pytest.mark.gpu


def _pair(orc, qtype, t, n, k, f32_x, seed):
    import torch
    say(f"noalloc {synth.NAMES[qtype]} t={t} n={n} k={k} f32_x={f32_x}")
    raw = weights(qtype, n, k, seed)
    x = synth.activations_f32(t, k, seed + 1) if f32_x else act_f16(t, k, seed + 1)
    w = to_dev(raw)
    xt = to_dev(x) if f32_x else to_dev(x).view(torch.float16)
    nbytes = qp.lib().qp_prefill_gemm_workspace_bytes(n, k, t)
    assert 0 < nbytes <= qp.NOALLOC_SCRATCH_BYTES, "this shape should split within the static scratch"
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y_ws = qp.prefill_gemm(qtype, w, n, k, xt, workspace=ws)
    y_na = torch.full((t, n), float("nan"), device="cuda")
    qp.prefill_gemm_noalloc(qtype, w, n, k, xt, y_na)
    torch.cuda.synchronize()
    y_ws, y_na = y_ws.cpu().numpy(), y_na.cpu().numpy()
    assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32)), "noalloc differs from the workspace call"
    assert_close(y_na, orc.prefill_gemm(qtype, raw, n, k, x), f"noalloc {synth.NAMES[qtype]} {t}x{n}x{k}")


def test_noalloc_two_calls_second_smaller(orc):
    # 8 tiles of 128 x 128 -> 8 K parts; then 2 x 3 tiles of a smaller ragged shape
    _pair(orc, Q8_0, 64, 1024, 1024, True, 9100)
    _pair(orc, Q4_K, 200, 300, 512, False, 9200)


def test_noalloc_unsplit_and_rejections(orc):
    import torch
    # a launch that fills the GPU (32 x 8 tiles of 128 x 128) does not split:
    # the same as qp_prefill_gemm
    t, n, k = 1024, 4096, 512
    raw = weights(Q6_K, n, k, 9300)
    x = act_f16(t, k, 9301)
    w, xt = to_dev(raw), to_dev(x).view(torch.float16)
    y = torch.empty((t, n), device="cuda")
    qp.prefill_gemm_noalloc(Q6_K, w, n, k, xt, y)
    y_ref = qp.prefill_gemm(Q6_K, w, n, k, xt, workspace=False)
    torch.cuda.synchronize()
    assert qp.lib().qp_prefill_gemm_workspace_bytes(n, k, t) == 0, "this shape fills the GPU: no split"
    assert np.array_equal(y.cpu().numpy(), y_ref.cpu().numpy())
    rows = np.array([0, 127, 128, 511, 640, 1023])
    assert_close(y.cpu().numpy()[rows], orc.prefill_gemm(Q6_K, raw, n, k, x, tokens=rows), "noalloc unsplit")
    # validation happens before any launch
    st = qp.lib().qp_prefill_gemm_noalloc(Q6_K, w.data_ptr(), n, 1000, xt.data_ptr(), qp.F16, t, k, y.data_ptr(), n,
                                          None)
    assert st == 1
