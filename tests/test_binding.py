"""Host-side checks of the Python binding (no GPU): the cached workspaces are
kept per stream, and undersized or mistyped tensors are refused before any
library call."""
import pytest
import torch

import quantized_prefill_amd as qp


def test_workspace_cache_keyed_by_stream():
    n, k, t = 1024, 4096, 64
    assert qp.lib().qp_prefill_gemm_workspace_bytes(n, k, t) > 0
    a1 = qp.gemm_workspace(n, k, t, "cpu", stream=1)
    b1 = qp.gemm_workspace(n, k, t, "cpu", stream=2)
    a2 = qp.gemm_workspace(n, k, t, "cpu", stream=1)
    assert a1 is a2, "one stream reuses its buffer"
    assert a1 is not b1 and a1.data_ptr() != b1.data_ptr(), "two streams never share a buffer"
    # a larger request replaces only that stream's buffer
    big = qp.gemm_workspace(4096, 4096, 64, "cpu", stream=2)
    assert big.numel() >= qp.lib().qp_prefill_gemm_workspace_bytes(4096, 4096, 64)
    assert qp.gemm_workspace(n, k, t, "cpu", stream=1) is a1
    q1 = qp.qkv_workspace(4096, 1024, 1024, 2048, "cpu", stream=1)
    q2 = qp.qkv_workspace(4096, 1024, 1024, 2048, "cpu", stream=3)
    assert q1 is not q2 and qp.qkv_workspace(4096, 1024, 1024, 2048, "cpu", stream=1) is q1
    assert qp._workspace_key("cpu", 5) != qp._workspace_key("cpu", 6)


def _w(qtype, rows, cols, short=0):
    return torch.zeros(rows * qp.row_bytes(qtype, cols) - short, dtype=torch.uint8)


def test_dequant_size_checks():
    with pytest.raises(ValueError, match="w holds"):
        qp.dequant_f32(qp.Q6_K, _w(qp.Q6_K, 2, 256, short=1), 2, 256, out=torch.empty(2, 256))
    with pytest.raises(ValueError, match="out holds"):
        qp.dequant_f32(qp.Q6_K, _w(qp.Q6_K, 2, 256), 2, 256, out=torch.empty(2, 255))
    with pytest.raises(TypeError):
        qp.dequant_f32(qp.Q6_K, _w(qp.Q6_K, 2, 256), 2, 256, out=torch.empty(2, 256, dtype=torch.float64))
    with pytest.raises(ValueError, match="out holds"):
        qp.dequant_f16(qp.Q2_K, _w(qp.Q2_K, 3, 512), 3, 512, out=torch.empty(3, 511, dtype=torch.float16))
    # right sizes: refused only for not being on the GPU
    with pytest.raises(ValueError, match="GPU tensor"):
        qp.dequant_f32(qp.Q6_K, _w(qp.Q6_K, 2, 256), 2, 256, out=torch.empty(2, 256))


def test_gemm_size_checks():
    x = torch.zeros(4, 256, dtype=torch.float16)
    y = torch.zeros(4, 512)
    with pytest.raises(ValueError, match="w holds"):
        qp.prefill_gemm(qp.Q4_K, _w(qp.Q4_K, 512, 256, short=144), 512, 256, x, out=y, workspace=False)
    with pytest.raises(ValueError, match="x is"):
        qp.prefill_gemm(qp.Q4_K, _w(qp.Q4_K, 512, 512), 512, 512, x, out=y, workspace=False)
    with pytest.raises(ValueError, match="out is"):
        qp.prefill_gemm(qp.Q4_K, _w(qp.Q4_K, 512, 256), 512, 256, x, out=torch.zeros(3, 512), workspace=False)
    with pytest.raises(TypeError):
        qp.prefill_gemm(qp.Q4_K, _w(qp.Q4_K, 512, 256), 512, 256, x, out=torch.zeros(4, 512, dtype=torch.float16),
                        workspace=False)
    with pytest.raises(ValueError, match="workspace holds"):
        qp.prefill_gemm(qp.Q4_K, _w(qp.Q4_K, 1024, 4096), 1024, 4096, torch.zeros(64, 4096, dtype=torch.float16),
                        out=torch.zeros(64, 1024), workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU tensor"):
        qp.prefill_gemm(qp.Q4_K, _w(qp.Q4_K, 512, 256), 512, 256, x, out=y, workspace=False)
    with pytest.raises(ValueError, match="out_up holds|out_up is"):
        qp.prefill_gemm_gate_up(qp.Q6_K, _w(qp.Q6_K, 512, 256), _w(qp.Q6_K, 512, 256), 512, 256, x, out_gate=y,
                                out_up=torch.zeros(4, 100))
    # per-head gains: 4 heads of 128 with a per-head stride need 512 floats
    with pytest.raises(ValueError, match="gain holds"):
        qp.prefill_gemm_qknorm(qp.Q4_K, _w(qp.Q4_K, 512, 256), 512, 256, x, 128, torch.ones(511), 128, out=y)
    with pytest.raises(ValueError, match="GPU tensor"):
        qp.prefill_gemm_qknorm(qp.Q4_K, _w(qp.Q4_K, 512, 256), 512, 256, x, 128, torch.ones(512), 128, out=y)
    with pytest.raises(ValueError, match="gain_k holds"):
        qp.prefill_gemm_qkv(qp.Q4_K, _w(qp.Q4_K, 512, 256), 512, _w(qp.Q4_K, 256, 256), 256, None, 0, 256, x, 128,
                            torch.ones(128), torch.ones(200), 0, 128, out_q=y, out_k=torch.zeros(4, 256),
                            workspace=False)


def test_moe_and_attention_size_checks():
    t, top_k, ne, hidden, inter = 8, 2, 4, 256, 256
    x = torch.zeros(t, hidden, dtype=torch.float16)
    ids = torch.zeros(t, top_k, dtype=torch.int32)
    wts = torch.zeros(t, top_k)
    ws = torch.zeros(qp.grouped_expert_workspace_bytes(t, top_k, ne, hidden, inter), dtype=torch.uint8)
    good = _w(qp.Q4_K, ne * inter, hidden)
    with pytest.raises(ValueError, match="w_down holds"):
        qp.grouped_expert_gemm(qp.Q4_K, good, good, _w(qp.Q4_K, ne * hidden, inter, short=1), ne, hidden, inter, x,
                               ids, wts, out=torch.zeros(t, hidden), workspace=ws)
    with pytest.raises(ValueError, match="workspace holds"):
        qp.grouped_expert_gemm(qp.Q4_K, good, good, good, ne, hidden, inter, x, ids, wts, out=torch.zeros(t, hidden),
                               workspace=ws[:-1])
    with pytest.raises(TypeError):
        qp.grouped_expert_gemm(qp.Q4_K, good, good, good, ne, hidden, inter, x, ids.long(), wts,
                               out=torch.zeros(t, hidden), workspace=ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        qp.grouped_expert_gemm(qp.Q4_K, good, good, good, ne, hidden, inter, x, ids, wts, out=torch.zeros(t, hidden),
                               workspace=ws)
    # attention: a Q8_0 cache of n_past + t tokens x 2 kv heads x 128 values
    q = torch.zeros(t, 4 * 128)
    need = (3 + t) * 2 * qp.row_bytes(qp.Q8_0, 128)
    kc = torch.zeros(need, dtype=torch.uint8)
    with pytest.raises(ValueError, match="v_cache holds"):
        qp.prompt_attention(qp.Q8_0, q, kc, kc[:-2], 3, 4, 2, out=torch.zeros(t, 512))
    with pytest.raises(ValueError, match="out is"):
        qp.prompt_attention(qp.Q8_0, q, kc, kc, 3, 4, 2, out=torch.zeros(t, 500))
    with pytest.raises(ValueError, match="GPU tensor"):
        qp.prompt_attention(qp.Q8_0, q, kc, kc, 3, 4, 2, out=torch.zeros(t, 512))
