"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/qprefill.h declares, answers the size queries, and rejects bad
arguments before launching anything (no call here reaches a kernel)."""
import os
import re

import pytest

import quantized_prefill_amd as qp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qprefill.h")

pytestmark = pytest.mark.skipif(not os.path.exists(qp.LIB_PATH), reason="libqprefill.so not built")

FAKE = 1 << 20  # a non-null, 256-byte aligned stand-in address; never dereferenced


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qp_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 12
    L = qp.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(qp.SIGNATURES), "binding and header disagree"


def test_geometry():
    assert [qp.block_size(t) for t in (qp.F16W, qp.Q8_0, qp.Q4_K, qp.Q5_K, qp.Q6_K, qp.Q2_K)] == [1, 32, 256, 256, 256,
                                                                                                256]
    assert [qp.type_size(t) for t in (qp.F16W, qp.Q8_0, qp.Q4_K, qp.Q5_K, qp.Q6_K, qp.Q2_K)] == [2, 34, 144, 176, 210,
                                                                                               84]
    assert qp.row_bytes(qp.Q6_K, 4173) == 17 * 210
    assert qp.row_bytes(qp.Q8_0, 33) == 2 * 34
    assert qp.block_size(3) == -1 and qp.row_bytes(qp.Q4_K, 0) == -1
    assert qp.block_size(qp.Q4_0) == 32 and qp.type_size(qp.Q4_0) == 18 and qp.row_bytes(qp.Q4_0, 128) == 4 * 18


def status_name(s):
    return qp.lib().qp_status_string(s).decode()


def test_status_strings():
    assert [status_name(i) for i in range(5)] == [qp.STATUS[i] for i in range(5)]


def test_dequant_rejections():
    L = qp.lib()
    assert L.qp_dequant_f32(2, FAKE, 4, 256, FAKE, None) == 2          # Q4_0: a KV cache format only
    assert b"no dequant kernel" in L.qp_last_error_detail()
    assert L.qp_dequant_f32(qp.Q4_K, FAKE, -1, 256, FAKE, None) == 1
    assert L.qp_dequant_f32(qp.Q4_K, FAKE, 4, 0, FAKE, None) == 1
    assert L.qp_dequant_f16(qp.Q4_K, None, 4, 256, FAKE, None) == 1
    assert L.qp_dequant_f16(qp.Q4_K, FAKE + 2, 4, 256, FAKE, None) == 1  # src not 16-byte aligned
    assert L.qp_dequant_f32(qp.Q4_K, FAKE, 4, 256, FAKE + 2, None) == 1  # dst not 4-byte aligned
    assert L.qp_dequant_f32(qp.Q4_K, None, 0, 256, None, None) == 0      # rows == 0: nothing to do


def test_gemm_rejections():
    L = qp.lib()
    g = L.qp_prefill_gemm
    assert g(7, FAKE, 64, 256, FAKE, qp.F16, 8, 256, FAKE, 64, None) == 2
    assert g(qp.Q8_0, FAKE, 64, 96, FAKE, qp.F16, 8, 96, FAKE, 64, None) == 1      # k % 256
    assert g(qp.Q4_K, FAKE, 64, 256, FAKE, 3, 8, 256, FAKE, 64, None) == 1        # x dtype
    assert g(qp.Q4_K, FAKE, 64, 256, FAKE, qp.F16, 8, 128, FAKE, 64, None) == 1   # ldx < k
    assert g(qp.Q4_K, FAKE, 64, 256, FAKE, qp.F16, 8, 256, FAKE, 32, None) == 1   # ldy < n
    assert g(qp.Q4_K, FAKE, 64, 256, FAKE, qp.F16, 8, 260, FAKE, 64, None) == 1   # ldx*2 % 16
    assert g(qp.Q4_K, FAKE + 8, 64, 256, FAKE, qp.F16, 8, 256, FAKE, 64, None) == 1
    assert g(qp.Q4_K, FAKE, 64, 256, FAKE, qp.F16, 0, 256, FAKE, 64, None) == 0   # t == 0
    q = L.qp_prefill_gemm_qknorm
    assert q(qp.Q4_K, FAKE, 256, 256, FAKE, 8, 256, 96, FAKE, 0, 1e-6, FAKE, 256, None) == 1   # head_dim
    assert q(qp.Q4_K, FAKE, 192, 256, FAKE, 8, 256, 128, FAKE, 0, 1e-6, FAKE, 192, None) == 1  # n % hd
    assert q(qp.Q4_K, FAKE, 256, 256, FAKE, 8, 256, 128, FAKE, 0, 0.0, FAKE, 256, None) == 1   # eps
    assert q(qp.Q4_K, FAKE, 256, 256, FAKE, 8, 256, 128, None, 0, 1e-6, FAKE, 256, None) == 1  # gain
    # head_dim 256 is accepted (t == 0: validated, nothing to launch); 192 and 512 are not
    assert q(qp.Q4_K, FAKE, 512, 256, FAKE, 0, 256, 256, FAKE, 256, 1e-6, FAKE, 512, None) == 0
    assert q(qp.Q4_K, FAKE, 768, 256, FAKE, 8, 256, 192, FAKE, 0, 1e-6, FAKE, 768, None) == 1
    assert q(qp.Q4_K, FAKE, 512, 256, FAKE, 8, 256, 512, FAKE, 0, 1e-6, FAKE, 512, None) == 1
    assert q(qp.Q4_K, FAKE, 384, 256, FAKE, 8, 256, 256, FAKE, 0, 1e-6, FAKE, 384, None) == 1  # n % 256
    # the K-split variant: same checks, plus its workspace
    gw = L.qp_prefill_gemm_ws
    assert gw(qp.Q4_K, FAKE, 64, 256, FAKE, qp.F16, 8, 128, FAKE, 64, None, 0, None) == 1   # ldx < k
    assert L.qp_prefill_gemm_workspace_bytes(0, 256, 8) == 0
    need = L.qp_prefill_gemm_workspace_bytes(128, 2048, 128)    # one tile: split into 8 parts of 256
    assert need == 8 * 128 * 128 * 4
    assert L.qp_prefill_gemm_workspace_bytes(128, 256, 128) == 0  # one 256-weight block: nothing to split
    assert gw(qp.Q4_K, FAKE, 128, 2048, FAKE, qp.F16, 128, 2048, FAKE, 128, FAKE, need - 16, None) == 3
    assert gw(qp.Q4_K, FAKE, 128, 2048, FAKE, qp.F16, 128, 2048, FAKE, 128, FAKE + 4, need, None) == 1
    f = L.qp_prefill_gemm_qkv
    good = [qp.Q4_K, FAKE, 256, FAKE, 128, FAKE, 128, 256, FAKE, 8, 256, 128, FAKE, 0, FAKE, 0, 1e-6,
            FAKE, 256, FAKE, 128, FAKE, 128, None, 0, None]
    assert f(*(good[:9] + [0] + good[10:])) == 0                  # t == 0: nothing to do
    hd256 = list(good)
    hd256[2], hd256[4], hd256[6], hd256[9], hd256[11] = 512, 256, 256, 0, 256
    hd256[18], hd256[20], hd256[22] = 512, 256, 256
    assert f(*hd256) == 0                                         # head_dim 256 accepted
    hd256[4] = 128
    assert f(*hd256) == 1                                         # n_k not a multiple of 256
    need = L.qp_prefill_gemm_qkv_workspace_bytes(256, 128, 128, 8)
    assert need == 2 * 8 * 256 * 4                                # partial sums of k and v, two halves
    assert L.qp_prefill_gemm_qkv_workspace_bytes(256, -1, 128, 8) == 0
    assert f(*(good[:23] + [FAKE, need - 4] + good[25:])) == 3    # workspace below the query
    assert f(*(good[:23] + [FAKE + 4, need] + good[25:])) == 1    # workspace misaligned
    for i, v, why in ((0, 7, "type"), (2, 192, "n_q % hd"), (4, 64, "n_k % hd"), (6, -1, "n_v"), (7, 96, "k"),
                      (11, 96, "head_dim"), (16, 0.0, "eps"), (12, None, "gain_q"), (14, None, "gain_k"),
                      (20, 64, "ldy_k < n_k"), (22, 64, "ldy_v < n_v")):
        bad = list(good)
        bad[i] = v
        want = 2 if why == "type" else 1
        assert f(*bad) == want, why


def test_moe_rejections():
    L = qp.lib()
    assert L.qp_moe_route_topk(FAKE, 4, 2000, 8, 0, FAKE, FAKE, None) == 1
    assert L.qp_moe_route_topk(FAKE, 4, 128, 0, 0, FAKE, FAKE, None) == 1
    ws = qp.grouped_expert_workspace_bytes(4096, 8, 128, 2048, 768)
    assert ws > 4096 * 8 * (2048 + 768) * 4
    assert qp.grouped_expert_workspace_bytes(4096, 0, 128, 2048, 768) == 0
    f = L.qp_grouped_expert_gemm
    args = [qp.Q4_K, FAKE, FAKE, FAKE, 128, 2048, 768, FAKE, 4096, 8, FAKE, FAKE, FAKE, FAKE]
    assert f(*args, ws - 1, None) == 3
    assert b"workspace" in L.qp_last_error_detail()
    bad = list(args)
    bad[6] = 700  # inter not a multiple of 256
    assert f(*bad, ws, None) == 1
    bad = list(args)
    bad[0] = 3
    assert f(*bad, ws, None) == 2
    # the dropped-pair reader: pointers checked before any copy is enqueued
    d = L.qp_grouped_expert_dropped_pairs
    assert d(None, FAKE, None) == 1
    assert d(FAKE, None, None) == 1
    assert d(FAKE + 16, FAKE, None) == 1      # workspace not 256-byte aligned
    assert d(FAKE, FAKE + 2, None) == 1       # count not 4-byte aligned


def test_attention_rejections():
    L = qp.lib()
    A = L.qp_prompt_attention
    # kv_type, q, ldq, k, v, n_past, t, n_head, n_kv, head_dim, scale, out, ldo, stream
    good = [qp.F16W, FAKE, 4096, FAKE, FAKE, 0, 8, 32, 8, 128, 0.088, FAKE, 4096, None]

    def call(**kw):
        a = list(good)
        names = ["kv", "q", "ldq", "k", "v", "n_past", "t", "n_head", "n_kv", "hd", "scale", "out", "ldo", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return A(*a)

    assert call(kv=qp.Q4_K) == 2
    assert b"KV cache" in L.qp_last_error_detail()
    assert call(hd=64) == 1
    assert call(n_kv=5) == 1            # 32 heads do not split into 5 groups
    assert call(n_head=0) == 1
    assert call(t=-1) == 1
    assert call(n_past=-3) == 1
    assert call(n_past=(1 << 31)) == 1
    assert call(t=(1 << 30), n_head=1024, n_kv=8, ldq=1 << 17, ldo=1 << 17) == 1   # grid beyond 2^32 threads
    assert b"grid too large" in L.qp_last_error_detail()
    assert call(ldq=4095) == 1          # below n_head * head_dim
    assert call(ldo=4098) == 1          # not a multiple of 4
    assert call(scale=float("inf")) == 1
    assert call(scale=float("nan")) == 1
    assert call(scale=0.0, t=0, q=None, k=None, v=None, out=None) == 0   # 0: the default 1/sqrt(head_dim)
    assert call(t=0, q=None, k=None, v=None, out=None) == 0   # empty chunk: nothing to do
    assert call(q=None) == 1
    assert call(q=FAKE + 4) == 1        # q not 16-byte aligned
    assert call(k=FAKE + 2) == 1        # binary16 cache not 16-byte aligned
    assert call(kv=qp.Q4_0, k=FAKE + 1) == 1   # Q4_0 cache on an odd byte
    assert call(out=FAKE + 8) == 1


def test_noalloc_rejections():
    """The allocation-free projection validates like qp_prefill_gemm, before
    anything is launched (t == 0 is a no-op that touches no device)."""
    L = qp.lib()
    assert L.qp_prefill_gemm_noalloc(2, FAKE, 64, 256, FAKE, qp.F16, 8, 256, FAKE, 64, None) == 2
    assert L.qp_prefill_gemm_noalloc(qp.Q4_K, FAKE, 64, 300, FAKE, qp.F16, 8, 304, FAKE, 64, None) == 1
    assert L.qp_prefill_gemm_noalloc(qp.Q4_K, FAKE, 64, 256, FAKE, 7, 8, 256, FAKE, 64, None) == 1
    assert L.qp_prefill_gemm_noalloc(qp.Q4_K, FAKE, 64, 256, FAKE + 8, qp.F16, 8, 256, FAKE, 64, None) == 1
    assert L.qp_prefill_gemm_noalloc(qp.Q4_K, FAKE, 64, 256, FAKE, qp.F16, 0, 256, FAKE, 64, None) == 0


def test_rope_and_kv_write_rejections():
    L = qp.lib()
    r = L.qp_rope
    # x, ldx, t, n_head, head_dim, pos0, base, stream
    assert r(FAKE, 4096, 8, 32, 127, 0, 1e6, None) == 1           # odd head_dim
    assert r(FAKE, 4095, 8, 32, 128, 0, 1e6, None) == 1           # ldx below the heads
    assert r(FAKE, 4096, 8, 32, 128, -1, 1e6, None) == 1          # negative position
    assert r(FAKE, 4096, 8, 32, 128, 0, 1.0, None) == 1           # base not > 1
    assert r(FAKE, 4096, 8, 32, 128, 0, float("inf"), None) == 1
    assert r(None, 4096, 8, 32, 128, 0, 1e6, None) == 1
    assert r(FAKE + 2, 4096, 8, 32, 128, 0, 1e6, None) == 1       # not 4-byte aligned
    assert r(None, 4096, 0, 32, 128, 0, 1e6, None) == 0           # t == 0: nothing to do
    w = L.qp_kv_cache_write
    # kv_type, src, lds, t, n_kv, head_dim, cache, row0, stream
    assert w(qp.Q4_K, FAKE, 1024, 8, 8, 128, FAKE, 0, None) == 2  # not a cache format
    assert w(qp.Q8_0, FAKE, 1024, 8, 8, 96 + 8, FAKE, 0, None) == 1   # head_dim % 32
    assert w(qp.Q8_0, FAKE, 1020, 8, 8, 128, FAKE, 0, None) == 1  # lds below the heads
    assert w(qp.Q8_0, FAKE, 1026, 8, 8, 128, FAKE, 0, None) == 1  # lds not a multiple of 4
    assert w(qp.Q8_0, FAKE, 1024, 8, 8, 128, FAKE, -1, None) == 1
    assert w(qp.Q8_0, FAKE + 4, 1024, 8, 8, 128, FAKE, 0, None) == 1  # src not 16-byte aligned
    assert w(qp.Q8_0, FAKE, 1024, 8, 8, 128, FAKE + 1, 0, None) == 1  # cache on an odd byte
    assert w(qp.F16W, FAKE, 1024, 8, 8, 128, FAKE + 2, 0, None) == 1  # binary16 cache needs 4 bytes
    assert w(qp.Q4_0, None, 1024, 0, 8, 128, None, 0, None) == 0  # t == 0



def test_attention_workspace_query_and_rejections():
    """qp_prompt_attention_workspace_bytes: two binary16 copies of the cache
    for Q8_0 and Q4_0, 0 otherwise; qp_prompt_attention_ws rejects a short or
    misaligned workspace before any launch."""
    L = qp.lib()
    q = L.qp_prompt_attention_workspace_bytes
    assert q(qp.Q8_0, 2048, 8, 128) == 2 * 2048 * 8 * 128 * 2
    assert q(qp.Q4_0, 1, 1, 128) == 2 * 256
    assert q(qp.F16W, 2048, 8, 128) == 0
    assert q(qp.Q8_0, 2048, 8, 64) == 0
    assert q(qp.Q8_0, 0, 8, 128) == 0
    assert q(qp.Q8_0, 16, 0, 128) == 0
    A = L.qp_prompt_attention_ws
    need = q(qp.Q8_0, 8, 8, 128)
    args = [qp.Q8_0, FAKE, 4096, FAKE, FAKE, 0, 8, 32, 8, 128, 0.0, FAKE, 4096]
    assert A(*args, FAKE, need - 1, None) == 3   # QP_ERR_WORKSPACE_TOO_SMALL
    assert b"workspace" in L.qp_last_error_detail()
    assert A(*args, FAKE + 8, need, None) == 1   # not 16-byte aligned
    assert A(*(args[:6] + [0] + args[7:]), None, 0, None) == 0   # empty chunk: nothing to do
