"""Python binding of libqprefill (include/qprefill.h): argument marshalling only.

Every step of the path runs in the HIP library; torch supplies device memory
and the current stream.  If the library is not built, or a tensor is not on
the GPU, the call raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqprefill.so")

F16W, Q8_0, Q2_K, Q4_K, Q5_K, Q6_K = 1, 8, 10, 12, 13, 14
Q4_0 = 2  # KV cache format of prompt_attention only
F32, F16 = 0, 1

STATUS = {0: "QP_OK", 1: "QP_ERR_INVALID_PARAMETER", 2: "QP_ERR_UNSUPPORTED_TYPE",
          3: "QP_ERR_WORKSPACE_TOO_SMALL", 4: "QP_ERR_DEVICE"}

# name -> (restype, argtypes) for every entry point of include/qprefill.h
_VP, _I64, _INT, _F32C, _SZ = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t
SIGNATURES = {
    "qp_block_size": (_I64, [_INT]),
    "qp_type_size": (_I64, [_INT]),
    "qp_row_bytes": (_I64, [_INT, _I64]),
    "qp_dequant_f32": (_INT, [_INT, _VP, _I64, _I64, _VP, _VP]),
    "qp_dequant_f16": (_INT, [_INT, _VP, _I64, _I64, _VP, _VP]),
    "qp_prefill_gemm": (_INT, [_INT, _VP, _I64, _I64, _VP, _INT, _I64, _I64, _VP, _I64, _VP]),
    "qp_prefill_gemm_ws": (_INT, [_INT, _VP, _I64, _I64, _VP, _INT, _I64, _I64, _VP, _I64, _VP, _SZ, _VP]),
    "qp_prefill_gemm_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "qp_prefill_gemm_noalloc": (_INT, [_INT, _VP, _I64, _I64, _VP, _INT, _I64, _I64, _VP, _I64, _VP]),
    "qp_prefill_gemm_gate_up": (_INT, [_INT, _VP, _VP, _I64, _I64, _VP, _I64, _I64, _VP, _I64, _VP, _I64, _VP]),
    "qp_prefill_gemm_qknorm": (_INT, [_INT, _VP, _I64, _I64, _VP, _I64, _I64, _I64, _VP, _I64, _F32C, _VP, _I64,
                                      _VP]),
    "qp_prefill_gemm_qkv": (_INT, [_INT, _VP, _I64, _VP, _I64, _VP, _I64, _I64, _VP, _I64, _I64, _I64, _VP, _I64,
                                   _VP, _I64, _F32C, _VP, _I64, _VP, _I64, _VP, _I64, _VP, _SZ, _VP]),
    "qp_prefill_gemm_qkv_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64]),
    "qp_moe_route_topk": (_INT, [_VP, _I64, _I64, _I64, _INT, _VP, _VP, _VP]),
    "qp_grouped_expert_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64]),
    "qp_grouped_expert_gemm": (_INT, [_INT, _VP, _VP, _VP, _I64, _I64, _I64, _VP, _I64, _I64, _VP, _VP, _VP, _VP,
                                      _SZ, _VP]),
    "qp_grouped_expert_dropped_pairs": (_INT, [_VP, _VP, _VP]),
    "qp_rope": (_INT, [_VP, _I64, _I64, _I64, _I64, _I64, C.c_double, _VP]),
    "qp_kv_cache_write": (_INT, [_INT, _VP, _I64, _I64, _I64, _I64, _VP, _I64, _VP]),
    "qp_prompt_attention": (_INT, [_INT, _VP, _I64, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _F32C, _VP, _I64, _VP]),
    "qp_prompt_attention_workspace_bytes": (_SZ, [_INT, _I64, _I64, _I64]),
    "qp_prompt_attention_ws": (_INT, [_INT, _VP, _I64, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _F32C, _VP, _I64, _VP,
                                      _SZ, _VP]),
    "qp_status_string": (C.c_char_p, [_INT]),
    "qp_last_error_detail": (C.c_char_p, []),
}


class QPError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib() -> C.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libqprefill.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != 0:
        raise QPError(status, lib().qp_last_error_detail().decode())


def block_size(qtype: int) -> int:
    return lib().qp_block_size(qtype)


def type_size(qtype: int) -> int:
    return lib().qp_type_size(qtype)


def row_bytes(qtype: int, cols: int) -> int:
    return lib().qp_row_bytes(qtype, cols)


# ---------------------------------------------------------------------------
# torch-facing calls

def _torch():
    import torch
    return torch


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _gpu(*named):
    """Raise unless every (tensor, name) is on the GPU (there is no CPU path)."""
    for t, name in named:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _need_bytes(t, nbytes: int, name: str) -> None:
    """Raise before any launch if tensor t holds fewer than nbytes bytes."""
    if _nbytes(t) < nbytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, the call reads or writes {nbytes}")


def _need_dtype(t, dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _need_rows(t, rows: int, cols: int, name: str) -> None:
    """A 2-D tensor with unit column stride covering rows x cols elements."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} is {tuple(t.shape)}, the call needs at least ({rows}, {cols})")


def _weights_bytes(qtype: int, rows: int, cols: int) -> int:
    rb = row_bytes(qtype, cols)
    if rb < 0:
        raise ValueError(f"type {qtype} has no block layout here")
    return rows * rb


def dequant_f32(qtype: int, w, rows: int, cols: int, out=None):
    torch = _torch()
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=w.device)
    if qtype in _BLOCK_TYPES and rows > 0 and cols > 0:
        _need_bytes(w, _weights_bytes(qtype, rows, cols), "w")
        _need_dtype(out, torch.float32, "out")
        _need_bytes(out, 4 * rows * cols, "out")
    check(lib().qp_dequant_f32(qtype, _dev(w, "w"), rows, cols, _dev(out, "out"), _stream()))
    return out


def dequant_f16(qtype: int, w, rows: int, cols: int, out=None):
    torch = _torch()
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float16, device=w.device)
    if qtype in _BLOCK_TYPES and rows > 0 and cols > 0:
        _need_bytes(w, _weights_bytes(qtype, rows, cols), "w")
        if out.element_size() != 2:
            raise TypeError("out must hold 2-byte elements (binary16 bit patterns)")
        _need_bytes(out, 2 * rows * cols, "out")
    check(lib().qp_dequant_f16(qtype, _dev(w, "w"), rows, cols, _dev(out, "out"), _stream()))
    return out


_BLOCK_TYPES = (F16W, Q8_0, Q2_K, Q4_K, Q5_K, Q6_K)

# Cached workspaces, one per (device, stream): calls on one stream run in
# order, so they may share a buffer; calls on two streams may overlap and
# get one each.  A buffer replaced by a larger one is released by the
# caching allocator only after the work already queued on its stream.
_GEMM_WORKSPACE = {}
_QKV_WORKSPACE = {}
_ATTN_WORKSPACE = {}


def _workspace_key(device, stream: int):
    return (_torch().device(device).index, int(stream or 0))


def _cached_workspace(cache: dict, nbytes: int, device, stream=None):
    torch = _torch()
    key = _workspace_key(device, _stream() if stream is None else stream)
    ws = cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        cache[key] = ws
    return ws


def gemm_workspace(n: int, k: int, t: int, device, stream=None):
    """Workspace for prefill_gemm's K split (None when it would not split),
    kept per device and stream (the current one by default) and grown as
    needed."""
    nbytes = lib().qp_prefill_gemm_workspace_bytes(n, k, t)
    if nbytes == 0:
        return None
    return _cached_workspace(_GEMM_WORKSPACE, nbytes, device, stream)


def _check_gemm_args(qtype: int, w, n: int, k: int, x, t: int, out, out_name="out"):
    torch = _torch()
    if qtype in _BLOCK_TYPES and n > 0 and k > 0:
        _need_bytes(w, _weights_bytes(qtype, n, k), "w")
    if t > 0:
        _need_rows(x, t, k, "x")
        _need_dtype(out, torch.float32, out_name)
        _need_rows(out, t, n, out_name)


def prefill_gemm(qtype: int, w, n: int, k: int, x, out=None, workspace=None):
    """y = x . W^T; x is [T, K] float16 or float32 (rows may be strided).
    workspace: a uint8 GPU tensor, None for the cached one (gemm_workspace),
    or False for none (qp_prefill_gemm exactly)."""
    torch = _torch()
    t = x.shape[0]
    if x.dtype == torch.float16:
        xd = F16
    elif x.dtype == torch.float32:
        xd = F32
    else:
        raise TypeError("x must be float16 or float32")
    if out is None:
        out = torch.empty((t, n), dtype=torch.float32, device=x.device)
    _check_gemm_args(qtype, w, n, k, x, t, out)
    ws = gemm_workspace(n, k, t, x.device) if workspace is None else (None if workspace is False else workspace)
    if ws is not None:
        _need_bytes(ws, lib().qp_prefill_gemm_workspace_bytes(n, k, t), "workspace")
    _gpu((x, "x"), (out, "out"))
    check(lib().qp_prefill_gemm_ws(qtype, _dev(w, "w"), n, k, x.data_ptr(), xd, t, x.stride(0), out.data_ptr(),
                                   out.stride(0), _dev(ws, "workspace") if ws is not None else None,
                                   ws.numel() if ws is not None else 0, _stream()))
    return out


# bytes of the library's static scratch behind prefill_gemm_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20


def prefill_gemm_noalloc(qtype: int, w, n: int, k: int, x, out):
    """y = x . W^T through qp_prefill_gemm_noalloc: the K split of prefill_gemm
    with its partial sums in the library's static device scratch, so the call
    allocates nothing (out must be given).  Calls on one GPU share that
    scratch and must not overlap."""
    torch = _torch()
    if x.dtype == torch.float16:
        xd = F16
    elif x.dtype == torch.float32:
        xd = F32
    else:
        raise TypeError("x must be float16 or float32")
    t = x.shape[0]
    _check_gemm_args(qtype, w, n, k, x, t, out)
    _gpu((x, "x"), (out, "out"))
    check(lib().qp_prefill_gemm_noalloc(qtype, _dev(w, "w"), n, k, x.data_ptr(), xd, t, x.stride(0),
                                        out.data_ptr(), out.stride(0), _stream()))
    return out


def prefill_gemm_gate_up(qtype: int, w_gate, w_up, n: int, k: int, x, out_gate=None, out_up=None):
    """The gate and up projections (each [T, n] f32) of one float16 x in one call."""
    torch = _torch()
    if x.dtype != torch.float16:
        raise TypeError("x must be float16")
    t = x.shape[0]
    if out_gate is None:
        out_gate = torch.empty((t, n), dtype=torch.float32, device=x.device)
    if out_up is None:
        out_up = torch.empty((t, n), dtype=torch.float32, device=x.device)
    _check_gemm_args(qtype, w_gate, n, k, x, t, out_gate, "out_gate")
    _check_gemm_args(qtype, w_up, n, k, x, t, out_up, "out_up")
    _gpu((x, "x"), (out_gate, "out_gate"), (out_up, "out_up"))
    check(lib().qp_prefill_gemm_gate_up(qtype, _dev(w_gate, "w_gate"), _dev(w_up, "w_up"), n, k, x.data_ptr(), t,
                                        x.stride(0), out_gate.data_ptr(), out_gate.stride(0), out_up.data_ptr(),
                                        out_up.stride(0), _stream()))
    return out_gate, out_up


def prefill_gemm_qknorm(qtype: int, w, n: int, k: int, x, head_dim: int, gain, gain_head_stride: int = 0,
                        eps: float = 1e-6, out=None):
    torch = _torch()
    if x.dtype != torch.float16:
        raise TypeError("x must be float16")
    t = x.shape[0]
    if out is None:
        out = torch.empty((t, n), dtype=torch.float32, device=x.device)
    _check_gemm_args(qtype, w, n, k, x, t, out)
    _check_gain(gain, n, head_dim, gain_head_stride, "gain")
    _gpu((x, "x"), (out, "out"))
    check(lib().qp_prefill_gemm_qknorm(qtype, _dev(w, "w"), n, k, x.data_ptr(), t, x.stride(0), head_dim,
                                       _dev(gain, "gain"), gain_head_stride, float(eps), out.data_ptr(),
                                       out.stride(0), _stream()))
    return out


def _check_gain(gain, n: int, head_dim: int, stride: int, name: str) -> None:
    """The f32 gains the norm reads: head h at h * stride, head_dim values."""
    torch = _torch()
    if head_dim > 0 and n >= head_dim and stride >= 0:
        _need_dtype(gain, torch.float32, name)
        _need_bytes(gain, 4 * ((n // head_dim - 1) * stride + head_dim), name)


def qkv_workspace(n_q: int, n_k: int, n_v: int, t: int, device, stream=None):
    """Workspace for prefill_gemm_qkv, kept per device and stream (the current
    one by default) and grown as needed."""
    nbytes = lib().qp_prefill_gemm_qkv_workspace_bytes(n_q, n_k, n_v, t)
    return _cached_workspace(_QKV_WORKSPACE, max(nbytes, 256), device, stream)


def prefill_gemm_qkv(qtype: int, w_q, n_q: int, w_k, n_k: int, w_v, n_v: int, k: int, x, head_dim: int,
                     gain_q, gain_k, gain_q_stride: int = 0, gain_k_stride: int = 0, eps: float = 1e-6,
                     out_q=None, out_k=None, out_v=None, workspace=None):
    """q and k with the per-head RMSNorm, v plain, over one float16 x, in one call.
    workspace: a uint8 GPU tensor, None for the cached one (qkv_workspace), or
    False for none (no K split)."""
    torch = _torch()
    if x.dtype != torch.float16:
        raise TypeError("x must be float16")
    t = x.shape[0]
    if workspace is None:
        ws = qkv_workspace(n_q, n_k, n_v, t, x.device)
    else:
        ws = None if workspace is False else workspace
    outs = []
    for o, n in ((out_q, n_q), (out_k, n_k), (out_v, n_v)):
        outs.append(o if o is not None else torch.empty((t, max(n, 1)), dtype=torch.float32, device=x.device))
    _check_gemm_args(qtype, w_q, n_q, k, x, t, outs[0], "out_q")
    _check_gemm_args(qtype, w_k, n_k, k, x, t, outs[1], "out_k")
    if n_v:
        _check_gemm_args(qtype, w_v, n_v, k, x, t, outs[2], "out_v")
    _check_gain(gain_q, n_q, head_dim, gain_q_stride, "gain_q")
    _check_gain(gain_k, n_k, head_dim, gain_k_stride, "gain_k")
    if ws is not None:
        _need_bytes(ws, lib().qp_prefill_gemm_qkv_workspace_bytes(n_q, n_k, n_v, t), "workspace")
    _gpu((x, "x"), *((o, "out") for o in outs))
    check(lib().qp_prefill_gemm_qkv(qtype, _dev(w_q, "w_q"), n_q, _dev(w_k, "w_k"), n_k,
                                    _dev(w_v, "w_v") if n_v else None, n_v, k, x.data_ptr(), t, x.stride(0),
                                    head_dim, _dev(gain_q, "gain_q"), gain_q_stride, _dev(gain_k, "gain_k"),
                                    gain_k_stride, float(eps), outs[0].data_ptr(), outs[0].stride(0),
                                    outs[1].data_ptr(), outs[1].stride(0), outs[2].data_ptr(), outs[2].stride(0),
                                    _dev(ws, "workspace") if ws is not None else None,
                                    ws.numel() if ws is not None else 0, _stream()))
    return tuple(outs)


def moe_route_topk(logits, top_k: int, renorm: bool = False, ids=None, weights=None):
    torch = _torch()
    t, e = logits.shape
    if ids is None:
        ids = torch.empty((t, top_k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((t, top_k), dtype=torch.float32, device=logits.device)
    _need_dtype(logits, torch.float32, "logits")
    _need_dtype(ids, torch.int32, "ids")
    _need_dtype(weights, torch.float32, "weights")
    _need_bytes(ids, 4 * t * top_k, "ids")
    _need_bytes(weights, 4 * t * top_k, "weights")
    check(lib().qp_moe_route_topk(_dev(logits, "logits"), t, e, top_k, int(bool(renorm)), _dev(ids, "ids"),
                                  _dev(weights, "weights"), _stream()))
    return ids, weights


def grouped_expert_workspace_bytes(t: int, top_k: int, n_experts: int, hidden: int, inter: int) -> int:
    return lib().qp_grouped_expert_workspace_bytes(t, top_k, n_experts, hidden, inter)


def grouped_expert_gemm(qtype: int, w_gate, w_up, w_down, n_experts: int, hidden: int, inter: int, x, ids, weights,
                        out=None, workspace=None):
    torch = _torch()
    t, top_k = ids.shape
    if out is None:
        out = torch.empty((t, hidden), dtype=torch.float32, device=x.device)
    nbytes = grouped_expert_workspace_bytes(t, top_k, n_experts, hidden, inter)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    if t > 0 and qtype in _BLOCK_TYPES:
        _need_bytes(w_gate, n_experts * _weights_bytes(qtype, inter, hidden), "w_gate")
        _need_bytes(w_up, n_experts * _weights_bytes(qtype, inter, hidden), "w_up")
        _need_bytes(w_down, n_experts * _weights_bytes(qtype, hidden, inter), "w_down")
        _need_dtype(x, torch.float16, "x")
        _need_bytes(x, 2 * t * hidden, "x")
        _need_dtype(ids, torch.int32, "ids")
        _need_dtype(weights, torch.float32, "weights")
        _need_bytes(weights, 4 * t * top_k, "weights")
        _need_dtype(out, torch.float32, "out")
        _need_bytes(out, 4 * t * hidden, "out")
        _need_bytes(workspace, nbytes, "workspace")
    check(lib().qp_grouped_expert_gemm(qtype, _dev(w_gate, "w_gate"), _dev(w_up, "w_up"), _dev(w_down, "w_down"),
                                       n_experts, hidden, inter, _dev(x, "x"), t, top_k, _dev(ids, "ids"),
                                       _dev(weights, "weights"), _dev(out, "out"), _dev(workspace, "workspace"),
                                       workspace.numel(), _stream()))
    return out


def grouped_expert_dropped_pairs(workspace) -> int:
    """Pairs the last grouped_expert_gemm call with this workspace dropped for
    an expert id outside [0, n_experts) (synchronizes with the current stream)."""
    torch = _torch()
    cnt = torch.zeros(1, dtype=torch.int32, device=workspace.device)
    check(lib().qp_grouped_expert_dropped_pairs(_dev(workspace, "workspace"), cnt.data_ptr(), _stream()))
    return int(cnt.item())


def rope(x, n_head: int, head_dim: int, pos0: int, base: float = 1e6):
    """Rotary step, in place, on x [T, >= n_head*head_dim] float32 (row i at
    position pos0 + i); returns x."""
    torch = _torch()
    t = x.shape[0]
    _need_dtype(x, torch.float32, "x")
    _need_rows(x, t, n_head * head_dim, "x")
    _gpu((x, "x"))
    check(lib().qp_rope(x.data_ptr(), x.stride(0), t, n_head, head_dim, pos0, float(base), _stream()))
    return x


def kv_cache_write(kv_type: int, src, n_kv_head: int, head_dim: int, cache, row0: int):
    """Write src [T, >= n_kv_head*head_dim] float32 (K or V rows of a chunk)
    into cache (flat uint8) at token rows row0 .. row0 + T - 1."""
    torch = _torch()
    t = src.shape[0]
    _need_dtype(src, torch.float32, "src")
    _need_rows(src, t, n_kv_head * head_dim, "src")
    rb = row_bytes(kv_type, head_dim)
    if t > 0 and rb > 0:
        _need_bytes(cache, (row0 + t) * n_kv_head * rb, "cache")
    _gpu((src, "src"), (cache, "cache"))
    check(lib().qp_kv_cache_write(kv_type, src.data_ptr(), src.stride(0), t, n_kv_head, head_dim, cache.data_ptr(),
                                  row0, _stream()))
    return cache


def attention_workspace(kv_type: int, kv_len: int, n_kv_head: int, head_dim: int, device, stream=None):
    """Workspace for prompt_attention over a Q8_0 or Q4_0 cache of kv_len
    tokens (None for a binary16 cache), kept per device and stream and grown
    as needed."""
    nbytes = lib().qp_prompt_attention_workspace_bytes(kv_type, kv_len, n_kv_head, head_dim)
    if nbytes == 0:
        return None
    return _cached_workspace(_ATTN_WORKSPACE, nbytes, device, stream)


def prompt_attention(kv_type: int, q, k_cache, v_cache, n_past: int, n_head: int, n_kv_head: int,
                     head_dim: int = 128, scale: float | None = None, out=None, workspace=None):
    """Causal prompt attention of a chunk of q.shape[0] queries over a KV cache of
    n_past + q.shape[0] tokens (flat byte tensors of binary16, Q8_0 or Q4_0 rows).
    scale None takes the library's default, 1 / sqrt(head_dim).  workspace: a
    uint8 GPU tensor, None for the cached one (attention_workspace: a quantized
    cache is decoded to binary16 rows once per call), or False for none (the
    kernel decodes as it stages; the output is the same bit for bit)."""
    torch = _torch()
    t = q.shape[0]
    if scale is None:
        scale = 0.0  # the library's default
    if out is None:
        out = torch.empty((t, n_head * head_dim), dtype=torch.float32, device=q.device)
    if t > 0:
        _need_dtype(q, torch.float32, "q")
        _need_rows(q, t, n_head * head_dim, "q")
        _need_dtype(out, torch.float32, "out")
        _need_rows(out, t, n_head * head_dim, "out")
        kv_bytes = (n_past + t) * n_kv_head * row_bytes(kv_type, head_dim) if row_bytes(kv_type, head_dim) > 0 else 0
        _need_bytes(k_cache, kv_bytes, "k_cache")
        _need_bytes(v_cache, kv_bytes, "v_cache")
    ptrs = (_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(out, "out"))
    ws = None
    if t > 0 and workspace is not False:
        ws = attention_workspace(kv_type, n_past + t, n_kv_head, head_dim, q.device) if workspace is None else workspace
        if ws is not None:
            _need_bytes(ws, lib().qp_prompt_attention_workspace_bytes(kv_type, n_past + t, n_kv_head, head_dim),
                        "workspace")
    check(lib().qp_prompt_attention_ws(kv_type, ptrs[0], q.stride(0), ptrs[1], ptrs[2], n_past, t, n_head, n_kv_head,
                                       head_dim, float(scale), ptrs[3], out.stride(0),
                                       _dev(ws, "workspace") if ws is not None else None,
                                       ws.numel() if ws is not None else 0, _stream()))
    return out
