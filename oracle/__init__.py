"""CPU oracle for the quantized prefill path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package.  The product library never links, loads or calls it; the
two share no code.  This file is argument marshalling (numpy <-> ctypes) for
`oracle.c`, which holds every step of the arithmetic.

Every output buffer handed to the C code carries a guard band of NaN-patterned
elements on both sides; `dequant_f32` / `dequant_f16` check the bands after the
call, so an out-of-bounds write is reported, never silently absorbed.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .build import library_path, build as _build

HERE = os.path.dirname(os.path.abspath(__file__))

F32 = 0
F16 = 1

GUARD = 256
GUARD_F32 = np.uint32(0x7FC0DEAD)
GUARD_F16 = np.uint16(0x7E01)


class OutOfBoundsWrite(AssertionError):
    pass


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


class Oracle:
    """ctypes view of one build of liboracle (the default one or a planted one)."""

    def __init__(self, path: str | None = None):
        path = path or library_path()
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library not built: {path}")
        self.path = path
        L = C.CDLL(path)
        self._L = L
        i64, vp, i32, dbl = C.c_int64, C.c_void_p, C.c_int, C.c_double
        L.or_half_to_double.argtypes = [C.c_uint16]
        L.or_half_to_double.restype = dbl
        L.or_half_to_float.argtypes = [C.c_uint16]
        L.or_half_to_float.restype = C.c_float
        L.or_float_to_half.argtypes = [C.c_float]
        L.or_float_to_half.restype = C.c_uint16
        L.or_half_to_float_array.argtypes = [vp, vp, i64]
        L.or_half_to_float_array.restype = None
        L.or_float_to_half_array.argtypes = [vp, vp, i64]
        L.or_float_to_half_array.restype = None
        for f in ("or_block_size", "or_type_size"):
            getattr(L, f).argtypes = [i32]
            getattr(L, f).restype = i64
        L.or_row_bytes.argtypes = [i32, i64]
        L.or_row_bytes.restype = i64
        L.or_dequant_f32.argtypes = [i32, vp, i64, i64, vp]
        L.or_dequant_f32.restype = i32
        L.or_dequant_f16.argtypes = [i32, vp, i64, i64, vp]
        L.or_dequant_f16.restype = i32
        L.or_prefill_gemm.argtypes = [i32, vp, i64, i64, vp, i32, i64, vp, i64, vp]
        L.or_prefill_gemm.restype = i32
        L.or_qknorm.argtypes = [vp, i64, i64, i64, vp, i64, dbl]
        L.or_qknorm.restype = i32
        L.or_route_topk.argtypes = [vp, i64, i64, i64, i32, vp, vp]
        L.or_route_topk.restype = i32
        L.or_moe.argtypes = [i32, vp, vp, vp, i64, i64, i64, vp, i64, i64, vp, vp, vp, i64, vp]
        L.or_moe.restype = i32
        L.or_attention.argtypes = [i32, vp, i64, vp, vp, i64, i64, i64, i64, i64, dbl, vp, i64, vp]
        L.or_attention.restype = i32
        L.or_rope.argtypes = [vp, i64, i64, i64, i64, i64, dbl]
        L.or_rope.restype = i32
        L.or_kv_quantize.argtypes = [i32, vp, i64, i64, i64, i64, vp]
        L.or_kv_quantize.restype = i32
        L.or_plant.restype = i32
        L.or_plant_count.restype = i32
        L.or_plant_name.argtypes = [i32]
        L.or_plant_name.restype = C.c_char_p
        L.or_num_threads.restype = i32
        L.or_set_num_threads.argtypes = [i32]
        L.or_set_num_threads.restype = None

    # -- small helpers -----------------------------------------------------
    @property
    def plant(self) -> int:
        return self._L.or_plant()

    def plant_names(self) -> list[str]:
        return [self._L.or_plant_name(i).decode() for i in range(self._L.or_plant_count())]

    def num_threads(self) -> int:
        return self._L.or_num_threads()

    def set_num_threads(self, n: int) -> None:
        """Threads of the oracle's parallel loops from now on (timing only)."""
        self._L.or_set_num_threads(int(n))

    def block_size(self, qtype: int) -> int:
        return self._L.or_block_size(qtype)

    def type_size(self, qtype: int) -> int:
        return self._L.or_type_size(qtype)

    def row_bytes(self, qtype: int, cols: int) -> int:
        return self._L.or_row_bytes(qtype, cols)

    def half_to_double(self, h: int) -> float:
        return self._L.or_half_to_double(int(h))

    def float_to_half(self, f: float) -> int:
        return self._L.or_float_to_half(float(np.float32(f)))

    def half_to_float_array(self, bits: np.ndarray) -> np.ndarray:
        src = np.ascontiguousarray(bits, dtype=np.uint16)
        dst = np.empty(src.shape, dtype=np.float32)
        self._L.or_half_to_float_array(_p(src), _p(dst), src.size)
        return dst

    def float_to_half_array(self, vals: np.ndarray) -> np.ndarray:
        src = np.ascontiguousarray(vals, dtype=np.float32)
        dst = np.empty(src.shape, dtype=np.uint16)
        self._L.or_float_to_half_array(_p(src), _p(dst), src.size)
        return dst

    # -- dequant -----------------------------------------------------------
    def _dequant(self, fn, fill, dtype, qtype, src, rows, cols):
        src = np.ascontiguousarray(src, dtype=np.uint8)
        buf = np.full(rows * cols + 2 * GUARD, fill, dtype=fill.dtype)
        rc = fn(qtype, _p(src), rows, cols, _p(buf[GUARD:]))
        if rc != 0:
            raise ValueError(f"oracle dequant rejected qtype={qtype} rows={rows} cols={cols}")
        if not (np.all(buf[:GUARD] == fill) and np.all(buf[GUARD + rows * cols:] == fill)):
            raise OutOfBoundsWrite("oracle dequant wrote outside rows x cols")
        return buf[GUARD:GUARD + rows * cols].view(dtype).reshape(rows, cols).copy()

    def dequant_f32(self, qtype, src, rows, cols) -> np.ndarray:
        return self._dequant(self._L.or_dequant_f32, GUARD_F32, np.float32, qtype, src, rows, cols)

    def dequant_f16_bits(self, qtype, src, rows, cols) -> np.ndarray:
        return self._dequant(self._L.or_dequant_f16, GUARD_F16, np.uint16, qtype, src, rows, cols)

    # -- GEMM / QK norm ----------------------------------------------------
    def prefill_gemm(self, qtype, w, n, k, x, tokens=None) -> np.ndarray:
        """float64 [len(tokens), n]; x is float32 [T, K] or uint16 binary16 bits [T, K]."""
        w = np.ascontiguousarray(w, dtype=np.uint8)
        if x.dtype == np.float32:
            xd = F32
        elif x.dtype == np.uint16:
            xd = F16
        else:
            raise TypeError("x must be float32 or uint16 (binary16 bits)")
        x = np.ascontiguousarray(x)
        t = x.shape[0]
        tok = np.arange(t, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
        y = np.empty((tok.size, n), dtype=np.float64)
        rc = self._L.or_prefill_gemm(qtype, _p(w), n, k, _p(x), xd, x.shape[1], _p(tok), tok.size, _p(y))
        if rc != 0:
            raise ValueError("oracle prefill_gemm rejected its arguments")
        return y

    def qknorm(self, y: np.ndarray, head_dim: int, gain: np.ndarray, gain_head_stride: int = 0,
               eps: float = 1e-6) -> np.ndarray:
        out = np.array(y, dtype=np.float64, copy=True, order="C")
        g = np.ascontiguousarray(gain, dtype=np.float32)
        rc = self._L.or_qknorm(_p(out), out.shape[0], out.shape[1], head_dim, _p(g), gain_head_stride,
                               float(eps))
        if rc != 0:
            raise ValueError("oracle qknorm rejected its arguments")
        return out

    def prefill_gemm_qknorm(self, qtype, w, n, k, x, head_dim, gain, gain_head_stride=0, eps=1e-6,
                            tokens=None) -> np.ndarray:
        return self.qknorm(self.prefill_gemm(qtype, w, n, k, x, tokens), head_dim, gain,
                           gain_head_stride, eps)

    # -- routed experts ----------------------------------------------------
    def route_topk(self, logits: np.ndarray, top_k: int, renorm: bool = False):
        lg = np.ascontiguousarray(logits, dtype=np.float32)
        t, e = lg.shape
        ids = np.empty((t, top_k), dtype=np.int32)
        wts = np.empty((t, top_k), dtype=np.float64)
        rc = self._L.or_route_topk(_p(lg), t, e, top_k, int(bool(renorm)), _p(ids), _p(wts))
        if rc != 0:
            raise ValueError("oracle route_topk rejected its arguments")
        return ids, wts

    def moe(self, qtype, wg, wu, wd, n_experts, hidden, inter, x, ids, weights, tokens=None):
        x = np.ascontiguousarray(x, dtype=np.uint16)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        weights = np.ascontiguousarray(weights, dtype=np.float64)
        t, top_k = ids.shape
        tok = np.arange(t, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
        out = np.empty((tok.size, hidden), dtype=np.float64)
        wg, wu, wd = (np.ascontiguousarray(a, dtype=np.uint8) for a in (wg, wu, wd))
        rc = self._L.or_moe(qtype, _p(wg), _p(wu), _p(wd), n_experts, hidden, inter, _p(x), x.shape[1],
                            top_k, _p(ids), _p(weights), _p(tok), tok.size, _p(out))
        if rc != 0:
            raise ValueError("oracle moe rejected its arguments")
        return out

    # -- prompt attention --------------------------------------------------
    def attention(self, kvtype, q, k_cache, v_cache, n_past, n_head, n_kv, head_dim, scale=None,
                  tokens=None) -> np.ndarray:
        """float64 [len(tokens), n_head * head_dim]; q is float32 [T, >= n_head*head_dim];
        the caches are flat uint8 arrays of (n_past + T) * n_kv rows of head_dim weights."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        t = q.shape[0]
        if scale is None:
            scale = 1.0 / np.sqrt(head_dim)
        kc = np.ascontiguousarray(k_cache, dtype=np.uint8).reshape(-1)
        vc = np.ascontiguousarray(v_cache, dtype=np.uint8).reshape(-1)
        need = (n_past + t) * n_kv * self.row_bytes(kvtype, head_dim)
        if kc.size < need or vc.size < need:
            raise ValueError(f"KV cache holds {min(kc.size, vc.size)} bytes, needs {need}")
        tok = np.arange(t, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
        out = np.empty((tok.size, n_head * head_dim), dtype=np.float64)
        rc = self._L.or_attention(kvtype, _p(q), q.shape[1], _p(kc), _p(vc), n_past, t, n_head, n_kv, head_dim,
                                  float(scale), _p(tok), tok.size, _p(out))
        if rc != 0:
            raise ValueError("oracle attention rejected its arguments")
        return out

    # -- rotary step and KV cache rows --------------------------------------
    def rope(self, x: np.ndarray, n_head: int, head_dim: int, pos0: int, base: float) -> np.ndarray:
        """float32 copy of x [T, >= n_head*head_dim] with each head of row i
        rotated to position pos0 + i (half-split pairs, binary64 angles)."""
        y = np.array(x, dtype=np.float32, order="C", copy=True)
        if y.ndim != 2:
            raise ValueError("x must be 2-D")
        rc = self._L.or_rope(_p(y), y.shape[1], y.shape[0], n_head, head_dim, pos0, float(base))
        if rc != 0:
            raise ValueError("oracle rope rejected its arguments")
        return y

    def kv_quantize(self, kvtype: int, src: np.ndarray, n_kv: int, head_dim: int) -> np.ndarray:
        """Cache rows (flat uint8, token-major then kv head) of src [T, >= n_kv*head_dim] f32."""
        x = np.ascontiguousarray(src, dtype=np.float32)
        if x.ndim != 2:
            raise ValueError("src must be 2-D")
        t = x.shape[0]
        rb = self.row_bytes(kvtype, head_dim)
        if rb <= 0:
            raise ValueError("unsupported cache type")
        out = np.zeros(t * n_kv * rb, dtype=np.uint8)
        rc = self._L.or_kv_quantize(kvtype, _p(x), x.shape[1], t, n_kv, head_dim, _p(out))
        if rc != 0:
            raise ValueError("oracle kv_quantize rejected its arguments")
        return out


_default: Oracle | None = None


def get() -> Oracle:
    """The default (unplanted) oracle, built on first use if needed."""
    global _default
    if _default is None:
        if not os.path.exists(library_path()):
            _build()
        _default = Oracle()
    return _default
