"""CPU oracle for the INT4 weight-only decode GEMV (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It loads ``liboracle_w4.so``, built from
``w4_oracle.c`` with gcc, and shares no code with the HIP library.

Definitions (restated from the pages: "How To Build Your Own LLM Runtime From
Scratch", aitrending.vip, "Technical Details" bullet 1 -- INT4 weights
dequantized at run time; noticiai.com.br, "As tres licoes", lesson 3 -- the
activations stay floating point; zero point 8 and one fp16 scale per group of G
inputs per row are the workload definition's format, the pages being silent):

    w[n, k] = (q[n, k] - 8) * s[n, k // G]
    y[n]    = sum_k w[n, k] * x[k]          (fp64, exact products)
    Y[m, n] = sum_k X[m, k] * w[n, k]       (prefill: one y per token row)
    o[h, :] = softmax_t(scale q[h] . K[t, g(h)]) V[t, g(h)]   (decode attention, paged KV)
    A[n]    = sum_k |w[n, k] * x[k]|
    h[j]    = silu(y[j]) * y[I + j],  silu(t) = t / (1 + exp(-t))
    argmax  = lowest index of max y
    W4A8:   c[k] = rint(x[k] * 127 / amax_g), s_g = amax_g / 127 (binary32),
            y[n] = sum_k w[n, k] * c[k] * s_g
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_w4.so")


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                           "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one build of the oracle library (the default build, or a
    mutated copy compiled by the self-tests)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_packed_weight_bytes.restype = i64
        lib.oracle_packed_weight_bytes.argtypes = [i64, i64, i32]
        lib.oracle_packed_scale_bytes.restype = i64
        lib.oracle_packed_scale_bytes.argtypes = [i64, i64, i32, i32]
        lib.oracle_pack.restype = ctypes.c_int
        lib.oracle_pack.argtypes = [p, p, i64, i64, i32, i32, p, p]
        lib.oracle_unpack.restype = ctypes.c_int
        lib.oracle_unpack.argtypes = [p, p, i64, i64, i32, i32, p, p]
        lib.oracle_gemv_rows.restype = None
        lib.oracle_gemv_rows.argtypes = [p, p, p, i64, i64, i32, p, i64, p, p]
        lib.oracle_gemv.restype = None
        lib.oracle_gemv.argtypes = [p, p, p, i64, i64, i32, p, p]
        lib.oracle_gemv_packed_rows.restype = None
        lib.oracle_gemv_packed_rows.argtypes = [p, p, p, i64, i64, i32, i32, p, i64, p, p]
        lib.oracle_gemm.restype = None
        lib.oracle_gemm.argtypes = [p, p, p, i64, i64, i64, i32, p, p]
        lib.oracle_gemm_packed.restype = None
        lib.oracle_gemm_packed.argtypes = [p, p, p, i64, i64, i32, i32, p, i64, p, i64, p, p]
        lib.oracle_attn_decode.restype = None
        lib.oracle_attn_decode.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, ctypes.c_double, p, p]
        lib.oracle_rmsnorm.restype = None
        lib.oracle_rmsnorm.argtypes = [p, i64, p, ctypes.c_double, p]
        lib.oracle_rmsnorm_given.restype = None
        lib.oracle_rmsnorm_given.argtypes = [p, i64, p, ctypes.c_double, ctypes.c_double, p]
        lib.oracle_sumsq_blocks.restype = None
        lib.oracle_sumsq_blocks.argtypes = [p, i64, i64, p]
        lib.oracle_rope.restype = None
        lib.oracle_rope.argtypes = [p, i32, i64, ctypes.c_double, p]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu_gate.restype = None
        lib.oracle_silu_gate.argtypes = [p, i64, p]
        lib.oracle_argmax.restype = i64
        lib.oracle_argmax.argtypes = [p, i64]
        lib.oracle_quantize_act8.restype = None
        lib.oracle_quantize_act8.argtypes = [p, i64, i32, p, p]
        lib.oracle_act8_block_order.restype = None
        lib.oracle_act8_block_order.argtypes = [p, i64, p]
        lib.oracle_gemv_a8_rows.restype = None
        lib.oracle_gemv_a8_rows.argtypes = [p, p, p, p, i64, i64, i32, p, i64, p, p]
        lib.oracle_gemv_a8_packed_rows.restype = None
        lib.oracle_gemv_a8_packed_rows.argtypes = [p, p, p, p, i64, i64, i32, i32, p, i64, p, p]
        self.lib = lib
        self.path = path

    def half_to_double(self, bits: int) -> float:
        return self.lib.oracle_half_to_double(int(bits) & 0xFFFF)

    def packed_sizes(self, n: int, k: int, group: int, gateup: bool = False) -> tuple[int, int]:
        return (int(self.lib.oracle_packed_weight_bytes(n, k, int(gateup))),
                int(self.lib.oracle_packed_scale_bytes(n, k, group, int(gateup))))

    def pack(self, q: np.ndarray, s_bits: np.ndarray, group: int, gateup: bool = False):
        """Logical q uint8 [n, k], s fp16 bits uint16 [n, k/group] -> (pw, ps) uint8."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s_bits = np.ascontiguousarray(s_bits, dtype=np.uint16)
        n, k = q.shape
        assert s_bits.shape == (n, k // group)
        wb, sb = self.packed_sizes(n, k, group, gateup)
        pw = np.empty(wb, np.uint8)
        ps = np.empty(sb, np.uint8)
        rc = self.lib.oracle_pack(_ptr(q), _ptr(s_bits), n, k, group, int(gateup), _ptr(pw), _ptr(ps))
        if rc != 0:
            raise ValueError("oracle_pack: shape not representable")
        return pw, ps

    def unpack(self, pw: np.ndarray, ps: np.ndarray, n: int, k: int, group: int,
               gateup: bool = False):
        """Packed buffers -> logical (q uint8 [n, k], s bits uint16 [n, k/group])."""
        pw = np.ascontiguousarray(pw, dtype=np.uint8)
        ps = np.ascontiguousarray(ps, dtype=np.uint8)
        wb, sb = self.packed_sizes(n, k, group, gateup)
        if pw.size < wb or ps.size < sb:
            raise ValueError("oracle.unpack: packed buffers too small")
        q = np.empty((n, k), np.uint8)
        s = np.empty((n, k // group), np.uint16)
        rc = self.lib.oracle_unpack(_ptr(pw), _ptr(ps), n, k, group, int(gateup), _ptr(q), _ptr(s))
        if rc != 0:
            raise ValueError("oracle_unpack: shape not representable")
        return q, s

    def gemv(self, q: np.ndarray, s_bits: np.ndarray, x_bits: np.ndarray, group: int, rows=None):
        """(y, A) in float64 for all rows, or for the listed rows."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s_bits = np.ascontiguousarray(s_bits, dtype=np.uint16)
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        n, k = q.shape
        assert s_bits.shape == (n, k // group) and x_bits.shape == (k,)
        if rows is None:
            y = np.empty(n, np.float64)
            a = np.empty(n, np.float64)
            self.lib.oracle_gemv(_ptr(q), _ptr(s_bits), _ptr(x_bits), n, k, group, _ptr(y), _ptr(a))
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            assert rows.size == 0 or (rows.min() >= 0 and rows.max() < n)
            y = np.empty(rows.size, np.float64)
            a = np.empty(rows.size, np.float64)
            self.lib.oracle_gemv_rows(_ptr(q), _ptr(s_bits), _ptr(x_bits), n, k, group,
                                      _ptr(rows), rows.size, _ptr(y), _ptr(a))
        return y, a

    def gemv_packed(self, pw: np.ndarray, ps: np.ndarray, x_bits: np.ndarray, n: int, k: int,
                    group: int, gateup: bool = False, rows=None):
        """(y, A) for the listed rows (default: all), reading the packed buffers."""
        pw = np.ascontiguousarray(pw, dtype=np.uint8)
        ps = np.ascontiguousarray(ps, dtype=np.uint8)
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        wb, sb = self.packed_sizes(n, k, group, gateup)
        assert pw.size >= wb and ps.size >= sb and x_bits.shape == (k,)
        if rows is None:
            rows = np.arange(n, dtype=np.int64)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < n)
        y = np.empty(rows.size, np.float64)
        a = np.empty(rows.size, np.float64)
        self.lib.oracle_gemv_packed_rows(_ptr(pw), _ptr(ps), _ptr(x_bits), n, k, group,
                                         int(gateup), _ptr(rows), rows.size, _ptr(y), _ptr(a))
        return y, a

    def gemm(self, q: np.ndarray, s_bits: np.ndarray, xm_bits: np.ndarray, group: int):
        """Prefill product: (Y, A) float64 [m, n] for token rows xm_bits [m, k]."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s_bits = np.ascontiguousarray(s_bits, dtype=np.uint16)
        xm_bits = np.ascontiguousarray(xm_bits, dtype=np.uint16)
        n, k = q.shape
        m = xm_bits.shape[0]
        assert s_bits.shape == (n, k // group) and xm_bits.shape == (m, k)
        y = np.empty((m, n), np.float64)
        a = np.empty((m, n), np.float64)
        self.lib.oracle_gemm(_ptr(q), _ptr(s_bits), _ptr(xm_bits), m, n, k, group, _ptr(y), _ptr(a))
        return y, a

    def gemm_packed(self, pw: np.ndarray, ps: np.ndarray, xm_bits: np.ndarray, n: int, k: int,
                    group: int, gateup: bool = False, mrows=None, ncols=None):
        """(Y, A) float64 [len(mrows), len(ncols)] from the packed buffers;
        defaults: every token row, every weight row."""
        pw = np.ascontiguousarray(pw, dtype=np.uint8)
        ps = np.ascontiguousarray(ps, dtype=np.uint8)
        xm_bits = np.ascontiguousarray(xm_bits, dtype=np.uint16)
        wb, sb = self.packed_sizes(n, k, group, gateup)
        assert pw.size >= wb and ps.size >= sb and xm_bits.ndim == 2 and xm_bits.shape[1] == k
        mt = xm_bits.shape[0]
        mrows = np.arange(mt, dtype=np.int64) if mrows is None else np.ascontiguousarray(mrows, dtype=np.int64)
        ncols = np.arange(n, dtype=np.int64) if ncols is None else np.ascontiguousarray(ncols, dtype=np.int64)
        assert mrows.size == 0 or (mrows.min() >= 0 and mrows.max() < mt)
        assert ncols.size == 0 or (ncols.min() >= 0 and ncols.max() < n)
        y = np.empty((mrows.size, ncols.size), np.float64)
        a = np.empty((mrows.size, ncols.size), np.float64)
        self.lib.oracle_gemm_packed(_ptr(pw), _ptr(ps), _ptr(xm_bits), n, k, group, int(gateup),
                                    _ptr(mrows), mrows.size, _ptr(ncols), ncols.size, _ptr(y), _ptr(a))
        return y, a

    def attn_decode(self, q_bits: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                    page_table: np.ndarray, ctx: int, n_kv: int, page: int, scale: float):
        """(o, A) float64 [n_heads, dim]: softmax(scale * q K^T) V of one token
        over the first ctx cached tokens; caches fp16 bits
        [num_pages, n_kv, page, dim], q fp16 bits [n_heads, dim]."""
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        k_cache = np.ascontiguousarray(k_cache, dtype=np.uint16)
        v_cache = np.ascontiguousarray(v_cache, dtype=np.uint16)
        page_table = np.ascontiguousarray(page_table, dtype=np.int32)
        n_heads, dim = q_bits.shape
        assert k_cache.shape == v_cache.shape and k_cache.shape[1:] == (n_kv, page, dim)
        assert n_heads % n_kv == 0 and 1 <= ctx <= page_table.size * page
        assert page_table[: (ctx + page - 1) // page].max() < k_cache.shape[0]
        o = np.empty((n_heads, dim), np.float64)
        a = np.empty((n_heads, dim), np.float64)
        self.lib.oracle_attn_decode(_ptr(q_bits), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), ctx, n_heads,
                                    n_kv, dim, page, float(scale), _ptr(o), _ptr(a))
        return o, a

    def rmsnorm(self, h: np.ndarray, gamma_bits: np.ndarray, eps: float) -> np.ndarray:
        """h / sqrt(mean(h^2) + eps) * gamma in float64 (h any float array)."""
        h = np.ascontiguousarray(h, dtype=np.float64)
        gamma_bits = np.ascontiguousarray(gamma_bits, dtype=np.uint16)
        assert gamma_bits.shape == h.shape and h.ndim == 1
        out = np.empty_like(h)
        self.lib.oracle_rmsnorm(_ptr(h), h.size, _ptr(gamma_bits), float(eps), _ptr(out))
        return out

    def rmsnorm_given(self, h: np.ndarray, gamma_bits: np.ndarray, sumsq: float, eps: float) -> np.ndarray:
        """h / sqrt(sumsq / n + eps) * gamma in float64, the sum of squares given."""
        h = np.ascontiguousarray(h, dtype=np.float64)
        gamma_bits = np.ascontiguousarray(gamma_bits, dtype=np.uint16)
        assert gamma_bits.shape == h.shape and h.ndim == 1
        out = np.empty_like(h)
        self.lib.oracle_rmsnorm_given(_ptr(h), h.size, _ptr(gamma_bits), float(sumsq), float(eps), _ptr(out))
        return out

    def sumsq_blocks(self, h: np.ndarray, rows: int) -> np.ndarray:
        """Sums of h^2 over consecutive blocks of `rows` values (the last may be short)."""
        h = np.ascontiguousarray(h, dtype=np.float64)
        assert h.ndim == 1 and rows >= 1
        out = np.empty((h.size + rows - 1) // rows, np.float64)
        self.lib.oracle_sumsq_blocks(_ptr(h), h.size, int(rows), _ptr(out))
        return out

    def rope(self, x: np.ndarray, pos: int, theta: float) -> np.ndarray:
        """Rotary embedding of each row of x [heads, dim] at position pos."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty_like(x)
        for r in range(x.shape[0]):
            self.lib.oracle_rope(_ptr(x[r]), x.shape[1], int(pos), float(theta), _ptr(out[r]))
        return out

    def silu(self, t: float) -> float:
        return self.lib.oracle_silu(float(t))

    def silu_gate(self, y: np.ndarray) -> np.ndarray:
        y = np.ascontiguousarray(y, dtype=np.float64)
        assert y.size % 2 == 0
        half = y.size // 2
        h = np.empty(half, np.float64)
        self.lib.oracle_silu_gate(_ptr(y), half, _ptr(h))
        return h

    def argmax(self, y: np.ndarray) -> int:
        y = np.ascontiguousarray(y, dtype=np.float64)
        return int(self.lib.oracle_argmax(_ptr(y), y.size))

    def quantize_act8(self, x_bits: np.ndarray, group: int):
        """(codes int8 [k] in logical order, scales float32 [k/G]) of fp16 x."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        k = x_bits.size
        assert k % group == 0
        codes = np.empty(k, np.int8)
        scales = np.empty(k // group, np.float32)
        self.lib.oracle_quantize_act8(_ptr(x_bits), k, group, _ptr(codes), _ptr(scales))
        return codes, scales

    def act8_block_order(self, codes: np.ndarray) -> np.ndarray:
        """The codes in the W4T4 byte order of the GEMV's activation buffer."""
        codes = np.ascontiguousarray(codes, dtype=np.int8)
        assert codes.size % 8 == 0
        out = np.empty_like(codes)
        self.lib.oracle_act8_block_order(_ptr(codes), codes.size, _ptr(out))
        return out

    def gemv_a8(self, q: np.ndarray, s_bits: np.ndarray, codes: np.ndarray, act_scales: np.ndarray, group: int,
                rows=None):
        """W4A8 (y, A) float64 for all rows, or for the listed rows."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s_bits = np.ascontiguousarray(s_bits, dtype=np.uint16)
        codes = np.ascontiguousarray(codes, dtype=np.int8)
        act_scales = np.ascontiguousarray(act_scales, dtype=np.float32)
        n, k = q.shape
        assert s_bits.shape == (n, k // group) and codes.shape == (k,) and act_scales.shape == (k // group,)
        rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        y = np.empty(rows.size, np.float64)
        a = np.empty(rows.size, np.float64)
        self.lib.oracle_gemv_a8_rows(_ptr(q), _ptr(s_bits), _ptr(codes), _ptr(act_scales), n, k, group,
                                     _ptr(rows), rows.size, _ptr(y), _ptr(a))
        return y, a

    def gemv_a8_packed(self, pw, ps, codes, act_scales, n: int, k: int, group: int, gateup: bool = False,
                       rows=None):
        """W4A8 (y, A) for the listed rows (default: all) from the packed buffers."""
        pw = np.ascontiguousarray(pw, dtype=np.uint8)
        ps = np.ascontiguousarray(ps, dtype=np.uint8)
        codes = np.ascontiguousarray(codes, dtype=np.int8)
        act_scales = np.ascontiguousarray(act_scales, dtype=np.float32)
        wb, sb = self.packed_sizes(n, k, group, gateup)
        assert pw.size >= wb and ps.size >= sb and codes.shape == (k,) and act_scales.shape == (k // group,)
        rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < n)
        y = np.empty(rows.size, np.float64)
        a = np.empty(rows.size, np.float64)
        self.lib.oracle_gemv_a8_packed_rows(_ptr(pw), _ptr(ps), _ptr(codes), _ptr(act_scales), n, k, group,
                                            int(gateup), _ptr(rows), rows.size, _ptr(y), _ptr(a))
        return y, a


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from w4_oracle.c (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def half_to_double(bits):
    return default().half_to_double(bits)


def packed_sizes(n, k, group, gateup=False):
    return default().packed_sizes(n, k, group, gateup)


def pack(q, s_bits, group, gateup=False):
    return default().pack(q, s_bits, group, gateup)


def unpack(pw, ps, n, k, group, gateup=False):
    return default().unpack(pw, ps, n, k, group, gateup)


def gemv(q, s_bits, x_bits, group, rows=None):
    return default().gemv(q, s_bits, x_bits, group, rows)


def gemm(q, s_bits, xm_bits, group):
    return default().gemm(q, s_bits, xm_bits, group)


def gemm_packed(pw, ps, xm_bits, n, k, group, gateup=False, mrows=None, ncols=None):
    return default().gemm_packed(pw, ps, xm_bits, n, k, group, gateup, mrows, ncols)


def gemv_packed(pw, ps, x_bits, n, k, group, gateup=False, rows=None):
    return default().gemv_packed(pw, ps, x_bits, n, k, group, gateup, rows)


def attn_decode(q_bits, k_cache, v_cache, page_table, ctx, n_kv, page, scale):
    return default().attn_decode(q_bits, k_cache, v_cache, page_table, ctx, n_kv, page, scale)


def rmsnorm(h, gamma_bits, eps):
    return default().rmsnorm(h, gamma_bits, eps)


def rmsnorm_given(h, gamma_bits, sumsq, eps):
    return default().rmsnorm_given(h, gamma_bits, sumsq, eps)


def sumsq_blocks(h, rows):
    return default().sumsq_blocks(h, rows)


def rope(x, pos, theta):
    return default().rope(x, pos, theta)


def silu(t):
    return default().silu(t)


def silu_gate(y):
    return default().silu_gate(y)


def argmax(y):
    return default().argmax(y)


def quantize_act8(x_bits, group):
    return default().quantize_act8(x_bits, group)


def act8_block_order(codes):
    return default().act8_block_order(codes)


def gemv_a8(q, s_bits, codes, act_scales, group, rows=None):
    return default().gemv_a8(q, s_bits, codes, act_scales, group, rows)


def gemv_a8_packed(pw, ps, codes, act_scales, n, k, group, gateup=False, rows=None):
    return default().gemv_a8_packed(pw, ps, codes, act_scales, n, k, group, gateup, rows)
