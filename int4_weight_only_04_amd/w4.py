"""Python binding of libw4.so (ctypes): argument marshalling only.

Every step of the GEMV runs in the HIP kernels behind the C ABI declared in
include/w4.h; PyTorch provides device memory and streams.  If the library is
not built, every call raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4.so")

OK, EINVAL, ESHAPE, EALIGN, EHIP, ENOMEM, ECAPTURE = range(7)
LAYOUT_PLAIN, LAYOUT_GATEUP = 0, 1
PROJ_PLAIN, PROJ_GATEUP_SILU, PROJ_LMHEAD_ARGMAX = 0, 1, 2
SWEEP_EAGER, SWEEP_GRAPH, SWEEP_PERSISTENT, SWEEP_PERSISTENT_EAGER = 0, 1, 2, 3

EXPORTED = (
    "w4_status_string", "w4_last_error", "w4_abi_version", "w4_packed_size", "w4_pack",
    "w4_gemv_workspace_size", "w4_gemv", "w4_gemv_argmax_noalloc", "w4_gemv_gateup_silu", "w4_gemm_workspace_size", "w4_gemm", "w4_gemm_gateup_silu",
    "w4_attn_decode_workspace_size", "w4_attn_decode",
    "w4_decode_linear_sweep_create", "w4_decode_linear_sweep", "w4_decode_linear_sweep_destroy",
    "w4_decode_linear_sweep_status", "w4_decode_linear_sweep_set_watchdog",
    "w4_embed", "w4_add_rmsnorm", "w4_rope_kv_append",
    "w4_decode_step_create", "w4_decode_step", "w4_decode_step_launches", "w4_decode_step_destroy",
    "w4_decode_step_trace_layout",
    "w4_quantize_act8", "w4_gemv_a8", "w4_gemv_gateup_silu_a8", "w4_read_probe",
    "w4_residual_parts", "w4_gemv_residual", "w4_gemv_rmsnorm", "w4_gemv_gateup_silu_rmsnorm",
)

TRACE_FIELDS = ("h_in", "x1", "qkv", "q", "attn", "o", "h_mid", "x2", "m", "d")


class W4Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {detail}")


class ProjDesc(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("packed_w", ctypes.c_void_p),
        ("packed_s", ctypes.c_void_p),
        ("x", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("argmax", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class LayerDesc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "attn_norm", "qkv_w", "qkv_s", "qkv_bias", "o_w", "o_s", "mlp_norm", "gateup_w", "gateup_s",
        "down_w", "down_s", "k_cache", "v_cache")]


class StepDesc(ctypes.Structure):
    _fields_ = [
        ("layers", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("vocab", ctypes.c_int64),
        ("group", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("rope_theta", ctypes.c_double),
        ("embed", ctypes.c_void_p),
        ("layer", ctypes.POINTER(LayerDesc)),
        ("final_norm", ctypes.c_void_p),
        ("lm_w", ctypes.c_void_p),
        ("lm_s", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("token", ctypes.c_void_p),
        ("pos", ctypes.c_void_p),
        ("logits", ctypes.c_void_p),
        ("trace", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """Load libw4.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950) first")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    L.w4_status_string.restype = ctypes.c_char_p
    L.w4_status_string.argtypes = [i32]
    L.w4_last_error.restype = ctypes.c_char_p
    L.w4_last_error.argtypes = []
    L.w4_abi_version.restype = i32
    L.w4_abi_version.argtypes = []
    L.w4_packed_size.restype = i32
    L.w4_packed_size.argtypes = [i64, i64, i32, i32, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.w4_pack.restype = i32
    L.w4_pack.argtypes = [vp, vp, i64, i64, i32, i32, vp, sz, vp, sz]
    L.w4_gemv_workspace_size.restype = i32
    L.w4_gemv_workspace_size.argtypes = [i64, i64, i32, i32, ctypes.POINTER(sz)]
    L.w4_gemv.restype = i32
    L.w4_gemv.argtypes = [vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, vp]
    L.w4_gemv_gateup_silu.restype = i32
    L.w4_gemv_argmax_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, vp]
    L.w4_gemv_argmax_noalloc.restype = i32
    L.w4_gemv_gateup_silu.argtypes = [vp, vp, vp, vp, i64, i64, i32, vp]
    L.w4_residual_parts.restype = i32
    L.w4_residual_parts.argtypes = [i64, i64, i32, ctypes.POINTER(i64)]
    L.w4_gemv_residual.restype = i32
    L.w4_gemv_residual.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, vp]
    L.w4_gemv_rmsnorm.restype = i32
    L.w4_gemv_rmsnorm.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.c_float, vp, vp, vp, vp, sz, i64, i64, i32, vp]
    L.w4_gemv_gateup_silu_rmsnorm.restype = i32
    L.w4_gemv_gateup_silu_rmsnorm.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.c_float, vp, vp, i64, i64, i32, vp]
    L.w4_gemm_workspace_size.restype = i32
    L.w4_gemm_workspace_size.argtypes = [i64, i64, i64, i32, ctypes.POINTER(sz)]
    L.w4_gemm.restype = i32
    L.w4_gemm.argtypes = [vp, vp, vp, vp, vp, sz, i64, i64, i64, i32, vp]
    L.w4_attn_decode_workspace_size.restype = i32
    L.w4_attn_decode_workspace_size.argtypes = [i32, i32, ctypes.POINTER(sz)]
    L.w4_attn_decode.restype = i32
    L.w4_attn_decode.argtypes = [vp, vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, ctypes.c_float, vp, sz, vp]
    L.w4_gemm_gateup_silu.restype = i32
    L.w4_gemm_gateup_silu.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp]
    L.w4_decode_linear_sweep_create.restype = i32
    L.w4_decode_linear_sweep_create.argtypes = [ctypes.POINTER(ProjDesc), i32, i32,
                                                ctypes.POINTER(vp)]
    L.w4_decode_linear_sweep.restype = i32
    L.w4_decode_linear_sweep.argtypes = [vp, vp]
    L.w4_decode_linear_sweep_destroy.restype = i32
    L.w4_decode_linear_sweep_destroy.argtypes = [vp]
    L.w4_decode_linear_sweep_status.argtypes = [vp, ctypes.POINTER(i32)]
    L.w4_decode_linear_sweep_status.restype = i32
    L.w4_decode_linear_sweep_set_watchdog.argtypes = [vp, ctypes.c_double]
    L.w4_decode_linear_sweep_set_watchdog.restype = i32
    L.w4_embed.restype = i32
    L.w4_embed.argtypes = [vp, i64, i64, vp, vp, vp]
    L.w4_add_rmsnorm.restype = i32
    L.w4_add_rmsnorm.argtypes = [vp, vp, vp, i64, ctypes.c_float, vp, vp]
    L.w4_rope_kv_append.restype = i32
    L.w4_rope_kv_append.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_double, vp, vp, vp, vp, i32, i32, i32,
                                    vp, vp]
    L.w4_decode_step_create.restype = i32
    L.w4_decode_step_create.argtypes = [ctypes.POINTER(StepDesc), i32, ctypes.POINTER(vp)]
    L.w4_decode_step.restype = i32
    L.w4_decode_step.argtypes = [vp, vp]
    L.w4_decode_step_launches.restype = i32
    L.w4_decode_step_launches.argtypes = [vp, ctypes.POINTER(i32)]
    L.w4_decode_step_destroy.restype = i32
    L.w4_decode_step_destroy.argtypes = [vp]
    L.w4_read_probe.restype = i32
    L.w4_read_probe.argtypes = [vp, sz, vp, vp]
    L.w4_quantize_act8.restype = i32
    L.w4_quantize_act8.argtypes = [vp, i64, i32, vp, vp, vp]
    L.w4_gemv_a8.restype = i32
    L.w4_gemv_a8.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, vp]
    L.w4_gemv_gateup_silu_a8.restype = i32
    L.w4_gemv_gateup_silu_a8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, vp]
    L.w4_decode_step_trace_layout.restype = i32
    L.w4_decode_step_trace_layout.argtypes = [ctypes.POINTER(StepDesc), ctypes.POINTER(sz), ctypes.POINTER(sz),
                                              ctypes.POINTER(sz)]
    _lib = L
    return L


def _check(status: int, where: str):
    if status != OK:
        detail = lib().w4_last_error().decode(errors="replace")
        raise W4Error(status, where, detail)


def status_string(status: int) -> str:
    return lib().w4_status_string(status).decode()


def last_error() -> str:
    return lib().w4_last_error().decode(errors="replace")


def _layout(layout) -> int:
    if layout in ("plain", LAYOUT_PLAIN):
        return LAYOUT_PLAIN
    if layout in ("gateup", LAYOUT_GATEUP):
        return LAYOUT_GATEUP
    return int(layout)


def packed_size(n: int, k: int, group: int, layout="plain") -> tuple[int, int]:
    wb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().w4_packed_size(n, k, group, _layout(layout), ctypes.byref(wb), ctypes.byref(sb)),
           "w4_packed_size")
    return wb.value, sb.value


def pack(q: np.ndarray, scales_bits: np.ndarray, group: int, layout="plain"):
    """Host packer: q uint8 [n, k] (values 0..15), scales fp16 bits uint16
    [n, k/group] -> (packed_w, packed_s) as uint8 numpy arrays."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    if q.ndim != 2:
        raise ValueError("q must be 2-D [n, k]")
    n, k = q.shape
    if scales_bits.shape != (n, k // group if group else 0):
        raise ValueError(f"scales must be [{n}, {k}//{group}], got {scales_bits.shape}")
    wb, sb = packed_size(n, k, group, layout)
    pw = np.empty(wb, np.uint8)
    ps = np.empty(sb, np.uint8)
    _check(lib().w4_pack(q.ctypes.data, scales_bits.ctypes.data, n, k, group, _layout(layout),
                         pw.ctypes.data, wb, ps.ctypes.data, sb), "w4_pack")
    return pw, ps


def gemv_workspace_size(n: int, k: int, group: int, with_argmax: bool) -> int:
    out = ctypes.c_size_t()
    _check(lib().w4_gemv_workspace_size(n, k, group, int(bool(with_argmax)), ctypes.byref(out)),
           "w4_gemv_workspace_size")
    return out.value


def _dev_ptr(t, name: str, dtype=None, numel: Optional[int] = None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def gemv(packed_w, packed_s, x, y, n: int, k: int, group: int, argmax=None, workspace=None,
         stream=None):
    """y[n] (fp32) = W x; with `argmax` (int32 [1]) and `workspace` (uint8,
    gemv_workspace_size bytes) also the lowest-index argmax of y."""
    import torch
    wb, sb = packed_size(n, k, group, "plain")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if argmax is not None and ws_bytes < gemv_workspace_size(n, k, group, True):
        raise ValueError("workspace too small for the argmax epilogue")
    _check(lib().w4_gemv(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                         _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                         _dev_ptr(x, "x", torch.float16, k),
                         _dev_ptr(y, "y", torch.float32, n),
                         _dev_ptr(argmax, "argmax", torch.int32, 1),
                         _dev_ptr(workspace, "workspace"), ws_bytes, n, k, group,
                         _stream(stream)), "w4_gemv")


def gemv_argmax_noalloc(packed_w, packed_s, x, y, argmax, n: int, k: int, group: int, stream=None):
    """y[n] (fp32) = W x and the lowest-index argmax of y, with the partials
    in the library's static device scratch (no workspace argument)."""
    import torch
    wb, sb = packed_size(n, k, group, "plain")
    _check(lib().w4_gemv_argmax_noalloc(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                                        _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                                        _dev_ptr(x, "x", torch.float16, k),
                                        _dev_ptr(y, "y", torch.float32, n),
                                        _dev_ptr(argmax, "argmax", torch.int32, 1),
                                        n, k, group, _stream(stream)), "w4_gemv_argmax_noalloc")


def gemv_gateup_silu(packed_w, packed_s, x, h, n_total: int, k: int, group: int, stream=None):
    """h[n_total/2] (fp16) = silu(gate) * up for a gate/up-layout matrix."""
    import torch
    wb, sb = packed_size(n_total, k, group, "gateup")
    _check(lib().w4_gemv_gateup_silu(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                                     _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                                     _dev_ptr(x, "x", torch.float16, k),
                                     _dev_ptr(h, "h", torch.float16, n_total // 2),
                                     n_total, k, group, _stream(stream)), "w4_gemv_gateup_silu")


def residual_parts(n: int, k: int, group: int) -> int:
    """Partial sums of squares gemv_residual writes for an n x k projection."""
    out = ctypes.c_int64()
    _check(lib().w4_residual_parts(n, k, group, ctypes.byref(out)), "w4_residual_parts")
    return out.value


def gemv_residual(packed_w, packed_s, x, y, h_in, h_out, ss_part, n: int, k: int, group: int, stream=None):
    """y = W x, h_out = h_in + y (fp32, h_out may be h_in) and the partial
    sums of squares of h_out (ss_part: fp32, residual_parts floats)."""
    import torch
    wb, sb = packed_size(n, k, group, "plain")
    _check(lib().w4_gemv_residual(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                                  _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                                  _dev_ptr(x, "x", torch.float16, k),
                                  _dev_ptr(y, "y", torch.float32, n),
                                  _dev_ptr(h_in, "h_in", torch.float32, n),
                                  _dev_ptr(h_out, "h_out", torch.float32, n),
                                  _dev_ptr(ss_part, "ss_part", torch.float32, residual_parts(n, k, group)),
                                  n, k, group, _stream(stream)), "w4_gemv_residual")


def _norm_args(h, gamma, ss_part, parts: int, eps: float, x_out, k: int):
    import torch
    return (_dev_ptr(h, "h", torch.float32, k), _dev_ptr(gamma, "gamma", torch.float16, k),
            _dev_ptr(ss_part, "ss_part", torch.float32, (parts + 3) // 4 * 4), parts, float(eps),
            _dev_ptr(x_out, "x_out", torch.float16, k))


def gemv_rmsnorm(packed_w, packed_s, h, gamma, ss_part, parts: int, eps: float, y, n: int, k: int, group: int,
                 x_out=None, argmax=None, workspace=None, stream=None):
    """y = W x with x = fp16(h * gamma / sqrt(sum(ss_part[:parts]) / k + eps))
    (ss_part padded to a multiple of 4 floats); x_out receives that x."""
    import torch
    wb, sb = packed_size(n, k, group, "plain")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if argmax is not None and ws_bytes < gemv_workspace_size(n, k, group, True):
        raise ValueError("workspace too small for the argmax epilogue")
    _check(lib().w4_gemv_rmsnorm(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                                 _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                                 *_norm_args(h, gamma, ss_part, parts, eps, x_out, k),
                                 _dev_ptr(y, "y", torch.float32, n),
                                 _dev_ptr(argmax, "argmax", torch.int32, 1),
                                 _dev_ptr(workspace, "workspace"), ws_bytes, n, k, group,
                                 _stream(stream)), "w4_gemv_rmsnorm")


def gemv_gateup_silu_rmsnorm(packed_w, packed_s, h, gamma, ss_part, parts: int, eps: float, h_mlp, n_total: int,
                             k: int, group: int, x_out=None, stream=None):
    """gemv_gateup_silu with its input normalized as in gemv_rmsnorm."""
    import torch
    wb, sb = packed_size(n_total, k, group, "gateup")
    _check(lib().w4_gemv_gateup_silu_rmsnorm(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                                             _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                                             *_norm_args(h, gamma, ss_part, parts, eps, x_out, k),
                                             _dev_ptr(h_mlp, "h_mlp", torch.float16, n_total // 2),
                                             n_total, k, group, _stream(stream)), "w4_gemv_gateup_silu_rmsnorm")


def read_probe(buf, nbytes: int, sink, stream=None):
    """Diagnostic: stream nbytes of a device buffer with the GEMVs' loads
    (sink: device int32/uint32 tensor of 1024 words)."""
    import torch
    if buf.numel() * buf.element_size() < nbytes:
        raise ValueError("buffer smaller than nbytes")
    _check(lib().w4_read_probe(_dev_ptr(buf, "buf"), nbytes, _dev_ptr(sink, "sink", None, 1024), _stream(stream)),
           "w4_read_probe")


def quantize_act8(x, group: int, codes, scales, stream=None):
    """codes int8 [k] (W4T4 block order) and scales fp32 [k/group] of fp16 x."""
    import torch
    k = x.numel()
    _check(lib().w4_quantize_act8(_dev_ptr(x, "x", torch.float16, k), k, group,
                                  _dev_ptr(codes, "codes", torch.int8, k),
                                  _dev_ptr(scales, "scales", torch.float32, k // group), _stream(stream)),
           "w4_quantize_act8")


def gemv_a8(packed_w, packed_s, codes, act_scales, y, n: int, k: int, group: int, argmax=None, workspace=None,
            stream=None):
    """W4A8 y[n] (fp32) from int8 codes and per-group scales (quantize_act8)."""
    import torch
    wb, sb = packed_size(n, k, group, "plain")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().w4_gemv_a8(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                            _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                            _dev_ptr(codes, "codes", torch.int8, k),
                            _dev_ptr(act_scales, "act_scales", torch.float32, k // group),
                            _dev_ptr(y, "y", torch.float32, n), _dev_ptr(argmax, "argmax", torch.int32, 1),
                            _dev_ptr(workspace, "workspace"), ws_bytes, n, k, group, _stream(stream)), "w4_gemv_a8")


def gemv_gateup_silu_a8(packed_w, packed_s, codes, act_scales, h, n_total: int, k: int, group: int, stream=None):
    """W4A8 h[n_total/2] (fp16) = silu(gate) * up."""
    import torch
    wb, sb = packed_size(n_total, k, group, "gateup")
    _check(lib().w4_gemv_gateup_silu_a8(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                                        _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                                        _dev_ptr(codes, "codes", torch.int8, k),
                                        _dev_ptr(act_scales, "act_scales", torch.float32, k // group),
                                        _dev_ptr(h, "h", torch.float16, n_total // 2), n_total, k, group,
                                        _stream(stream)), "w4_gemv_gateup_silu_a8")


def gemm_workspace_size(m: int, n: int, k: int, group: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().w4_gemm_workspace_size(m, n, k, group, ctypes.byref(out)), "w4_gemm_workspace_size")
    return int(out.value)


def gemm(packed_w, packed_s, x, y, m: int, n: int, k: int, group: int, workspace=None, stream=None):
    """Prefill product y[m, n] (fp32) = x[m, k] (fp16) times W^T; `workspace`
    (uint8, gemm_workspace_size bytes) is needed when that size is nonzero."""
    import torch
    wb, sb = packed_size(n, k, group, "plain")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().w4_gemm(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                         _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                         _dev_ptr(x, "x", torch.float16, m * k),
                         _dev_ptr(y, "y", torch.float32, m * n),
                         _dev_ptr(workspace, "workspace"), ws_bytes,
                         m, n, k, group, _stream(stream)), "w4_gemm")


def gemm_gateup_silu(packed_w, packed_s, x, h, m: int, n_total: int, k: int, group: int,
                     stream=None):
    """Prefill gate/up + SiLU: h[m, n_total/2] (fp16) = silu(gate) * up per token row."""
    import torch
    wb, sb = packed_size(n_total, k, group, "gateup")
    _check(lib().w4_gemm_gateup_silu(_dev_ptr(packed_w, "packed_w", torch.uint8, wb),
                                     _dev_ptr(packed_s, "packed_s", torch.uint8, sb),
                                     _dev_ptr(x, "x", torch.float16, m * k),
                                     _dev_ptr(h, "h", torch.float16, m * (n_total // 2)),
                                     m, n_total, k, group, _stream(stream)), "w4_gemm_gateup_silu")


def attn_decode_workspace_size(n_heads: int, max_ctx: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().w4_attn_decode_workspace_size(n_heads, max_ctx, ctypes.byref(out)),
           "w4_attn_decode_workspace_size")
    return int(out.value)


def attn_decode(q, k_cache, v_cache, page_table, ctx_len, max_ctx: int, out, n_kv_heads: int,
                page_size: int, scale: float, workspace, stream=None):
    """o[n_heads, 128] (fp16) = softmax(scale q K^T) V over the paged cache;
    ctx_len is a device int32 tensor of one element."""
    import torch
    n_heads = q.shape[0]
    num_pages = k_cache.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().w4_attn_decode(_dev_ptr(q, "q", torch.float16, n_heads * 128),
                                _dev_ptr(k_cache, "k_cache", torch.float16),
                                _dev_ptr(v_cache, "v_cache", torch.float16, k_cache.numel()),
                                _dev_ptr(page_table, "page_table", torch.int32, -(-max_ctx // page_size)),
                                num_pages, _dev_ptr(ctx_len, "ctx_len", torch.int32, 1), max_ctx,
                                _dev_ptr(out, "out", torch.float16, n_heads * 128),
                                n_heads, n_kv_heads, 128, page_size, float(scale),
                                _dev_ptr(workspace, "workspace"), ws_bytes, _stream(stream)),
           "w4_attn_decode")


@dataclass
class Proj:
    """One projection of a sweep (device tensors are kept alive by the Sweep)."""
    kind: int
    n: int
    k: int
    group: int
    packed_w: object
    packed_s: object
    x: object
    out: object
    argmax: object = None
    workspace: object = None


class Sweep:
    """Per-token linear sweep: eager launches, one captured HIP graph, or the
    persistent kernel (mode SWEEP_PERSISTENT / SWEEP_PERSISTENT_EAGER)."""

    def __init__(self, projs: Sequence[Proj], use_graph: bool = True, mode: Optional[int] = None):
        import torch
        self._projs = list(projs)  # keep device buffers alive while the graph exists
        arr = (ProjDesc * len(self._projs))()
        for i, p in enumerate(self._projs):
            d = arr[i]
            d.kind = p.kind
            d.group = p.group
            d.n = p.n
            d.k = p.k
            wb, sb = packed_size(p.n, p.k, p.group,
                                 "gateup" if p.kind == PROJ_GATEUP_SILU else "plain")
            d.packed_w = _dev_ptr(p.packed_w, "packed_w", torch.uint8, wb)
            d.packed_s = _dev_ptr(p.packed_s, "packed_s", torch.uint8, sb)
            d.x = _dev_ptr(p.x, "x", torch.float16, p.k)
            if p.kind == PROJ_GATEUP_SILU:
                d.out = _dev_ptr(p.out, "out", torch.float16, p.n // 2)
            else:
                d.out = _dev_ptr(p.out, "out", torch.float32, p.n)
            d.argmax = _dev_ptr(p.argmax, "argmax", torch.int32, 1)
            d.workspace = _dev_ptr(p.workspace, "workspace")
            d.workspace_bytes = (p.workspace.numel() * p.workspace.element_size()
                                 if p.workspace is not None else 0)
        if mode is None:
            mode = SWEEP_GRAPH if use_graph else SWEEP_EAGER
        handle = ctypes.c_void_p()
        _check(lib().w4_decode_linear_sweep_create(arr, len(self._projs), int(mode), ctypes.byref(handle)),
               "w4_decode_linear_sweep_create")
        self._handle = handle
        self.mode = int(mode)
        self.use_graph = self.mode in (SWEEP_GRAPH, SWEEP_PERSISTENT)

    def status(self) -> bool:
        """True if a watchdog timeout happened since the last call (persistent modes)."""
        out = ctypes.c_int32()
        _check(lib().w4_decode_linear_sweep_status(self._handle, ctypes.byref(out)), "w4_decode_linear_sweep_status")
        return bool(out.value)

    def set_watchdog(self, seconds: float):
        _check(lib().w4_decode_linear_sweep_set_watchdog(self._handle, float(seconds)),
               "w4_decode_linear_sweep_set_watchdog")

    def run(self, stream=None):
        if not self._handle:
            raise RuntimeError("sweep destroyed")
        _check(lib().w4_decode_linear_sweep(self._handle, _stream(stream)), "w4_decode_linear_sweep")

    def close(self):
        if self._handle:
            _check(lib().w4_decode_linear_sweep_destroy(self._handle), "w4_decode_linear_sweep_destroy")
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def embed(table, token, h, stream=None):
    """h[hidden] (fp32) = table[*token] for an fp16 table [vocab, hidden] and a
    device int32 token of one element."""
    import torch
    vocab, hidden = table.shape
    _check(lib().w4_embed(_dev_ptr(table, "table", torch.float16), vocab, hidden,
                          _dev_ptr(token, "token", torch.int32, 1),
                          _dev_ptr(h, "h", torch.float32, hidden), _stream(stream)), "w4_embed")


def add_rmsnorm(h, y, gamma, eps: float, x, stream=None):
    """h += y (when y is given), then x (fp16) = rmsnorm(h) * gamma."""
    import torch
    n = h.numel()
    _check(lib().w4_add_rmsnorm(_dev_ptr(h, "h", torch.float32, n), _dev_ptr(y, "y", torch.float32, n),
                                _dev_ptr(gamma, "gamma", torch.float16, n), n, float(eps),
                                _dev_ptr(x, "x", torch.float16, n), _stream(stream)), "w4_add_rmsnorm")


def rope_kv_append(qkv, bias, pos, n_heads: int, n_kv_heads: int, theta: float, q_out, k_cache, v_cache,
                   page_table, max_ctx: int, ctx_len=None, stream=None):
    """Rotate q and k of the fused projection output at device position *pos,
    write q (fp16) to q_out and k, v to the paged caches; ctx_len <- pos + 1."""
    import torch
    rows = (n_heads + 2 * n_kv_heads) * 128
    num_pages, _, page_size, _ = k_cache.shape
    _check(lib().w4_rope_kv_append(_dev_ptr(qkv, "qkv", torch.float32, rows),
                                   _dev_ptr(bias, "bias", torch.float32, rows),
                                   _dev_ptr(pos, "pos", torch.int32, 1), n_heads, n_kv_heads, 128, float(theta),
                                   _dev_ptr(q_out, "q_out", torch.float16, n_heads * 128),
                                   _dev_ptr(k_cache, "k_cache", torch.float16),
                                   _dev_ptr(v_cache, "v_cache", torch.float16, k_cache.numel()),
                                   _dev_ptr(page_table, "page_table", torch.int32, -(-max_ctx // page_size)),
                                   num_pages, page_size, max_ctx, _dev_ptr(ctx_len, "ctx_len", torch.int32, 1),
                                   _stream(stream)), "w4_rope_kv_append")


@dataclass
class StepLayer:
    """Device tensors of one decoder layer (packed matrices as uint8)."""
    attn_norm: object
    qkv_w: object
    qkv_s: object
    o_w: object
    o_s: object
    mlp_norm: object
    gateup_w: object
    gateup_s: object
    down_w: object
    down_s: object
    k_cache: object
    v_cache: object
    qkv_bias: object = None


def trace_layout(desc: "StepDesc") -> tuple[list[int], int, int]:
    """(field offsets, layer stride, total bytes) of a step's trace buffer."""
    offs = (ctypes.c_size_t * len(TRACE_FIELDS))()
    stride, total = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().w4_decode_step_trace_layout(ctypes.byref(desc), offs, ctypes.byref(stride), ctypes.byref(total)),
           "w4_decode_step_trace_layout")
    return list(offs), stride.value, total.value


def step_trace_bytes(*, hidden, n_heads, n_kv_heads, inter, layers) -> int:
    """Bytes of the trace buffer a DecodeStep with these dimensions fills."""
    d = StepDesc()
    d.layers, d.hidden, d.n_heads, d.n_kv_heads, d.inter = layers, hidden, n_heads, n_kv_heads, inter
    return trace_layout(d)[2]


class DecodeStep:
    """One full greedy decode step (embedding .. argmax, position advance) as
    eager launches or one captured HIP graph; token and pos are device int32
    tensors of one element that the step reads and advances."""

    def __init__(self, *, hidden, n_heads, n_kv_heads, inter, vocab, group, page_size, max_ctx, rms_eps,
                 rope_theta, embed, layers: Sequence[StepLayer], final_norm, lm_w, lm_s, page_table, token, pos,
                 logits, trace=None, use_graph=True):
        import torch
        self._keep = (embed, list(layers), final_norm, lm_w, lm_s, page_table, token, pos, logits, trace)
        qkv_rows = (n_heads + 2 * n_kv_heads) * 128
        arr = (LayerDesc * len(layers))()
        num_pages = None
        for i, L in enumerate(layers):
            d = arr[i]
            d.attn_norm = _dev_ptr(L.attn_norm, "attn_norm", torch.float16, hidden)
            d.mlp_norm = _dev_ptr(L.mlp_norm, "mlp_norm", torch.float16, hidden)
            for name, (n, k, lay) in (("qkv", (qkv_rows, hidden, "plain")), ("o", (hidden, n_heads * 128, "plain")),
                                      ("gateup", (2 * inter, hidden, "gateup")), ("down", (hidden, inter, "plain"))):
                wb, sb = packed_size(n, k, group, lay)
                setattr(d, name + "_w", _dev_ptr(getattr(L, name + "_w"), name + "_w", torch.uint8, wb))
                setattr(d, name + "_s", _dev_ptr(getattr(L, name + "_s"), name + "_s", torch.uint8, sb))
            d.qkv_bias = _dev_ptr(L.qkv_bias, "qkv_bias", torch.float32, qkv_rows)
            if tuple(L.k_cache.shape[1:]) != (n_kv_heads, page_size, 128) or L.v_cache.shape != L.k_cache.shape:
                raise ValueError("caches must be fp16 [num_pages, n_kv_heads, page_size, 128]")
            if num_pages is not None and L.k_cache.shape[0] != num_pages:
                raise ValueError("every layer's cache must have the same number of pages")
            num_pages = L.k_cache.shape[0]
            d.k_cache = _dev_ptr(L.k_cache, "k_cache", torch.float16)
            d.v_cache = _dev_ptr(L.v_cache, "v_cache", torch.float16)
        desc = StepDesc()
        desc.layers, desc.hidden, desc.n_heads, desc.n_kv_heads = len(layers), hidden, n_heads, n_kv_heads
        desc.head_dim, desc.inter, desc.vocab, desc.group = 128, inter, vocab, group
        desc.page_size, desc.num_pages, desc.max_ctx = page_size, num_pages or 0, max_ctx
        desc.rms_eps, desc.rope_theta = float(rms_eps), float(rope_theta)
        desc.embed = _dev_ptr(embed, "embed", torch.float16, vocab * hidden)
        desc.layer = arr
        desc.final_norm = _dev_ptr(final_norm, "final_norm", torch.float16, hidden)
        wb, sb = packed_size(vocab, hidden, group, "plain")
        desc.lm_w = _dev_ptr(lm_w, "lm_w", torch.uint8, wb)
        desc.lm_s = _dev_ptr(lm_s, "lm_s", torch.uint8, sb)
        desc.page_table = _dev_ptr(page_table, "page_table", torch.int32, -(-max_ctx // page_size))
        desc.token = _dev_ptr(token, "token", torch.int32, 1)
        desc.pos = _dev_ptr(pos, "pos", torch.int32, 1)
        desc.logits = _dev_ptr(logits, "logits", torch.float32, vocab)
        self.layout = trace_layout(desc)
        desc.trace = _dev_ptr(trace, "trace", torch.uint8, self.layout[2] if trace is not None else None)
        self.dims = dict(hidden=hidden, n_heads=n_heads, n_kv_heads=n_kv_heads, inter=inter,
                         layers=len(layers))
        self.trace = trace
        handle = ctypes.c_void_p()
        _check(lib().w4_decode_step_create(ctypes.byref(desc), int(bool(use_graph)), ctypes.byref(handle)),
               "w4_decode_step_create")
        self._handle = handle
        self.use_graph = use_graph

    def read_trace(self) -> list[dict]:
        """Host copy of the trace: one dict per layer (fp32 fields as float32,
        fp16 fields as uint16 bits), then {"h_in", "x1"} of the final record."""
        import numpy as np
        if self.trace is None:
            raise RuntimeError("step built without a trace buffer")
        raw = self.trace.cpu().numpy()
        offs, stride, _ = self.layout
        H, nh, nkv, inter = (self.dims[k] for k in ("hidden", "n_heads", "n_kv_heads", "inter"))
        spec = {"h_in": (np.float32, H), "x1": (np.uint16, H), "qkv": (np.float32, (nh + 2 * nkv) * 128),
                "q": (np.uint16, nh * 128), "attn": (np.uint16, nh * 128), "o": (np.float32, H),
                "h_mid": (np.float32, H), "x2": (np.uint16, H), "m": (np.uint16, inter), "d": (np.float32, H)}
        out = []
        for l in range(self.dims["layers"] + 1):
            rec = {}
            for f, name in enumerate(TRACE_FIELDS):
                if l == self.dims["layers"] and name not in ("h_in", "x1"):
                    continue
                dt, n = spec[name]
                start = l * stride + offs[f]
                rec[name] = raw[start:start + n * np.dtype(dt).itemsize].view(dt).copy()
            out.append(rec)
        return out

    def launches(self) -> int:
        n = ctypes.c_int32()
        _check(lib().w4_decode_step_launches(self._handle, ctypes.byref(n)), "w4_decode_step_launches")
        return n.value

    def run(self, stream=None):
        if not self._handle:
            raise RuntimeError("decode step destroyed")
        _check(lib().w4_decode_step(self._handle, _stream(stream)), "w4_decode_step")

    def close(self):
        if self._handle:
            _check(lib().w4_decode_step_destroy(self._handle), "w4_decode_step_destroy")
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
