"""Helpers for the GPU parity tests: device upload and the tolerances.

Tolerance (plain outputs): |y_gpu - y_ref| <= 1e-3 * A + 1e-5 per element,
A = sum_k |w x| from the oracle.

Tolerance (fused gate/up, derived from the plain one): with g, u the gate and
up rows, |silu'| <= 1.0998 (its maximum, near t = 2.3994), so
  |silu(g')u' - silu(g)u| <= 1.0998 E_g (|u| + E_u) + |silu(g)| E_u
plus the fp16 rounding of h (half an ulp, <= 2^-11 |h| for normal values),
the fast exponential's relative error (~1e-6), covered together by
2^-10 |h|, plus 2^-24 (the fp16 subnormal step) absolute.
"""
from __future__ import annotations

import numpy as np

SILU_SLOPE_MAX = 1.0998


def tol_plain(a: np.ndarray) -> np.ndarray:
    return 1e-3 * a + 1e-5


def tol_gateup(yg, ag, yu, au, h_ref) -> np.ndarray:
    eg = tol_plain(ag)
    eu = tol_plain(au)
    silu_g = yg / (1.0 + np.exp(-yg))
    return (SILU_SLOPE_MAX * eg * (np.abs(yu) + eu) + np.abs(silu_g) * eu
            + 2.0 ** -10 * np.abs(h_ref) + 2.0 ** -24)


def dev_u8(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def dev_f16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).cuda().view(
        torch.float16)


def host_f16(t) -> np.ndarray:
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.float16).astype(np.float64)


def half_bits(v) -> np.ndarray:
    return np.asarray(v, np.float16).view(np.uint16)


def near_tie_set(y_ref: np.ndarray, a_ref: np.ndarray) -> np.ndarray:
    """Indices whose reference value is within the combined tolerance of the max."""
    e = tol_plain(a_ref)
    i_star = int(np.argmax(y_ref))
    return np.nonzero(y_ref >= y_ref[i_star] - (e + e[i_star]))[0]
