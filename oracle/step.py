"""Oracle of one full decode step (test infrastructure only).

The pages name the model (Qwen2.5-Coder-7B: 28 decoder layers, hidden 3584,
MLP 18944, vocabulary 152064 -- "How to Build Your Own LLM Runtime from
Scratch", brifing.si, section 7 "Model Dimensions and Structure") and the parts
of its runtime (INT4 weights, paged KV cache, attention -- "How To Build Your
Own LLM Runtime From Scratch", aitrending.vip, "Technical Details", first
bullet), not the decoder's equations.  They are read as that model family's
pre-norm decoder, composed here from the oracle's pinned pieces in fp64:

    x1 = rmsnorm(h) g1                         (stored fp16: the GEMV input)
    qkv = W_qkv x1 (+ bias)                    q heads, then k heads, then v heads
    q, k = rope(q, pos), rope(k, pos)          (stored fp16: attention input, KV cache)
    a  = attention(q, K[0..pos], V[0..pos])    (stored fp16)
    h' = h + W_o a
    x2 = rmsnorm(h') g2                        (stored fp16)
    m  = silu(gate x2) * (up x2)               (stored fp16)
    h'' = h' + W_down m
and, after the last layer, logits = W_lm (rmsnorm(h) g_f) with the greedy
argmax.  The fp16 storage points are the ones where the step's operations are
defined on fp16 operands (GEMV input x, attention q and cache, gate/up output);
rounding there is to nearest even.  Everything else is fp64.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import default

HEAD_DIM = 128


def to_half_bits(v) -> np.ndarray:
    """Round to fp16 (nearest even) and return the bit patterns."""
    return np.asarray(v, np.float64).astype(np.float16).view(np.uint16)


def half_bits_to_double(b) -> np.ndarray:
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


@dataclass
class Proj:
    """Logical INT4 matrix: q uint8 [n, k] in 0..15, s fp16 bits [n, k/G]."""
    q: np.ndarray
    s: np.ndarray


@dataclass
class Layer:
    attn_norm: np.ndarray   # fp16 bits [hidden]
    qkv: Proj
    o: Proj
    mlp_norm: np.ndarray
    gateup: Proj            # rows [0, I) gate, [I, 2I) up
    down: Proj
    qkv_bias: np.ndarray | None = None   # float64 [(nh + 2 nkv) * 128], values exact in fp32


@dataclass
class Config:
    hidden: int
    n_heads: int
    n_kv: int
    inter: int
    group: int
    page: int
    eps: float
    theta: float


@dataclass
class LayerResult:
    """Stage values of one layer.  fp16 stages hold the unrounded fp64 value
    (the stored operand is its fp16 rounding); a_* are the sums of |terms|."""
    x1: np.ndarray = field(default=None)       # fp64 [hidden], stored fp16
    qkv: np.ndarray = field(default=None)      # fp64, the projection (bias not added)
    a_qkv: np.ndarray = field(default=None)
    q: np.ndarray = field(default=None)        # fp64 [nh, 128] rotated, stored fp16
    k: np.ndarray = field(default=None)        # fp64 [nkv, 128] rotated, stored fp16 in the cache
    v: np.ndarray = field(default=None)        # fp64 [nkv, 128], stored fp16 in the cache
    attn: np.ndarray = field(default=None)     # fp64 [nh, 128], stored fp16
    a_attn: np.ndarray = field(default=None)
    o: np.ndarray = field(default=None)
    a_o: np.ndarray = field(default=None)
    h_mid: np.ndarray = field(default=None)
    x2: np.ndarray = field(default=None)       # fp64 [hidden], stored fp16
    gu: np.ndarray = field(default=None)       # fp64 [2I]
    a_gu: np.ndarray = field(default=None)
    m: np.ndarray = field(default=None)        # fp64 [I], stored fp16
    d: np.ndarray = field(default=None)
    a_d: np.ndarray = field(default=None)
    h_out: np.ndarray = field(default=None)


def _take(forced, name, own):
    """The value the next stage consumes: the forced one when given."""
    if forced is not None and name in forced:
        return forced[name]
    return own


def decoder_layer(h: np.ndarray, layer: Layer, cfg: Config, pos: int, k_cache: np.ndarray,
                  v_cache: np.ndarray, page_table: np.ndarray, orc=None, forced: dict | None = None) -> LayerResult:
    """One layer for the token at position pos.  h is the fp64 residual
    stream; k_cache / v_cache (fp16 bits [pages, nkv, page, 128]) hold the
    earlier tokens and receive this token's k and v (modified in place).

    forced (teacher forcing) maps stage names to values that replace this
    function's own stored results as the input of the following stages, so a
    stage can be checked from another implementation's input: "x1", "q", "k",
    "v", "attn", "x2", "m" as fp16 bits; "qkv", "o", "h_mid", "d" as float64.
    Each stage's own result (computed from the forced inputs) is returned."""
    orc = orc or default()
    r = LayerResult()
    nh, nkv, G = cfg.n_heads, cfg.n_kv, cfg.group
    r.x1 = orc.rmsnorm(h, layer.attn_norm, cfg.eps)
    x1 = _take(forced, "x1", to_half_bits(r.x1))
    r.qkv, r.a_qkv = orc.gemv(layer.qkv.q, layer.qkv.s, x1, G)
    qkv = _take(forced, "qkv", r.qkv)
    if layer.qkv_bias is not None:
        qkv = qkv + layer.qkv_bias
    parts = qkv.reshape(nh + 2 * nkv, HEAD_DIM)
    r.q = orc.rope(parts[:nh], pos, cfg.theta)
    r.k = orc.rope(parts[nh:nh + nkv], pos, cfg.theta)
    r.v = parts[nh + nkv:].copy()
    pg, slot = page_table[pos // cfg.page], pos % cfg.page
    k_cache[pg, :, slot, :] = _take(forced, "k", to_half_bits(r.k))
    v_cache[pg, :, slot, :] = _take(forced, "v", to_half_bits(r.v))
    q = _take(forced, "q", to_half_bits(r.q))
    r.attn, r.a_attn = orc.attn_decode(q, k_cache, v_cache, page_table, pos + 1, nkv, cfg.page,
                                       1.0 / np.sqrt(float(HEAD_DIM)))
    attn = _take(forced, "attn", to_half_bits(r.attn))
    r.o, r.a_o = orc.gemv(layer.o.q, layer.o.s, np.asarray(attn).reshape(-1), G)
    r.h_mid = h + _take(forced, "o", r.o)
    h_mid = _take(forced, "h_mid", r.h_mid)
    r.x2 = orc.rmsnorm(h_mid, layer.mlp_norm, cfg.eps)
    x2 = _take(forced, "x2", to_half_bits(r.x2))
    r.gu, r.a_gu = orc.gemv(layer.gateup.q, layer.gateup.s, x2, G)
    r.m = orc.silu_gate(r.gu)
    m = _take(forced, "m", to_half_bits(r.m))
    r.d, r.a_d = orc.gemv(layer.down.q, layer.down.s, m, G)
    r.h_out = h_mid + _take(forced, "d", r.d)
    return r


def final_logits(h: np.ndarray, final_norm: np.ndarray, lm: Proj, cfg: Config, orc=None, forced_xf=None):
    """(x_f fp64 (stored fp16), logits fp64, A, argmax) after the last layer;
    forced_xf (fp16 bits) replaces the stored x_f as the lm_head input."""
    orc = orc or default()
    xf = orc.rmsnorm(h, final_norm, cfg.eps)
    xin = to_half_bits(xf) if forced_xf is None else forced_xf
    y, a = orc.gemv(lm.q, lm.s, xin, cfg.group)
    return xf, y, a, orc.argmax(y)


def embed_row(table_bits: np.ndarray, token: int) -> np.ndarray:
    """Residual stream at the first layer: the token's fp16 embedding row."""
    return half_bits_to_double(table_bits[int(token)])
