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
    x1: np.ndarray = field(default=None)       # fp16 bits
    qkv: np.ndarray = field(default=None)      # fp64 (bias added)
    a_qkv: np.ndarray = field(default=None)    # sum |w x| of the qkv rows
    q: np.ndarray = field(default=None)        # fp64 rotated [nh, 128]
    k: np.ndarray = field(default=None)        # fp64 rotated [nkv, 128]
    v: np.ndarray = field(default=None)        # fp64 [nkv, 128]
    attn: np.ndarray = field(default=None)     # fp64 [nh, 128]
    a_attn: np.ndarray = field(default=None)
    o: np.ndarray = field(default=None)
    a_o: np.ndarray = field(default=None)
    h_mid: np.ndarray = field(default=None)
    x2: np.ndarray = field(default=None)       # fp16 bits
    gu: np.ndarray = field(default=None)       # fp64 [2I]
    a_gu: np.ndarray = field(default=None)
    m: np.ndarray = field(default=None)        # fp64 [I]
    d: np.ndarray = field(default=None)
    a_d: np.ndarray = field(default=None)
    h_out: np.ndarray = field(default=None)


def decoder_layer(h: np.ndarray, layer: Layer, cfg: Config, pos: int, k_cache: np.ndarray,
                  v_cache: np.ndarray, page_table: np.ndarray, orc=None) -> LayerResult:
    """One layer for the token at position pos.  h is the fp64 residual
    stream; k_cache / v_cache (fp16 bits [pages, nkv, page, 128]) hold the
    earlier tokens and receive this token's k and v (modified in place)."""
    orc = orc or default()
    r = LayerResult()
    nh, nkv, G = cfg.n_heads, cfg.n_kv, cfg.group
    r.x1 = to_half_bits(orc.rmsnorm(h, layer.attn_norm, cfg.eps))
    r.qkv, r.a_qkv = orc.gemv(layer.qkv.q, layer.qkv.s, r.x1, G)
    if layer.qkv_bias is not None:
        r.qkv = r.qkv + layer.qkv_bias
    parts = r.qkv.reshape(nh + 2 * nkv, HEAD_DIM)
    r.q = orc.rope(parts[:nh], pos, cfg.theta)
    r.k = orc.rope(parts[nh:nh + nkv], pos, cfg.theta)
    r.v = parts[nh + nkv:].copy()
    pg, slot = page_table[pos // cfg.page], pos % cfg.page
    k_cache[pg, :, slot, :] = to_half_bits(r.k)
    v_cache[pg, :, slot, :] = to_half_bits(r.v)
    r.attn, r.a_attn = orc.attn_decode(to_half_bits(r.q), k_cache, v_cache, page_table, pos + 1, nkv, cfg.page,
                                       1.0 / np.sqrt(float(HEAD_DIM)))
    r.o, r.a_o = orc.gemv(layer.o.q, layer.o.s, to_half_bits(r.attn).reshape(-1), G)
    r.h_mid = h + r.o
    r.x2 = to_half_bits(orc.rmsnorm(r.h_mid, layer.mlp_norm, cfg.eps))
    r.gu, r.a_gu = orc.gemv(layer.gateup.q, layer.gateup.s, r.x2, G)
    r.m = orc.silu_gate(r.gu)
    r.d, r.a_d = orc.gemv(layer.down.q, layer.down.s, to_half_bits(r.m), G)
    r.h_out = r.h_mid + r.d
    return r


def final_logits(h: np.ndarray, final_norm: np.ndarray, lm: Proj, cfg: Config, orc=None):
    """(x_f fp16 bits, logits fp64, A, argmax) after the last layer."""
    orc = orc or default()
    xf = to_half_bits(orc.rmsnorm(h, final_norm, cfg.eps))
    y, a = orc.gemv(lm.q, lm.s, xf, cfg.group)
    return xf, y, a, orc.argmax(y)


def embed_row(table_bits: np.ndarray, token: int) -> np.ndarray:
    """Residual stream at the first layer: the token's fp16 embedding row."""
    return half_bits_to_double(table_bits[int(token)])
