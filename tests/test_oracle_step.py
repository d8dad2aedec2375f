"""Pins of the full-step oracle (oracle/step.py), no GPU.

The composition is checked against an independent dense numpy formulation
(dequantized matrices, complex-number rotary embedding, scipy softmax over the
gathered cache), against closed forms (zero projections leave the residual
stream unchanged; a one-token context returns V; position 0 leaves k
unrotated) and against the cache-slot rule.  Plausible wiring mistakes are
planted in copies of the module and must each fail a pin."""
from __future__ import annotations

import importlib.util
import os
import sys

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synthetic
from oracle import step as ostep

CFG = ostep.Config(hidden=256, n_heads=4, n_kv=2, inter=512, group=64, page=16, eps=1e-6, theta=1e6)
MAX_CTX, PAGES = 64, 6


def _half(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def _r16(v):
    return np.asarray(v, np.float64).astype(np.float16).astype(np.float64)


def model(seed=3, bias=True, layers=1):
    m = synthetic.step_model(seed, hidden=CFG.hidden, n_heads=CFG.n_heads, n_kv=CFG.n_kv, inter=CFG.inter,
                             vocab=300, group=CFG.group, layers=layers, bias=bias)
    out = []
    for L in m["layers"]:
        out.append(ostep.Layer(attn_norm=L["attn_norm"], qkv=ostep.Proj(*L["qkv"]), o=ostep.Proj(*L["o"]),
                               mlp_norm=L["mlp_norm"], gateup=ostep.Proj(*L["gateup"]),
                               down=ostep.Proj(*L["down"]),
                               qkv_bias=None if L["qkv_bias"] is None else L["qkv_bias"].astype(np.float64)))
    return m, out


def cache(seed=4):
    kc, vc = synthetic.kv_prefix(seed, PAGES, CFG.n_kv, CFG.page)
    table = synthetic.page_table(seed, PAGES, MAX_CTX // CFG.page)
    return kc.copy(), vc.copy(), table


def _deq(P):
    return (P.q.astype(np.float64) - 8.0) * np.repeat(_half(P.s), CFG.group, axis=1)


def _rms(v, g):
    return v / np.sqrt(np.mean(v * v) + CFG.eps) * _half(g)


def _rope_complex(x, pos):
    half = x.shape[-1] // 2
    ang = pos * CFG.theta ** (-2.0 * np.arange(half) / x.shape[-1])
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def layer_numpy(h, L, pos, kc, vc, table):
    nh, nkv = CFG.n_heads, CFG.n_kv
    x1u = _rms(h, L.attn_norm)
    x1 = _r16(x1u)
    qkv = _deq(L.qkv) @ x1
    parts = (qkv + (L.qkv_bias if L.qkv_bias is not None else 0.0)).reshape(nh + 2 * nkv, 128)
    q = _rope_complex(parts[:nh], pos)
    k = _rope_complex(parts[nh:nh + nkv], pos)
    v = parts[nh + nkv:]
    kc, vc = kc.copy(), vc.copy()
    kc[table[pos // CFG.page], :, pos % CFG.page] = ostep.to_half_bits(k)
    vc[table[pos // CFG.page], :, pos % CFG.page] = ostep.to_half_bits(v)
    toks = np.arange(pos + 1)
    K = _half(kc[table[toks // CFG.page], :, toks % CFG.page])  # [t, nkv, 128]
    V = _half(vc[table[toks // CFG.page], :, toks % CFG.page])
    att = np.empty((nh, 128))
    for hh in range(nh):
        g = hh // (nh // nkv)
        p = softmax(K[:, g] @ _r16(q[hh]) / np.sqrt(128.0))
        att[hh] = p @ V[:, g]
    o = _deq(L.o) @ _r16(att).reshape(-1)
    h_mid = h + o
    x2u = _rms(h_mid, L.mlp_norm)
    x2 = _r16(x2u)
    gu = _deq(L.gateup) @ x2
    gate, up = gu[:CFG.inter], gu[CFG.inter:]
    m = gate / (1.0 + np.exp(-gate)) * up
    d = _deq(L.down) @ _r16(m)
    return dict(x1=x1u, qkv=qkv, q=q, k=k, v=v, attn=att, o=o, h_mid=h_mid, x2=x2u, gu=gu, m=m, d=d,
                h_out=h_mid + d, kc=kc, vc=vc)


def _close(a, b, rtol=1e-10, atol=1e-12):
    return np.allclose(a, b, rtol=rtol, atol=atol)


def pin_step_layer_vs_numpy(st, orc):
    m, layers = model()
    kc, vc, table = cache()
    h = _half(m["embed"][7]) * 3.0
    pos = 37
    ref = layer_numpy(h, layers[0], pos, kc, vc, table)
    r = st.decoder_layer(h, layers[0], CFG, pos, kc, vc, table, orc=orc)
    for name in ("x1", "qkv", "q", "k", "v", "attn", "o", "h_mid", "x2", "gu", "m", "d", "h_out"):
        assert _close(getattr(r, name), ref[name]), name
    assert np.array_equal(kc, ref["kc"]) and np.array_equal(vc, ref["vc"])


def pin_step_residual_identity(st, orc):
    """All-zero o_proj and down weights (nibble 8) leave h unchanged exactly."""
    _, layers = model(seed=5)
    L = layers[0]
    L.o = ostep.Proj(np.full_like(L.o.q, 8), L.o.s)
    L.down = ostep.Proj(np.full_like(L.down.q, 8), L.down.s)
    kc, vc, table = cache(6)
    h = np.random.default_rng(1).standard_normal(CFG.hidden)
    r = st.decoder_layer(h, L, CFG, 20, kc, vc, table, orc=orc)
    assert np.array_equal(r.h_mid, h) and np.array_equal(r.h_out, h)
    assert not np.array_equal(r.attn, 0.0 * r.attn)


def pin_step_first_token(st, orc):
    """At position 0: k is unrotated, and attention over one token returns
    that token's V (each query head the V of its KV head)."""
    _, layers = model(seed=7)
    kc, vc, table = cache(8)
    h = np.random.default_rng(2).standard_normal(CFG.hidden)
    r = st.decoder_layer(h, layers[0], CFG, 0, kc, vc, table, orc=orc)
    nh, nkv = CFG.n_heads, CFG.n_kv
    parts = (r.qkv + layers[0].qkv_bias).reshape(nh + 2 * nkv, 128)
    assert np.array_equal(r.k, parts[nh:nh + nkv]) and np.array_equal(r.q, parts[:nh])
    vh = _r16(parts[nh + nkv:])
    for hh in range(nh):
        assert np.array_equal(r.attn[hh], vh[hh // (nh // nkv)])


def pin_step_cache_slot(st, orc):
    """Only the slot of token pos changes, in the page the table names."""
    _, layers = model(seed=9)
    kc, vc, table = cache(10)
    k0, v0 = kc.copy(), vc.copy()
    pos = 49
    r = st.decoder_layer(np.ones(CFG.hidden), layers[0], CFG, pos, kc, vc, table, orc=orc)
    pg, sl = table[pos // CFG.page], pos % CFG.page
    mask = np.zeros(kc.shape, bool)
    mask[pg, :, sl, :] = True
    assert np.array_equal(kc[~mask], k0[~mask]) and np.array_equal(vc[~mask], v0[~mask])
    assert np.array_equal(kc[pg, :, sl], ostep.to_half_bits(r.k))
    assert np.array_equal(vc[pg, :, sl], ostep.to_half_bits(r.v))


def pin_step_final_logits(st, orc):
    m, _ = model(seed=11)
    h = np.random.default_rng(3).standard_normal(CFG.hidden) * 2.0
    lm = ostep.Proj(*m["lm"])
    xf, y, a, best = st.final_logits(h, m["final_norm"], lm, CFG, orc=orc)
    assert _close(xf, _rms(h, m["final_norm"]))
    x_ref = _r16(xf)
    y_ref = _deq(lm) @ x_ref
    assert _close(y, y_ref) and best == int(np.argmax(y_ref))
    assert _close(a, np.abs(_deq(lm) * x_ref).sum(axis=1))


def pin_step_forcing(st, orc):
    """Teacher forcing: forcing every stage with the layer's own stored values
    changes nothing; a forced zero attention output gives o = 0 and leaves the
    residual stream unchanged; a forced x2 is what the gate/up product reads."""
    _, layers = model(seed=13)
    L = layers[0]
    kc, vc, table = cache(14)
    h = np.random.default_rng(4).standard_normal(CFG.hidden)
    pos = 29
    k1, v1 = kc.copy(), vc.copy()
    r0 = st.decoder_layer(h, L, CFG, pos, k1, v1, table, orc=orc)
    hb = ostep.to_half_bits
    forced = dict(x1=hb(r0.x1), qkv=r0.qkv, q=hb(r0.q), k=hb(r0.k), v=hb(r0.v), attn=hb(r0.attn), o=r0.o,
                  h_mid=r0.h_mid, x2=hb(r0.x2), m=hb(r0.m), d=r0.d)
    k2, v2 = kc.copy(), vc.copy()
    r1 = st.decoder_layer(h, L, CFG, pos, k2, v2, table, orc=orc, forced=forced)
    for name in ("x1", "qkv", "q", "k", "v", "attn", "o", "h_mid", "x2", "gu", "m", "d", "h_out"):
        assert np.array_equal(getattr(r0, name), getattr(r1, name)), name
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    r2 = st.decoder_layer(h, L, CFG, pos, kc.copy(), vc.copy(), table, orc=orc,
                          forced=dict(attn=np.zeros((CFG.n_heads, 128), np.uint16)))
    assert np.array_equal(r2.o, np.zeros(CFG.hidden)) and np.array_equal(r2.h_mid, h)
    x2 = hb(np.random.default_rng(5).standard_normal(CFG.hidden))
    r3 = st.decoder_layer(h, L, CFG, pos, kc.copy(), vc.copy(), table, orc=orc, forced=dict(x2=x2))
    assert np.array_equal(r3.gu, orc.gemv(L.gateup.q, L.gateup.s, x2, CFG.group)[0])


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_step_")]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_step_pin(pin):
    pin(ostep, oracle.default())


SRC = os.path.join(os.path.dirname(oracle.__file__), "step.py")

MUTANTS = [
    ("v_from_k_part", "r.v = parts[nh + nkv:].copy()", "r.v = parts[nh:nh + nkv].copy()"),
    ("k_unrotated", "r.k = orc.rope(parts[nh:nh + nkv], pos, cfg.theta)", "r.k = parts[nh:nh + nkv].copy()"),
    ("q_position_shift", "r.q = orc.rope(parts[:nh], pos, cfg.theta)", "r.q = orc.rope(parts[:nh], pos + 1, cfg.theta)"),
    ("context_short", "page_table, pos + 1, nkv", "page_table, max(pos, 1), nkv"),
    ("attn_residual_dropped", "r.h_mid = h + _take(forced, \"o\", r.o)", "r.h_mid = _take(forced, \"o\", r.o)"),
    ("mlp_norm_of_layer_input", "orc.rmsnorm(h_mid, layer.mlp_norm", "orc.rmsnorm(h, layer.mlp_norm"),
    ("mlp_residual_base", "r.h_out = h_mid + _take(forced, \"d\", r.d)", "r.h_out = h + _take(forced, \"d\", r.d)"),
    ("bias_dropped", "qkv = qkv + layer.qkv_bias", "qkv = qkv"),
    ("cache_slot_shift", "pos % cfg.page", "(pos + 1) % cfg.page"),
    ("norm_weights_swapped", "orc.rmsnorm(h, layer.attn_norm", "orc.rmsnorm(h, layer.mlp_norm"),
    ("final_norm_dropped", "xf = orc.rmsnorm(h, final_norm, cfg.eps)", "xf = h"),
    ("attn_transposed_into_o", "np.asarray(attn).reshape(-1)", "np.asarray(attn).T.reshape(-1)"),
    ("forced_attn_ignored", 'attn = _take(forced, "attn", to_half_bits(r.attn))', "attn = to_half_bits(r.attn)"),
    ("forced_x2_ignored", 'x2 = _take(forced, "x2", to_half_bits(r.x2))', "x2 = to_half_bits(r.x2)"),
    ("down_input_from_gate", "r.d, r.a_d = orc.gemv(layer.down.q, layer.down.s, m, G)",
     "r.d, r.a_d = orc.gemv(layer.down.q, layer.down.s, to_half_bits(r.gu[:cfg.inter]), G)"),
]


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_step_mutant_is_caught(name, find, repl, tmp_path):
    text = open(SRC).read()
    assert find in text, find
    mutated = text.replace(find, repl).replace("from . import default", "from oracle import default")
    path = tmp_path / f"step_{name}.py"
    path.write_text(mutated)
    spec = importlib.util.spec_from_file_location(f"step_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod  # dataclasses look their module up by name
    try:
        spec.loader.exec_module(mod)
    finally:
        sys.modules.pop(spec.name, None)
    failed = []
    for pin in PINS:
        try:
            pin(mod, oracle.default())
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
