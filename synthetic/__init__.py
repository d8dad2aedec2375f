"""Seeded synthetic inputs for the INT4 weight-only GEMV (shared by tests,
the oracle checks and the benchmark).

This module only draws random numbers; it holds none of the method's
arithmetic.  Every draw comes from numpy's Philox counter-based generator keyed
by the seed, in a fixed order: nibbles, then scales, then activations.

Recipe (the pages give the model dimensions -- "How To Build Your Own LLM
Runtime From Scratch", aitrending.vip, section 技术解析, first bullet: 28 layers,
hidden 3584, MLP width 18944, vocabulary 152064 -- but no weights and no value
distributions; the distributions below are the workload definition's):

  * q  ~ uniform on {0..15}, i.i.d. per weight (zero point 8 is applied by the
    method, not here);
  * s  ~ uniform on [s_lo, s_hi] drawn in float32, rounded to fp16;
  * x  ~ N(0, 1) drawn in float32, rounded to fp16.

Trained Qwen2.5-Coder-7B weights are not available and are not needed: the
GEMV has no data-dependent control flow, so uniform nibbles time the same as
real ones and exercise every nibble value.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HIDDEN = 3584
MLP = 18944
VOCAB = 152064
LAYERS = 28
QKV = 4608
GROUP = 128
PROMPT = 512   # prompt tokens of the prefill workload (the pages' 512-token first-token latency)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=int(seed)))


def _nibbles(rng: np.random.Generator, count: int) -> np.ndarray:
    """`count` i.i.d. uniform values in {0..15} (one per byte)."""
    words = (count + 7) // 8
    b = rng.bit_generator.random_raw(words).view(np.uint8)[:count]
    np.bitwise_and(b, 15, out=b)
    return b


def _scales(rng: np.random.Generator, count: int, lo: float, hi: float) -> np.ndarray:
    u = rng.random(count, dtype=np.float32)
    return (u * np.float32(hi - lo) + np.float32(lo)).astype(np.float16).view(np.uint16)


def _acts(rng: np.random.Generator, count: int) -> np.ndarray:
    return rng.standard_normal(count, dtype=np.float32).astype(np.float16).view(np.uint16)


def logical(seed: int, n: int, k: int, group: int, s_lo: float = 0.001, s_hi: float = 0.02):
    """Logical inputs: q uint8 [n, k], s fp16 bits uint16 [n, k/group], x fp16 bits [k]."""
    rng = _rng(seed)
    q = _nibbles(rng, n * k).reshape(n, k)
    s = _scales(rng, n * (k // group), s_lo, s_hi).reshape(n, k // group)
    x = _acts(rng, k)
    return q, s, x


def packed_random(seed: int, weight_bytes: int, scale_count: int, k: int,
                  s_lo: float = 0.001, s_hi: float = 0.02):
    """Inputs drawn directly in packed form, for shapes without padding slots:
    uniform random weight bytes (two i.i.d. uniform nibbles each), scale_count
    fp16 scales, and x.  Returns (pw uint8 [weight_bytes], ps uint8
    [2*scale_count], x fp16 bits [k])."""
    rng = _rng(seed)
    pw = rng.bit_generator.random_raw((weight_bytes + 7) // 8).view(np.uint8)[:weight_bytes]
    ps = _scales(rng, scale_count, s_lo, s_hi).view(np.uint8)
    x = _acts(rng, k)
    return np.ascontiguousarray(pw), ps, x


def prompt_acts(seed: int, m: int, k: int) -> np.ndarray:
    """A block of m token activation rows for the prefill product: fp16 bits
    [m, k], N(0, 1) drawn in float32 and rounded to fp16, row after row."""
    return _acts(_rng(seed), m * k).reshape(m, k)


@dataclass(frozen=True)
class Proj:
    """One projection of the decode-step linear sweep."""
    name: str
    kind: str          # "plain" | "gateup" | "lmhead"
    n: int             # output rows (gate/up: 2 * MLP width)
    k: int
    group: int
    seed: int


# Per-projection seeds: layer l, projection p in {0 qkv, 1 o, 2 gate/up, 3 down}
# uses 1000 + 10*l + p; lm_head uses 1280.
CONFIG_TINY = dict(name="tiny", kind="plain", n=512, k=256, group=64, seed=0, s_lo=0.005, s_hi=0.02)
CONFIG_DOWN = dict(name="down", kind="plain", n=HIDDEN, k=MLP, group=GROUP, seed=1, s_lo=0.001, s_hi=0.02)
CONFIG_GATEUP = dict(name="gateup", kind="gateup", n=2 * MLP, k=HIDDEN, group=GROUP, seed=2,
                     s_lo=0.001, s_hi=0.02)
CONFIG_LMHEAD = dict(name="lmhead", kind="lmhead", n=VOCAB, k=HIDDEN, group=GROUP, seed=3,
                     s_lo=0.001, s_hi=0.02)


def prefill_projections(layers: int = LAYERS) -> list[Proj]:
    """The 28 layers' four prefill products in order (lm_head runs as the
    decode GEMV on the last prompt token).  Weights of layer l, projection p
    use seed 2000 + 10*l + p; the token block feeding it uses that seed + 5."""
    out = []
    for l in range(layers):
        out.append(Proj(f"L{l}.qkv", "plain", QKV, HIDDEN, GROUP, 2000 + 10 * l + 0))
        out.append(Proj(f"L{l}.o", "plain", HIDDEN, HIDDEN, GROUP, 2000 + 10 * l + 1))
        out.append(Proj(f"L{l}.gateup", "gateup", 2 * MLP, HIDDEN, GROUP, 2000 + 10 * l + 2))
        out.append(Proj(f"L{l}.down", "plain", HIDDEN, MLP, GROUP, 2000 + 10 * l + 3))
    return out


def sweep_projections(layers: int = LAYERS) -> list[Proj]:
    """The 28-layer decode-step sweep in decode order, then lm_head."""
    out = []
    for l in range(layers):
        out.append(Proj(f"L{l}.qkv", "plain", QKV, HIDDEN, GROUP, 1000 + 10 * l + 0))
        out.append(Proj(f"L{l}.o", "plain", HIDDEN, HIDDEN, GROUP, 1000 + 10 * l + 1))
        out.append(Proj(f"L{l}.gateup", "gateup", 2 * MLP, HIDDEN, GROUP, 1000 + 10 * l + 2))
        out.append(Proj(f"L{l}.down", "plain", HIDDEN, MLP, GROUP, 1000 + 10 * l + 3))
    out.append(Proj("lm_head", "lmhead", VOCAB, HIDDEN, GROUP, 1280))
    return out


# Decoder of the full decode step (the pages' model: 28 query heads over 4 KV
# heads of 128 give the 4608-wide fused QKV projection).
HEADS = 28
KV_HEADS = 4
PAGE = 16
MAX_CTX = 4096


def norm_weights(seed: int, n: int) -> np.ndarray:
    """RMSNorm weights: U[0.5, 1.5] drawn in float32, rounded to fp16 (bits)."""
    return _scales(_rng(seed), n, 0.5, 1.5)


def step_model(seed: int, *, hidden: int, n_heads: int, n_kv: int, inter: int, vocab: int, group: int,
               layers: int, bias: bool = False, s_lo: float = 0.001, s_hi: float = 0.02,
               embed: bool = True) -> dict:
    """Logical weights of a small decoder for the full-step tests.

    Layer l draws from seed * 1000 + 10 * l + p with p = 0 qkv, 1 o_proj,
    2 gate/up, 3 down (nibbles then scales, as `logical`), 4 attention norm,
    5 MLP norm, 6 qkv bias; the embedding table, final norm and lm_head use
    seed * 1000 + 900, 901, 902 (embed=False skips the table).  Norm weights ~ U[0.5, 1.5] and embeddings
    ~ N(0, 1) (float32 draws rounded to fp16); biases ~ N(0, 0.5) in float32.
    Returns plain arrays: {"embed", "final_norm", "lm": (q, s), "layers":
    [{"attn_norm", "qkv", "qkv_bias", "o", "mlp_norm", "gateup", "down"}]}."""
    def proj(sd, n, k):
        rng = _rng(sd)
        q = _nibbles(rng, n * k).reshape(n, k)
        s = _scales(rng, n * (k // group), s_lo, s_hi).reshape(n, k // group)
        return q, s

    def norm(sd, n):
        return norm_weights(sd, n)

    base = seed * 1000
    qkv_rows = (n_heads + 2 * n_kv) * 128
    out = {"layers": []}
    for l in range(layers):
        b = base + 10 * l
        layer = {
            "qkv": proj(b + 0, qkv_rows, hidden),
            "o": proj(b + 1, hidden, n_heads * 128),
            "gateup": proj(b + 2, 2 * inter, hidden),
            "down": proj(b + 3, hidden, inter),
            "attn_norm": norm(b + 4, hidden),
            "mlp_norm": norm(b + 5, hidden),
            "qkv_bias": (_rng(b + 6).standard_normal(qkv_rows, dtype=np.float32) * np.float32(0.5)) if bias else None,
        }
        out["layers"].append(layer)
    out["embed"] = _acts(_rng(base + 900), vocab * hidden).reshape(vocab, hidden) if embed else None
    out["final_norm"] = norm(base + 901, hidden)
    out["lm"] = proj(base + 902, vocab, hidden)
    return out


def kv_prefix(seed: int, num_pages: int, n_kv: int, page: int) -> tuple[np.ndarray, np.ndarray]:
    """Cache contents standing in for earlier tokens of the sequence: fp16 bits
    [num_pages, n_kv, page, 128] for K then V, N(0, 1) rounded to fp16."""
    rng = _rng(seed)
    shape = (num_pages, n_kv, page, 128)
    count = int(np.prod(shape))
    return _acts(rng, count).reshape(shape), _acts(rng, count).reshape(shape)


def page_table(seed: int, num_pages: int, entries: int) -> np.ndarray:
    """A random assignment of distinct physical pages to the logical pages."""
    return _rng(seed).permutation(num_pages).astype(np.int32)[:entries]


def half_bits_uniform(seed: int, count: int, lo_exp: int = 14) -> np.ndarray:
    """Cheap fp16 bit patterns for very large tables: random sign and
    mantissa with a fixed exponent (magnitudes in [2^(lo_exp-15), 2^(lo_exp-14)),
    i.e. [0.5, 1) by default)."""
    raw = _rng(seed).bit_generator.random_raw((count + 3) // 4).view(np.uint16)[:count]
    return (raw & np.uint16(0x83FF)) | np.uint16(lo_exp << 10)


def residual(seed: int, n: int, scale: float = 4.0) -> np.ndarray:
    """A residual-stream vector: N(0, scale^2) drawn in float32."""
    return (_rng(seed).standard_normal(n, dtype=np.float32) * np.float32(scale)).astype(np.float32)
