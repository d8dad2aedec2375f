"""Pins that tie the CPU oracle to facts outside itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with something the pages, the mathematics or an independent library
routine fixes:

  * the hand-derived packing and GEMV example in tests/golden/ (bytes and
    products worked out by hand from the layout rules);
  * IEEE binary16 decoding checked against numpy's float16 for every pattern;
  * the plain GEMV and the prefill GEMM checked against numpy's float64
    matrix product of the dequantized matrix (a library routine, independent
    of the C loops);
  * closed forms (zero point, constant nibbles, one-hot activations, one-hot
    token rows selecting weight columns);
  * exact invariants (power-of-two scaling, A >= |y|);
  * silu against scipy's logistic function, argmax against numpy.argmax;
  * decode attention against scipy's softmax on the gathered KV cache, and its
    closed forms (uniform weights, one token, one dominating key) and
    page-layout invariance.

The same pins run against deliberately mutated copies of the oracle
(test_oracle_mutants.py) to show that each plausible mistake trips one.
"""
from __future__ import annotations

import os

import numpy as np
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pack_2x64_g32.txt")


def load_golden(path: str = GOLDEN) -> dict:
    out: dict = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key in ("n", "k", "group"):
                out[key] = int(vals[0])
            elif key.endswith("_pw") or key.endswith("_ps"):
                out.setdefault(key, []).extend(int(v, 16) for v in vals)
            else:
                out[key] = [float(v) for v in vals]
    for key in list(out):
        if key.endswith("_pw") or key.endswith("_ps"):
            out[key] = np.array(out[key], np.uint8)
    return out


def golden_logical():
    """The golden matrix as described in words in the fixture header."""
    k = 64
    kk = np.arange(k)
    q = np.stack([kk % 16, 15 - (kk % 16)]).astype(np.uint8)
    s = np.array([[0x3C00, 0x4000], [0x3800, 0xBC00]], np.uint16)
    return q, s


def _h(v) -> np.ndarray:
    """float values -> fp16 bit patterns (numpy's conversion)."""
    return np.asarray(v, np.float16).view(np.uint16)


def _dequant_numpy(q, s_bits, group):
    s = s_bits.view(np.float16).astype(np.float64)
    return (q.astype(np.float64) - 8.0) * np.repeat(s, group, axis=1)


# --------------------------------------------------------------------------- pins


def pin_half_decode_all(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_golden_pack(orc):
    g = load_golden()
    q, s = golden_logical()
    pw, ps = orc.pack(q, s, g["group"], gateup=False)
    assert np.array_equal(pw, g["plain_pw"]), "plain weight bytes differ from the hand-derived ones"
    assert np.array_equal(ps, g["plain_ps"]), "plain scale bytes differ from the hand-derived ones"
    pw, ps = orc.pack(q, s, g["group"], gateup=True)
    assert np.array_equal(pw, g["gateup_pw"]), "gate/up weight bytes differ"
    assert np.array_equal(ps, g["gateup_ps"]), "gate/up scale bytes differ"


def pin_golden_unpack(orc):
    g = load_golden()
    q, s = golden_logical()
    for layout in ("plain", "gateup"):
        uq, us = orc.unpack(g[layout + "_pw"], g[layout + "_ps"], g["n"], g["k"], g["group"],
                            gateup=(layout == "gateup"))
        assert np.array_equal(uq, q), layout
        assert np.array_equal(us, s), layout


def pin_golden_gemv(orc):
    g = load_golden()
    q, s = golden_logical()
    ones = _h(np.ones(g["k"]))
    onehot = _h(np.eye(g["k"])[33])
    for x, yk, ak in ((ones, "y_ones", "a_ones"), (onehot, "y_onehot33", "a_onehot33")):
        y, a = orc.gemv(q, s, x, g["group"])
        assert np.array_equal(y, g[yk]), (yk, y)
        assert np.array_equal(a, g[ak]), (ak, a)
        for layout in ("plain", "gateup"):
            y2, a2 = orc.gemv_packed(g[layout + "_pw"], g[layout + "_ps"], x, g["n"], g["k"],
                                     g["group"], gateup=(layout == "gateup"))
            assert np.array_equal(y2, g[yk]), (layout, yk, y2)
            assert np.array_equal(a2, g[ak]), (layout, ak, a2)


def pin_pack_roundtrip(orc):
    rng = np.random.default_rng(7)
    for n, k, group, gateup in ((1, 32, 32, False), (3, 64, 32, False), (5, 96, 32, False),
                                (7, 128, 64, False), (9, 256, 128, False), (2, 64, 32, True),
                                (6, 128, 64, True), (10, 256, 128, True), (16, 64, 64, True)):
        q = rng.integers(0, 16, (n, k), dtype=np.uint8)
        s = _h(rng.uniform(-2, 2, (n, k // group)))
        pw, ps = orc.pack(q, s, group, gateup)
        wb, sb = orc.packed_sizes(n, k, group, gateup)
        assert pw.size == wb and ps.size == sb
        uq, us = orc.unpack(pw, ps, n, k, group, gateup)
        assert np.array_equal(uq, q), (n, k, group, gateup)
        assert np.array_equal(us, s), (n, k, group, gateup)


def pin_packed_sizes(orc):
    # closed forms: ceil(n/4) tiles of k/2 * 4 bytes, and (k/G) * 8 scale bytes
    assert orc.packed_sizes(512, 256, 64) == (128 * 512, 128 * 4 * 8)
    assert orc.packed_sizes(3584, 18944, 128) == (3584 * 18944 // 2, 896 * 148 * 8)
    assert orc.packed_sizes(5, 32, 32) == (2 * 64, 2 * 8)
    assert orc.packed_sizes(6, 32, 32, True) == (2 * 64, 2 * 8)    # halves of 3 rows, 1 tile each
    assert orc.packed_sizes(10, 32, 32, True) == (4 * 64, 4 * 8)   # halves of 5 rows, 2 tiles each


def pin_gemv_vs_numpy(orc):
    rng = np.random.default_rng(11)
    for n, k, group in ((512, 256, 64), (37, 384, 128), (6, 96, 32)):
        q = rng.integers(0, 16, (n, k), dtype=np.uint8)
        s = _h(rng.uniform(0.001, 0.02, (n, k // group)))
        x = _h(rng.standard_normal(k))
        w = _dequant_numpy(q, s, group)
        xf = x.view(np.float16).astype(np.float64)
        ref = w @ xf
        refa = np.abs(w) @ np.abs(xf)
        y, a = orc.gemv(q, s, x, group)
        assert np.all(np.abs(y - ref) <= 1e-12 * refa + 1e-300), (n, k, group)
        assert np.allclose(a, refa, rtol=1e-12, atol=0), (n, k, group)


def pin_closed_forms(orc):
    n, k, group = 5, 256, 64
    ones = _h(np.ones(k))
    one_s = _h(np.ones((n, k // group)))
    rng = np.random.default_rng(3)
    xr = _h(rng.integers(-4, 5, k))          # small integers: every sum exact
    s_r = _h(rng.uniform(0.001, 0.02, (n, k // group)))
    # zero point: q == 8 gives a zero matrix
    y, a = orc.gemv(np.full((n, k), 8, np.uint8), s_r, xr, group)
    assert np.all(y == 0) and np.all(a == 0)
    # q == 15, s == 1, x == 1  ->  7K
    y, _ = orc.gemv(np.full((n, k), 15, np.uint8), one_s, ones, group)
    assert np.all(y == 7 * k)
    # q == 0, s == 1  ->  -8 * sum(x)
    y, _ = orc.gemv(np.zeros((n, k), np.uint8), one_s, xr, group)
    assert np.all(y == -8 * xr.view(np.float16).astype(np.float64).sum())
    # q == 9, s == 0.5, x == 1  ->  K/2
    y, _ = orc.gemv(np.full((n, k), 9, np.uint8), _h(np.full((n, k // group), 0.5)), ones, group)
    assert np.all(y == k / 2)


def pin_onehot(orc):
    rng = np.random.default_rng(5)
    n, k, group = 9, 256, 64
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = _h(rng.uniform(-0.02, 0.02, (n, k // group)))
    sv = s.view(np.float16).astype(np.float64)
    for kk in (0, 1, 7, 8, group - 1, group, 2 * group + 3, k - 1):
        x = _h(np.eye(k)[kk])
        y, a = orc.gemv(q, s, x, group)
        expect = (q[:, kk].astype(np.float64) - 8.0) * sv[:, kk // group]
        assert np.array_equal(y, expect), kk
        assert np.array_equal(a, np.abs(expect)), kk


def pin_scaling(orc):
    rng = np.random.default_rng(9)
    n, k, group = 13, 384, 128
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = _h(rng.uniform(0.001, 0.02, (n, k // group)))
    x = _h(rng.standard_normal(k))
    x2 = _h(2.0 * x.view(np.float16).astype(np.float64))
    y, a = orc.gemv(q, s, x, group)
    y2, a2 = orc.gemv(q, s, x2, group)
    assert np.array_equal(y2, 2 * y) and np.array_equal(a2, 2 * a)
    assert np.all(a >= np.abs(y))
    # all terms non-negative -> A == y
    qp = rng.integers(8, 16, (n, k), dtype=np.uint8)
    xp = _h(np.abs(x.view(np.float16)))
    yp, ap = orc.gemv(qp, s, xp, group)
    assert np.array_equal(yp, ap)


def pin_rows_subset(orc):
    rng = np.random.default_rng(13)
    n, k, group = 21, 128, 32
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = _h(rng.uniform(0.001, 0.02, (n, k // group)))
    x = _h(rng.standard_normal(k))
    y, a = orc.gemv(q, s, x, group)
    rows = np.array([20, 0, 7, 7, 13], np.int64)
    yr, ar = orc.gemv(q, s, x, group, rows=rows)
    assert np.array_equal(yr, y[rows]) and np.array_equal(ar, a[rows])
    for gateup in (False, True):
        pw, ps = orc.pack(q[:20], s[:20], group, gateup)
        yp, ap = orc.gemv_packed(pw, ps, x, 20, k, group, gateup, rows=rows[rows < 20])
        assert np.array_equal(yp, y[rows[rows < 20]]) and np.array_equal(ap, a[rows[rows < 20]])


def pin_silu(orc):
    t = np.linspace(-20, 20, 4001)
    ref = t * scipy.special.expit(t)
    got = np.array([orc.silu(v) for v in t])
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)
    assert orc.silu(0.0) == 0.0
    # silu(-t) = silu(t) - t
    for v in (0.5, 2.399, 7.0, 19.0):
        assert abs(orc.silu(-v) - (orc.silu(v) - v)) <= 1e-14 * max(1.0, v)


def pin_silu_gate(orc):
    g = np.array([-3.0, 0.0, 1.5, 4.0])
    u = np.array([2.0, 5.0, -1.0, 0.25])
    h = orc.silu_gate(np.concatenate([g, u]))
    assert np.allclose(h, g * scipy.special.expit(g) * u, rtol=1e-14, atol=0)
    # gate rows come first: a zero up half gives zero regardless of the gate
    assert np.all(orc.silu_gate(np.concatenate([g, np.zeros(4)])) == 0)


def pin_argmax(orc):
    rng = np.random.default_rng(17)
    for _ in range(20):
        y = rng.standard_normal(1000)
        assert orc.argmax(y) == int(np.argmax(y))
    y = np.array([1.0, 3.0, 2.0, 3.0, 3.0])
    assert orc.argmax(y) == int(np.argmax(y)) == 1
    y = np.array([np.nan, -1.0, 5.0, np.nan, 5.0])
    assert orc.argmax(y) == 2


def pin_gemm_vs_numpy(orc):
    """The prefill product against numpy's float64 matrix product of the
    dequantized weights, for the logical and both packed layouts."""
    rng = np.random.default_rng(19)
    for m, n, k, group in ((7, 37, 384, 128), (3, 10, 256, 64), (1, 6, 96, 32)):
        q = rng.integers(0, 16, (n, k), dtype=np.uint8)
        s = _h(rng.uniform(0.001, 0.02, (n, k // group)))
        xm = _h(rng.standard_normal((m, k)))
        w = _dequant_numpy(q, s, group)
        xf = xm.view(np.float16).astype(np.float64)
        ref = xf @ w.T
        refa = np.abs(xf) @ np.abs(w).T
        y, a = orc.gemm(q, s, xm, group)
        assert y.shape == (m, n) and a.shape == (m, n)
        assert np.all(np.abs(y - ref) <= 1e-12 * refa + 1e-300), (m, n, k, group)
        assert np.allclose(a, refa, rtol=1e-12, atol=0), (m, n, k, group)
        for gateup in (False, True):
            if gateup and n % 2:
                continue
            pw, ps = orc.pack(q, s, group, gateup)
            yp, ap = orc.gemm_packed(pw, ps, xm, n, k, group, gateup)
            assert np.array_equal(yp, y) and np.array_equal(ap, a), (m, n, k, group, gateup)


def pin_gemm_onehot_rows(orc):
    """Token row m one-hot at input k_m selects column k_m of the weights:
    Y[m, n] = w[n, k_m] exactly (catches a transposed operand or a wrong x row)."""
    rng = np.random.default_rng(23)
    n, k, group = 12, 256, 64
    ks = np.array([0, 1, 7, 8, 63, 64, 130, 255])
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = _h(rng.uniform(-0.02, 0.02, (n, k // group)))
    sv = s.view(np.float16).astype(np.float64)
    xm = _h(np.eye(k)[ks])
    expect = ((q[:, ks].astype(np.float64) - 8.0) * sv[:, ks // group]).T
    y, a = orc.gemm(q, s, xm, group)
    assert np.array_equal(y, expect) and np.array_equal(a, np.abs(expect))
    for gateup in (False, True):
        pw, ps = orc.pack(q, s, group, gateup)
        yp, _ = orc.gemm_packed(pw, ps, xm, n, k, group, gateup)
        assert np.array_equal(yp, expect), gateup


def pin_gemm_rows_and_subsets(orc):
    """Token rows are independent: doubling one row of X doubles that row of Y
    only, equal rows give equal outputs, and the (token, weight) subsets pick
    the matching entries of the full product."""
    rng = np.random.default_rng(29)
    m, n, k, group = 6, 14, 128, 32
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = _h(rng.uniform(0.001, 0.02, (n, k // group)))
    xm = _h(rng.standard_normal((m, k)))
    xm[4] = xm[1]
    y, a = orc.gemm(q, s, xm, group)
    assert np.array_equal(y[4], y[1])
    x2 = xm.copy()
    x2[2] = _h(2.0 * xm[2].view(np.float16).astype(np.float64))
    y2, _ = orc.gemm(q, s, x2, group)
    assert np.array_equal(y2[2], 2 * y[2])
    keep = np.arange(m) != 2
    assert np.array_equal(y2[keep], y[keep])
    pw, ps = orc.pack(q, s, group, False)
    mr = np.array([5, 0, 3, 3], np.int64)
    nc = np.array([13, 2, 2, 0, 7], np.int64)
    ys, as_ = orc.gemm_packed(pw, ps, xm, n, k, group, False, mrows=mr, ncols=nc)
    assert np.array_equal(ys, y[np.ix_(mr, nc)]) and np.array_equal(as_, a[np.ix_(mr, nc)])


def _attn_numpy(q_bits, kc, vc, table, ctx, n_kv, page, scale):
    """softmax(scale Q K^T) V with numpy/scipy on the gathered cache."""
    n_heads, dim = q_bits.shape
    qf = q_bits.view(np.float16).astype(np.float64)
    t = np.arange(ctx)
    kf = kc.view(np.float16).astype(np.float64)[table[t // page], :, t % page, :]   # [ctx, n_kv, dim]
    vf = vc.view(np.float16).astype(np.float64)[table[t // page], :, t % page, :]
    group = n_heads // n_kv
    o = np.empty((n_heads, dim))
    a = np.empty((n_heads, dim))
    for h in range(n_heads):
        sc = scale * (kf[:, h // group, :] @ qf[h])
        p = scipy.special.softmax(sc)
        o[h] = p @ vf[:, h // group, :]
        a[h] = p @ np.abs(vf[:, h // group, :])
    return o, a


def _attn_inputs(rng, n_heads, n_kv, dim, page, pages, ctx):
    q = _h(rng.standard_normal((n_heads, dim)))
    kc = _h(rng.standard_normal((pages, n_kv, page, dim)))
    vc = _h(rng.standard_normal((pages, n_kv, page, dim)))
    table = rng.permutation(pages).astype(np.int32)[: (ctx + page - 1) // page]
    return q, kc, vc, table


def pin_attn_vs_numpy(orc):
    """Decode attention against numpy/scipy softmax on the gathered cache, with
    grouped KV heads, permuted page tables and ragged page tails."""
    rng = np.random.default_rng(37)
    for n_heads, n_kv, dim, page, ctx in ((4, 1, 16, 4, 13), (28, 4, 128, 16, 37), (6, 2, 8, 8, 8), (3, 3, 32, 16, 1)):
        pages = (ctx + page - 1) // page + 3
        q, kc, vc, table = _attn_inputs(rng, n_heads, n_kv, dim, page, pages, ctx)
        scale = 1.0 / np.sqrt(dim)
        o, a = orc.attn_decode(q, kc, vc, table, ctx, n_kv, page, scale)
        ro, ra = _attn_numpy(q, kc, vc, table, ctx, n_kv, page, scale)
        assert np.allclose(o, ro, rtol=1e-12, atol=1e-13), (n_heads, n_kv, ctx)
        assert np.allclose(a, ra, rtol=1e-12, atol=1e-13), (n_heads, n_kv, ctx)


def pin_attn_closed_forms(orc):
    """q = 0 averages V uniformly; one cached token returns its V exactly; one
    key that dominates by a huge score returns its V exactly (and needs the
    max subtracted before exp to stay finite)."""
    rng = np.random.default_rng(41)
    n_heads, n_kv, dim, page, ctx = 4, 2, 16, 8, 21
    q, kc, vc, table = _attn_inputs(rng, n_heads, n_kv, dim, page, 4, ctx)
    t = np.arange(ctx)
    vf = vc.view(np.float16).astype(np.float64)[table[t // page], :, t % page, :]
    o, a = orc.attn_decode(np.zeros_like(q), kc, vc, table, ctx, n_kv, page, 0.25)
    for h in range(n_heads):
        assert np.allclose(o[h], vf[:, h // 2, :].mean(axis=0), rtol=1e-13, atol=1e-15)
        assert np.allclose(a[h], np.abs(vf[:, h // 2, :]).mean(axis=0), rtol=1e-13, atol=1e-15)
    o, _ = orc.attn_decode(q, kc, vc, table, 1, n_kv, page, 0.25)
    for h in range(n_heads):
        assert np.array_equal(o[h], vf[0, h // 2, :])
    # token 11 gets key = 64 * q-direction: its score exceeds the others by far more than exp's range
    q1 = _h(np.ones((n_heads, dim)))
    kc2 = kc.copy()
    tstar = 11
    kc2[table[tstar // page], :, tstar % page, :] = _h(np.full((n_kv, dim), 64.0))
    o, _ = orc.attn_decode(q1, kc2, vc, table, ctx, n_kv, page, 1.0)
    assert np.all(np.isfinite(o))
    for h in range(n_heads):
        assert np.array_equal(o[h], vf[tstar, h // 2, :])


def pin_attn_page_layouts(orc):
    """The same logical cache laid out with another page size and another page
    order gives the same result bit for bit (the sum runs in token order)."""
    rng = np.random.default_rng(43)
    n_heads, n_kv, dim, ctx = 8, 2, 32, 45
    q = _h(rng.standard_normal((n_heads, dim)))
    k_log = _h(rng.standard_normal((ctx, n_kv, dim)))
    v_log = _h(rng.standard_normal((ctx, n_kv, dim)))
    outs = []
    for page, seed in ((4, 1), (16, 2), (64, 3)):
        npages = (ctx + page - 1) // page
        table = np.random.default_rng(seed).permutation(npages + 2).astype(np.int32)[:npages]
        kc = np.zeros((npages + 2, n_kv, page, dim), np.uint16)
        vc = np.zeros_like(kc)
        for t in range(ctx):
            kc[table[t // page], :, t % page, :] = k_log[t]
            vc[table[t // page], :, t % page, :] = v_log[t]
        outs.append(orc.attn_decode(q, kc, vc, table, ctx, n_kv, page, 0.2))
    for o, a in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(a, outs[0][1])


def pin_rmsnorm(orc):
    """RMSNorm: scale invariance (with eps scaled alike), constant vectors map
    to gamma, unit gamma gives a root-mean-square of 1 (eps = 0)."""
    rng = np.random.default_rng(47)
    n = 3584
    h = rng.standard_normal(n) * 3.0
    g = _h(rng.uniform(0.5, 1.5, n))
    gv = g.view(np.float16).astype(np.float64)
    out = orc.rmsnorm(h, g, 1e-6)
    assert np.allclose(orc.rmsnorm(4.0 * h, g, 16e-6), out, rtol=1e-14, atol=0)
    assert np.allclose(orc.rmsnorm(np.full(n, 2.5), g, 0.0), gv, rtol=1e-14, atol=0)
    ones = _h(np.ones(n))
    o1 = orc.rmsnorm(h, ones, 0.0)
    assert abs(np.sqrt(np.mean(o1 ** 2)) - 1.0) < 1e-14
    assert np.allclose(o1 * np.sqrt(np.mean(h ** 2)), h, rtol=1e-13, atol=0)


def pin_rmsnorm_given_and_sumsq_blocks(orc):
    """The norm with its sum of squares given: a unit mean square with eps = 0
    returns h * gamma exactly, a mean square of 4 halves it, and fed the sum of
    the block sums it is the plain RMSNorm.  Block sums: rows = 1 gives the
    squares, the blocks of a ragged length cover every value once, and a
    hand-worked case."""
    rng = np.random.default_rng(59)
    n = 1000
    h = rng.standard_normal(n) * 2.0
    g = _h(rng.uniform(0.5, 1.5, n))
    hg = h * g.view(np.float16).astype(np.float64)
    assert np.array_equal(orc.rmsnorm_given(h, g, float(n), 0.0), hg)
    assert np.array_equal(orc.rmsnorm_given(h, g, 4.0 * n, 0.0), hg / 2.0)
    for rows in (1, 4, 7, 1000, 1024):
        parts = orc.sumsq_blocks(h, rows)
        assert parts.size == -(-n // rows)
        assert np.allclose(orc.rmsnorm_given(h, g, float(np.sum(parts)), 1e-6), orc.rmsnorm(h, g, 1e-6),
                           rtol=1e-13, atol=0)
        assert abs(np.sum(parts) - np.sum(h ** 2)) <= 1e-12 * np.sum(h ** 2)
    assert np.array_equal(orc.sumsq_blocks(h, 1), h * h)
    assert np.array_equal(orc.sumsq_blocks(np.array([1.0, 2.0, 3.0, 4.0, 5.0]), 2), np.array([5.0, 25.0, 25.0]))


def pin_rope(orc):
    """RoPE against the complex-number form (x_i + j x_{i+d/2}) e^{j a_i},
    identity at position 0, norm preservation, composition of positions and
    dependence of q . k on the position difference only."""
    rng = np.random.default_rng(53)
    dim, theta = 128, 1e6
    x = rng.standard_normal((5, dim))
    for pos in (0, 1, 17, 4095):
        out = orc.rope(x, pos, theta)
        a = pos * theta ** (-np.arange(dim // 2) * 2.0 / dim)
        z = (x[:, : dim // 2] + 1j * x[:, dim // 2:]) * np.exp(1j * a)
        assert np.allclose(out[:, : dim // 2], z.real, rtol=0, atol=1e-12)
        assert np.allclose(out[:, dim // 2:], z.imag, rtol=0, atol=1e-12)
    assert np.array_equal(orc.rope(x, 0, theta), x)
    out = orc.rope(x, 333, theta)
    pairs = lambda v: v[:, : dim // 2] ** 2 + v[:, dim // 2:] ** 2
    assert np.allclose(pairs(out), pairs(x), rtol=1e-12, atol=0)
    assert np.allclose(orc.rope(orc.rope(x, 100, theta), 23, theta), orc.rope(x, 123, theta), rtol=0, atol=1e-10)
    q, k = x[0:1], x[1:2]
    d1 = float((orc.rope(q, 500, theta) @ orc.rope(k, 480, theta).T)[0, 0])
    d2 = float((orc.rope(q, 1020, theta) @ orc.rope(k, 1000, theta).T)[0, 0])
    assert abs(d1 - d2) < 1e-9


def pin_act8_hand_examples(orc):
    """Codes worked by hand.  Group 0 has amax 1, so inv = 127 exactly and
    c = rint(127 x): 0.5 -> 63.5 -> 64 (tie to even), -0.25 -> -31.75 -> -32,
    0.125 -> 15.875 -> 16, 0.75 -> 95.25 -> 95, fp16(0.3) = 0.2998046875 ->
    38.075 -> 38.  Group 1 has amax 2, inv = 63.5: 1 -> 63.5 -> 64,
    -0.5 -> -31.75 -> -32, 1.5 -> 95.25 -> 95, 0.25 -> 15.875 -> 16."""
    x = _h([1.0, 0.5, -0.25, 0.0, 0.125, -1.0, 0.75, 0.3, 2.0, 1.0, -0.5, 0.0, 1.5, -2.0, 0.25, 0.0])
    c, sc = orc.quantize_act8(x, 8)
    assert c.tolist() == [127, 64, -32, 0, 16, -127, 95, 38, 127, 64, -32, 0, 95, -127, 16, 0]
    assert sc[0] == np.float32(1.0) / np.float32(127.0) and sc[1] == np.float32(2.0) / np.float32(127.0)
    c0, s0 = orc.quantize_act8(np.zeros(16, np.uint16), 8)
    assert not c0.any() and not s0.any()


def pin_act8_properties(orc):
    """Bounded codes; each group's largest |x| maps to +-127; the
    dequantization error is at most half a step; sign symmetry; doubling x
    doubles the scales and keeps the codes (every step is exact under a
    power-of-two scaling)."""
    rng = np.random.default_rng(61)
    k, g = 512, 64
    xf = rng.standard_normal(k) * 2.0
    x = _h(xf)
    xv = x.view(np.float16).astype(np.float64)
    c, sc = orc.quantize_act8(x, g)
    assert np.abs(c.astype(int)).max() <= 127
    for j in range(k // g):
        seg = slice(j * g, (j + 1) * g)
        i = int(np.argmax(np.abs(xv[seg])))
        assert abs(int(c[seg][i])) == 127
        err = np.abs(xv[seg] - c[seg].astype(np.float64) * float(sc[j]))
        assert np.all(err <= 0.5 * float(sc[j]) * (1 + 1e-6))
    cn, sn = orc.quantize_act8(_h(-xv), g)
    assert np.array_equal(cn, -c) and np.array_equal(sn, sc)
    c2, s2 = orc.quantize_act8(_h(2.0 * xv), g)
    assert np.array_equal(c2, c) and np.array_equal(s2, 2.0 * sc)


def pin_act8_block_order(orc):
    """The byte order of the codes is the packed nibble order: for a row whose
    8 weights are q = 0..7, the bytes of (word & 0x0F0F0F0F) and of
    ((word >> 4) & 0x0F0F0F0F) list the inputs in the order the codes use."""
    q = np.zeros((4, 8), np.uint8)
    q[0] = np.arange(8)
    s = np.full((4, 1), 0x3C00, np.uint16)
    pw, _ = orc.pack(q, s, 8)
    word = int.from_bytes(bytes(pw[:4]), "little")
    order = [(word >> (8 * b)) & 0xF for b in range(4)] + [(word >> (8 * b + 4)) & 0xF for b in range(4)]
    assert order == [0, 4, 1, 5, 2, 6, 3, 7]
    assert orc.act8_block_order(np.arange(16, dtype=np.int8)).tolist() == order + [8 + v for v in order]


def pin_gemv_a8_vs_numpy(orc):
    rng = np.random.default_rng(67)
    n, k, g = 37, 256, 64
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = _h(rng.uniform(0.001, 0.02, (n, k // g)))
    c, sc = orc.quantize_act8(_h(rng.standard_normal(k)), g)
    xhat = c.astype(np.float64) * np.repeat(sc.astype(np.float64), g)
    w = _dequant_numpy(q, s, g)
    y, a = orc.gemv_a8(q, s, c, sc, g)
    assert np.allclose(y, w @ xhat, rtol=1e-12, atol=1e-15)
    assert np.allclose(a, np.abs(w * xhat).sum(axis=1), rtol=1e-12, atol=1e-15)
    rows = np.array([36, 0, 5], np.int64)
    y2, _ = orc.gemv_a8(q, s, c, sc, g, rows=rows)
    assert np.array_equal(y2, y[rows])


def pin_gemv_a8_closed_forms(orc):
    """q = 8 gives 0; unit weights (q = 9, s = 1) give sum_k c[k] s_g exactly;
    a one-hot activation v e_k gives (q - 8) s (+-127 * fl(|v| / 127))."""
    rng = np.random.default_rng(71)
    n, k, g = 8, 128, 32
    c, sc = orc.quantize_act8(_h(rng.standard_normal(k)), g)
    ones = np.full((n, k // g), 0x3C00, np.uint16)
    y0, _ = orc.gemv_a8(np.full((n, k), 8, np.uint8), ones, c, sc, g)
    assert np.array_equal(y0, np.zeros(n))
    y1, _ = orc.gemv_a8(np.full((n, k), 9, np.uint8), ones, c, sc, g)
    exact = sum(int(c[i]) * float(sc[i // g]) for i in range(k))
    assert np.all(y1 == exact)
    x = np.zeros(k, np.uint16)
    x[77] = _h([-0.375])[0]
    c1, s1 = orc.quantize_act8(x, g)
    assert c1[77] == -127 and s1[77 // g] == np.float32(0.375) / np.float32(127.0)
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = _h(rng.uniform(0.001, 0.02, (n, k // g)))
    y, _ = orc.gemv_a8(q, s, c1, s1, g)
    ref = (q[:, 77].astype(np.float64) - 8) * s[:, 77 // g].view(np.float16).astype(np.float64) * (
        -127.0 * float(s1[77 // g]))
    assert np.array_equal(y, ref)


def pin_gemv_a8_packed_matches_logical(orc):
    rng = np.random.default_rng(73)
    k, g = 192, 64
    c, sc = orc.quantize_act8(_h(rng.standard_normal(k)), g)
    for n, gateup in ((13, False), (10, True)):
        q = rng.integers(0, 16, (n, k), dtype=np.uint8)
        s = _h(rng.uniform(0.001, 0.02, (n, k // g)))
        pw, ps = orc.pack(q, s, g, gateup)
        y1, a1 = orc.gemv_a8(q, s, c, sc, g)
        y2, a2 = orc.gemv_a8_packed(pw, ps, c, sc, n, k, g, gateup)
        assert np.array_equal(y1, y2) and np.array_equal(a1, a2)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
