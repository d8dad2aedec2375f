"""GPU parity of the prefill GEMM (w4_gemm / w4_gemm_gateup_silu through the C
ABI) against the CPU oracle's prefill product on the same seeded inputs.

Bars: within 1e-3*sum|w x| + 1e-5 per element (the GEMM rounds each
dequantized weight once to fp16, a relative error of at most 2^-11, and
accumulates in fp32); the propagated bound of gpu_util for the fused SiLU;
bit-exact for the one-hot nibble probe (unit scales: every weight and every
sum is an exact small integer) and for run-to-run determinism."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import dev_f16, dev_u8, host_f16, tol_gateup, tol_plain

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_04_amd import w4
    w4.lib()  # fail loudly if the HIP library is missing


def _w4():
    from int4_weight_only_04_amd import w4
    return w4


def gemm_plain(pw, ps, xm, n, k, group):
    w4 = _w4()
    m = xm.shape[0]
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    wsb = w4.gemm_workspace_size(m, n, k, group)
    ws = torch.full((max(wsb, 16),), 0xFF, dtype=torch.uint8, device="cuda") if wsb else None
    w4.gemm(dev_u8(pw), dev_u8(ps), dev_f16(xm), y, m, n, k, group, workspace=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def gemm_gateup(pw, ps, xm, n_total, k, group):
    w4 = _w4()
    m = xm.shape[0]
    h = torch.full((m, n_total // 2), float("nan"), dtype=torch.float16, device="cuda")
    w4.gemm_gateup_silu(dev_u8(pw), dev_u8(ps), dev_f16(xm), h, m, n_total, k, group)
    torch.cuda.synchronize()
    return host_f16(h)


def _logical(seed, m, n, k, group, s_lo=0.001, s_hi=0.02):
    q, s, _ = synthetic.logical(seed, n, k, group, s_lo, s_hi)
    xm = synthetic.prompt_acts(seed + 1, m, k)
    return q, s, xm


# (m, n, k, group): several tiles in every direction and ragged tails in each:
# m vs the 64/128-row tiles, n vs the 4-row packing tiles and the 64/128-column
# tiles, k vs the 64-input k steps (k = 200: 25 blocks of 8, G = 8); from 256
# token rows on the tiles are 128 rows, split over k to fill 512 workgroups
# (300 x 200 x 992: 6 tiles, 8 splits over 15.5 k steps).
PLAIN_SHAPES = [
    (5, 512, 256, 64),
    (1, 37, 96, 32),
    (64, 64, 64, 64),
    (130, 301, 448, 64),
    (200, 130, 200, 8),
    (129, 260, 576, 64),
    (257, 1030, 320, 32),
    (300, 200, 992, 32),
    (256, 96, 128, 32),     # the tile policy's boundary: 128-row tiles, two of them
    (255, 96, 128, 32),     # one row fewer: 64-row tiles, the last one ragged
]


@pytest.mark.parametrize("m,n,k,group", PLAIN_SHAPES)
def test_gemm_plain_vs_oracle(m, n, k, group):
    q, s, xm = _logical(100 + m + n, m, n, k, group)
    pw, ps = _w4().pack(q, s, group, "plain")
    y = gemm_plain(pw, ps, xm, n, k, group)
    y_ref, a_ref = oracle.gemm(q, s, xm, group)
    err = np.abs(y - y_ref)
    assert np.all(np.isfinite(y))
    assert np.all(err <= tol_plain(a_ref)), (float((err / tol_plain(a_ref)).max()), m, n, k, group)


# From 256 token rows gate/up runs on 128-row tiles with one LDS buffer (three
# workgroups per CU): 300 and 257 rows end in ragged tiles, 448 inputs are an
# odd number of k steps (the ring's tail), and 200 inputs end inside a step.
@pytest.mark.parametrize("m,half,k,group", [(70, 136, 256, 64), (33, 64, 128, 32), (130, 200, 384, 128),
                                            (1, 9, 64, 64), (300, 200, 448, 64), (257, 70, 200, 8)])
def test_gemm_gateup_vs_oracle(m, half, k, group):
    n = 2 * half
    q, s, xm = _logical(300 + m + half, m, n, k, group)
    pw, ps = _w4().pack(q, s, group, "gateup")
    h = gemm_gateup(pw, ps, xm, n, k, group)
    y_ref, a_ref = oracle.gemm(q, s, xm, group)
    h_ref = np.stack([oracle.silu_gate(row) for row in y_ref])
    tol = tol_gateup(y_ref[:, :half], a_ref[:, :half], y_ref[:, half:], a_ref[:, half:], h_ref)
    err = np.abs(h - h_ref)
    assert np.all(np.isfinite(h))
    assert np.all(err <= tol), (float((err / tol).max()), m, half, k, group)


def test_gemm_onehot_nibbles_exact():
    """Unit scales and one-hot token rows: Y[t, j] = q[j, k_t] - 8 exactly, so
    the nibbles the GEMM unpacks are recovered bit for bit."""
    n, k, group = 260, 512, 128
    ks = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 15, 63, 64, 127, 128, 129, 255, 256, 448, 510, 511] * 7)
    m = ks.size
    rng = np.random.default_rng(31)
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = np.full((n, k // group), 0x3C00, np.uint16)  # fp16 1.0
    xm = np.zeros((m, k), np.uint16)
    xm[np.arange(m), ks] = 0x3C00
    for layout in ("plain", "gateup"):
        pw, ps = _w4().pack(q, s, group, layout)
        if layout == "plain":
            y = gemm_plain(pw, ps, xm, n, k, group)
            assert np.array_equal(y + 8, q[:, ks].T.astype(np.float64))
        else:
            # silu(g) * u with u one-hot exact: check the gate half through u = 1 rows
            q2 = q.copy()
            q2[n // 2:] = 9  # up rows: q - 8 = 1 everywhere
            pw2, ps2 = _w4().pack(q2, s, group, "gateup")
            h = gemm_gateup(pw2, ps2, xm, n, k, group)
            g = q2[: n // 2, ks].T.astype(np.float64) - 8.0
            h_ref = np.stack([oracle.silu_gate(np.concatenate([row, np.ones_like(row)])) for row in g])
            assert np.all(np.abs(h - h_ref) <= 2.0 ** -10 * np.abs(h_ref) + 2.0 ** -24)


def test_gemm_deterministic():
    m, n, k, group = 130, 301, 448, 64
    q, s, xm = _logical(7, m, n, k, group)
    pw, ps = _w4().pack(q, s, group, "plain")
    y1 = gemm_plain(pw, ps, xm, n, k, group)
    y2 = gemm_plain(pw, ps, xm, n, k, group)
    assert np.array_equal(y1, y2)


FULL = [("qkv", "plain", synthetic.QKV, synthetic.HIDDEN), ("o", "plain", synthetic.HIDDEN, synthetic.HIDDEN),
        ("gateup", "gateup", 2 * synthetic.MLP, synthetic.HIDDEN), ("down", "plain", synthetic.HIDDEN, synthetic.MLP)]


@pytest.mark.parametrize("name,kind,n,k", FULL, ids=[f[0] for f in FULL])
def test_gemm_full_size_sampled(name, kind, n, k):
    """The 512-token prefill shapes in the launch configuration the benchmark
    times, checked on sampled (token, output) pairs at tile boundaries."""
    w4 = _w4()
    m, group = synthetic.PROMPT, synthetic.GROUP
    wb, sb = w4.packed_size(n, k, group, kind)
    pw, ps, _ = synthetic.packed_random(5000 + n + k, wb, sb // 2, k)
    xm = synthetic.prompt_acts(5001 + n + k, m, k)
    mrows = np.array([0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 383, 384, 510, 511], np.int64)
    rng = np.random.default_rng(n + k)
    if kind == "gateup":
        half = n // 2
        h = gemm_gateup(pw, ps, xm, n, k, group)
        cols = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, 65, half - 1], rng.integers(0, half, 40)]))
        yg, ag = oracle.gemm_packed(pw, ps, xm, n, k, group, True, mrows, cols)
        yu, au = oracle.gemm_packed(pw, ps, xm, n, k, group, True, mrows, cols + half)
        h_ref = np.stack([oracle.silu_gate(np.concatenate([yg[i], yu[i]])) for i in range(mrows.size)])
        tol = tol_gateup(yg, ag, yu, au, h_ref)
        err = np.abs(h[np.ix_(mrows, cols)] - h_ref)
    else:
        y = gemm_plain(pw, ps, xm, n, k, group)
        cols = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, 127, 128, n - 1], rng.integers(0, n, 40)]))
        y_ref, a_ref = oracle.gemm_packed(pw, ps, xm, n, k, group, False, mrows, cols)
        tol = tol_plain(a_ref)
        err = np.abs(y[np.ix_(mrows, cols)] - y_ref)
        assert np.all(np.isfinite(y))
    assert np.all(err <= tol), (name, float((err / tol).max()))
