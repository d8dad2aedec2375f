"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: bit-exact where the result is an integer or exact by construction
(one-hot nibble probes, integer closed forms, argmax vs the GPU's own logits,
graph vs eager, replay determinism); within 1e-3*sum|w x| + 1e-5 per element
for floating-point outputs; the propagated bound of gpu_util for the fused
SiLU epilogue."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import (dev_f16, dev_u8, half_bits, host_f16, near_tie_set, tol_gateup, tol_plain)

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


def run_plain(q, s, x, group, argmax=False):
    w4 = _w4()
    n, k = q.shape
    pw, ps = w4.pack(q, s, group, "plain")
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    am = ws = None
    if argmax:
        am = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        ws = torch.zeros(w4.gemv_workspace_size(n, k, group, True), dtype=torch.uint8, device="cuda")
    w4.gemv(dev_u8(pw), dev_u8(ps), dev_f16(x), y, n, k, group, argmax=am, workspace=ws)
    torch.cuda.synchronize()
    yh = y.cpu().numpy().astype(np.float64)
    if argmax:
        return yh, int(am.item()), ws
    return yh


def run_gateup(q, s, x, group):
    w4 = _w4()
    n, k = q.shape
    pw, ps = w4.pack(q, s, group, "gateup")
    h = torch.empty(n // 2, dtype=torch.float16, device="cuda")
    w4.gemv_gateup_silu(dev_u8(pw), dev_u8(ps), dev_f16(x), h, n, k, group)
    torch.cuda.synchronize()
    return host_f16(h)


def check_plain(y, q, s, x, group):
    y_ref, a_ref = oracle.gemv(q, s, x, group)
    err = np.abs(y - y_ref)
    bound = tol_plain(a_ref)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{bad.size} rows out of tolerance, first {bad[:5]}, "
                           f"err {err[bad[:5]]}, bound {bound[bad[:5]]}")
    return y_ref, a_ref


def check_gateup(h, q, s, x, group):
    y_ref, a_ref = oracle.gemv(q, s, x, group)
    half = q.shape[0] // 2
    h_ref = oracle.silu_gate(y_ref)
    bound = tol_gateup(y_ref[:half], a_ref[:half], y_ref[half:], a_ref[half:], h_ref)
    err = np.abs(h - h_ref)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{bad.size} outputs out of tolerance, first {bad[:5]}, "
                           f"err {err[bad[:5]]}, bound {bound[bad[:5]]}")


# ----------------------------------------------------------------- plain GEMV


def test_tiny_config():
    c = synthetic.CONFIG_TINY
    q, s, x = synthetic.logical(c["seed"], c["n"], c["k"], c["group"], c["s_lo"], c["s_hi"])
    check_plain(run_plain(q, s, x, c["group"]), q, s, x, c["group"])


RAGGED = [
    # (n, k, group): tiles of 4 rows with ragged n, k blocks not a multiple of
    # the 64 lanes, more blocks than one round of in-flight loads, tiny k
    (1, 8, 8), (3, 32, 32), (5, 64, 32), (7, 72, 8), (63, 520, 8), (65, 1032, 8),
    (130, 4104, 8), (257, 4096, 128), (33, 8192, 256), (4099, 384, 128), (9, 32768, 128),
]


@pytest.mark.parametrize("n,k,group", RAGGED)
def test_ragged_shapes(n, k, group):
    q, s, x = synthetic.logical(7000 + n + k, n, k, group)
    check_plain(run_plain(q, s, x, group), q, s, x, group)


def test_onehot_nibbles_exact_tiny():
    """s = 1 and x = e_k give y[n] = q[n][k] - 8 exactly: recover every nibble."""
    w4 = _w4()
    n, k, group = 512, 256, 64
    q, _, _ = synthetic.logical(0, n, k, group)
    s = np.full((n, k // group), 0x3C00, np.uint16)
    pw, ps = w4.pack(q, s, group)
    dpw, dps = dev_u8(pw), dev_u8(ps)
    ys = torch.empty((k, n), dtype=torch.float32, device="cuda")
    xs = [dev_f16(half_bits(np.eye(k)[kk])) for kk in range(k)]
    for kk in range(k):
        w4.gemv(dpw, dps, xs[kk], ys[kk], n, k, group)
    torch.cuda.synchronize()
    rec = ys.cpu().numpy().T + 8.0
    assert np.array_equal(rec, q.astype(np.float64))


# the down and QKV shapes (5 and 2 k iterations per wave), and shapes whose
# waves take 8 iterations at G = 256 and 1 iteration at G = 512: with groups
# of 128 inputs or more a wave loads each tile's scale words once and hands
# each 16-lane row its word, which random scales and one-hot x pin exactly
@pytest.mark.parametrize("n,k,group", [(3584, 18944, 128), (4608, 3584, 128), (40, 32768, 256),
                                       (48, 2048, 512)])
def test_onehot_nibbles_exact_big(n, k, group):
    w4 = _w4()
    q, s_rand, _ = synthetic.logical(31, n, k, group)
    s = np.full_like(s_rand, 0x3C00)
    pw, ps = w4.pack(q, s, group)
    dpw, dps = dev_u8(pw), dev_u8(ps)
    # random scales too: y = (q - 8) * s exactly (a 4-bit integer times an fp16)
    pw2, ps2 = w4.pack(q, s_rand, group)
    dpw2, dps2 = dev_u8(pw2), dev_u8(ps2)
    sv = s_rand.view(np.float16).astype(np.float64)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    for kk in (0, 1, 7, 8, 127, 128, 511, 512, 513, k // 2 + 3, k - 1):
        xk = dev_f16(half_bits(np.eye(1, k, kk)[0]))
        w4.gemv(dpw, dps, xk, y, n, k, group)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy() + 8.0, q[:, kk].astype(np.float32)), kk
        w4.gemv(dpw2, dps2, xk, y, n, k, group)
        torch.cuda.synchronize()
        expect = (q[:, kk].astype(np.float64) - 8.0) * sv[:, kk // group]
        assert np.array_equal(y.cpu().numpy().astype(np.float64), expect), kk


@pytest.mark.parametrize("k", [256, 3584, 18944])
def test_integer_closed_forms(k):
    n, group = 37, 128
    ones = half_bits(np.ones(k))
    one_s = half_bits(np.ones((n, k // group)))
    rng = np.random.default_rng(k)
    xr = half_bits(rng.integers(-3, 4, k))
    sr = half_bits(rng.uniform(0.001, 0.02, (n, k // group)))
    assert np.all(run_plain(np.full((n, k), 8, np.uint8), sr, xr, group) == 0.0)
    assert np.all(run_plain(np.full((n, k), 15, np.uint8), one_s, ones, group) == 7 * k)
    y = run_plain(np.zeros((n, k), np.uint8), one_s, xr, group)
    assert np.all(y == -8 * xr.view(np.float16).astype(np.float64).sum())
    half_s = half_bits(np.full((n, k // group), 0.5))
    assert np.all(run_plain(np.full((n, k), 9, np.uint8), half_s, ones, group) == k / 2)


def test_down_config():
    c = synthetic.CONFIG_DOWN
    q, s, x = synthetic.logical(c["seed"], c["n"], c["k"], c["group"], c["s_lo"], c["s_hi"])
    check_plain(run_plain(q, s, x, c["group"]), q, s, x, c["group"])


def test_qkv_and_o_shapes():
    for n, seed in ((4608, 1000), (3584, 1001)):
        q, s, x = synthetic.logical(seed, n, 3584, 128)
        check_plain(run_plain(q, s, x, 128), q, s, x, 128)


def test_determinism_repeat_bitwise():
    c = synthetic.CONFIG_DOWN
    q, s, x = synthetic.logical(c["seed"], c["n"], c["k"], c["group"])
    w4 = _w4()
    pw, ps = w4.pack(q, s, c["group"])
    dpw, dps, dx = dev_u8(pw), dev_u8(ps), dev_f16(x)
    ys = [torch.empty(c["n"], dtype=torch.float32, device="cuda") for _ in range(3)]
    for y in ys:
        w4.gemv(dpw, dps, dx, y, c["n"], c["k"], c["group"])
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])


# ----------------------------------------------------------------- gate/up + SiLU


def test_gateup_config():
    c = synthetic.CONFIG_GATEUP
    q, s, x = synthetic.logical(c["seed"], c["n"], c["k"], c["group"], c["s_lo"], c["s_hi"])
    check_gateup(run_gateup(q, s, x, c["group"]), q, s, x, c["group"])


@pytest.mark.parametrize("n_total,k,group", [(2, 64, 32), (6, 128, 64), (10, 256, 128),
                                             (14, 96, 32), (130, 1032, 8), (8194, 3584, 128)])
def test_gateup_ragged(n_total, k, group):
    q, s, x = synthetic.logical(9000 + n_total, n_total, k, group)
    check_gateup(run_gateup(q, s, x, group), q, s, x, group)


def test_gateup_zero_rows_give_zero():
    n_total, k, group = 64, 3584, 128
    q, s, x = synthetic.logical(77, n_total, k, group)
    half = n_total // 2
    qg = q.copy()
    qg[:half] = 8         # gate == 0 -> silu(0) * u == 0
    assert np.all(run_gateup(qg, s, x, group) == 0.0)
    qu = q.copy()
    qu[half:] = 8         # up == 0 -> silu(g) * 0 == 0
    assert np.all(run_gateup(qu, s, x, group) == 0.0)


def test_gateup_silu_over_range():
    """Planted gate values over [-20, 20] with up == 1: h follows silu."""
    half, k, group = 256, 64, 64
    g_target = np.linspace(-20, 20, half)
    q = np.full((2 * half, k), 8, np.uint8)
    s = np.zeros((2 * half, 1), np.uint16)
    q[:half, 0] = 15                                  # g = 7 * s_g
    s[:half, 0] = half_bits(g_target / 7.0)
    q[half:, 0] = 9                                   # u = 1
    s[half:, 0] = half_bits(np.ones(half))
    x = half_bits(np.eye(1, k, 0)[0])
    check_gateup(run_gateup(q, s, x, group), q, s, x, group)


# ----------------------------------------------------------------- lm_head argmax


def test_lmhead_config():
    c = synthetic.CONFIG_LMHEAD
    q, s, x = synthetic.logical(c["seed"], c["n"], c["k"], c["group"], c["s_lo"], c["s_hi"])
    y, idx, _ = run_plain(q, s, x, c["group"], argmax=True)
    y_ref, a_ref = check_plain(y, q, s, x, c["group"])
    # the argmax decision is taken in the kernel's precision: bit-exact against
    # the first maximum of the GPU's own fp32 logits
    assert idx == oracle.argmax(y)
    tie = near_tie_set(y_ref, a_ref)
    assert idx in tie
    if tie.size == 1:
        assert idx == oracle.argmax(y_ref)


@pytest.mark.parametrize("n,k", [(65536, 256), (70001, 512), (65540, 8)])
def test_tall_matrix_short_rows(n, k):
    """16384 tiles or more run two tiles per unit; with k <= 512 there is one
    k iteration and a single wave per unit (a launch shape of its own), with
    and without the argmax epilogue."""
    group = 8 if k == 8 else 64
    q, s, x = synthetic.logical(n + k, n, k, group)
    check_plain(run_plain(q, s, x, group), q, s, x, group)
    y, idx, _ = run_plain(q, s, x, group, argmax=True)
    y_ref, a_ref = check_plain(y, q, s, x, group)
    assert idx == oracle.argmax(y)
    assert idx in near_tie_set(y_ref, a_ref)


def test_argmax_planted_and_ties():
    n, k, group = 4099, 256, 64
    q, s, x = synthetic.logical(55, n, k, group)
    xs = half_bits(np.abs(x.view(np.float16)))      # x >= 0
    qq = q.copy()
    qq[3001] = 15                                     # planted winner: 7 * s * sum x
    y, idx, _ = run_plain(qq, s, xs, group, argmax=True)
    assert idx == 3001 == oracle.argmax(y)
    # two identical winning rows -> the lower index
    qq[1234] = 15
    ss = s.copy()
    ss[1234] = ss[3001]
    y, idx, _ = run_plain(qq, ss, xs, group, argmax=True)
    assert idx == 1234 == oracle.argmax(y)
    # all rows equal -> index 0
    qc = np.full((n, k), 11, np.uint8)
    sc = np.full((n, k // group), 0x2000, np.uint16)
    y, idx, _ = run_plain(qc, sc, xs, group, argmax=True)
    assert idx == 0 and np.all(y == y[0])


def _argmax_grid(n, k, group):
    """Number of per-workgroup partials the finalize reduces, recovered from the
    workspace size (partial values, a 256-byte aligned offset, partial rows)."""
    wsb = _w4().gemv_workspace_size(n, k, group, True)
    for g in range(max(1, wsb // 8 - 64), wsb // 8 + 64):
        if ((4 * g + 255) // 256) * 256 + 4 * g == wsb:
            return g
    raise AssertionError(f"no grid gives a workspace of {wsb} bytes")


# (n rows at k = 64): partial counts of every residue mod 4, so the finalize's
# scalar tail loads and its 16-byte loads both carry the winner, and 1.05M rows
# for more partials than one load round of the finalize covers
@pytest.mark.parametrize("n", [4112, 4128, 4144, 4160, 1_050_000])
def test_argmax_finalize_tails_and_rounds(n):
    k, group = 64, 64
    grid = _argmax_grid(n, k, group)
    print(f"[argmax] n={n} partials={grid}", flush=True)
    q, s, x = synthetic.logical(900 + n % 97, n, k, group)
    xs = half_bits(np.abs(x.view(np.float16)))
    top = s.max()
    cases = []
    for rows in ([n - 1], [1], [n // 2], [n - 1, n - 2], [n - 3, 7]):
        qq, ss = q.copy(), s.copy()
        for r in rows:
            qq[r] = 15
            ss[r] = top
        cases.append((rows, qq, ss))
    for rows, qq, ss in cases:
        y, idx, _ = run_plain(qq, ss, xs, group, argmax=True)
        # the setup makes the planted rows the maxima of the GPU's own logits
        # (identical rows give bit-identical sums), so the lowest one must win
        assert np.all(y[rows] == y.max()), rows
        assert idx == min(rows) == oracle.argmax(y), (rows, idx)
    if n > 1_000_000:
        assert grid > 24576


def test_argmax_workspace_reuse():
    """The workspace needs no initial contents: starting from garbage, repeated
    calls agree bit for bit."""
    w4 = _w4()
    c = synthetic.CONFIG_LMHEAD
    n, k, group = c["n"], c["k"], c["group"]
    q, s, x = synthetic.logical(4, n, k, group)
    pw, ps = w4.pack(q, s, group)
    dpw, dps, dx = dev_u8(pw), dev_u8(ps), dev_f16(x)
    ws = torch.full((w4.gemv_workspace_size(n, k, group, True),), 0xA5, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(4):
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        am = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        w4.gemv(dpw, dps, dx, y, n, k, group, argmax=am, workspace=ws)
        outs.append((y, am))
    torch.cuda.synchronize()
    for y, am in outs[1:]:
        assert torch.equal(y, outs[0][0]) and int(am.item()) == int(outs[0][1].item())
    assert int(outs[0][1].item()) == oracle.argmax(outs[0][0].cpu().numpy().astype(np.float64))


# ----------------------------------------------------------------- ABI on device


def test_device_validation_errors():
    w4 = _w4()
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    L = w4.lib()
    p = buf.data_ptr()
    assert L.w4_gemv(p + 8, p, p, p, None, None, 0, 4, 64, 32, None) == w4.EALIGN
    assert L.w4_gemv(p, p, p + 2, p, None, None, 0, 4, 64, 32, None) == w4.EALIGN
    with pytest.raises(ValueError):
        w4.gemv(buf[:10], buf, buf.view(torch.float16), buf.view(torch.float32), 4, 64, 32)
