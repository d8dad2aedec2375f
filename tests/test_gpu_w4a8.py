"""GPU parity of the W4A8 variant (w4_quantize_act8, w4_gemv_a8,
w4_gemv_gateup_silu_a8 through the C ABI) against the oracle.

Bars:
  * the activation codes and their scales are integer / binary32 results of
    a rule fixed to the last bit (binary32, round to nearest even): bit-exact,
    in the W4T4 byte order the oracle derives from the layout;
  * a one-hot activation of 127/128 has the scale 2^-7 and the code 127, so
    with unit weight scales every output is (q - 8) * 127 * 2^-7 exactly:
    the nibbles come back bit-exact;
  * outputs: 1e-3 sum|w x^| + 1e-5 with x^ = c * s_g (the GPU's block sums
    are exact integers; one fp32 rounding of s * s_g and fp32 accumulation
    remain); gate/up through the propagated bar; the argmax bit-exact against
    the GPU's own logits and inside the oracle's near-tie set.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import dev_f16, dev_u8, host_f16, near_tie_set, tol_gateup, tol_plain

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


def quantize(x_bits, group):
    w4 = _w4()
    k = x_bits.size
    codes = torch.full((k,), 99, dtype=torch.int8, device="cuda")
    scales = torch.full((k // group,), float("nan"), dtype=torch.float32, device="cuda")
    w4.quantize_act8(dev_f16(x_bits), group, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def check_codes(x_bits, group):
    codes, scales = quantize(x_bits, group)
    c_ref, s_ref = oracle.quantize_act8(x_bits, group)
    assert np.array_equal(codes.cpu().numpy(), oracle.act8_block_order(c_ref))
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    return codes, scales, c_ref, s_ref


@pytest.mark.parametrize("k,group", [(8, 8), (256, 64), (448, 64), (3584, 128), (18944, 128), (4096, 1024),
                                     (32768, 32768)])
def test_quantize_bit_exact(k, group):
    rng = np.random.default_rng(k + group)
    x = (rng.standard_normal(k) * rng.choice([1e-3, 1.0, 30.0], k)).astype(np.float16).view(np.uint16)
    check_codes(x, group)


def test_quantize_ties_zeros_and_subnormals():
    """Exact ties (x * inv = m + 0.5) round to even; an all-zero group gives
    zero codes and a zero scale; subnormal inputs and a -0 are handled."""
    x = np.zeros(64, np.float16)
    x[:8] = [1.0, 0.5, -0.5, 1.5 / 127, 2.5 / 127, -3.5 / 127, 0.0, -0.0]
    x[16:24] = [6.1e-5, -6.1e-6, 3e-7, -1e-7, 2e-6, 0, 0, 5.9e-8]   # one group of subnormal-scale values
    x[40:48] = [2.0, 1.0, -1.0, 0.25, 0.75, -0.75, 1.25, -2.0]
    _, scales, c_ref, s_ref = check_codes(x.view(np.uint16), 8)
    assert s_ref[1] == 0.0 and not c_ref[8:16].any()


def _one_hot_codes(k, positions):
    x = np.zeros(k, np.float16)
    x[positions] = 127.0 / 128.0
    return x.view(np.uint16)


@pytest.mark.parametrize("layout", ["plain", "gateup"])
def test_gemv_a8_one_hot_nibbles_exact(layout):
    """x = (127/128) e_k with unit weight scales: code 127, scale 2^-7, so
    y[n] = (q[n][k] - 8) * 127 / 128 exactly and q is recovered bit for bit,
    for every position of an 8-input block and across group boundaries."""
    w4 = _w4()
    n, k, group = 260, 512, 128
    rng = np.random.default_rng(41)
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = np.full((n, k // group), 0x3C00, np.uint16)
    pw, ps = w4.pack(q, s, group, layout)
    for kk in [0, 1, 2, 3, 4, 5, 6, 7, 8, 127, 128, 129, 300, 504, 511]:
        x = np.zeros(k, np.uint16)
        x[kk] = _one_hot_codes(k, [kk])[kk]
        codes, scales = quantize(x, group)
        assert float(scales.cpu()[kk // group]) == 2.0 ** -7
        if layout == "plain":
            y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
            w4.gemv_a8(dev_u8(pw), dev_u8(ps), codes, scales, y, n, k, group)
            torch.cuda.synchronize()
            got = y.cpu().numpy().astype(np.float64) * 128.0 / 127.0 + 8.0
            assert np.array_equal(got, q[:, kk].astype(np.float64)), kk
        else:
            # up rows fixed at q = 9 (weight 1): h = silu(g) * 127/128 with g exact
            q2 = q.copy()
            q2[n // 2:] = 9
            pw2, ps2 = w4.pack(q2, s, group, "gateup")
            h = torch.full((n // 2,), float("nan"), dtype=torch.float16, device="cuda")
            w4.gemv_gateup_silu_a8(dev_u8(pw2), dev_u8(ps2), codes, scales, h, n, k, group)
            torch.cuda.synchronize()
            g = (q2[: n // 2, kk].astype(np.float64) - 8.0) * 127.0 / 128.0
            h_ref = np.array([oracle.silu(v) for v in g]) * 127.0 / 128.0
            assert np.all(np.abs(host_f16(h) - h_ref) <= 2.0 ** -10 * np.abs(h_ref) + 2.0 ** -24), kk


PLAIN = [(5, 512, 256, 64), (1, 37, 96, 32), (130, 301, 448, 64), (200, 130, 200, 8), (7, 4608, 3584, 128),
         (3, 3584, 18944, 128)]


@pytest.mark.parametrize("seed,n,k,group", PLAIN)
def test_gemv_a8_vs_oracle(seed, n, k, group):
    w4 = _w4()
    q, s, x = synthetic.logical(seed * 7 + n, n, k, group)
    pw, ps = w4.pack(q, s, group, "plain")
    codes, scales, c_ref, s_ref = check_codes(x, group)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    w4.gemv_a8(dev_u8(pw), dev_u8(ps), codes, scales, y, n, k, group)
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.gemv_a8(q, s, c_ref, s_ref, group)
    err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
    assert np.all(err <= tol_plain(a_ref)), float((err / tol_plain(a_ref)).max())


@pytest.mark.parametrize("half,k,group", [(96, 256, 64), (9, 64, 64), (200, 384, 128), (18944, 3584, 128)])
def test_gemv_gateup_a8_vs_oracle(half, k, group):
    w4 = _w4()
    n = 2 * half
    if n * k > 50_000_000:
        wb, sb = w4.packed_size(n, k, group, "gateup")
        pw, ps, x = synthetic.packed_random(77 + half, wb, sb // 2, k)
        rows = np.unique(np.concatenate([[0, 1, 63, 64, half - 1], np.random.default_rng(1).integers(0, half, 60)]))
    else:
        q, s, x = synthetic.logical(half + k, n, k, group)
        pw, ps = w4.pack(q, s, group, "gateup")
        rows = np.arange(half)
    codes, scales, c_ref, s_ref = check_codes(x, group)
    h = torch.full((half,), float("nan"), dtype=torch.float16, device="cuda")
    w4.gemv_gateup_silu_a8(dev_u8(pw), dev_u8(ps), codes, scales, h, n, k, group)
    torch.cuda.synchronize()
    yg, ag = oracle.gemv_a8_packed(pw, ps, c_ref, s_ref, n, k, group, True, rows)
    yu, au = oracle.gemv_a8_packed(pw, ps, c_ref, s_ref, n, k, group, True, rows + half)
    h_ref = np.array([oracle.silu(g) * u for g, u in zip(yg, yu)])
    tol = tol_gateup(yg, ag, yu, au, h_ref)
    err = np.abs(host_f16(h)[rows] - h_ref)
    assert np.all(err <= tol), float((err / tol).max())


def test_gemv_a8_lm_head_argmax():
    """The lm_head shape with the argmax epilogue, sampled rows plus the
    argmax against the full oracle product."""
    w4 = _w4()
    n, k, group = synthetic.VOCAB, synthetic.HIDDEN, synthetic.GROUP
    wb, sb = w4.packed_size(n, k, group, "plain")
    pw, ps, x = synthetic.packed_random(4321, wb, sb // 2, k)
    codes, scales, c_ref, s_ref = check_codes(x, group)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    am = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    ws = torch.empty(w4.gemv_workspace_size(n, k, group, True), dtype=torch.uint8, device="cuda")
    w4.gemv_a8(dev_u8(pw), dev_u8(ps), codes, scales, y, n, k, group, argmax=am, workspace=ws)
    torch.cuda.synchronize()
    yh = y.cpu().numpy().astype(np.float64)
    y_ref, a_ref = oracle.gemv_a8_packed(pw, ps, c_ref, s_ref, n, k, group)
    assert np.all(np.abs(yh - y_ref) <= tol_plain(a_ref))
    assert int(am.item()) == int(np.argmax(yh))
    assert int(am.item()) in set(near_tie_set(y_ref, a_ref).tolist())


def test_gemv_a8_deterministic_and_close_to_w4a16():
    """Run-to-run bit-identical; and the W4A8 result differs from the fp16
    activation GEMV by no more than the activation rounding allows:
    |y8 - y16| <= sum_k |w_k| s_g / 2 + both bars."""
    w4 = _w4()
    n, k, group = 512, 3584, 128
    q, s, x = synthetic.logical(99, n, k, group)
    pw, ps = w4.pack(q, s, group, "plain")
    codes, scales, c_ref, s_ref = check_codes(x, group)
    outs = []
    for _ in range(2):
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        w4.gemv_a8(dev_u8(pw), dev_u8(ps), codes, scales, y, n, k, group)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    y16 = torch.empty(n, dtype=torch.float32, device="cuda")
    w4.gemv(dev_u8(pw), dev_u8(ps), dev_f16(x), y16, n, k, group)
    torch.cuda.synchronize()
    wabs = np.abs(q.astype(np.float64) - 8) * np.repeat(s.view(np.float16).astype(np.float64), group, axis=1)
    step = np.repeat(s_ref.astype(np.float64), group) / 2
    _, a16 = oracle.gemv(q, s, x, group)
    _, a8 = oracle.gemv_a8(q, s, c_ref, s_ref, group)
    bound = wabs @ step + tol_plain(a16) + tol_plain(a8)
    assert np.all(np.abs(outs[0].astype(np.float64) - y16.cpu().numpy()) <= bound)
