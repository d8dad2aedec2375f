"""GPU parity of the residual add and RMSNorm folded into the projections
(w4_residual_parts, w4_gemv_residual, w4_gemv_rmsnorm,
w4_gemv_gateup_silu_rmsnorm through the C ABI) against the oracle.

Bars:
  * y: the GEMV bar 1e-3 * A + 1e-5, with A from the oracle on the x the
    kernel wrote to x_out.  Every workgroup computes that x itself; a matrix
    of one unit weight per row checks bit for bit that they all used it;
  * h_out: bit-exact against fp32(h_in + y_gpu), one fp32 addition;
  * partial sums of squares: a rounded square per row and at most 7 additions
    (a part covers at most 8 rows): |err| <= 9 * 2^-24 * sum;
  * x = fp16((h r) gamma) with r = 1 / sqrt(S / k + eps): S takes at most 21
    fp32 additions of the given parts, then S / k, + eps, sqrt, 1 / ., and two
    products, so before the fp16 rounding (half an ulp, 2^-11 relative, or
    2^-25 absolute below the normal range) x is within (21 / 2 + 8) 2^-24
    relative of the oracle's; the bar uses t = 24 (t = 32 where the parts
    themselves come from the GPU, for their own rounding);
  * gate/up: the propagated form of the plain bar; argmax: the GPU logits'
    own first argmax, inside the oracle's near-tie set.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import dev_f16, dev_u8, host_f16, near_tie_set, tol_gateup, tol_plain

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U = 2.0 ** -24
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_04_amd import w4
    w4.lib()  # fail loudly if the HIP library is missing


def _w4():
    from int4_weight_only_04_amd import w4
    return w4


def tol_norm(x_ref, t):
    return (2.0 ** -11 + (t / 2 + 8) * U) * np.abs(x_ref) + 2.0 ** -25


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def parts_buffer(parts_f32, pad_value=float("nan")):
    """The partial sums on the device, padded to whole float4 with `pad_value`
    (the kernel must ignore the padding)."""
    n = parts_f32.size
    buf = np.full((n + 3) // 4 * 4, pad_value, np.float32)
    buf[:n] = parts_f32
    return dev_f32(buf)


def given_parts(h32, rows):
    """Partial sums of squares of h over blocks of `rows` values, rounded to fp32."""
    return oracle.sumsq_blocks(h32.astype(np.float64), rows).astype(np.float32)


def check_x(x_out, h32, gamma, parts_f32, t):
    s = float(np.sum(parts_f32.astype(np.float64)))
    x_ref = oracle.rmsnorm_given(h32.astype(np.float64), gamma, s, EPS)
    got = host_f16(x_out)
    err = np.abs(got - x_ref)
    tol = tol_norm(x_ref, t)
    assert np.all(err <= tol), float((err / tol).max())
    return got.astype(np.float16).view(np.uint16)


RESIDUAL = [(1, 512, 256, 64), (2, 37, 96, 32), (3, 3584, 3584, 128), (4, 3584, 18944, 128), (5, 130, 448, 64),
            (6, 65540, 256, 64)]


@pytest.mark.parametrize("seed,n,k,group", RESIDUAL)
@pytest.mark.parametrize("in_place", [False, True])
def test_gemv_residual_vs_oracle(seed, n, k, group, in_place):
    w4 = _w4()
    q, s, x = synthetic.logical(seed * 11 + n, n, k, group)
    pw, ps = w4.pack(q, s, group, "plain")
    h_in = synthetic.residual(seed, n)
    parts = w4.residual_parts(n, k, group)
    tiles = -(-n // 4)
    rows_per_part = 4 * (-(-tiles // parts))
    assert parts == -(-n // rows_per_part) and rows_per_part in (4, 8)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    hi = dev_f32(h_in)
    ho = hi if in_place else torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    ss = torch.full(((parts + 3) // 4 * 4,), float("nan"), dtype=torch.float32, device="cuda")
    w4.gemv_residual(dev_u8(pw), dev_u8(ps), dev_f16(x), y, hi, ho, ss, n, k, group)
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    y_ref, a_ref = oracle.gemv(q, s, x, group)
    assert np.all(np.abs(yg.astype(np.float64) - y_ref) <= tol_plain(a_ref))
    hg = ho.cpu().numpy()
    assert np.array_equal(hg, (h_in + yg).astype(np.float32))   # one fp32 addition, bit for bit
    ss_ref = oracle.sumsq_blocks(hg.astype(np.float64), rows_per_part)
    got = ss.cpu().numpy()[:parts].astype(np.float64)
    assert np.all(np.abs(got - ss_ref) <= 9 * U * ss_ref + 1e-30)


PLAIN_NORM = [  # seed, n, k, group, rows per given part
    (1, 5, 512, 64, 512), (2, 37, 96, 32, 7), (3, 130, 448, 64, 4), (4, 4608, 3584, 128, 4),
    (5, 200, 4096, 128, 4), (6, 3, 3584, 128, 4), (7, 260, 1024, 64, 1), (8, 8, 32768, 128, 32)]


@pytest.mark.parametrize("seed,n,k,group,rows", PLAIN_NORM)
def test_gemv_rmsnorm_vs_oracle(seed, n, k, group, rows):
    w4 = _w4()
    q, s, _ = synthetic.logical(seed * 13 + n, n, k, group)
    pw, ps = w4.pack(q, s, group, "plain")
    h = synthetic.residual(seed + 100, k)
    gamma = synthetic.norm_weights(seed + 200, k)
    parts = given_parts(h, rows)
    assert 1 <= parts.size <= 1024
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    x_out = torch.full((k,), float("nan"), dtype=torch.float16, device="cuda")
    w4.gemv_rmsnorm(dev_u8(pw), dev_u8(ps), dev_f32(h), dev_f16(gamma), parts_buffer(parts), parts.size, EPS, y,
                    n, k, group, x_out=x_out)
    torch.cuda.synchronize()
    xb = check_x(x_out, h, gamma, parts, 24)
    y_ref, a_ref = oracle.gemv(q, s, xb, group)
    err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
    assert np.all(err <= tol_plain(a_ref)), float((err / tol_plain(a_ref)).max())


@pytest.mark.parametrize("n,k", [(4096, 3584), (1000, 448)])
def test_every_workgroup_uses_the_same_x(n, k):
    """Row r holds a single unit weight at column c(r) (nibble 9, scale 1.0),
    so y[r] is x[c(r)] exactly: every workgroup's own normalized x must equal
    the x that workgroup 0 wrote, bit for bit."""
    w4 = _w4()
    group = 64
    cols = (np.arange(n) * 7 + 3) % k
    q = np.full((n, k), 8, np.uint8)
    q[np.arange(n), cols] = 9
    s = np.full((n, k // group), 0x3C00, np.uint16)
    pw, ps = w4.pack(q, s, group, "plain")
    h = synthetic.residual(77, k)
    gamma = synthetic.norm_weights(78, k)
    parts = given_parts(h, 4)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    x_out = torch.empty(k, dtype=torch.float16, device="cuda")
    w4.gemv_rmsnorm(dev_u8(pw), dev_u8(ps), dev_f32(h), dev_f16(gamma), parts_buffer(parts), parts.size, EPS, y,
                    n, k, group, x_out=x_out)
    torch.cuda.synchronize()
    xg = host_f16(x_out)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), xg[cols])


def test_gemv_rmsnorm_argmax_lm_head():
    """The lm_head shape with the norm prologue and the argmax epilogue:
    sampled rows against the oracle on x_out, the argmax against the GPU's
    own logits and inside the oracle's near-tie set."""
    w4 = _w4()
    n, k, group = synthetic.VOCAB, synthetic.HIDDEN, synthetic.GROUP
    wb, sb = w4.packed_size(n, k, group, "plain")
    pw, ps, _ = synthetic.packed_random(4322, wb, sb // 2, k)
    h = synthetic.residual(4323, k)
    gamma = synthetic.norm_weights(4324, k)
    parts = given_parts(h, 4)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    am = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    ws = torch.empty(w4.gemv_workspace_size(n, k, group, True), dtype=torch.uint8, device="cuda")
    x_out = torch.empty(k, dtype=torch.float16, device="cuda")
    w4.gemv_rmsnorm(dev_u8(pw), dev_u8(ps), dev_f32(h), dev_f16(gamma), parts_buffer(parts), parts.size, EPS, y,
                    n, k, group, x_out=x_out, argmax=am, workspace=ws)
    torch.cuda.synchronize()
    xb = check_x(x_out, h, gamma, parts, 24)
    yh = y.cpu().numpy().astype(np.float64)
    y_ref, a_ref = oracle.gemv_packed(pw, ps, xb, n, k, group)
    assert np.all(np.abs(yh - y_ref) <= tol_plain(a_ref))
    assert int(am.item()) == int(np.argmax(yh))
    assert int(am.item()) in set(near_tie_set(y_ref, a_ref).tolist())


@pytest.mark.parametrize("half,k,group,rows", [(96, 256, 64, 4), (9, 64, 64, 64), (200, 448, 64, 3),
                                                (18944, 3584, 128, 4)])
def test_gemv_gateup_rmsnorm_vs_oracle(half, k, group, rows):
    w4 = _w4()
    n = 2 * half
    if n * k > 50_000_000:
        wb, sb = w4.packed_size(n, k, group, "gateup")
        pw, ps, _ = synthetic.packed_random(91 + half, wb, sb // 2, k)
        sel = np.unique(np.concatenate([[0, 1, 63, 64, half - 1], np.random.default_rng(2).integers(0, half, 60)]))
    else:
        q, s, _ = synthetic.logical(half + k + 5, n, k, group)
        pw, ps = w4.pack(q, s, group, "gateup")
        sel = np.arange(half)
    h = synthetic.residual(half + 1, k)
    gamma = synthetic.norm_weights(half + 2, k)
    parts = given_parts(h, rows)
    hm = torch.full((half,), float("nan"), dtype=torch.float16, device="cuda")
    x_out = torch.full((k,), float("nan"), dtype=torch.float16, device="cuda")
    w4.gemv_gateup_silu_rmsnorm(dev_u8(pw), dev_u8(ps), dev_f32(h), dev_f16(gamma), parts_buffer(parts), parts.size,
                                EPS, hm, n, k, group, x_out=x_out)
    torch.cuda.synchronize()
    xb = check_x(x_out, h, gamma, parts, 24)
    yg, ag = oracle.gemv_packed(pw, ps, xb, n, k, group, True, sel)
    yu, au = oracle.gemv_packed(pw, ps, xb, n, k, group, True, sel + half)
    h_ref = np.array([oracle.silu(g) * u for g, u in zip(yg, yu)])
    tol = tol_gateup(yg, ag, yu, au, h_ref)
    err = np.abs(host_f16(hm)[sel] - h_ref)
    assert np.all(err <= tol), float((err / tol).max())


@pytest.mark.parametrize("hidden,k_o", [(3584, 3584), (512, 512), (200, 96)])
def test_residual_then_norm_chain(hidden, k_o):
    """o_proj-style producer then a qkv-style consumer on its partial sums:
    the consumer's x is the RMSNorm of the producer's h_out."""
    w4 = _w4()
    group = 8 if hidden % 64 else 64
    q, s, x = synthetic.logical(5 + hidden, hidden, k_o, group)
    pw, ps = w4.pack(q, s, group, "plain")
    h_in = synthetic.residual(6 + hidden, hidden)
    parts = w4.residual_parts(hidden, k_o, group)
    y = torch.empty(hidden, dtype=torch.float32, device="cuda")
    h_out = torch.empty(hidden, dtype=torch.float32, device="cuda")
    ss = torch.full(((parts + 3) // 4 * 4,), float("nan"), dtype=torch.float32, device="cuda")
    w4.gemv_residual(dev_u8(pw), dev_u8(ps), dev_f16(x), y, dev_f32(h_in), h_out, ss, hidden, k_o, group)
    n2 = 64
    q2, s2, _ = synthetic.logical(7 + hidden, n2, hidden, group)
    pw2, ps2 = w4.pack(q2, s2, group, "plain")
    gamma = synthetic.norm_weights(8 + hidden, hidden)
    y2 = torch.empty(n2, dtype=torch.float32, device="cuda")
    x_out = torch.empty(hidden, dtype=torch.float16, device="cuda")
    w4.gemv_rmsnorm(dev_u8(pw2), dev_u8(ps2), h_out, dev_f16(gamma), ss, parts, EPS, y2, n2, hidden, group,
                    x_out=x_out)
    torch.cuda.synchronize()
    hg = h_out.cpu().numpy().astype(np.float64)
    x_ref = oracle.rmsnorm(hg, gamma, EPS)
    err = np.abs(host_f16(x_out) - x_ref)
    assert np.all(err <= tol_norm(x_ref, 32)), float((err / tol_norm(x_ref, 32)).max())
    xb = host_f16(x_out).astype(np.float16).view(np.uint16)
    y_ref, a_ref = oracle.gemv(q2, s2, xb, group)
    assert np.all(np.abs(y2.cpu().numpy().astype(np.float64) - y_ref) <= tol_plain(a_ref))
