"""The persistent sweep (one cooperative kernel for every projection) through
the C ABI: bit for bit the outputs of the graph-captured one-kernel-per-
projection sweep, on a small mixed sweep with ragged per-workgroup shares and
on the full 28-layer + lm_head sweep bench.py times; identical across replays;
the lm_head argmax against the oracle; and the watchdog: a wait limit too
short for any hand-off is reported as a timeout, the kernel still ends, and
the next run with the normal limit is correct again."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import host_f16, near_tie_set, tol_gateup, tol_plain

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_04_amd import w4
    w4.lib()  # fail loudly if the HIP library is missing


def _proj(w4, kind, n, k, group, seed):
    layout = "gateup" if kind == "gateup" else "plain"
    wb, sb = w4.packed_size(n, k, group, layout)
    pw, ps, x = synthetic.packed_random(seed, wb, sb // 2, k)
    dpw = torch.from_numpy(pw).cuda()
    dps = torch.from_numpy(ps).cuda()
    dx = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
    host = (pw, ps, x)
    if kind == "gateup":
        out = torch.empty(n // 2, dtype=torch.float16, device="cuda")
        return w4.Proj(w4.PROJ_GATEUP_SILU, n, k, group, dpw, dps, dx, out), host
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    if kind == "lmhead":
        am = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        ws = torch.zeros(w4.gemv_workspace_size(n, k, group, True), dtype=torch.uint8, device="cuda")
        return w4.Proj(w4.PROJ_LMHEAD_ARGMAX, n, k, group, dpw, dps, dx, out, am, ws), host
    return w4.Proj(w4.PROJ_PLAIN, n, k, group, dpw, dps, dx, out), host


# A small sweep whose projections give the workgroups unequal shares (tile
# counts not multiples of 256), every launch-table shape (splits 4, 8 and 2,
# one and two tiles per unit), several group sizes and a short lm_head.
SMALL = [("plain", 1000, 512, 128, 11), ("plain", 4100, 3584, 128, 12), ("gateup", 2 * 1030, 1024, 64, 13),
         ("plain", 700, 6144, 256, 14), ("gateup", 2 * 18944, 3584, 128, 15), ("plain", 3584, 18944, 128, 16),
         ("plain", 96, 2048, 512, 17), ("lmhead", 70000, 3584, 128, 18)]


def _outputs(projs):
    from int4_weight_only_04_amd import w4
    outs = []
    for p in projs:
        outs.append(p.out.clone())
        if p.kind == w4.PROJ_LMHEAD_ARGMAX:
            outs.append(p.argmax.clone())
    return outs


def _poison(projs):
    for p in projs:
        p.out.fill_(float("nan"))
        if p.argmax is not None:
            p.argmax.fill_(-5)


def _run(sweep, projs, stream):
    _poison(projs)
    torch.cuda.synchronize()
    sweep.run(stream)
    stream.synchronize()
    return _outputs(projs)


def _bits(t):
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype == torch.float16:
        return t.view(torch.int16)
    return t


def _same(a, b):
    return len(a) == len(b) and all(torch.equal(_bits(x), _bits(y)) for x, y in zip(a, b))


def _check_against_graph(projs, modes):
    from int4_weight_only_04_amd import w4
    stream = torch.cuda.Stream()
    ref_sweep = w4.Sweep(projs, mode=w4.SWEEP_GRAPH)
    ref = _run(ref_sweep, projs, stream)
    ref_sweep.close()
    for mode in modes:
        print(f"[persist] mode {mode}: {len(projs)} projections", flush=True)
        sw = w4.Sweep(projs, mode=mode)
        for rep in range(3):
            got = _run(sw, projs, stream)
            assert not sw.status(), f"watchdog timeout, mode {mode} replay {rep}"
            assert _same(ref, got), f"mode {mode} replay {rep} differs from the graph sweep"
        sw.close()
    return ref


def test_persistent_small_sweep_bitwise_vs_graph():
    from int4_weight_only_04_amd import w4
    built = [_proj(w4, *spec) for spec in SMALL]
    projs = [p for p, _ in built]
    ref = _check_against_graph(projs, (w4.SWEEP_PERSISTENT, w4.SWEEP_PERSISTENT_EAGER))
    # the lm_head logits and argmax against the oracle
    (pw, ps, x), p = built[-1][1], projs[-1]
    _, n, k, g, _ = SMALL[-1]
    y = ref[-2].cpu().numpy().astype(np.float64)
    y_ref, a_ref = oracle.gemv_packed(pw, ps, x, n, k, g, False)
    assert np.all(np.abs(y - y_ref) <= tol_plain(a_ref))
    idx = int(ref[-1].item())
    assert idx == int(np.argmax(y))
    assert idx in set(near_tie_set(y_ref, a_ref).tolist())
    # a gate/up projection with G = 64 against the oracle on sampled rows
    (pw, ps, x) = built[2][1]
    _, n, k, g, _ = SMALL[2]
    half = n // 2
    j = np.unique(np.concatenate([[0, 1, 2, 3, half - 1], np.random.default_rng(7).integers(0, half, 40)]))
    yr, ar = oracle.gemv_packed(pw, ps, x, n, k, g, True, np.concatenate([j, half + j]))
    m = j.size
    h_ref = oracle.silu_gate(yr)
    bound = tol_gateup(yr[:m], ar[:m], yr[m:], ar[m:], h_ref)
    assert np.all(np.abs(host_f16(ref[2])[j] - h_ref) <= bound)


def test_persistent_full_sweep_bitwise_vs_graph():
    import bench
    from int4_weight_only_04_amd import w4
    specs, projs = bench.build_sweep()
    _check_against_graph(projs, (w4.SWEEP_PERSISTENT,))


def test_persistent_watchdog_timeout_reported_then_recovers():
    from int4_weight_only_04_amd import w4
    built = [_proj(w4, *spec) for spec in SMALL[:4]]
    projs = [p for p, _ in built]
    stream = torch.cuda.Stream()
    ref_sweep = w4.Sweep(projs, mode=w4.SWEEP_GRAPH)
    ref = _run(ref_sweep, projs, stream)
    ref_sweep.close()
    sw = w4.Sweep(projs, mode=w4.SWEEP_PERSISTENT)
    assert not sw.status()
    # 10 ns: every wait that has to wait at all gives up; the kernel still ends
    sw.set_watchdog(1e-8)
    print("[persist] watchdog 10 ns", flush=True)
    _run(sw, projs, stream)
    assert sw.status(), "a 10 ns wait limit must be reported as a timeout"
    assert not sw.status(), "the status is cleared once read"
    sw.set_watchdog(0.2)
    print("[persist] watchdog 200 ms", flush=True)
    got = _run(sw, projs, stream)
    assert not sw.status()
    assert _same(ref, got)
    sw.close()
