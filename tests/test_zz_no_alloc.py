"""GPU check of the allocation-free argmax GEMV (w4_gemv_argmax_noalloc)
through the C ABI: on two calls in a row, the second one smaller, its logits
and argmax equal those of w4_gemv with a caller workspace (the same kernels,
so bit for bit), and on the small case both lie within the oracle's bar."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import dev_f16, dev_u8, near_tie_set, tol_plain

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_04_amd import w4
    w4.lib()  # fail loudly if the HIP library is missing


def _both(w4, pw, ps, x, n, k, group):
    """(y, argmax) from the workspace entry point and from the allocation-free one."""
    y_ws = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    am_ws = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(w4.gemv_workspace_size(n, k, group, True), dtype=torch.uint8, device="cuda")
    w4.gemv(pw, ps, x, y_ws, n, k, group, argmax=am_ws, workspace=ws)
    y_na = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    am_na = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    w4.gemv_argmax_noalloc(pw, ps, x, y_na, am_na, n, k, group)
    torch.cuda.synchronize()
    return (y_ws.cpu().numpy(), int(am_ws.item()), y_na.cpu().numpy(), int(am_na.item()))


def test_noalloc_matches_workspace_entry_point_two_calls():
    from int4_weight_only_04_amd import w4
    # call 1: the lm_head shape (152064 x 3584, G = 128), drawn in packed form
    n1, k1, g1 = synthetic.VOCAB, synthetic.HIDDEN, synthetic.GROUP
    wb, sb = w4.packed_size(n1, k1, g1, "plain")
    pw1, ps1, x1 = synthetic.packed_random(9101, wb, sb // 2, k1)
    print(f"[no_alloc] call 1 n={n1} k={k1} group={g1}", flush=True)
    y_ws, a_ws, y_na, a_na = _both(w4, dev_u8(pw1), dev_u8(ps1), dev_f16(x1), n1, k1, g1)
    assert np.array_equal(y_ws.view(np.uint32), y_na.view(np.uint32))
    assert a_na == a_ws == int(np.argmax(y_na))
    rows = np.unique(np.concatenate([[0, n1 - 1, a_na], np.random.default_rng(5).integers(0, n1, 200)]))
    y_ref, a_ref = oracle.gemv_packed(pw1, ps1, x1, n1, k1, g1, rows=rows)
    assert np.all(np.abs(y_na[rows].astype(np.float64) - y_ref) <= tol_plain(a_ref))

    # call 2: smaller (the tiny config, 512 x 256, G = 64); the scratch still
    # holds call 1's partials past this call's workgroups
    n2, k2, g2 = 512, 256, 64
    q, s, x2 = synthetic.logical(0, n2, k2, g2, 0.005, 0.02)
    pw2, ps2 = w4.pack(q, s, g2, "plain")
    print(f"[no_alloc] call 2 n={n2} k={k2} group={g2}", flush=True)
    y_ws, a_ws, y_na, a_na = _both(w4, dev_u8(pw2), dev_u8(ps2), dev_f16(x2), n2, k2, g2)
    assert np.array_equal(y_ws.view(np.uint32), y_na.view(np.uint32))
    assert a_na == a_ws == int(np.argmax(y_na))
    y_ref, a_ref = oracle.gemv(q, s, x2, g2)
    assert np.all(np.abs(y_na.astype(np.float64) - y_ref) <= tol_plain(a_ref))
    assert a_na in set(near_tie_set(y_ref, a_ref).tolist())
