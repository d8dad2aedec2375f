"""C-ABI checks that need no GPU: the library loads and exports every symbol
include/w4.h declares, the host packer is bit-exact against the oracle's
packer (integer/byte work: bit-exact is the bar), and argument validation
rejects bad calls before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synthetic
from int4_weight_only_04_amd import w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_exactly_the_exports():
    assert _declared_functions() == sorted(w4.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = w4.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.w4_abi_version() == 1


def test_status_strings():
    names = ["W4_OK", "W4_EINVAL", "W4_ESHAPE", "W4_EALIGN", "W4_EHIP", "W4_ENOMEM", "W4_ECAPTURE"]
    for code, name in enumerate(names):
        assert w4.status_string(code) == name
    assert w4.status_string(99) == "W4_UNKNOWN"


PACK_CASES = [
    # (n, k, group, layout)
    (1, 8, 8, "plain"), (3, 32, 32, "plain"), (5, 64, 32, "plain"), (7, 72, 8, "plain"),
    (130, 1032, 8, "plain"), (512, 256, 64, "plain"), (65, 4104, 8, "plain"),
    (2, 64, 32, "gateup"), (6, 128, 64, "gateup"), (10, 256, 128, "gateup"),
    (14, 96, 32, "gateup"), (64, 384, 128, "gateup"),
]


@pytest.mark.parametrize("n,k,group,layout", PACK_CASES)
def test_packer_bit_exact_vs_oracle(n, k, group, layout):
    q, s, _ = synthetic.logical(100 + n + k, n, k, group)
    pw, ps = w4.pack(q, s, group, layout)
    opw, ops = oracle.pack(q, s, group, layout == "gateup")
    assert np.array_equal(pw, opw)
    assert np.array_equal(ps, ops)
    assert w4.packed_size(n, k, group, layout) == oracle.packed_sizes(n, k, group, layout == "gateup")


def test_packer_golden_bytes():
    import oracle_pins
    g = oracle_pins.load_golden()
    q, s = oracle_pins.golden_logical()
    pw, ps = w4.pack(q, s, g["group"], "plain")
    assert np.array_equal(pw, g["plain_pw"]) and np.array_equal(ps, g["plain_ps"])
    pw, ps = w4.pack(q, s, g["group"], "gateup")
    assert np.array_equal(pw, g["gateup_pw"]) and np.array_equal(ps, g["gateup_ps"])


@pytest.mark.parametrize("cfg", [synthetic.CONFIG_DOWN, synthetic.CONFIG_GATEUP],
                         ids=["down", "gateup"])
def test_packer_full_size_bit_exact(cfg):
    q, s, _ = synthetic.logical(cfg["seed"], cfg["n"], cfg["k"], cfg["group"], cfg["s_lo"], cfg["s_hi"])
    layout = "gateup" if cfg["kind"] == "gateup" else "plain"
    pw, ps = w4.pack(q, s, cfg["group"], layout)
    opw, ops = oracle.pack(q, s, cfg["group"], layout == "gateup")
    assert np.array_equal(pw, opw) and np.array_equal(ps, ops)


def test_pack_rejects_bad_nibble():
    q = np.zeros((4, 32), np.uint8)
    q[2, 17] = 16
    s = np.zeros((4, 1), np.uint16)
    with pytest.raises(w4.W4Error) as ei:
        w4.pack(q, s, 32)
    assert ei.value.status == w4.EINVAL
    assert "q[2][17] = 16" in str(ei.value)


@pytest.mark.parametrize("n,k,group,layout,status", [
    (0, 64, 32, "plain", w4.ESHAPE),
    (4, 4, 8, "plain", w4.ESHAPE),
    (4, 64, 48, "plain", w4.ESHAPE),      # group not a power of two
    (4, 64, 4, "plain", w4.ESHAPE),       # group < 8
    (4, 96, 64, "plain", w4.ESHAPE),      # k % group != 0
    (4, 64, 128, "plain", w4.ESHAPE),     # group > k
    (4, 65536, 128, "plain", w4.ESHAPE),  # k above the LDS staging limit
    (5, 64, 32, "gateup", w4.ESHAPE),     # odd n_total
    (4, 64, 32, 7, w4.EINVAL),            # unknown layout
])
def test_packed_size_validation(n, k, group, layout, status):
    with pytest.raises(w4.W4Error) as ei:
        w4.packed_size(n, k, group, layout)
    assert ei.value.status == status
    assert w4.last_error()


def test_pack_rejects_wrong_buffer_sizes():
    L = w4.lib()
    q = np.zeros((4, 32), np.uint8)
    s = np.zeros((4, 1), np.uint16)
    pw = np.zeros(64, np.uint8)
    ps = np.zeros(8, np.uint8)
    st = L.w4_pack(q.ctypes.data, s.ctypes.data, 4, 32, 32, 0, pw.ctypes.data, 63, ps.ctypes.data, 8)
    assert st == w4.EINVAL and "buffer sizes" in w4.last_error()
    st = L.w4_pack(None, s.ctypes.data, 4, 32, 32, 0, pw.ctypes.data, 64, ps.ctypes.data, 8)
    assert st == w4.EINVAL


def test_workspace_sizes():
    assert w4.gemv_workspace_size(152064, 3584, 128, False) == 0
    ws = w4.gemv_workspace_size(152064, 3584, 128, True)
    assert 0 < ws <= 1 << 20


def test_gemv_validation_before_launch():
    """Calls that fail validation never reach the device (safe without a GPU)."""
    L = w4.lib()
    A = 1 << 20  # 16-byte aligned fake addresses: only used where validation must fail first
    # null pointers
    assert L.w4_gemv(None, A, A, A, None, None, 0, 4, 64, 32, None) == w4.EINVAL
    assert L.w4_gemv(A, A, A, None, None, None, 0, 4, 64, 32, None) == w4.EINVAL
    # misalignment
    assert L.w4_gemv(A + 4, A, A, A, None, None, 0, 4, 64, 32, None) == w4.EALIGN
    assert L.w4_gemv(A, A + 8, A, A, None, None, 0, 4, 64, 32, None) == w4.EALIGN
    assert L.w4_gemv(A, A, A + 2, A, None, None, 0, 4, 64, 32, None) == w4.EALIGN
    # shapes
    assert L.w4_gemv(A, A, A, A, None, None, 0, 0, 64, 32, None) == w4.ESHAPE
    assert L.w4_gemv(A, A, A, A, None, None, 0, 4, 96, 64, None) == w4.ESHAPE
    # argmax without workspace / too small workspace
    assert L.w4_gemv(A, A, A, A, A, None, 0, 4, 64, 32, None) == w4.EINVAL
    assert L.w4_gemv(A, A, A, A, A, A, 16, 4, 64, 32, None) == w4.EINVAL
    assert L.w4_gemv(A, A, A, A, A, A + 8, 1 << 20, 4, 64, 32, None) == w4.EALIGN
    # gate/up: odd n_total
    assert L.w4_gemv_gateup_silu(A, A, A, A, 5, 64, 32, None) == w4.ESHAPE
    assert L.w4_gemv_gateup_silu(A, None, A, A, 6, 64, 32, None) == w4.EINVAL


def test_gemv_argmax_noalloc_validation_before_launch():
    """The allocation-free argmax entry point rejects bad arguments, and shapes
    whose partials exceed its static scratch, before any device call."""
    L = w4.lib()
    A = 1 << 20
    assert L.w4_gemv_argmax_noalloc(A, A, A, A, None, 4, 64, 32, None) == w4.EINVAL    # no argmax
    assert L.w4_gemv_argmax_noalloc(None, A, A, A, A, 4, 64, 32, None) == w4.EINVAL    # null weights
    assert L.w4_gemv_argmax_noalloc(A + 4, A, A, A, A, 4, 64, 32, None) == w4.EALIGN
    assert L.w4_gemv_argmax_noalloc(A, A, A, A, A, 4, 96, 64, None) == w4.ESHAPE       # k % group
    # 600000 x 3584 needs 37500 workgroups of partials, past the 256 KiB scratch
    assert L.w4_gemv_argmax_noalloc(A, A, A, A, A, 600000, 3584, 128, None) == w4.ESHAPE
    assert "scratch" in w4.last_error()


def test_gemm_validation_before_launch():
    """Prefill GEMM argument checks run before any device call."""
    L = w4.lib()
    A = 1 << 20
    W = 1 << 30  # a workspace size large enough for the small shapes below
    assert L.w4_gemm(None, A, A, A, A, W, 8, 4, 64, 32, None) == w4.EINVAL
    assert L.w4_gemm(A, A, A, None, A, W, 8, 4, 64, 32, None) == w4.EINVAL
    assert L.w4_gemm(A, A, A + 2, A, A, W, 8, 4, 64, 32, None) == w4.EALIGN
    assert L.w4_gemm(A + 8, A, A, A, A, W, 8, 4, 64, 32, None) == w4.EALIGN
    assert L.w4_gemm(A, A, A, A + 2, A, W, 8, 4, 64, 32, None) == w4.EALIGN
    assert L.w4_gemm(A, A, A, A, A, W, 0, 4, 64, 32, None) == w4.ESHAPE
    assert L.w4_gemm(A, A, A, A, A, W, (1 << 20) + 1, 4, 64, 32, None) == w4.ESHAPE
    assert L.w4_gemm(A, A, A, A, A, W, 8, 4, 96, 64, None) == w4.ESHAPE
    assert L.w4_gemm(A, A, A, A, A, W, 8, 0, 64, 32, None) == w4.ESHAPE
    # a split shape without (or with too small, or misaligned) workspace
    need = w4.gemm_workspace_size(512, 3584, 18944, 128)
    assert need > 0
    assert L.w4_gemm(A, A, A, A, None, 0, 512, 3584, 18944, 128, None) == w4.EINVAL
    assert L.w4_gemm(A, A, A, A, A, need - 1, 512, 3584, 18944, 128, None) == w4.EINVAL
    assert L.w4_gemm(A, A, A, A, A + 4, need, 512, 3584, 18944, 128, None) == w4.EALIGN
    assert L.w4_gemm_gateup_silu(A, A, A, A, 8, 5, 64, 32, None) == w4.ESHAPE
    assert L.w4_gemm_gateup_silu(A, A, A, A + 1, 8, 6, 64, 32, None) == w4.EALIGN
    assert L.w4_gemm_gateup_silu(A, None, A, A, 8, 6, 64, 32, None) == w4.EINVAL
    assert "w4_gemm_gateup_silu" in w4.last_error()


def test_gemm_workspace_sizes():
    # split-k partials: splits x m x n fp32; no split once the grid covers the chip.
    # From 256 token rows the tiles are 128 x 128, split to fit 512 workgroups:
    assert w4.gemm_workspace_size(512, 4608, 3584, 128) == 3 * 512 * 4608 * 4    # 144 tiles, 3 splits
    assert w4.gemm_workspace_size(512, 3584, 18944, 128) == 4 * 512 * 3584 * 4   # 112 tiles, 4 splits
    assert w4.gemm_workspace_size(512, 3584, 3584, 128) == 4 * 512 * 3584 * 4
    assert w4.gemm_workspace_size(4096, 37888, 3584, 128) == 0                   # 9472 tiles
    # below 256 rows, 64 x 128 tiles split to reach 256 workgroups: 112 tiles, 3 splits
    assert w4.gemm_workspace_size(200, 3584, 3584, 128) == 3 * 200 * 3584 * 4
    assert w4.gemm_workspace_size(1, 64, 64, 64) == 0  # one k step: nothing to split


def test_attn_validation_before_launch():
    """Decode-attention argument checks run before any device call."""
    L = w4.lib()
    A = 1 << 20
    W = 1 << 30

    def call(q=A, kc=A, vc=A, tab=A, npages=4, ctx=A, max_ctx=64, out=A, nh=28, nkv=4, dim=128, page=16,
             ws=A, wsb=W):
        return L.w4_attn_decode(q, kc, vc, tab, npages, ctx, max_ctx, out, nh, nkv, dim, page, 0.088, ws, wsb,
                                None)

    assert call(q=None) == w4.EINVAL
    assert call(ctx=None) == w4.EINVAL
    assert call(ws=None) == w4.EINVAL
    assert call(dim=64) == w4.ESHAPE
    assert call(nh=30) == w4.ESHAPE            # not a multiple of n_kv
    assert call(nh=40) == w4.ESHAPE            # 10 query heads per KV head
    assert call(page=24) == w4.ESHAPE          # not a power of two
    assert call(max_ctx=0) == w4.ESHAPE
    assert call(npages=0) == w4.ESHAPE
    assert call(q=A + 2) == w4.EALIGN
    assert call(ctx=A + 2) == w4.EALIGN
    need = w4.attn_decode_workspace_size(28, 64)
    assert need == 28 * 130 * 4
    assert call(wsb=need - 1) == w4.EINVAL
    # one (128 partial outputs, max, sum) record per query head and 128-token chunk
    assert w4.attn_decode_workspace_size(28, 128) == 28 * 130 * 4
    assert w4.attn_decode_workspace_size(28, 129) == 2 * 28 * 130 * 4
    assert w4.attn_decode_workspace_size(28, 4096) == 32 * 28 * 130 * 4


def test_sweep_create_validation():
    L = w4.lib()
    A = 1 << 20
    handle = ctypes.c_void_p()
    assert L.w4_decode_linear_sweep_create(None, 0, 1, ctypes.byref(handle)) == w4.EINVAL
    descs = (w4.ProjDesc * 2)()
    for d in descs:
        d.kind, d.group, d.n, d.k = w4.PROJ_PLAIN, 32, 4, 64
        d.packed_w = d.packed_s = d.x = d.out = A
    descs[1].kind = 9
    assert L.w4_decode_linear_sweep_create(descs, 2, 1, ctypes.byref(handle)) == w4.EINVAL
    assert "projection 1" in w4.last_error()
    descs[1].kind = w4.PROJ_LMHEAD_ARGMAX  # no workspace
    assert L.w4_decode_linear_sweep_create(descs, 2, 0, ctypes.byref(handle)) == w4.EINVAL
    descs[1].kind = w4.PROJ_GATEUP_SILU
    descs[1].n = 7
    assert L.w4_decode_linear_sweep_create(descs, 2, 0, ctypes.byref(handle)) == w4.ESHAPE
    assert not handle.value
    assert L.w4_decode_linear_sweep_destroy(None) == w4.OK
    assert L.w4_decode_linear_sweep(None, None) == w4.EINVAL


def test_persistent_sweep_validation_before_launch():
    """The persistent modes' shape limits (k a multiple of 512, 64 <= G <= 512,
    at most 256 projections), the mode range and the status / watchdog calls'
    argument checks all fail before any device call."""
    L = w4.lib()
    A = 1 << 20
    handle = ctypes.c_void_p()
    descs = (w4.ProjDesc * 2)()
    for d in descs:
        d.kind, d.group, d.n, d.k = w4.PROJ_PLAIN, 128, 64, 1024
        d.packed_w = d.packed_s = d.x = d.out = A
    assert L.w4_decode_linear_sweep_create(descs, 2, 4, ctypes.byref(handle)) == w4.EINVAL
    assert "mode" in w4.last_error()
    assert L.w4_decode_linear_sweep_create(descs, 2, -1, ctypes.byref(handle)) == w4.EINVAL
    descs[1].k = 768  # a multiple of G = 128 and of 256, not of 512
    for mode in (w4.SWEEP_PERSISTENT, w4.SWEEP_PERSISTENT_EAGER):
        assert L.w4_decode_linear_sweep_create(descs, 2, mode, ctypes.byref(handle)) == w4.ESHAPE
        assert "projection 1" in w4.last_error() and "512" in w4.last_error()
    descs[1].k = 1024
    descs[0].group = 32
    assert L.w4_decode_linear_sweep_create(descs, 2, w4.SWEEP_PERSISTENT, ctypes.byref(handle)) == w4.ESHAPE
    assert "projection 0" in w4.last_error() and "group" in w4.last_error()
    many = (w4.ProjDesc * 257)()
    for d in many:
        d.kind, d.group, d.n, d.k = w4.PROJ_PLAIN, 128, 64, 1024
        d.packed_w = d.packed_s = d.x = d.out = A
    assert L.w4_decode_linear_sweep_create(many, 257, w4.SWEEP_PERSISTENT, ctypes.byref(handle)) == w4.ESHAPE
    assert "257" in w4.last_error()
    assert not handle.value
    flag = ctypes.c_int32(5)
    assert L.w4_decode_linear_sweep_status(None, ctypes.byref(flag)) == w4.EINVAL
    assert L.w4_decode_linear_sweep_set_watchdog(None, ctypes.c_double(0.1)) == w4.EINVAL


def test_step_glue_validation_before_launch():
    """Embedding, residual + RMSNorm and rotary/KV-append checks run before
    any device call."""
    L = w4.lib()
    A = 1 << 20
    assert L.w4_embed(None, 10, 64, A, A, None) == w4.EINVAL
    assert L.w4_embed(A, 10, 0, A, A, None) == w4.ESHAPE
    assert L.w4_embed(A, 0, 64, A, A, None) == w4.ESHAPE
    assert L.w4_embed(A + 1, 10, 64, A, A, None) == w4.EALIGN
    assert L.w4_embed(A, 10, 64, A + 2, A, None) == w4.EALIGN
    assert L.w4_add_rmsnorm(A, None, A, 0, 1e-6, A, None) == w4.ESHAPE
    assert L.w4_add_rmsnorm(A, None, A, 64, -1.0, A, None) == w4.EINVAL
    assert L.w4_add_rmsnorm(A, None, A, 64, float("nan"), A, None) == w4.EINVAL
    assert L.w4_add_rmsnorm(None, None, A, 64, 1e-6, A, None) == w4.EINVAL
    assert L.w4_add_rmsnorm(A + 2, None, A, 64, 1e-6, A, None) == w4.EALIGN

    def rope(qkv=A, bias=None, pos=A, nh=28, nkv=4, dim=128, theta=1e6, q=A, kc=A, vc=A, tab=A, npages=4,
             page=16, max_ctx=64, ctx=A):
        return L.w4_rope_kv_append(qkv, bias, pos, nh, nkv, dim, theta, q, kc, vc, tab, npages, page, max_ctx,
                                   ctx, None)

    assert rope(dim=64) == w4.ESHAPE
    assert rope(nh=30) == w4.ESHAPE
    assert rope(page=12) == w4.ESHAPE
    assert rope(max_ctx=0) == w4.ESHAPE
    assert rope(theta=0.0) == w4.EINVAL
    assert rope(pos=None) == w4.EINVAL
    assert rope(kc=None) == w4.EINVAL
    assert rope(qkv=A + 2) == w4.EALIGN
    assert rope(bias=A + 1) == w4.EALIGN
    # the caches are read by the attention in 16-byte words
    assert rope(kc=A + 2) == w4.EALIGN
    assert rope(vc=A + 8) == w4.EALIGN
    assert "16-byte" in w4.last_error()


def test_read_probe_validation_before_launch():
    L = w4.lib()
    A = 1 << 20
    assert L.w4_read_probe(None, 1024, A, None) == w4.EINVAL
    assert L.w4_read_probe(A, 0, A, None) == w4.ESHAPE
    assert L.w4_read_probe(A, 1000, A, None) == w4.ESHAPE
    assert L.w4_read_probe(A + 8, 1024, A, None) == w4.EALIGN


def test_w4a8_validation_before_launch():
    L = w4.lib()
    A = 1 << 20
    assert L.w4_quantize_act8(None, 256, 64, A, A, None) == w4.EINVAL
    assert L.w4_quantize_act8(A, 250, 64, A, A, None) == w4.ESHAPE      # k % G
    assert L.w4_quantize_act8(A, 256, 48, A, A, None) == w4.ESHAPE      # G not a power of two
    assert L.w4_quantize_act8(A + 8, 256, 64, A, A, None) == w4.EALIGN  # x not 16-byte aligned
    assert L.w4_quantize_act8(A, 256, 64, A + 4, A, None) == w4.EALIGN  # codes not 8-byte aligned
    assert L.w4_gemv_a8(A, A, A, None, A, None, None, 0, 4, 64, 32, None) == w4.EINVAL
    assert L.w4_gemv_a8(A, A, A, A + 2, A, None, None, 0, 4, 64, 32, None) == w4.EALIGN
    assert L.w4_gemv_a8(A, A, A + 8, A, A, None, None, 0, 4, 64, 32, None) == w4.EALIGN
    assert L.w4_gemv_a8(A, A, A, A, A, A, A, 16, 4, 64, 32, None) == w4.EINVAL   # argmax workspace too small
    assert L.w4_gemv_gateup_silu_a8(A, A, A, A, A, 7, 64, 32, None) == w4.ESHAPE
    assert L.w4_gemv_gateup_silu_a8(A, A, A, None, A, 8, 64, 32, None) == w4.EINVAL


def test_fused_norm_validation_before_launch():
    """The residual and norm-prologue GEMVs reject bad calls on the host."""
    L = w4.lib()
    A = 1 << 20
    f = ctypes.c_float
    assert L.w4_gemv_residual(A, A, A, A, A, None, A, 64, 256, 64, None) == w4.EINVAL        # null h_out
    assert L.w4_gemv_residual(A, A, A, A, None, A, A, 64, 256, 64, None) == w4.EINVAL        # null h_in
    assert L.w4_gemv_residual(A, A, A, A, A, A, None, 64, 256, 64, None) == w4.EINVAL        # null ss_part
    assert L.w4_gemv_residual(A, A, A, A, A, A, A + 4, 64, 256, 64, None) == w4.EALIGN       # ss_part 16-byte
    assert L.w4_gemv_residual(A, A, A, A, A + 2, A, A, 64, 256, 64, None) == w4.EALIGN       # h_in 4-byte
    assert L.w4_gemv_residual(A, A, A, A, A, A, A, 64, 250, 64, None) == w4.ESHAPE           # k % G
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("w", A), ("s", A), ("h", A), ("g", A), ("ss", A), ("parts", 4), ("eps", f(1e-6)), ("xo", None), ("y", A),
        ("am", None), ("ws", None), ("wsb", 0), ("n", 64), ("k", 256), ("group", 64), ("st", None))]
    assert L.w4_gemv_rmsnorm(*args(h=None)) == w4.EINVAL
    assert L.w4_gemv_rmsnorm(*args(g=None)) == w4.EINVAL
    assert L.w4_gemv_rmsnorm(*args(ss=None)) == w4.EINVAL
    assert L.w4_gemv_rmsnorm(*args(parts=0)) == w4.ESHAPE
    assert L.w4_gemv_rmsnorm(*args(parts=1025)) == w4.ESHAPE
    assert L.w4_gemv_rmsnorm(*args(eps=f(-1.0))) == w4.EINVAL
    assert L.w4_gemv_rmsnorm(*args(eps=f(float("inf")))) == w4.EINVAL
    assert L.w4_gemv_rmsnorm(*args(h=A + 4)) == w4.EALIGN
    assert L.w4_gemv_rmsnorm(*args(g=A + 8)) == w4.EALIGN
    assert L.w4_gemv_rmsnorm(*args(ss=A + 4)) == w4.EALIGN
    assert L.w4_gemv_rmsnorm(*args(xo=A + 8)) == w4.EALIGN
    assert L.w4_gemv_rmsnorm(*args(am=A, ws=A, wsb=16)) == w4.EINVAL   # argmax workspace too small
    assert L.w4_gemv_gateup_silu_rmsnorm(A, A, A, A, A, 4, f(1e-6), None, A, 63, 256, 64, None) == w4.ESHAPE
    assert L.w4_gemv_gateup_silu_rmsnorm(A, A, A, A, A, 2000, f(1e-6), None, A, 64, 256, 64, None) == w4.ESHAPE
    assert L.w4_gemv_gateup_silu_rmsnorm(A, A, None, A, A, 4, f(1e-6), None, A, 64, 256, 64, None) == w4.EINVAL


@pytest.mark.parametrize("n,k,group,parts", [(3584, 3584, 128, 896), (3584, 18944, 128, 896), (37, 96, 32, 10),
                                             (65536, 256, 64, 8192), (65540, 256, 64, 8193)])
def test_residual_parts(n, k, group, parts):
    """One partial per 4-row tile, or per pair of tiles once the matrix has
    16384 tiles or more (the launch's two-tile units)."""
    assert w4.residual_parts(n, k, group) == parts


def _step_desc(layers_arr, **kw):
    A = 1 << 20
    d = w4.StepDesc()
    vals = dict(layers=len(layers_arr), hidden=256, n_heads=2, n_kv_heads=1, head_dim=128, inter=512, vocab=300,
                group=64, page_size=16, num_pages=4, max_ctx=64, rms_eps=1e-6, rope_theta=1e6)
    vals.update(kw)
    for k, v in vals.items():
        setattr(d, k, v)
    d.layer = layers_arr
    for name in ("embed", "final_norm", "lm_w", "lm_s", "page_table", "token", "pos", "logits"):
        setattr(d, name, A)
    return d


def _layer_arr(n):
    A = 1 << 20
    arr = (w4.LayerDesc * n)()
    for L in arr:
        for name, _ in w4.LayerDesc._fields_:
            setattr(L, name, A)
        L.qkv_bias = None
    return arr


def test_decode_step_create_validation():
    """Every descriptor rule is checked before anything is allocated."""
    L = w4.lib()
    handle = ctypes.c_void_p()

    def create(d):
        return L.w4_decode_step_create(ctypes.byref(d), 1, ctypes.byref(handle))

    arr = _layer_arr(2)
    assert L.w4_decode_step_create(None, 1, ctypes.byref(handle)) == w4.EINVAL
    assert create(_step_desc(arr, layers=0)) == w4.EINVAL
    assert create(_step_desc(arr, head_dim=64)) == w4.ESHAPE
    assert create(_step_desc(arr, n_heads=3, n_kv_heads=2)) == w4.ESHAPE
    assert create(_step_desc(arr, rms_eps=-1.0)) == w4.EINVAL
    assert create(_step_desc(arr, rope_theta=0.0)) == w4.EINVAL
    assert create(_step_desc(arr, hidden=200)) == w4.ESHAPE        # k % G for qkv
    assert "layer 0 qkv" in w4.last_error()
    assert create(_step_desc(arr, inter=500)) == w4.ESHAPE         # k % G for down
    assert "down" in w4.last_error()
    d = _step_desc(arr)
    d.token = None
    assert create(d) == w4.EINVAL
    d = _step_desc(arr)
    d.trace = (1 << 20) + 16
    assert create(d) == w4.EALIGN
    bad = _layer_arr(2)
    bad[1].k_cache = None
    assert create(_step_desc(bad)) == w4.EINVAL
    assert "layer 1" in w4.last_error()
    bad = _layer_arr(2)
    bad[1].gateup_w = (1 << 20) + 8
    assert create(_step_desc(bad)) == w4.EALIGN
    for field, off in (("k_cache", 2), ("v_cache", 8)):
        bad = _layer_arr(2)
        setattr(bad[0], field, (1 << 20) + off)  # element-aligned, not 16-byte aligned
        assert create(_step_desc(bad)) == w4.EALIGN
        assert "layer 0" in w4.last_error()
    bad = _layer_arr(2)
    bad[1].attn_norm = (1 << 20) + 8         # read 16 bytes at a time by the qkv norm prologue
    assert create(_step_desc(bad)) == w4.EALIGN
    bad = _layer_arr(2)
    bad[1].mlp_norm = (1 << 20) + 4
    assert create(_step_desc(bad)) == w4.EALIGN
    d = _step_desc(arr)
    d.final_norm = (1 << 20) + 4
    assert create(d) == w4.EALIGN
    assert not handle.value
    assert L.w4_decode_step(None, None) == w4.EINVAL
    assert L.w4_decode_step_destroy(None) == w4.OK


def test_decode_step_trace_layout():
    d = _step_desc(_layer_arr(3), hidden=512, n_heads=4, n_kv_heads=2, inter=1024)
    offs, stride, total = w4.trace_layout(d)
    sizes = [4 * 512, 2 * 512, 4 * 1024, 2 * 512, 2 * 512, 4 * 512, 4 * 512, 2 * 512, 2 * 1024, 4 * 512]
    expect, o = [], 0
    for b in sizes:
        expect.append(o)
        o += -(-b // 256) * 256
    assert offs == expect and stride == o
    assert total == 3 * stride + expect[2]
    assert w4.step_trace_bytes(hidden=512, n_heads=4, n_kv_heads=2, inter=1024, layers=3) == total


def test_launch_without_device_reports_hip_error():
    """With no GPU present, a validated call fails with W4_EHIP (no launch)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this case only runs where no device exists")
    L = w4.lib()
    A = 1 << 20
    st = L.w4_gemv(A, A, A, A, None, None, 0, 4, 64, 32, None)
    assert st == w4.EHIP, w4.last_error()
