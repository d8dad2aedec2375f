"""GPU parity of decode attention over a paged KV cache (w4_attn_decode through
the C ABI) against the CPU oracle on the same seeded inputs.

Tolerance per output element: |o_gpu - o_ref| <= 2e-3 * A + 1e-5 with
A = sum_t p_t |V_t| from the oracle.  Derivation: the fp16 output rounds by at
most 2^-11 |o| <= 2^-11 A (4.9e-4 A); the softmax weights are rounded to fp16
for the matrix-core product P V, and the sum that normalises them adds the
same rounded weights, so the output is a convex combination whose weights are
each off by a relative 2 * 2^-11 at most: <= 2^-10 A (9.8e-4 A; weights below
2^-14 round to subnormals with an absolute error under 2^-25 each, inside the
1e-5 term); scores are fp32 sums of 128 exact fp16 products (for N(0,1) data
|ds| <~ 6e-5, moving the weighted sum by <~ 1.2e-4 A); the fast exponential
and the fp32 sums over the chunk's tokens plus the wave and chunk merges add
< 2e-5 A.  That is <~ 1.6e-3 A in the worst case, under the 2e-3 A bar.

Shapes follow the model (28 query heads over 4 KV heads of 128) and the
pages' context of up to 4096 tokens; the context lengths straddle page and
chunk boundaries, where the pages' softmax bug showed (page tails)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle

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


def _h(v):
    return np.asarray(v, np.float16).view(np.uint16)


def make_cache(seed, n_heads, n_kv, page, max_ctx, extra_pages=3):
    rng = np.random.default_rng(seed)
    npages = (max_ctx + page - 1) // page
    pages = npages + extra_pages
    q = _h(rng.standard_normal((n_heads, 128)))
    kc = _h(rng.standard_normal((pages, n_kv, page, 128)))
    vc = _h(rng.standard_normal((pages, n_kv, page, 128)))
    table = rng.permutation(pages).astype(np.int32)[:npages]
    return q, kc, vc, table


class Dev:
    """Device copies of one cache and the buffers of an attention call."""

    def __init__(self, q, kc, vc, table, n_kv, page, max_ctx):
        w4 = _w4()
        self.n_heads = q.shape[0]
        self.n_kv, self.page, self.max_ctx = n_kv, page, max_ctx
        f16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.float16)
        self.q, self.kc, self.vc = f16(q), f16(kc), f16(vc)
        self.table = torch.from_numpy(table).cuda()
        self.ctx = torch.ones(1, dtype=torch.int32, device="cuda")
        self.out = torch.full((self.n_heads, 128), float("nan"), dtype=torch.float16, device="cuda")
        self.ws = torch.full((w4.attn_decode_workspace_size(self.n_heads, max_ctx),), 0xFF, dtype=torch.uint8,
                             device="cuda")
        self.scale = 1.0 / np.sqrt(128.0)

    def launch(self, stream=None):
        _w4().attn_decode(self.q, self.kc, self.vc, self.table, self.ctx, self.max_ctx, self.out, self.n_kv,
                          self.page, self.scale, self.ws, stream=stream)

    def run(self, ctx):
        self.ctx.fill_(ctx)
        self.launch()
        torch.cuda.synchronize()
        return self.out.cpu().view(torch.int16).numpy().view(np.float16).astype(np.float64)


def check(o, q, kc, vc, table, ctx, n_kv, page):
    ref, a = oracle.attn_decode(q, kc, vc, table, ctx, n_kv, page, 1.0 / np.sqrt(128.0))
    assert np.all(np.isfinite(o))
    err = np.abs(o - ref)
    tol = 2e-3 * a + 1e-5
    assert np.all(err <= tol), (ctx, float((err / tol).max()))


CTXS = [1, 2, 15, 16, 17, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 1000, 4095, 4096]


def test_attn_qwen_shape_page_tails():
    """28 query heads over 4 KV heads, pages of 16 tokens, one cache of 4096
    tokens; every context length runs on the same buffers (the kernel reads
    the length from device memory)."""
    q, kc, vc, table = make_cache(1, 28, 4, 16, 4096)
    d = Dev(q, kc, vc, table, 4, 16, 4096)
    for ctx in CTXS:
        check(d.run(ctx), q, kc, vc, table, ctx, 4, 16)


@pytest.mark.parametrize("n_heads,n_kv,page,max_ctx,ctx", [
    (8, 8, 32, 300, 77),       # one query head per KV head
    (16, 2, 8, 300, 300),      # eight per KV head
    (12, 4, 64, 1000, 999),
    (7, 1, 128, 200, 129),
    (28, 4, 1, 50, 50),        # one token per page
    (4, 2, 256, 600, 513),
])
def test_attn_shapes(n_heads, n_kv, page, max_ctx, ctx):
    q, kc, vc, table = make_cache(n_heads * 100 + page, n_heads, n_kv, page, max_ctx)
    d = Dev(q, kc, vc, table, n_kv, page, max_ctx)
    check(d.run(ctx), q, kc, vc, table, ctx, n_kv, page)


@pytest.mark.parametrize("ctx", [1, 200, 8193, 8320, 8321, 9000])
def test_attn_long_context_combine(ctx):
    """A workspace of more than 64 chunks of 128 tokens (max_ctx 9000) takes the
    combine's blocked path (the chunk maxima in blocks of 64 lanes), whatever
    the context: 1 and 200 tokens use one and two chunks of it, 8193 tokens
    end one token into the 65th chunk, 8320 and 8321 straddle the 66th, 9000
    needs 71 chunks."""
    q, kc, vc, table = make_cache(11, 8, 2, 16, 9000)
    d = Dev(q, kc, vc, table, 2, 16, 9000)
    check(d.run(ctx), q, kc, vc, table, ctx, 2, 16)


@pytest.mark.parametrize("max_ctx,ctx", [(4096, 4096), (4096, 2049), (2000, 1999)])
def test_attn_combine_one_round_widths(max_ctx, ctx):
    """The combine's one-round path loads 8 partials per thread for at most 32
    chunks (max_ctx <= 4096) and 16 for 33..64 chunks (max_ctx 8192, the same
    contexts); 1999 tokens use 16 chunks, the last one ragged."""
    q, kc, vc, table = make_cache(12 + ctx, 8, 2, 16, max_ctx)
    d = Dev(q, kc, vc, table, 2, 16, max_ctx)
    check(d.run(ctx), q, kc, vc, table, ctx, 2, 16)
    if max_ctx == 4096:
        q2, kc2, vc2, table2 = make_cache(13, 8, 2, 16, 8192)
        d2 = Dev(q2, kc2, vc2, table2, 2, 16, 8192)
        check(d2.run(ctx), q2, kc2, vc2, table2, ctx, 2, 16)


def test_attn_context_clamped():
    """ctx above max_ctx uses max_ctx; ctx below 1 uses 1."""
    q, kc, vc, table = make_cache(5, 8, 2, 16, 100)
    d = Dev(q, kc, vc, table, 2, 16, 100)
    check(d.run(1000), q, kc, vc, table, 100, 2, 16)
    check(d.run(0), q, kc, vc, table, 1, 2, 16)


def test_attn_out_of_range_page_entry_is_clamped():
    """A page-table entry outside the cache reads the nearest page inside it
    (wrong by contract, never a fault)."""
    q, kc, vc, table = make_cache(6, 8, 2, 16, 64)
    bad = table.copy()
    bad[1] = 10 ** 6
    d = Dev(q, kc, vc, bad, 2, 16, 64)
    o = d.run(64)
    fixed = bad.copy()
    fixed[1] = kc.shape[0] - 1
    check(o, q, kc, vc, fixed, 64, 2, 16)


def test_attn_dominant_key_and_uniform():
    """One key far above the others returns its V row; q = 0 averages V."""
    n_heads, n_kv, page, ctx = 8, 2, 16, 200
    q, kc, vc, table = make_cache(7, n_heads, n_kv, page, ctx)
    tstar = 133
    q1 = _h(np.full((n_heads, 128), 0.125))
    kc[table[tstar // page], :, tstar % page, :] = _h(np.full((n_kv, 128), 32.0))  # score 45 above the rest
    d = Dev(q1, kc, vc, table, n_kv, page, ctx)
    o = d.run(ctx)
    check(o, q1, kc, vc, table, ctx, n_kv, page)
    v_star = vc.view(np.float16)[table[tstar // page], :, tstar % page, :].astype(np.float64)
    for h in range(n_heads):
        assert np.array_equal(o[h], v_star[h // 4])
    d0 = Dev(np.zeros_like(q), kc, vc, table, n_kv, page, ctx)
    check(d0.run(ctx), np.zeros_like(q), kc, vc, table, ctx, n_kv, page)


def test_attn_graph_replay_as_context_grows():
    """One captured graph, replayed while the device context length grows:
    every replay equals the eager call bit for bit and the oracle within E."""
    q, kc, vc, table = make_cache(8, 28, 4, 16, 600)
    d = Dev(q, kc, vc, table, 4, 16, 600)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    d.ctx.fill_(1)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        d.launch(torch.cuda.current_stream())
    for ctx in (5, 16, 17, 300, 599, 600):
        d.ctx.fill_(ctx)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = d.out.clone()
        eager = d.run(ctx)
        assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.float16).astype(np.float64), eager)
        check(eager, q, kc, vc, table, ctx, 4, 16)


def test_attn_deterministic():
    q, kc, vc, table = make_cache(9, 28, 4, 16, 2000)
    d = Dev(q, kc, vc, table, 4, 16, 2000)
    assert np.array_equal(d.run(1777), d.run(1777))
