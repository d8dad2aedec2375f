"""GPU parity of the full decode step (embedding, residual add + RMSNorm,
rotary embedding + KV append, the INT4 projections, paged attention, lm_head
+ argmax, position advance) through the C ABI, against the oracle.

Each operation is checked on its own, then the whole step with teacher
forcing: the step copies every intermediate into a trace buffer, the oracle's
layer (oracle/step.py) takes the GPU's value of each stage as the input of the
next one, and every GPU stage is held to the bar of its own operation:

  * RMSNorm (fp16 output): 2^-11 |x| (the fp16 rounding) plus
    (t/2 + 8) 2^-24 |x| with t = max(ceil(n/1024) + 21, 25) bounding the
    additions a square passes through in the fp32 sum of squares (the
    one-workgroup norm kernel, or the norm folded into qkv), plus the
    sqrt, reciprocal and two products; plus 2^-25 below the fp16 normal range;
  * INT4 products: 1e-3 sum|w x| + 1e-5 (fused gate/up: its propagated form);
  * rotary embedding (fp16 output): 2^-11 |r| plus 5 2^-24 (|x_i| + |x_i+64|)
    for the fp32 bias add, the fp32 sine and cosine and the rotation; v: the
    bias add and the fp16 rounding;
  * attention: 2e-3 sum p|V| + 1e-5 (its own derived bar);
  * residual adds: bit-exact (fp32 additions of the same operands);
  * argmax: the GPU token is the lowest-index maximum of the GPU's logits
    (bit-exact) and lies in the oracle's near-tie set.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import dev_f16, dev_u8, near_tie_set, tol_gateup, tol_plain
from oracle import step as ostep

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_04_amd import w4
    w4.lib()  # fail loudly if the HIP library is missing


def _w4():
    from int4_weight_only_04_amd import w4
    return w4


def _half(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def _host16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def tol_rmsnorm(x_ref, n):
    # t bounds the fp32 roundings any square passes through on its way into
    # the sum of squares: the single-workgroup norm kernel has ceil(n/1024) +
    # 21 (per-thread terms, 6 shuffle levels, the cross-wave sum); the norm
    # folded into the qkv projection has the square, 3 additions in the down
    # projection's part (up to 8 rows), 15 per-lane additions of the parts and
    # 6 shuffle levels, i.e. 25
    t = max(math.ceil(n / 1024) + 21, 25)
    return (2.0 ** -11 + (t / 2 + 8) * U) * np.abs(x_ref) + 2.0 ** -25


def tol_rope(r_ref, x):
    half = x.shape[-1] // 2
    mag = np.abs(x[..., :half]) + np.abs(x[..., half:])
    return 2.0 ** -11 * np.abs(r_ref) + 5 * U * np.concatenate([mag, mag], axis=-1) + 2.0 ** -25


def assert_within(got, ref, tol, what):
    err = np.abs(np.asarray(got, np.float64) - ref)
    assert np.all(np.isfinite(got)), what
    bad = err > tol
    assert not bad.any(), (what, float((err / tol).max()), int(bad.sum()))


# ---------------------------------------------------------------- single ops


def test_embed_rows_exact_and_clamped():
    w4 = _w4()
    vocab, hidden = 1000, 3584
    tb = synthetic.half_bits_uniform(11, vocab * hidden, lo_exp=13).reshape(vocab, hidden)
    dt = dev_f16(tb)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    h = torch.full((hidden,), float("nan"), dtype=torch.float32, device="cuda")
    for t, row in ((0, 0), (1, 1), (517, 517), (999, 999), (-5, 0), (10 ** 6, 999)):
        tok.fill_(t)
        w4.embed(dt, tok, h)
        torch.cuda.synchronize()
        assert np.array_equal(h.cpu().numpy().astype(np.float64), _half(tb[row])), t


@pytest.mark.parametrize("n", [1, 100, 1024, 1025, 3584, 18944])
def test_add_rmsnorm_vs_oracle(n):
    w4 = _w4()
    rng = np.random.default_rng(n)
    h0 = (rng.standard_normal(n) * 3.0).astype(np.float32)
    y0 = rng.standard_normal(n).astype(np.float32)
    g = synthetic._scales(synthetic._rng(n), n, 0.5, 1.5)
    h = torch.from_numpy(h0.copy()).cuda()
    y = torch.from_numpy(y0).cuda()
    x = torch.full((n,), float("nan"), dtype=torch.float16, device="cuda")
    w4.add_rmsnorm(h, y, dev_f16(g), 1e-6, x)
    torch.cuda.synchronize()
    h_new = h0 + y0  # the same fp32 addition
    assert np.array_equal(h.cpu().numpy(), h_new)
    ref = oracle.rmsnorm(h_new.astype(np.float64), g, 1e-6)
    assert_within(_half(_host16(x)), ref, tol_rmsnorm(ref, n), "x")
    # without a residual: h is only read
    w4.add_rmsnorm(h, None, dev_f16(g), 0.0, x)
    torch.cuda.synchronize()
    assert np.array_equal(h.cpu().numpy(), h_new)
    ref0 = oracle.rmsnorm(h_new.astype(np.float64), g, 0.0)
    assert_within(_half(_host16(x)), ref0, tol_rmsnorm(ref0, n), "x, no residual")


def test_add_rmsnorm_deterministic():
    w4 = _w4()
    n = 3584
    rng = np.random.default_rng(5)
    h = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    g = dev_f16(synthetic._scales(synthetic._rng(5), n, 0.5, 1.5))
    x1 = torch.empty(n, dtype=torch.float16, device="cuda")
    x2 = torch.empty_like(x1)
    w4.add_rmsnorm(h, None, g, 1e-6, x1)
    w4.add_rmsnorm(h, None, g, 1e-6, x2)
    torch.cuda.synchronize()
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16))


@pytest.mark.parametrize("pos", [0, 1, 15, 16, 17, 2000, 4095])
@pytest.mark.parametrize("with_bias", [False, True])
def test_rope_kv_append_vs_oracle(pos, with_bias):
    w4 = _w4()
    nh, nkv, page, max_ctx = 28, 4, 16, 4096
    rows = (nh + 2 * nkv) * 128
    rng = np.random.default_rng(pos * 2 + with_bias)
    qkv = (rng.standard_normal(rows) * 2.0).astype(np.float32)
    bias = (rng.standard_normal(rows) * 0.5).astype(np.float32) if with_bias else None
    npages = max_ctx // page + 2
    kc0, vc0 = synthetic.kv_prefix(pos + 1, npages, nkv, page)
    table = synthetic.page_table(pos + 2, npages, max_ctx // page)
    kc, vc = dev_f16(kc0).view(npages, nkv, page, 128), dev_f16(vc0).view(npages, nkv, page, 128)
    q_out = torch.full((nh, 128), float("nan"), dtype=torch.float16, device="cuda")
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = torch.full((1,), pos, dtype=torch.int32, device="cuda")
    w4.rope_kv_append(torch.from_numpy(qkv).cuda(), None if bias is None else torch.from_numpy(bias).cuda(), p,
                      nh, nkv, 1e6, q_out, kc, vc, torch.from_numpy(table).cuda(), max_ctx, ctx)
    torch.cuda.synchronize()
    assert int(ctx.item()) == pos + 1
    x = (qkv + bias if bias is not None else qkv).astype(np.float64).reshape(nh + 2 * nkv, 128)
    q_ref = oracle.rope(x[:nh], pos, 1e6)
    k_ref = oracle.rope(x[nh:nh + nkv], pos, 1e6)
    v_ref = x[nh + nkv:]
    assert_within(_half(_host16(q_out)), q_ref, tol_rope(q_ref, x[:nh]), "q")
    kh, vh = _host16(kc), _host16(vc)
    pg, sl = table[pos // page], pos % page
    assert_within(_half(kh[pg, :, sl]), k_ref, tol_rope(k_ref, x[nh:nh + nkv]), "k")
    assert_within(_half(vh[pg, :, sl]), v_ref, (2.0 ** -11 + U) * np.abs(v_ref) + 2.0 ** -25, "v")
    mask = np.zeros(kh.shape, bool)
    mask[pg, :, sl] = True
    assert np.array_equal(kh[~mask], kc0[~mask]) and np.array_equal(vh[~mask], vc0[~mask])


def test_rope_kv_append_position_clamped():
    """A position outside [0, max_ctx) writes the nearest slot inside it."""
    w4 = _w4()
    nh, nkv, page, max_ctx = 8, 2, 16, 64
    rows = (nh + 2 * nkv) * 128
    qkv = torch.from_numpy(np.random.default_rng(3).standard_normal(rows).astype(np.float32)).cuda()
    table = torch.arange(4, dtype=torch.int32, device="cuda")
    for pos, used in ((1000, 63), (-7, 0)):
        kc = torch.zeros((4, nkv, page, 128), dtype=torch.float16, device="cuda")
        vc = torch.zeros_like(kc)
        q1 = torch.empty((nh, 128), dtype=torch.float16, device="cuda")
        q2 = torch.empty_like(q1)
        kc2, vc2 = torch.zeros_like(kc), torch.zeros_like(kc)
        ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
        w4.rope_kv_append(qkv, None, torch.full((1,), pos, dtype=torch.int32, device="cuda"), nh, nkv, 1e6, q1, kc,
                          vc, table, max_ctx, ctx)
        w4.rope_kv_append(qkv, None, torch.full((1,), used, dtype=torch.int32, device="cuda"), nh, nkv, 1e6, q2,
                          kc2, vc2, table, max_ctx)
        torch.cuda.synchronize()
        assert int(ctx.item()) == used + 1
        assert torch.equal(q1.view(torch.int16), q2.view(torch.int16))
        assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
        assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))


# ---------------------------------------------------------------- full step


class Model:
    """A seeded decoder on the device plus its logical weights for the oracle."""

    def __init__(self, seed, *, hidden, n_heads, n_kv, inter, vocab, group, layers, page, max_ctx, bias):
        w4 = _w4()
        self.cfg = ostep.Config(hidden=hidden, n_heads=n_heads, n_kv=n_kv, inter=inter, group=group, page=page,
                                eps=1e-6, theta=1e6)
        self.vocab, self.max_ctx, self.n_layers = vocab, max_ctx, layers
        m = synthetic.step_model(seed, hidden=hidden, n_heads=n_heads, n_kv=n_kv, inter=inter, vocab=vocab,
                                 group=group, layers=layers, bias=bias)
        self.m = m
        self.layers = []
        dev_layers = []
        entries = -(-max_ctx // page)  # logical pages covering max_ctx tokens
        self.num_pages = entries + 2
        self.table = synthetic.page_table(seed + 1, self.num_pages, entries)
        self.kc0, self.vc0 = [], []
        for l, L in enumerate(m["layers"]):
            lay = ostep.Layer(attn_norm=L["attn_norm"], qkv=ostep.Proj(*L["qkv"]), o=ostep.Proj(*L["o"]),
                              mlp_norm=L["mlp_norm"], gateup=ostep.Proj(*L["gateup"]), down=ostep.Proj(*L["down"]),
                              qkv_bias=None if L["qkv_bias"] is None else L["qkv_bias"].astype(np.float64))
            self.layers.append(lay)
            packed = {}
            for name, layout in (("qkv", "plain"), ("o", "plain"), ("gateup", "gateup"), ("down", "plain")):
                q, s = L[name]
                pw, ps = w4.pack(q, s, group, layout)
                packed[name] = (dev_u8(pw), dev_u8(ps))
            kc, vc = synthetic.kv_prefix(seed * 7 + l, self.num_pages, n_kv, page)
            self.kc0.append(kc)
            self.vc0.append(vc)
            shape = (self.num_pages, n_kv, page, 128)
            dev_layers.append(w4.StepLayer(
                attn_norm=dev_f16(L["attn_norm"]), qkv_w=packed["qkv"][0], qkv_s=packed["qkv"][1],
                o_w=packed["o"][0], o_s=packed["o"][1], mlp_norm=dev_f16(L["mlp_norm"]),
                gateup_w=packed["gateup"][0], gateup_s=packed["gateup"][1], down_w=packed["down"][0],
                down_s=packed["down"][1], k_cache=dev_f16(kc).view(shape), v_cache=dev_f16(vc).view(shape),
                qkv_bias=None if L["qkv_bias"] is None else torch.from_numpy(L["qkv_bias"]).cuda()))
        self.dev_layers = dev_layers
        pw, ps = w4.pack(*m["lm"], group, "plain")
        self.lm_w, self.lm_s = dev_u8(pw), dev_u8(ps)
        self.embed = dev_f16(m["embed"]).view(vocab, hidden)
        self.final_norm = dev_f16(m["final_norm"])
        self.page_table = torch.from_numpy(self.table).cuda()
        self.token = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.pos = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.logits = torch.full((vocab,), float("nan"), dtype=torch.float32, device="cuda")
        self.w_abs = None

    def step(self, use_graph, trace=True):
        w4 = _w4()
        c = self.cfg
        tr = None
        if trace:
            nbytes = w4.step_trace_bytes(hidden=c.hidden, n_heads=c.n_heads, n_kv_heads=c.n_kv, inter=c.inter,
                                         layers=self.n_layers)
            tr = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        return w4.DecodeStep(hidden=c.hidden, n_heads=c.n_heads, n_kv_heads=c.n_kv, inter=c.inter, vocab=self.vocab,
                             group=c.group, page_size=c.page, max_ctx=self.max_ctx, rms_eps=c.eps,
                             rope_theta=c.theta, embed=self.embed, layers=self.dev_layers,
                             final_norm=self.final_norm, lm_w=self.lm_w, lm_s=self.lm_s,
                             page_table=self.page_table, token=self.token, pos=self.pos, logits=self.logits,
                             trace=tr, use_graph=use_graph)

    def caches(self):
        return [(_host16(L.k_cache), _host16(L.v_cache)) for L in self.dev_layers]


def check_step(model: Model, st, token, pos, caches_before):
    """Teacher-forced check of one traced step that consumed (token, pos)."""
    c = model.cfg
    nh, nkv, H = c.n_heads, c.n_kv, c.hidden
    trace = st.read_trace()
    caches_after = model.caches()
    assert np.array_equal(trace[0]["h_in"].astype(np.float64), _half(model.m["embed"][token]))
    for l, L in enumerate(model.layers):
        t = trace[l]
        kc, vc = (a.copy() for a in caches_before[l])
        ka, va = caches_after[l]
        pg, sl = model.table[pos // c.page], pos % c.page
        forced = dict(x1=t["x1"], qkv=t["qkv"].astype(np.float64), q=t["q"].reshape(nh, 128),
                      k=ka[pg, :, sl], v=va[pg, :, sl], attn=t["attn"].reshape(nh, 128),
                      o=t["o"].astype(np.float64), h_mid=t["h_mid"].astype(np.float64), x2=t["x2"], m=t["m"],
                      d=t["d"].astype(np.float64))
        h_in = t["h_in"].astype(np.float64)
        r = ostep.decoder_layer(h_in, L, c, pos, kc, vc, model.table, forced=forced)
        tag = f"layer {l} pos {pos}"
        assert_within(_half(t["x1"]), r.x1, tol_rmsnorm(r.x1, H), tag + " x1")
        assert_within(t["qkv"], r.qkv, tol_plain(r.a_qkv), tag + " qkv")
        xb = (t["qkv"] + (L.qkv_bias.astype(np.float32) if L.qkv_bias is not None else np.float32(0)))
        xb = xb.astype(np.float64).reshape(nh + 2 * nkv, 128)
        assert_within(_half(t["q"]).reshape(nh, 128), r.q, tol_rope(r.q, xb[:nh]), tag + " q")
        assert_within(_half(ka[pg, :, sl]), r.k, tol_rope(r.k, xb[nh:nh + nkv]), tag + " k")
        assert_within(_half(va[pg, :, sl]), r.v, (2.0 ** -11 + U) * np.abs(r.v) + 2.0 ** -25, tag + " v")
        # the rest of each cache is untouched
        mask = np.zeros(ka.shape, bool)
        mask[pg, :, sl] = True
        assert np.array_equal(ka[~mask], caches_before[l][0][~mask]), tag + " k cache"
        assert np.array_equal(va[~mask], caches_before[l][1][~mask]), tag + " v cache"
        assert_within(_half(t["attn"]).reshape(nh, 128), r.attn, 2e-3 * r.a_attn + 1e-5, tag + " attn")
        assert_within(t["o"], r.o, tol_plain(r.a_o), tag + " o")
        assert np.array_equal(t["h_mid"], t["h_in"] + t["o"]), tag + " h_mid"
        assert_within(_half(t["x2"]), r.x2, tol_rmsnorm(r.x2, H), tag + " x2")
        I = c.inter
        tol_m = tol_gateup(r.gu[:I], r.a_gu[:I], r.gu[I:], r.a_gu[I:], r.m)
        assert_within(_half(t["m"]), r.m, tol_m, tag + " m")
        assert_within(t["d"], r.d, tol_plain(r.a_d), tag + " d")
        nxt = trace[l + 1]["h_in"]
        assert np.array_equal(nxt, t["h_mid"] + t["d"]), tag + " residual"
    fin = trace[model.n_layers]
    lm = ostep.Proj(*model.m["lm"])
    xf, y_ref, a_ref, _ = ostep.final_logits(fin["h_in"].astype(np.float64), model.m["final_norm"], lm, c,
                                             forced_xf=fin["x1"])
    assert_within(_half(fin["x1"]), xf, tol_rmsnorm(xf, H), "final norm")
    logits = model.logits.cpu().numpy()
    assert_within(logits, y_ref, tol_plain(a_ref), "logits")
    tok_out = int(model.token.item())
    assert tok_out == int(np.argmax(logits)), "token is the GPU logits' first argmax"
    assert tok_out in set(near_tie_set(y_ref, a_ref).tolist()), "token in the oracle's near-tie set"
    assert int(model.pos.item()) == pos + 1
    return tok_out


SMALL = dict(hidden=512, n_heads=4, n_kv=2, inter=1024, vocab=1000, group=64, layers=3, page=16, max_ctx=128)


@pytest.mark.parametrize("use_graph", [False, True], ids=["eager", "graph"])
def test_step_teacher_forced_small(use_graph):
    """Three layers, grouped KV heads, qkv bias; five consecutive steps from
    position 37 (page tails, a page boundary at 48 not reached, context
    growing), each checked stage by stage."""
    model = Model(21, bias=True, **SMALL)
    st = model.step(use_graph)
    # 7 kernels per layer (qkv with the attention norm folded in from layer 1
    # on, rotary + append + attention x2, o_proj, residual add + MLP norm,
    # gate/up, down with the residual add) + embedding with the first norm, the
    # last down's residual add + final norm, and lm_head (2: the GEMV, then
    # the argmax finalize, which also advances the position); the trace adds
    # 10 copies per layer and 2 for the first record
    assert st.launches() == 7 * 3 + 4 + 10 * 3 + 2
    model.token.fill_(5)
    model.pos.fill_(37)
    torch.cuda.synchronize()
    for i in range(5):
        token, pos = int(model.token.item()), int(model.pos.item())
        before = model.caches()
        st.run()
        torch.cuda.synchronize()
        check_step(model, st, token, pos, before)


def test_step_graph_equals_eager_and_untraced():
    """The captured graph and the eager launches give the same bits (logits,
    tokens, caches), traced or not, over several steps across a page boundary."""
    results = []
    for use_graph, trace in ((False, True), (True, True), (True, False)):
        model = Model(33, bias=False, **SMALL)
        st = model.step(use_graph, trace=trace)
        model.token.fill_(17)
        model.pos.fill_(44)
        toks, logits = [], []
        for _ in range(6):
            st.run()
            torch.cuda.synchronize()
            toks.append(int(model.token.item()))
            logits.append(model.logits.cpu().numpy().copy())
        results.append((toks, logits, model.caches()))
        st.close()
    for toks, logits, caches in results[1:]:
        assert toks == results[0][0]
        for a, b in zip(logits, results[0][1]):
            assert np.array_equal(a, b)
        for (k1, v1), (k0, v0) in zip(caches, results[0][2]):
            assert np.array_equal(k1, k0) and np.array_equal(v1, v0)


def test_step_first_position():
    """Position 0: one-token attention (the output is the new token's V)."""
    model = Model(45, bias=True, **SMALL)
    st = model.step(True)
    model.token.fill_(999)
    model.pos.fill_(0)
    torch.cuda.synchronize()
    before = model.caches()
    st.run()
    torch.cuda.synchronize()
    check_step(model, st, 999, 0, before)


@pytest.mark.parametrize("n_heads,n_kv,page,max_ctx,start", [
    (2, 2, 1, 40, 37),      # one query head per KV head, one token per page
    (8, 2, 64, 100, 97),    # the last chunk's reads past max_ctx are clamped onto the slot being appended
    (6, 3, 16, 70, 63),     # steps across a wave boundary inside the chunk (63 -> 64)
    (4, 1, 8, 129, 126),    # four query heads on one KV head; steps across the chunk boundary (127 -> 128)
                            # into a last chunk of one token, ending at max_ctx - 1 = 128
])
def test_step_fused_attention_edges(n_heads, n_kv, page, max_ctx, start):
    """The rotary + KV append fused into attention at the cache's edges:
    every step teacher-forced, up to the last position of the cache."""
    cfg = dict(hidden=256, n_heads=n_heads, n_kv=n_kv, inter=512, vocab=300, group=64, layers=2, page=page,
               max_ctx=max_ctx)
    model = Model(60 + n_heads + page, bias=True, **cfg)
    st = model.step(True)
    model.token.fill_(3)
    model.pos.fill_(start)
    torch.cuda.synchronize()
    for _ in range(max_ctx - start):
        token, pos = int(model.token.item()), int(model.pos.item())
        before = model.caches()
        st.run()
        torch.cuda.synchronize()
        check_step(model, st, token, pos, before)


def test_step_separate_norms_above_4096():
    """Hidden 4224 (33 heads over 11 KV heads): the partial sums of squares
    would exceed the norm prologue's 1024, so the step runs a separate residual
    + RMSNorm kernel before every qkv (8 kernels per layer); teacher-forced
    like the rest."""
    cfg = dict(hidden=4224, n_heads=33, n_kv=11, inter=256, vocab=500, group=64, layers=2, page=16, max_ctx=64)
    model = Model(88, bias=True, **cfg)
    st = model.step(True)
    assert st.launches() == 8 * 2 + 3 + 10 * 2 + 2
    model.token.fill_(7)
    model.pos.fill_(30)
    torch.cuda.synchronize()
    for _ in range(2):
        token, pos = int(model.token.item()), int(model.pos.item())
        before = model.caches()
        st.run()
        torch.cuda.synchronize()
        check_step(model, st, token, pos, before)


@pytest.mark.slow
def test_step_teacher_forced_full_width():
    """The model's real widths (hidden 3584, 28 query / 4 KV heads, MLP 18944,
    vocabulary 152064, G = 128), two layers, pages of 16 and a 4096-token
    context, at a position deep in the context."""
    model = Model(7, hidden=synthetic.HIDDEN, n_heads=synthetic.HEADS, n_kv=synthetic.KV_HEADS,
                  inter=synthetic.MLP, vocab=synthetic.VOCAB, group=synthetic.GROUP, layers=2,
                  page=synthetic.PAGE, max_ctx=synthetic.MAX_CTX, bias=True)
    st = model.step(True)
    model.token.fill_(151000)
    model.pos.fill_(3000)
    torch.cuda.synchronize()
    for _ in range(2):
        token, pos = int(model.token.item()), int(model.pos.item())
        before = model.caches()
        st.run()
        torch.cuda.synchronize()
        check_step(model, st, token, pos, before)
