"""Benchmark: the per-token INT4 linear sweep of a 28-layer decode step.

One step = one replay of the captured HIP graph that runs, in decode order,
28 x (QKV 3584->4608, o_proj 3584->3584, gate/up 3584->2x18944 + SiLU,
down 18944->3584) and lm_head 3584->152064 + argmax: 113 GEMVs over
3,650,274,304 algorithmic bytes (packed nibbles + fp16 scales + fp16 x +
outputs), all resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5]

prints one JSON line: achieved GB/s over the whole sweep (value), ms per
sweep, the eager-launch sweep for comparison, the dominant kernel's roofline
(gate/up + SiLU, timed per launch with HIP events on the launch stream) and
the CPU oracle timed on a bounded sample on the host.

    python bench.py --workload attention

times 28 layers' decode attention over a paged fp16 KV cache at a
4096-token context (GB/s against the HBM peak).

    python bench.py --workload prefill [--steps 10] [--warmup 2]

times the prefill counterpart instead: the 28 layers' four INT4 products for
a 512-token prompt (112 GEMMs on the matrix cores) plus lm_head on the last
token, captured in one HIP graph; value is TFLOP/s over the sweep, the
roofline is the gate/up GEMM's against the fp16 matrix-core peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synthetic  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix-core peak
METRIC = "achieved HBM GB/s (% of peak) and ms per 28-layer+lm_head INT4 linear sweep"
PREFILL_METRIC = "prefill TFLOP/s (% of fp16 MFMA peak) and ms per 28-layer 512-token INT4 linear sweep"
ATTN_METRIC = "decode attention GB/s (% of HBM peak) and ms per 28-layer paged-KV attention at 4096-token context"
ATTN_HEADS, ATTN_KV_HEADS, ATTN_PAGE, ATTN_CTX = 28, 4, 16, 4096
KERNEL_SRC = os.path.join(ROOT, "int4_weight_only_04_amd", "csrc", "w4_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gateup_silu_37888x3584.json")
GEMM_SRC = os.path.join(ROOT, "int4_weight_only_04_amd", "csrc", "w4_gemm.hip")
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_gateup_512x37888x3584.json")


def algorithmic_bytes(kind: str, n: int, k: int, group: int) -> int:
    """Bytes a GEMV must move at least once: nibbles, scales, x, outputs."""
    b = n * k // 2 + 2 * n * (k // group) + 2 * k
    if kind == "gateup":
        b += 2 * (n // 2)
    else:
        b += 4 * n
    if kind == "lmhead":
        b += 4
    return b


def sweep_bytes(projs) -> int:
    return sum(algorithmic_bytes(p.kind, p.n, p.k, p.group) for p in projs)


def build_sweep(layers: int = synthetic.LAYERS, device: str = "cuda"):
    """Device buffers of the sweep: each projection's inputs are drawn already
    packed (uniform random bytes = i.i.d. uniform nibbles; all row counts are
    multiples of 4, so there are no padding slots) from its own seed."""
    import torch
    from int4_weight_only_04_amd import w4

    specs = synthetic.sweep_projections(layers)
    projs = []
    for p in specs:
        layout = "gateup" if p.kind == "gateup" else "plain"
        wb, sb = w4.packed_size(p.n, p.k, p.group, layout)
        pw, ps, x = synthetic.packed_random(p.seed, wb, sb // 2, p.k)
        dpw = torch.from_numpy(pw).to(device)
        dps = torch.from_numpy(ps).to(device)
        dx = torch.from_numpy(x.view(np.int16)).to(device).view(torch.float16)
        if p.kind == "gateup":
            out = torch.empty(p.n // 2, dtype=torch.float16, device=device)
            projs.append(w4.Proj(w4.PROJ_GATEUP_SILU, p.n, p.k, p.group, dpw, dps, dx, out))
        elif p.kind == "lmhead":
            out = torch.empty(p.n, dtype=torch.float32, device=device)
            am = torch.full((1,), -1, dtype=torch.int32, device=device)
            ws = torch.zeros(w4.gemv_workspace_size(p.n, p.k, p.group, True), dtype=torch.uint8,
                             device=device)
            projs.append(w4.Proj(w4.PROJ_LMHEAD_ARGMAX, p.n, p.k, p.group, dpw, dps, dx, out, am, ws))
        else:
            out = torch.empty(p.n, dtype=torch.float32, device=device)
            projs.append(w4.Proj(w4.PROJ_PLAIN, p.n, p.k, p.group, dpw, dps, dx, out))
    return specs, projs


def kernel_source_hash(path: str = KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(launch_bytes_alg: int = 0, path: str = TRAFFIC_FILE, src: str = KERNEL_SRC):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if absent or taken on another kernel source."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    return t.get("hbm_bytes_per_launch")


def time_graph(sweep, stream, steps: int, warmup: int):
    import torch
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            sweep.run(stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        sweep.run(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = start.elapsed_time(end) / steps
    return ev_ms, wall * 1e3 / steps


def time_dominant_kernel(projs, stream, replays: int = 4):
    """Average duration of one gate/up + SiLU launch (the kernel that moves the
    most bytes in the sweep): the 28 layers' gate/up launches are captured in
    their own HIP graph (1.96 GB of weights, so nothing is served from the
    256 MB Infinity Cache), replayed once to warm up, then `replays` times
    between HIP events recorded on the launch stream.  The per-launch figure
    includes the time between graph nodes (about 1.4 us from the last wave of
    one kernel to the first wave of the next).  The loop is kept short: after
    a few milliseconds of back-to-back gate/up launches (about 5 TB/s
    sustained) the kernel was seen to slow down in steps, which the sweep, at
    a lower average bandwidth, does not show."""
    import torch
    from int4_weight_only_04_amd import w4
    gu = [p for p in projs if p.kind == w4.PROJ_GATEUP_SILU]
    g = w4.Sweep(gu, use_graph=True)
    g.run(stream)
    stream.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.run(stream)
    b.record(stream)
    stream.synchronize()
    g.close()
    launches = replays * len(gu)
    return a.elapsed_time(b) / launches, launches


def cpu_baseline():
    """The oracle as it stands (single thread, fp64) on a bounded sample: all
    rows of layer 0's four projections, inputs drawn exactly as in the sweep."""
    import oracle
    from int4_weight_only_04_amd import w4
    specs = synthetic.sweep_projections(1)
    total_bytes = 0
    t_total = 0.0
    for p in specs:
        layout = "gateup" if p.kind == "gateup" else "plain"
        wb, sb = w4.packed_size(p.n, p.k, p.group, layout)
        pw, ps, x = synthetic.packed_random(p.seed, wb, sb // 2, p.k)
        t0 = time.perf_counter()
        y, _ = oracle.gemv_packed(pw, ps, x, p.n, p.k, p.group, gateup=(layout == "gateup"))
        if p.kind == "gateup":
            oracle.silu_gate(y)
        t_total += time.perf_counter() - t0
        total_bytes += algorithmic_bytes(p.kind, p.n, p.k, p.group)
    return {
        "value": total_bytes / t_total / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "layer 0 of the sweep (qkv, o_proj, gate/up+silu, down), all rows, "
                  f"{total_bytes} algorithmic bytes in {t_total:.1f} s, single-threaded fp64 C",
        "seconds": t_total,
    }


def build_prefill(layers: int, device: str = "cuda"):
    """Device buffers of the prefill sweep: packed weights drawn like the decode
    sweep's, one seeded 512-row token block per projection, and lm_head as
    the decode GEMV (with argmax) on one token."""
    import torch
    from int4_weight_only_04_amd import w4

    m = synthetic.PROMPT
    items = []
    for p in synthetic.prefill_projections(layers):
        layout = "gateup" if p.kind == "gateup" else "plain"
        wb, sb = w4.packed_size(p.n, p.k, p.group, layout)
        pw, ps, _ = synthetic.packed_random(p.seed, wb, sb // 2, p.k)
        xm = synthetic.prompt_acts(p.seed + 5, m, p.k)
        dx = torch.from_numpy(xm.view(np.int16)).to(device).view(torch.float16)
        cols = p.n // 2 if p.kind == "gateup" else p.n
        out = torch.empty((m, cols), dtype=torch.float16 if p.kind == "gateup" else torch.float32,
                          device=device)
        items.append((p, torch.from_numpy(pw).to(device), torch.from_numpy(ps).to(device), dx, out))
    # one split-k workspace serves every product: they run one after another
    ws_bytes = max([w4.gemm_workspace_size(m, p.n, p.k, p.group) for (p, *_r) in items if p.kind != "gateup"]
                   + [16])
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    lm = synthetic.sweep_projections(0)[-1]
    wb, sb = w4.packed_size(lm.n, lm.k, lm.group, "plain")
    pw, ps, x = synthetic.packed_random(lm.seed, wb, sb // 2, lm.k)
    lm_buf = (lm, torch.from_numpy(pw).to(device), torch.from_numpy(ps).to(device),
              torch.from_numpy(x.view(np.int16)).to(device).view(torch.float16),
              torch.empty(lm.n, dtype=torch.float32, device=device),
              torch.full((1,), -1, dtype=torch.int32, device=device),
              torch.zeros(w4.gemv_workspace_size(lm.n, lm.k, lm.group, True), dtype=torch.uint8,
                          device=device))
    return items, lm_buf, workspace


def prefill_flops(items, lm_buf) -> int:
    m = synthetic.PROMPT
    return sum(2 * m * p.n * p.k for (p, *_rest) in items) + 2 * lm_buf[0].n * lm_buf[0].k


def launch_prefill(items, lm_buf, workspace, stream, only_gateup: bool = False):
    from int4_weight_only_04_amd import w4
    m = synthetic.PROMPT
    for p, pw, ps, x, out in items:
        if p.kind == "gateup":
            w4.gemm_gateup_silu(pw, ps, x, out, m, p.n, p.k, p.group, stream=stream)
        elif not only_gateup:
            w4.gemm(pw, ps, x, out, m, p.n, p.k, p.group, workspace=workspace, stream=stream)
    if not only_gateup:
        lm, pw, ps, x, y, am, ws = lm_buf
        w4.gemv(pw, ps, x, y, lm.n, lm.k, lm.group, argmax=am, workspace=ws, stream=stream)


def capture(fn, stream):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn(torch.cuda.current_stream())
    return g


def replay_ms(g, stream, steps: int, warmup: int) -> float:
    import torch
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        a.record(stream)
        for _ in range(steps):
            g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def prefill_cpu_baseline(tokens: int = 4):
    """The oracle's prefill product (single thread, fp64) on a bounded sample:
    layer 0's four projections, all weight rows, for the first `tokens` rows
    of their token blocks."""
    import oracle
    from int4_weight_only_04_amd import w4
    flops = 0
    t_total = 0.0
    for p in synthetic.prefill_projections(1):
        layout = "gateup" if p.kind == "gateup" else "plain"
        wb, sb = w4.packed_size(p.n, p.k, p.group, layout)
        pw, ps, _ = synthetic.packed_random(p.seed, wb, sb // 2, p.k)
        xm = synthetic.prompt_acts(p.seed + 5, tokens, p.k)
        t0 = time.perf_counter()
        y, _ = oracle.gemm_packed(pw, ps, xm, p.n, p.k, p.group, gateup=(layout == "gateup"))
        if p.kind == "gateup":
            for row in y:
                oracle.silu_gate(row)
        t_total += time.perf_counter() - t0
        flops += 2 * tokens * p.n * p.k
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"layer 0 of the prefill sweep (qkv, o_proj, gate/up+silu, down), all rows, first "
                  f"{tokens} prompt tokens: {flops} flops in {t_total:.1f} s, single-threaded fp64 C",
        "seconds": t_total,
    }


def run_prefill(args) -> int:
    import torch
    print(f"[bench] building prefill sweep ({args.layers} layers, {synthetic.PROMPT} tokens)",
          file=sys.stderr, flush=True)
    items, lm_buf, workspace = build_prefill(args.layers)
    flops = prefill_flops(items, lm_buf)
    stream = torch.cuda.Stream()
    print("[bench] prefill graph", file=sys.stderr, flush=True)
    g = capture(lambda s: launch_prefill(items, lm_buf, workspace, s), stream)
    ms = replay_ms(g, stream, args.steps, args.warmup)
    print("[bench] dominant kernel (gate/up GEMM)", file=sys.stderr, flush=True)
    gg = capture(lambda s: launch_prefill(items, lm_buf, workspace, s, only_gateup=True), stream)
    n_gu = sum(1 for it in items if it[0].kind == "gateup")
    reps = 3
    gu_ms = replay_ms(gg, stream, reps, 1) / n_gu
    gp = next(it[0] for it in items if it[0].kind == "gateup")
    gu_flops = 2 * synthetic.PROMPT * gp.n * gp.k
    gu_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    value = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": (f"512-token prefill INT4 linear sweep, hipGraph: {args.layers} x (qkv 3584->4608, "
                         "o_proj 3584->3584, gate/up 3584->2x18944 + silu, down 18944->3584) as GEMMs on "
                         "512 token rows + lm_head 3584->152064 + argmax on the last token; int4 zero point "
                         "8, fp16 scales per 128 inputs dequantized to fp16, fp16 activations, fp32 "
                         "accumulation"),
            "prompt_tokens": synthetic.PROMPT,
            "gemms_per_step": len(items),
            "flops_per_step": flops,
            "pct_of_mfma_f16_peak": round(100.0 * value / MFMA_F16_PEAK_TFLOPS, 2),
        },
        "roofline": {
            "kernel": "gemm_w4_kernel<gate/up+silu> 512x37888x3584 g128",
            "bound": "mfma",
            "achieved": round(gu_tflops, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gu_tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": read_traffic(path=GEMM_TRAFFIC_FILE, src=GEMM_SRC),
            "algorithmic_flops_per_launch": gu_flops,
            "algorithmic_bytes_per_launch": (gp.n * gp.k // 2 + 2 * gp.n * (gp.k // gp.group)
                                             + 2 * synthetic.PROMPT * gp.k + synthetic.PROMPT * gp.n),
            "avg_launch_us": round(gu_ms * 1e3, 3),
            "launches_timed": reps * n_gu,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle prefill product)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = prefill_cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


def attn_bytes(ctx: int) -> int:
    """K and V rows of the context, q, the output and the page table."""
    return 2 * ctx * ATTN_KV_HEADS * 128 * 2 + 2 * ATTN_HEADS * 128 * 2 + 4 * (-(-ctx // ATTN_PAGE))


def attn_cpu_baseline(layers: int = 12):
    """The oracle's attention (single thread, fp64) on `layers` layers' caches
    at the full context."""
    import oracle
    rng = np.random.default_rng(4000)
    npages = ATTN_CTX // ATTN_PAGE
    total = 0.0
    for _ in range(layers):
        q = rng.standard_normal((ATTN_HEADS, 128)).astype(np.float16).view(np.uint16)
        kc = rng.standard_normal((npages, ATTN_KV_HEADS, ATTN_PAGE, 128)).astype(np.float16).view(np.uint16)
        vc = rng.standard_normal((npages, ATTN_KV_HEADS, ATTN_PAGE, 128)).astype(np.float16).view(np.uint16)
        table = rng.permutation(npages).astype(np.int32)
        t0 = time.perf_counter()
        oracle.attn_decode(q, kc, vc, table, ATTN_CTX, ATTN_KV_HEADS, ATTN_PAGE, 1.0 / np.sqrt(128.0))
        total += time.perf_counter() - t0
    nbytes = layers * attn_bytes(ATTN_CTX)
    return {
        "value": nbytes / total / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{layers} layers' attention at context {ATTN_CTX} (28 query heads, 4 KV heads, pages of "
                  f"{ATTN_PAGE}): {nbytes} algorithmic bytes in {total:.1f} s, single-threaded fp64 C",
        "seconds": total,
    }


def run_attention(args) -> int:
    """28 layers' decode attention at a 4096-token context: two sets of 28
    caches (470 MB, beyond the 256 MB Infinity Cache) alternate, each layer
    with its own seeded cache and a permuted page table, in one HIP graph."""
    import torch
    from int4_weight_only_04_amd import w4
    layers = args.layers
    npages = ATTN_CTX // ATTN_PAGE
    dev = "cuda"
    g = torch.Generator(device="cpu").manual_seed(4001)
    calls = []
    for i in range(2 * layers):
        kc = torch.randn((npages, ATTN_KV_HEADS, ATTN_PAGE, 128), generator=g).to(torch.float16).to(dev)
        vc = torch.randn((npages, ATTN_KV_HEADS, ATTN_PAGE, 128), generator=g).to(torch.float16).to(dev)
        q = torch.randn((ATTN_HEADS, 128), generator=g).to(torch.float16).to(dev)
        table = torch.randperm(npages, generator=g).to(torch.int32).to(dev)
        out = torch.empty((ATTN_HEADS, 128), dtype=torch.float16, device=dev)
        calls.append((q, kc, vc, table, out))
    ctx = torch.full((1,), ATTN_CTX, dtype=torch.int32, device=dev)
    ws = torch.empty(w4.attn_decode_workspace_size(ATTN_HEADS, ATTN_CTX), dtype=torch.uint8, device=dev)
    scale = 1.0 / float(np.sqrt(128.0))

    def launch(s, subset=None):
        for (q, kc, vc, table, out) in (calls if subset is None else subset):
            w4.attn_decode(q, kc, vc, table, ctx, ATTN_CTX, out, ATTN_KV_HEADS, ATTN_PAGE, scale, ws, stream=s)

    stream = torch.cuda.Stream()
    print(f"[bench] attention graph ({2 * layers} calls over two cache sets)", file=sys.stderr, flush=True)
    graph = capture(lambda s: launch(s), stream)
    per_call_ms = replay_ms(graph, stream, args.steps, args.warmup) / (2 * layers)
    ms = per_call_ms * layers
    nbytes = attn_bytes(ATTN_CTX)
    gbs = nbytes / (per_call_ms * 1e-3) / 1e9
    out = {
        "metric": ATTN_METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"batch-1 decode attention, hipGraph: {layers} layers x softmax(q K^T / sqrt(128)) V over "
                         f"a paged fp16 KV cache, context {ATTN_CTX}, pages of {ATTN_PAGE} tokens, {ATTN_HEADS} query "
                         f"heads over {ATTN_KV_HEADS} KV heads of 128, fp32 arithmetic, fp16 output"),
            "algorithmic_bytes_per_layer": nbytes,
            "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        },
        "roofline": {
            "kernel": "attn_partial_kernel<7> + attn_combine_kernel, 4096 tokens",
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": nbytes,
            "avg_launch_us": round(per_call_ms * 1e3, 3),
            "launches_timed": args.steps * 2 * layers,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle attention)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = attn_cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=synthetic.LAYERS)
    ap.add_argument("--eager-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=("decode", "prefill", "attention"), default="decode",
                    help="decode: the per-token GEMV sweep (default); prefill: the 512-token GEMM sweep; "
                         "attention: 28 layers' paged-KV decode attention at a 4096-token context")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the INT4 decode GEMV sweep is a single-GPU path here; "
              "run it with --gpus 1", file=sys.stderr)
        return 2

    import torch
    from int4_weight_only_04_amd import w4
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    w4.lib()

    if args.copy_probe:
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3}), flush=True)
        return 0

    if args.workload == "prefill":
        return run_prefill(args)
    if args.workload == "attention":
        return run_attention(args)

    print(f"[bench] building sweep ({args.layers} layers)", file=sys.stderr, flush=True)
    specs, projs = build_sweep(args.layers)
    alg_bytes = sweep_bytes(specs)
    stream = torch.cuda.Stream()

    print("[bench] graph sweep", file=sys.stderr, flush=True)
    graph = w4.Sweep(projs, use_graph=True)
    ev_ms, wall_ms = time_graph(graph, stream, args.steps, args.warmup)

    print("[bench] eager sweep", file=sys.stderr, flush=True)
    eager = w4.Sweep(projs, use_graph=False)
    eager_ms, eager_wall_ms = time_graph(eager, stream, args.eager_steps, 2)
    eager.close()

    print("[bench] dominant kernel", file=sys.stderr, flush=True)
    gu_mean_ms, gu_launches = time_dominant_kernel(projs, stream)
    gp = next(p for p in specs if p.kind == "gateup")
    gu_bytes = algorithmic_bytes("gateup", gp.n, gp.k, gp.group)
    gu_gbs = gu_bytes / (gu_mean_ms * 1e-3) / 1e9
    graph.close()

    value = alg_bytes / (ev_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ev_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"batch-1 decode-step INT4 linear sweep, hipGraph: {args.layers} x (qkv 3584->4608, "
                         "o_proj 3584->3584, gate/up 3584->2x18944 + silu, down 18944->3584) + lm_head "
                         "3584->152064 + argmax; int4 zero point 8, fp16 scales per 128 inputs, fp16 x, "
                         "fp32 accumulation"),
            "gemvs_per_step": len(specs),
            "algorithmic_bytes_per_step": alg_bytes,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "wall_ms_per_step": round(wall_ms, 4),
            "eager_ms_per_step": round(eager_ms, 4),
            "graph_speedup_vs_eager": round(eager_ms / ev_ms, 3),
        },
        "roofline": {
            "kernel": "gemv_w4_kernel<2, gate/up+silu> 37888x3584 g128",
            "bound": "hbm",
            "achieved": round(gu_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(gu_bytes),
            "algorithmic_bytes_per_launch": gu_bytes,
            "avg_launch_us": round(gu_mean_ms * 1e3, 3),
            "launches_timed": gu_launches,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
