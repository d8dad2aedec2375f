"""Benchmark: the per-token INT4 linear sweep of a 28-layer decode step.

One step = one replay of the captured HIP graph that runs, in decode order,
28 x (QKV 3584->4608, o_proj 3584->3584, gate/up 3584->2x18944 + SiLU,
down 18944->3584) and lm_head 3584->152064 + argmax: 113 GEMVs over
3,650,274,304 algorithmic bytes (packed nibbles + fp16 scales + fp16 x +
outputs), all resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5]

prints one JSON line: achieved GB/s over the whole sweep (value) and ms per
sweep; the graph and the library's eager launches timed in alternating rounds
(and a Python-driven eager loop); each config's GEMV (tiny, down, gate/up +
SiLU, lm_head + argmax) on cold buffers, with its counter-calibrated HBM
bytes when they were taken on this kernel source; the dominant kernel's
roofline (gate/up + SiLU, timed per launch with HIP events on the launch
stream) with the GPU clocks sampled around it and a sustained series; the
pages' H100 figures as context; and the CPU oracle timed on the host's cores,
single-threaded and on all available cores.

    python bench.py --workload configs
    python bench.py --traffic-from FETCH.csv WRITE.csv COPYF.csv COPYW.csv

run only the per-config timings (the run the FETCH_SIZE / WRITE_SIZE
counters are taken over), and turn those counters into
profiles/traffic_configs.json (host only).

    python bench.py --workload attention

times 28 layers' decode attention over a paged fp16 KV cache at a
4096-token context (GB/s against the HBM peak).

    python bench.py --workload step [--steps 128] [--warmup 5]

times the full batch-1 decode step (embedding, 28 pre-norm decoder layers
with RMSNorm, the INT4 projections, RoPE + paged KV append and attention,
final norm, lm_head + greedy argmax, position advance) as one captured HIP
graph per token, for tokens 512..512+steps-1 after a 512-token prompt (the
pages' pp512/tg128 protocol), and the same step as eager launches.

    python bench.py --workload w4a8

times the W4A8 variant of the linear sweep (int8 activations, integer
dot products): each projection's fp16 x is quantized per group of 128 and the
GEMV reads the codes; reported next to the W4A16 sweep of the same weights,
with and without the quantization launches.

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
W4A8_METRIC = "W4A8 achieved HBM GB/s (% of peak) and ms per 28-layer+lm_head INT4 linear sweep with int8 activations"
STEP_METRIC = "batch-1 decode tokens/s and ms per full 28-layer decode step (hipGraph), tokens 512..639"
ATTN_HEADS, ATTN_KV_HEADS, ATTN_PAGE, ATTN_CTX = 28, 4, 16, 4096
KERNEL_SRC = os.path.join(ROOT, "int4_weight_only_04_amd", "csrc", "w4_kernels.hip")
# every file the decode GEMV kernels are compiled from (the GEMV's math and its
# launch table, and lm_head's argmax finalize, whose bytes the lm_head config counts)
GEMV_SRCS = tuple(os.path.join(ROOT, "int4_weight_only_04_amd", "csrc", f)
                  for f in ("w4_kernels.hip", "w4_argmax.hip", "w4_gemv_math.h", "w4_internal.h"))
CONFIG_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_configs.json")
COLD_BYTES = 576 << 20      # per-config working set: past the 256 MB Infinity Cache
# The pages' own figures (H100, whole decode step, INT4 weights, batch 1): context, not targets.
PAGES_CONTEXT_H100 = {"runtime_ms_per_token": 16.7, "eager_ms_per_token": 119, "graph_ms_per_token": 17,
                      "llama_cpp_q4km_ms_per_token": 4.95,
                      "note": "whole decode step on an NVIDIA H100 as the pages report it; not this path's "
                              "metric and not a target"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gateup_silu_37888x3584.json")
GEMM_SRC = os.path.join(ROOT, "int4_weight_only_04_amd", "csrc", "w4_gemm.hip")
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_gateup_512x37888x3584.json")
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_4096.json")
ATTN_SRC = os.path.join(ROOT, "int4_weight_only_04_amd", "csrc", "w4_attn.hip")
A8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gateup_silu_a8_37888x3584.json")


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


def kernel_source_hash(path=KERNEL_SRC) -> str:
    """sha256 prefix of a kernel's source file, or of several concatenated."""
    h = hashlib.sha256()
    for f in ((path,) if isinstance(path, str) else path):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(launch_bytes_alg: int = 0, path: str = TRAFFIC_FILE, src=GEMV_SRCS):
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


def time_dominant_kernel(projs, stream, replays: int = 4, sustained: int = 200):
    """Average duration of one gate/up + SiLU launch (the kernel that moves the
    most bytes in the sweep): the 28 layers' gate/up launches are captured in
    their own HIP graph (1.96 GB of weights, so nothing is served from the
    256 MB Infinity Cache), replayed once to warm up, then `replays` times
    between HIP events recorded on the launch stream.  The per-launch figure
    includes the time between graph nodes (about 1.4 us from the last wave of
    one kernel to the first wave of the next).

    Then `sustained` more replays back to back (about 80 ms), each between its
    own events, with the GPU's clocks, power and throttle status sampled
    throughout (the metrics refresh more slowly than a few milliseconds, so
    the series is long enough to span several refreshes): it shows whether a
    longer run at this bandwidth slows down, and why.
    Returns (ms per launch in the short window, launches, sustained summary)."""
    import torch
    from int4_weight_only_04_amd import w4
    gu = [p for p in projs if p.kind == w4.PROJ_GATEUP_SILU]
    g = w4.Sweep(gu, use_graph=True)
    g.run(stream)
    stream.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    with ClockSampler() as short_clk:
        a.record(stream)
        for _ in range(replays):
            g.run(stream)
        b.record(stream)
        stream.synchronize()
    launches = replays * len(gu)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(sustained + 1)]
    with ClockSampler() as long_clk:
        ev[0].record(stream)
        for i in range(sustained):
            g.run(stream)
            ev[i + 1].record(stream)
        stream.synchronize()
    g.close()
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 / len(gu) for i in range(sustained)]
    q = max(1, sustained // 8)
    sus = {"replays": sustained, "launches": sustained * len(gu),
           "us_per_launch_first": round(sum(per[:q]) / q, 3),
           "us_per_launch_last": round(sum(per[-q:]) / q, 3),
           "us_per_launch_min": round(min(per), 3), "us_per_launch_max": round(max(per), 3),
           "ms_total": round(ev[0].elapsed_time(ev[-1]), 3),
           "clocks": long_clk.summary()}
    return a.elapsed_time(b) / launches, launches, sus, short_clk.summary()


def time_pure_read_sweep(specs, stream, steps: int, warmup: int):
    """The ceiling of a sweep built from one kernel per projection: a graph of
    113 launches of the library's read-only probe kernel (the GEMVs' 16-byte
    non-temporal loads and nothing else), each over exactly the packed weight +
    scale bytes of one projection, in sweep order, from one buffer.  Also one
    1 GiB read, the streaming ceiling of the loads themselves."""
    import torch
    from int4_weight_only_04_amd import w4
    sizes = []
    for p in specs:
        layout = "gateup" if p.kind == "gateup" else "plain"
        wb, sb = w4.packed_size(p.n, p.k, p.group, layout)
        sizes.append((wb + sb + 255) // 256 * 256)
    total = sum(sizes)
    buf = torch.empty(max(total, 1 << 30), dtype=torch.uint8, device="cuda")
    buf[: 1 << 20].fill_(1)
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)

    def launch(s):
        for off, nb in zip(offs, sizes):
            w4.read_probe(buf[int(off):], nb, sink, stream=s)

    g = capture(launch, stream)
    ms = replay_ms(g, stream, steps, warmup)
    big = capture(lambda s: w4.read_probe(buf, 1 << 30, sink, stream=s), stream)
    big_ms = replay_ms(big, stream, 10, 2)
    del g, big
    return ms, total, (1 << 30) / (big_ms * 1e-3) / 1e9


CONFIGS = (synthetic.CONFIG_TINY, synthetic.CONFIG_DOWN, synthetic.CONFIG_GATEUP, synthetic.CONFIG_LMHEAD)


def config_label(c) -> str:
    extra = {"gateup": " + silu", "lmhead": " + argmax"}.get(c["kind"], "")
    return f'{c["name"]} {c["n"]}x{c["k"]} g{c["group"]}{extra}'


def config_inputs(c):
    """A config's packed inputs, drawn in packed form from its seed (row counts
    are multiples of 4, so no padding slots), with its scale range."""
    from int4_weight_only_04_amd import w4
    layout = "gateup" if c["kind"] == "gateup" else "plain"
    wb, sb = w4.packed_size(c["n"], c["k"], c["group"], layout)
    pw, ps, x = synthetic.packed_random(c["seed"], wb, sb // 2, c["k"], c["s_lo"], c["s_hi"])
    return layout, wb, sb, pw, ps, x


def time_configs(stream, replays: int = 5, max_calls=None):
    """Per config (tiny, down, gate/up + SiLU, lm_head + argmax): microseconds
    per GEMV call on cold buffers.  The packed matrix is replicated on the
    device until the copies span COLD_BYTES (more than the 256 MB Infinity
    Cache), a HIP graph of max(copies, 32) back-to-back calls cycles through
    them, and the graph is replayed `replays` times after one warm-up; the
    figure is the replay time over the calls, so it includes the gap between
    consecutive kernels (and, for lm_head, the argmax finalize launch).
    `max_calls` caps the calls per graph (the counter runs, where every
    dispatch is serialized): the copies used are then the first ones written,
    which the later copies have pushed out of the caches."""
    import torch
    from int4_weight_only_04_amd import w4
    traffic = read_config_traffic()
    out = []
    for c in CONFIGS:
        layout, wb, sb, pw, ps, x = config_inputs(c)
        n, k, g = c["n"], c["k"], c["group"]
        wpad, spad = (wb + 4095) // 4096 * 4096, (sb + 255) // 256 * 256
        copies = max(2, -(-COLD_BYTES // (wpad + spad)))
        big_w = torch.empty((copies, wpad), dtype=torch.uint8, device="cuda")
        big_s = torch.empty((copies, spad), dtype=torch.uint8, device="cuda")
        big_w[0, :wb].copy_(torch.from_numpy(pw))
        big_s[0, :sb].copy_(torch.from_numpy(ps))
        big_w[1:] = big_w[0]
        big_s[1:] = big_s[0]
        dx = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
        if c["kind"] == "gateup":
            y = torch.empty(n // 2, dtype=torch.float16, device="cuda")
        else:
            y = torch.empty(n, dtype=torch.float32, device="cuda")
        am = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        ws = torch.zeros(w4.gemv_workspace_size(n, k, g, True), dtype=torch.uint8, device="cuda")
        calls = max(copies, 32) if max_calls is None else min(max(copies, 32), max_calls)
        print(f"[configs] {config_label(c)}: {copies} copies, {calls} calls x {replays} replays",
              file=sys.stderr, flush=True)

        def launch(st, c=c):
            for i in range(calls):
                cw, cs = big_w[i % copies], big_s[i % copies]
                if c["kind"] == "gateup":
                    w4.gemv_gateup_silu(cw, cs, dx, y, n, k, g, stream=st)
                elif c["kind"] == "lmhead":
                    w4.gemv(cw, cs, dx, y, n, k, g, argmax=am, workspace=ws, stream=st)
                else:
                    w4.gemv(cw, cs, dx, y, n, k, g, stream=st)

        graph = capture(launch, stream)
        ms = replay_ms(graph, stream, replays, 1)
        del graph
        us = ms * 1e3 / calls
        alg = algorithmic_bytes(c["kind"], n, k, g)
        gbs = alg / (us * 1e-6) / 1e9
        t = traffic.get(c["name"]) if traffic else None
        hbm = t["hbm_bytes_per_launch"] if t else None
        out.append({
            "config": config_label(c),
            "us_per_gemv": round(us, 3),
            "algorithmic_bytes": alg,
            "gbs": round(gbs, 1),
            "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
            "floor_us_at_8tbs": round(alg / (HBM_PEAK_GBS * 1e9) * 1e6, 3),
            "hbm_bytes_per_launch_fetch_write": hbm,
            "fetch_gbs": round(hbm / (us * 1e-6) / 1e9, 1) if hbm else None,
            "calls_timed": calls * replays,
            "cold_copies": copies,
            "cold_working_set_bytes": copies * (wb + sb),
        })
        del big_w, big_s
        torch.cuda.synchronize()
    return out


def read_config_traffic(path: str = CONFIG_TRAFFIC_FILE):
    """Per-config HBM bytes per call from the committed counter summary, or
    None if absent or taken on another kernel source."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash(GEMV_SRCS):
        return None
    return t.get("configs")


def write_traffic(fetch_csv: str, write_csv: str, copyf_csv: str, copyw_csv: str) -> int:
    """Turn four `rocprofv3 --pmc` CSVs (FETCH_SIZE and WRITE_SIZE over
    `bench.py --workload configs`, then over `bench.py --copy-probe`) into the
    per-config traffic summary and the dominant kernel's: HBM bytes per call =
    mean FETCH_SIZE x f + mean WRITE_SIZE x w (KiB), with f and w the ratios of
    a plain 1 GiB copy's known bytes to what the same counters read for it."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        order = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], int(r["Grid_Size"]))
                if key not in acc:
                    acc[key] = []
                    order.append(key)
                acc[key].append(float(r["Counter_Value"]))
        return order, {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    _, cf, _ = per_kernel(copyf_csv, "FETCH_SIZE")
    _, cw, _ = per_kernel(copyw_csv, "WRITE_SIZE")
    copy_kib = float(1 << 20)
    ff = copy_kib / max(v for k, v in cf.items() if "copyBuffer" in k[0])
    wf = copy_kib / max(v for k, v in cw.items() if "copyBuffer" in k[0])
    order, fetch, count = per_kernel(fetch_csv, "FETCH_SIZE")
    _, write, _ = per_kernel(write_csv, "WRITE_SIZE")
    ours = [k for k in order if "w4i::" in k[0]]
    # --workload configs launches, in this order: tiny, down, gate/up, lm_head GEMV, argmax finalize
    names = ["tiny", "down", "gateup", "lmhead", "lmhead_finalize"]
    if len(ours) != len(names):
        print(f"expected {len(names)} kernels of the library, found {len(ours)}: {ours}", file=sys.stderr)
        return 1
    per = {}
    for name, key in zip(names, ours):
        per[name] = {"kernel": key[0][:160], "grid": key[1], "dispatches": count[key],
                     "fetch_kib": round(fetch[key], 1), "write_kib": round(write.get(key, 0.0), 1),
                     "hbm_bytes": int(round((fetch[key] * ff + write.get(key, 0.0) * wf) * 1024))}
    fin = per.pop("lmhead_finalize")
    per["lmhead"]["hbm_bytes"] += fin["hbm_bytes"]
    per["lmhead"]["finalize"] = fin
    configs = {}
    for c in CONFIGS:
        alg = algorithmic_bytes(c["kind"], c["n"], c["k"], c["group"])
        e = per[c["name"]]
        configs[c["name"]] = {"hbm_bytes_per_launch": e["hbm_bytes"], "algorithmic_bytes": alg,
                              "ratio": round(e["hbm_bytes"] / alg, 4), "counters": e}
    src_hash = kernel_source_hash(GEMV_SRCS)
    summary = {"what": "HBM bytes per call of each config's kernels on cold buffers "
                       "(rocprofv3 FETCH_SIZE and WRITE_SIZE means, calibrated by a 1 GiB copy)",
               "kernel_source_sha256_16": src_hash, "fetch_factor": round(ff, 6), "write_factor": round(wf, 6),
               "configs": configs,
               "source": "bench.py --traffic-from over the four CSVs of the commands in "
                         "gemv_configs_traffic.md (same folder)"}
    with open(CONFIG_TRAFFIC_FILE, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    gu = configs["gateup"]
    dom = {"kernel": "gemv_w4_kernel<2, gate/up, split 2, depth 4, full, fp16 x> 37888x3584 g128",
           "kernel_source_sha256_16": src_hash, "hbm_bytes_per_launch": gu["hbm_bytes_per_launch"],
           "fetch_factor": round(ff, 6), "write_factor": round(wf, 6),
           "source": "the gate/up config of traffic_configs.json (same folder)"}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(dom, f, indent=1)
        f.write("\n")
    print(json.dumps(summary, indent=1))
    return 0


class ClockSampler:
    """Samples the GPU's engine and memory clocks, power and throttle status
    (amdsmi GPU metrics) from a background thread while a measured loop runs."""

    KEYS = ("current_gfxclk", "average_gfxclk_frequency", "current_uclk", "average_uclk_frequency",
            "current_socket_power", "average_socket_power", "temperature_hotspot", "temperature_mem",
            "throttle_status", "indep_throttle_status")

    def __init__(self, period_s: float = 0.0005):
        self.period = period_s
        self.samples = []
        self.error = None
        self._stop = None
        self._thread = None
        self._handle = None

    def _read(self):
        import amdsmi
        m = amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        row = {}
        for key in self.KEYS:
            v = m.get(key)
            if isinstance(v, (int, float)) and v not in (0xFFFF, 0xFFFFFFFF, 0xFFFFFFFFFFFFFFFF):
                row[key] = v
        gfx = m.get("current_gfxclks")
        if isinstance(gfx, (list, tuple)):
            vals = [v for v in gfx if isinstance(v, (int, float)) and 0 < v < 0xFFFF]
            if vals:
                row["current_gfxclks_min"] = min(vals)
                row["current_gfxclks_max"] = max(vals)
        return row

    def __enter__(self):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
            self.samples.append(self._read())
        except Exception as e:  # clocks are context; the measurement does not depend on them
            self.error = f"{type(e).__name__}: {e}"
            return self
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    self.samples.append(self._read())
                except Exception as e:
                    self.error = f"{type(e).__name__}: {e}"
                    return
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if self._handle is not None:
            try:
                import amdsmi
                self.samples.append(self._read())
                amdsmi.amdsmi_shut_down()
            except Exception:
                pass
        return False

    def summary(self):
        if not self.samples:
            return {"error": self.error or "no samples"}
        keys = sorted({k for r in self.samples for k in r})
        out = {"samples": len(self.samples)}
        for k in keys:
            vals = [r[k] for r in self.samples if k in r]
            if "throttle" in k:
                out[k] = sorted({int(v) for v in vals})
            else:
                out[k] = {"min": min(vals), "max": max(vals), "first": vals[0], "last": vals[-1]}
        if self.error:
            out["error"] = self.error
        return out


def time_graph_vs_eager(projs, stream, steps: int, rounds: int = 3):
    """The captured sweep and the same launches issued eagerly by the
    library, timed the same way (HIP events around `steps` sweeps) in
    alternating rounds after one shared warm-up; medians of the rounds."""
    from int4_weight_only_04_amd import w4
    graph = w4.Sweep(projs, mode=w4.SWEEP_GRAPH)
    eager = w4.Sweep(projs, mode=w4.SWEEP_EAGER)
    for sw in (graph, eager):
        time_graph(sw, stream, 2, 2)
    g_ms, e_ms = [], []
    for _ in range(rounds):
        g_ms.append(time_graph(graph, stream, steps, 0)[0])
        e_ms.append(time_graph(eager, stream, steps, 0)[0])
    graph.close()
    eager.close()
    med = lambda v: sorted(v)[len(v) // 2]
    return med(g_ms), med(e_ms), g_ms, e_ms


def py_eager_sweep(projs, stream):
    """One sweep launched projection by projection from Python through the
    binding (the host-driven eager loop the pages compare graph capture with)."""
    from int4_weight_only_04_amd import w4
    for p in projs:
        if p.kind == w4.PROJ_GATEUP_SILU:
            w4.gemv_gateup_silu(p.packed_w, p.packed_s, p.x, p.out, p.n, p.k, p.group, stream=stream)
        elif p.kind == w4.PROJ_LMHEAD_ARGMAX:
            w4.gemv(p.packed_w, p.packed_s, p.x, p.out, p.n, p.k, p.group, argmax=p.argmax, workspace=p.workspace,
                    stream=stream)
        else:
            w4.gemv(p.packed_w, p.packed_s, p.x, p.out, p.n, p.k, p.group, stream=stream)


def time_py_eager(projs, stream, steps: int, warmup: int = 2):
    import torch
    for _ in range(warmup):
        py_eager_sweep(projs, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        py_eager_sweep(projs, stream)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def host_info():
    """Host cores and CPU model, as the process sees them."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = min(avail, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else avail
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": avail, "omp_num_threads": omp, "threads": threads,
            "cpu_model": model}


def oracle_gemv_timed(pw, ps, x, n, k, g, kind, threads: int):
    """The oracle's GEMV (fp64 C, unchanged) over all rows, the rows split in
    `threads` contiguous ranges run by a thread pool (the C call releases the
    interpreter lock); gate/up adds the SiLU gate.  Seconds."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    gateup = kind == "gateup"
    t0 = time.perf_counter()
    if threads == 1:
        y, _ = oracle.gemv_packed(pw, ps, x, n, k, g, gateup=gateup)
    else:
        cuts = np.linspace(0, n, threads + 1).astype(np.int64)
        parts = [np.arange(cuts[i], cuts[i + 1], dtype=np.int64) for i in range(threads)]
        with ThreadPoolExecutor(max_workers=threads) as ex:
            ys = list(ex.map(lambda r: oracle.gemv_packed(pw, ps, x, n, k, g, gateup=gateup, rows=r)[0], parts))
        y = np.concatenate(ys)
    if gateup:
        oracle.silu_gate(y)
    if kind == "lmhead":
        int(np.argmax(y))
    return time.perf_counter() - t0


def cpu_baseline():
    """The oracle as it stands (fp64 C, never tuned), on the host's cores: once
    single-threaded and once over all available cores (rows split across a
    thread pool).  Per config one call each; the sweep figure is layer 0's
    four projections, run in full, with the whole sweep estimated as
    28 x layer 0 + lm_head."""
    from int4_weight_only_04_amd import w4
    host = host_info()
    nt = host["threads"]
    per_config = {}
    lm_s = {}
    for c in CONFIGS:
        layout, wb, sb, pw, ps, x = config_inputs(c)
        alg = algorithmic_bytes(c["kind"], c["n"], c["k"], c["group"])
        t1 = oracle_gemv_timed(pw, ps, x, c["n"], c["k"], c["group"], c["kind"], 1)
        tn = oracle_gemv_timed(pw, ps, x, c["n"], c["k"], c["group"], c["kind"], nt)
        per_config[c["name"]] = {"ms_1_thread": round(t1 * 1e3, 3), f"ms_{nt}_threads": round(tn * 1e3, 3),
                                 "gbs_1_thread": round(alg / t1 / 1e9, 4),
                                 f"gbs_{nt}_threads": round(alg / tn / 1e9, 4)}
        if c["name"] == "lmhead":
            lm_s = {1: t1, nt: tn}
    layer = synthetic.sweep_projections(1)
    total = 0
    t = {1: 0.0, nt: 0.0}
    for p in layer:
        layout = "gateup" if p.kind == "gateup" else "plain"
        wb, sb = w4.packed_size(p.n, p.k, p.group, layout)
        pw, ps, x = synthetic.packed_random(p.seed, wb, sb // 2, p.k)
        for th in (1, nt):
            t[th] += oracle_gemv_timed(pw, ps, x, p.n, p.k, p.group, p.kind, th)
        total += algorithmic_bytes(p.kind, p.n, p.k, p.group)
    layers = synthetic.LAYERS
    est = {th: (layers * t[th] + lm_s[th]) * 1e3 for th in (1, nt)}
    return {
        "value": round(total / t[nt] / 1e9, 4),
        "unit": "GB/s",
        "cores": nt,
        "kind": "oracle",
        "sample": f"layer 0 of the sweep (qkv, o_proj, gate/up+silu, down), all rows, {total} algorithmic "
                  f"bytes in {t[nt]:.2f} s on {nt} threads (rows split across a thread pool; fp64 C oracle)",
        "single_thread": {"value": round(total / t[1] / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "seconds": round(t[1], 3)},
        "sweep_ms_estimate": {"1_thread": round(est[1], 1), f"{nt}_threads": round(est[nt], 1),
                              "how": f"{layers} x layer 0 + lm_head, each timed in full"},
        "per_config": per_config,
        "host": host,
    }


def run_persistent(args) -> int:
    """The same 28-layer sweep in its persistent form (one cooperative kernel
    for all 113 projections, graph-captured) against the graph of one kernel
    per projection, timed alike (HIP events around `steps` sweeps after
    `warmup`), in alternating rounds; the outputs of the two are bit-identical
    (tests/test_gpu_persist.py)."""
    import torch
    from int4_weight_only_04_amd import w4
    specs, projs = build_sweep(args.layers)
    alg_bytes = sweep_bytes(specs)
    stream = torch.cuda.Stream()
    forms = {"graph": w4.Sweep(projs, mode=w4.SWEEP_GRAPH),
             "persistent": w4.Sweep(projs, mode=w4.SWEEP_PERSISTENT)}
    for sw in forms.values():
        time_graph(sw, stream, 2, args.warmup)
    rounds = {k: [] for k in forms}
    for _ in range(3):
        for k, sw in forms.items():
            rounds[k].append(time_graph(sw, stream, args.steps, 0)[0])
    timed_out = forms["persistent"].status()
    for sw in forms.values():
        sw.close()
    med = {k: sorted(v)[len(v) // 2] for k, v in rounds.items()}
    ms = med["persistent"]
    value = alg_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "persistent-kernel sweep: achieved HBM GB/s and ms per 28-layer+lm_head INT4 linear sweep",
        "value": round(value, 1),
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
            "workload": (f"the decode-step INT4 linear sweep ({args.layers} layers + lm_head) as one persistent "
                         "cooperative kernel (one workgroup per CU, hand-off through tagged words and arrival "
                         "counters), graph-captured, against the graph of one kernel per projection"),
            "graph_ms_per_step": round(med["graph"], 4),
            "persistent_vs_graph_time": round(ms / med["graph"], 3),
            "rounds_ms": {k: [round(x, 4) for x in v] for k, v in rounds.items()},
            "watchdog_timeout": bool(timed_out),
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        },
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


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


PREFILL_PRODUCTS = ("qkv", "o", "gateup", "down")


def product_of(p) -> str:
    """The product a projection is, from its name (``L<layer>.<product>``)."""
    return p.name.split(".", 1)[1]


def launch_prefill(items, lm_buf, workspace, stream, only: str | None = None):
    """The prefill sweep, or with `only` just that product's launches (no lm_head)."""
    from int4_weight_only_04_amd import w4
    m = synthetic.PROMPT
    for p, pw, ps, x, out in items:
        if only is not None and product_of(p) != only:
            continue
        if p.kind == "gateup":
            w4.gemm_gateup_silu(pw, ps, x, out, m, p.n, p.k, p.group, stream=stream)
        else:
            w4.gemm(pw, ps, x, out, m, p.n, p.k, p.group, workspace=workspace, stream=stream)
    if only is None:
        lm, pw, ps, x, y, am, ws = lm_buf
        w4.gemv(pw, ps, x, y, lm.n, lm.k, lm.group, argmax=am, workspace=ws, stream=stream)


def time_prefill_products(items, lm_buf, workspace, stream, reps: int = 3):
    """Each product on its own: its launches over every layer (each layer's
    weights are distinct, 0.2-1 GB per product, beyond the 256 MB Infinity
    Cache) captured in one graph, replayed once to warm up and `reps` times
    between events; microseconds per launch, the split-k reduction included."""
    m = synthetic.PROMPT
    rows = []
    for prod in PREFILL_PRODUCTS:
        sel = [it[0] for it in items if product_of(it[0]) == prod]
        if not sel:
            continue
        g = capture(lambda s, prod=prod: launch_prefill(items, lm_buf, workspace, s, only=prod), stream)
        us = replay_ms(g, stream, reps, 1) / len(sel) * 1e3
        del g
        p = sel[0]
        flops = 2 * m * p.n * p.k
        rows.append({"product": prod, "shape_m_n_k": [m, p.n, p.k], "launches": len(sel) * reps,
                     "w4_us_per_launch": round(us, 2),
                     "w4_tflops": round(flops / (us * 1e-6) / 1e12, 1),
                     "w4_pct_of_mfma_f16_peak": round(100.0 * flops / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 2)})
    return rows


def dense_f16_library_times(reps: int = 20) -> dict:
    """Context, not the INT4 path: the same products as dense fp16 weight
    matrices [n][k] through the vendor GEMM library (torch's F.linear, which
    calls hipBLASLt), x of 512 token rows.  Each shape cycles through enough
    weight copies to span >= 512 MiB, so every call reads its weights from
    HBM; one warm-up call per copy, then `reps` timed calls between events.
    The dense form reads 4x the INT4 weight bytes and dequantizes nothing;
    gate/up is timed without the SiLU (37888 output columns)."""
    import torch
    m = synthetic.PROMPT
    shapes = {"qkv": (synthetic.QKV, synthetic.HIDDEN), "o": (synthetic.HIDDEN, synthetic.HIDDEN),
              "gateup": (2 * synthetic.MLP, synthetic.HIDDEN), "down": (synthetic.HIDDEN, synthetic.MLP)}
    gen = torch.Generator(device="cuda").manual_seed(5150)
    out = {}
    for prod, (n, k) in shapes.items():
        copies = max(2, -(-(512 << 20) // (2 * n * k)))
        x = torch.randn((m, k), generator=gen, device="cuda", dtype=torch.float16)
        ws = [torch.randn((n, k), generator=gen, device="cuda", dtype=torch.float16) for _ in range(copies)]
        for w in ws:
            torch.nn.functional.linear(x, w)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            torch.nn.functional.linear(x, ws[i % copies])
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        tflops = 2 * m * n * k / (us * 1e-6) / 1e12
        out[prod] = {"dense_f16_library_us": round(us, 2), "dense_f16_library_tflops": round(tflops, 1),
                     "dense_f16_library_pct_of_mfma_f16_peak": round(100.0 * tflops / MFMA_F16_PEAK_TFLOPS, 2)}
        del ws, x
        torch.cuda.empty_cache()
    return out


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


def _pool_map(fn, items, threads: int):
    """fn over items on a thread pool of `threads` (the oracle's C calls release
    the interpreter lock), results in order."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


def _row_ranges(n: int, parts: int):
    cuts = np.linspace(0, n, parts + 1).astype(np.int64)
    return [np.arange(cuts[i], cuts[i + 1], dtype=np.int64) for i in range(parts)]


def prefill_cpu_baseline(tokens: int = 4):
    """The oracle's prefill product (fp64 C, unchanged) on a bounded sample:
    layer 0's four projections, all weight rows, for the first `tokens` rows
    of their token blocks; once single-threaded and once with the weight rows
    split over all available cores."""
    import oracle
    from int4_weight_only_04_amd import w4
    host = host_info()
    nt = host["threads"]
    flops = 0
    t = {1: 0.0, nt: 0.0}
    for p in synthetic.prefill_projections(1):
        gateup = p.kind == "gateup"
        layout = "gateup" if gateup else "plain"
        wb, sb = w4.packed_size(p.n, p.k, p.group, layout)
        pw, ps, _ = synthetic.packed_random(p.seed, wb, sb // 2, p.k)
        xm = synthetic.prompt_acts(p.seed + 5, tokens, p.k)
        for th in (1, nt):
            t0 = time.perf_counter()
            if th == 1:
                y, _ = oracle.gemm_packed(pw, ps, xm, p.n, p.k, p.group, gateup=gateup)
            else:
                ys = _pool_map(lambda r: oracle.gemm_packed(pw, ps, xm, p.n, p.k, p.group, gateup=gateup,
                                                            ncols=r)[0], _row_ranges(p.n, th), th)
                y = np.concatenate(ys, axis=1)
            if gateup:
                for row in y:
                    oracle.silu_gate(row)
            t[th] += time.perf_counter() - t0
        flops += 2 * tokens * p.n * p.k
    return {
        "value": flops / t[nt] / 1e12,
        "unit": "TFLOP/s",
        "cores": nt,
        "kind": "oracle",
        "sample": f"layer 0 of the prefill sweep (qkv, o_proj, gate/up+silu, down), all rows, first "
                  f"{tokens} prompt tokens: {flops} flops in {t[nt]:.2f} s on {nt} threads (weight rows split "
                  f"across a thread pool; fp64 C oracle)",
        "seconds": t[nt],
        "single_thread": {"value": flops / t[1] / 1e12, "unit": "TFLOP/s", "cores": 1, "seconds": round(t[1], 3)},
        "host": host,
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
    print("[bench] each product alone, and the dense fp16 library GEMM at the same shapes",
          file=sys.stderr, flush=True)
    reps = 3
    per_product = time_prefill_products(items, lm_buf, workspace, stream, reps)
    del g
    dense = dense_f16_library_times()
    for row in per_product:
        d = dense.get(row["product"])
        if d:
            row.update(d)
            row["w4_time_vs_dense_f16_library"] = round(row["w4_us_per_launch"] / d["dense_f16_library_us"], 3)
    gu_row = next(r for r in per_product if r["product"] == "gateup")
    gu_ms = gu_row["w4_us_per_launch"] / 1e3
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
            "per_product": per_product,
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
            "launches_timed": gu_row["launches"],
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
    """The oracle's attention (fp64 C, unchanged) on `layers` layers' caches at
    the full context: once single-threaded, one layer after another, and once
    with the layers spread over all available cores (a thread pool of
    min(cores, layers) threads; the oracle computes one call's heads in
    order)."""
    import oracle
    host = host_info()
    nt = host["threads"]
    rng = np.random.default_rng(4000)
    npages = ATTN_CTX // ATTN_PAGE
    calls = []
    for _ in range(layers):
        q = rng.standard_normal((ATTN_HEADS, 128)).astype(np.float16).view(np.uint16)
        kc = rng.standard_normal((npages, ATTN_KV_HEADS, ATTN_PAGE, 128)).astype(np.float16).view(np.uint16)
        vc = rng.standard_normal((npages, ATTN_KV_HEADS, ATTN_PAGE, 128)).astype(np.float16).view(np.uint16)
        table = rng.permutation(npages).astype(np.int32)
        calls.append((q, kc, vc, table))

    def one(c):
        q, kc, vc, table = c
        return oracle.attn_decode(q, kc, vc, table, ATTN_CTX, ATTN_KV_HEADS, ATTN_PAGE, 1.0 / np.sqrt(128.0))

    t0 = time.perf_counter()
    for c in calls:
        one(c)
    t1 = time.perf_counter() - t0
    th = min(nt, layers)
    t0 = time.perf_counter()
    _pool_map(one, calls, th)
    tn = time.perf_counter() - t0
    nbytes = layers * attn_bytes(ATTN_CTX)
    return {
        "value": nbytes / tn / 1e9,
        "unit": "GB/s",
        "cores": th,
        "kind": "oracle",
        "sample": f"{layers} layers' attention at context {ATTN_CTX} (28 query heads, 4 KV heads, pages of "
                  f"{ATTN_PAGE}): {nbytes} algorithmic bytes in {tn:.2f} s on {th} threads (one layer per "
                  f"task; fp64 C oracle)",
        "seconds": tn,
        "single_thread": {"value": nbytes / t1 / 1e9, "unit": "GB/s", "cores": 1, "seconds": round(t1, 3)},
        "host": host,
    }


def run_attention(args) -> int:
    """28 layers' decode attention at a 4096-token context: two sets of 28
    caches (470 MB, beyond the 256 MB Infinity Cache) alternate, each layer
    with its own seeded cache, all of one sequence's permuted page table, in
    one HIP graph."""
    import torch
    from int4_weight_only_04_amd import w4
    layers = args.layers
    npages = ATTN_CTX // ATTN_PAGE
    dev = "cuda"
    g = torch.Generator(device="cpu").manual_seed(4001)
    # one sequence: its page table (a permutation of the pages) is shared by
    # every layer, as a paged cache's block table belongs to the sequence
    table = torch.randperm(npages, generator=g).to(torch.int32).to(dev)
    calls = []
    for i in range(2 * layers):
        kc = torch.randn((npages, ATTN_KV_HEADS, ATTN_PAGE, 128), generator=g).to(torch.float16).to(dev)
        vc = torch.randn((npages, ATTN_KV_HEADS, ATTN_PAGE, 128), generator=g).to(torch.float16).to(dev)
        q = torch.randn((ATTN_HEADS, 128), generator=g).to(torch.float16).to(dev)
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
            "traffic": read_traffic(path=ATTN_TRAFFIC_FILE, src=ATTN_SRC),
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


def build_step(layers: int, device: str = "cuda"):
    """Device model of the full decode step: the sweep's packed weights (same
    seeds), seeded RMSNorm weights, an fp16 embedding table of uniform random
    magnitudes in [0.25, 0.5), and per layer a paged fp16 KV cache of
    4096 tokens (pages of 16) filled with N(0, 1) values standing in for the
    prompt, one shared permuted page table.  No qkv bias (the pages give none)."""
    import torch
    from int4_weight_only_04_amd import w4
    H, V = synthetic.HIDDEN, synthetic.VOCAB
    nkv, page, max_ctx = synthetic.KV_HEADS, synthetic.PAGE, synthetic.MAX_CTX
    num_pages = max_ctx // page
    specs = synthetic.sweep_projections(layers)

    def packed(p):
        layout = "gateup" if p.kind == "gateup" else "plain"
        wb, sb = w4.packed_size(p.n, p.k, p.group, layout)
        pw, ps, _ = synthetic.packed_random(p.seed, wb, sb // 2, p.k)
        return torch.from_numpy(pw).to(device), torch.from_numpy(ps).to(device)

    def f16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.float16)

    g = torch.Generator(device="cpu").manual_seed(5000)
    step_layers = []
    for l in range(layers):
        pq, po, pg, pd = specs[4 * l: 4 * l + 4]
        (qw, qs), (ow, os_), (gw, gs), (dw, ds) = packed(pq), packed(po), packed(pg), packed(pd)
        shape = (num_pages, nkv, page, 128)
        kc = torch.randn(shape, generator=g).to(torch.float16).to(device)
        vc = torch.randn(shape, generator=g).to(torch.float16).to(device)
        step_layers.append(w4.StepLayer(
            attn_norm=f16(synthetic.norm_weights(6000 + 10 * l, H)), qkv_w=qw, qkv_s=qs, o_w=ow, o_s=os_,
            mlp_norm=f16(synthetic.norm_weights(6001 + 10 * l, H)), gateup_w=gw, gateup_s=gs, down_w=dw,
            down_s=ds, k_cache=kc, v_cache=vc))
    lw, ls = packed(specs[-1])
    embed = f16(synthetic.half_bits_uniform(6900, V * H, lo_exp=13)).view(V, H)
    model = dict(
        layers=step_layers, embed=embed, final_norm=f16(synthetic.norm_weights(6901, H)), lm_w=lw, lm_s=ls,
        page_table=torch.from_numpy(synthetic.page_table(6902, num_pages, num_pages)).to(device),
        token=torch.zeros(1, dtype=torch.int32, device=device),
        pos=torch.zeros(1, dtype=torch.int32, device=device),
        logits=torch.empty(V, dtype=torch.float32, device=device))
    return specs, model


def make_step(model, use_graph: bool):
    from int4_weight_only_04_amd import w4
    return w4.DecodeStep(hidden=synthetic.HIDDEN, n_heads=synthetic.HEADS, n_kv_heads=synthetic.KV_HEADS,
                         inter=synthetic.MLP, vocab=synthetic.VOCAB, group=synthetic.GROUP,
                         page_size=synthetic.PAGE, max_ctx=synthetic.MAX_CTX, rms_eps=1e-6, rope_theta=1e6,
                         use_graph=use_graph, **model)


def step_bytes(specs, layers: int, ctx: int) -> int:
    """Algorithmic bytes of one decode step at context ctx: the 113 INT4
    products (as in the sweep), each layer's attention over ctx cached tokens,
    the embedding row, the norm weights and the residual traffic."""
    H = synthetic.HIDDEN
    glue = 2 * H + (2 * layers + 1) * (2 * H + 4 * H * 3)  # embedding row; per norm: gamma, h, y, h
    return sweep_bytes(specs) + layers * attn_bytes(ctx) + glue


def run_steps(step, model, stream, start_token: int, start_pos: int, n: int, record: bool = False):
    """Run n steps from (start_token, start_pos); return the tokens if record."""
    import torch
    model["token"].fill_(start_token)
    model["pos"].fill_(start_pos)
    torch.cuda.synchronize()
    toks = []
    for _ in range(n):
        step.run(stream)
        if record:
            stream.synchronize()
            toks.append(int(model["token"].item()))
    return toks


class PyEagerStep:
    """The same decode step issued op by op from Python through the per-op C
    ABI (w4_embed, w4_add_rmsnorm, w4_gemv, w4_rope_kv_append, w4_attn_decode,
    w4_gemv_gateup_silu): what a host-driven eager loop costs."""

    def __init__(self, model):
        import torch
        from int4_weight_only_04_amd import w4
        H, I = synthetic.HIDDEN, synthetic.MLP
        nh, nkv = synthetic.HEADS, synthetic.KV_HEADS
        self.m, self.w4 = model, w4
        dev = "cuda"
        self.h = torch.empty(H, dtype=torch.float32, device=dev)
        self.y = torch.empty(H, dtype=torch.float32, device=dev)
        self.x = torch.empty(H, dtype=torch.float16, device=dev)
        self.qkv = torch.empty((nh + 2 * nkv) * 128, dtype=torch.float32, device=dev)
        self.q = torch.empty((nh, 128), dtype=torch.float16, device=dev)
        self.ao = torch.empty((nh, 128), dtype=torch.float16, device=dev)
        self.mh = torch.empty(I, dtype=torch.float16, device=dev)
        self.ctx = torch.zeros(1, dtype=torch.int32, device=dev)
        self.attn_ws = torch.empty(w4.attn_decode_workspace_size(nh, synthetic.MAX_CTX), dtype=torch.uint8,
                                   device=dev)
        self.lm_ws = torch.empty(w4.gemv_workspace_size(synthetic.VOCAB, H, synthetic.GROUP, True),
                                 dtype=torch.uint8, device=dev)
        self.scale = 1.0 / float(np.sqrt(128.0))

    def run(self, stream):
        w4, m = self.w4, self.m
        H, I, G = synthetic.HIDDEN, synthetic.MLP, synthetic.GROUP
        nh, nkv = synthetic.HEADS, synthetic.KV_HEADS
        rows = (nh + 2 * nkv) * 128
        w4.embed(m["embed"], m["token"], self.h, stream=stream)
        for l, L in enumerate(m["layers"]):
            w4.add_rmsnorm(self.h, None if l == 0 else self.y, L.attn_norm, 1e-6, self.x, stream=stream)
            w4.gemv(L.qkv_w, L.qkv_s, self.x, self.qkv, rows, H, G, stream=stream)
            w4.rope_kv_append(self.qkv, L.qkv_bias, m["pos"], nh, nkv, 1e6, self.q, L.k_cache, L.v_cache,
                              m["page_table"], synthetic.MAX_CTX, self.ctx, stream=stream)
            w4.attn_decode(self.q, L.k_cache, L.v_cache, m["page_table"], self.ctx, synthetic.MAX_CTX, self.ao,
                           nkv, synthetic.PAGE, self.scale, self.attn_ws, stream=stream)
            w4.gemv(L.o_w, L.o_s, self.ao, self.y, H, nh * 128, G, stream=stream)
            w4.add_rmsnorm(self.h, self.y, L.mlp_norm, 1e-6, self.x, stream=stream)
            w4.gemv_gateup_silu(L.gateup_w, L.gateup_s, self.x, self.mh, 2 * I, H, G, stream=stream)
            w4.gemv(L.down_w, L.down_s, self.mh, self.y, H, I, G, stream=stream)
        w4.add_rmsnorm(self.h, self.y, m["final_norm"], 1e-6, self.x, stream=stream)
        w4.gemv(m["lm_w"], m["lm_s"], self.x, m["logits"], synthetic.VOCAB, H, G, argmax=m["token"],
                workspace=self.lm_ws, stream=stream)
        import torch
        with torch.cuda.stream(stream):
            m["pos"].add_(1)


def step_cpu_baseline(ctx: int):
    """The oracle's decode step (single thread, fp64) on a bounded sample: one
    full-width layer at context ctx and the lm_head, scaled to 28 layers."""
    import oracle
    from oracle import step as ostep
    H, I, V, G = synthetic.HIDDEN, synthetic.MLP, synthetic.VOCAB, synthetic.GROUP
    nh, nkv, page = synthetic.HEADS, synthetic.KV_HEADS, synthetic.PAGE
    m = synthetic.step_model(6100, hidden=H, n_heads=nh, n_kv=nkv, inter=I, vocab=V, group=G, layers=1,
                             embed=False)
    L = m["layers"][0]
    lay = ostep.Layer(attn_norm=L["attn_norm"], qkv=ostep.Proj(*L["qkv"]), o=ostep.Proj(*L["o"]),
                      mlp_norm=L["mlp_norm"], gateup=ostep.Proj(*L["gateup"]), down=ostep.Proj(*L["down"]))
    cfg = ostep.Config(hidden=H, n_heads=nh, n_kv=nkv, inter=I, group=G, page=page, eps=1e-6, theta=1e6)
    pages = -(-(ctx + 1) // page)
    kc, vc = synthetic.kv_prefix(6101, pages, nkv, page)
    table = np.arange(pages, dtype=np.int32)
    h = np.random.default_rng(6102).standard_normal(H)
    oracle.default()
    t0 = time.perf_counter()
    r = ostep.decoder_layer(h, lay, cfg, ctx, kc, vc, table)
    t_layer = time.perf_counter() - t0
    t0 = time.perf_counter()
    ostep.final_logits(r.h_out, m["final_norm"], ostep.Proj(*m["lm"]), cfg)
    t_lm = time.perf_counter() - t0
    per_token = synthetic.LAYERS * t_layer + t_lm
    return {
        "value": 1.0 / per_token,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"one full-width decoder layer at context {ctx + 1} ({t_layer:.2f} s) and the lm_head with "
                   f"argmax ({t_lm:.2f} s), single-threaded fp64, scaled to {synthetic.LAYERS} layers"),
        "seconds": t_layer + t_lm,
    }


def run_step(args) -> int:
    """The full decode step, graph and eager, on the 7B-class shapes."""
    import torch
    layers = args.layers
    prompt = synthetic.PROMPT
    steps, warmup = args.steps, args.warmup
    if prompt + steps > synthetic.MAX_CTX or warmup > prompt:
        print("bench.py: prompt + steps must stay within the 4096-token context", file=sys.stderr)
        return 2
    print(f"[bench] building the decode-step model ({layers} layers)", file=sys.stderr, flush=True)
    specs, model = build_step(layers)
    stream = torch.cuda.Stream()
    graph = make_step(model, True)
    eager = make_step(model, False)
    launches = graph.launches()

    print("[bench] graph vs eager token check", file=sys.stderr, flush=True)
    check_n = 12
    toks_graph = run_steps(graph, model, stream, 1234, prompt, check_n, record=True)
    toks_eager = run_steps(eager, model, stream, 1234, prompt, check_n, record=True)
    pyeager = PyEagerStep(model)
    toks_py = run_steps(pyeager, model, stream, 1234, prompt, check_n, record=True)

    def timed(step, n_warm, n):
        run_steps(step, model, stream, 1234, prompt - n_warm, n_warm)
        stream.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(n):
            step.run(stream)
        b.record(stream)
        stream.synchronize()
        return a.elapsed_time(b) / n, (time.perf_counter() - t0) * 1e3 / n

    print(f"[bench] graph: {warmup} warmup + {steps} timed tokens", file=sys.stderr, flush=True)
    ms, wall_ms = timed(graph, warmup, steps)
    print(f"[bench] eager: 2 warmup + {args.eager_steps} timed tokens", file=sys.stderr, flush=True)
    eager_ms, eager_wall = timed(eager, 2, args.eager_steps)
    print(f"[bench] python-driven eager: 2 warmup + {args.eager_steps} timed tokens", file=sys.stderr, flush=True)
    py_ms, py_wall = timed(pyeager, 2, args.eager_steps)

    print("[bench] dominant kernel", file=sys.stderr, flush=True)
    from int4_weight_only_04_amd import w4
    x = torch.zeros(synthetic.HIDDEN, dtype=torch.float16, device="cuda")
    hbuf = torch.empty(synthetic.MLP, dtype=torch.float16, device="cuda")
    gu = [w4.Proj(w4.PROJ_GATEUP_SILU, 2 * synthetic.MLP, synthetic.HIDDEN, synthetic.GROUP, L.gateup_w, L.gateup_s,
                  x, hbuf) for L in model["layers"]]
    gu_mean_ms, gu_launches, _, _ = time_dominant_kernel(gu, stream)
    gu_bytes = algorithmic_bytes("gateup", 2 * synthetic.MLP, synthetic.HIDDEN, synthetic.GROUP)
    gu_gbs = gu_bytes / (gu_mean_ms * 1e-3) / 1e9
    graph.close()
    eager.close()

    mid_ctx = prompt + steps // 2
    nbytes = step_bytes(specs, layers, mid_ctx)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": STEP_METRIC,
        "value": round(1000.0 / ms, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"batch-1 greedy decode, one hipGraph per token: embedding, {layers} pre-norm decoder "
                         "layers (RMSNorm, INT4 qkv 3584->4608, RoPE + paged fp16 KV append, attention with 28 "
                         "query / 4 KV heads, INT4 o_proj, RMSNorm, INT4 gate/up 3584->2x18944 + silu, INT4 down "
                         "18944->3584, fp32 residual), final RMSNorm, INT4 lm_head 3584->152064 + argmax, "
                         f"tokens {prompt}..{prompt + steps - 1} after a {prompt}-token prompt"),
            "kernels_per_step": launches,
            "algorithmic_bytes_per_step_at_mid_context": nbytes,
            "achieved_gbs": round(gbs, 1),
            "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
            "wall_ms_per_step": round(wall_ms, 4),
            "eager_ms_per_step": round(eager_ms, 4),
            "eager_wall_ms_per_step": round(eager_wall, 4),
            "graph_speedup_vs_eager": round(eager_ms / ms, 3),
            "graph_eager_tokens_equal": toks_graph == toks_eager,
            "python_eager_ms_per_step": round(py_ms, 4),
            "python_eager_wall_ms_per_step": round(py_wall, 4),
            "graph_speedup_vs_python_eager": round(py_wall / wall_ms, 3),
            "python_eager_tokens_equal": toks_graph == toks_py,
            "pages_context_h100": {"runtime_ms_per_token": 16.7, "eager_ms_per_token": 119,
                                   "llama_cpp_q4_k_m_ms_per_token": 4.95},
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
        print("[bench] cpu baseline (oracle decode step)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = step_cpu_baseline(mid_ctx)
    print(json.dumps(out), flush=True)
    return 0


def a8_bytes(kind: str, n: int, k: int, group: int) -> int:
    """Bytes of one W4A8 GEMV: the W4A16 GEMV's with int8 codes (k bytes) and
    fp32 group scales in place of the fp16 x."""
    return algorithmic_bytes(kind, n, k, group) - 2 * k + k + 4 * (k // group)


def quant_bytes(k: int, group: int) -> int:
    """Bytes of one activation quantization: fp16 x in, codes and scales out."""
    return 2 * k + k + 4 * (k // group)


def w4a8_cpu_baseline():
    """The oracle's W4A8 product (fp64 C, unchanged) on layer 0's four
    projections, all rows, plus the oracle's quantization of their inputs:
    once single-threaded and once with the rows split over all available
    cores (the quantization runs once, on one thread, in both)."""
    import oracle
    from int4_weight_only_04_amd import w4
    host = host_info()
    nt = host["threads"]
    total = 0
    t = {1: 0.0, nt: 0.0}
    for p in synthetic.sweep_projections(1):
        gateup = p.kind == "gateup"
        layout = "gateup" if gateup else "plain"
        wb, sb = w4.packed_size(p.n, p.k, p.group, layout)
        pw, ps, x = synthetic.packed_random(p.seed, wb, sb // 2, p.k)
        for th in (1, nt):
            t0 = time.perf_counter()
            c, sc = oracle.quantize_act8(x, p.group)
            if th == 1:
                y, _ = oracle.gemv_a8_packed(pw, ps, c, sc, p.n, p.k, p.group, gateup=gateup)
            else:
                ys = _pool_map(lambda r: oracle.gemv_a8_packed(pw, ps, c, sc, p.n, p.k, p.group, gateup=gateup,
                                                               rows=r)[0], _row_ranges(p.n, th), th)
                y = np.concatenate(ys)
            if gateup:
                oracle.silu_gate(y)
            t[th] += time.perf_counter() - t0
        total += a8_bytes(p.kind, p.n, p.k, p.group) + quant_bytes(p.k, p.group)
    return {
        "value": total / t[nt] / 1e9,
        "unit": "GB/s",
        "cores": nt,
        "kind": "oracle",
        "sample": f"layer 0 of the W4A8 sweep (quantize + qkv, o_proj, gate/up+silu, down), all rows, {total} "
                  f"algorithmic bytes in {t[nt]:.2f} s on {nt} threads (rows split across a thread pool; fp64 C "
                  f"oracle)",
        "seconds": t[nt],
        "single_thread": {"value": total / t[1] / 1e9, "unit": "GB/s", "cores": 1, "seconds": round(t[1], 3)},
        "host": host,
    }


def run_w4a8(args) -> int:
    """The linear sweep with int8 activations, next to the W4A16 sweep."""
    import torch
    from int4_weight_only_04_amd import w4
    print(f"[bench] building sweep ({args.layers} layers)", file=sys.stderr, flush=True)
    specs, projs = build_sweep(args.layers)
    stream = torch.cuda.Stream()
    bufs = []
    for p, pr in zip(specs, projs):
        codes = torch.empty(p.k, dtype=torch.int8, device="cuda")
        scales = torch.empty(p.k // p.group, dtype=torch.float32, device="cuda")
        bufs.append((p, pr, codes, scales))

    def launch(s, quant: bool, only=None):
        for p, pr, codes, scales in bufs:
            if only is not None and p.kind != only:
                continue
            if quant:
                w4.quantize_act8(pr.x, p.group, codes, scales, stream=s)
            if p.kind == "gateup":
                w4.gemv_gateup_silu_a8(pr.packed_w, pr.packed_s, codes, scales, pr.out, p.n, p.k, p.group, stream=s)
            elif p.kind == "lmhead":
                w4.gemv_a8(pr.packed_w, pr.packed_s, codes, scales, pr.out, p.n, p.k, p.group, argmax=pr.argmax,
                           workspace=pr.workspace, stream=s)
            else:
                w4.gemv_a8(pr.packed_w, pr.packed_s, codes, scales, pr.out, p.n, p.k, p.group, stream=s)

    with torch.cuda.stream(stream):
        launch(stream, True)   # fill the codes once for the GEMV-only graph
    stream.synchronize()
    print("[bench] W4A8 sweep with quantization (graph)", file=sys.stderr, flush=True)
    g_q = capture(lambda s: launch(s, True), stream)
    ms_q = replay_ms(g_q, stream, args.steps, args.warmup)
    print("[bench] W4A8 sweep, GEMVs only (graph)", file=sys.stderr, flush=True)
    g_g = capture(lambda s: launch(s, False), stream)
    ms_g = replay_ms(g_g, stream, args.steps, args.warmup)
    print("[bench] W4A16 sweep (graph)", file=sys.stderr, flush=True)
    sweep16 = w4.Sweep(projs, use_graph=True)
    ms16, _ = time_graph(sweep16, stream, args.steps, args.warmup)
    sweep16.close()

    print("[bench] dominant kernel (W4A8 gate/up)", file=sys.stderr, flush=True)
    g_gu = capture(lambda s: launch(s, False, only="gateup"), stream)
    with torch.cuda.stream(stream):
        g_gu.replay()
    stream.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    replays = 4
    with torch.cuda.stream(stream):
        a.record(stream)
        for _ in range(replays):
            g_gu.replay()
        b.record(stream)
    stream.synchronize()
    n_gu = sum(1 for p in specs if p.kind == "gateup")
    gu_ms = a.elapsed_time(b) / (replays * n_gu)
    gp = next(p for p in specs if p.kind == "gateup")
    gu_bytes = a8_bytes("gateup", gp.n, gp.k, gp.group)
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9

    bytes_q = sum(a8_bytes(p.kind, p.n, p.k, p.group) + quant_bytes(p.k, p.group) for p in specs)
    bytes_g = sum(a8_bytes(p.kind, p.n, p.k, p.group) for p in specs)
    value = bytes_q / (ms_q * 1e-3) / 1e9
    out = {
        "metric": W4A8_METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_q, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8xi4->i32, f32",
        "data": "synthetic",
        "config": {
            "workload": (f"batch-1 decode-step INT4 linear sweep with int8 activations, hipGraph: {args.layers} x "
                         "(quantize x + qkv 3584->4608, o_proj, gate/up 3584->2x18944 + silu, down 18944->3584) + "
                         "lm_head 3584->152064 + argmax; activations per group of 128 (symmetric int8, fp32 scale), "
                         "integer 8-input block sums, fp32 accumulation"),
            "algorithmic_bytes_per_step": bytes_q,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "gemv_only_ms_per_step": round(ms_g, 4),
            "gemv_only_gbs": round(bytes_g / (ms_g * 1e-3) / 1e9, 1),
            "w4a16_ms_per_step": round(ms16, 4),
            "w4a16_gbs": round(sweep_bytes(specs) / (ms16 * 1e-3) / 1e9, 1),
            "w4a8_vs_w4a16_time_ratio": round(ms_q / ms16, 3),
            "w4a8_gemv_only_vs_w4a16_time_ratio": round(ms_g / ms16, 3),
        },
        "roofline": {
            "kernel": "gemv_w4_kernel<2, gate/up+silu, A8> 37888x3584 g128",
            "bound": "hbm",
            "achieved": round(gu_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(gu_bytes, A8_TRAFFIC_FILE),
            "algorithmic_bytes_per_launch": gu_bytes,
            "avg_launch_us": round(gu_ms * 1e3, 3),
            "launches_timed": replays * n_gu,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle W4A8)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = w4a8_cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; 128 for --workload step, the pages' tg128)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=synthetic.LAYERS)
    ap.add_argument("--eager-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=("decode", "prefill", "attention", "step", "w4a8", "configs", "persistent"),
                    default="decode",
                    help="decode: the per-token GEMV sweep (default); prefill: the 512-token GEMM sweep; "
                         "attention: 28 layers' paged-KV decode attention at a 4096-token context; "
                         "step: the full decode step (tokens 512.. after a 512-token prompt); "
                         "w4a8: the sweep with int8 activations; configs: only the per-config GEMV "
                         "timings on cold buffers (the run the traffic counters are taken over); "
                         "persistent: the sweep as one cooperative kernel against the graph")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic_configs.json (and the dominant kernel's traffic file) from "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE CSVs of --workload configs and --copy-probe; "
                         "host only")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args(argv)
    if args.traffic_from:
        return write_traffic(*args.traffic_from)
    if args.steps is None:
        args.steps = 128 if args.workload == "step" else 50

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
    if args.workload == "step":
        return run_step(args)
    if args.workload == "w4a8":
        return run_w4a8(args)
    if args.workload == "persistent":
        return run_persistent(args)
    if args.workload == "configs":
        stream = torch.cuda.Stream()
        print(json.dumps({"per_config": time_configs(stream, replays=1, max_calls=32)}), flush=True)
        return 0

    print(f"[bench] building sweep ({args.layers} layers)", file=sys.stderr, flush=True)
    specs, projs = build_sweep(args.layers)
    alg_bytes = sweep_bytes(specs)
    stream = torch.cuda.Stream()

    print("[bench] graph sweep", file=sys.stderr, flush=True)
    graph = w4.Sweep(projs, use_graph=True)
    ev_ms, wall_ms = time_graph(graph, stream, args.steps, args.warmup)
    graph.close()

    print("[bench] graph vs eager (alternating rounds)", file=sys.stderr, flush=True)
    g_med, e_med, g_rounds, e_rounds = time_graph_vs_eager(projs, stream, args.steps)
    print("[bench] python-driven eager sweep", file=sys.stderr, flush=True)
    py_ms = time_py_eager(projs, stream, args.eager_steps)

    print("[bench] dominant kernel (+ clocks)", file=sys.stderr, flush=True)
    gu_mean_ms, gu_launches, gu_sustained, gu_clocks = time_dominant_kernel(projs, stream)
    print("[bench] pure-read ceiling (113 read-only launches)", file=sys.stderr, flush=True)
    read_ms, read_bytes, stream_gbs = time_pure_read_sweep(specs, stream, args.steps, args.warmup)
    gp = next(p for p in specs if p.kind == "gateup")
    gu_bytes = algorithmic_bytes("gateup", gp.n, gp.k, gp.group)
    gu_gbs = gu_bytes / (gu_mean_ms * 1e-3) / 1e9
    del projs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print("[bench] per-config GEMVs on cold buffers", file=sys.stderr, flush=True)
    per_config = time_configs(stream)

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
            "graph_ms_per_step_alternating": round(g_med, 4),
            "eager_ms_per_step": round(e_med, 4),
            "graph_speedup_vs_eager": round(e_med / g_med, 3),
            "graph_vs_eager_rounds_ms": {"graph": [round(v, 4) for v in g_rounds],
                                         "eager": [round(v, 4) for v in e_rounds]},
            "python_eager_ms_per_step": round(py_ms, 4),
            "graph_speedup_vs_python_eager": round(py_ms / g_med, 3),
            "pure_read_sweep_ms": round(read_ms, 4),
            "pure_read_sweep_gbs": round(read_bytes / (read_ms * 1e-3) / 1e9, 1),
            "sweep_time_vs_pure_read": round(ev_ms / read_ms, 3),
            "stream_read_1gib_gbs": round(stream_gbs, 1),
            "per_config": per_config,
            "pages_context_h100": PAGES_CONTEXT_H100,
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
            "clocks": gu_clocks,
            "sustained": gu_sustained,
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
