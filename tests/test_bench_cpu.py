"""bench.py's accounting and contract, checked without a GPU.

The roofline's `achieved` figure is algorithmic bytes (or flops) per launch
divided by the measured time, so the byte counts are pinned here against
closed forms: nibbles K/2 per row, one fp16 scale per G inputs, the fp16
input once, the output once (fp32 y, fp16 h for gate/up, plus the 4-byte
argmax).  At the 7B shapes the sweep moves 3,650,274,308 bytes (3,650,274,304
without the argmax index), i.e. 0.456 ms at 8 TB/s."""
from __future__ import annotations

import subprocess
import sys
import os

import pytest

import bench
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_gemv_bytes_closed_forms():
    H, I, V, G = synthetic.HIDDEN, synthetic.MLP, synthetic.VOCAB, synthetic.GROUP
    assert bench.algorithmic_bytes("plain", 4608, H, G) == 4608 * H // 2 + 2 * 4608 * (H // G) + 2 * H + 4 * 4608
    assert bench.algorithmic_bytes("plain", H, I, G) == 35_060_736           # down
    assert bench.algorithmic_bytes("gateup", 2 * I, H, G) == 70_062_080      # gate/up + SiLU, fp16 h
    assert bench.algorithmic_bytes("lmhead", V, H, G) == 281_629_696 + 4     # + the 4-byte argmax index
    assert bench.algorithmic_bytes("plain", 512, 256, 64) == 72_192          # the tiny config
    specs = synthetic.sweep_projections()
    assert len(specs) == 113
    assert bench.sweep_bytes(specs) == 3_650_274_304 + 4


def test_w4a8_and_quantizer_bytes():
    H, G = synthetic.HIDDEN, synthetic.GROUP
    # codes (k bytes) and fp32 group scales replace the fp16 x
    assert bench.a8_bytes("plain", 4608, H, G) == bench.algorithmic_bytes("plain", 4608, H, G) - H + 4 * (H // G)
    assert bench.quant_bytes(H, G) == 2 * H + H + 4 * (H // G)


def test_attention_bytes():
    # K and V rows of ctx tokens for 4 KV heads of 128 fp16, q and the output, the page-table entries
    ctx = 4096
    assert bench.attn_bytes(ctx) == 2 * ctx * 4 * 128 * 2 + 2 * 28 * 128 * 2 + 4 * (ctx // 16)


def test_step_bytes_are_the_sweep_attention_and_glue():
    """Per step: the 113 products, 28 attentions at the context, the
    embedding row (fp16) and per norm (57 of them) gamma (fp16) plus the
    residual stream read, the producing GEMV's output read and h written back
    (fp32)."""
    specs = synthetic.sweep_projections()
    H = synthetic.HIDDEN
    glue = 2 * H + 57 * (2 * H + 3 * 4 * H)
    assert bench.step_bytes(specs, 28, 576) == bench.sweep_bytes(specs) + 28 * bench.attn_bytes(576) + glue


def test_prefill_flops():
    class P:
        def __init__(self, n, k):
            self.n, self.k = n, k
    items = [(P(4608, 3584),), (P(37888, 3584),)]
    lm = (P(152064, 3584),)
    assert bench.prefill_flops(items, lm) == 2 * 512 * (4608 + 37888) * 3584 + 2 * 152064 * 3584


def test_more_than_one_gpu_is_refused():
    """The build measures one GPU: --gpus N > 1 exits with a message, before
    touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("workload", ["decode", "prefill", "attention", "step", "w4a8"])
def test_workloads_are_selectable(workload):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0 and workload in r.stdout
