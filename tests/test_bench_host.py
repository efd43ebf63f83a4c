"""Host-side checks of the benchmark script (no GPU): the MFU numerator of
the headline workload, and the refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from decoder_only_transformer_02_amd import gpt2 as G  # noqa: E402
from decoder_only_transformer_02_amd.inputs import PRESETS  # noqa: E402


def test_flops_per_token_of_the_124m_step():
    # 6N + 6 L C (T + 1) with N = all parameters but wpe, counted at the
    # unpadded vocabulary (padding earns no credit)
    import ctypes as ct
    p = PRESETS["gpt2_124m"]
    cfg = G.make_config(**{**p, "max_batch": p["B"], "max_seq": p["T"]})
    n_total = G.lib().gpt2_num_params(ct.byref(cfg))
    n = n_total - p["block_size"] * p["n_embd"] - (p["padded_vocab"] - p["vocab_size"]) * p["n_embd"]
    assert n == 123_653_376
    assert bench.flops_per_token(12, 768, 1024, n) == 798_598_656
    assert bench.flops_per_token(12, 768, 512, n) == 6 * n + 6 * 12 * 768 * 513


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_class_work_matches_the_scope_table_figures():
    """Per-step algorithmic work of the B=16 T=1024 step per timing class:
    GEMMs 3 x 2.783 TF (layers) + 3 x 1.266 TF (classifier); attention
    0.3095 TF forward, twice that backward; LayerNorm (6C+8) and (14C+8)
    bytes per token over 25 LayerNorms; cross-entropy (4 Vp + 8) bytes per
    token; norm 4 and AdamW 30 bytes per parameter."""
    p = PRESETS["gpt2_124m"]
    w = bench.class_work(p, 16, 1024, 124_475_904)
    assert w["gemm"][1] == 3 * 2 * 16384 * (12 * 12 * 768 * 768 + 50304 * 768)
    assert abs(w["gemm"][1] / 1e12 - (3 * 2.783 + 3 * 1.266)) < 0.01
    assert abs(w["lmhead_fwd"][1] / 1e12 - 1.266) < 0.001
    assert abs(w["attn_fwd"][1] / 1e12 - 0.3095) < 0.0005
    assert w["attn_bwd"][1] == 2 * w["attn_fwd"][1]
    assert abs(w["ln_fwd"][1] / 1e9 - 1.89) < 0.01
    assert abs(w["ln_bwd"][1] / 1e9 - 4.41) < 0.01
    assert abs(w["xent"][1] / 1e9 - 3.30) < 0.01
    assert abs(w["norm"][1] / 1e9 - 0.498) < 0.001
    assert abs(w["adamw"][1] / 1e9 - 3.734) < 0.001
    assert {k: v[0] for k, v in w.items()} == {
        "lmhead_fwd": "mfma", "gemm": "mfma", "attn_fwd": "mfma", "attn_bwd": "mfma", "ln_fwd": "hbm",
        "ln_bwd": "hbm", "xent": "hbm", "norm": "hbm", "adamw": "hbm"}


def test_roofline_entry_and_percentiles():
    e = bench.roofline_entry("mfma", 1.25e12, 1.0)   # 1.25 TF in 1 ms
    assert e["achieved"] == 1250.0 and e["frac"] == 0.5 and e["unit"] == "TFLOP/s"
    e = bench.roofline_entry("hbm", 4e9, 1.0)        # 4 GB in 1 ms
    assert e["achieved"] == 4000.0 and e["frac"] == 0.5 and e["unit"] == "GB/s"
    xs = [5.0, 1.0, 3.0, 2.0, 4.0]
    assert bench.percentile(xs, 50) == 3.0
    assert bench.percentile(xs, 10) == 1.4
    assert bench.percentile(xs, 90) == 4.6
    assert bench.percentile([7.0], 90) == 7.0


def test_bench_control_flow_on_the_emulated_library(monkeypatch, capsys):
    """bench.main() end to end with the library's CPU emulation standing in
    for the GPU and small presets standing in for the 124M shapes: every leg
    runs (timed steps with the classifier's launches bracketed, per-class
    timing, unpadded vocabulary, accumulated step, single block, oracle
    baseline) and one JSON line with the contract's keys is
    printed.  Timings here mean nothing; only the control flow is checked."""
    import json
    import time as _time

    import torch

    from decoder_only_transformer_02_amd import inputs
    from tests.emu.binding import EmuStep

    class Ev:
        def __init__(self, enable_timing=True):
            self.t = 0.0

        def record(self):
            self.t = _time.perf_counter()

        def elapsed_time(self, other):
            return (other.t - self.t) * 1e3

    small = dict(n_layer=2, n_head=2, n_embd=128, block_size=64, vocab_size=1000, padded_vocab=1024,
                 B=2, T=32, compute="bf16", tokens="zipf")
    presets = {"gpt2_124m": small, "gpt2_124m_v50257": {**small, "padded_vocab": 1000},
               "gpt2_124m_accum": {**small, "B": 2, "T": 16, "accum": 2, "lr_step": 132},
               "block124m": {**small, "tokens": "none"}}
    monkeypatch.setattr(inputs, "PRESETS", presets)
    monkeypatch.setattr(G, "GPT2Step", EmuStep)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    monkeypatch.setattr(torch.cuda, "Event", Ev)
    monkeypatch.setattr(torch.Tensor, "cuda", lambda self, *a, **k: self)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "3", "--warmup", "1"])
    bench.main()
    line = capsys.readouterr().out.strip().splitlines()[-1]
    rec = json.loads(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "kernels",
                "padding", "accumulated_step", "block", "ms_per_step_median", "ms_per_step_p10",
                "ms_per_step_p90"):
        assert key in rec, key
    assert rec["metric"] == bench.METRIC and rec["steps"] == 3 and rec["n_gpus"] == 1
    assert rec["roofline"]["bound"] == "mfma" and rec["roofline"]["launches"] == 1
    assert set(rec["kernels"]) >= {"gemm", "attn_fwd", "attn_bwd", "ln_fwd", "ln_bwd", "xent", "adamw",
                                   "norm", "embed"}
    assert rec["kernels"]["attn_fwd"]["launches_per_step"] == small["n_layer"]
    assert "transpose" not in rec["kernels"] and "colsum" not in rec["kernels"]
    assert rec["kernels"]["ln_fwd"]["launches_per_step"] == 2 * small["n_layer"] + 1
    assert rec["cpu_baseline"]["kind"] == "oracle" and rec["cpu_baseline"]["cores"] >= 1
    assert rec["accumulated_step"]["tokens_per_step"] == 2 * 16 * 2 and rec["accumulated_step"]["steps"] == 10
    assert rec["block"]["runs"] == 20 and rec["block"]["ms_median"] > 0
