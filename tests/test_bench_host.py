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
