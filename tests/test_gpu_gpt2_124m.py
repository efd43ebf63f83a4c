"""GPU parity at the GPT-2 124M shapes: one block in isolation at its full
size (B=16, T=1024), the full step on a one-sequence batch against the
whole oracle step, the full B=16 batch on sampled rows the oracle computes
one by one, the unpadded vocabulary, and gradient accumulation."""
import numpy as np
import pytest

from decoder_only_transformer_02_amd import gpt2 as G
from decoder_only_transformer_02_amd import inputs
from oracle import gpt2_oracle as O
from tests.gpu_helpers import (configs, cosine, gpu_grads, oracle_init, rel_l2, say, to_dev)
from tests.test_gpu_parity import assert_bf16, run_step

pytestmark = pytest.mark.gpu

import torch  # noqa: E402

G124 = inputs.PRESETS["gpt2_124m"]
G124U = inputs.PRESETS["gpt2_124m_v50257"]


def test_block_124m_full_size():
    """One 124M block, B=16 T=1024, bf16: x ~ N(0,1), dy ~ N(0, 1e-3^2)."""
    B, T, C = 16, 1024, 768
    lc, oc, p = configs(inputs.PRESETS["block124m"], B, T)
    x, dy = inputs.block_inputs(0, B, T, C)
    say("block 124m B=16 T=1024")
    m = G.GPT2Step(lc, seed=0)
    y, dx = m.block_fwd_bwd(0, to_dev(x), to_dev(dy))
    y = y.cpu().numpy()
    dx = dx.cpu().numpy()
    names = [n for n in m.param_names() if n.startswith("h0.")]
    gg = gpu_grads(m, names)
    m.close()
    P = oracle_init(oc, 0)
    Pl = {n: P[n] for n in names}
    yr, dxr, gr = O.block_fwd_bwd(x, dy, Pl, 0, oc, dt=np.float32)
    say("y relL2", rel_l2(y, yr), "cos", cosine(y, yr), "dx cos", cosine(dx, dxr))
    assert rel_l2(y, yr) <= 2e-2 and cosine(y, yr) >= 0.999
    assert cosine(dx, dxr) >= 0.999
    for n in names:
        c = cosine(gg[n], gr[n])
        say(n, c)
        assert c >= 0.999, n


def test_gpt2_124m_step_one_sequence():
    """Full 124M step (vocab 50304, Zipf ids), one sequence of 1024, against
    the whole oracle step (float32 storage, float64 reductions)."""
    assert_bf16(*run_step(G124, 1, 1024, seed=0, data_seed=0, dt=np.float32))


def test_gpt2_124m_full_batch_sampled_rows():
    """B=16 T=1024 (the benchmark's launch configuration): per-position losses
    of sampled rows equal the oracle's forward of those rows alone; each
    logits-gradient row sums to zero; backward + AdamW finish with a finite
    norm and are bitwise reproducible."""
    B, T = 16, 1024
    lc, oc, p = configs(G124, B, T)
    s = inputs.zipf_stream(0, B * T + 1)
    x, y = inputs.batch_from_stream(s, B, T)
    runs = []
    for rep in range(2):
        m = G.GPT2Step(lc, seed=0)
        loss = m.forward(to_dev(x), to_dev(y))
        per = m.view("losses")[:B * T].cpu().numpy().reshape(B, T)
        dz = m.view("logits")[:B * T]
        rows = torch.tensor([0, 777, B * T - 1], device="cuda")
        sums = dz[rows].float().sum(dim=1).cpu().numpy()
        m.backward(1.0)
        norm = m.step(6e-4)
        wte = m.view("wte")[:64].clone().cpu()
        runs.append((loss, per, sums, norm, wte))
        m.close()
    loss, per, sums, norm, wte = runs[0]
    assert runs[1][0] == loss and runs[1][3] == norm and torch.equal(runs[1][4], wte)
    assert np.isfinite(norm) and 0 < norm
    assert np.all(np.abs(sums) <= 1e-2 / (B * T)), sums
    P = oracle_init(oc, 0)
    for b in (0, B - 1):
        _, per_ref, _ = O.forward(P, x[b:b + 1], y[b:b + 1], oc, np.float32, keep_logits=False)
        d = np.abs(per[b] - per_ref[0])
        say("row", b, "mean", per[b].mean(), per_ref[0].mean(), "max |diff|", d.max())
        assert abs(per[b].mean() - per_ref[0].mean()) <= 2e-3 * per_ref[0].mean()
        assert d.max() <= 0.05
    assert abs(loss - per.mean()) <= 1e-5 * loss


def test_unpadded_vocabulary_and_padding_effect():
    """Vocab 50257 (ragged classifier tiles): loss parity, and with shared
    weights the padded model's loss exceeds the unpadded one by the oracle's
    margin (the softmax of the padded model spans 47 more logits)."""
    B, T = 1, 1024
    res = {}
    for name, pr in (("padded", G124), ("unpadded", G124U)):
        lc, oc, p = configs(pr, B, T)
        x, y = inputs.batch_from_stream(inputs.zipf_stream(0, B * T + 1), B, T)
        m = G.GPT2Step(lc, seed=0)
        loss = m.forward(to_dev(x), to_dev(y))
        m.close()
        lref = O.forward(oracle_init(oc, 0), x, y, oc, np.float32, keep_logits=False)[0]
        say(name, loss, lref)
        assert abs(loss - lref) <= 2e-2 * lref
        res[name] = (loss, lref)
    dg = res["padded"][0] - res["unpadded"][0]
    dr = res["padded"][1] - res["unpadded"][1]
    say("padding margin gpu", dg, "oracle", dr)
    assert dr > 0 and dg > 0
    assert abs(dg - dr) <= 0.3 * dr


def test_accumulated_step_two_micro_steps():
    """Gradient accumulation at the accumulated-step shape (T=512): two
    micro-steps at loss scale 1/2, then clip and AdamW at lr(132) = 6e-4."""
    assert_bf16(*run_step(inputs.PRESETS["gpt2_124m_accum"], 1, 512, seed=0, data_seed=0,
                          lr=O.lr_at(132), dt=np.float32, micro=2))
