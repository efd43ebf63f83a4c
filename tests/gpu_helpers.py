"""Shared helpers of the parity tests: configuration pairs for the library
and the oracle, running one step through the C ABI on a backend (the HIP
library on the GPU, or its CPU emulation), and the comparison measures with
the tolerances of the two arithmetic paths."""
from __future__ import annotations

import functools
import sys
import time

import numpy as np

from decoder_only_transformer_02_amd import gpt2 as G
from decoder_only_transformer_02_amd import inputs
from oracle import gpt2_oracle as O


# pytest's config, set by conftest.py: lets say() write past output capture.
PYTEST_CONFIG = None


def say(*a):
    """Print a progress line on the real stdout, also while pytest captures
    the test's output (a run without -s still shows that a long oracle
    computation is advancing)."""
    capman = PYTEST_CONFIG.pluginmanager.getplugin("capturemanager") if PYTEST_CONFIG else None
    if capman is not None:
        with capman.global_and_fixture_disabled():
            print(*a, flush=True)
    else:
        print(*a, flush=True)
    sys.stdout.flush()


def oracle_progress(label: str):
    """A train_step progress callback: a line per oracle micro-batch once the
    computation has run for more than 5 s (short ones stay quiet)."""
    t0 = time.perf_counter()

    def report(i, k):
        dt = time.perf_counter() - t0
        if dt > 5.0:
            say(f"  oracle {label}: micro-batch {i + 1}/{k} done, {dt:.0f} s")
    return report


def configs(p: dict, B: int, T: int, **over):
    p = {**p, **over}
    lc = G.make_config(**{**p, "max_batch": B, "max_seq": T})
    oc = O.Config(p["n_layer"], p["n_head"], p["n_embd"], p["block_size"], p["vocab_size"],
                  p["padded_vocab"])
    return lc, oc, p


@functools.lru_cache(maxsize=4)
def oracle_init(oc: O.Config, seed: int):
    return O.init_params(oc, seed)


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


class Backend:
    """Where the library runs: `make(cfg, seed)` returns a GPT2Step-like
    context and `dev(array)` moves an input array to that backend."""

    def __init__(self, name, make, dev):
        self.name, self.make, self.dev = name, make, dev


GPU = Backend("gpu", lambda cfg, seed: G.GPT2Step(cfg, seed=seed), to_dev)


def emu_backend() -> Backend:
    import torch
    from tests.emu.binding import EmuStep
    return Backend("emu", lambda cfg, seed: EmuStep(cfg, seed=seed),
                   lambda a: torch.from_numpy(np.ascontiguousarray(a)))


def gpu_grads(m: G.GPT2Step, names):
    return {n: m.view("grad." + n).double().cpu().numpy() for n in names}


def gpu_params(m: G.GPT2Step, names):
    return {n: m.view(n).double().cpu().numpy() for n in names}


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def rel_l2(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_post_adamw(new_gpu, new_ref, g_gpu, g_ref, lr, exact: bool):
    """fp32 path: max |diff| <= 1e-3 everywhere.  bf16 path: <= 1e-3 where the
    two gradients agree in sign, <= 2 lr + 1e-4 everywhere (the first AdamW
    step moves each weight by about lr * sign(g)).  Returns the fraction of
    sign disagreements."""
    flips = 0
    total = 0
    for n in new_ref:
        d = np.abs(new_gpu[n] - new_ref[n].astype(np.float64))
        if exact:
            assert d.max() <= 1e-3, (n, d.max())
            continue
        same = np.sign(g_gpu[n]) == np.sign(g_ref[n])
        flips += int((~same).sum())
        total += same.size
        if same.any():
            assert d[same].max() <= 1e-3, (n, d[same].max())
        assert d.max() <= 2 * lr + 1e-4, (n, d.max())
    return flips / max(total, 1)


def stream_for(p, n, seed):
    if p["tokens"] == "zipf":
        return inputs.zipf_stream(seed, n, p["vocab_size"])
    return inputs.uniform_stream(seed, n, p["vocab_size"])


def run_step(p, B, T, seed=0, data_seed=1, lr=6e-4, dt=np.float64, micro=1, be: Backend = GPU):
    """One optimizer step of `micro` micro-batches (B, T) through the C ABI on
    backend `be`, and the oracle's step on the same seeded inputs.  Returns
    (mean micro loss, pre-clip norm, gradients, post-step parameters, oracle
    result)."""
    lc, oc, p = configs(p, B, T)
    s = stream_for(p, B * T * micro + 1, data_seed)
    batches = [inputs.batch_from_stream(s, B, T, k) for k in range(micro)]
    say(f"case [{be.name}] layers={p['n_layer']} C={p['n_embd']} V={p['vocab_size']}/{p['padded_vocab']} "
        f"B={B} T={T} micro={micro} {p['compute']}")
    m = be.make(lc, seed)
    losses = []
    for x, y in batches:
        losses.append(m.forward(be.dev(x), be.dev(y)))
        m.backward(1.0 / micro)
    names = m.param_names()
    norm = m.step(lr, 1.0)
    gg = gpu_grads(m, names)
    pp = gpu_params(m, names)
    m.check_arena()
    m.close()
    P = oracle_init(oc, seed)
    ref = O.train_step(P, batches, oc, lr=lr, clip=1.0, t=1, dt=dt, progress=oracle_progress("step"))
    return float(np.mean(losses)), norm, gg, pp, ref


def assert_fp32(loss, norm, gg, pp, ref, lr=6e-4):
    """The fp32 path: loss and norm within 1e-4 relative, every gradient
    within 1e-4 relative L2, post-AdamW parameters within 1e-3."""
    say("loss", loss, ref["loss"], "norm", norm, ref["norm"])
    assert abs(loss - ref["loss"]) <= 1e-4 * abs(ref["loss"])
    assert abs(norm - ref["norm"]) <= 1e-4 * ref["norm"]
    for n in ref["grads"]:
        assert rel_l2(gg[n], ref["grads"][n]) <= 1e-4, (n, rel_l2(gg[n], ref["grads"][n]))
    check_post_adamw(pp, ref["params"], gg, ref["grads"], lr, exact=True)


def assert_bf16(loss, norm, gg, pp, ref, lr=6e-4):
    """The bf16 path: loss within 2e-2 relative, per-tensor gradient cosine
    >= 0.999, the post-AdamW rule of check_post_adamw; the pre-clip norm
    within 5e-2 relative is a looser extra check."""
    say("loss", loss, ref["loss"], "norm", norm, ref["norm"])
    assert abs(loss - ref["loss"]) <= 2e-2 * abs(ref["loss"])
    assert abs(norm - ref["norm"]) <= 5e-2 * ref["norm"]
    worst = min((cosine(gg[n], ref["grads"][n]), n) for n in ref["grads"])
    say("worst gradient cosine", worst)
    assert worst[0] >= 0.999, worst
    flips = check_post_adamw(pp, ref["params"], gg, ref["grads"], lr, exact=False)
    say("sign-disagreement fraction", flips)
    assert flips < 0.01
