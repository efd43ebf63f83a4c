"""Parity cases of the training step against the CPU oracle, each a function
of the backend it runs on: the HIP library on the GPU (tests marked `gpu`)
or the CPU emulation of the same sources (tests/test_emu_*.py).  Shapes are
arguments, so the GPU tests run the workloads at their real sizes and the
emulation runs the same code paths at sizes the CPU finishes quickly.

Tolerances (see gpu_helpers): fp32 path 1e-4 relative on the loss and every
gradient, 1e-3 on the post-AdamW parameters; bf16 path 2e-2 relative on the
loss, per-tensor gradient cosine >= 0.999, post-AdamW 1e-3 where the two
gradients agree in sign and 2 lr + 1e-4 everywhere."""
from __future__ import annotations

import numpy as np
import torch

from decoder_only_transformer_02_amd import gpt2 as G
from decoder_only_transformer_02_amd import inputs
from oracle import gpt2_oracle as O
from tests.gpu_helpers import (Backend, assert_bf16, assert_fp32, check_post_adamw, configs, cosine,
                               gpu_grads, gpu_params, oracle_init, oracle_progress, rel_l2, run_step, say,
                               stream_for)

SMALL_BF16 = dict(n_layer=2, n_head=2, n_embd=128, block_size=128, vocab_size=1000,
                  padded_vocab=1000, compute="bf16", tokens="uniform")
SMALL_FP32 = dict(n_layer=2, n_head=4, n_embd=64, block_size=64, vocab_size=301,
                  padded_vocab=320, compute="fp32", tokens="uniform")
G124 = inputs.PRESETS["gpt2_124m"]
G124U = inputs.PRESETS["gpt2_124m_v50257"]
G124A = inputs.PRESETS["gpt2_124m_accum"]
G124F = inputs.PRESETS["gpt2_124m_fp32"]
SMALL_F16 = {**SMALL_BF16, "compute": "fp16"}


# ---------------------------------------------------------------------------- small configurations

def tiny_fp32_step(be: Backend):
    """Tiny GPT-2-shaped decoder, fp32 throughout, B=4 T=64, seed 0."""
    assert_fp32(*run_step(inputs.PRESETS["tiny"], 4, 64, seed=0, data_seed=0, be=be))


def fp32_ragged_shapes(be: Backend):
    """Ragged M, T and vocabulary tiles; the generic attention kernels."""
    assert_fp32(*run_step(SMALL_FP32, 3, 37, seed=3, data_seed=5, be=be))


def bf16_ragged_mfma_paths(be: Backend):
    """head_dim 64 (matrix-core attention), T=100 (ragged key and query
    tiles), M=300 (ragged GEMM rows and weight-gradient token stages),
    vocabulary 1000 (ragged classifier tiles, unaligned cross-entropy rows)."""
    assert_bf16(*run_step(SMALL_BF16, 3, 100, seed=1, data_seed=2, be=be))


def bf16_accumulation_matches_one_big_batch(be: Backend):
    """4 micro-steps at loss scale 1/4 equal one batch 4x as large."""
    lc, oc, p = configs(SMALL_BF16, 8, 64)
    x, y = inputs.batch_from_stream(stream_for(p, 8 * 64 + 1, 9), 8, 64)
    m = be.make(lc, 0)
    m.forward(be.dev(x), be.dev(y))
    m.backward(1.0)
    names = m.param_names()
    g1 = gpu_grads(m, names)
    m.zero_grad()
    for k in range(4):
        m.forward(be.dev(x[2 * k:2 * k + 2]), be.dev(y[2 * k:2 * k + 2]))
        m.backward(0.25)
    g4 = gpu_grads(m, names)
    m.close()
    for n in names:
        assert cosine(g1[n], g4[n]) >= 0.9999, n


def causality_bitwise(be: Backend, preset: str):
    """Perturbing token t+1 leaves the logits of positions <= t bitwise
    unchanged and changes position t+1."""
    p = SMALL_FP32 if preset == "fp32" else SMALL_BF16
    B, T = 2, 64
    lc, oc, p = configs(p, B, T)
    m = be.make(lc, 0)
    x, _ = inputs.batch_from_stream(stream_for(p, B * T + 1, 4), B, T)
    t = 40
    m.forward(be.dev(x))
    Vp = p["padded_vocab"]
    z0 = m.view("logits")[:B * T, :Vp].clone().view(B, T, -1)
    x2 = x.copy()
    x2[:, t + 1] = (x2[:, t + 1] + 11) % p["vocab_size"]
    m.forward(be.dev(x2))
    z1 = m.view("logits")[:B * T, :Vp].clone().view(B, T, -1)
    m.close()
    assert torch.equal(z0[:, :t + 1], z1[:, :t + 1])
    assert not torch.equal(z0[:, t + 1], z1[:, t + 1])


def determinism_bitwise(be: Backend):
    """Two runs of the same step are bitwise equal (no atomics, fixed
    reduction orders)."""
    outs = []
    for _ in range(2):
        lc, oc, pp = configs(SMALL_BF16, 3, 100)
        x, y = inputs.batch_from_stream(stream_for(pp, 301, 7), 3, 100)
        m = be.make(lc, 0)
        loss = m.forward(be.dev(x), be.dev(y))
        m.backward(1.0)
        norm = m.step(6e-4)
        names = m.param_names()
        outs.append((loss, norm, gpu_grads(m, names), gpu_params(m, names)))
        m.close()
    assert outs[0][0] == outs[1][0] and outs[0][1] == outs[1][1]
    for n in outs[0][2]:
        assert np.array_equal(outs[0][2][n], outs[1][2][n]), n
        assert np.array_equal(outs[0][3][n], outs[1][3][n]), n


def device_init_equals_host_init(be: Backend):
    """gpt2_create's parameters equal gpt2_init_host's bitwise and the
    oracle's within one float32 ulp."""
    lc, oc, p = configs(SMALL_BF16, 2, 16)
    m = be.make(lc, 5)
    flat = np.concatenate([m.view(n).cpu().numpy().ravel() for n in m.param_names()])
    m.close()
    host = G.init_host(lc, 5)
    assert np.array_equal(flat, host)
    ref = np.concatenate([v.ravel() for v in O.init_params(oc, 5).values()])
    assert np.all(np.abs(flat - ref) <= np.spacing(np.abs(ref)))


def error_paths(be: Backend):
    """Out-of-order calls, shapes beyond the arena, ids and targets outside
    the vocabulary, and a non-finite gradient (the update is skipped and the
    parameters stay bitwise unchanged)."""
    import pytest
    lc, oc, p = configs(SMALL_FP32, 2, 16)
    m = be.make(lc, 0)
    x, y = inputs.batch_from_stream(stream_for(p, 33, 1), 2, 16)
    with pytest.raises(G.GPT2Error) as e:
        m.backward(1.0)
    assert e.value.status == G.GPT2_E_STATE
    with pytest.raises(G.GPT2Error) as e:
        m.step(1e-3)
    assert e.value.status == G.GPT2_E_STATE
    with pytest.raises(G.GPT2Error) as e:
        m.forward(be.dev(np.zeros((3, 16), np.int32)), be.dev(np.zeros((3, 16), np.int32)))
    assert e.value.status == G.GPT2_E_SHAPE
    bad = x.copy()
    bad[1, 3] = p["vocab_size"]
    with pytest.raises(G.GPT2Error) as e:
        m.forward(be.dev(bad), be.dev(y))
    assert e.value.status == G.GPT2_E_TOKEN
    badt = y.copy()
    badt[0, 0] = -1
    with pytest.raises(G.GPT2Error) as e:
        m.forward(be.dev(x), be.dev(badt))
    assert e.value.status == G.GPT2_E_TOKEN
    m.forward(be.dev(x), be.dev(y))
    m.backward(1.0)
    before = {n: m.view(n).clone() for n in m.param_names()}
    m.view("grad.h0.fc.w")[0, 0] = float("nan")
    with pytest.raises(G.GPT2Error) as e:
        m.step(1e-3)
    assert e.value.status == G.GPT2_E_NONFINITE
    for n in before:
        assert torch.equal(before[n], m.view(n)), n
    loss = m.forward(be.dev(x), be.dev(y))
    m.backward(1.0)
    assert np.isfinite(m.step(1e-3)) and np.isfinite(loss)
    m.close()


def overfit_single_batch_tracks_oracle(be: Backend, steps: int = 25):
    """The chapter "optimization loop: overfit a single batch": repeated steps
    on one tiny fp32 batch; the loss curve follows the oracle's."""
    lc, oc, p = configs(inputs.PRESETS["tiny"], 4, 64)
    x, y = inputs.batch_from_stream(stream_for(p, 257, 0), 4, 64)
    m = be.make(lc, 0)
    gl = []
    for _ in range(steps):
        gl.append(m.forward(be.dev(x), be.dev(y)))
        m.backward(1.0)
        m.step(1e-3)
    m.close()
    P = oracle_init(oc, 0)
    Ms = Vs = None
    ol = []
    for t in range(1, 6):
        r = O.train_step(P, [(x, y)], oc, lr=1e-3, clip=1.0, t=t, M_state=Ms, V_state=Vs)
        ol.append(r["loss"])
        P, Ms, Vs = r["params"], r["m"], r["v"]
    say("library", gl[:5], "oracle", ol)
    for a, b in zip(gl[:5], ol):
        assert abs(a - b) <= 1e-4 * abs(b)
    assert gl[-1] < gl[0] - 1.0


def checkpoint_resume_bitwise(be: Backend, preset: str):
    """Save after two steps (parameters, both moments, step count through the
    tensor table), restore into a fresh context created from another seed,
    and the third step of both is bitwise the same: loss, norm, parameters,
    moments and the step count."""
    p = SMALL_FP32 if preset == "fp32" else SMALL_BF16
    B, T = 2, 32
    lc, oc, p = configs(p, B, T)
    s = stream_for(p, 3 * B * T + 1, 11)
    batches = [inputs.batch_from_stream(s, B, T, k) for k in range(3)]
    a = be.make(lc, 0)
    for x, y in batches[:2]:
        a.forward(be.dev(x), be.dev(y))
        a.backward(1.0)
        a.step(1e-3)
    sd = a.state_dict()
    assert sd["__step__"] == 2
    x, y = batches[2]
    la = a.forward(be.dev(x), be.dev(y))
    a.backward(1.0)
    na = a.step(1e-3)
    ra = a.state_dict()
    a.check_arena()
    a.close()
    b = be.make(lc, 7)
    b.load_state_dict(sd)
    lb = b.forward(be.dev(x), be.dev(y))
    b.backward(1.0)
    nb = b.step(1e-3)
    rb = b.state_dict()
    b.check_arena()
    b.close()
    assert la == lb and na == nb
    assert ra["__step__"] == rb["__step__"] == 3
    for n in ra:
        if n != "__step__":
            assert torch.equal(ra[n], rb[n]), n


def arena_guard_detects_overrun(be: Backend):
    """The guards after the arena regions are intact after a step, and one
    byte changed right after a region's end is reported, naming the region."""
    import pytest
    lc, oc, p = configs(SMALL_BF16, 2, 16)
    m = be.make(lc, 0)
    x, y = inputs.batch_from_stream(stream_for(p, 33, 3), 2, 16)
    m.forward(be.dev(x), be.dev(y))
    m.backward(1.0)
    m.step(1e-3)
    m.check_arena()
    t = m.tensors["losses"]
    end = t["offset"] + t["bytes"]
    m.arena[end + 5] = 0
    with pytest.raises(G.GPT2Error) as e:
        m.check_arena()
    assert e.value.status == G.GPT2_E_ARENA and "losses" in str(e.value)
    m.close()


def weight_copies_follow_weights(be: Backend, preset: str):
    """Every 16-bit GEMM weight copy (which the forward and the dX GEMMs both
    read, the latter in place as a [k][n] operand) is bitwise its fp32
    parameter rounded to nearest even, right after create and after each
    optimizer step (AdamW writes the copy with the parameter)."""
    p = SMALL_F16 if preset == "fp16" else SMALL_BF16
    tt = torch.float16 if preset == "fp16" else torch.bfloat16
    lc, oc, p = configs(p, 2, 24)
    m = be.make(lc, 0)
    names = [n[5:] for n in m.tensors if n.startswith("bf16.")]
    assert names and len(names) == 4 * p["n_layer"] + 1, names

    def check():
        for n in names:
            w16 = m.view("bf16." + n).cpu()
            w = m.view(n).cpu()
            assert w16.dtype == tt and w16.shape == w.shape, n
            assert torch.equal(w16.view(torch.int16), w.to(tt).view(torch.int16)), n

    check()
    for k in range(2):
        x, y = inputs.batch_from_stream(stream_for(p, 2 * 24 + 1, 11 + k), 2, 24)
        m.forward(be.dev(x), be.dev(y))
        m.backward(1.0)
        m.step(1e-2)
        check()
    m.check_arena()
    m.close()


def eval_loss_forward_only(be: Backend, preset: str):
    """gpt2_eval_loss gives the forward's loss bitwise, leaves the raw logits
    in place (bitwise those of a forward without targets), does not arm
    backward, disarms a backward armed before, and matches the oracle."""
    import pytest
    p = SMALL_FP32 if preset == "fp32" else SMALL_BF16
    B, T = 3, 40
    lc, oc, p = configs(p, B, T)
    x, y = inputs.batch_from_stream(stream_for(p, B * T + 1, 6), B, T)
    m = be.make(lc, 0)
    m.forward(be.dev(x))
    z_raw = m.view("logits")[:B * T].clone()
    l_fwd = m.forward(be.dev(x), be.dev(y))
    l_eval = m.eval_loss(be.dev(x), be.dev(y))
    assert l_eval == l_fwd
    assert torch.equal(m.view("logits")[:B * T], z_raw)
    with pytest.raises(G.GPT2Error) as e:
        m.backward(1.0)
    assert e.value.status == G.GPT2_E_STATE
    m.check_arena()
    m.close()
    ref = O.eval_loss(oracle_init(oc, 0), x, y, oc)
    tol = 1e-4 if preset == "fp32" else 2e-2
    assert abs(l_eval - ref) <= tol * ref


def generate_matches_oracle(be: Backend, preset: str, B: int = 2, T0: int = 7, T: int = 48, n_layer=None):
    """Sampling with the key/value cache against the oracle by teacher
    forcing: one oracle forward over the generated sequence gives the logits
    before every new token; the token must be the oracle's inverse-CDF pick
    at the step's draw, or lie within `band` of a cumulative-probability
    boundary (floating point may then decide either way), and its
    log-probability must match.  The library's own full forward over the
    output agrees with the cached decode path too.  Prefix unchanged."""
    p = {"fp32": SMALL_FP32, "bf16": SMALL_BF16, "124m": G124}[preset]
    band, lp_tol = (1e-5, 1e-4) if preset == "fp32" else (2e-2, 5e-2)
    over = {} if n_layer is None else {"n_layer": n_layer}
    lc, oc, p = configs(p, B, T, **over)
    rng = np.random.default_rng(12)
    tok = np.zeros((B, T), np.int32)
    tok[:, :T0] = stream_for(p, B * T0, 8).reshape(B, T0)
    u = rng.random((B, T - T0)).astype(np.float32)
    m = be.make(lc, 0)
    td = be.dev(tok)
    lpd = be.dev(np.zeros((B, T - T0), np.float32))
    m.generate(td, T0, be.dev(u), lpd)
    out = td.cpu().numpy()
    lp = lpd.cpu().numpy().astype(np.float64)
    m.forward(be.dev(out))
    z_lib = m.view("logits")[:B * T, :p["padded_vocab"]].double().cpu().numpy().reshape(B, T, -1)
    m.check_arena()
    m.close()
    assert np.array_equal(out[:, :T0], tok[:, :T0])
    assert out.min() >= 0 and out.max() < p["vocab_size"]
    _, _, cache = O.forward(oracle_init(oc, 0), out.astype(np.int64), None, oc,
                            np.float32 if preset == "124m" else np.float64)
    z = cache["z"].reshape(B, T, -1)
    exact = 0
    for b in range(B):
        for t in range(T0, T):
            zr = z[b, t - 1, :p["vocab_size"]]
            e = np.exp(zr - zr.max())
            c = np.cumsum(e) / e.sum()
            v = int(out[b, t])
            uu = float(u[b, t - T0])
            lo = c[v - 1] if v > 0 else 0.0
            assert lo - band <= uu < c[v] + band, (b, t, v, lo, c[v], uu)
            exact += int(O.sample_token(zr, uu, p["vocab_size"])[0] == v)
            ref_lp = float(np.log(e[v] / e.sum()))
            assert abs(lp[b, t - T0] - ref_lp) <= lp_tol, (b, t, lp[b, t - T0], ref_lp)
            zl = z_lib[b, t - 1, :p["vocab_size"]]
            el = np.exp(zl - zl.max())
            assert abs(lp[b, t - T0] - float(np.log(el[v] / el.sum()))) <= lp_tol
    say(f"[{be.name}] generate {preset}: {exact} of {B * (T - T0)} picks equal the oracle's")
    # fp32: nearly every pick is the oracle's.  bf16: logit rounding moves
    # cumulative boundaries by up to ~1e-3, and with 50257 near-uniform ids
    # (intervals ~2e-5 wide) a fair share of picks may then differ; a wrong
    # distribution would still match almost none.
    assert exact >= (0.9 if preset == "fp32" else 0.5) * B * (T - T0)


def fp16_ragged_step(be: Backend):
    """fp16 operands with dynamic loss scaling (scale 65536 at create) on the
    ragged configuration: the bf16 tolerances apply (fp16 has more mantissa
    bits, the loss scale keeps small gradients representable)."""
    assert_bf16(*run_step(SMALL_F16, 3, 100, seed=1, data_seed=2, be=be))


def fp16_loss_scaler(be: Backend):
    """The dynamic loss scale: 65536 at create; an overflow (scale 2^40
    makes the fp16 gradients non-finite) skips the step on the device
    (parameters, moments and step count bitwise unchanged, norm reported as
    +inf, status OK) and halves the scale; after `growth_interval` finite
    steps the scale doubles; and two finite scales give the same update up
    to fp16 rounding (scaling is divided out)."""
    lc, oc, p = configs(SMALL_F16, 2, 32)
    x, y = inputs.batch_from_stream(stream_for(p, 65, 3), 2, 32)
    m = be.make(lc, 0)
    assert m.loss_scale() == 65536.0
    m.set_loss_scale(2.0 ** 40, 2000)
    before = {n: v.clone() for n, v in m.state_dict().items() if n != "__step__"}
    m.forward(be.dev(x), be.dev(y))
    m.backward(1.0)
    assert m.step(1e-3) == float("inf")
    after = m.state_dict()
    assert after["__step__"] == 0
    for n in before:
        assert torch.equal(before[n], after[n]), n
    assert m.loss_scale() == 2.0 ** 39
    m.set_loss_scale(256.0, 2)
    norms = []
    for k in range(3):
        m.forward(be.dev(x), be.dev(y))
        m.backward(1.0)
        norms.append(m.step(1e-3))
    assert all(np.isfinite(norms))
    assert m.loss_scale() == 512.0 and m.step_count() == 3
    m.check_arena()
    m.close()
    outs = []
    for S in (256.0, 4096.0):
        m = be.make(lc, 0)
        m.set_loss_scale(S, 2000)
        m.forward(be.dev(x), be.dev(y))
        m.backward(1.0)
        nrm = m.step(1e-3)
        names = m.param_names()
        outs.append((nrm, gpu_params(m, names)))
        m.close()
    assert abs(outs[0][0] - outs[1][0]) <= 1e-2 * outs[1][0]
    for n in outs[0][1]:
        assert np.abs(outs[0][1][n] - outs[1][1][n]).max() <= 2 * 1e-3 + 1e-6, n


# ---------------------------------------------------------------------------- GPT-2 124M shapes

def block_124m(be: Backend, B: int = 16, T: int = 1024):
    """One 124M block in isolation, bf16: x ~ N(0,1), dy ~ N(0, 1e-3^2);
    y (relative L2 2e-2, cosine 0.999), dx and the 12 block gradients
    (cosine 0.999) against the oracle in float32 storage."""
    C = 768
    lc, oc, p = configs(inputs.PRESETS["block124m"], B, T)
    x, dy = inputs.block_inputs(0, B, T, C)
    say(f"[{be.name}] block 124m B={B} T={T}")
    m = be.make(lc, 0)
    y, dx = m.block_fwd_bwd(0, be.dev(x), be.dev(dy))
    y = y.cpu().numpy()
    dx = dx.cpu().numpy()
    names = [n for n in m.param_names() if n.startswith("h0.")]
    gg = gpu_grads(m, names)
    m.check_arena()
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


def _one_sequence_batches(x, y):
    return [(x[b:b + 1], y[b:b + 1]) for b in range(x.shape[0])]


def full_step_vs_oracle(be: Backend, preset: dict, B: int, T: int, lr: float = 6e-4, n_layer=None,
                        compute=None):
    """A whole step (forward, backward, clip, AdamW) of B sequences of T
    Zipf ids in ONE forward/backward of the library, against the oracle's
    step over the same B sequences taken as B one-sequence micro-batches at
    loss scale 1/B, which equals the one-batch step exactly (gradient
    accumulation is linear; pinned on the CPU).  Loss 2e-2, per-tensor
    gradient cosine 0.999, post-AdamW rule."""
    over = {} if n_layer is None else {"n_layer": n_layer}
    if compute:
        over["compute"] = compute
    lc, oc, p = configs(preset, B, T, **over)
    x, y = inputs.batch_from_stream(stream_for(p, B * T + 1, 0), B, T)
    say(f"[{be.name}] full step layers={p['n_layer']} V={p['vocab_size']}/{p['padded_vocab']} B={B} T={T} "
        f"{p['compute']}")
    m = be.make(lc, 0)
    loss = m.forward(be.dev(x), be.dev(y))
    per = m.view("losses")[:B * T].cpu().numpy()
    m.backward(1.0)
    names = m.param_names()
    norm = m.step(lr, 1.0)
    gg = gpu_grads(m, names)
    pp = gpu_params(m, names)
    m.check_arena()
    m.close()
    assert abs(loss - float(np.mean(per, dtype=np.float64))) <= 1e-5 * loss
    ref = O.train_step(oracle_init(oc, 0), _one_sequence_batches(x, y), oc, lr=lr, clip=1.0, t=1,
                       dt=np.float32, progress=oracle_progress(f"B={B} T={T}"))
    assert_bf16(loss, norm, gg, pp, ref, lr=lr)


def full_step_fp32_vs_oracle(be: Backend, B: int, T: int, n_layer=None):
    """The whole step in fp32 throughout at the 124M width (the GEMMs on the
    fp32 matrix cores from 2^27 multiply-adds up): loss and norm within
    1e-4 relative, every gradient within 1e-4 relative L2, and the
    post-AdamW rule with 1e-3 where the gradients agree in sign (at 124M
    some near-zero gradients may differ in sign even in fp32; they must be
    under 0.1 % of the elements)."""
    over = {} if n_layer is None else {"n_layer": n_layer}
    lc, oc, p = configs(G124F, B, T, **over)
    x, y = inputs.batch_from_stream(stream_for(p, B * T + 1, 0), B, T)
    say(f"[{be.name}] fp32 full step layers={p['n_layer']} B={B} T={T}")
    m = be.make(lc, 0)
    loss = m.forward(be.dev(x), be.dev(y))
    m.backward(1.0)
    names = m.param_names()
    norm = m.step(6e-4, 1.0)
    gg = gpu_grads(m, names)
    pp = gpu_params(m, names)
    m.check_arena()
    m.close()
    ref = O.train_step(oracle_init(oc, 0), _one_sequence_batches(x, y), oc, lr=6e-4, clip=1.0, t=1,
                       dt=np.float32, progress=oracle_progress(f"fp32 B={B} T={T}"))
    say("loss", loss, ref["loss"], "norm", norm, ref["norm"])
    assert abs(loss - ref["loss"]) <= 1e-4 * ref["loss"]
    assert abs(norm - ref["norm"]) <= 1e-4 * ref["norm"]
    worst = max((rel_l2(gg[n], ref["grads"][n]), n) for n in ref["grads"])
    say("worst gradient relative L2", worst)
    assert worst[0] <= 1e-4, worst
    flips = check_post_adamw(pp, ref["params"], gg, ref["grads"], 6e-4, exact=False)
    say("sign-disagreement fraction", flips)
    assert flips < 1e-3


def accumulated_step_vs_oracle(be: Backend, B: int = 32, T: int = 512, micro: int = 2, n_layer=None):
    """The accumulated optimizer step's shape (B=32, T=512 micro-batches, Zipf
    ids, lr(132) = 6e-4, fresh optimizer t = 1) with `micro` real micro-steps
    at loss scale 1/micro, against the oracle over the same micro*B
    sequences as one-sequence micro-batches at scale 1/(micro*B)."""
    over = {} if n_layer is None else {"n_layer": n_layer}
    lc, oc, p = configs(G124A, B, T, **over)
    lr = O.lr_at(132)
    s = stream_for(p, micro * B * T + 1, 0)
    batches = [inputs.batch_from_stream(s, B, T, k) for k in range(micro)]
    say(f"[{be.name}] accumulated step layers={p['n_layer']} B={B} T={T} micro={micro} lr={lr}")
    m = be.make(lc, 0)
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
    seqs = []
    for x, y in batches:
        seqs += _one_sequence_batches(x, y)
    ref = O.train_step(oracle_init(oc, 0), seqs, oc, lr=lr, clip=1.0, t=1, dt=np.float32,
                       progress=oracle_progress(f"{micro} x B={B} T={T}"))
    assert_bf16(float(np.mean(losses)), norm, gg, pp, ref, lr=lr)


def _flat_grads(m):
    """One view over the whole fp32 gradient array (every tensor, canonical
    order, as the arena lays them out)."""
    t0 = m.tensors["grad.wte"]
    last = max((t for n, t in m.tensors.items() if t["kind"] == "grad"), key=lambda t: t["offset"])
    nbytes = last["offset"] + last["bytes"] - t0["offset"]
    return m.arena[t0["offset"]:t0["offset"] + nbytes].view(torch.float32)


def accumulation_equals_sum_of_micro_steps(be: Backend, B: int = 32, T: int = 512, micro: int = 32,
                                           n_layer=None):
    """The full accumulated step: `micro` micro-steps at scale 1/micro
    accumulate (beta = 1 after the first) to the sum of the micro-steps'
    gradients each computed alone; cosine >= 0.99999 and relative L2
    <= 1e-4 over the whole gradient."""
    over = {} if n_layer is None else {"n_layer": n_layer}
    lc, oc, p = configs(G124A, B, T, **over)
    s = stream_for(p, micro * B * T + 1, 0)
    m = be.make(lc, 0)
    say(f"[{be.name}] accumulation sum layers={p['n_layer']} B={B} T={T} micro={micro}")
    total = None
    for k in range(micro):
        x, y = inputs.batch_from_stream(s, B, T, k)
        m.zero_grad()
        m.forward(be.dev(x), be.dev(y))
        m.backward(1.0 / micro)
        g = _flat_grads(m).double()
        total = g.clone() if total is None else total + g
    m.zero_grad()
    for k in range(micro):
        x, y = inputs.batch_from_stream(s, B, T, k)
        m.forward(be.dev(x), be.dev(y))
        m.backward(1.0 / micro)
    acc = _flat_grads(m).double()
    m.close()
    cos = float((acc @ total) / (acc.norm() * total.norm()))
    rl = float((acc - total).norm() / total.norm())
    say("accumulated vs summed: cosine", cos, "rel L2", rl)
    assert cos >= 0.99999 and rl <= 1e-4


def step_124m_one_sequence(be: Backend, T: int = 1024):
    """Full 124M step (vocabulary 50304, Zipf ids), one sequence, against the
    whole oracle step (float32 storage, float64 reductions)."""
    assert_bf16(*run_step(G124, 1, T, seed=0, data_seed=0, dt=np.float32, be=be))


def unpadded_vocabulary_and_padding_effect(be: Backend, T: int = 1024, n_layer=None):
    """Vocabulary 50257 (ragged classifier tiles): loss parity, and with
    shared weights the padded model's loss exceeds the unpadded one by the
    oracle's margin (its softmax spans 47 more logits)."""
    B = 1
    res = {}
    over = {} if n_layer is None else {"n_layer": n_layer}
    for name, pr in (("padded", G124), ("unpadded", G124U)):
        lc, oc, p = configs(pr, B, T, **over)
        x, y = inputs.batch_from_stream(inputs.zipf_stream(0, B * T + 1), B, T)
        m = be.make(lc, 0)
        loss = m.forward(be.dev(x), be.dev(y))
        m.close()
        lref = O.forward(oracle_init(oc, 0), x, y, oc, np.float32, keep_logits=False)[0]
        say(name, loss, lref)
        assert abs(loss - lref) <= 2e-2 * lref
        res[name] = (loss, lref)
    dg = res["padded"][0] - res["unpadded"][0]
    dr = res["padded"][1] - res["unpadded"][1]
    say("padding margin library", dg, "oracle", dr)
    assert dr > 0 and dg > 0
    assert abs(dg - dr) <= 0.3 * dr


def full_batch_rows_and_determinism(be: Backend, B: int = 16, T: int = 1024, n_layer=None):
    """The benchmark's launch configuration: per-position losses of sampled
    rows equal the oracle's forward of those rows alone; each
    logits-gradient row sums to zero; two whole steps are bitwise equal."""
    over = {} if n_layer is None else {"n_layer": n_layer}
    lc, oc, p = configs(G124, B, T, **over)
    x, y = inputs.batch_from_stream(inputs.zipf_stream(0, B * T + 1), B, T)
    runs = []
    for rep in range(2):
        m = be.make(lc, 0)
        loss = m.forward(be.dev(x), be.dev(y))
        per = m.view("losses")[:B * T].cpu().numpy().reshape(B, T)
        dz = m.view("logits")[:B * T]
        rows = torch.tensor([0, (B * T) // 2 + 1, B * T - 1], device=m.device)
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
