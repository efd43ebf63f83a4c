"""Throughput of one GPT-2 124M training step (forward, backward, global-norm
clip, AdamW) at B=16, T=1024, bf16, on one MI355X, through the C ABI.

Prints one JSON line:
  * value: tokens/s of the whole job (wall clock over exactly `--steps`
    steps between two device synchronizations), ms/step (mean), and the
    median / p10 / p90 of per-step HIP-event times on the library stream;
  * mfu: (6N + 6 L C (T+1)) flops per token against the bf16 dense peak;
  * roofline: the dominant kernel (the classifier forward GEMM), its
    algorithmic flops over its launch time, from HIP events around each of
    its launches during the timed steps;
  * kernels: every timing class of the library with its algorithmic work
    per step (the scope table's per-unit figures times the units of one
    step), its time per step and its fraction of the MI355X roofline;
  * padding: the classifier GEMMs + cross-entropy and the whole step at the
    unpadded vocabulary 50257 against the padded 50304;
  * accumulated_step: one optimizer step of 32 micro-steps of B=32, T=512
    (524,288 tokens) with clip and AdamW at lr(132), median of 10;
  * block: one transformer block's forward and backward alone at B=16,
    T=1024, median of 20;
  * cpu_baseline: the CPU oracle on a bounded sample of the same workload.
Inputs are resident in device memory before every timed region.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15     # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12      # MI355X HBM3E, bytes/s
METRIC = "train tokens/sec + ms/step, GPT-2 124M B=16 T=1024 bf16; MFU vs peak"


def flops_per_token(L, C, T, n_nonemb):
    """6N + 6 L C (T + 1): causal attention scores counted once per (i <= j)."""
    return 6 * n_nonemb + 6 * L * C * (T + 1)


def percentile(xs, q):
    """Linear-interpolation percentile (q in [0, 100]) of a non-empty list."""
    s = sorted(xs)
    if len(s) == 1:
        return s[0]
    pos = (len(s) - 1) * q / 100.0
    lo = int(pos)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (pos - lo)


def class_work(p, B, T, n_params):
    """Algorithmic work of one training step per timing class: (bound, amount,
    unit) with flops for matrix-core classes and bytes for bandwidth classes.

    GEMMs: 2 M K N per product; per layer the four weight products
    (3C, C, 4C, 4C outputs of widths C, C, C, 4C) three times (forward, dX,
    dW), plus the classifier (M x Vp x C) three times.  Attention: 4 hd flops
    per causal score (QK^T and PV) forward, twice that backward (recompute
    not credited).  LayerNorm forward (6C+8) and backward (14C+8) bytes per
    token over 2L+1 LayerNorms; cross-entropy (4 Vp + 8) bytes per token;
    gradient norm 4 bytes and AdamW 30 bytes per parameter."""
    L, C, H, Vp = p["n_layer"], p["n_embd"], p["n_head"], p["padded_vocab"]
    M = B * T
    hd = C // H
    gemm = 3 * 2 * M * (L * 12 * C * C + Vp * C)
    lm = 2 * M * Vp * C
    attn = L * B * H * (T * (T + 1) // 2) * hd * 4
    return {
        "lmhead_fwd": ("mfma", lm, "flop"),
        "gemm": ("mfma", gemm, "flop"),
        "attn_fwd": ("mfma", attn, "flop"),
        "attn_bwd": ("mfma", 2 * attn, "flop"),
        "ln_fwd": ("hbm", (2 * L + 1) * M * (6 * C + 8), "byte"),
        "ln_bwd": ("hbm", (2 * L + 1) * M * (14 * C + 8), "byte"),
        "xent": ("hbm", M * (4 * Vp + 8), "byte"),
        "norm": ("hbm", 4 * n_params, "byte"),
        "adamw": ("hbm", 30 * n_params, "byte"),
    }


def roofline_entry(bound, work, ms):
    """Achieved rate and fraction of the MI355X peak for `work` done in `ms`."""
    if bound == "mfma":
        ach = work / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": round(ach * 1e12 / PEAK_BF16, 4)}
    ach = work / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(ach * 1e9 / PEAK_HBM, 4)}


def cpu_baseline(preset, n_seq=2):
    """The oracle as it stands, one full step of the same model on `n_seq`
    sequences of T tokens (a bounded sample of the benchmark batch, taken as
    one-sequence micro-batches, as the parity tests take it)."""
    import numpy as np
    from decoder_only_transformer_02_amd import inputs
    from oracle import gpt2_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas_threads = None
    oc = O.Config(preset["n_layer"], preset["n_head"], preset["n_embd"], preset["block_size"],
                  preset["vocab_size"], preset["padded_vocab"])
    P = O.init_params(oc, 0)
    T = preset["T"]
    x, y = inputs.batch_from_stream(inputs.zipf_stream(0, n_seq * T + 1, preset["vocab_size"]), n_seq, T)
    t0 = time.perf_counter()
    O.train_step(P, [(x[b:b + 1], y[b:b + 1]) for b in range(n_seq)], oc, lr=6e-4, clip=1.0, t=1,
                 dt=np.float32)
    dt = time.perf_counter() - t0
    cores = blas_threads or len(os.sched_getaffinity(0))
    return {"value": round(n_seq * T / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one full step (forward, backward, clip, AdamW) of the same model on {n_seq} sequences "
                      f"of {T} tokens ({n_seq}/{preset['B']} of the benchmark batch), float32 storage with "
                      f"float64 reductions, {dt:.1f} s; host has {os.cpu_count()} CPUs, "
                      f"{len(os.sched_getaffinity(0))} in this process's affinity, BLAS threads "
                      f"{blas_threads}"}


def block_leg(G, inputs, torch, runs=20, warmup=3):
    """One transformer block in isolation (forward and backward of layer 0,
    bf16): the median of `runs` HIP-event timed calls, with its algorithmic
    work: the 12 GEMMs (3 x 2 M 12 C^2) and the causal attention forward and
    backward (3 x 4 hd flops per score, T(T+1)/2 scores per head)."""
    pb = inputs.PRESETS["block124m"]
    B, T, C, H = pb["B"], pb["T"], pb["n_embd"], pb["n_head"]
    cfg = G.make_config(**{**pb, "max_batch": B, "max_seq": T})
    m = G.GPT2Step(cfg, seed=0)
    x, dy = inputs.block_inputs(0, B, T, C)
    x = torch.from_numpy(x).cuda()
    dy = torch.from_numpy(dy).cuda()
    for _ in range(warmup):
        m.block_fwd_bwd(0, x, dy)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for a, b in ev:
        a.record()
        m.block_fwd_bwd(0, x, dy)
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    m.close()
    torch.cuda.synchronize()
    M = B * T
    gemm = 3 * 2 * M * 12 * C * C
    attn = 3 * B * H * (T * (T + 1) // 2) * (C // H) * 4
    med = percentile(ms, 50)
    e = roofline_entry("mfma", gemm + attn, med)
    return {"workload": f"one 124M block, forward and backward, B={B}, T={T}, bf16", "runs": runs,
            "ms_median": round(med, 4), "ms_p10": round(percentile(ms, 10), 4),
            "ms_p90": round(percentile(ms, 90), 4), "flops": gemm + attn, "tokens_per_s": round(M / (med * 1e-3), 1),
            "achieved_tflops": e["achieved"], "frac_of_bf16_peak": e["frac"]}


class Runner:
    """One library context with device-resident inputs of a preset."""

    def __init__(self, G, inputs, torch, preset, micro=1):
        self.torch = torch
        self.p = preset
        self.B, self.T = preset["B"], preset["T"]
        cfg = G.make_config(**{**preset, "max_batch": self.B, "max_seq": self.T})
        self.cfg = cfg
        self.m = G.GPT2Step(cfg, seed=0)
        n = self.B * self.T
        s = inputs.zipf_stream(0, n * micro + 1, preset["vocab_size"])
        self.batches = []
        for k in range(micro):
            x, y = inputs.batch_from_stream(s, self.B, self.T, k)
            self.batches.append((torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()))
        torch.cuda.synchronize()

    def step(self, lr=6e-4):
        k = len(self.batches)
        for x, y in self.batches:
            self.m.forward(x, y, sync=False)
            self.m.backward(1.0 / k)
        self.m.step(lr, 1.0, sync=False)

    def timed(self, steps, warmup, lr=6e-4, kernel_class=None):
        """Wall-clock seconds of exactly `steps` steps between two device
        synchronizations, and the per-step HIP-event times (ms).  With
        `kernel_class`, the library also brackets that class's launches with
        HIP events on its stream during the timed steps; the summed time
        and launch count are kept in self.class_timed."""
        torch = self.torch
        if kernel_class:
            self.m.timing_enable(kernel_class)   # warm-up creates the events
        for _ in range(warmup):
            self.step(lr)
        torch.cuda.synchronize()
        if kernel_class:
            self.m.timing_read()                 # drop the warm-up brackets
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in ev:
            a.record()
            self.step(lr)
            b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if kernel_class:
            self.class_timed = self.m.timing_read()
            self.m.timing_enable("none")
        return wall, [a.elapsed_time(b) for a, b in ev]

    def class_ms(self, cls, steps=3):
        """Milliseconds per step and brackets per step of one timing class."""
        self.m.timing_enable(cls)
        for _ in range(steps):
            self.step()
        ms, n = self.m.timing_read()
        self.m.timing_enable("none")
        return ms / steps, n / steps

    def close(self):
        self.m.close()
        self.torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the unpadded-vocabulary and accumulated-step measurements")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the data-parallel exchange is not built)", file=sys.stderr)
        sys.exit(2)

    import ctypes
    import torch
    from decoder_only_transformer_02_amd import gpt2 as G
    from decoder_only_transformer_02_amd import inputs

    p = inputs.PRESETS["gpt2_124m"]
    B, T = p["B"], p["T"]
    print(f"config 124M B={B} T={T}: warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr,
          flush=True)
    r = Runner(G, inputs, torch, p)
    wall, ev_ms = r.timed(args.steps, args.warmup, kernel_class="lmhead_fwd")
    lm_ms, lm_n = r.class_timed
    ms = wall / args.steps * 1e3
    tokens = B * T * args.steps / wall
    n_total = G.lib().gpt2_num_params(ctypes.byref(r.cfg))
    n_mfu = n_total - p["block_size"] * p["n_embd"] - (p["padded_vocab"] - p["vocab_size"]) * p["n_embd"]
    fpt = flops_per_token(p["n_layer"], p["n_embd"], T, n_mfu)
    work = class_work(p, B, T, n_total)

    print("per-class kernel timing", file=sys.stderr, flush=True)
    kernels = {}
    for cls in ("lmhead_fwd", "gemm", "attn_fwd", "attn_bwd", "ln_fwd", "ln_bwd", "xent", "norm", "adamw",
                "embed"):
        c_ms, c_n = r.class_ms(cls)
        k = {"ms_per_step": round(c_ms, 4), "launches_per_step": c_n}
        if cls in work:
            bound, amount, unit = work[cls]
            k.update({"work_per_step": amount, "work_unit": unit})
            k.update(roofline_entry(bound, amount, c_ms))
        kernels[cls] = k
    loss = r.m.forward(*r.batches[0], sync=True)
    r.close()
    del r

    # the dominant kernel's rate over the timed steps themselves
    lm = roofline_entry("mfma", work["lmhead_fwd"][1], lm_ms / max(args.steps, 1))
    out = {
        "metric": METRIC,
        "value": round(tokens, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "ms_per_step_median": round(percentile(ev_ms, 50), 3),
        "ms_per_step_p10": round(percentile(ev_ms, 10), 3),
        "ms_per_step_p90": round(percentile(ev_ms, 90), 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"GPT-2 124M train step (forward, backward, clip, AdamW), B={B}, T={T}, "
                               f"vocabulary {p['vocab_size']} padded to {p['padded_vocab']}, Zipf(1.1) ids",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "mfu": round(tokens * fpt / PEAK_BF16, 4),
        "flops_per_token": fpt,
        "loss": round(loss, 5),
        "roofline": {"kernel": "classifier GEMM forward (k_gemm_nt 256x256, EPI_LOGITS)",
                     "bound": "mfma", "achieved": lm["achieved"], "peak": lm["peak"], "unit": "TFLOP/s",
                     "frac": lm["frac"], "traffic": None,
                     "avg_launch_ms": round(lm_ms / max(lm_n, 1), 4),
                     "launches": lm_n / max(args.steps, 1),
                     "timed_over": f"HIP events on the library stream around each classifier launch "
                                   f"of the {args.steps} timed steps"},
        "kernels": kernels,
    }

    if not args.no_extra:
        print("unpadded vocabulary", file=sys.stderr, flush=True)
        u = Runner(G, inputs, torch, inputs.PRESETS["gpt2_124m_v50257"])
        u_wall, u_ev = u.timed(max(5, args.steps // 2), 2)
        u_lm, _ = u.class_ms("lmhead_fwd")
        u_gemm_x = u.class_ms("xent")[0]
        u.close()
        del u
        pad_ms = kernels["lmhead_fwd"]["ms_per_step"] + kernels["xent"]["ms_per_step"]
        unpad_ms = u_lm + u_gemm_x
        out["padding"] = {
            "classifier_fwd_plus_xent_ms": {"vocab_50304": round(pad_ms, 4), "vocab_50257": round(unpad_ms, 4)},
            "step_ms_median": {"vocab_50304": round(percentile(ev_ms, 50), 3),
                               "vocab_50257": round(percentile(u_ev, 50), 3)},
            "step_speedup_from_padding": round(percentile(u_ev, 50) / percentile(ev_ms, 50) - 1.0, 4),
        }
        print("accumulated step (32 x B=32 T=512)", file=sys.stderr, flush=True)
        pa = inputs.PRESETS["gpt2_124m_accum"]
        a = Runner(G, inputs, torch, pa, micro=pa["accum"])
        a_steps = 10
        a_wall, a_ev = a.timed(a_steps, 3, lr=G.lr_at(pa["lr_step"]))
        a.close()
        del a
        a_tok = pa["B"] * pa["T"] * pa["accum"]
        a_ms = percentile(a_ev, 50)
        out["accumulated_step"] = {
            "tokens_per_step": a_tok, "steps": a_steps, "warmup": 3, "ms_per_step_median": round(a_ms, 2),
            "ms_per_step_p10": round(percentile(a_ev, 10), 2), "ms_per_step_p90": round(percentile(a_ev, 90), 2),
            "ms_per_step_wall_mean": round(a_wall / a_steps * 1e3, 2),
            "tokens_per_s": round(a_tok / (a_ms * 1e-3), 1),
            "mfu": round(a_tok / (a_ms * 1e-3) * flops_per_token(pa["n_layer"], pa["n_embd"], pa["T"], n_mfu)
                         / PEAK_BF16, 4)}
    if not args.no_extra:
        print("single block (B=16 T=1024)", file=sys.stderr, flush=True)
        out["block"] = block_leg(G, inputs, torch)
    if not args.no_cpu_baseline:
        print("cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(p)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
