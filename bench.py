"""Throughput of one GPT-2 124M training step (forward, backward, global-norm
clip, AdamW) at B=16, T=1024, bf16, on one MI355X, through the C ABI.

Prints one JSON line: tokens/s (whole job), ms/step, MFU, the roofline of
the dominant kernel (the classifier GEMM, timed live with HIP events on the
library stream over the timed region), and the CPU oracle timed on a
bounded sample of the same workload on this host."""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15     # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12      # bytes/s


def flops_per_token(L, C, T, n_nonemb):
    """6N + 6 L C (T + 1): causal attention scores counted once per (i <= j)."""
    return 6 * n_nonemb + 6 * L * C * (T + 1)


def cpu_baseline(preset, seconds_hint=True):
    import numpy as np
    from decoder_only_transformer_02_amd import inputs
    from oracle import gpt2_oracle as O
    oc = O.Config(preset["n_layer"], preset["n_head"], preset["n_embd"], preset["block_size"],
                  preset["vocab_size"], preset["padded_vocab"])
    P = O.init_params(oc, 0)
    T = preset["T"]
    x, y = inputs.batch_from_stream(inputs.zipf_stream(0, T + 1, preset["vocab_size"]), 1, T)
    t0 = time.perf_counter()
    O.train_step(P, [(x, y)], oc, lr=6e-4, clip=1.0, t=1, dt=np.float32)
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one full step (forward, backward, clip, AdamW) of the same model on one "
                      f"sequence of {T} tokens, float32 storage with float64 reductions, "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--preset", default="gpt2_124m")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the data-parallel exchange is not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from decoder_only_transformer_02_amd import gpt2 as G
    from decoder_only_transformer_02_amd import inputs

    p = inputs.PRESETS[args.preset]
    B, T = p["B"], p["T"]
    cfg = G.make_config(**{**p, "max_batch": B, "max_seq": T})
    m = G.GPT2Step(cfg, seed=0)
    x, y = inputs.batch_from_stream(inputs.zipf_stream(0, B * T + 1, p["vocab_size"]), B, T)
    xd = torch.from_numpy(x).cuda()
    yd = torch.from_numpy(y).cuda()
    lr = 6e-4

    def step():
        m.forward(xd, yd, sync=False)
        m.backward(1.0)
        m.step(lr, 1.0, sync=False)

    print(f"warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    m.timing_enable("lmhead_fwd")
    print(f"timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    k_ms, k_n = m.timing_read()
    m.timing_enable("none")
    loss = m.forward(xd, yd, sync=True)

    ms = dt / args.steps * 1e3
    tokens = B * T * args.steps / dt
    n_total = G.lib().gpt2_num_params(__import__("ctypes").byref(cfg))
    n_mfu = n_total - p["block_size"] * p["n_embd"] - (p["padded_vocab"] - p["vocab_size"]) * p["n_embd"]
    fpt = flops_per_token(p["n_layer"], p["n_embd"], T, n_mfu)
    mfu = tokens * fpt / PEAK_BF16
    avg_k = k_ms / max(k_n, 1) * 1e-3
    k_flops = 2.0 * B * T * p["padded_vocab"] * p["n_embd"]
    achieved = k_flops / avg_k / 1e12
    out = {
        "metric": "train tokens/sec + ms/step, GPT-2 124M B=16 T=1024 bf16; MFU vs peak",
        "value": round(tokens, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.preset}: GPT-2 124M train step, B={B}, T={T}, vocab "
                               f"{p['vocab_size']} padded to {p['padded_vocab']}, Zipf(1.1) ids",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "mfu": round(mfu, 4),
        "flops_per_token": fpt,
        "loss": round(loss, 5),
        "roofline": {"kernel": "classifier GEMM forward (k_gemm_nt, EPI_LOGITS)",
                     "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16 / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved * 1e12 / PEAK_BF16, 4),
                     "traffic": None, "avg_launch_ms": round(avg_k * 1e3, 4),
                     "launches": k_n},
    }
    del m
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        print("cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(p)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
