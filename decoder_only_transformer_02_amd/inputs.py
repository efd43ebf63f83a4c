"""Seeded synthetic inputs and the named workload presets.

This module holds no arithmetic of the training step.  It only draws token
streams and block inputs from fixed seeds, so that the HIP library and the
CPU oracle can be fed identical arrays.

Token streams stand in for the FineWeb-Edu shards named on the pages
("Let's reproduce GPT-2 (124M)", bullet "Data Set and Evaluation"): ids in
[0, 50257) with a skewed, Zipf-like frequency profile.  Targets are the
stream shifted by one, as the chapter "data loader lite" describes.
"""
from __future__ import annotations

import numpy as np

# Sizes of the named workloads.  `compute` is the arithmetic type of the
# path ("fp32" throughout, or "bf16" operands with fp32 accumulation and
# fp32 master weights).
PRESETS = {
    # tiny GPT-2-shaped decoder, fp32 throughout
    "tiny": dict(n_layer=2, n_head=4, n_embd=64, block_size=64, vocab_size=512,
                 padded_vocab=512, B=4, T=64, compute="fp32", tokens="uniform"),
    # one GPT-2 124M block in isolation
    "block124m": dict(n_layer=12, n_head=12, n_embd=768, block_size=1024, vocab_size=50257,
                      padded_vocab=50304, B=16, T=1024, compute="bf16", tokens="none"),
    # full GPT-2 124M step, vocabulary padded to 50304
    "gpt2_124m": dict(n_layer=12, n_head=12, n_embd=768, block_size=1024, vocab_size=50257,
                      padded_vocab=50304, B=16, T=1024, compute="bf16", tokens="zipf"),
    # same, unpadded vocabulary (ragged classifier tiles)
    "gpt2_124m_v50257": dict(n_layer=12, n_head=12, n_embd=768, block_size=1024,
                             vocab_size=50257, padded_vocab=50257, B=16, T=1024,
                             compute="bf16", tokens="zipf"),
    # the same step in fp32 throughout (matrix-core fp32 GEMMs)
    "gpt2_124m_fp32": dict(n_layer=12, n_head=12, n_embd=768, block_size=1024, vocab_size=50257,
                           padded_vocab=50304, B=16, T=1024, compute="fp32", tokens="zipf"),
    # accumulated optimizer step: 32 micro-steps of B=32, T=512
    "gpt2_124m_accum": dict(n_layer=12, n_head=12, n_embd=768, block_size=1024,
                            vocab_size=50257, padded_vocab=50304, B=32, T=512, accum=32,
                            compute="bf16", tokens="zipf", lr_step=132),
}


def uniform_stream(seed: int, n: int, vocab: int) -> np.ndarray:
    """n ids uniform in [0, vocab)."""
    return np.random.default_rng(seed).integers(0, vocab, n).astype(np.int32)


def zipf_stream(seed: int, n: int, vocab: int = 50257, s: float = 1.1) -> np.ndarray:
    """n ids with P(id = k) proportional to (k + 1)^-s on [0, vocab), drawn by
    inverse CDF (a float64 cumulative table searched with uniform draws)."""
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = np.random.default_rng(seed).random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def batch_from_stream(stream: np.ndarray, B: int, T: int, k: int = 0):
    """Micro-batch k of a stream: x = s[kBT : (k+1)BT], y = x shifted by one,
    both [B, T] row-major int32."""
    n = B * T
    x = stream[k * n:(k + 1) * n].reshape(B, T)
    y = stream[k * n + 1:(k + 1) * n + 1].reshape(B, T)
    return np.ascontiguousarray(x, dtype=np.int32), np.ascontiguousarray(y, dtype=np.int32)


def tokens_for(preset: dict, seed: int = 0, B: int | None = None, T: int | None = None,
               micro_steps: int = 1):
    """The stream of a preset (B*T*micro_steps + 1 ids)."""
    B = preset["B"] if B is None else B
    T = preset["T"] if T is None else T
    n = B * T * micro_steps + 1
    if preset["tokens"] == "uniform":
        return uniform_stream(seed, n, preset["vocab_size"])
    return zipf_stream(seed, n, preset["vocab_size"])


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), kept in
    float32 storage."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def block_inputs(seed: int, B: int, T: int, C: int, dy_std: float = 1e-3):
    """Block-in-isolation inputs: x ~ N(0, 1) and dy ~ N(0, dy_std^2), both
    rounded to bf16 (exact in float32 / float64)."""
    rng = np.random.default_rng(seed)
    x = round_to_bf16(rng.standard_normal((B, T, C)).astype(np.float32))
    dy = round_to_bf16((dy_std * rng.standard_normal((B, T, C))).astype(np.float32))
    return x, dy
