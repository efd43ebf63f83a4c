"""Plain CPU oracle for one GPT-2 (124M-family) training step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes follows the pages as follows (page titles as printed):
  * "Let's reproduce GPT-2 (124M)" (signalextractor key takeaways), bullet
    "GPT-2 Architecture Specifics": decoder-only, LayerNorm before attention
    and before the MLP, an extra LayerNorm before the classifier, GELU.
  * same page, bullet "Weight Tying & Numerical Padding": the token
    embedding is the classifier weight; the vocabulary may be padded
    (50257 -> 50304) and the padded size is then the model's vocabulary.
  * same page, bullets "Optimization Hyperparameters" and "Scaling Training
    with Gradient Accumulation & DDP": AdamW (0.9, 0.95, 1e-8), global-norm
    clip at 1.0, weight decay 0.1 on 2-D tensors only, warm-up + cosine LR
    down to 10 % of max, loss divided by the number of accumulation steps.
  * "From Scratch: Building GPT-2 for Efficient Language Modeling", Key
    Features (token + position embeddings, multi-head self-attention,
    residual connections, GELU MLP) and the Training Setup table (warm-up
    132, 3400 iterations, vocabulary 50304).
  * "Let's reproduce GPT-2 (124M)" chapter list: cross entropy loss,
    parameter sharing wte/lm_head, "model initialization: std 0.02, residual
    init".

Readings where the pages are silent (each is also listed in the design
notes): tanh-GELU; LayerNorm eps 1e-5 with the biased variance; attention
scale 1/sqrt(head_dim) with query i seeing keys j <= i; q, k, v as the
three contiguous thirds of the qkv projection, heads as contiguous chunks;
weights stored [out, in]; clip coefficient min(1, clip / (norm + 1e-6));
decoupled weight decay lr * wd * p; residual projections initialised with
std 0.02 / sqrt(2 * n_layer); sampling draws token t from the softmax over
the vocab_size real ids (padding ids excluded, temperature 1, no
truncation) by the inverse of its cumulative distribution in id order at a
uniform draw that the caller supplies.

Precision: every function takes a storage dtype.  float64 (default) is the
reference for small configurations and finite differences; float32 storage
keeps every reduction (LayerNorm statistics, softmax sums, loss mean,
gradient norm, bias / LayerNorm-parameter gradient sums) in float64.

Every function here is pinned by tests/test_oracle_*.py against closed
forms, invariants, finite differences, published generator outputs or an
independent library (PyTorch CPU).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F64 = np.float64

# ----------------------------------------------------------------------------
# configuration and canonical parameter list
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    n_layer: int
    n_head: int
    n_embd: int
    block_size: int
    vocab_size: int
    padded_vocab: int
    ln_eps: float = 1e-5
    beta1: float = 0.9
    beta2: float = 0.95
    adam_eps: float = 1e-8
    weight_decay: float = 0.1


def param_specs(cfg: Config):
    """Canonical tensor order: (name, shape, init std, decayed?).

    Initialization per the chapter "model initialization: std 0.02, residual
    init": N(0, 0.02) for embeddings and input projections, the residual
    (output) projections scaled by 1/sqrt(2 * n_layer), biases 0, LayerNorm
    gain 1 and bias 0.  Decay applies to 2-D tensors only ("Optimization
    Hyperparameters").
    """
    C, L = cfg.n_embd, cfg.n_layer
    res_std = 0.02 / math.sqrt(2.0 * L)
    specs = [("wte", (cfg.padded_vocab, C), 0.02, True),
             ("wpe", (cfg.block_size, C), 0.02, True)]
    for l in range(L):
        p = f"h{l}."
        specs += [
            (p + "ln1.w", (C,), "one", False),
            (p + "ln1.b", (C,), "zero", False),
            (p + "qkv.w", (3 * C, C), 0.02, True),
            (p + "qkv.b", (3 * C,), "zero", False),
            (p + "proj.w", (C, C), res_std, True),
            (p + "proj.b", (C,), "zero", False),
            (p + "ln2.w", (C,), "one", False),
            (p + "ln2.b", (C,), "zero", False),
            (p + "fc.w", (4 * C, C), 0.02, True),
            (p + "fc.b", (4 * C,), "zero", False),
            (p + "mproj.w", (C, 4 * C), res_std, True),
            (p + "mproj.b", (C,), "zero", False),
        ]
    specs += [("lnf.w", (C,), "one", False), ("lnf.b", (C,), "zero", False)]
    return specs


def num_params(cfg: Config) -> int:
    return sum(int(np.prod(s)) for _, s, _, _ in param_specs(cfg))


# ----------------------------------------------------------------------------
# initialization RNG: SplitMix64 (Steele, Lea & Flood, "Fast splittable
# pseudorandom number generators", OOPSLA 2014) + Box-Muller (1958)
# ----------------------------------------------------------------------------

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, index: np.ndarray) -> np.ndarray:
    """Output number `index` (0-based) of the SplitMix64 stream started at
    state `seed`: the state after i+1 increments is seed + (i+1)*golden."""
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (idx + np.uint64(1)) * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
    return z ^ (z >> np.uint64(31))


def normal_init(seed: int, tensor_index: int, n: int, std: float) -> np.ndarray:
    """n draws of N(0, std^2), rounded to float32.

    Tensor j draws from its own stream seeded with seed XOR (j << 32).
    Pair q uses outputs 2q (-> u1 in (0, 1]) and 2q+1 (-> u2 in [0, 1));
    Box-Muller gives r cos(2 pi u2) and r sin(2 pi u2), r = sqrt(-2 ln u1).
    """
    s = (int(seed) ^ (int(tensor_index) << 32)) & ((1 << 64) - 1)
    npair = (n + 1) // 2
    q = np.arange(npair, dtype=np.uint64)
    a = splitmix64(s, 2 * q)
    b = splitmix64(s, 2 * q + np.uint64(1))
    u1 = ((a >> np.uint64(11)).astype(F64) + 1.0) * (2.0 ** -53)
    u2 = (b >> np.uint64(11)).astype(F64) * (2.0 ** -53)
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * npair, dtype=F64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    return (z[:n] * std).astype(np.float32)


def init_params(cfg: Config, seed: int) -> dict:
    """All parameters as float32 arrays, in canonical order."""
    params = {}
    for j, (name, shape, std, _) in enumerate(param_specs(cfg)):
        n = int(np.prod(shape))
        if std == "one":
            params[name] = np.ones(shape, np.float32)
        elif std == "zero":
            params[name] = np.zeros(shape, np.float32)
        else:
            params[name] = normal_init(seed, j, n, std).reshape(shape)
    return params


# ----------------------------------------------------------------------------
# building blocks (each the textbook definition)
# ----------------------------------------------------------------------------

def layernorm_fwd(x, w, b, eps, dt):
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * w + b,
    var the biased (divide-by-C) variance; statistics in float64."""
    x64 = x.astype(F64)
    mu = x64.mean(axis=-1, keepdims=True)
    var = ((x64 - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x64 - mu) * rstd
    y = (xhat * w.astype(F64) + b.astype(F64)).astype(dt)
    return y, (xhat.astype(dt), rstd.astype(F64))


def layernorm_bwd(dy, cache, w, dt):
    """Chain rule through LayerNorm: with g = dy * w,
    dx = rstd * (g - mean(g) - xhat * mean(g * xhat)); dw = sum dy*xhat,
    db = sum dy (sums over all rows, float64)."""
    xhat, rstd = cache
    dy64 = dy.astype(F64)
    xh = xhat.astype(F64)
    g = dy64 * w.astype(F64)
    dx = rstd * (g - g.mean(axis=-1, keepdims=True)
                 - xh * (g * xh).mean(axis=-1, keepdims=True))
    C = dy.shape[-1]
    dw = (dy64 * xh).reshape(-1, C).sum(axis=0)
    db = dy64.reshape(-1, C).sum(axis=0)
    return dx.astype(dt), dw, db


_GELU_K = math.sqrt(2.0 / math.pi)
_GELU_A = 0.044715


def gelu_tanh(u):
    """tanh-approximate GELU (Hendrycks & Gimpel 2016)."""
    u64 = u.astype(F64)
    return 0.5 * u64 * (1.0 + np.tanh(_GELU_K * (u64 + _GELU_A * u64 ** 3)))


def gelu_tanh_grad(u):
    """d/du of gelu_tanh, differentiated by hand."""
    u64 = u.astype(F64)
    t = np.tanh(_GELU_K * (u64 + _GELU_A * u64 ** 3))
    return 0.5 * (1.0 + t) + 0.5 * u64 * (1.0 - t * t) * _GELU_K * (1.0 + 3.0 * _GELU_A * u64 ** 2)


def _softmax_rows(s):
    """Row softmax of s (last axis); max and sum in float64."""
    s64 = s.astype(F64)
    e = np.exp(s64 - s64.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def causal_attention_fwd(q, k, v, dt):
    """q, k, v: [B, H, T, hd].  S = q k^T / sqrt(hd) with S[i, j] = -inf for
    j > i (diagonal kept), P = row softmax(S), o = P v.  Computed one batch
    row at a time so the T x T scores never exist for all rows at once."""
    B, H, T, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    o = np.empty(q.shape, dtype=dt)
    for b in range(B):
        s = np.matmul(q[b], np.swapaxes(k[b], -1, -2)).astype(F64) * scale
        s[:, mask] = -np.inf
        p = _softmax_rows(s)
        o[b] = np.matmul(p.astype(dt), v[b]).astype(dt)
    return o


def causal_attention_bwd(q, k, v, o, do, dt):
    """Backward of causal_attention_fwd; P is recomputed from q, k:
    dV = P^T dO; dP = dO V^T; dS = P * (dP - rowsum(dP * P));
    dQ = dS K / sqrt(hd); dK = dS^T Q / sqrt(hd)."""
    B, H, T, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        s = np.matmul(q[b], np.swapaxes(k[b], -1, -2)).astype(F64) * scale
        s[:, mask] = -np.inf
        p = _softmax_rows(s)
        pd = p.astype(dt)
        dv[b] = np.matmul(np.swapaxes(pd, -1, -2), do[b]).astype(dt)
        dp = np.matmul(do[b], np.swapaxes(v[b], -1, -2)).astype(F64)
        dsm = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
        dsd = (dsm * scale).astype(dt)
        dq[b] = np.matmul(dsd, k[b]).astype(dt)
        dk[b] = np.matmul(np.swapaxes(dsd, -1, -2), q[b]).astype(dt)
    return dq, dk, dv


def _linear(x, w, b, dt):
    """y = x w^T + b with w stored [out, in]."""
    y = np.matmul(x, w.astype(dt).T)
    if b is not None:
        y = y + b.astype(dt)
    return y.astype(dt)


def _split_heads(t, H):
    M_B, T, C = t.shape
    return np.ascontiguousarray(t.reshape(M_B, T, H, C // H).transpose(0, 2, 1, 3))


def _merge_heads(t):
    B, H, T, hd = t.shape
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3).reshape(B, T, H * hd))


# ----------------------------------------------------------------------------
# one transformer block (pre-norm: x + attn(ln1(x)), then + mlp(ln2(.)))
# ----------------------------------------------------------------------------

def block_fwd(x, P, l, cfg: Config, dt):
    p = f"h{l}."
    C, H = cfg.n_embd, cfg.n_head
    a1, ln1c = layernorm_fwd(x, P[p + "ln1.w"], P[p + "ln1.b"], cfg.ln_eps, dt)
    qkv = _linear(a1, P[p + "qkv.w"], P[p + "qkv.b"], dt)
    q = _split_heads(qkv[..., 0:C], H)
    k = _split_heads(qkv[..., C:2 * C], H)
    v = _split_heads(qkv[..., 2 * C:3 * C], H)
    oh = causal_attention_fwd(q, k, v, dt)
    o = _merge_heads(oh)
    h1 = (x.astype(dt) + _linear(o, P[p + "proj.w"], P[p + "proj.b"], dt)).astype(dt)
    a2, ln2c = layernorm_fwd(h1, P[p + "ln2.w"], P[p + "ln2.b"], cfg.ln_eps, dt)
    u = _linear(a2, P[p + "fc.w"], P[p + "fc.b"], dt)
    g = gelu_tanh(u).astype(dt)
    h2 = (h1 + _linear(g, P[p + "mproj.w"], P[p + "mproj.b"], dt)).astype(dt)
    cache = dict(a1=a1, ln1c=ln1c, q=q, k=k, v=v, oh=oh, o=o, a2=a2, ln2c=ln2c, u=u, g=g)
    return h2, cache


def block_bwd(dh2, cache, P, l, cfg: Config, dt, grads):
    """Given dL/d(block output), returns dL/d(block input) and adds this
    block's parameter gradients into `grads` (float64 accumulators)."""
    p = f"h{l}."
    C, H = cfg.n_embd, cfg.n_head
    c = cache
    B, T, _ = dh2.shape
    dh2 = dh2.astype(dt)
    # h2 = h1 + g W_mp^T + b_mp
    grads[p + "mproj.w"] += np.matmul(dh2.reshape(-1, C).T, c["g"].reshape(-1, 4 * C)).astype(F64)
    grads[p + "mproj.b"] += dh2.astype(F64).reshape(-1, C).sum(axis=0)
    dg = np.matmul(dh2, P[p + "mproj.w"].astype(dt))
    du = (dg.astype(F64) * gelu_tanh_grad(c["u"])).astype(dt)
    # u = a2 W_fc^T + b_fc
    grads[p + "fc.w"] += np.matmul(du.reshape(-1, 4 * C).T, c["a2"].reshape(-1, C)).astype(F64)
    grads[p + "fc.b"] += du.astype(F64).reshape(-1, 4 * C).sum(axis=0)
    da2 = np.matmul(du, P[p + "fc.w"].astype(dt)).astype(dt)
    dx2, dw, db = layernorm_bwd(da2, c["ln2c"], P[p + "ln2.w"], dt)
    grads[p + "ln2.w"] += dw
    grads[p + "ln2.b"] += db
    dh1 = (dh2 + dx2).astype(dt)
    # h1 = x + o W_proj^T + b_proj
    grads[p + "proj.w"] += np.matmul(dh1.reshape(-1, C).T, c["o"].reshape(-1, C)).astype(F64)
    grads[p + "proj.b"] += dh1.astype(F64).reshape(-1, C).sum(axis=0)
    do = np.matmul(dh1, P[p + "proj.w"].astype(dt)).astype(dt)
    doh = _split_heads(do, H)
    dq, dk, dv = causal_attention_bwd(c["q"], c["k"], c["v"], c["oh"], doh, dt)
    dqkv = np.concatenate([_merge_heads(dq), _merge_heads(dk), _merge_heads(dv)], axis=-1)
    grads[p + "qkv.w"] += np.matmul(dqkv.reshape(-1, 3 * C).T, c["a1"].reshape(-1, C)).astype(F64)
    grads[p + "qkv.b"] += dqkv.astype(F64).reshape(-1, 3 * C).sum(axis=0)
    da1 = np.matmul(dqkv, P[p + "qkv.w"].astype(dt)).astype(dt)
    dx1, dw, db = layernorm_bwd(da1, c["ln1c"], P[p + "ln1.w"], dt)
    grads[p + "ln1.w"] += dw
    grads[p + "ln1.b"] += db
    dx = (dh1 + dx1).astype(dt)
    return dx


# ----------------------------------------------------------------------------
# full model: embeddings -> blocks -> ln_f -> tied classifier -> mean CE
# ----------------------------------------------------------------------------

def forward(P, idx, targets, cfg: Config, dt=F64, keep_logits=True):
    """idx, targets: int arrays [B, T] (targets may be None).
    Returns (loss or None, per-position losses [B, T] or None, cache)."""
    B, T = idx.shape
    C = cfg.n_embd
    h = (P["wte"].astype(dt)[idx] + P["wpe"].astype(dt)[np.arange(T)][None]).astype(dt)
    caches = []
    hs = [h]
    for l in range(cfg.n_layer):
        h, c = block_fwd(h, P, l, cfg, dt)
        caches.append(c)
        hs.append(h)
    hf, lnfc = layernorm_fwd(h, P["lnf.w"], P["lnf.b"], cfg.ln_eps, dt)
    z = np.matmul(hf.reshape(-1, C), P["wte"].astype(dt).T).astype(dt)    # [M, Vp]
    cache = dict(idx=idx, hf=hf, lnfc=lnfc, blocks=caches, B=B, T=T, hs=hs)
    if keep_logits:
        cache["z"] = z
    if targets is None:
        return None, None, cache
    y = targets.reshape(-1)
    z64 = z.astype(F64)
    zmax = z64.max(axis=1, keepdims=True)
    lse = (np.log(np.exp(z64 - zmax).sum(axis=1, keepdims=True)) + zmax)[:, 0]
    per = lse - z64[np.arange(y.size), y]
    loss = per.sum() / y.size
    cache["z"] = z
    cache["y"] = y
    return float(loss), per.reshape(B, T), cache


def cross_entropy_grad(z, y, scale):
    """d(mean CE)/dz * scale = (softmax(z) - onehot(y)) / M * scale."""
    p = _softmax_rows(z)
    p[np.arange(y.size), y] -= 1.0
    return p * (scale / y.size)


def backward(P, cache, cfg: Config, dt=F64, grad_scale=1.0):
    """Gradients (float64 arrays, one per parameter) of grad_scale * loss."""
    C = cfg.n_embd
    B, T = cache["B"], cache["T"]
    grads = {name: np.zeros(shape, F64) for name, shape, _, _ in param_specs(cfg)}
    dz = cross_entropy_grad(cache["z"], cache["y"], grad_scale).astype(dt)   # [M, Vp]
    hf = cache["hf"].reshape(-1, C)
    # tied classifier z = hf wte^T: head part of dwte
    grads["wte"] += np.matmul(dz.T, hf).astype(F64)
    dhf = np.matmul(dz, P["wte"].astype(dt)).astype(dt).reshape(B, T, C)
    dh, dw, db = layernorm_bwd(dhf, cache["lnfc"], P["lnf.w"], dt)
    grads["lnf.w"] += dw
    grads["lnf.b"] += db
    for l in reversed(range(cfg.n_layer)):
        dh = block_bwd(dh, cache["blocks"][l], P, l, cfg, dt, grads)
    # embedding part of the tied dwte, and dwpe
    dh64 = dh.astype(F64)
    np.add.at(grads["wte"], cache["idx"].reshape(-1), dh64.reshape(-1, C))
    grads["wpe"][:T] += dh64.sum(axis=0)
    return grads


# ----------------------------------------------------------------------------
# optimizer: global-norm clip, AdamW, LR schedule
# ----------------------------------------------------------------------------

def grad_norm(grads) -> float:
    """sqrt of the sum of squares of every gradient element (tied wte counted
    once, because it is one tensor), in float64."""
    return math.sqrt(sum(float((g.astype(F64) ** 2).sum()) for g in grads.values()))


def clip_coef(norm: float, clip: float) -> float:
    """PyTorch clip_grad_norm_ convention: min(1, clip / (norm + 1e-6))."""
    return min(1.0, clip / (norm + 1e-6))


def adamw_update(p, g, m, v, t, lr, cfg: Config, decay: bool):
    """One decoupled-decay Adam step (float64 math), returns (p, m, v):
    m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2; mhat = m/(1-b1^t),
    vhat = v/(1-b2^t); p = p - lr*(mhat/(sqrt(vhat)+eps) + wd*p)."""
    p64, g64, m64, v64 = (a.astype(F64) for a in (p, g, m, v))
    m64 = cfg.beta1 * m64 + (1.0 - cfg.beta1) * g64
    v64 = cfg.beta2 * v64 + (1.0 - cfg.beta2) * g64 * g64
    mhat = m64 / (1.0 - cfg.beta1 ** t)
    vhat = v64 / (1.0 - cfg.beta2 ** t)
    wd = cfg.weight_decay if decay else 0.0
    p64 = p64 - lr * (mhat / (np.sqrt(vhat) + cfg.adam_eps) + wd * p64)
    return p64, m64, v64


def optimizer_step(P, grads, M_state, V_state, t, lr, clip, cfg: Config):
    """Clip all gradients by the global norm, then AdamW on every tensor.
    Returns (new params (float32), new m, new v (float64), norm, coef)."""
    n = grad_norm(grads)
    c = clip_coef(n, clip)
    newP, newM, newV = {}, {}, {}
    for name, shape, _, decay in param_specs(cfg):
        p, m, v = adamw_update(P[name], grads[name] * c, M_state[name], V_state[name],
                               t, lr, cfg, decay)
        newP[name] = p.astype(np.float32)
        newM[name] = m
        newV[name] = v
    return newP, newM, newV, n, c


def lr_at(it: int, max_lr=6e-4, warmup=132, max_steps=3400, min_ratio=0.1) -> float:
    """Linear warm-up then cosine decay to min_ratio * max_lr.
    lr = max*(it+1)/W for it < W; min for it > S; else
    min + 0.5*(1 + cos(pi*(it-W)/(S-W)))*(max-min)."""
    min_lr = max_lr * min_ratio
    if it < warmup:
        return max_lr * (it + 1) / warmup
    if it > max_steps:
        return min_lr
    ratio = (it - warmup) / (max_steps - warmup)
    return min_lr + 0.5 * (1.0 + math.cos(math.pi * ratio)) * (max_lr - min_lr)


def train_step(P, micro_batches, cfg: Config, lr, clip=1.0, t=1, dt=F64, M_state=None, V_state=None,
               progress=None):
    """micro_batches: list of (idx, targets).  Loss of each micro-batch is
    scaled by 1/len(micro_batches) and gradients summed, then one clipped
    AdamW step.  Returns dict with loss (mean of micro losses), grads (the
    summed, unclipped ones), norm, coef, params, m, v.  `progress`, if
    given, is called as progress(i, k) after micro-batch i of k (reporting
    only; it takes no part in the arithmetic)."""
    k = len(micro_batches)
    total = None
    losses = []
    for i, (idx, tgt) in enumerate(micro_batches):
        loss, _, cache = forward(P, idx, tgt, cfg, dt)
        losses.append(loss)
        g = backward(P, cache, cfg, dt, grad_scale=1.0 / k)
        del cache
        if progress is not None:
            progress(i, k)
        if total is None:
            total = g
        else:
            for n_ in total:
                total[n_] += g[n_]
    if M_state is None:
        M_state = {n_: np.zeros(s, F64) for n_, s, _, _ in param_specs(cfg)}
        V_state = {n_: np.zeros(s, F64) for n_, s, _, _ in param_specs(cfg)}
    newP, newM, newV, n, c = optimizer_step(P, total, M_state, V_state, t, lr, clip, cfg)
    return dict(loss=float(np.mean(losses)), grads=total, norm=n, coef=c,
                params=newP, m=newM, v=newV)


def block_fwd_bwd(x, dy, P, l, cfg: Config, dt=F64):
    """One block in isolation: y = block(x); dx and the block's parameter
    gradients of sum(y * dy)."""
    y, cache = block_fwd(x.astype(dt), P, l, cfg, dt)
    grads = {name: np.zeros(shape, F64) for name, shape, _, _ in param_specs(cfg)
             if name.startswith(f"h{l}.")}
    dx = block_bwd(dy.astype(dt), cache, P, l, cfg, dt, grads)
    return y, dx, grads


# ----------------------------------------------------------------------------
# forward-only workloads: validation loss and sampling ("Let's reproduce
# GPT-2 (124M)" chapters "sampling init, prefix tokens", "sampling loop" and
# "validation data split, validation loss, sampling revive")
# ----------------------------------------------------------------------------

def eval_loss(P, idx, targets, cfg: Config, dt=F64) -> float:
    """Mean cross-entropy of a batch, forward only (the loss of forward())."""
    loss, _, _ = forward(P, idx, targets, cfg, dt, keep_logits=False)
    return loss


def sample_token(z_row, u: float, vocab_size: int):
    """Next token from one row of logits and a uniform draw u in [0, 1):
    p = softmax(z[:vocab_size]) in float64 (padding ids are not tokens), and
    the token is the smallest id v with p_0 + ... + p_v > u, i.e. the
    inverse of the cumulative distribution in id order.  Returns (token,
    log p_token)."""
    z = np.asarray(z_row[:vocab_size], dtype=F64)
    z = z - z.max()
    e = np.exp(z)
    S = e.sum()
    c = np.cumsum(e) / S
    v = int(np.searchsorted(c, u, side="right"))
    v = min(v, vocab_size - 1)
    while e[v] == 0.0 and v > 0:  # the top of the distribution: last id with mass
        v -= 1
    return v, float(z[v] - math.log(S))


def generate(P, tokens, T0: int, uniforms, cfg: Config, dt=F64):
    """Autoregressive sampling, the plain way: for t = T0 .. T-1 run the whole
    forward over positions [0, t) and sample token t from the logits of
    position t-1 with uniforms[:, t - T0].  tokens: int [B, T] with the
    prefix in [:, :T0].  Returns (tokens, log-probabilities [B, T - T0])."""
    tok = np.array(tokens, dtype=np.int64, copy=True)
    B, T = tok.shape
    lp = np.zeros((B, T - T0), F64)
    for t in range(T0, T):
        _, _, cache = forward(P, tok[:, :t], None, cfg, dt)
        z = cache["z"].reshape(B, t, -1)[:, t - 1]
        for b in range(B):
            tok[b, t], lp[b, t - T0] = sample_token(z[b], float(uniforms[b, t - T0]), cfg.vocab_size)
    return tok, lp
