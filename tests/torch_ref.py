"""An independent PyTorch-CPU (float64, autograd) rendering of the same model,
built from library primitives (F.layer_norm, F.scaled_dot_product_attention
with is_causal, F.gelu(approximate="tanh"), F.cross_entropy,
torch.nn.utils.clip_grad_norm_, torch.optim.AdamW).  Used only to pin the
oracle's hand-derived forward and backward; it shares no code with it."""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def to_torch(params: dict):
    return {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True)
            for k, v in params.items()}


def model_loss(P: dict, idx: np.ndarray, tgt: np.ndarray | None, n_layer: int, n_head: int,
               eps: float = 1e-5, return_logits: bool = False):
    idx_t = torch.tensor(idx, dtype=torch.long)
    B, T = idx_t.shape
    C = P["wte"].shape[1]
    x = P["wte"][idx_t] + P["wpe"][:T][None]
    for l in range(n_layer):
        p = f"h{l}."
        a = F.layer_norm(x, (C,), P[p + "ln1.w"], P[p + "ln1.b"], eps)
        qkv = a @ P[p + "qkv.w"].T + P[p + "qkv.b"]
        q, k, v = qkv.split(C, dim=-1)
        q = q.view(B, T, n_head, C // n_head).transpose(1, 2)
        k = k.view(B, T, n_head, C // n_head).transpose(1, 2)
        v = v.view(B, T, n_head, C // n_head).transpose(1, 2)
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        o = o.transpose(1, 2).reshape(B, T, C)
        x = x + o @ P[p + "proj.w"].T + P[p + "proj.b"]
        a = F.layer_norm(x, (C,), P[p + "ln2.w"], P[p + "ln2.b"], eps)
        u = a @ P[p + "fc.w"].T + P[p + "fc.b"]
        x = x + F.gelu(u, approximate="tanh") @ P[p + "mproj.w"].T + P[p + "mproj.b"]
    x = F.layer_norm(x, (C,), P["lnf.w"], P["lnf.b"], eps)
    logits = x @ P["wte"].T
    if tgt is None:
        return logits
    loss = F.cross_entropy(logits.reshape(-1, logits.shape[-1]),
                           torch.tensor(tgt, dtype=torch.long).reshape(-1))
    if return_logits:
        return loss, logits
    return loss
