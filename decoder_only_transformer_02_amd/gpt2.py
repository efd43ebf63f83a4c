"""Thin Python binding of the C ABI in include/gpt2.h (libgpt2mi.so).

Argument marshalling only: every step of the training step runs in the HIP
kernels behind the ABI.  PyTorch provides the device arena, the int32 token
buffers and the stream; nothing here computes.  If the library is missing
the binding raises; there is no fallback.
"""
from __future__ import annotations

import ctypes as ct
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgpt2mi.so")

GPT2_OK, GPT2_E_ARG, GPT2_E_SHAPE, GPT2_E_STATE = 0, -1, -2, -3
GPT2_E_HIP, GPT2_E_TOKEN, GPT2_E_NONFINITE, GPT2_E_ARENA = -4, -5, -6, -7
STATUS = {0: "OK", -1: "E_ARG", -2: "E_SHAPE", -3: "E_STATE", -4: "E_HIP", -5: "E_TOKEN",
          -6: "E_NONFINITE", -7: "E_ARENA"}
GPT2_FP32, GPT2_BF16, GPT2_FP16 = 0, 1, 2
KINDS = ["param", "grad", "adam_m", "adam_v", "shadow", "act", "logits", "scalar"]
TIMING = {"none": 0, "lmhead_fwd": 1, "gemm": 2, "attn_fwd": 3, "attn_bwd": 4, "ln_fwd": 5,
          "ln_bwd": 6, "xent": 7, "adamw": 8, "norm": 9, "embed": 10}

# every symbol declared in include/gpt2.h
EXPORTS = ["gpt2_default_config", "gpt2_arena_bytes", "gpt2_num_params", "gpt2_init_host",
           "gpt2_create", "gpt2_destroy", "gpt2_last_error", "gpt2_forward", "gpt2_backward",
           "gpt2_zero_grad", "gpt2_step", "gpt2_lr_at", "gpt2_block_fwd_bwd", "gpt2_num_tensors",
           "gpt2_tensor_info", "gpt2_timing_enable", "gpt2_timing_read", "gpt2_sync_weight_copies",
           "gpt2_get_step_count", "gpt2_set_step_count", "gpt2_check_arena", "gpt2_eval_loss",
           "gpt2_kv_cache_bytes", "gpt2_generate", "gpt2_get_loss_scale", "gpt2_set_loss_scale"]


class Config(ct.Structure):
    _fields_ = [("n_layer", ct.c_int32), ("n_head", ct.c_int32), ("n_embd", ct.c_int32),
                ("block_size", ct.c_int32), ("vocab_size", ct.c_int32),
                ("padded_vocab", ct.c_int32), ("max_batch", ct.c_int32), ("max_seq", ct.c_int32),
                ("compute", ct.c_int32), ("ln_eps", ct.c_float), ("beta1", ct.c_float),
                ("beta2", ct.c_float), ("adam_eps", ct.c_float), ("weight_decay", ct.c_float)]


class TensorDesc(ct.Structure):
    _fields_ = [("name", ct.c_char * 48), ("kind", ct.c_int32), ("dtype", ct.c_int32),
                ("ndim", ct.c_int32), ("decay", ct.c_int32), ("shape", ct.c_int64 * 4),
                ("offset", ct.c_uint64), ("bytes", ct.c_uint64)]


class GPT2Error(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def bind(L):
    """Sets the argument and result types of every call in include/gpt2.h on
    a loaded library handle."""
    P, I32, I64, SZ, F = ct.c_void_p, ct.c_int32, ct.c_int64, ct.c_size_t, ct.c_float
    cfgp = ct.POINTER(Config)
    sig = {
        "gpt2_default_config": (None, [cfgp, I32, I32]),
        "gpt2_arena_bytes": (SZ, [cfgp]),
        "gpt2_num_params": (I64, [cfgp]),
        "gpt2_init_host": (I32, [cfgp, ct.c_uint64, P]),
        "gpt2_create": (I32, [cfgp, ct.c_uint64, P, SZ, P, ct.POINTER(P)]),
        "gpt2_destroy": (None, [P]),
        "gpt2_last_error": (ct.c_char_p, [P]),
        "gpt2_forward": (I32, [P, P, P, I32, I32, ct.POINTER(F)]),
        "gpt2_backward": (I32, [P, F]),
        "gpt2_zero_grad": (I32, [P]),
        "gpt2_step": (I32, [P, F, F, ct.POINTER(F)]),
        "gpt2_lr_at": (ct.c_double, [I64, ct.c_double, ct.c_double, I64, I64]),
        "gpt2_block_fwd_bwd": (I32, [P, I32, P, P, P, P, I32, I32]),
        "gpt2_num_tensors": (I32, [P]),
        "gpt2_tensor_info": (I32, [P, I32, ct.POINTER(TensorDesc)]),
        "gpt2_timing_enable": (I32, [P, I32]),
        "gpt2_timing_read": (I32, [P, ct.POINTER(ct.c_double), ct.POINTER(I64)]),
        "gpt2_sync_weight_copies": (I32, [P]),
        "gpt2_get_step_count": (I32, [P, ct.POINTER(I64)]),
        "gpt2_set_step_count": (I32, [P, I64]),
        "gpt2_check_arena": (I32, [P, ct.POINTER(I32)]),
        "gpt2_eval_loss": (I32, [P, P, P, I32, I32, ct.POINTER(F)]),
        "gpt2_kv_cache_bytes": (SZ, [cfgp]),
        "gpt2_generate": (I32, [P, P, SZ, P, I32, I32, I32, P, P]),
        "gpt2_get_loss_scale": (I32, [P, ct.POINTER(F)]),
        "gpt2_set_loss_scale": (I32, [P, F, I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    """Loads libgpt2mi.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    _lib = bind(ct.CDLL(LIB_PATH))
    return _lib


def make_config(n_layer, n_head, n_embd, block_size, vocab_size, padded_vocab, max_batch, max_seq,
                compute="bf16", **_):
    c = Config()
    lib().gpt2_default_config(ct.byref(c), max_batch, max_seq)
    c.n_layer, c.n_head, c.n_embd = n_layer, n_head, n_embd
    c.block_size, c.vocab_size, c.padded_vocab = block_size, vocab_size, padded_vocab
    c.compute = {"bf16": GPT2_BF16, "fp16": GPT2_FP16, "fp32": GPT2_FP32}[compute]
    return c


def lr_at(it: int, max_lr: float = 6e-4, min_lr: float = 6e-5, warmup: int = 132,
          decay_end: int = 3400) -> float:
    """Learning rate at optimizer iteration `it` (include/gpt2.h, gpt2_lr_at)."""
    return lib().gpt2_lr_at(it, max_lr, min_lr, warmup, decay_end)


def init_host(cfg: Config, seed: int) -> np.ndarray:
    """Initial parameters computed by the library on the host (no GPU)."""
    n = lib().gpt2_num_params(ct.byref(cfg))
    out = np.empty(n, np.float32)
    st = lib().gpt2_init_host(ct.byref(cfg), ct.c_uint64(seed), out.ctypes.data_as(ct.c_void_p))
    if st != 0:
        raise GPT2Error(st, "gpt2_init_host")
    return out


class GPT2Step:
    """One context of the training step on the current HIP device."""

    def __init__(self, cfg: Config, seed: int = 0, device="cuda:0"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        self._L = L = lib()
        nbytes = L.gpt2_arena_bytes(ct.byref(cfg))
        if nbytes == 0:
            raise GPT2Error(GPT2_E_ARG, "invalid config")
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.stream = torch.cuda.current_stream(self.device)
        ctx = ct.c_void_p()
        st = L.gpt2_create(ct.byref(cfg), ct.c_uint64(seed), ct.c_void_p(self.arena.data_ptr()),
                           nbytes, ct.c_void_p(self.stream.cuda_stream), ct.byref(ctx))
        if st != 0:
            raise GPT2Error(st, "gpt2_create")
        self.ctx = ctx
        self._tables()

    def _tables(self):
        L = self._L
        self.tensors = {}
        d = TensorDesc()
        for i in range(L.gpt2_num_tensors(self.ctx)):
            self._check(L.gpt2_tensor_info(self.ctx, i, ct.byref(d)))
            self.tensors[d.name.decode()] = dict(kind=KINDS[d.kind], dtype=d.dtype,
                                                 shape=tuple(d.shape[:d.ndim]), offset=d.offset,
                                                 bytes=d.bytes, decay=bool(d.decay))

    def close(self):
        if getattr(self, "ctx", None):
            self._L.gpt2_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st):
        if st != 0:
            msg = self._L.gpt2_last_error(self.ctx) if getattr(self, "ctx", None) else b""
            raise GPT2Error(st, (msg or b"").decode())

    # ------------------------------------------------------------------ calls
    def forward(self, tokens, targets=None, sync=True):
        B, T = tokens.shape
        loss = ct.c_float(0.0)
        st = self._L.gpt2_forward(self.ctx, ct.c_void_p(tokens.data_ptr()),
                                ct.c_void_p(targets.data_ptr()) if targets is not None else None,
                                B, T, ct.byref(loss) if sync else None)
        self._check(st)
        return loss.value if (sync and targets is not None) else None

    def eval_loss(self, tokens, targets, sync=True):
        """Forward-only mean cross-entropy (no logits gradient, backward not
        armed)."""
        B, T = tokens.shape
        loss = ct.c_float(0.0)
        self._check(self._L.gpt2_eval_loss(self.ctx, ct.c_void_p(tokens.data_ptr()),
                                           ct.c_void_p(targets.data_ptr()), B, T,
                                           ct.byref(loss) if sync else None))
        return loss.value if sync else None

    def generate(self, tokens, T0, uniforms, logprobs=None):
        """Samples positions [T0, T) of the int32 [B, T] device tensor
        `tokens` in place from its prefix [0, T0), with the float32 [B, T - T0]
        uniform draws; fills `logprobs` (same shape, optional).  The key/value
        cache is allocated once per context (gpt2_kv_cache_bytes)."""
        B, T = tokens.shape
        if getattr(self, "_kv", None) is None:
            n = self._L.gpt2_kv_cache_bytes(ct.byref(self.cfg))
            self._kv = self.torch.empty(n, dtype=self.torch.uint8, device=self.device)
        self._check(self._L.gpt2_generate(self.ctx, ct.c_void_p(self._kv.data_ptr()), self._kv.numel(),
                                          ct.c_void_p(tokens.data_ptr()), B, T0, T,
                                          ct.c_void_p(uniforms.data_ptr()),
                                          ct.c_void_p(logprobs.data_ptr()) if logprobs is not None else None))

    def backward(self, grad_scale=1.0):
        self._check(self._L.gpt2_backward(self.ctx, grad_scale))

    def zero_grad(self):
        self._check(self._L.gpt2_zero_grad(self.ctx))

    def step(self, lr, clip=1.0, sync=True):
        norm = ct.c_float(0.0)
        self._check(self._L.gpt2_step(self.ctx, lr, clip, ct.byref(norm) if sync else None))
        return norm.value if sync else None

    def block_fwd_bwd(self, layer, x, dy):
        """x, dy: float32 cuda [B, T, C]; returns (y, dx)."""
        B, T, C = x.shape
        y = self.torch.empty_like(x)
        dx = self.torch.empty_like(x)
        self._check(self._L.gpt2_block_fwd_bwd(self.ctx, layer, ct.c_void_p(x.data_ptr()),
                                             ct.c_void_p(dy.data_ptr()), ct.c_void_p(y.data_ptr()),
                                             ct.c_void_p(dx.data_ptr()), B, T))
        return y, dx

    def timing_enable(self, kernel_class: str):
        self._check(self._L.gpt2_timing_enable(self.ctx, TIMING[kernel_class]))

    def timing_read(self):
        ms = ct.c_double(0.0)
        n = ct.c_int64(0)
        self._check(self._L.gpt2_timing_read(self.ctx, ct.byref(ms), ct.byref(n)))
        return ms.value, n.value

    def check_arena(self):
        """Raises GPT2Error (E_ARENA) if a kernel wrote past its arena region."""
        n = ct.c_int32(0)
        self._check(self._L.gpt2_check_arena(self.ctx, ct.byref(n)))

    def loss_scale(self):
        v = ct.c_float(0.0)
        self._check(self._L.gpt2_get_loss_scale(self.ctx, ct.byref(v)))
        return v.value

    def set_loss_scale(self, scale: float, growth_interval: int = 2000):
        self._check(self._L.gpt2_set_loss_scale(self.ctx, scale, growth_interval))

    def sync_weight_copies(self):
        self._check(self._L.gpt2_sync_weight_copies(self.ctx))

    def step_count(self):
        t = ct.c_int64(0)
        self._check(self._L.gpt2_get_step_count(self.ctx, ct.byref(t)))
        return t.value

    def set_step_count(self, t: int):
        self._check(self._L.gpt2_set_step_count(self.ctx, t))

    def state_dict(self):
        """Checkpoint: host copies of the parameters, both AdamW moments and
        the step count."""
        kinds = ("param", "adam_m", "adam_v")
        out = {n: self.view(n).clone().cpu() for n, t in self.tensors.items() if t["kind"] in kinds}
        out["__step__"] = self.step_count()
        return out

    def load_state_dict(self, sd):
        """Resume from state_dict(): writes the tensors back through the
        arena views, sets the step count and refreshes the bf16 copies."""
        for n, v in sd.items():
            if n != "__step__":
                self.view(n).copy_(v)
        self.set_step_count(sd["__step__"])
        self.sync_weight_copies()

    # ------------------------------------------------------------------ views
    def view(self, name):
        """Zero-copy torch view of a tensor in the arena."""
        t = self.tensors[name]
        torch = self.torch
        dt = {0: torch.float32, 1: torch.bfloat16, 2: torch.int32, 3: torch.float64,
              4: torch.float16}[t["dtype"]]
        raw = self.arena[t["offset"]:t["offset"] + t["bytes"]]
        return raw.view(dt).view(t["shape"])

    def param_names(self):
        return [n for n, t in self.tensors.items() if t["kind"] == "param"]
