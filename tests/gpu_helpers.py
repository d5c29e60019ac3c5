"""Shared helpers of the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import sys

import numpy as np

import synthetic as syn


def say(*a):
    """Print what names the case before each GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def to_dev(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def max_rel(a, r) -> float:
    a = np.asarray(a, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-30))


def cosine(a, r) -> float:
    a = np.asarray(a, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    na, nr = np.linalg.norm(a), np.linalg.norm(r)
    if na == 0 and nr == 0:
        return 1.0
    return float(a @ r / (na * nr))


def ocfg(o, m: syn.Model, seed: int = 0):
    # the dropout probability as the GPU's fp32 config holds it
    return o.make_cfg(m.vocab, m.block_size, m.n_embd, m.n_head, m.n_layer, m.mlp_hidden, m.bias, m.ln_eps,
                      gelu_erf=m.gelu_erf, untied=m.untied, dropout=float(np.float32(m.dropout)), seed=seed)


def gcfg(b, m: syn.Model, dtype: str):
    return b.make_config(m.vocab, m.block_size, m.n_embd, m.n_head, m.n_layer, m.mlp_hidden, m.bias,
                         b.DTYPE_F32 if dtype == "f32" else b.DTYPE_BF16, m.ln_eps, gelu_erf=m.gelu_erf,
                         untied_head=m.untied, dropout=m.dropout)


def gpu_model(b, m: syn.Model, dtype: str, B: int, T: int, named: dict, mode=None):
    mode = b.MODE_TRAIN if mode is None else mode
    g = b.Model(gcfg(b, m, dtype), B, T, mode)
    g.load_named(named)
    g.init()
    return g


def gpu_named_grads(g) -> dict:
    flat = g.grads.detach().cpu().numpy().astype(np.float64)
    return {k: np.array(v) for k, v in g.named(flat).items()}


def gpu_named_params(g) -> dict:
    flat = g.params.detach().cpu().numpy()
    return {k: np.array(v) for k, v in g.named(flat).items()}


def oracle_grads(o, m: syn.Model, named: dict, x, y, dtype=np.float64, loss_scale=1.0, seed=0):
    cfg = ocfg(o, m, seed)
    p = o.pack(cfg, named, dtype)
    g = np.zeros_like(p)
    B, T = x.shape
    loss, _, _ = o.step(cfg, B, T, p, x, y, g, loss_scale=loss_scale)
    return loss, {k: np.array(v, dtype=np.float64) for k, v in o.unpack(cfg, g).items()}
