"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module holds the workload descriptions and random draws only: model
shapes, token streams and initial weights. It contains none of the model's
arithmetic, and neither the HIP library nor the oracle imports it; each side
receives the arrays it draws.

Workloads (the nanogpt page's train_gpt2.py sizes and the minigpt page's
GPTConfig defaults; token and init recipes are the synthetic stand-ins for
OpenWebText / Shakespeare, which are not available):
  tiny_f32   V65  T64   C128 H4  L4  F512,  no bias, B4,  uniform tokens, fp32
  char_bf16  V65  T256  C384 H6  L6  F1536, no bias, B64, Zipf s=1.1,     bf16
  gpt2_124m  V50257 T1024 C768 H12 L12 F3072, bias, B12, Zipf s=1.05,     bf16
  gpt2_124m_accum  as gpt2_124m, 40 micro-batches per optimiser step
  gpt2_124m_eval   as gpt2_124m, B64, forward + loss only
  tiny_f32_literal, char_bf16_literal, gpt2_124m_literal  as tiny_f32 / char_bf16 /
                   gpt2_124m with the minigpt page's literal model: exact-erf GELU
                   and an lm_head of its own
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Model:
    vocab: int
    block_size: int
    n_embd: int
    n_head: int
    n_layer: int
    mlp_hidden: int
    bias: bool
    ln_eps: float = 1e-5
    gelu_erf: bool = False  # exact erf GELU (nn.GELU() default) instead of the tanh form
    untied: bool = False    # separate lm_head [V, C] instead of the head tied to wte
    dropout: float = 0.0    # training-mode dropout probability (the minigpt page's literal model: 0.1)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: Model
    batch: int
    seq: int
    dtype: str            # "f32" or "bf16"
    tokens: str           # "uniform" or "zipf"
    zipf_s: float = 0.0
    steps: int = 1
    accum: int = 1
    clip: float = 0.0
    lr: float = 6e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    cosine: bool = False  # warmup + cosine schedule (max 6e-4, min 6e-5, warmup 2000, 600k iters)
    train: bool = True


GPT2_124M = Model(50257, 1024, 768, 12, 12, 3072, True)

WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", Model(65, 64, 128, 4, 4, 512, False), 4, 64, "f32", "uniform"),
    "char_bf16": Workload("char_bf16", Model(65, 256, 384, 6, 6, 1536, False), 64, 256, "bf16", "zipf",
                          zipf_s=1.1, steps=10),
    "gpt2_124m": Workload("gpt2_124m", GPT2_124M, 12, 1024, "bf16", "zipf", zipf_s=1.05),
    "gpt2_124m_accum": Workload("gpt2_124m_accum", GPT2_124M, 12, 1024, "bf16", "zipf", zipf_s=1.05,
                                accum=40, clip=1.0, cosine=True),
    "gpt2_124m_eval": Workload("gpt2_124m_eval", GPT2_124M, 64, 1024, "bf16", "zipf", zipf_s=1.05,
                               train=False),
    "gpt2_124m_literal": Workload("gpt2_124m_literal", dataclasses.replace(GPT2_124M, gelu_erf=True, untied=True), 12,
                                  1024, "bf16", "zipf", zipf_s=1.05),
    "tiny_f32_literal": Workload("tiny_f32_literal", Model(65, 64, 128, 4, 4, 512, False, gelu_erf=True, untied=True),
                                 4, 64, "f32", "uniform"),
    "char_bf16_literal": Workload("char_bf16_literal",
                                  Model(65, 256, 384, 6, 6, 1536, False, gelu_erf=True, untied=True), 64, 256,
                                  "bf16", "zipf", zipf_s=1.1, steps=10),
}

PARAM_SEED = 1234
DATA_SEED = 5678


def tensor_shapes(m: Model):
    """Named parameter tensors in module order, with shapes (the head is tied to
    wte unless the model is untied, then lm_head comes last, after ln_f)."""
    C, F = m.n_embd, m.mlp_hidden
    out = [("wte", (m.vocab, C)), ("wpe", (m.block_size, C))]
    for l in range(m.n_layer):
        p = f"h{l}."
        out += [(p + "ln1_g", (C,)), (p + "ln1_b", (C,)), (p + "w_qkv", (3 * C, C))]
        if m.bias:
            out.append((p + "b_qkv", (3 * C,)))
        out.append((p + "w_proj", (C, C)))
        if m.bias:
            out.append((p + "b_proj", (C,)))
        out += [(p + "ln2_g", (C,)), (p + "ln2_b", (C,)), (p + "w_fc", (F, C))]
        if m.bias:
            out.append((p + "b_fc", (F,)))
        out.append((p + "w_fc2", (C, F)))
        if m.bias:
            out.append((p + "b_fc2", (C,)))
    out += [("lnf_g", (C,)), ("lnf_b", (C,))]
    if m.untied:
        out.append(("lm_head", (m.vocab, C)))
    return out


def init_params(m: Model, seed: int = PARAM_SEED, std: float = 0.02) -> dict:
    """N(0, std) for embeddings and Linear weights, the two residual projections
    (w_proj, w_fc2) at std / sqrt(2 L), zero biases, LayerNorm gain 1 / bias 0.
    Each tensor draws from its own stream (seed, tensor index), fp32."""
    out = {}
    for i, (name, shape) in enumerate(tensor_shapes(m)):
        base = name.split(".")[-1]
        if base.endswith("_g"):
            out[name] = np.ones(shape, np.float32)
        elif base.endswith("_b") or base.startswith("b_"):
            out[name] = np.zeros(shape, np.float32)
        else:
            s = std / math.sqrt(2 * m.n_layer) if base in ("w_proj", "w_fc2") else std
            rng = np.random.Generator(np.random.PCG64([seed, i]))
            out[name] = (rng.standard_normal(shape, dtype=np.float32) * np.float32(s)).astype(np.float32)
    return out


def zipf_cdf(V: int, s: float) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def draw_tokens(rng: np.random.Generator, V: int, n: int, kind: str, s: float = 0.0) -> np.ndarray:
    """n iid token ids in [0, V): uniform, or Zipf with p(k) ~ (k+1)^-s (inverse CDF)."""
    if kind == "uniform":
        return rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)
    if kind == "zipf":
        u = rng.random(n)
        ids = np.searchsorted(zipf_cdf(V, s), u, side="right")
        return np.minimum(ids, V - 1).astype(np.int32)
    raise ValueError(kind)


def batch(w: Workload, step: int = 0, seed: int = DATA_SEED, B: int | None = None, T: int | None = None):
    """One batch: B rows of T+1 ids; x = row[:T], y = row[1:T+1] (targets are the
    inputs shifted by one, as get_batch builds them)."""
    B = w.batch if B is None else B
    T = w.seq if T is None else T
    rng = np.random.Generator(np.random.PCG64([seed, step]))
    rows = draw_tokens(rng, w.model.vocab, B * (T + 1), w.tokens, w.zipf_s).reshape(B, T + 1)
    return np.ascontiguousarray(rows[:, :T]), np.ascontiguousarray(rows[:, 1:])


def n_params_exact(m: Model) -> int:
    return int(sum(int(np.prod(s)) for _, s in tensor_shapes(m)))
