#!/usr/bin/env python3
"""Benchmark of one GPT-2 training step on one MI355X.

A step is the whole hot path: forward, backward and AdamW over one micro-batch
of the 124M model (12 x 1024 tokens, bf16 operands, fp32 master weights and
optimizer state), inputs resident in HBM before the timed region. Prints one
JSON line with training tokens/s, MFU against the bf16 dense MFMA peak, the
roofline of the step's dominant kernel (timed live with HIP events over the
timed region) and the CPU oracle timed on the host cores as a baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic as syn  # noqa: E402

METRIC = "GPT-2 124M train tokens/sec (fwd+bwd+AdamW, T=1024) + bf16 MFU % on 1 GPU"
PEAK_BF16 = 2.5e15     # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12      # MI355X HBM3E, bytes/s


def flops_per_token(m: syn.Model, T: int) -> int:
    """6 N per trained token plus causal attention (6 L C (T+1)): the score and
    value products, forward and backward, over the j <= i half of each row.
    N counts every parameter once (a tied head's products are wte's); an untied
    model's wte is only looked up, so it is left out of N."""
    n = syn.n_params_exact(m) - (m.vocab * m.n_embd if m.untied else 0)
    return 6 * n + 6 * m.n_layer * m.n_embd * (T + 1)


def kernel_work(label: str, w: syn.Workload):
    """(bound, algorithmic work per step for this label, unit) for the roofline."""
    m = w.model
    M, C, F, V, L, H = w.batch * w.seq, m.n_embd, m.mlp_hidden, m.vocab, m.n_layer, m.n_head
    T, B = w.seq, w.batch
    gemm = {"qkv": 2 * M * 3 * C * C, "proj": 2 * M * C * C, "fc": 2 * M * F * C, "fc2": 2 * M * C * F,
            "head": 2 * M * V * C}
    if label.startswith("gemm."):
        _, kind, which = label.split(".")
        per = gemm[which]
        return "mfma", per * (1 if which == "head" else L), "TFLOP/s"
    causal = B * H * (T * (T + 1) // 2) * (C // H) * 2   # one causal T x T x d product
    if label == "attn.fwd":
        return "mfma", 2 * causal * L, "TFLOP/s"
    # backward: 4 causal products per layer (dV, dP, dK, dQ); the dK/dV kernel is
    # credited with dV, dP and dK, the dQ kernel with dQ (recomputed S and dP are
    # not counted as algorithmic work)
    if label == "attn.bwd":
        return "mfma", 4 * causal * L, "TFLOP/s"
    if label == "attn.bwd.dkdv":
        return "mfma", 3 * causal * L, "TFLOP/s"
    if label == "attn.bwd.dq":
        return "mfma", causal * L, "TFLOP/s"
    Vp = (V + 127) // 128 * 128
    n = syn.n_params_exact(m)
    bytes_ = {
        "ce": M * Vp * 2 * 2 + M * 8,                 # read logits, write dlogits (bf16)
        "adamw": n * (4 * 4 + 3 * 4 + 2),             # read p, g, m, v; write p, m, v, bf16 p
        "gradnorm": n * 4,
        "ln.fwd": (2 * L + 1) * M * C * (4 + 2),      # fp32 in, bf16 out
        "ln.bwd": (2 * L + 1) * M * C * (4 * 4 + 2),  # dy, x, dres in/out (fp32), bf16 copy
        "embed.fwd": M * C * 4 * 3,
        "embed.bwd": M * C * 4 * 2,
    }
    if label in bytes_:
        return "hbm", bytes_[label], "GB/s"
    return None, None, None


LABELS = ["gemm.fwd.qkv", "gemm.fwd.proj", "gemm.fwd.fc", "gemm.fwd.fc2", "gemm.fwd.head",
          "gemm.dgrad.head", "gemm.wgrad.head", "gemm.dgrad.fc2", "gemm.wgrad.fc2", "gemm.dgrad.fc",
          "gemm.wgrad.fc", "gemm.dgrad.proj", "gemm.wgrad.proj", "gemm.dgrad.qkv", "gemm.wgrad.qkv",
          "attn.fwd", "attn.bwd.dq", "attn.bwd.dkdv", "ln.fwd", "ln.bwd", "ce", "loss", "colsum",
          "bias", "embed.fwd", "embed.bwd", "gradnorm", "adamw", "dropout.mask"]


# Labels whose launches run with no other work of the step beside them: the
# forward pass, the head's input gradient, the optimizer. The rest of the
# backward overlaps the weight gradients, which run on the library's second
# stream, so a per-launch duration there covers a kernel and its neighbour
# sharing the GPU; the roofline kernel is the largest of these labels.
SOLO = {"gemm.fwd.qkv", "gemm.fwd.proj", "gemm.fwd.fc", "gemm.fwd.fc2", "gemm.fwd.head", "gemm.dgrad.head",
        "attn.fwd", "ln.fwd", "ce", "loss", "embed.fwd", "gradnorm", "adamw"}

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gpt2_124m_12x1024.json")


def measured_traffic(label: str):
    """HBM bytes per launch of `label` (FETCH_SIZE + WRITE_SIZE, calibrated on a
    copy of known size; written by bench_traffic.py), or None when there is no
    measurement or the kernel sources changed after it was taken."""
    try:
        import bench_traffic
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
        if t.get("source_sha256") != bench_traffic.source_hash():
            return None
        e = t["labels"][label]
        return {"bytes": e["fetch_size_bytes_per_launch"] + e["write_size_bytes_per_launch"],
                "fetch": e["fetch_size_bytes_per_launch"], "write": e["write_size_bytes_per_launch"]}
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w: syn.Workload, named: dict, seq: int):
    """The oracle (fp32 instantiation, as it stands) on one sequence of `seq`
    tokens, forward + backward, plus one AdamW pass over every parameter;
    extrapolated to the full batch (B*T/seq sequences) to give tokens/s."""
    import numpy as np
    import oracle as o
    if not os.path.exists(o.LIB_PATH):
        from oracle import build
        build.build()
    m = w.model
    cfg = o.make_cfg(m.vocab, m.block_size, m.n_embd, m.n_head, m.n_layer, m.mlp_hidden, m.bias, m.ln_eps,
                     gelu_erf=m.gelu_erf, untied=m.untied)
    p = o.pack(cfg, named, np.float32)
    g = np.zeros_like(p)
    x, y = syn.batch(w, step=0, B=1, T=seq)
    t0 = time.perf_counter()
    o.step(cfg, 1, seq, p, x, y, g)
    t1 = time.perf_counter()
    mm = np.zeros_like(p)
    vv = np.zeros_like(p)
    o.adamw(p, g, mm, vv, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1)
    t2 = time.perf_counter()
    per_step = (t1 - t0) * (w.batch * w.seq / seq) + (t2 - t1)
    return {"value": round(w.batch * w.seq / per_step, 3), "unit": "tokens/s", "cores": o.max_threads(),
            "kind": "oracle",
            "sample": f"fp32 oracle, 1 sequence x {seq} tokens fwd+bwd ({t1 - t0:.2f} s) extrapolated x"
                      f"{w.batch * w.seq // seq} to the {w.batch}x{w.seq} batch, plus one AdamW pass over all "
                      f"{syn.n_params_exact(m)} parameters ({t2 - t1:.2f} s)"}


def bench_generate(args, b):
    """Generation with the key/value cache: B sequences, a Zipf prompt of P tokens,
    N new tokens at temperature 1. A position step runs B rows through the model;
    P + N - 1 steps feed the prompt and every new token but the last, and the N
    steps that end a feed also run the head and the sampler. Throughput is new
    tokens per second (B N / time, prompt included in the time) and position
    rows per second. The roofline is HBM: one position step reads every weight
    once (bf16 copy), so its algorithmic bytes are 2 bytes per flat-buffer element
    (without the head's on steps that skip it), timed per label."""
    import numpy as np
    import torch
    w = syn.WORKLOADS[args.workload]
    m = w.model
    B, P, N = args.gen_batch, args.gen_prompt, args.gen_new
    if P + N > m.block_size:
        sys.exit("prompt + new tokens must fit in block_size for this measurement (no window slide)")
    cfg = b.make_config(m.vocab, m.block_size, m.n_embd, m.n_head, m.n_layer, m.mlp_hidden, m.bias, b.DTYPE_BF16,
                        m.ln_eps, gelu_erf=m.gelu_erf, untied_head=m.untied)
    g = b.Model(cfg, B, m.block_size, b.MODE_GENERATE)
    g.load_named(syn.init_params(m))
    g.init()
    rng = np.random.default_rng(syn.DATA_SEED)
    prompt = torch.from_numpy(syn.draw_tokens(rng, m.vocab, B * P, "zipf", w.zipf_s).reshape(B, P)).cuda()
    u = torch.from_numpy(rng.random((B, N)).astype(np.float32)).cuda()
    out = torch.empty((B, P + N), dtype=torch.int32, device="cuda")
    g.generate(prompt, N, 1.0, u, out)  # warm-up
    torch.cuda.synchronize()
    labels = ["gen.embed", "gen.ln", "gen.gemm", "gen.attn", "gen.head", "gen.sample"]
    breakdown = {}
    for lab in labels:
        g.timing_begin(lab)
        g.generate(prompt, N, 1.0, u, out)
        ms, n = g.timing_end()
        breakdown[lab] = {"ms": round(ms, 4), "launches": n}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(1, args.steps // 5)
    ev0.record()
    for _ in range(reps):
        g.generate(prompt, N, 1.0, u, out)
    ev1.record()
    torch.cuda.synchronize()
    sec = ev0.elapsed_time(ev1) / 1e3 / reps
    status = g.sync_status()
    steps = P + N - 1
    n_head = sum(int(np.prod(d["shape"])) for d in g.table if d["name"] == ("lm_head" if m.untied else "wte"))
    n_body = g.n_flat - g.vocab_pad * m.n_embd * (2 if m.untied else 1)  # layer and LN weights (+ wpe)
    gemm_ms = breakdown["gen.gemm"]["ms"] / breakdown["gen.gemm"]["launches"] * 4 * m.n_layer  # per step
    body_bytes = 2 * (n_body - m.block_size * m.n_embd)
    head_ms = breakdown["gen.head"]["ms"] / max(1, breakdown["gen.head"]["launches"])
    head_bytes = 2 * g.vocab_pad * m.n_embd
    out_line = {
        "metric": "GPT-2 124M generation, new tokens/sec with the key/value cache (bf16 weights)",
        "value": round(B * N / sec, 1), "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic (Zipf s=1.05 prompts, N(0,0.02) init, uniform draws)",
        "config": {"workload": f"{w.name}: B={B} sequences, prompt {P}, {N} new tokens, temperature 1",
                   "batch": B, "prompt": P, "new_tokens": N},
        "ms_per_generate": round(sec * 1e3, 3), "position_rows_per_s": round(B * steps / sec, 1),
        "status": status,
        "roofline": {"bound": "hbm", "kernel": "gen.gemm (the four layer products of one position step)",
                     "achieved": round(body_bytes / (gemm_ms / 1e3) / 1e9, 2), "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": round(body_bytes / (gemm_ms / 1e3) / PEAK_HBM, 4), "traffic": None,
                     "bytes_per_step": body_bytes, "ms_per_step": round(gemm_ms, 4)},
        "head_roofline": {"achieved": round(head_bytes / (head_ms / 1e3) / 1e9, 2), "unit": "GB/s",
                          "ms_per_launch": round(head_ms, 4), "bytes": head_bytes},
        "breakdown": breakdown,
    }
    print(json.dumps(out_line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2_124m", choices=["gpt2_124m", "gpt2_124m_literal"],
                    help="gpt2_124m_literal: the same model with exact erf GELU and an untied lm_head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seq", type=int, default=1024, help="tokens in the oracle's timed sample")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-kernel-class timing pass")
    ap.add_argument("--roofline-kernel", default=None, help="timing label for the roofline (default: the "
                    "label with the largest time in the breakdown pass)")
    ap.add_argument("--dropout", type=float, default=0.0, help="training-mode dropout p (the minigpt page's "
                    "literal model uses 0.1); fresh masks every step")
    ap.add_argument("--generate", action="store_true", help="measure generation instead of the training step "
                    "(prints its own JSON line)")
    ap.add_argument("--gen-batch", type=int, default=12)
    ap.add_argument("--gen-prompt", type=int, default=32)
    ap.add_argument("--gen-new", type=int, default=64)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    from decoder_only_transformer_04_amd import binding as b

    if args.generate:
        bench_generate(args, b)
        return
    w = syn.WORKLOADS[args.workload]
    m = w.model
    cfg = b.make_config(m.vocab, m.block_size, m.n_embd, m.n_head, m.n_layer, m.mlp_hidden, m.bias, b.DTYPE_BF16,
                        m.ln_eps, gelu_erf=m.gelu_erf, untied_head=m.untied,
                        dropout=args.dropout)
    named = syn.init_params(m)
    g = b.Model(cfg, w.batch, w.seq, b.MODE_TRAIN)
    g.load_named(named)
    g.init()
    nb = args.warmup + args.steps + len(LABELS)
    xs, ys = [], []
    for k in range(nb):
        x, y = syn.batch(w, step=k)
        xs.append(torch.from_numpy(x.reshape(-1)).cuda())
        ys.append(torch.from_numpy(y.reshape(-1)).cuda())
    torch.cuda.synchronize()
    t = 0

    def step(k):
        nonlocal t
        t += 1
        if args.dropout > 0:
            g.set_dropout_seed(k)
        g.forward(xs[k], ys[k])
        g.backward(1.0, True)
        g.adamw_step(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # per-kernel-class time of one step each (untimed), to name the dominant kernel
    breakdown = {}
    if not args.no_breakdown:
        for i, lab in enumerate(LABELS):
            g.timing_begin(lab)
            step(args.warmup + i)
            ms, n = g.timing_end()
            breakdown[lab] = round(ms, 4)
    if args.roofline_kernel:
        dominant = args.roofline_kernel
    elif breakdown:
        dominant = max((l for l in breakdown if kernel_work(l, w)[0] and l in SOLO), key=lambda l: breakdown[l])
    else:
        dominant = "gemm.fwd.head"
    if kernel_work(dominant, w)[0] is None:
        sys.exit(f"no roofline work defined for label {dominant!r}")

    # timed region: exactly K steps, the dominant kernel's launches bracketed by events
    base = args.warmup + len(LABELS)
    torch.cuda.synchronize()
    g.timing_begin(dominant)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for k in range(args.steps):
        step(base + k)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom_ms, dom_n = g.timing_end()
    status = g.sync_status()
    loss = float(g.loss.item())
    elapsed = max(ev0.elapsed_time(ev1) / 1e3, 1e-9)
    wall = t1 - t0
    tokens = w.batch * w.seq * args.steps
    value = tokens / elapsed
    fpt = flops_per_token(m, w.seq)
    mfu = value * fpt / PEAK_BF16
    bound, work, unit = kernel_work(dominant, w)
    launches_per_step = max(1, dom_n // max(args.steps, 1))
    avg_launch_s = dom_ms / 1e3 / max(dom_n, 1)
    per_launch = work / launches_per_step
    if bound == "mfma":
        achieved = per_launch / avg_launch_s / 1e12
        peak = PEAK_BF16 / 1e12
    else:
        achieved = per_launch / avg_launch_s / 1e9
        peak = PEAK_HBM / 1e9
    tr = measured_traffic(dominant)
    roofline = {"bound": bound, "kernel": dominant, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": round(tr["bytes"]) if tr else None,
                "traffic_fetch_write": [round(tr["fetch"]), round(tr["write"])] if tr else None,
                "avg_launch_ms": round(avg_launch_s * 1e3, 4), "launches_timed": dom_n,
                "work_per_launch": per_launch}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (Zipf s=1.05 token ids, N(0,0.02) init, seeds 1234/5678)",
        "config": {"workload": ("gpt2_124m: V50257 T1024 C768 H12 L12 F3072, biases, tied head; "
                                "micro-batch 12 x 1024, one fwd+bwd+AdamW per step") if not m.untied else
                               ("gpt2_124m_literal: V50257 T1024 C768 H12 L12 F3072, biases, exact erf GELU, "
                                "untied lm_head; micro-batch 12 x 1024, one fwd+bwd+AdamW per step"),
                   "global_batch": w.batch, "seq_len": w.seq, "parallelism": "none (1 GPU)",
                   "dropout": args.dropout},
        "mfu": round(mfu, 4),
        "flops_per_token": fpt,
        "wall_s": round(wall, 3),
        "final_loss": round(loss, 5),
        "status": status,
        "roofline": roofline,
        "breakdown_ms_per_step": breakdown,
    }
    if not args.no_cpu_baseline and args.dropout == 0:  # the oracle baseline times the plain step
        out["cpu_baseline"] = cpu_baseline(w, named, args.cpu_seq)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
