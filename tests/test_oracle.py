"""Pins for the CPU oracle: checks against things other than the oracle itself.

- whole-model gradients against central finite differences (double);
- the whole model against an independent torch-CPU autograd model built from
  library primitives (F.layer_norm, F.linear, scaled_dot_product_attention,
  F.gelu(approximate="tanh"), F.cross_entropy) in float64, also for the minigpt
  page's literal variants (exact erf GELU, a separate lm_head);
- closed forms and invariants: initial loss ~ ln V, LayerNorm moments, softmax
  rows, the causal mask, the worked softmax example printed on the minigpt page,
  GELU identities, AdamW's first step, the LR schedule, clipping, parameter counts.
"""
import math
import os

import numpy as np
import pytest

import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ocfg(o, m: syn.Model):
    return o.make_cfg(m.vocab, m.block_size, m.n_embd, m.n_head, m.n_layer, m.mlp_hidden, m.bias, m.ln_eps,
                      gelu_erf=m.gelu_erf, untied=m.untied)


def rand_named(m: syn.Model, seed, std=0.3):
    """Non-degenerate parameters: all tensors random (LayerNorm gains around 1)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in syn.tensor_shapes(m):
        base = name.split(".")[-1]
        if base.endswith("_g"):
            out[name] = 1.0 + 0.2 * rng.standard_normal(shape)
        else:
            out[name] = std * rng.standard_normal(shape)
    return out


TINY = syn.Model(vocab=11, block_size=8, n_embd=16, n_head=2, n_layer=2, mlp_hidden=64, bias=True)
TINY_NB = syn.Model(vocab=11, block_size=8, n_embd=16, n_head=2, n_layer=2, mlp_hidden=64, bias=False)
# the minigpt page's literal model: exact erf GELU, lm_head of its own
TINY_LIT = syn.Model(vocab=11, block_size=8, n_embd=16, n_head=2, n_layer=2, mlp_hidden=64, bias=True,
                     gelu_erf=True, untied=True)


def tiny_batch(m, B, T, seed):
    rng = np.random.default_rng(seed)
    x = rng.integers(0, m.vocab, size=(B, T)).astype(np.int32)
    y = rng.integers(0, m.vocab, size=(B, T)).astype(np.int32)
    return x, y


# ----------------------------------------------------------------- finite differences
@pytest.mark.parametrize("model", [TINY, TINY_NB, TINY_LIT], ids=["bias", "nobias", "erf_untied"])
def test_gradients_match_finite_differences(oracle, model):
    cfg = ocfg(oracle, model)
    B, T = 2, 8
    named = rand_named(model, 1)
    p = oracle.pack(cfg, named, np.float64)
    x, y = tiny_batch(model, B, T, 2)
    scale = 0.7
    g = np.zeros_like(p)
    loss, _, _ = oracle.step(cfg, B, T, p, x, y, g, loss_scale=scale)
    assert np.isfinite(loss)
    rng = np.random.default_rng(3)
    for name, off, shape in oracle.param_table(cfg):
        n = int(np.prod(shape))
        picks = np.arange(n) if n <= 48 else rng.choice(n, size=48, replace=False)
        fd = np.empty(len(picks))
        for i, j in enumerate(picks):
            h = 1e-6 * max(1.0, abs(p[off + j]))
            pp = p.copy(); pp[off + j] += h
            lp, _, _ = oracle.step(cfg, B, T, pp, x, y)
            pm = p.copy(); pm[off + j] -= h
            lm, _, _ = oracle.step(cfg, B, T, pm, x, y)
            fd[i] = scale * (lp - lm) / (2 * h)
        an = g[off + picks]
        err = np.max(np.abs(an - fd)) / max(np.max(np.abs(fd)), 1e-30)
        assert err <= 1e-5, (name, err)


def test_fp32_instantiation_tracks_fp64(oracle):
    m = syn.WORKLOADS["tiny_f32"].model
    cfg = ocfg(oracle, m)
    B, T = 4, 64
    named = syn.init_params(m)
    x, y = syn.batch(syn.WORKLOADS["tiny_f32"])
    p64 = oracle.pack(cfg, named, np.float64)
    p32 = oracle.pack(cfg, named, np.float32)
    g64 = np.zeros_like(p64)
    g32 = np.zeros_like(p32)
    l64, _, _ = oracle.step(cfg, B, T, p64, x, y, g64)
    l32, _, _ = oracle.step(cfg, B, T, p32, x, y, g32)
    assert abs(l32 - l64) / abs(l64) <= 1e-6
    for name, off, shape in oracle.param_table(cfg):
        n = int(np.prod(shape))
        a, r = g32[off:off + n].astype(np.float64), g64[off:off + n]
        assert np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-30) <= 1e-4, name


# ----------------------------------------------------------------- independent torch model
def torch_model_loss(named, m: syn.Model, x, y, scale=1.0, masks=None):
    """masks (training-mode dropout): {(layer, site): keep flags} with the
    attention site [B, H, T, T] and the residual sites [B, T, C], plus "p"."""
    import torch
    import torch.nn.functional as F
    P = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in named.items()}
    B, T = x.shape
    C, H = m.n_embd, m.n_head
    d = C // H
    idx = torch.tensor(x, dtype=torch.long)
    h = P["wte"][idx] + P["wpe"][:T]

    def drop(t, l, site):  # nn.Dropout in training mode with a given keep mask
        if masks is None:
            return t
        return t * torch.tensor(masks[(l, site)], dtype=torch.float64) / (1.0 - masks["p"])

    for l in range(m.n_layer):
        q = lambda s: P[f"h{l}.{s}"] if f"h{l}.{s}" in P else None
        a = F.layer_norm(h, (C,), q("ln1_g"), q("ln1_b"), eps=m.ln_eps)
        qkv = F.linear(a, q("w_qkv"), q("b_qkv"))
        qq, kk, vv = qkv.split(C, dim=-1)
        qq = qq.view(B, T, H, d).transpose(1, 2)
        kk = kk.view(B, T, H, d).transpose(1, 2)
        vv = vv.view(B, T, H, d).transpose(1, 2)
        if masks is None:
            att = F.scaled_dot_product_attention(qq, kk, vv, is_causal=True)
        else:  # Head.forward: masked softmax of the scaled scores, dropout, weights @ v
            wei = (qq @ kk.transpose(-2, -1)) / math.sqrt(d)
            wei = wei.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
            att = drop(torch.softmax(wei, dim=-1), l, 0) @ vv
        att = att.transpose(1, 2).reshape(B, T, C)
        h = h + drop(F.linear(att, q("w_proj"), q("b_proj")), l, 1)
        a2 = F.layer_norm(h, (C,), q("ln2_g"), q("ln2_b"), eps=m.ln_eps)
        gelu = F.gelu(F.linear(a2, q("w_fc"), q("b_fc")), approximate="none" if m.gelu_erf else "tanh")
        h = h + drop(F.linear(gelu, q("w_fc2"), q("b_fc2")), l, 2)
    hf = F.layer_norm(h, (C,), P["lnf_g"], P["lnf_b"], eps=m.ln_eps)
    logits = hf @ (P["lm_head"] if m.untied else P["wte"]).T
    if y is None:
        return logits.detach().numpy()
    loss = F.cross_entropy(logits.view(-1, m.vocab), torch.tensor(y, dtype=torch.long).view(-1))
    (loss * scale).backward()
    return float(loss.detach()), {k: v.grad.numpy() for k, v in P.items()}


@pytest.mark.parametrize("model", [TINY, TINY_NB, syn.Model(13, 16, 24, 3, 3, 96, True), TINY_LIT,
                                   syn.Model(13, 16, 24, 3, 3, 96, False, untied=True)],
                         ids=["bias", "nobias", "h3", "erf_untied", "untied_tanh"])
def test_oracle_matches_independent_torch_model(oracle, model):
    cfg = ocfg(oracle, model)
    B, T = 3, model.block_size
    named = rand_named(model, 11)
    x, y = tiny_batch(model, B, T, 12)
    p = oracle.pack(cfg, named, np.float64)
    g = np.zeros_like(p)
    loss, _, _ = oracle.step(cfg, B, T, p, x, y, g, loss_scale=0.5)
    tl, tg = torch_model_loss(named, model, x, y, scale=0.5)
    assert abs(loss - tl) <= 1e-12 * abs(tl)
    og = oracle.unpack(cfg, g)
    for name in og:
        r = tg[name]
        assert np.max(np.abs(og[name] - r)) <= 1e-10 * max(1.0, np.max(np.abs(r))), name


# ----------------------------------------------------------------- dropout
def test_philox_known_answer_vectors(oracle):
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(w, 16) for w in line.split()])
    assert len(rows) == 3
    for r in rows:
        out = oracle.philox4x32_10(r[0:4], r[4:6])
        assert [int(v) for v in out] == r[6:10], [hex(v) for v in out]


def test_dropout_keep_rate_and_independence(oracle):
    """Each element is kept with probability 1 - round(65536 p) / 65536 (a
    binomial 6-sigma band over 2M draws); p = 0 keeps everything; sites, layers
    and seeds draw different masks; a stretch equals the same stretch of a longer
    run (element e is a function of e alone)."""
    n = 2_000_000
    for p in (0.1, 0.5):
        k = oracle.dropout_keep(p, 99, oracle.DROP_ATTN, 0, n)
        q = 1.0 - round(65536 * p) / 65536
        assert abs(k.mean() - q) <= 6 * math.sqrt(q * (1 - q) / n), (p, k.mean())
    assert oracle.dropout_keep(0.0, 99, oracle.DROP_PROJ, 3, 4096).all()
    a = oracle.dropout_keep(0.5, 7, oracle.DROP_PROJ, 1, 4096)
    for other in (oracle.dropout_keep(0.5, 7, oracle.DROP_FC2, 1, 4096),
                  oracle.dropout_keep(0.5, 7, oracle.DROP_PROJ, 2, 4096),
                  oracle.dropout_keep(0.5, 8, oracle.DROP_PROJ, 1, 4096)):
        assert 0.4 < np.mean(a == other) < 0.6
    np.testing.assert_array_equal(oracle.dropout_keep(0.5, 7, oracle.DROP_PROJ, 1, 1000, e0=1234),
                                  oracle.dropout_keep(0.5, 7, oracle.DROP_PROJ, 1, 4096)[1234:2234])
    # element e uses half e mod 8 of Philox at counter e / 8: low half of word 0 first
    r = oracle.philox4x32_10([5, 0, oracle.DROP_FC2, 2], [7, 0])
    halves = np.array([[w & 0xFFFF, w >> 16] for w in r.tolist()]).ravel()
    np.testing.assert_array_equal(oracle.dropout_keep(0.5, 7, oracle.DROP_FC2, 2, 8, e0=40),
                                  (halves >= 32768).astype(np.uint8))


def dropout_masks(oracle, m: syn.Model, B, T, p, seed):
    masks = {"p": p}
    C, H = m.n_embd, m.n_head
    for l in range(m.n_layer):
        masks[(l, 0)] = oracle.dropout_keep(p, seed, oracle.DROP_ATTN, l, B * H * T * T).reshape(B, H, T, T)
        masks[(l, 1)] = oracle.dropout_keep(p, seed, oracle.DROP_PROJ, l, B * T * C).reshape(B, T, C)
        masks[(l, 2)] = oracle.dropout_keep(p, seed, oracle.DROP_FC2, l, B * T * C).reshape(B, T, C)
    return masks


@pytest.mark.parametrize("model", [TINY, TINY_LIT], ids=["gpt2", "literal"])
def test_dropout_step_matches_torch_model(oracle, model):
    """Training-mode dropout (p = 0.1) at the three sites of minigpt.py's block
    -- the attention weights after the softmax, the projection output and the
    FeedForward output -- against torch with the same keep masks: loss and every
    gradient."""
    p, seed = 0.1, 2024
    cfg = oracle.make_cfg(model.vocab, model.block_size, model.n_embd, model.n_head, model.n_layer,
                          model.mlp_hidden, model.bias, model.ln_eps, gelu_erf=model.gelu_erf,
                          untied=model.untied, dropout=p, seed=seed)
    B, T = 3, model.block_size
    named = rand_named(model, 31)
    x, y = tiny_batch(model, B, T, 32)
    pf = oracle.pack(cfg, named, np.float64)
    g = np.zeros_like(pf)
    loss, _, _ = oracle.step(cfg, B, T, pf, x, y, g)
    masks = dropout_masks(oracle, model, B, T, p, seed)
    assert 0 < sum(int((masks[k] == 0).sum()) for k in masks if k != "p")   # something was dropped
    tl, tg = torch_model_loss(named, model, x, y, masks=masks)
    assert abs(loss - tl) <= 1e-12 * abs(tl)
    og = oracle.unpack(cfg, g)
    for name in og:
        r = tg[name]
        assert np.max(np.abs(og[name] - r)) <= 1e-10 * max(1.0, np.max(np.abs(r))), name
    # the eval-mode model (and p = 0) has no dropout at all
    l0, _, _ = oracle.step(oracle.eval_cfg(cfg), B, T, pf, x, y)
    assert abs(l0 - torch_model_loss(named, model, x, y)[0]) <= 1e-12 * abs(l0)
    assert l0 != loss


def test_shorter_sequence_than_block_size(oracle):
    """T < block_size uses positions 0..T-1 only (forward asserts T <= block_size)."""
    m = TINY
    cfg = ocfg(oracle, m)
    named = rand_named(m, 21)
    x, y = tiny_batch(m, 2, 5, 22)
    p = oracle.pack(cfg, named, np.float64)
    g = np.zeros_like(p)
    loss, _, _ = oracle.step(cfg, 2, 5, p, x, y, g)
    tl, tg = torch_model_loss(named, m, x, y)
    assert abs(loss - tl) <= 1e-12 * abs(tl)
    wpe = oracle.unpack(cfg, g)["wpe"]
    assert np.all(wpe[5:] == 0)
    np.testing.assert_allclose(wpe[:5], tg["wpe"][:5], rtol=0, atol=1e-10)


def test_rejects_bad_inputs(oracle):
    m = TINY
    cfg = ocfg(oracle, m)
    p = oracle.pack(cfg, rand_named(m, 1), np.float64)
    x, y = tiny_batch(m, 1, 8, 1)
    bad = x.copy(); bad[0, 3] = m.vocab
    assert math.isnan(oracle.step(cfg, 1, 8, p, bad, y)[0])
    assert math.isnan(oracle.step(cfg, 1, 9, p, np.zeros((1, 9), np.int32), np.zeros((1, 9), np.int32))[0])


# ----------------------------------------------------------------- loss at init
@pytest.mark.parametrize("wname", ["tiny_f32", "char_bf16"])
def test_initial_loss_near_ln_vocab(oracle, wname):
    w = syn.WORKLOADS[wname]
    m = w.model
    cfg = ocfg(oracle, m)
    B, T = (4, 64) if wname == "tiny_f32" else (2, 256)
    p = oracle.pack(cfg, syn.init_params(m), np.float64)
    x, y = syn.batch(w, B=B, T=T)
    # targets independent of the logits: for small logits E[loss] ~ ln V + var/2
    yu = np.random.default_rng(13).integers(0, m.vocab, size=y.shape).astype(np.int32)
    loss, logits, _ = oracle.step(cfg, B, T, p, x, yu, want_logits=True)
    s2 = float(np.mean(np.var(logits, axis=1)))
    assert abs(loss - (math.log(m.vocab) + s2 / 2)) < 0.05
    loss_y, _, _ = oracle.step(cfg, B, T, p, x, y)
    assert abs(loss_y - math.log(m.vocab)) < 0.1


def test_initial_loss_124m_slice(oracle):
    m = syn.GPT2_124M
    # one short sequence through the full-width 124M model (two layers suffice for the check)
    m2 = syn.Model(m.vocab, m.block_size, m.n_embd, m.n_head, 2, m.mlp_hidden, True)
    cfg = ocfg(oracle, m2)
    p = oracle.pack(cfg, syn.init_params(m2), np.float32)
    x, y = syn.batch(syn.WORKLOADS["gpt2_124m"], B=1, T=32)
    loss, _, _ = oracle.step(cfg, 1, 32, p, x, y)
    assert abs(loss - math.log(50257)) < 0.3


def test_zero_logits_give_exactly_ln_v(oracle):
    m = TINY
    cfg = ocfg(oracle, m)
    named = rand_named(m, 5)
    named["wte"] = np.zeros_like(named["wte"])
    p = oracle.pack(cfg, named, np.float64)
    x, y = tiny_batch(m, 2, 8, 6)
    loss, _, _ = oracle.step(cfg, 2, 8, p, x, y)
    assert abs(loss - math.log(m.vocab)) <= 1e-14


# ----------------------------------------------------------------- LayerNorm
def test_layernorm_moments(oracle):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 768)) * 3 + 1.5
    y, mean, rstd = oracle.layernorm(x, np.ones(768), np.zeros(768), eps=1e-5)
    var = np.var(x, axis=1)
    assert np.max(np.abs(y.mean(axis=1))) <= 1e-12
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-13)
    np.testing.assert_allclose(rstd, 1 / np.sqrt(var + 1e-5), rtol=1e-12)
    # gain and bias act per channel
    g = rng.standard_normal(768); b = rng.standard_normal(768)
    y2, _, _ = oracle.layernorm(x, g, b)
    np.testing.assert_allclose(y2, y * g + b, rtol=1e-12, atol=1e-12)


def test_layernorm_backward_is_projection(oracle):
    """With g = 1 and eps = 0 the input gradient is orthogonal to 1 and to xhat
    (LayerNorm output is invariant to shifting and scaling its input row)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 96))
    y, mean, rstd = oracle.layernorm(x, np.ones(96), np.zeros(96), eps=0.0)
    dy = rng.standard_normal((16, 96))
    dx, dg, db = oracle.layernorm_bwd(dy, x, mean, rstd, np.ones(96))
    assert np.max(np.abs(dx.sum(axis=1))) < 1e-12
    assert np.max(np.abs((dx * y).sum(axis=1))) < 1e-10
    np.testing.assert_allclose(db, dy.sum(axis=0), rtol=1e-13)
    np.testing.assert_allclose(dg, (dy * y).sum(axis=0), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------- attention / softmax
def read_golden_softmax():
    scores, printed, tol = [], [], None
    with open(os.path.join(GOLDEN, "softmax_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            if k == "scores":
                scores.append([float(t) for t in v])
            elif k == "printed":
                printed.append([float(t) for t in v])
            elif k == "tol":
                tol = float(v[0])
    return np.array(scores), np.array(printed), tol


def test_softmax_worked_example_from_page(oracle):
    S, printed, tol = read_golden_softmax()
    T = 3
    d = 3
    # q_i . k_j / sqrt(d) = S[i, j] with k_j = sqrt(d) e_j and q_i = S[i]; v = I gives out = P
    k = math.sqrt(d) * np.eye(T)
    out, P = oracle.head_attention(S.copy(), k, np.eye(T))
    np.testing.assert_allclose(P, out, rtol=0, atol=1e-15)
    assert np.max(np.abs(P - printed)) <= tol
    exact = [[1, 0, 0], [0.4256, 0.5744, 0], [0.1769, 0.2917, 0.5314]]
    np.testing.assert_allclose(P, exact, atol=1e-4)


def test_causal_mask_and_row_sums(oracle):
    mask = np.loadtxt(os.path.join(GOLDEN, "causal_mask_4x4.txt"))
    rng = np.random.default_rng(2)
    T, d = 4, 8
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    out, P = oracle.head_attention(q, k, v)
    assert np.all(P[mask == 0] == 0.0)          # exactly zero above the diagonal
    assert np.all(P[mask == 1] > 0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    T = 64
    q, k, v = (rng.standard_normal((T, 32)) * 4 for _ in range(3))
    out, P = oracle.head_attention(q, k, v)
    assert np.all(np.triu(P, 1) == 0.0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(out, P @ v, atol=1e-13)
    assert np.all(np.isfinite(out))


def test_attention_special_cases(oracle):
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, 16))
    out, _ = oracle.head_attention(rng.standard_normal((1, 16)), rng.standard_normal((1, 16)), v)
    assert np.array_equal(out, v)               # T = 1: attends only to itself
    T = 10
    v = rng.standard_normal((T, 16))
    out, P = oracle.head_attention(np.zeros((T, 16)), rng.standard_normal((T, 16)), v)
    np.testing.assert_allclose(P, np.tril(np.ones((T, T))) / np.arange(1, T + 1)[:, None], atol=1e-15)
    np.testing.assert_allclose(out, np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None], atol=1e-14)


def test_fused_qkv_equals_per_head_modules(oracle):
    """Fused [3C, C] QKV with head h at rows h*d of each third equals separate
    per-head query/key/value Linears followed by concatenation (minigpt Head and
    MultiHeadAttention)."""
    rng = np.random.default_rng(4)
    B, T, C, H = 2, 12, 24, 3
    d = C // H
    x = rng.standard_normal((B * T, C))
    W = rng.standard_normal((3 * C, C)) * 0.3
    fused = oracle.attention(oracle.linear(x, W), B, T, C, H)
    outs = []
    for h in range(H):
        Wq, Wk, Wv = W[h * d:(h + 1) * d], W[C + h * d:C + (h + 1) * d], W[2 * C + h * d:2 * C + (h + 1) * d]
        per_b = []
        for b in range(B):
            xb = x[b * T:(b + 1) * T]
            q, k, v = xb @ Wq.T, xb @ Wk.T, xb @ Wv.T
            wei = (q @ k.T) * d ** -0.5
            wei = np.where(np.tril(np.ones((T, T), bool)), wei, -np.inf)
            wei = np.exp(wei - wei.max(axis=1, keepdims=True))
            wei /= wei.sum(axis=1, keepdims=True)
            per_b.append(wei @ v)
        outs.append(np.concatenate(per_b, axis=0))
    ref = np.concatenate(outs, axis=1)
    np.testing.assert_allclose(fused, ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- GELU
def test_gelu_identities(oracle):
    u = np.linspace(-8, 8, 4001)
    y, dy = oracle.gelu(u)
    assert y[2000] == 0.0                                       # GELU(0) = 0
    np.testing.assert_allclose(y - y[::-1], u, atol=1e-14)      # GELU(u) - GELU(-u) = u
    exact = np.array([0.5 * t * (1 + math.erf(t / math.sqrt(2))) for t in u])
    assert np.max(np.abs(y - exact)) < 5e-4                     # tanh form approximates u*Phi(u)
    assert np.max(np.abs(y[u > 6] - u[u > 6])) < 1e-8
    assert np.max(np.abs(y[u < -6])) < 1e-8
    h = 1e-6
    yp, _ = oracle.gelu(u + h)
    ym, _ = oracle.gelu(u - h)
    np.testing.assert_allclose(dy, (yp - ym) / (2 * h), atol=1e-8)


def test_erf_gelu_identities(oracle):
    from scipy.stats import norm
    u = np.linspace(-8, 8, 4001)
    y, dy = oracle.gelu(u, erf_form=True)
    assert y[2000] == 0.0                                       # GELU(0) = 0
    np.testing.assert_allclose(y - y[::-1], u, atol=1e-14)      # Phi(u) + Phi(-u) = 1
    np.testing.assert_allclose(y, u * norm.cdf(u), rtol=1e-13, atol=1e-15)  # u Phi(u), Phi from scipy
    np.testing.assert_allclose(dy, norm.cdf(u) + u * norm.pdf(u), rtol=1e-12, atol=1e-15)
    h = 1e-6
    yp, _ = oracle.gelu(u + h, erf_form=True)
    ym, _ = oracle.gelu(u - h, erf_form=True)
    np.testing.assert_allclose(dy, (yp - ym) / (2 * h), atol=1e-8)
    t, _ = oracle.gelu(u)                                       # the tanh form stays within 5e-4 of it
    assert 0 < np.max(np.abs(t - y)) < 5e-4


def test_erf_gelu_matches_torch_exact_gelu(oracle):
    import torch
    u = np.linspace(-10, 10, 2001)
    y, _ = oracle.gelu(u, erf_form=True)
    ref = torch.nn.functional.gelu(torch.tensor(u), approximate="none").numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-15)


def test_gelu_matches_torch_tanh_gelu(oracle):
    import torch
    u = np.linspace(-10, 10, 2001)
    y, _ = oracle.gelu(u)
    ref = torch.nn.functional.gelu(torch.tensor(u), approximate="tanh").numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-15)


# ----------------------------------------------------------------- cross-entropy
def test_cross_entropy_properties(oracle):
    from scipy.special import logsumexp
    rng = np.random.default_rng(5)
    z = rng.standard_normal((32, 100)) * 5
    y = rng.integers(0, 100, 32).astype(np.int32)
    lr, dz = oracle.cross_entropy(z, y, scale=0.25)
    np.testing.assert_allclose(lr, logsumexp(z, axis=1) - z[np.arange(32), y], rtol=1e-13)
    assert np.all(lr >= 0)
    np.testing.assert_allclose(dz.sum(axis=1), 0, atol=1e-15)
    assert np.all(dz[np.arange(32), y] < 0)
    lr0, _ = oracle.cross_entropy(np.zeros((3, 50257)), np.array([0, 7, 50256], np.int32))
    np.testing.assert_allclose(lr0, math.log(50257), rtol=1e-14)
    zz = np.zeros((1, 10)); zz[0, 3] = 100
    lr1, _ = oracle.cross_entropy(zz, np.array([3], np.int32))
    assert lr1[0] < 1e-40


# ----------------------------------------------------------------- optimiser
def test_adamw_first_and_second_step_closed_form(oracle):
    rng = np.random.default_rng(6)
    p0 = rng.standard_normal(1000)
    g1 = rng.standard_normal(1000)
    g2 = rng.standard_normal(1000)
    lr, b1, b2, eps, wd = 6e-4, 0.9, 0.95, 1e-8, 0.1
    p = p0.copy(); m = np.zeros(1000); v = np.zeros(1000)
    oracle.adamw(p, g1, m, v, lr, b1, b2, eps, wd, 1)
    p1 = p0 * (1 - lr * wd) - lr * g1 / (np.abs(g1) + eps)   # m_hat = g, v_hat = g^2
    np.testing.assert_allclose(p, p1, rtol=1e-14, atol=1e-16)
    oracle.adamw(p, g2, m, v, lr, b1, b2, eps, wd, 2)
    m2 = b1 * (1 - b1) * g1 + (1 - b1) * g2
    v2 = b2 * (1 - b2) * g1 ** 2 + (1 - b2) * g2 ** 2
    p2 = p1 * (1 - lr * wd) - lr * (m2 / (1 - b1 ** 2)) / (np.sqrt(v2 / (1 - b2 ** 2)) + eps)
    np.testing.assert_allclose(p, p2, rtol=1e-13, atol=1e-16)


def test_adamw_matches_torch_adamw(oracle):
    import torch
    rng = np.random.default_rng(7)
    p0 = rng.standard_normal(512)
    tp = torch.tensor(p0.copy(), requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=1e-3, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)
    p = p0.copy(); m = np.zeros(512); v = np.zeros(512)
    for t in range(1, 6):
        g = rng.standard_normal(512)
        tp.grad = torch.tensor(g)
        opt.step()
        oracle.adamw(p, g, m, v, 1e-3, 0.9, 0.95, 1e-8, 0.1, t)
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)
    # decay mask: masked entries follow plain Adam
    p = p0.copy(); m = np.zeros(512); v = np.zeros(512)
    mask = np.zeros(512, np.uint8)
    g = rng.standard_normal(512)
    oracle.adamw(p, g, m, v, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1, decay=mask)
    np.testing.assert_allclose(p, p0 - 1e-3 * g / (np.abs(g) + 1e-8), rtol=1e-14)


def test_lr_schedule_values(oracle):
    assert oracle.lr_at(0) == pytest.approx(3e-7, rel=1e-12)
    assert oracle.lr_at(1999) == pytest.approx(6e-4, rel=1e-12)
    assert oracle.lr_at(2000) == pytest.approx(6e-4, rel=1e-12)
    assert oracle.lr_at(301000) == pytest.approx(3.3e-4, rel=1e-12)
    assert oracle.lr_at(600000) == pytest.approx(6e-5, rel=1e-12)
    assert oracle.lr_at(10 ** 7) == pytest.approx(6e-5, rel=1e-12)
    vals = [oracle.lr_at(i) for i in range(2000, 600000, 1000)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))


def test_clip(oracle):
    rng = np.random.default_rng(8)
    g = rng.standard_normal(10000)
    n0 = float(np.linalg.norm(g))
    gg = g.copy()
    n = oracle.clip(gg, 1.0)
    assert n == pytest.approx(n0, rel=1e-14)
    assert float(np.linalg.norm(gg)) == pytest.approx(1.0 * n0 / (n0 + 1e-6), rel=1e-12)
    small = g * 1e-4
    s2 = small.copy()
    oracle.clip(s2, 1.0)
    assert np.array_equal(s2, small)
    s3 = g.copy()
    oracle.clip(s3, 0.0)
    assert np.array_equal(s3, g)


# ----------------------------------------------------------------- sizes
def read_counts():
    out = {}
    with open(os.path.join(GOLDEN, "param_counts.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


@pytest.mark.parametrize("wname", ["tiny_f32", "char_bf16", "gpt2_124m", "tiny_f32_literal"])
def test_param_counts(oracle, wname):
    import torch.nn as nn
    counts = read_counts()
    m = syn.WORKLOADS[wname].model
    n = oracle.n_params(ocfg(oracle, m))
    assert n == int(counts[wname]) == syn.n_params_exact(m)
    # independent count from torch layers of the same shapes
    mods = [nn.Embedding(m.vocab, m.n_embd), nn.Embedding(m.block_size, m.n_embd), nn.LayerNorm(m.n_embd)]
    for _ in range(m.n_layer):
        mods += [nn.LayerNorm(m.n_embd), nn.LayerNorm(m.n_embd),
                 nn.Linear(m.n_embd, 3 * m.n_embd, bias=m.bias), nn.Linear(m.n_embd, m.n_embd, bias=m.bias),
                 nn.Linear(m.n_embd, m.mlp_hidden, bias=m.bias), nn.Linear(m.mlp_hidden, m.n_embd, bias=m.bias)]
    if m.untied:
        mods.append(nn.Linear(m.n_embd, m.vocab, bias=False))
    assert n == sum(p.numel() for mod in mods for p in mod.parameters())
    if wname == "gpt2_124m":
        assert abs(n - counts["page_approx_124m"]) / counts["page_approx_124m"] < 0.005


# ----------------------------------------------------------------- generation
def test_inverse_cdf_sampling_boundaries(oracle):
    # dyadic probabilities, so the cumulative sums 0.125 | 0.375 | 0.75 | 1 are exact
    p = np.array([[0.125, 0.25, 0.375, 0.25]] * 7)
    u = np.array([0.0, 0.124, 0.125, 0.374, 0.375, 0.75, 0.9999])
    # the smallest k whose cumulative probability exceeds u
    assert list(oracle.sample_inverse_cdf(p, u)) == [0, 0, 1, 1, 2, 3, 3]
    q = np.array([[0.0, 0.5, 0.0, 0.5]] * 3)
    assert list(oracle.sample_inverse_cdf(q, np.array([0.0, 0.49, 0.5]))) == [1, 1, 3]  # p = 0 never drawn


def test_inverse_cdf_sampling_frequencies(oracle):
    from scipy.stats import chisquare
    rng = np.random.default_rng(8)
    p = rng.dirichlet(np.ones(12))
    n = 60000
    draws = oracle.sample_inverse_cdf(np.broadcast_to(p, (n, 12)), rng.random(n))
    counts = np.bincount(draws, minlength=12)
    assert chisquare(counts, p * n).pvalue > 1e-3


def test_next_token_probs_match_torch_softmax_and_crop(oracle):
    import torch
    m = TINY
    cfg = ocfg(oracle, m)
    named = rand_named(m, 21)
    p = oracle.pack(cfg, named, np.float64)
    rng = np.random.default_rng(22)
    ctx = rng.integers(0, m.vocab, size=(3, 5)).astype(np.int32)
    probs = oracle.next_token_probs(cfg, p, ctx, temperature=0.7)
    z = torch.tensor(torch_model_loss(named, m, ctx, None)[:, -1, :] / 0.7)
    np.testing.assert_allclose(probs, torch.softmax(z, dim=-1).numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(probs.sum(axis=1), 1.0, rtol=1e-14)
    # the model sees only the last block_size tokens: anything before them is cropped away
    full = rng.integers(0, m.vocab, size=(3, m.block_size)).astype(np.int32)
    longer = np.concatenate([rng.integers(0, m.vocab, size=(3, 4)).astype(np.int32), full], axis=1)
    np.testing.assert_array_equal(oracle.next_token_probs(cfg, p, longer, 1.0),
                                  oracle.next_token_probs(cfg, p, full, 1.0))


def test_low_temperature_generation_is_greedy(oracle):
    m = TINY
    cfg = ocfg(oracle, m)
    p = oracle.pack(cfg, rand_named(m, 23), np.float64)
    prompt = np.array([[1, 2], [3, 4]], dtype=np.int32)
    u = np.random.default_rng(24).random((2, 12))
    seq = oracle.generate(cfg, p, prompt, 12, 1e-6, u)      # crosses block_size = 8
    assert seq.shape == (2, 14) and np.array_equal(seq[:, :2], prompt)
    for i in range(2, 14):
        probs = oracle.next_token_probs(cfg, p, seq[:, :i], 1.0)
        assert np.array_equal(seq[:, i], probs.argmax(axis=1)), i


# ----------------------------------------------------------------- synthetic inputs
def test_batch_targets_are_inputs_shifted_by_one():
    w = syn.WORKLOADS["char_bf16"]
    rng = np.random.Generator(np.random.PCG64([syn.DATA_SEED, 3]))
    rows = syn.draw_tokens(rng, w.model.vocab, w.batch * (w.seq + 1), w.tokens, w.zipf_s).reshape(w.batch, -1)
    x, y = syn.batch(w, step=3)
    assert np.array_equal(x, rows[:, :-1]) and np.array_equal(y, rows[:, 1:])
    assert np.array_equal(x[:, 1:], y[:, :-1])
    assert x.min() >= 0 and x.max() < w.model.vocab


def test_zipf_frequencies_chi_square():
    from scipy.stats import chisquare
    V, s = 65, 1.1
    rng = np.random.default_rng(9)
    t = syn.draw_tokens(rng, V, 200000, "zipf", s)
    p = np.diff(np.concatenate([[0.0], syn.zipf_cdf(V, s)]))
    obs = np.bincount(t, minlength=V)
    assert chisquare(obs, p * obs.sum()).pvalue > 1e-3
    assert abs(obs[0] / obs.sum() - 1 / np.sum(np.arange(1, V + 1) ** -s)) < 0.01
