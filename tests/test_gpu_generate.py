"""Generation (gpt2_generate) against the oracle's generate loop (GPU required).

Every draw is checked re-synced: the oracle computes the next-token
probabilities from the GPU's own prefix, and the GPU's token k must satisfy
cdf(k-1) - tol <= u <= cdf(k) + tol (the inverse-CDF rule; tol covers rounding in
the probabilities: fp32 logits in fp32 mode, bf16 GEMM operands in bf16 mode).
Where no boundary lies within tol of u the token is unique and must equal the
oracle's own draw (fp32); in bf16 mode, whose small-vocabulary distributions put
a boundary within the rounding tolerance of nearly every u, the share of draws
equal to the oracle's is checked instead.
"""
import numpy as np
import pytest

import synthetic as syn
from gpu_helpers import gcfg, ocfg, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from decoder_only_transformer_04_amd import binding
    binding.lib()
    return binding


def gen_gpu(b, m, dtype, named, prompt, n_new, temperature, u):
    import torch
    B, T0 = prompt.shape
    g = b.Model(gcfg(b, m, dtype), B, m.block_size, b.MODE_GENERATE)
    g.load_named(named)
    g.init()
    out = torch.full((B, T0 + n_new), -1, dtype=torch.int32, device="cuda")
    g.generate(torch.from_numpy(np.ascontiguousarray(prompt, np.int32)).cuda(), n_new, temperature,
               torch.from_numpy(np.ascontiguousarray(u, np.float32)).cuda(), out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), g


def check_draws(oracle, m, named, seq, T0, temperature, u, tol):
    cfg = ocfg(oracle, m)
    p = oracle.pack(cfg, named, np.float64)
    B, n_new = u.shape
    rows = np.arange(B)
    same, unique, same_all = 0, 0, 0
    margin = 0.0
    for i in range(n_new):
        probs = oracle.next_token_probs(cfg, p, seq[:, :T0 + i], temperature)
        k = seq[:, T0 + i]
        assert np.all((k >= 0) & (k < m.vocab)), (i, k)
        c = np.cumsum(probs, axis=1)
        lo = np.where(k > 0, c[rows, np.maximum(k - 1, 0)], 0.0)
        hi = c[rows, k]
        uu = u[:, i].astype(np.float64)
        assert np.all(lo - tol <= uu) and np.all(uu <= hi + tol), (i, k, lo, hi, uu)
        margin = max(margin, float(np.max(np.maximum(lo - uu, uu - hi))))
        ref = oracle.sample_inverse_cdf(probs, uu)
        same_all += int((ref == k).sum())
        clear = np.abs(c - uu[:, None]).min(axis=1) > tol  # no boundary near u: one valid token
        unique += int(clear.sum())
        same += int((ref == k)[clear].sum())
    say(f"  draws {B * n_new}: equal to the oracle's {same_all}, CDF margin needed {margin:.2e}")
    return same, unique, same_all


def test_generate_tiny_f32_with_crop(b, oracle):
    """fp32: 70 new tokens after a 5-token prompt crosses block_size (64), so the
    window slides and is recomputed; every draw where u is clear of a boundary
    equals the oracle's."""
    w = syn.WORKLOADS["tiny_f32"]
    m = w.model
    say("generate tiny_f32 3 x (5 + 70)")
    named = syn.init_params(m, seed=5)
    rng = np.random.default_rng(6)
    prompt = rng.integers(0, m.vocab, size=(3, 5)).astype(np.int32)
    u = rng.random((3, 70)).astype(np.float32)
    seq, g = gen_gpu(b, m, "f32", named, prompt, 70, 0.9, u)
    assert np.array_equal(seq[:, :5], prompt)
    same, unique, _ = check_draws(oracle, m, named, seq, 5, 0.9, u, tol=1e-5)
    assert unique >= 200 and same == unique, (same, unique)
    assert g.sync_status() == 0


def test_generate_greedy_and_literal_model(b, oracle):
    """The literal model (erf GELU, own lm_head) at a very low temperature: every
    draw is the most probable token given the GPU's prefix."""
    w = syn.WORKLOADS["tiny_f32_literal"]
    m = w.model
    say("generate tiny_f32_literal greedy 2 x (3 + 20)")
    named = syn.init_params(m, seed=7)
    rng = np.random.default_rng(8)
    prompt = rng.integers(0, m.vocab, size=(2, 3)).astype(np.int32)
    u = rng.random((2, 20)).astype(np.float32)
    seq, g = gen_gpu(b, m, "f32", named, prompt, 20, 1e-3, u)
    cfg = ocfg(oracle, m)
    p = oracle.pack(cfg, named, np.float64)
    for i in range(20):
        logits_p = oracle.next_token_probs(cfg, p, seq[:, :3 + i], 1.0)
        top2 = np.sort(logits_p, axis=1)[:, -2:]
        decided = top2[:, 1] > top2[:, 0] * (1 + 1e-3)
        assert np.all(seq[decided, 3 + i] == logits_p.argmax(axis=1)[decided]), i
    same, unique, _ = check_draws(oracle, m, named, seq, 3, 1e-3, u, tol=1e-5)
    assert same == unique
    assert g.sync_status() == 0


def test_generate_char_bf16(b, oracle):
    """bf16 operands: draws valid within the bf16 rounding of the logits and
    mostly equal to the oracle's."""
    w = syn.WORKLOADS["char_bf16"]
    m = w.model
    say("generate char_bf16 2 x (8 + 32)")
    named = syn.init_params(m, seed=9)
    rng = np.random.default_rng(10)
    prompt = syn.draw_tokens(rng, m.vocab, 16, "zipf", 1.1).reshape(2, 8)
    u = rng.random((2, 32)).astype(np.float32)
    seq, g = gen_gpu(b, m, "bf16", named, prompt, 32, 1.0, u)
    _, _, same_all = check_draws(oracle, m, named, seq, 8, 1.0, u, tol=1e-2)
    assert same_all >= 0.75 * u.size, same_all
    assert g.sync_status() == 0


def test_generate_gpt2_124m_bf16(b, oracle):
    """The 124M model (tied head, biases): a short continuation of two Zipf prompts."""
    w = syn.WORKLOADS["gpt2_124m"]
    m = w.model
    say("generate gpt2_124m 2 x (12 + 4)")
    named = syn.init_params(m)
    rng = np.random.default_rng(11)
    prompt = syn.draw_tokens(rng, m.vocab, 24, "zipf", 1.05).reshape(2, 12)
    u = rng.random((2, 4)).astype(np.float32)
    seq, g = gen_gpu(b, m, "bf16", named, prompt, 4, 1.0, u)
    assert np.array_equal(seq[:, :12], prompt)
    check_draws(oracle, m, named, seq, 12, 1.0, u, tol=3e-2)
    assert g.sync_status() == 0


def test_generate_edges_and_errors(b):
    import torch
    m = syn.WORKLOADS["tiny_f32"].model
    named = syn.init_params(m)
    prompt = np.array([[1, 2, 3]], dtype=np.int32)
    seq, g = gen_gpu(b, m, "f32", named, prompt, 0, 1.0, np.zeros((1, 0), np.float32))
    assert np.array_equal(seq, prompt)                      # no new tokens: the prompt alone
    out = torch.zeros((1, 5), dtype=torch.int32, device="cuda")
    u = torch.full((1, 2), 0.5, dtype=torch.float32, device="cuda")
    pr = torch.tensor([[1, 99, 3]], dtype=torch.int32, device="cuda")  # 99 >= V = 65
    g.generate(pr, 2, 1.0, u, out)
    assert g.sync_status() & b.STATUS_TOKEN_RANGE
    g.clear_status()
    with pytest.raises(b.GPT2Error):
        g.generate(pr, 2, 0.0, u, out)                      # temperature must be > 0
    with pytest.raises(b.GPT2Error):
        g.forward(pr.reshape(-1))                           # the training forward is not for this mode
    with pytest.raises(b.GPT2Error):
        b.Model(gcfg(b, m, "f32"), 1, m.block_size - 1, b.MODE_GENERATE)  # T must be block_size
