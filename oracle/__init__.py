"""ctypes wrapper over the CPU oracle (oracle/liboracle.so).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only users. The product path never
imports this package. Parameters travel between the harness and the oracle as
a dict of named float arrays; the oracle packs them into its own compact layout
(``oracle_param_table``), independent of the HIP library's layout.
"""
from __future__ import annotations

import ctypes as ct
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

KIND_NAMES = ["wte", "wpe", "ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj",
              "ln2_g", "ln2_b", "w_fc", "b_fc", "w_fc2", "b_fc2", "lnf_g", "lnf_b", "lm_head"]
GELU_ERF, UNTIED = 1, 2  # variant bits: exact erf GELU, separate lm_head


class OracleCfg(ct.Structure):
    _fields_ = [("vocab", ct.c_int32), ("block_size", ct.c_int32), ("n_embd", ct.c_int32),
                ("n_head", ct.c_int32), ("n_layer", ct.c_int32), ("mlp_hidden", ct.c_int32),
                ("bias", ct.c_int32), ("variant", ct.c_int32), ("ln_eps", ct.c_double),
                ("dropout", ct.c_double), ("seed", ct.c_uint64)]


DROP_ATTN, DROP_PROJ, DROP_FC2 = 0, 1, 2  # dropout sites of a block


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ct.CDLL(LIB_PATH)
        P = ct.c_void_p
        i64, i32, dbl = ct.c_int64, ct.c_int32, ct.c_double
        L.oracle_n_params.restype = i64
        L.oracle_n_params.argtypes = [P]
        L.oracle_param_table.restype = ct.c_int
        L.oracle_param_table.argtypes = [P, P, ct.c_int]
        for suf in ("f32", "f64"):
            f = getattr(L, f"oracle_step_{suf}")
            f.restype = dbl
            f.argtypes = [P, ct.c_int, ct.c_int, P, P, P, P, dbl, P, P]
            getattr(L, f"oracle_layernorm_{suf}").argtypes = [i64, ct.c_int, P, P, P, dbl, P, P, P]
            getattr(L, f"oracle_layernorm_bwd_{suf}").argtypes = [i64, ct.c_int, P, P, P, P, P, P, P, P]
            getattr(L, f"oracle_linear_{suf}").argtypes = [i64, ct.c_int, ct.c_int, P, P, P, P]
            getattr(L, f"oracle_linear_bwd_{suf}").argtypes = [i64, ct.c_int, ct.c_int, P, P, P, P, P, P]
            getattr(L, f"oracle_gelu_{suf}").argtypes = [i64, P, P, P, ct.c_int]
            getattr(L, f"oracle_head_attention_{suf}").argtypes = [ct.c_int, ct.c_int, P, P, P, P, P]
            getattr(L, f"oracle_attention_{suf}").argtypes = [ct.c_int] * 4 + [P, P]
            getattr(L, f"oracle_attention_bwd_{suf}").argtypes = [ct.c_int] * 4 + [P, P, P]
            getattr(L, f"oracle_cross_entropy_{suf}").argtypes = [i64, ct.c_int, P, P, P, P, dbl]
            getattr(L, f"oracle_adamw_{suf}").argtypes = [i64, P, P, P, P, dbl, dbl, dbl, dbl, dbl,
                                                          ct.c_int, P]
            c = getattr(L, f"oracle_clip_{suf}")
            c.restype = dbl
            c.argtypes = [i64, P, dbl]
        L.oracle_lr.restype = dbl
        L.oracle_lr.argtypes = [i64, dbl, dbl, i64, i64]
        L.oracle_argmax_f32.argtypes = [i64, ct.c_int, P, P]
        L.oracle_philox4x32_10.argtypes = [P, P, P]
        L.oracle_dropout_keep.argtypes = [dbl, ct.c_uint64, ct.c_int, ct.c_int, ct.c_uint64, i64, P]
        L.oracle_set_threads.argtypes = [ct.c_int]
        L.oracle_max_threads.restype = ct.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ct.c_void_p)


def _dt(dtype):
    dtype = np.dtype(dtype)
    if dtype == np.float32:
        return "f32"
    if dtype == np.float64:
        return "f64"
    raise TypeError(dtype)


def make_cfg(vocab, block_size, n_embd, n_head, n_layer, mlp_hidden, bias, ln_eps=1e-5, gelu_erf=False,
             untied=False, dropout=0.0, seed=0):
    """dropout > 0: the training-mode model (step() applies dropout keyed by seed)."""
    variant = (GELU_ERF if gelu_erf else 0) | (UNTIED if untied else 0)
    return OracleCfg(vocab, block_size, n_embd, n_head, n_layer, mlp_hidden, int(bias), variant, ln_eps,
                     float(dropout), int(seed))


def eval_cfg(cfg: OracleCfg) -> OracleCfg:
    """The same model in eval mode (model.eval(): no dropout)."""
    c = OracleCfg.from_buffer_copy(cfg)
    c.dropout = 0.0
    return c


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 of one 4-word counter under a 2-word key (uint32)."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def dropout_keep(p: float, seed: int, site: int, layer: int, n: int, e0: int = 0) -> np.ndarray:
    """uint8 keep flags of elements e0 .. e0 + n - 1 of one dropout site."""
    out = np.zeros(n, dtype=np.uint8)
    lib().oracle_dropout_keep(float(p), int(seed), int(site), int(layer), int(e0), int(n), _p(out))
    return out


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def n_params(cfg: OracleCfg) -> int:
    return int(lib().oracle_n_params(ct.byref(cfg)))


def param_table(cfg: OracleCfg):
    """[(name, offset, shape)] of the oracle's compact layout."""
    cap = 16 * (cfg.n_layer + 2)
    buf = np.zeros((cap, 5), dtype=np.int64)
    n = lib().oracle_param_table(ct.byref(cfg), _p(buf), cap)
    out = []
    for kind, layer, off, rows, cols in buf[:n]:
        base = KIND_NAMES[kind]
        name = base if layer < 0 else f"h{layer}.{base}"
        shape = (int(cols),) if rows == 1 and base not in ("wte", "wpe") else (int(rows), int(cols))
        out.append((name, int(off), shape))
    return out


def pack(cfg: OracleCfg, named: dict, dtype=np.float64) -> np.ndarray:
    flat = np.zeros(n_params(cfg), dtype=dtype)
    for name, off, shape in param_table(cfg):
        a = np.asarray(named[name], dtype=dtype)
        assert a.shape == shape, (name, a.shape, shape)
        flat[off:off + a.size] = a.ravel()
    return flat


def unpack(cfg: OracleCfg, flat: np.ndarray) -> dict:
    return {name: flat[off:off + int(np.prod(shape))].reshape(shape)
            for name, off, shape in param_table(cfg)}


def step(cfg: OracleCfg, B: int, T: int, params_flat: np.ndarray, idx: np.ndarray,
         targets: np.ndarray | None, grads: np.ndarray | None = None, loss_scale: float = 1.0,
         want_logits: bool = False, want_loss_rows: bool = False):
    """Forward (+ backward into ``grads`` when given, accumulating) of the whole
    model. Returns (loss, logits or None, loss_rows or None)."""
    dt = params_flat.dtype
    suf = _dt(dt)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1)
    tg = None if targets is None else np.ascontiguousarray(targets, dtype=np.int32).reshape(-1)
    assert idx.size == B * T
    logits = np.empty((B * T, cfg.vocab), dtype=dt) if want_logits else None
    rows = np.empty(B * T, dtype=dt) if want_loss_rows else None
    if grads is not None:
        assert grads.dtype == dt and grads.size == params_flat.size
    loss = getattr(lib(), f"oracle_step_{suf}")(ct.byref(cfg), B, T, _p(params_flat), _p(idx), _p(tg),
                                                _p(grads), loss_scale, _p(logits), _p(rows))
    return loss, logits, rows


# ---------------------------------------------------------------- generation
# The generate loop of the minigpt page (section 二, MiniGPT.generate; walkthrough
# 3.8) written out: crop the sequence to its last block_size tokens, run the whole
# forward, take the last position's logits, divide by the temperature, softmax,
# draw one token, append. The draw: torch.multinomial's internal procedure is not
# on the pages, so a draw is inverse-CDF sampling with a uniform number u in [0, 1)
# supplied by the caller (one per sequence and step): the token is the smallest k
# whose cumulative probability, summed in index order, exceeds u.
def next_token_probs(cfg: OracleCfg, params_flat: np.ndarray, ctx: np.ndarray, temperature: float) -> np.ndarray:
    """[B, V] float64 probabilities of the next token after each row of ``ctx``
    ([B, n] int32, n >= 1), with the crop to the last block_size tokens."""
    ctx = np.asarray(ctx, dtype=np.int32)
    B, n = ctx.shape
    win = ctx[:, max(0, n - cfg.block_size):]
    T = win.shape[1]
    _, logits, _ = step(eval_cfg(cfg), B, T, params_flat, win, None, want_logits=True)
    z = logits.reshape(B, T, cfg.vocab)[:, -1, :].astype(np.float64) / temperature
    z -= z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def sample_inverse_cdf(probs: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Per row, the smallest k with sum_{j<=k} p_j > u (the last token with p > 0
    if rounding leaves the total below u)."""
    out = np.empty(probs.shape[0], dtype=np.int32)
    for r in range(probs.shape[0]):
        c = np.cumsum(probs[r])
        k = int(np.searchsorted(c, u[r], side="right"))
        if k >= probs.shape[1]:
            k = int(np.nonzero(probs[r] > 0)[0][-1])
        out[r] = k
    return out


def generate(cfg: OracleCfg, params_flat: np.ndarray, prompt: np.ndarray, n_new: int, temperature: float,
             uniforms: np.ndarray) -> np.ndarray:
    """[B, T0 + n_new] int32: the prompt followed by n_new drawn tokens, the i-th
    new token of row b drawn with uniforms[b, i]."""
    seq = np.asarray(prompt, dtype=np.int32)
    for i in range(n_new):
        p = next_token_probs(cfg, params_flat, seq, temperature)
        seq = np.concatenate([seq, sample_inverse_cdf(p, uniforms[:, i])[:, None]], axis=1)
    return seq


# ---------------------------------------------------------------- unit functions
def layernorm(x, g, b, eps=1e-5):
    x = np.ascontiguousarray(x)
    suf = _dt(x.dtype)
    rows, C = x.reshape(-1, x.shape[-1]).shape
    y = np.empty_like(x)
    mean = np.empty(rows, dtype=x.dtype)
    rstd = np.empty(rows, dtype=x.dtype)
    getattr(lib(), f"oracle_layernorm_{suf}")(rows, C, _p(x), _p(np.ascontiguousarray(g, x.dtype)),
                                               _p(np.ascontiguousarray(b, x.dtype)), eps, _p(y), _p(mean),
                                               _p(rstd))
    return y, mean, rstd


def layernorm_bwd(dy, x, mean, rstd, g):
    x = np.ascontiguousarray(x)
    suf = _dt(x.dtype)
    rows, C = x.reshape(-1, x.shape[-1]).shape
    dx = np.zeros_like(x)
    dg = np.zeros(C, dtype=x.dtype)
    db = np.zeros(C, dtype=x.dtype)
    getattr(lib(), f"oracle_layernorm_bwd_{suf}")(rows, C, _p(np.ascontiguousarray(dy, x.dtype)), _p(x),
                                                   _p(mean), _p(rstd), _p(np.ascontiguousarray(g, x.dtype)),
                                                   _p(dx), _p(dg), _p(db))
    return dx, dg, db


def linear(X, W, b=None):
    X = np.ascontiguousarray(X)
    suf = _dt(X.dtype)
    M, K = X.shape
    N = W.shape[0]
    Y = np.empty((M, N), dtype=X.dtype)
    getattr(lib(), f"oracle_linear_{suf}")(M, N, K, _p(X), _p(np.ascontiguousarray(W, X.dtype)),
                                            None if b is None else _p(np.ascontiguousarray(b, X.dtype)), _p(Y))
    return Y


def linear_bwd(dY, X, W, with_bias=True):
    X = np.ascontiguousarray(X)
    suf = _dt(X.dtype)
    M, K = X.shape
    N = W.shape[0]
    dX = np.empty((M, K), dtype=X.dtype)
    dW = np.zeros((N, K), dtype=X.dtype)
    db = np.zeros(N, dtype=X.dtype) if with_bias else None
    getattr(lib(), f"oracle_linear_bwd_{suf}")(M, N, K, _p(np.ascontiguousarray(dY, X.dtype)), _p(X),
                                                _p(np.ascontiguousarray(W, X.dtype)), _p(dX), _p(dW), _p(db))
    return dX, dW, db


def gelu(u, erf_form=False):
    """GELU and its derivative: the tanh approximation, or the exact erf form."""
    u = np.ascontiguousarray(u)
    y = np.empty_like(u)
    dy = np.empty_like(u)
    getattr(lib(), f"oracle_gelu_{_dt(u.dtype)}")(u.size, _p(u), _p(y), _p(dy), int(bool(erf_form)))
    return y, dy


def head_attention(q, k, v):
    """One causal head (T x d each). Returns (out, P)."""
    q = np.ascontiguousarray(q)
    T, d = q.shape
    out = np.empty_like(q)
    P = np.empty((T, T), dtype=q.dtype)
    getattr(lib(), f"oracle_head_attention_{_dt(q.dtype)}")(T, d, _p(q), _p(np.ascontiguousarray(k, q.dtype)),
                                                             _p(np.ascontiguousarray(v, q.dtype)), _p(out), _p(P))
    return out, P


def attention(qkv, B, T, C, H):
    qkv = np.ascontiguousarray(qkv)
    out = np.empty((B * T, C), dtype=qkv.dtype)
    getattr(lib(), f"oracle_attention_{_dt(qkv.dtype)}")(B, T, C, H, _p(qkv), _p(out))
    return out


def attention_bwd(qkv, dout, B, T, C, H):
    qkv = np.ascontiguousarray(qkv)
    dqkv = np.empty_like(qkv)
    getattr(lib(), f"oracle_attention_bwd_{_dt(qkv.dtype)}")(B, T, C, H, _p(qkv),
                                                              _p(np.ascontiguousarray(dout, qkv.dtype)), _p(dqkv))
    return dqkv


def cross_entropy(z, y, scale=None):
    """Per-row losses, and dlogits*(scale) when scale is given."""
    z = np.ascontiguousarray(z)
    rows, V = z.shape
    y = np.ascontiguousarray(y, dtype=np.int32)
    lr = np.empty(rows, dtype=z.dtype)
    dz = np.empty_like(z) if scale is not None else None
    getattr(lib(), f"oracle_cross_entropy_{_dt(z.dtype)}")(rows, V, _p(z), _p(y), _p(lr), _p(dz),
                                                            0.0 if scale is None else float(scale))
    return lr, dz


def adamw(p, g, m, v, lr, b1, b2, eps, wd, t, decay=None):
    """In place on p, m, v."""
    suf = _dt(p.dtype)
    d = None if decay is None else np.ascontiguousarray(decay, dtype=np.uint8)
    getattr(lib(), f"oracle_adamw_{suf}")(p.size, _p(p), _p(np.ascontiguousarray(g, p.dtype)), _p(m), _p(v),
                                           lr, b1, b2, eps, wd, int(t), _p(d))


def clip(g, clip_value):
    """In place; returns the pre-clip global norm."""
    return float(getattr(lib(), f"oracle_clip_{_dt(g.dtype)}")(g.size, _p(g), float(clip_value)))


def lr_at(it, max_lr=6e-4, min_lr=6e-5, warmup=2000, max_iters=600000):
    return float(lib().oracle_lr(int(it), max_lr, min_lr, int(warmup), int(max_iters)))


def argmax_rows(z):
    z = np.ascontiguousarray(z, dtype=np.float32)
    rows, V = z.shape
    out = np.empty(rows, dtype=np.int32)
    lib().oracle_argmax_f32(rows, V, _p(z), _p(out))
    return out
