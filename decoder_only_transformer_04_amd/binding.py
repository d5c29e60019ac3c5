"""ctypes binding over libgpt2mi.so (the C ABI in include/gpt2.h).

Argument marshalling only: every step of the training path runs in the HIP
library. torch supplies device memory (torch.empty on "cuda") and the current
stream handle. If the library has not been built this module raises; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes as ct
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2mi.so")

GPT2_OK, GPT2_EINVAL, GPT2_ENOSPC, GPT2_EHIP, GPT2_EDEVICE, GPT2_ESTATE = 0, -1, -2, -3, -4, -5
DTYPE_F32, DTYPE_BF16 = 0, 1
MODE_TRAIN, MODE_EVAL, MODE_GENERATE = 0, 1, 2
DECAY_ALL, DECAY_MATRICES = 0, 1
STATUS_TOKEN_RANGE, STATUS_NONFINITE_LOSS, STATUS_NONFINITE_GNORM, STATUS_WINDOW_RANGE = 1, 2, 4, 8

EXPORTS = [
    "gpt2_query_sizes", "gpt2_num_params", "gpt2_param_table", "gpt2_lr_cosine", "gpt2_strerror", "gpt2_init",
    "gpt2_refresh_weights", "gpt2_forward", "gpt2_backward", "gpt2_adamw_step", "gpt2_generate", "gpt2_sync_status",
    "gpt2_clear_status", "gpt2_arena_tensor", "gpt2_destroy", "gpt2_op_linear_fwd", "gpt2_op_linear_bwd",
    "gpt2_op_layernorm_fwd", "gpt2_op_layernorm_bwd", "gpt2_op_attention_fwd", "gpt2_op_attention_bwd",
    "gpt2_op_cross_entropy", "gpt2_timing_begin", "gpt2_timing_end", "gpt2_char_vocab", "gpt2_char_encode",
    "gpt2_char_decode", "gpt2_split_point", "gpt2_batch_windows", "gpt2_set_dropout_seed",
]


class Config(ct.Structure):
    _fields_ = [("vocab", ct.c_int32), ("block_size", ct.c_int32), ("n_embd", ct.c_int32), ("n_head", ct.c_int32),
                ("n_layer", ct.c_int32), ("mlp_hidden", ct.c_int32), ("bias", ct.c_int32), ("dtype", ct.c_int32),
                ("ln_eps", ct.c_float), ("gelu_erf", ct.c_int32), ("untied_head", ct.c_int32),
                ("dropout", ct.c_float)]


class TensorDesc(ct.Structure):
    _fields_ = [("name", ct.c_char * 24), ("layer", ct.c_int32), ("decay", ct.c_int32), ("offset", ct.c_int64),
                ("rows", ct.c_int64), ("cols", ct.c_int64), ("reserved", ct.c_int64)]


class Buffers(ct.Structure):
    _fields_ = [("params", ct.c_void_p), ("grads", ct.c_void_p), ("adam_m", ct.c_void_p), ("adam_v", ct.c_void_p),
                ("arena", ct.c_void_p), ("arena_bytes", ct.c_size_t)]


class GPT2Error(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})")


_lib = None


def lib():
    """Load libgpt2mi.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m decoder_only_transformer_04_amd.build)")
        # torch first: it loads the HIP runtime it was built with, and the library
        # then binds to that one; loaded the other way round, the process can end up
        # with two runtimes, and the library's sees no device
        import torch  # noqa: F401
        L = ct.CDLL(LIB_PATH)
        P, i32, i64, f32, f64 = ct.c_void_p, ct.c_int32, ct.c_int64, ct.c_float, ct.c_double
        sz = ct.POINTER(ct.c_size_t)
        sig = {
            "gpt2_query_sizes": (ct.c_int, [P, i32, i32, i32, sz, sz]),
            "gpt2_num_params": (i64, [P]),
            "gpt2_param_table": (ct.c_int, [P, P, i32]),
            "gpt2_lr_cosine": (f64, [i64, f64, f64, i64, i64]),
            "gpt2_strerror": (ct.c_char_p, [ct.c_int]),
            "gpt2_init": (ct.c_int, [ct.POINTER(P), P, P, i32, i32, i32, P]),
            "gpt2_refresh_weights": (ct.c_int, [P]),
            "gpt2_forward": (ct.c_int, [P, P, P, P, P]),
            "gpt2_backward": (ct.c_int, [P, f32, i32]),
            "gpt2_adamw_step": (ct.c_int, [P, f32, f32, f32, f32, f32, i32, f32, i32, P]),
            "gpt2_generate": (ct.c_int, [P, P, i32, i32, f32, P, P]),
            "gpt2_set_dropout_seed": (ct.c_int, [P, ct.c_uint64]),
            "gpt2_char_vocab": (i32, [P, i64, P]),
            "gpt2_char_encode": (ct.c_int, [P, i64, P, i32, P]),
            "gpt2_char_decode": (ct.c_int, [P, i64, P, i32, P]),
            "gpt2_split_point": (i64, [i64, f64]),
            "gpt2_batch_windows": (ct.c_int, [P, i64, P, i32, i32, P, P, P, P]),
            "gpt2_sync_status": (ct.c_int, [P, ct.POINTER(ct.c_uint32)]),
            "gpt2_clear_status": (ct.c_int, [P]),
            "gpt2_arena_tensor": (ct.c_int, [P, ct.c_char_p, i32, sz, ct.POINTER(i32), ct.POINTER(i64),
                                             ct.POINTER(i64)]),
            "gpt2_destroy": (None, [P]),
            "gpt2_timing_begin": (ct.c_int, [P, ct.c_char_p]),
            "gpt2_timing_end": (ct.c_int, [P, ct.POINTER(f32), ct.POINTER(i32)]),
            "gpt2_op_linear_fwd": (ct.c_int, [i32, i64, i32, i32, P, P, P, P, P]),
            "gpt2_op_linear_bwd": (ct.c_int, [i32, i64, i32, i32, P, P, P, P, P, P, i32, P]),
            "gpt2_op_layernorm_fwd": (ct.c_int, [i32, i64, i32, P, P, P, f32, P, P, P, P]),
            "gpt2_op_layernorm_bwd": (ct.c_int, [i64, i32, P, P, P, P, P, P, P, P, P]),
            "gpt2_op_attention_fwd": (ct.c_int, [i32, i32, i32, i32, i32, P, P, P, P]),
            "gpt2_op_attention_bwd": (ct.c_int, [i32, i32, i32, i32, i32, P, P, P, P, P, P]),
            "gpt2_op_cross_entropy": (ct.c_int, [i32, i64, i32, i32, P, P, P, P, i32, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().gpt2_strerror(int(code)).decode()


def check(code: int, what: str) -> int:
    if code < 0:
        raise GPT2Error(code, what)
    return code


def make_config(vocab, block_size, n_embd, n_head, n_layer, mlp_hidden, bias, dtype, ln_eps=1e-5, gelu_erf=False,
                untied_head=False, dropout=0.0) -> Config:
    return Config(vocab, block_size, n_embd, n_head, n_layer, mlp_hidden, int(bias), int(dtype), ln_eps,
                  int(bool(gelu_erf)), int(bool(untied_head)), float(dropout))


def query_sizes(cfg: Config, B: int, T: int, mode: int):
    n = ct.c_size_t()
    a = ct.c_size_t()
    check(lib().gpt2_query_sizes(ct.byref(cfg), B, T, mode, ct.byref(n), ct.byref(a)), "gpt2_query_sizes")
    return int(n.value), int(a.value)


def num_params(cfg: Config) -> int:
    return check(int(lib().gpt2_num_params(ct.byref(cfg))), "gpt2_num_params")


def param_table(cfg: Config):
    n = check(lib().gpt2_param_table(ct.byref(cfg), None, 0), "gpt2_param_table")
    arr = (TensorDesc * n)()
    check(lib().gpt2_param_table(ct.byref(cfg), arr, n), "gpt2_param_table")
    out = []
    for d in arr:
        name = d.name.decode()
        shape = (int(d.cols),) if d.rows == 1 and name not in ("wte", "wpe") else (int(d.rows), int(d.cols))
        out.append({"name": name, "layer": d.layer, "decay": d.decay, "offset": int(d.offset), "shape": shape,
                    "reserved": int(d.reserved)})
    return out


# ------------------------------------------------------------------ character-level data
def char_vocab(text: bytes) -> list:
    buf = (ct.c_uint8 * 256)()
    v = check(int(lib().gpt2_char_vocab(text, len(text), buf)), "gpt2_char_vocab")
    return list(buf[:v])


def char_encode(text: bytes, vocab: list):
    import numpy as np
    ids = np.empty(len(text), dtype=np.int32)
    ch = (ct.c_uint8 * 256)(*vocab)
    check(lib().gpt2_char_encode(text, len(text), ch, len(vocab), ids.ctypes.data_as(ct.c_void_p)),
          "gpt2_char_encode")
    return ids


def char_decode(ids, vocab: list) -> bytes:
    import numpy as np
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    out = ct.create_string_buffer(max(1, ids.size))
    ch = (ct.c_uint8 * 256)(*vocab)
    check(lib().gpt2_char_decode(ids.ctypes.data_as(ct.c_void_p), ids.size, ch, len(vocab), out), "gpt2_char_decode")
    return out.raw[:ids.size]


def split_point(n: int, ratio: float = 0.9) -> int:
    return check(int(lib().gpt2_split_point(int(n), float(ratio))), "gpt2_split_point")


def batch_windows(data, offsets, x, y, status=None, stream=None) -> None:
    """data: int32 [n] (cuda); offsets: int64 [B] (cuda); x, y: int32 [B, T] (cuda)."""
    B, T = x.shape
    check(lib().gpt2_batch_windows(_ptr(data), data.numel(), _ptr(offsets), B, T, _ptr(x), _ptr(y), _ptr(status),
                                   _s(stream)), "gpt2_batch_windows")


def lr_cosine(it, max_lr=6e-4, min_lr=6e-5, warmup=2000, max_iters=600000) -> float:
    return float(lib().gpt2_lr_cosine(int(it), max_lr, min_lr, int(warmup), int(max_iters)))


def _ptr(t):
    return None if t is None else ct.c_void_p(t.data_ptr())


def _stream_handle(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ct.c_void_p(stream.cuda_stream)


class Model:
    """Owns the device buffers (torch tensors) of one training (or eval) step and
    the library context. Methods map one-to-one onto the C ABI."""

    def __init__(self, cfg: Config, B: int, T: int, mode: int = MODE_TRAIN, device="cuda", stream=None):
        import torch
        self.cfg, self.B, self.T, self.mode = cfg, B, T, mode
        self.n_flat, self.arena_bytes = query_sizes(cfg, B, T, mode)
        self.table = param_table(cfg)
        self.by_name = {d["name"]: d for d in self.table}
        self.vocab_pad = (cfg.vocab + 127) // 128 * 128  # wte rows reserved in the flat layout
        f32 = torch.float32
        self.params = torch.zeros(self.n_flat, dtype=f32, device=device)
        train = mode == MODE_TRAIN
        self.grads = torch.zeros(self.n_flat, dtype=f32, device=device) if train else None
        self.adam_m = torch.zeros(self.n_flat, dtype=f32, device=device) if train else None
        self.adam_v = torch.zeros(self.n_flat, dtype=f32, device=device) if train else None
        self.arena = torch.empty(self.arena_bytes, dtype=torch.uint8, device=device)
        self.loss = torch.zeros(1, dtype=f32, device=device)
        self.grad_norm = torch.zeros(1, dtype=f32, device=device)
        self._stream = stream
        self.ctx = None

    # -------------------------------------------------------------- parameters
    def load_named(self, named: dict) -> None:
        """Copy a dict of named host arrays (fp32) into the flat parameter buffer."""
        import numpy as np
        import torch
        host = np.zeros(self.n_flat, dtype=np.float32)
        for d in self.table:
            a = np.asarray(named[d["name"]], dtype=np.float32)
            assert a.shape == d["shape"], (d["name"], a.shape, d["shape"])
            host[d["offset"]:d["offset"] + a.size] = a.ravel()
        self.params.copy_(torch.from_numpy(host))
        if self.ctx is not None:
            check(lib().gpt2_refresh_weights(self.ctx), "gpt2_refresh_weights")

    def named(self, flat) -> dict:
        """Split a flat host array (numpy) into named views."""
        out = {}
        for d in self.table:
            n = 1
            for s in d["shape"]:
                n *= s
            out[d["name"]] = flat[d["offset"]:d["offset"] + n].reshape(d["shape"])
        return out

    def init(self) -> None:
        bufs = Buffers(self.params.data_ptr(), self.grads.data_ptr() if self.grads is not None else None,
                       self.adam_m.data_ptr() if self.adam_m is not None else None,
                       self.adam_v.data_ptr() if self.adam_v is not None else None,
                       self.arena.data_ptr(), self.arena_bytes)
        ctx = ct.c_void_p()
        check(lib().gpt2_init(ct.byref(ctx), ct.byref(self.cfg), ct.byref(bufs), self.B, self.T, self.mode,
                              _stream_handle(self._stream)), "gpt2_init")
        self.ctx = ctx

    def refresh_weights(self) -> None:
        check(lib().gpt2_refresh_weights(self.ctx), "gpt2_refresh_weights")

    # -------------------------------------------------------------- the step
    def forward(self, idx, targets=None, argmax=None, loss=None) -> None:
        loss = self.loss if loss is None else loss
        check(lib().gpt2_forward(self.ctx, _ptr(idx), _ptr(targets), _ptr(loss) if targets is not None else None,
                                 _ptr(argmax)), "gpt2_forward")

    def backward(self, loss_scale: float = 1.0, zero_grads: bool = True) -> None:
        check(lib().gpt2_backward(self.ctx, float(loss_scale), int(bool(zero_grads))), "gpt2_backward")

    def adamw_step(self, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, t=1, clip=0.0,
                   decay_mode=DECAY_ALL, want_norm=False) -> None:
        check(lib().gpt2_adamw_step(self.ctx, lr, beta1, beta2, eps, weight_decay, int(t), clip, decay_mode,
                                    _ptr(self.grad_norm) if want_norm else None), "gpt2_adamw_step")

    def set_dropout_seed(self, seed: int) -> None:
        """Key of the dropout masks of the following training forwards."""
        check(lib().gpt2_set_dropout_seed(self.ctx, int(seed)), "gpt2_set_dropout_seed")

    def generate(self, prompt, n_new: int, temperature: float, uniforms, out) -> None:
        """prompt: int32 [B, T0] (cuda); uniforms: fp32 [B, n_new] (cuda); out:
        int32 [B, T0 + n_new] (cuda), written on the context's stream."""
        T0 = int(prompt.shape[1])
        check(lib().gpt2_generate(self.ctx, _ptr(prompt), T0, int(n_new), float(temperature), _ptr(uniforms),
                                  _ptr(out)), "gpt2_generate")

    def sync_status(self) -> int:
        bits = ct.c_uint32()
        rc = lib().gpt2_sync_status(self.ctx, ct.byref(bits))
        if rc not in (GPT2_OK, GPT2_EDEVICE):
            raise GPT2Error(rc, "gpt2_sync_status")
        return int(bits.value)

    def timing_begin(self, prefix: str) -> None:
        check(lib().gpt2_timing_begin(self.ctx, prefix.encode()), "gpt2_timing_begin")

    def timing_end(self):
        """(total milliseconds, launches) of the launches timed since timing_begin."""
        ms = ct.c_float()
        n = ct.c_int32()
        check(lib().gpt2_timing_end(self.ctx, ct.byref(ms), ct.byref(n)), "gpt2_timing_end")
        return float(ms.value), int(n.value)

    def clear_status(self) -> None:
        check(lib().gpt2_clear_status(self.ctx), "gpt2_clear_status")

    def arena_tensor(self, name: str, layer: int = 0):
        """A torch view of an activation inside the arena (for inspection)."""
        import torch
        off = ct.c_size_t()
        eb = ct.c_int32()
        rows = ct.c_int64()
        cols = ct.c_int64()
        check(lib().gpt2_arena_tensor(self.ctx, name.encode(), layer, ct.byref(off), ct.byref(eb), ct.byref(rows),
                                      ct.byref(cols)), "gpt2_arena_tensor")
        n = int(rows.value) * int(cols.value)
        raw = self.arena[off.value:off.value + n * eb.value]
        dt = {4: torch.float32, 2: torch.bfloat16, 8: torch.int64}[eb.value]
        return raw.view(dt).view(int(rows.value), int(cols.value))

    def close(self) -> None:
        if self.ctx is not None:
            lib().gpt2_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------ single operations
def _s(stream):
    return _stream_handle(stream)


def op_linear_fwd(dtype, X, W, bias, Y, stream=None):
    M, K = X.shape
    N = W.shape[0]
    check(lib().gpt2_op_linear_fwd(dtype, M, N, K, _ptr(X), _ptr(W), _ptr(bias), _ptr(Y), _s(stream)),
          "gpt2_op_linear_fwd")


def op_linear_bwd(dtype, dY, X, W, dX, dW, db, accumulate=False, stream=None):
    M, K = X.shape
    N = W.shape[0]
    check(lib().gpt2_op_linear_bwd(dtype, M, N, K, _ptr(dY), _ptr(X), _ptr(W), _ptr(dX), _ptr(dW), _ptr(db),
                                   int(accumulate), _s(stream)), "gpt2_op_linear_bwd")


def op_layernorm_fwd(dtype, x, g, b, eps, y, mean, rstd, stream=None):
    rows, C = x.shape
    check(lib().gpt2_op_layernorm_fwd(dtype, rows, C, _ptr(x), _ptr(g), _ptr(b), eps, _ptr(y), _ptr(mean),
                                      _ptr(rstd), _s(stream)), "gpt2_op_layernorm_fwd")


def op_layernorm_bwd(dy, x, mean, rstd, g, dx, dg, db, stream=None):
    rows, C = x.shape
    check(lib().gpt2_op_layernorm_bwd(rows, C, _ptr(dy), _ptr(x), _ptr(mean), _ptr(rstd), _ptr(g), _ptr(dx),
                                      _ptr(dg), _ptr(db), _s(stream)), "gpt2_op_layernorm_bwd")


def op_attention_fwd(dtype, B, T, C, H, qkv, out, lse, stream=None):
    check(lib().gpt2_op_attention_fwd(dtype, B, T, C, H, _ptr(qkv), _ptr(out), _ptr(lse), _s(stream)),
          "gpt2_op_attention_fwd")


def op_attention_bwd(dtype, B, T, C, H, qkv, out, lse, dout, dqkv, stream=None):
    check(lib().gpt2_op_attention_bwd(dtype, B, T, C, H, _ptr(qkv), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dqkv),
                                      _s(stream)), "gpt2_op_attention_bwd")


def op_cross_entropy(dtype, logits, V, targets, loss_rows, argmax=None, write_grad=False, stream=None):
    rows, ld = logits.shape
    check(lib().gpt2_op_cross_entropy(dtype, rows, V, ld, _ptr(logits), _ptr(targets), _ptr(loss_rows),
                                      _ptr(argmax), int(write_grad), _s(stream)), "gpt2_op_cross_entropy")
