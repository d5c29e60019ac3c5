"""The character-level data path (the minigpt page's prepare_data / get_batch):
the oracle pinned by hand-worked values, the native tokenizer compared with it
byte for byte (host only), and the device window gather bit-exact (GPU)."""
import ctypes as ct

import numpy as np
import pytest

from oracle import chardata as cd


@pytest.fixture(scope="module")
def b():
    import os
    from decoder_only_transformer_04_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from decoder_only_transformer_04_amd import build
        build.build()
    binding.lib()
    return binding


def test_oracle_hand_worked_example():
    text = b"hello world"
    vocab = cd.char_vocab(text)
    assert vocab == list(b" dehlorw")                      # sorted distinct characters
    ids = cd.encode(text, vocab)
    assert ids[:5] == [3, 2, 4, 4, 5]                      # h e l l o
    assert cd.decode(ids, vocab) == text
    assert cd.split_point(11) == 9 and cd.split_point(10) == 9   # int(0.9 n)
    xs, ys = cd.get_batch(ids, [0, 6], 4)
    assert xs == [[3, 2, 4, 4], [7, 5, 6, 4]] and ys == [[2, 4, 4, 5], [5, 6, 4, 1]]
    for x, y in zip(xs, ys):
        assert x[1:] == y[:-1]                             # targets are inputs shifted by one


def synthetic_text(seed, n, alphabet):
    rng = np.random.default_rng(seed)
    return bytes(rng.choice(np.frombuffer(alphabet, dtype=np.uint8), size=n).tolist())


@pytest.mark.parametrize("seed,n,alphabet", [(1, 5000, b"abcdefgh ijkl\nmnop,.;!?ABCDEFG"),
                                             (2, 3000, bytes(range(256))), (3, 1, b"z")])
def test_native_tokenizer_matches_oracle(b, seed, n, alphabet):
    text = synthetic_text(seed, n, alphabet)
    vocab, ids = b.char_vocab(text), None
    assert vocab == cd.char_vocab(text)
    ids = b.char_encode(text, vocab)
    assert ids.tolist() == cd.encode(text, vocab)
    assert b.char_decode(ids, vocab) == text
    for r in (0.9, 0.5, 0.1):
        assert b.split_point(len(text), r) == cd.split_point(len(text), r)


def test_native_tokenizer_errors(b):
    vocab = b.char_vocab(b"abc")
    with pytest.raises(b.GPT2Error):
        b.char_encode(b"abd", vocab)                       # 'd' is not in the vocabulary
    with pytest.raises(b.GPT2Error):
        b.char_decode(np.array([0, 3], dtype=np.int32), vocab)  # id 3 >= vocabulary size


@pytest.mark.gpu
def test_batch_windows_bit_exact(b):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    text = synthetic_text(4, 20000, b"the quick brown fox jumps over a lazy dog\n")
    vocab = cd.char_vocab(text)
    data = cd.encode(text, vocab)
    T, B = 64, 32
    rng = np.random.default_rng(5)
    offs = rng.integers(0, len(data) - T - 1, size=B).tolist()   # get_batch's range
    offs[0], offs[1] = 0, len(data) - T - 1                      # both ends of the valid range
    d = torch.tensor(data, dtype=torch.int32, device="cuda")
    o = torch.tensor(offs, dtype=torch.int64, device="cuda")
    x = torch.empty((B, T), dtype=torch.int32, device="cuda")
    y = torch.empty((B, T), dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    b.batch_windows(d, o, x, y, st)
    torch.cuda.synchronize()
    xs, ys = cd.get_batch(data, offs, T)
    assert x.cpu().numpy().tolist() == xs and y.cpu().numpy().tolist() == ys
    assert int(st.item()) == 0
    o2 = torch.tensor([5, len(data) - T], dtype=torch.int64, device="cuda")  # second one runs past the end
    x2 = torch.full((2, T), 7, dtype=torch.int32, device="cuda")
    y2 = torch.full((2, T), 7, dtype=torch.int32, device="cuda")
    b.batch_windows(d, o2, x2, y2, st)
    torch.cuda.synchronize()
    assert int(st.item()) & b.STATUS_WINDOW_RANGE
    assert x2[0].cpu().numpy().tolist() == data[5:5 + T]
    assert np.all(x2[1].cpu().numpy() == 0) and np.all(y2[1].cpu().numpy() == 0)
