"""Character-level data preparation of the minigpt page, written out plainly.

TEST INFRASTRUCTURE ONLY (like the rest of oracle/): the tests are its only users.

Follows prepare_data and get_batch of minigpt.py (the minigpt page, section 二;
walkthrough 3.2): the vocabulary is the sorted set of distinct characters of the
text, ids are positions in it, the first int(ratio * n) ids are the training
split, and a batch takes windows data[i : i + T] as inputs and data[i + 1 : i + T + 1]
as targets. Reading: a character is one byte of the text (the same thing for ASCII
text; the native library works on bytes), and the window starts i, which
get_batch draws uniformly from [0, n - T - 1), are supplied by the caller.
"""
from __future__ import annotations


def char_vocab(text: bytes) -> list[int]:
    """Sorted distinct byte values of the text."""
    return sorted(set(text))


def encode(text: bytes, vocab: list[int]) -> list[int]:
    stoi = {ch: i for i, ch in enumerate(vocab)}
    return [stoi[c] for c in text]


def decode(ids: list[int], vocab: list[int]) -> bytes:
    return bytes(vocab[i] for i in ids)


def split_point(n: int, ratio: float = 0.9) -> int:
    return int(ratio * n)


def get_batch(data: list[int], offsets: list[int], T: int):
    """x[b] = data[i_b : i_b + T], y[b] = data[i_b + 1 : i_b + T + 1]."""
    xs = [data[i:i + T] for i in offsets]
    ys = [data[i + 1:i + T + 1] for i in offsets]
    return xs, ys
