"""Python access to the CPU oracle.  TEST INFRASTRUCTURE ONLY.

``topk_ragged_oracle`` runs the C++ oracle (``oracle_topk.cpp``: per-row
nth_element under the order "larger value first, then lower index", chosen
indices sorted ascending, -1 padding).

Source of the op: vLLM persistent_topk pages -- PR #54110 ("low shared
memory fallback"), its code excerpt: the per-row decode top-K takes the
logits, next_n, the lengths, the output and both logits strides, and next_n
is the second dimension of a 2-D lengths tensor, else 1; PR #41189 (deadlock
fix), its code excerpt: fp32 logits in, int32 indices out.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_topk.so")
_lib = None


def load_library():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build_oracle
            build_oracle.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_topk_ragged.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32]
        lib.oracle_topk_ragged.restype = ctypes.c_int
        _lib = lib
    return _lib


def _next_n_of(lengths: np.ndarray) -> int:
    # PR #54110 excerpt: a 2-D lengths tensor [batch, next_n] is the
    # multi-token layout, a 1-D one is plain decode (next_n = 1).
    return int(lengths.shape[1]) if lengths.ndim == 2 else 1


def topk_ragged_oracle(scores: np.ndarray, lengths: np.ndarray, K: int,
                       next_n: int | None = None, threads: int = 0) -> np.ndarray:
    """int32 [num_rows, K]: per row, the indices of the K best of the first
    lengths[r] scores ("best": larger value, then lower index), ascending,
    padded with -1.  Raises on a NaN inside a valid prefix (out of contract).
    """
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    assert scores.ndim == 2
    lengths = np.asarray(lengths)
    if next_n is None:
        next_n = _next_n_of(lengths)
    flat = np.ascontiguousarray(lengths.reshape(-1), dtype=np.int32)
    num_rows, stride = scores.shape
    assert flat.shape[0] == num_rows, "one length per row"
    out = np.empty((num_rows, K), dtype=np.int32)
    lib = load_library()
    rc = lib.oracle_topk_ragged(scores.ctypes.data, stride, flat.ctypes.data, num_rows,
                                next_n, K, out.ctypes.data, int(threads))
    if rc == -2:
        raise ValueError("NaN inside a valid prefix: outside the op's contract")
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return out


def topk_ragged_offsets_oracle(scores: np.ndarray, lengths: np.ndarray, K: int, row_offsets,
                               next_n: int | None = None, threads: int = 0) -> np.ndarray:
    """The same selection with every chosen index of row r reported as
    row_offsets[r] + index; the -1 padding is unchanged.

    Reading of the PR #41189 page, whose fallback calls a "RaggedTransform"
    variant of the ragged top-K without defining it: a row whose scores start
    at row_offsets[r] in a flat layout (the rows' valid prefixes laid end to
    end) reports positions in that layout.  Raises if a shifted index falls
    outside [0, 2^31 - 1] (out of contract).
    """
    out = topk_ragged_oracle(scores, lengths, K, next_n=next_n, threads=threads).astype(np.int64)
    off = np.asarray(row_offsets, dtype=np.int64).reshape(-1)
    assert off.shape[0] == out.shape[0], "one offset per row"
    shifted = np.where(out >= 0, out + off[:, None], -1)
    chosen = out >= 0
    if chosen.any() and (shifted[chosen].min() < 0 or shifted[chosen].max() > 2**31 - 1):
        raise ValueError("row_offsets[r] + index leaves [0, 2^31 - 1]: outside the op's contract")
    return shifted.astype(np.int32)


def topk_ragged_values_oracle(scores: np.ndarray, lengths: np.ndarray, K: int, row_offsets=None,
                              next_n: int | None = None, threads: int = 0):
    """(indices, values): the selection (shifted by row_offsets when given)
    and, at each chosen position, the score itself (its exact fp32 bits);
    -inf where the index is -1.  Not on the pages: a convenience output."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    if row_offsets is None:
        idx = topk_ragged_oracle(scores, lengths, K, next_n=next_n, threads=threads)
        off = np.zeros(scores.shape[0], dtype=np.int64)
    else:
        idx = topk_ragged_offsets_oracle(scores, lengths, K, row_offsets, next_n=next_n, threads=threads)
        off = np.asarray(row_offsets, dtype=np.int64).reshape(-1)
    vals = np.full(idx.shape, -np.inf, dtype=np.float32)
    rows, cols = np.nonzero(idx >= 0)
    vals[rows, cols] = scores[rows, idx[rows, cols].astype(np.int64) - off[rows]]
    return idx, vals


def topk_ragged_strided_oracle(flat: np.ndarray, row_stride: int, col_stride: int, num_cols: int,
                               num_rows: int, lengths: np.ndarray, K: int, next_n: int | None = None,
                               threads: int = 0) -> np.ndarray:
    """The selection over rows with a column stride (the PR #54110 page
    passes both logits strides to the per-row top-K): entry (r, c) is
    flat[r * row_stride + c * col_stride], lengths are clamped to
    [0, num_cols].  Only valid entries are read; the rest of each dense row
    is NaN, which the selection never reads."""
    flat = np.asarray(flat, dtype=np.float32).reshape(-1)
    L = np.asarray(lengths).reshape(-1).astype(np.int64)
    dense = np.full((num_rows, num_cols), np.nan, dtype=np.float32)
    for r in range(num_rows):
        n = int(min(max(L[r], 0), num_cols))
        if n:
            dense[r, :n] = flat[r * row_stride + np.arange(n, dtype=np.int64) * col_stride]
    return topk_ragged_oracle(dense, np.asarray(lengths), K, next_n=next_n, threads=threads)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 values (their 16 bits as uint16) as fp32: the 16 bits become the
    high half of the fp32 word, which is exact."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def topk_ragged_bf16_oracle(bits: np.ndarray, lengths: np.ndarray, K: int, next_n: int | None = None,
                            threads: int = 0) -> np.ndarray:
    """The selection over bf16 scores (given as uint16 bits [num_rows,
    row_stride]): the same rule on their exact fp32 widening."""
    return topk_ragged_oracle(widen_bf16(bits), lengths, K, next_n=next_n, threads=threads)
