"""Seeded synthetic inputs for ragged per-row top-K.

This module only draws numbers. It holds none of the selection arithmetic, so
both the CPU oracle and the HIP path can be fed from it without sharing any
of the method's code.

The pages (vLLM ``persistent_topk``: PR #41189 "deadlock fix" excerpt, PR
#54110 "low shared memory fallback" excerpt) describe the op as taking an fp32
``logits`` matrix with a row stride, int32 ragged ``lengths`` (1-D for decode,
2-D ``[batch, next_n]`` for multi-token rows) and returning int32 indices,
``[num_rows, TopK]``. No public dataset is involved; the five workloads below
stand in for the sparse-attention indexer's decode, multi-token and prefill
score rows.

Recipe shared by every workload:

* ``numpy.random.default_rng(seed)`` (PCG64); values via
  ``standard_normal(dtype=float32)``.
* Entries past a row's length are filled with uniformly random 32-bit
  patterns reinterpreted as fp32 (NaN, inf and huge values included), so any
  read past ``lengths[r]`` that leaks into the result breaks parity.
"""

from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_workload", "fill_tails", "valid_bytes"]


@dataclasses.dataclass
class Workload:
    name: str
    scores: np.ndarray  # float32 [num_rows, row_stride], C-contiguous
    lengths: np.ndarray  # int32 [num_rows] or [batch, next_n]
    K: int
    next_n: int
    description: str

    @property
    def num_rows(self) -> int:
        return int(self.scores.shape[0])

    @property
    def row_stride(self) -> int:
        return int(self.scores.shape[1])

    @property
    def flat_lengths(self) -> np.ndarray:
        return np.ascontiguousarray(self.lengths.reshape(-1), dtype=np.int32)


def fill_tails(rng: np.random.Generator, scores: np.ndarray, lengths: np.ndarray) -> None:
    """Overwrite every entry at or past its row's length with random bits."""
    flat = lengths.reshape(-1)
    stride = scores.shape[1]
    bits = scores.view(np.uint32)
    for r, n in enumerate(flat):
        n = int(min(max(int(n), 0), stride))
        if n < stride:
            bits[r, n:] = rng.integers(0, 2**32, size=stride - n, dtype=np.uint32)


def valid_bytes(lengths: np.ndarray, row_stride: int) -> int:
    """Bytes of valid fp32 scores: 4 * sum of the clamped lengths."""
    n = np.clip(lengths.reshape(-1).astype(np.int64), 0, row_stride)
    return int(4 * n.sum())


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _c1(seed: int) -> Workload:
    rng = np.random.default_rng(seed)
    rows, stride = 4, 8192
    s = _normal(rng, (rows, stride))
    lengths = np.full(rows, stride, dtype=np.int32)
    return Workload("small", s, lengths, 512, 1,
                    "4 rows x 8192 fp32 N(0,1), all lengths 8192, K=512, next_n=1")


def _c2(seed: int) -> Workload:
    rng = np.random.default_rng(seed)
    rows, stride, K = 64, 32768, 2048
    s = _normal(rng, (rows, stride))
    lengths = rng.integers(1, stride + 1, size=rows, dtype=np.int64).astype(np.int32)
    fill_tails(rng, s, lengths)
    return Workload("decode", s, lengths, K, 1,
                    "decode: 64 rows, row_stride 32768, lengths U{1..32768}, K=2048, "
                    "N(0,1), random-bit tails")


def _c3(seed: int) -> Workload:
    rng = np.random.default_rng(seed)
    batch, next_n, stride, K = 32, 2, 65536, 2048
    ctx = rng.integers(16384, 65536 + 1, size=batch, dtype=np.int64)
    # Row (b, j) of a multi-token step sees c_b - 1 + j context positions.
    lengths = (ctx[:, None] - 1 + np.arange(next_n)[None, :]).astype(np.int32)
    s = _normal(rng, (batch * next_n, stride))
    fill_tails(rng, s, lengths)
    return Workload("mtp", s, lengths, K, next_n,
                    "MTP: batch 32 x next_n 2 = 64 rows, row_stride 65536, "
                    "c_b U{16384..65536}, len(b,j) = c_b-1+j, K=2048, N(0,1)")


def _c4(seed: int, K: int = 2048) -> Workload:
    rng = np.random.default_rng(seed)
    rows, stride = 16, 131072
    lengths = rng.integers(65536, stride + 1, size=rows, dtype=np.int64).astype(np.int32)
    z = _normal(rng, (rows, stride))
    # Rows 8..15: 64 levels (q - 31.5)/8, q = clip(floor((z + 4) * 8), 0, 63).
    # Every level is exact in fp32 and none is zero; ties are heavy.
    q = np.clip(np.floor((z[8:] + np.float32(4.0)) * np.float32(8.0)), 0, 63)
    z[8:] = ((q - np.float32(31.5)) / np.float32(8.0)).astype(np.float32)
    fill_tails(rng, z, lengths)
    return Workload(f"long_k{K}", z, lengths, K, 1,
                    f"long rows: 16 x 131072, lengths U{{65536..131072}}, K={K}; rows 0-7 "
                    "N(0,1), rows 8-15 quantised to 64 levels")


def _c5(seed: int) -> Workload:
    rng = np.random.default_rng(seed)
    rows, stride, K = 4096, 65536, 2048
    s = _normal(rng, (rows, stride))
    off = rng.uniform(-4.0, 4.0, size=rows).astype(np.float32)
    s += off[:, None]
    lengths = (61440 + np.arange(rows)).astype(np.int32)
    fill_tails(rng, s, lengths)
    return Workload("prefill", s, lengths, K, 1,
                    "prefill-shaped: 4096 rows, row_stride 65536, len_i = 61440+i, "
                    "N(0,1) + per-row offset U(-4,4), K=2048")


# name -> (builder, seed)
WORKLOADS = {
    "small": (_c1, 101),
    "decode": (_c2, 102),
    "mtp": (_c3, 103),
    "long_k1024": (lambda seed: _c4(seed, 1024), 104),
    "long_k2048": (lambda seed: _c4(seed, 2048), 104),
    "prefill": (_c5, 105),
}


def make_workload(name: str, seed: int | None = None) -> Workload:
    builder, default_seed = WORKLOADS[name]
    return builder(default_seed if seed is None else seed)


def random_rows(seed: int, num_rows: int, row_stride: int, lengths, dist: str = "normal",
                levels: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Small ad-hoc inputs for edge-case tests.

    ``dist``: "normal", "levels" (``levels`` distinct integers, heavy ties),
    "const" (one value per row), "inc"/"dec" (strictly monotone rows),
    "signed_zero" (a mix of +0.0, -0.0 and a few +-1), "denorm" (subnormal
    magnitudes of both signs), "inf" (normal values with +-inf mixed in).
    """
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32).reshape(-1)
    assert lengths.shape[0] == num_rows
    if dist == "normal":
        s = rng.standard_normal((num_rows, row_stride), dtype=np.float32)
    elif dist == "levels":
        s = rng.integers(0, max(levels, 1), size=(num_rows, row_stride)).astype(np.float32)
    elif dist == "const":
        s = np.repeat(rng.standard_normal((num_rows, 1), dtype=np.float32), row_stride, axis=1)
    elif dist == "inc":
        s = np.tile(np.arange(row_stride, dtype=np.float32), (num_rows, 1)) * np.float32(0.5)
    elif dist == "dec":
        s = np.tile(-np.arange(row_stride, dtype=np.float32), (num_rows, 1)) * np.float32(0.5)
    elif dist == "signed_zero":
        choice = rng.integers(0, 8, size=(num_rows, row_stride))
        s = np.where(choice < 3, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        s[choice == 6] = np.float32(1.0)
        s[choice == 7] = np.float32(-1.0)
    elif dist == "denorm":
        mant = rng.integers(1, 1 << 23, size=(num_rows, row_stride), dtype=np.uint32)
        sign = rng.integers(0, 2, size=(num_rows, row_stride), dtype=np.uint32) << np.uint32(31)
        s = (mant | sign).view(np.float32)
        s = np.ascontiguousarray(s)
    elif dist == "inf":
        s = rng.standard_normal((num_rows, row_stride), dtype=np.float32)
        pick = rng.integers(0, 16, size=(num_rows, row_stride))
        s[pick == 0] = np.float32(np.inf)
        s[pick == 1] = np.float32(-np.inf)
    else:
        raise ValueError(dist)
    s = np.ascontiguousarray(s, dtype=np.float32)
    fill_tails(rng, s, lengths)
    return s, lengths
