"""GPU parity for split rows: rows cut into chunks that separate workgroups
stream, each publishing its candidates to the workspace, the last one to
arrive selecting over all of them (or streaming the whole row itself when
the shared bound turns out unusable).  Compared element by element with the
CPU oracle."""

from __future__ import annotations

import numpy as np
import pytest

import row_radix_top_amd as rrt
from oracle import topk_ragged_oracle
from row_radix_top_amd import workloads
from tests.gpu_util import assert_same, require_gpu, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("name,G,chunk", [
    ("decode", 4, 8192), ("decode", 2, 16384),
    ("mtp", 8, 8192), ("mtp", 4, 16384), ("mtp", 16, 4096),
    ("long_k1024", 16, 8192), ("long_k2048", 16, 8192), ("long_k2048", 8, 16384),
])
def test_workloads_split_rows(name, G, chunk):
    w = workloads.make_workload(name)
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=f"{name} split G={G} chunk={chunk}", force_path=1,
                        split_rows=w.num_rows, split_g=G, split_chunk=chunk)
    assert plan["path"] == rrt.PATH_SINGLE and plan["split_rows"] == w.num_rows
    assert plan["split_g"] == G and plan["split_chunk"] == chunk
    assert_same(got, exp, f"{name} G={G}")


@pytest.mark.parametrize("split_rows,G", [(512, 4), (1024, 2), (4096, 4)])
def test_prefill_split_tail(split_rows, G):
    w = workloads.make_workload("prefill")
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=f"prefill split tail {split_rows} G={G}",
                        split_rows=split_rows, split_g=G)
    assert plan["split_rows"] == split_rows and plan["grid"] < w.num_rows
    assert_same(got, exp, f"prefill split {split_rows} G={G}")


def _adversarial_rows(stride: int, seed: int):
    """Rows that defeat a bound taken from the quarter starts in every way
    the split path must survive, with lengths at and around chunk edges."""
    rng = np.random.default_rng(seed)
    Q = stride // 4
    rows, lens = [], []

    def add(x, n):
        rows.append(x.astype(np.float32))
        lens.append(n)

    z = lambda: rng.standard_normal(stride, dtype=np.float32)
    add(z(), stride)                                     # ordinary
    x = z(); x[2 * Q:3 * Q] += 10.0; add(x, stride)      # one chunk holds every large value
    x = z(); x[Q + 2048:Q + 4096] += 10.0; add(x, stride)  # a hot stretch the sample misses
    x = z(); x[Q + 8:Q + 40] += 10.0; add(x, stride - 3)   # a few large values, off the sample
    add(-np.arange(stride, dtype=np.float32), stride)    # decreasing: the bound overshoots
    add(np.arange(stride, dtype=np.float32), stride)     # increasing: one chunk overflows
    add(np.full(stride, 1.5, dtype=np.float32), stride)  # constant: too many to gather
    add(rng.integers(0, 3, size=stride).astype(np.float32), stride)  # three levels
    x = z(); x[::7] = -0.0; x[1::7] = 0.0; add(x, stride)  # signed zeros
    for n in (16384, 16385, 2 * 16384, 2 * 16384 + 1, 3 * 8192 - 1, 40000, 8191, 100, 0):
        add(z(), n)
    s = np.ascontiguousarray(np.stack(rows))
    L = np.array(lens, dtype=np.int32)
    workloads.fill_tails(rng, s, L)
    return s, L


@pytest.mark.parametrize("G,chunk", [(4, 16384), (8, 8192), (3, 24576)])
def test_split_adversarial_rows(G, chunk):
    s, L = _adversarial_rows(65536, 70 + G)
    for K in (1, 129, 700, 2048):
        exp = topk_ragged_oracle(s, L, K)
        for grid in (0, 1, 3):
            got, plan = run_gpu(s, L, K, tag=f"split adversarial G={G} chunk={chunk} K={K} grid={grid}",
                                force_path=1, split_rows=s.shape[0], split_g=G, split_chunk=chunk, max_grid=grid)
            assert plan["split_rows"] == s.shape[0]
            assert_same(got, exp, f"split adversarial G={G} K={K} grid={grid}")


@pytest.mark.parametrize("offset", [0, 1, 2])
def test_split_load_widths(offset):
    stride = {0: 65536, 1: 65529, 2: 65530}[offset]   # load widths 4, 1, 2
    s, L = _adversarial_rows(stride, 90 + offset)
    for K in (129, 2048):
        exp = topk_ragged_oracle(s, L, K)
        got, _ = run_gpu(s, L, K, offset=offset, tag=f"split offset={offset} K={K}", force_path=1,
                         split_rows=s.shape[0], split_g=4, split_chunk=16384)
        assert_same(got, exp, f"split offset={offset} K={K}")


def test_split_32bit_indices():
    # Rows longer than 65536 elements: the 32-bit-index instance.
    s, L = _adversarial_rows(131072, 95)
    for K in (129, 2048):
        exp = topk_ragged_oracle(s, L, K)
        for G, chunk in ((8, 16384), (16, 8192)):
            got, plan = run_gpu(s, L, K, tag=f"split 32-bit G={G} K={K}", force_path=1,
                                split_rows=s.shape[0], split_g=G, split_chunk=chunk)
            assert plan["idx16"] == 0
            assert_same(got, exp, f"split 32-bit G={G} K={K}")


def test_split_some_rows_only():
    # Whole rows first, the last rows split: both kinds of unit in one launch,
    # with more units than workgroups.
    rng = np.random.default_rng(97)
    lens = rng.integers(0, 65537, size=300)
    s, L = workloads.random_rows(97, 300, 65536, lens, dist="normal")
    for K in (64, 2048):
        exp = topk_ragged_oracle(s, L, K)
        for split, grid in ((100, 0), (300, 50), (1, 7)):
            got, plan = run_gpu(s, L, K, tag=f"split last {split} grid={grid} K={K}", force_path=1,
                                split_rows=split, split_g=4, max_grid=grid)
            assert plan["split_rows"] == split
            assert_same(got, exp, f"split last {split} grid={grid} K={K}")
