"""The multi-workgroup path's chunks speculate from their first two tiles.

A chunk keeps the elements that reach its bound; if fewer than K do, the
bound was above the chunk's K-th best and the chunk streams again without
one.  Decreasing rows make every chunk's first tiles hold its largest
values (each bound fails), increasing rows the smallest (bounds that keep
almost everything), constant and few-level rows put ties at the bound, and
a row whose chunks alternate between the two fails some bounds and not
others.  Each case runs at several workgroups per row and K, and must equal
the oracle and leave the workspace all-zero.
"""

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


@pytest.mark.parametrize("dist", ["dec", "inc", "const", "levels", "normal"])
@pytest.mark.parametrize("G", [8, 16])
def test_multi_chunk_bounds(dist, G):
    stride = 131072
    lens = [stride, stride - 1, 100000, 65537, 40000, 8193, 4096, 2049]
    s, L = workloads.random_rows(4000 + G, len(lens), stride, lens, dist=dist, levels=7)
    for K in (129, 1024, 2048):
        exp = topk_ragged_oracle(s, L, K)
        got, plan = run_gpu(s, L, K, tag=f"multi spec {dist} G={G} K={K}", force_path=2, force_wg_per_row=G)
        assert plan["path"] == rrt.PATH_MULTI and plan["wg_per_row"] == G
        assert_same(got, exp, f"multi spec {dist} G={G} K={K}")


def test_multi_chunk_bounds_mixed():
    # Chunks of 8192 elements alternate decreasing and increasing runs.
    stride, G = 131072, 16
    rng = np.random.default_rng(77)
    x = np.empty(stride, np.float32)
    for c in range(stride // 8192):
        run = np.sort(rng.standard_normal(8192).astype(np.float32))
        x[c * 8192:(c + 1) * 8192] = run[::-1] if c % 2 == 0 else run
    s = np.stack([x, x[::-1].copy(), np.roll(x, 4096)])
    L = np.array([stride, stride - 5, 90000], np.int32)
    workloads.fill_tails(rng, s, L)
    for K in (700, 2048):
        exp = topk_ragged_oracle(s, L, K)
        got, plan = run_gpu(s, L, K, tag=f"multi spec mixed K={K}", force_path=2, force_wg_per_row=G)
        assert plan["path"] == rrt.PATH_MULTI and plan["chunk"] == 8192
        assert_same(got, exp, f"multi spec mixed K={K}")
