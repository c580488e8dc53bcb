"""GPU parity for K above 2048 (the large layout: 7168 candidates, two
workgroups per CU), compared element by element with the oracle."""

from __future__ import annotations

import numpy as np
import pytest

import row_radix_top_amd as rrt
from oracle import topk_ragged_bf16_oracle, topk_ragged_oracle, topk_ragged_values_oracle
from row_radix_top_amd import workloads
from tests.gpu_util import assert_same, require_gpu, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("K", [2049, 3000, 4096])
@pytest.mark.parametrize("name", ["decode", "mtp", "long_k2048", "prefill"])
def test_large_k_workloads(name, K):
    w = workloads.make_workload(name)
    exp = topk_ragged_oracle(w.scores, w.lengths, K)
    paths = [{}, dict(force_path=1)]
    if name != "prefill":
        paths += [dict(force_path=2), dict(force_path=1, max_grid=5), dict(force_idx32=1)]
    if name in ("mtp", "long_k2048"):
        paths.append(dict(force_path=2, force_block=512))
    for ov in paths:
        got, plan = run_gpu(w.scores, w.lengths, K, tag=f"{name} K={K} {ov}", **ov)
        assert plan["kmax"] == 4096
        assert_same(got, exp, f"{name} K={K} {ov}")


@pytest.mark.parametrize("dist", ["normal", "levels", "const", "inc", "dec", "signed_zero"])
def test_large_k_edges(dist):
    K = 3333
    stride = 40000
    lens = [0, 1, K - 1, K, K + 1, 2 * K, 6143, 6144, 6145, 16384, 16385, 30000, stride, stride + 9]
    s, L = workloads.random_rows(71, len(lens), stride, lens, dist=dist, levels=40)
    exp = topk_ragged_oracle(s, L, K)
    for ov in ({}, dict(force_path=2, force_wg_per_row=3), dict(force_idx32=1), dict(force_path=1, max_grid=2)):
        got, _ = run_gpu(s, L, K, tag=f"large K edges {dist} {ov}", **ov)
        assert_same(got, exp, f"large K edges {dist} {ov}")


def test_large_k_values_offsets_bf16():
    import torch
    dev = torch.device("cuda:0")
    w = workloads.make_workload("decode")
    K = 4000
    n = np.clip(w.flat_lengths.astype(np.int64), 0, w.row_stride)
    starts = np.concatenate([[0], np.cumsum(n)[:-1]])
    s = torch.from_numpy(w.scores).to(dev)
    L = torch.from_numpy(w.flat_lengths).to(dev)
    ro = torch.from_numpy(starts.astype(np.int32)).to(dev)
    ei, ev = topk_ragged_values_oracle(w.scores, w.lengths, K, starts)
    ws = rrt.new_workspace(rrt.workspace_size(w.num_rows, w.row_stride, K, device=dev, force_idx32=1), dev)
    vals = torch.empty((w.num_rows, K), dtype=torch.float32, device=dev)
    gi, gv = rrt.topk_ragged_values(s, L, K, workspace=ws, out_values=vals, row_offsets=ro)
    torch.cuda.synchronize()
    assert_same(gi.cpu().numpy(), ei, "large K values")
    assert np.array_equal(gv.cpu().numpy().view(np.uint32), ev.view(np.uint32))
    tb = s.to(torch.bfloat16)
    bits = tb.view(torch.int16).cpu().numpy().view(np.uint16)
    exp = topk_ragged_bf16_oracle(bits, w.lengths, K)
    got = rrt.topk_ragged_bf16(tb, L, K, workspace=ws)
    torch.cuda.synchronize()
    assert_same(got.cpu().numpy(), exp, "large K bf16")
