"""hipGraph capture and replay of the launch (through torch.cuda.CUDAGraph on
the capture stream), with the lengths buffer rewritten between replays.

The point is the in-kernel workspace cleanup (PR #41748 page: the per-call
memset was replaced by cleanup at the end of the kernel, which also makes
graph replay possible; its review warns that a counter reset can race with
the histogram zeroing).  Every replay must leave the workspace all-zero and
produce exactly the oracle's output for the lengths it saw.
"""

from __future__ import annotations

import numpy as np
import pytest

import row_radix_top_amd as rrt
from oracle import topk_ragged_oracle
from row_radix_top_amd import workloads
from tests.gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _length_patterns(rng, npat, rows, stride):
    pats = []
    for i in range(npat):
        if i == 0:
            pats.append(np.full(rows, stride, np.int32))
        elif i == 1:
            pats.append(rng.integers(0, 3000, size=rows).astype(np.int32))  # mostly short
        else:
            pats.append(rng.integers(0, stride + 1, size=rows).astype(np.int32))
    return pats


@pytest.mark.parametrize("path,G,grid,block", [(2, 0, 0, 0), (2, 7, 0, 0), (1, 0, 0, 0), (1, 0, 5, 0),
                                                (2, 0, 0, 512), (1, 0, 5, 512)])
def test_graph_replay_changing_lengths(path, G, grid, block):
    # grid=5 < 12 rows: the one-workgroup path hands rows out by a ticket
    # counter in the workspace, which must be back at zero after each replay.
    # The cooperative path's counters, slots and published lists too, at both
    # widths.
    import torch
    dev = torch.device("cuda:0")
    rows, stride, K = 12, 65536, 2048
    rng = np.random.default_rng(50 + path + G + block)
    s_np, _ = workloads.random_rows(51, rows, stride, [stride] * rows, dist="levels", levels=4000)
    pats = _length_patterns(rng, 8, rows, stride)
    exps = [torch.from_numpy(topk_ragged_oracle(s_np, p, K)).to(dev) for p in pats]
    pats_d = [torch.from_numpy(p).to(dev) for p in pats]

    scores = torch.from_numpy(s_np).to(dev)
    L = pats_d[0].clone()
    out = torch.empty((rows, K), dtype=torch.int32, device=dev)
    ov = dict(force_path=path, force_wg_per_row=G) if G else dict(force_path=path)
    if grid:
        ov["max_grid"] = grid
    if block:
        ov["force_block"] = block
    plan = rrt.query_plan(scores, K, **ov)
    note(f"replay plan={plan}")
    assert plan["path"] == path
    nbytes = rrt.workspace_size(rows, stride, K, scores=scores, **ov)
    ws = rrt.new_workspace(nbytes, dev) if nbytes else None

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rrt.topk_ragged(scores, L, K, out=out, workspace=ws, **ov)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out, exps[0])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rrt.topk_ragged(scores, L, K, out=out, workspace=ws, **ov)
    torch.cuda.synchronize()

    n_replay = 3000
    for it in range(n_replay):
        i = (it * 5 + 3) % len(pats)
        L.copy_(pats_d[i])
        out.fill_(-7)
        g.replay()
        if it % 25 == 0 or it < 40:
            torch.cuda.synchronize()
            assert torch.equal(out, exps[i]), f"replay {it} pattern {i}"
            if ws is not None:
                assert int(ws.count_nonzero().item()) == 0, f"workspace not zero after replay {it}"
    torch.cuda.synchronize()
    if ws is not None:
        assert rrt.workspace_status(ws) == 0
    note(f"{n_replay} replays ok")


def test_back_to_back_launches_share_workspace():
    # Many stream-ordered launches with one workspace and no host sync
    # between them: each must see the workspace the previous one cleaned.
    import torch
    dev = torch.device("cuda:0")
    w = workloads.make_workload("long_k1024")
    scores = torch.from_numpy(w.scores).to(dev)
    L = torch.from_numpy(w.flat_lengths).to(dev)
    exp = torch.from_numpy(topk_ragged_oracle(w.scores, w.lengths, w.K)).to(dev)
    ws = rrt.new_workspace(rrt.workspace_size(w.num_rows, w.row_stride, w.K, device=dev), dev)
    outs = [rrt.topk_ragged(scores, L, w.K, workspace=ws) for _ in range(200)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, exp), f"launch {i}"
    assert int(ws.count_nonzero().item()) == 0
