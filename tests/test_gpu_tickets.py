"""The one-workgroup path's row tickets, at the boundaries of their scheme.

With G workgroups and U > G rows, workgroup b takes row b, then row b + G,
then rows 2G, 2G + 1, ... from a counter in the workspace header, drawn when
each row starts; the draw that hands out the last ticket resets the counter.
Row counts around G, 2G and 3G, and grids from 1 to 9 workgroups, must give
the oracle's output on every launch of a workspace reused without
re-initialisation, and leave it all-zero each time (a counter left behind
would skip or repeat rows on the next launch).
"""

from __future__ import annotations

import numpy as np
import pytest

import row_radix_top_amd as rrt
from oracle import topk_ragged_oracle
from row_radix_top_amd import workloads
from tests.gpu_util import assert_same, note, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _cases():
    out = []
    for G in (1, 2, 3, 5, 9):
        for U in sorted({G + 1, 2 * G - 1, 2 * G, 2 * G + 1, 3 * G + 2}):
            if U > G:
                out.append((G, U))
    return out


@pytest.mark.parametrize("G,U", _cases())
def test_ticket_boundaries(G, U):
    import torch
    dev = torch.device("cuda:0")
    stride, K = 20000, 512
    rng = np.random.default_rng(1000 + 17 * G + U)
    # Long rows (wave by wave), general-path rows and rows with n <= K.
    lengths = rng.choice([stride, 17000, 9000, 3000, K, 100, 0], size=U).astype(np.int32)
    s_np, L_np = workloads.random_rows(2000 + U, U, stride, lengths, dist="normal")
    exp = topk_ragged_oracle(s_np, L_np, K)
    scores = torch.from_numpy(s_np).to(dev)
    L = torch.from_numpy(L_np).to(dev)
    plan = rrt.query_plan(scores, K, max_grid=G)
    note(f"tickets G={G} U={U} plan={plan}")
    assert plan["path"] == rrt.PATH_SINGLE and plan["grid"] == G
    nbytes = rrt.workspace_size(U, stride, K, scores=scores, max_grid=G)
    assert nbytes > 0, "rows past the grid need the ticket counter"
    ws = rrt.new_workspace(nbytes, dev)
    for launch in range(3):
        out = rrt.topk_ragged(scores, L, K, workspace=ws, max_grid=G)
        torch.cuda.synchronize()
        assert_same(out.cpu().numpy(), exp, f"G={G} U={U} launch {launch}")
        assert int(ws.count_nonzero().item()) == 0, f"G={G} U={U}: workspace not all-zero after launch {launch}"


@pytest.mark.parametrize("G,U,block", [(2, 5, 512), (3, 7, 1024), (4, 9, 512)])
def test_ticket_boundaries_wide(G, U, block):
    # The same scheme on 512- and 1024-thread workgroups, with rows longer
    # than 16-bit indices hold.
    import torch
    dev = torch.device("cuda:0")
    stride, K = 70000, 1024
    s_np, L_np = workloads.random_rows(3000 + U, U, stride, [stride, 69000, 40000, 70000, 5000, 66000, 70000,
                                                              1000, 68000][:U], dist="normal")
    exp = topk_ragged_oracle(s_np, L_np, K)
    scores = torch.from_numpy(s_np).to(dev)
    L = torch.from_numpy(L_np).to(dev)
    ov = dict(force_path=1, max_grid=G, force_block=block)
    plan = rrt.query_plan(scores, K, **ov)
    note(f"tickets wide G={G} U={U} block={block} plan={plan}")
    assert plan["block"] == block and plan["grid"] == G
    ws = rrt.new_workspace(rrt.workspace_size(U, stride, K, scores=scores, **ov), dev)
    for launch in range(3):
        out = rrt.topk_ragged(scores, L, K, workspace=ws, **ov)
        torch.cuda.synchronize()
        assert_same(out.cpu().numpy(), exp, f"wide G={G} U={U} block={block} launch {launch}")
        assert int(ws.count_nonzero().item()) == 0, f"wide G={G} U={U} block={block}: workspace not all-zero"
