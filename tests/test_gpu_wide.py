"""GPU parity of the wide instances (512 and 1024 threads per workgroup, 8 and
16 wavefronts on one row) against the CPU oracle, through the C ABI.

The wide instances share every code path with the 256-thread ones, at other
sizes: tiles of 4096 or 8192 elements, samples of 8192 or 16384 for the
speculative bound, 8 or 16 wave segments per row, candidate buffers of 6144
to 12288.  Each test forces a width with the force_block override and
compares element by element (bit-exact, integer output).
"""

from __future__ import annotations

import numpy as np
import pytest

import row_radix_top_amd as rrt
from oracle import topk_ragged_oracle
from row_radix_top_amd import workloads
from tests.gpu_util import assert_same, require_gpu, run_gpu

pytestmark = pytest.mark.gpu

BLOCKS = [512, 1024]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("name", ["small", "decode", "mtp", "long_k1024", "long_k2048", "prefill"])
def test_workloads_single_path(name, block):
    w = workloads.make_workload(name)
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=f"{name} block={block}", force_path=1, force_block=block)
    assert plan["path"] == rrt.PATH_SINGLE and plan["block"] == block, plan
    assert_same(got, exp, f"{name} block={block}")


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("name,G", [("long_k1024", 0), ("long_k2048", 0), ("long_k2048", 5), ("mtp", 3)])
def test_workloads_multi_path(name, G, block):
    w = workloads.make_workload(name)
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    ov = dict(force_path=2, force_block=block)
    if G:
        ov["force_wg_per_row"] = G
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=f"{name} multi G={G} block={block}", **ov)
    assert plan["path"] == rrt.PATH_MULTI and plan["block"] == block, plan
    assert_same(got, exp, f"{name} multi G={G} block={block}")


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("dist", ["normal", "levels", "const", "inc", "dec", "signed_zero", "denorm", "inf"])
def test_edge_rows(dist, block):
    stride = 20000
    for K in (1, 300, 2048):
        lens = [0, 1, K - 1, K, K + 1, 4095, 4096, 4097, 8191, 8192, 8193, 12288, 16383, 16384, 16385,
                stride, -5, 99999]
        s, L = workloads.random_rows(3000 + K + block, len(lens), stride, lens, dist=dist, levels=3)
        exp = topk_ragged_oracle(s, L, K)
        got, _ = run_gpu(s, L, K, tag=f"wide edge {dist} K={K} block={block}", force_path=1, force_block=block)
        assert_same(got, exp, f"wide edge {dist} K={K} block={block}")
        got, _ = run_gpu(s, L, K, tag=f"wide edge multi {dist} K={K} block={block}", force_path=2,
                         force_wg_per_row=3, force_block=block)
        assert_same(got, exp, f"wide edge multi {dist} K={K} block={block}")


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("offset,stride", [(1, 40001), (2, 40002), (0, 40000)])
def test_narrow_loads(offset, stride, block):
    lens = [stride, stride - 1, 20000, 16385, 9000, 4099, 17]
    s, L = workloads.random_rows(88 + offset, len(lens), stride, lens, dist="levels", levels=60)
    for K in (16, 2048):
        exp = topk_ragged_oracle(s, L, K)
        for path in (1, 2):
            got, plan = run_gpu(s, L, K, offset=offset, tag=f"wide narrow off={offset} path={path} block={block}",
                                force_path=path, force_block=block)
            assert plan["block"] == block
            assert_same(got, exp, f"wide narrow offset={offset} K={K} path={path} block={block}")


@pytest.mark.parametrize("block", BLOCKS)
def test_wave_segments(block):
    """Rows streamed wave by wave with 8 or 16 segments: lengths at the
    segment edges, a last segment holding every large value (its part of
    the buffer overflows and the row goes again on the general path),
    heavy ties, monotone rows, and rows whose bound fails."""
    W = block // 64
    rng = np.random.default_rng(900 + block)
    stride = 65536
    edge = W * 1024
    lens = [edge - 1, edge, edge + 1, edge + 511, edge + 512, 2 * edge, 2 * edge + 3, 3 * edge - 7,
            40000, stride - 1, stride, 50001, 24576, 24577, 32768, 20000]
    rows = []
    for i, n in enumerate(lens):
        kind = i % 5
        if kind == 0:
            x = rng.standard_normal(stride, dtype=np.float32)
        elif kind == 1:
            x = rng.standard_normal(stride, dtype=np.float32)
            x[(W - 1) * n // W:] += np.float32(5.0)        # the last segment holds the largest values
        elif kind == 2:
            x = rng.integers(0, 3, size=stride).astype(np.float32)
        elif kind == 3:
            x = np.arange(stride, dtype=np.float32) * np.float32(0.25)
            if i % 2:
                x = -x
        else:
            x = rng.standard_normal(stride, dtype=np.float32)
            x[2048 * W:] -= np.float32(10.0)                # the sample holds the largest values
        rows.append(x)
    s = np.ascontiguousarray(np.stack(rows))
    workloads.fill_tails(rng, s, np.array(lens))
    L = np.array(lens, dtype=np.int32)
    for K in (129, 1000, 2048):
        exp = topk_ragged_oracle(s, L, K)
        for grid in (0, 1):
            got, plan = run_gpu(s, L, K, tag=f"wide segments K={K} grid={grid} block={block}", force_path=1,
                                max_grid=grid, force_block=block)
            assert plan["path"] == rrt.PATH_SINGLE and plan["block"] == block
            assert_same(got, exp, f"wide segments K={K} grid={grid} block={block}")


@pytest.mark.parametrize("block", BLOCKS)
def test_large_k_values_and_offsets(block):
    import torch
    dev = torch.device("cuda:0")
    lens = [70000, 65536, 50000, 4096, 4097, 3000, 0, 9000]
    s, L = workloads.random_rows(77 + block, len(lens), 70000, lens, dist="levels", levels=5000)
    for K in (4096, 2048):
        exp = topk_ragged_oracle(s, L, K)
        for path in (1, 2):
            got, plan = run_gpu(s, L, K, tag=f"wide K={K} path={path} block={block}", force_path=path,
                                force_block=block)
            assert plan["block"] == block
            assert_same(got, exp, f"wide K={K} path={path} block={block}")
    # Values and row offsets on the wide instances (32-bit indices for K = 4096).
    K = 2048
    sd = torch.from_numpy(s).to(dev)
    Ld = torch.from_numpy(L).to(dev)
    offs = torch.arange(len(lens), dtype=torch.int32, device=dev) * 100000
    ws = rrt.new_workspace(rrt.workspace_size(len(lens), 70000, K, scores=sd, force_path=1, force_block=block), dev)
    idx, val = rrt.topk_ragged_values(sd, Ld, K, workspace=ws, row_offsets=offs, force_path=1, force_block=block)
    torch.cuda.synchronize()
    exp = topk_ragged_oracle(s, L, K)
    exp_off = np.where(exp >= 0, exp + np.arange(len(lens))[:, None] * 100000, -1)
    assert_same(idx.cpu().numpy(), exp_off, f"wide values/offsets block={block}")
    v = val.cpu().numpy()
    for r in range(len(lens)):
        m = int(min(K, max(lens[r], 0)))
        assert np.array_equal(v[r, :m].view(np.uint32), s[r, exp[r, :m]].view(np.uint32))
        assert np.all(np.isneginf(v[r, m:]))


def test_bf16_on_512_threads():
    import torch
    dev = torch.device("cuda:0")
    w = workloads.make_workload("mtp")
    sb = torch.from_numpy(w.scores).to(dev).to(torch.bfloat16)
    widened = (sb.cpu().view(torch.int16).numpy().astype(np.uint32) << 16).view(np.float32)
    # The tails become other bit patterns after rounding; the oracle reads only the prefixes.
    exp = topk_ragged_oracle(np.ascontiguousarray(widened), w.flat_lengths, w.K)
    L = torch.from_numpy(w.flat_lengths).to(dev)
    for path in (1, 2):
        ws = rrt.new_workspace(rrt.workspace_size(w.num_rows, w.row_stride, w.K, device=dev, force_path=path,
                                                  force_block=512), dev)
        out = rrt.topk_ragged_bf16(sb, L, w.K, workspace=ws, force_path=path, force_block=512)
        torch.cuda.synchronize()
        assert_same(out.cpu().numpy(), exp, f"bf16 512 path={path}")


def test_graph_replay_wide():
    """Two wide launches captured in one graph (a 1024-thread one-workgroup
    launch with a ticket counter, a 512-thread cooperative one), replayed
    while the lengths change; every replay exact, the workspaces all-zero."""
    import torch
    dev = torch.device("cuda:0")
    rows, stride, K = 12, 65536, 2048
    rng = np.random.default_rng(55)
    s_np, _ = workloads.random_rows(56, rows, stride, [stride] * rows, dist="levels", levels=4000)
    pats = [np.full(rows, stride, np.int32)] + [rng.integers(0, stride + 1, size=rows).astype(np.int32)
                                               for _ in range(5)]
    exps = [topk_ragged_oracle(s_np, p, K) for p in pats]
    scores = torch.from_numpy(s_np).to(dev)
    L = torch.from_numpy(pats[0]).to(dev)
    cfgs = [dict(force_path=1, force_block=1024, max_grid=5), dict(force_path=2, force_block=512)]
    outs = [torch.empty((rows, K), dtype=torch.int32, device=dev) for _ in cfgs]
    wss = [rrt.new_workspace(rrt.workspace_size(rows, stride, K, scores=scores, **c), dev) for c in cfgs]
    for c, o, ws in zip(cfgs, outs, wss):
        rrt.topk_ragged(scores, L, K, out=o, workspace=ws, **c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for c, o, ws in zip(cfgs, outs, wss):
                rrt.topk_ragged(scores, L, K, out=o, workspace=ws, stream=st, **c)
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(30):
        i = rep % len(pats)
        L.copy_(torch.from_numpy(pats[i]).to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for c, o, ws in zip(cfgs, outs, wss):
            assert_same(o.cpu().numpy(), exps[i], f"replay {rep} {c}")
            if ws is not None:
                assert int(ws.count_nonzero().item()) == 0, f"workspace not clean after replay {rep} {c}"
    del g


def _above_sample_rows(seed: int, rows: int, stride: int, K: int, levels: bool) -> tuple[np.ndarray, np.ndarray]:
    """Rows whose K best all lie outside the speculative sample and above its
    largest value: N(0, 1) everywhere, plus K + K // 2 values of 100 or more
    at random positions p with p mod 4096 >= 2048.  The sample is at most the
    first 1024 elements of each wave segment, and segments start at multiples
    of 4096 in these rows, so it holds none of them; the final selection's
    first pass then finds the K-th best in its open top bin.  With levels the
    large values take 11 distinct values (ties at the threshold)."""
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((rows, stride), dtype=np.float32)
    pos = np.nonzero(np.arange(stride) % 4096 >= 2048)[0]
    m = K + K // 2
    for r in range(rows):
        p = rng.choice(pos, size=m, replace=False)
        if levels:
            s[r, p] = np.float32(100.0) + rng.integers(0, 11, size=m).astype(np.float32)
        else:
            s[r, p] = np.float32(100.0) + rng.random(m, dtype=np.float32) * np.float32(50.0)
    return s, np.full(rows, stride, np.int32)


@pytest.mark.parametrize("levels", [False, True])
@pytest.mark.parametrize("block", BLOCKS)
def test_threshold_above_sample(block, levels):
    """The final selection of a row streamed wave by wave starts from the
    bound and the sample's largest key, with keys above that in its top bin:
    rows whose threshold lies in that bin, one workgroup per row."""
    s, L = _above_sample_rows(300 + block + int(levels), 6, 65536, 2048, levels)
    for K in (1000, 2048):
        exp = topk_ragged_oracle(s, L, K)
        got, plan = run_gpu(s, L, K, tag=f"above sample K={K} block={block} levels={levels}", force_path=1,
                            force_block=block)
        assert plan["path"] == rrt.PATH_SINGLE and plan["block"] == block
        assert_same(got, exp, f"above sample K={K} block={block} levels={levels}")


@pytest.mark.parametrize("levels", [False, True])
def test_threshold_above_sample_cooperative(levels):
    """The same on the cooperative path (rows of 131072, 8 or 16 workgroups
    per row): the union's selection starts from the shared bound and the
    shared sample's largest key."""
    s, L = _above_sample_rows(400 + int(levels), 4, 131072, 2048, levels)
    for K, G in ((1024, 8), (2048, 16)):
        exp = topk_ragged_oracle(s, L, K)
        got, plan = run_gpu(s, L, K, tag=f"above sample coop K={K} G={G} levels={levels}", force_path=2,
                            force_wg_per_row=G, force_block=512)
        assert plan["path"] == rrt.PATH_MULTI and plan["wg_per_row"] == G
        assert_same(got, exp, f"above sample coop K={K} G={G} levels={levels}")
