"""Seeded random sweep: shapes, strides (both index widths), K, value
distributions, lengths, paths, group sizes, workgroup widths, grid caps, load
widths, row offsets, values and bf16 scores, each case compared element by
element with the oracle.  Every case prints its parameters first, so a
failure names its case."""

from __future__ import annotations

import numpy as np
import pytest

import row_radix_top_amd as rrt
from oracle import topk_ragged_bf16_oracle, topk_ragged_offsets_oracle, topk_ragged_values_oracle
from row_radix_top_amd import workloads
from tests.gpu_util import assert_same, note, require_gpu

pytestmark = pytest.mark.gpu

DISTS = ["normal", "levels", "const", "inc", "dec", "signed_zero", "denorm", "inf"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _case(seed: int):
    rng = np.random.default_rng(1000 + seed)
    big = rng.random() < 0.3
    stride = int(rng.integers(65537, 140001)) if big else int(rng.integers(1, 65537))
    rows = int(rng.integers(1, max(2, min(300, 3_000_000 // stride))))
    K = int(rng.choice([1, 2, 7, 64, 100, 511, 512, 1024, 1500, 2047, 2048]))
    dist = str(rng.choice(DISTS))
    kind = rng.integers(0, 4)
    if kind == 0:
        lens = rng.integers(0, stride + 1, size=rows)
    elif kind == 1:
        lens = np.full(rows, stride)
    elif kind == 2:
        lens = rng.choice([0, 1, K - 1, K, K + 1, 2047, 2048, 2049, 8191, 8192, 8193, 8703, 8704, 16383, 16384,
                           16385, stride, stride + 5, -3],
                          size=rows)
    else:
        lens = stride - rng.integers(0, 64, size=rows)
    lens = np.asarray(lens, dtype=np.int64).clip(-5, stride + 10).astype(np.int32)
    s, L = workloads.random_rows(2000 + seed, rows, stride, lens, dist=dist, levels=int(rng.integers(2, 50)))
    ov = {}
    path = rng.integers(0, 4)
    if path == 1:
        ov["force_path"] = 1
        if rng.random() < 0.5:
            ov["max_grid"] = int(rng.integers(1, 9))
    elif path == 2:
        ov["force_path"] = 2
        if rng.random() < 0.5:
            ov["force_wg_per_row"] = int(rng.integers(1, 17))
    elif path == 3 and stride >= 4096:
        ov["force_path"] = int(rng.integers(1, 3))
        ov["force_block"] = 512
    offset = int(rng.choice([0, 0, 1, 2]))
    return dict(stride=stride, rows=rows, K=K, dist=dist, s=s, L=L, ov=ov, offset=offset,
                offsets=rng.random() < 0.3, values=rng.random() < 0.3, bf16=rng.random() < 0.2)


@pytest.mark.parametrize("seed", range(40))
def test_random_case(seed):
    import torch
    dev = torch.device("cuda:0")
    c = _case(seed)
    s, L, K, ov = c["s"], c["L"], c["K"], c["ov"]
    rows, stride = s.shape
    note(f"random seed={seed} rows={rows} stride={stride} K={K} dist={c['dist']} ov={ov} "
         f"offset={c['offset']} offsets={c['offsets']} values={c['values']} bf16={c['bf16']}")
    n = np.clip(L.astype(np.int64), 0, stride)
    starts = np.concatenate([[0], np.cumsum(n)[:-1]]) if c["offsets"] else None
    Ld = torch.from_numpy(L).to(dev)
    ro = torch.from_numpy(starts.astype(np.int32)).to(dev) if starts is not None else None
    if c["bf16"]:
        t = torch.from_numpy(s).to(torch.bfloat16)
        bits = t.view(torch.int16).numpy().view(np.uint16)
        exp = topk_ragged_bf16_oracle(bits, L, K)
        if starts is not None:
            exp = np.where(exp >= 0, exp + starts[:, None], -1).astype(np.int32)
        flat = np.zeros(bits.size + c["offset"], dtype=np.uint16)
        flat[c["offset"]:] = bits.reshape(-1)
        sd = torch.from_numpy(flat.view(np.int16)).to(dev).view(torch.bfloat16)[c["offset"]:].view(rows, stride)
        ws = rrt.new_workspace(rrt.workspace_size(rows, stride, K, device=dev, **ov), dev)
        got = rrt.topk_ragged_bf16(sd, Ld, K, workspace=ws, row_offsets=ro, **ov)
        torch.cuda.synchronize()
        assert_same(got.cpu().numpy(), exp, f"random {seed} bf16")
        return
    flat = np.zeros(s.size + c["offset"] + 4, dtype=np.float32)
    flat[c["offset"]:c["offset"] + s.size] = s.reshape(-1)
    sd = torch.from_numpy(flat).to(dev)[c["offset"]:c["offset"] + s.size].view(rows, stride)
    ws = rrt.new_workspace(rrt.workspace_size(rows, stride, K, scores=sd, **ov), dev)
    if c["values"]:
        ei, ev = topk_ragged_values_oracle(s, L, K, starts)
        vals = torch.empty((rows, K), dtype=torch.float32, device=dev)
        gi, gv = rrt.topk_ragged_values(sd, Ld, K, workspace=ws, out_values=vals, row_offsets=ro, **ov)
        torch.cuda.synchronize()
        assert_same(gi.cpu().numpy(), ei, f"random {seed} values")
        assert np.array_equal(gv.cpu().numpy().view(np.uint32), ev.view(np.uint32)), f"random {seed} values"
    else:
        exp = topk_ragged_offsets_oracle(s, L, K, starts) if starts is not None else None
        if exp is None:
            from oracle import topk_ragged_oracle
            exp = topk_ragged_oracle(s, L, K)
        got = rrt.topk_ragged(sd, Ld, K, workspace=ws, row_offsets=ro, **ov)
        torch.cuda.synchronize()
        assert_same(got.cpu().numpy(), exp, f"random {seed}")
    if ws is not None:
        assert int(ws.count_nonzero().item()) == 0, f"random {seed}: workspace not zero"
