"""The allocation-free entry point (topk_ragged_noalloc) against topk_ragged
with a caller-owned workspace, through the C ABI.

topk_ragged_noalloc is topk_ragged for callers that cannot allocate device
memory: where a launch needs a workspace it uses the library's static
per-device scratch array instead.  Each case makes two calls in a row on the
same scratch, the second with a smaller input, and both must equal what
topk_ragged returns for the same input, bit for bit (integer output).  A
launch whose workspace would exceed the scratch must be refused before
anything runs.
"""

from __future__ import annotations


import numpy as np
import pytest

import row_radix_top_amd as rrt
from oracle import topk_ragged_oracle
from row_radix_top_amd import binding, workloads
from tests.gpu_util import assert_same, note, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _abi_noalloc(s, L, K, next_n, out):
    import torch
    lib = binding.load()
    sp = int(torch.cuda.current_stream(s.device).cuda_stream)
    return lib.topk_ragged_noalloc(s.data_ptr(), s.stride(0), L.data_ptr(), s.shape[0], next_n, K, out.data_ptr(),
                                   sp)


def _with_workspace(s, L, K, next_n):
    import torch
    ws = rrt.new_workspace(rrt.workspace_size(s.shape[0], s.stride(0), K, device=s.device), s.device)
    out = rrt.topk_ragged(s, L, K, workspace=ws, next_n=next_n)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (0 if ws is None else ws.numel())


def _case(scores_np, lengths_np, K, next_n, tag):
    import torch
    dev = torch.device("cuda:0")
    s = torch.from_numpy(scores_np).to(dev)
    L = torch.from_numpy(np.ascontiguousarray(lengths_np, dtype=np.int32)).to(dev)
    exp, ws_bytes = _with_workspace(s, L, K, next_n)
    note(f"noalloc {tag}: rows={s.shape[0]} stride={s.stride(0)} K={K} workspace={ws_bytes} "
         f"plan={rrt.query_plan(s, K)}")
    out = torch.full((s.shape[0], K), -7, dtype=torch.int32, device=dev)
    rc = _abi_noalloc(s, L, K, next_n, out)
    assert rc == 0, f"{tag}: topk_ragged_noalloc returned {rc}: {binding.last_error()}"
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert_same(got, exp, f"noalloc {tag} vs topk_ragged")
    return got


# (workload for the first call, the second call's smaller input)
CASES = [
    # Long rows on the multi-workgroup path: a block per row in the scratch.
    ("long_k2048", dict(rows=5, stride=131072, n_lo=65536, n_hi=131072, K=2048)),
    ("long_k1024", dict(rows=3, stride=98304, n_lo=40000, n_hi=98304, K=1024)),
    # One workgroup per row with more rows than workgroups: the ticket counter.
    ("prefill", dict(rows=1500, stride=65536, n_lo=1, n_hi=65536, K=2048)),
    # No workspace at all.
    ("decode", dict(rows=7, stride=32768, n_lo=0, n_hi=32768, K=2048)),
]


@pytest.mark.parametrize("name,small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_topk_ragged_twice(name, small):
    w = workloads.make_workload(name)
    first = _case(w.scores, w.flat_lengths, w.K, w.next_n, f"{name} (first call)")
    rows = [0, w.num_rows // 2, w.num_rows - 1]
    assert_same(first[rows], topk_ragged_oracle(w.scores[rows], w.flat_lengths[rows], w.K), f"noalloc {name} oracle")
    rng = np.random.default_rng(700 + len(name))
    n = rng.integers(small["n_lo"], small["n_hi"] + 1, size=small["rows"]).astype(np.int32)
    s_np, L = workloads.random_rows(701 + len(name), small["rows"], small["stride"], n, dist="normal")
    second = _case(s_np, L, small["K"], 1, f"{name} (second, smaller call)")
    assert_same(second, topk_ragged_oracle(s_np, L, small["K"]), f"noalloc {name} second call vs oracle")


def test_noalloc_refuses_more_than_its_scratch():
    import torch
    dev = torch.device("cuda:0")
    limit = binding.NOALLOC_SCRATCH_BYTES
    # The first of a few long-row shapes whose workspace exceeds the scratch
    # (the large-K layout has the larger per-workgroup lists).
    shape = None
    for K in (2048, 4096):
        for rows in (16, 32, 64, 96, 128):
            for stride in (131072, 262144, 1 << 20):
                need = rrt.workspace_size(rows, stride, K, device=dev)
                if need > limit and shape is None:
                    shape = (rows, stride, K, need)
    assert shape is not None, "no shape needs more workspace than the scratch holds"
    rows, stride, K, need = shape
    note(f"noalloc refusal: rows={rows} stride={stride} K={K} needs {need} > {limit}")
    s = torch.zeros((rows, stride), dtype=torch.float32, device=dev)
    L = torch.full((rows,), stride, dtype=torch.int32, device=dev)
    out = torch.full((rows, K), -7, dtype=torch.int32, device=dev)
    rc = _abi_noalloc(s, L, K, 1, out)
    assert rc == -3, f"expected TOPK_EWORKSPACE, got {rc}"
    assert "scratch" in binding.last_error()
    torch.cuda.synchronize()
    assert bool((out == -7).all().item()), "a refused call must launch nothing"
    # The scratch still works afterwards.
    w = workloads.make_workload("long_k2048")
    _case(w.scores, w.flat_lengths, w.K, w.next_n, "long_k2048 after a refusal")
