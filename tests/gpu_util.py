"""Helpers for the GPU tests: run the HIP path through the C ABI on numpy
inputs and compare with the CPU oracle."""

from __future__ import annotations

import sys

import numpy as np

import row_radix_top_amd as rrt
from row_radix_top_amd import binding


def require_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    binding.load()
    return torch.device("cuda:0")


def note(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(scores: np.ndarray, lengths: np.ndarray, K: int, *, next_n=None, offset: int = 0,
            check_workspace: bool = True, tag: str = "", row_offsets=None, **overrides):
    """Copies inputs to the GPU, runs topk_ragged, returns (out, plan).

    offset > 0 places row 0 at element `offset` of the device buffer, so the
    scores pointer is only 4- or 8-byte aligned (narrower loads)."""
    import torch
    dev = torch.device("cuda:0")
    num_rows, stride = scores.shape
    flat = np.ascontiguousarray(scores.reshape(-1))
    buf = torch.empty(flat.size + offset + 4, dtype=torch.float32, device=dev)
    buf[offset:offset + flat.size].copy_(torch.from_numpy(flat))
    s = buf[offset:offset + flat.size].view(num_rows, stride)
    L = torch.from_numpy(np.ascontiguousarray(lengths, dtype=np.int32)).to(dev)
    plan = rrt.query_plan(s, K, **overrides)
    note(f"{tag} rows={num_rows} stride={stride} K={K} offset={offset} plan={plan}")
    nbytes = rrt.workspace_size(num_rows, stride, K, scores=s, **overrides)
    ws = rrt.new_workspace(nbytes, dev)
    ro = None
    if row_offsets is not None:
        ro = torch.from_numpy(np.ascontiguousarray(row_offsets, dtype=np.int32)).to(dev)
    out = rrt.topk_ragged(s, L, K, workspace=ws, next_n=next_n, row_offsets=ro, **overrides)
    torch.cuda.synchronize()
    if check_workspace and ws is not None:
        assert int(ws.count_nonzero().item()) == 0, "workspace must be all-zero after a launch"
        assert rrt.workspace_status(ws) == 0
    return out.cpu().numpy(), plan


def assert_same(got: np.ndarray, exp: np.ndarray, what: str = "") -> None:
    if not np.array_equal(got, exp):
        bad = np.nonzero((got != exp).any(axis=1))[0]
        r = int(bad[0])
        col = int(np.nonzero(got[r] != exp[r])[0][0])
        raise AssertionError(
            f"{what}: {bad.size} rows differ; first row {r} col {col}: got {got[r, col:col + 8]} "
            f"expected {exp[r, col:col + 8]}")
