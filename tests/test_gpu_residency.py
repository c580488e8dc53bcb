"""Residency and fallback on the GPU (PR #41189 page: cooperative waits
deadlock unless every workgroup of a row is resident; PR #54110 page: fall
back to one workgroup per row when a device cannot hold the cooperative
launch).

The planner is run as if the device kept only one or two workgroups per CU
(max_occupancy), so its headroom, group sizing and fallback decisions are
exercised on real hardware.  The device itself keeps more, so every launch
here is resident whatever the plan.  Bounded waits are checked by forcing a
one-poll spin limit from the host: the launch must still finish, report the
timeout in the workspace header, and a fresh workspace must give exact
results again."""

from __future__ import annotations

import numpy as np
import pytest

import row_radix_top_amd as rrt
from oracle import topk_ragged_oracle
from row_radix_top_amd import workloads
from tests.gpu_util import assert_same, note, require_gpu, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("occ", [1, 2])
@pytest.mark.parametrize("name", ["mtp", "long_k1024", "long_k2048"])
def test_emulated_low_occupancy(name, occ):
    w = workloads.make_workload(name)
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    for ov in ({}, dict(force_path=2), dict(force_path=2, force_wg_per_row=16), dict(force_path=1)):
        got, plan = run_gpu(w.scores, w.lengths, w.K, tag=f"{name} occ={occ} {ov}", max_occupancy=occ, **ov)
        assert plan["resident_cap"] <= 256 * occ
        if plan["path"] == rrt.PATH_MULTI:
            assert plan["grid"] <= plan["resident_cap"] - plan["headroom"]
            assert plan["headroom"] == (256 if occ > 1 else 1)
        elif ov.get("force_path") == 2:
            assert plan["fell_back"] == 1
        assert_same(got, exp, f"{name} occ={occ} {ov}")


def test_emulated_low_occupancy_many_rows():
    # Prefill at one workgroup per CU: 16 rows per workgroup through the ticket.
    w = workloads.make_workload("prefill")
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag="prefill occ=1", max_occupancy=1)
    assert plan["path"] == rrt.PATH_SINGLE and plan["grid"] <= 256
    assert_same(got, exp, "prefill occ=1")


def test_bounded_wait_times_out_and_recovers():
    import torch
    dev = torch.device("cuda:0")
    w = workloads.make_workload("long_k2048")
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    s = torch.from_numpy(w.scores).to(dev)
    L = torch.from_numpy(w.flat_lengths).to(dev)
    ov = dict(force_path=2, force_wg_per_row=16)
    plan = rrt.query_plan(s, w.K, **ov)
    assert plan["path"] == rrt.PATH_MULTI
    ws = rrt.new_workspace(rrt.workspace_size(w.num_rows, w.row_stride, w.K, scores=s, **ov), dev)
    note(f"bounded wait: spin_limit=1 plan={plan}")
    # Every wait's target is set one arrival beyond what can come, from the
    # host: each wait gives up after one poll, so the timeout is certain.
    rrt.topk_ragged(s, L, w.K, workspace=ws, spin_limit=1, force_wait_timeout=1, **ov)
    torch.cuda.synchronize()  # the launch ends although its waits gave up
    flags = rrt.workspace_status(ws)
    note(f"bounded wait: flags={flags}")
    assert flags & 1, "every cooperative wait was made to time out"
    assert flags & ~3 == 0
    # After an error the workspace is undefined: initialise it again.
    rrt.workspace_init(ws)
    out = rrt.topk_ragged(s, L, w.K, workspace=ws, **ov)
    torch.cuda.synchronize()
    assert rrt.workspace_status(ws) == 0
    assert int(ws.count_nonzero().item()) == 0
    assert_same(out.cpu().numpy(), exp, "after re-initialising the workspace")


@pytest.mark.parametrize("name", ["decode", "mtp", "long_k2048"])
def test_one_workgroup_grid(name):
    # The one-workgroup path never waits: a grid of one workgroup must take
    # every row in turn through the ticket counter.
    w = workloads.make_workload(name)
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=f"{name} grid=1", force_path=1, max_grid=1)
    assert plan["grid"] == 1
    assert_same(got, exp, f"{name} grid=1")
