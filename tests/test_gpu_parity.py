"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle,
element by element (int32 indices, padding included).  Bit-exact is the bar:
the output is integer and the selection rule makes it unique.
"""

from __future__ import annotations

import numpy as np
import pytest

import row_radix_top_amd as rrt
from oracle import topk_ragged_oracle
from row_radix_top_amd import workloads
from tests.gpu_util import assert_same, note, require_gpu, run_gpu
from tests.pins import check_invariants

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# ---------------------------------------------------------------------------
# Key transform: every fp32 bit pattern
# ---------------------------------------------------------------------------

def test_key_transform_exhaustive():
    """Walk all 2^32 patterns in IEEE value order (-NaNs, -inf .. -0, +0 ..
    +inf, +NaNs): keys must rise strictly, except -0 -> +0 which are equal."""
    import torch
    dev = torch.device("cuda:0")
    chunk = 1 << 27
    # Negative floats in increasing value: bits 0xFFFFFFFF down to 0x80000000.
    # Non-negative floats in increasing value: 0x00000000 up to 0x7FFFFFFF.
    prev_last = None
    for neg in (True, False):
        for c in range(0, 1 << 31, chunk):
            ar = torch.arange(c, c + chunk, dtype=torch.int64, device=dev)
            bits = (0xFFFFFFFF - ar) if neg else ar
            bits32 = (bits - (bits >= (1 << 31)).to(torch.int64) * (1 << 32)).to(torch.int32)
            keys = rrt.debug_keys(bits32).to(torch.int64) & 0xFFFFFFFF
            d = keys[1:] - keys[:-1]
            assert bool((d > 0).all()), f"keys not increasing near chunk {c} neg={neg}"
            if prev_last is not None:
                step = int(keys[0].item()) - prev_last
                if neg is False and c == 0:
                    assert step == 0, "-0.0 and +0.0 must share a key"
                else:
                    assert step > 0
            prev_last = int(keys[-1].item())
    # -0.0 and +0.0 -> 0x80000000; -inf -> 0x007FFFFF; +inf -> 0xFF800000.
    probe = torch.tensor([0x80000000 - (1 << 32), 0, 0xFF800000 - (1 << 32), 0x7F800000],
                         dtype=torch.int32, device=dev)
    k = (rrt.debug_keys(probe).to(torch.int64) & 0xFFFFFFFF).tolist()
    assert k == [0x80000000, 0x80000000, 0x007FFFFF, 0xFF800000]


# ---------------------------------------------------------------------------
# The five workloads (the long-row one at both K), full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["small", "decode", "mtp", "long_k1024", "long_k2048", "prefill"])
def test_workload_parity(name):
    w = workloads.make_workload(name)
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=name)
    assert_same(got, exp, name)
    if name in ("long_k1024", "long_k2048"):
        assert plan["path"] == rrt.PATH_MULTI and plan["wg_per_row"] >= 4, plan
    if name == "mtp":
        # Rows of at most 65536 elements stay on one workgroup each.
        assert plan["path"] == rrt.PATH_SINGLE and plan["idx16"] == 1, plan
    if name == "prefill":
        assert plan["path"] == rrt.PATH_SINGLE and plan["grid"] < w.num_rows, plan


@pytest.mark.parametrize("name", ["long_k1024", "long_k2048"])
def test_long_rows_one_workgroup_per_row(name):
    # The same long rows with the cooperative path switched off: 32-bit
    # candidate indices, streamed wave by wave.
    w = workloads.make_workload(name)
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=name + "/single", force_path=1)
    assert plan["path"] == rrt.PATH_SINGLE and plan["idx16"] == 0
    assert_same(got, exp, name + " single path")


@pytest.mark.parametrize("G", [0, 2, 4])
def test_mtp_rows_shared_by_workgroups(G):
    # The multi-token rows with the cooperative path forced on.
    w = workloads.make_workload("mtp")
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    ov = dict(force_path=2, force_wg_per_row=G) if G else dict(force_path=2)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=f"mtp/multi G={G}", **ov)
    assert plan["path"] == rrt.PATH_MULTI
    assert_same(got, exp, f"mtp multi G={G}")


@pytest.mark.parametrize("G", [1, 2, 3, 5, 16, 31, 64])
def test_long_rows_group_sizes(G):
    # 256-thread workgroups (up to 3 per CU on the cooperative path), so that
    # every G up to 64 per row can be resident for the 16 rows or not.
    w = workloads.make_workload("long_k2048")
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=f"long G={G}", force_path=2, force_wg_per_row=G,
                        force_block=256)
    if plan["path"] == rrt.PATH_MULTI:
        assert plan["wg_per_row"] == G
    else:
        # Not co-resident on this device: the planner must have fallen back.
        assert plan["fell_back"] == 1 and 16 * G > plan["resident_cap"] - plan["headroom"]
    assert_same(got, exp, f"G={G}")


@pytest.mark.parametrize("grid", [1, 3, 64, 200])
def test_persistent_grid_caps(grid):
    w = workloads.make_workload("decode")
    exp = topk_ragged_oracle(w.scores, w.lengths, w.K)
    got, plan = run_gpu(w.scores, w.lengths, w.K, tag=f"decode grid={grid}", max_grid=grid)
    assert plan["grid"] == min(grid, w.num_rows)
    assert_same(got, exp, f"grid={grid}")


def test_decode_short_rows_and_next_n():
    w = workloads.make_workload("mtp")
    got2d, _ = run_gpu(w.scores, w.lengths, w.K, tag="mtp 2-D lengths")
    got1d, _ = run_gpu(w.scores, w.flat_lengths, w.K, next_n=1, tag="mtp 1-D lengths")
    assert np.array_equal(got2d, got1d)
    w = workloads.make_workload("decode")
    got, _ = run_gpu(w.scores, w.lengths, w.K, tag="decode invariants")
    for r in range(w.num_rows):
        check_invariants(w.scores[r], int(w.flat_lengths[r]), w.K, got[r])


# ---------------------------------------------------------------------------
# Edge rows: every length class, special values, both paths, narrow loads
# ---------------------------------------------------------------------------

EDGE_DISTS = ["normal", "levels", "const", "inc", "dec", "signed_zero", "denorm", "inf"]


@pytest.mark.parametrize("dist", EDGE_DISTS)
@pytest.mark.parametrize("K", [1, 7, 300, 1024, 2048])
def test_edge_rows_single_path(dist, K):
    stride = 9000
    lens = [0, 1, K - 1, K, K + 1, stride, 2047, 2048, 2049, 4097, 6143, 8191, 8999, -5, 99999]
    lens = [min(max(v, -5), 99999) for v in lens]
    s, L = workloads.random_rows(1000 + K, len(lens), stride, lens, dist=dist, levels=3)
    exp = topk_ragged_oracle(s, L, K)
    got, _ = run_gpu(s, L, K, tag=f"edge {dist} K={K}")
    assert_same(got, exp, f"{dist} K={K}")


@pytest.mark.parametrize("dist", EDGE_DISTS)
@pytest.mark.parametrize("K", [5, 2048])
def test_edge_rows_multi_path(dist, K):
    stride = 40000
    lens = [0, 1, K, K + 1, 2049, 8192, 8193, 16384 + 3, 39999, 40000]
    s, L = workloads.random_rows(2000 + K, len(lens), stride, lens, dist=dist, levels=4)
    exp = topk_ragged_oracle(s, L, K)
    for G in (2, 5):
        got, plan = run_gpu(s, L, K, tag=f"edge-multi {dist} K={K} G={G}", force_path=2,
                            force_wg_per_row=G)
        assert plan["path"] == rrt.PATH_MULTI
        assert_same(got, exp, f"multi {dist} K={K} G={G}")


@pytest.mark.parametrize("offset,stride", [(1, 5001), (2, 5002), (3, 5003), (0, 5003), (0, 5002)])
def test_narrow_loads(offset, stride):
    lens = [stride, stride - 1, 4099, 3000, 17]
    s, L = workloads.random_rows(77 + offset, len(lens), stride, lens, dist="levels", levels=50)
    for K in (16, 2048):
        exp = topk_ragged_oracle(s, L, K)
        got, plan = run_gpu(s, L, K, offset=offset, tag=f"narrow off={offset} stride={stride}")
        want_vec = 4 if (offset % 4 == 0 and stride % 4 == 0) else (2 if offset % 2 == 0 and stride % 2 == 0 else 1)
        assert plan["vec"] == want_vec
        assert_same(got, exp, f"offset={offset} stride={stride} K={K}")


def test_forced_vec_widths():
    s, L = workloads.random_rows(5, 6, 12000, [12000, 11999, 5000, 2048, 2049, 1], dist="normal")
    exp = topk_ragged_oracle(s, L, 777)
    for vec in (1, 2, 4):
        for path in (1, 2):
            got, plan = run_gpu(s, L, 777, tag=f"vec={vec} path={path}", force_vec=vec, force_path=path,
                                force_wg_per_row=3 if path == 2 else 0)
            assert plan["vec"] == vec
            assert_same(got, exp, f"vec={vec} path={path}")


def test_all_ties_long_rows():
    # Constant rows far longer than the candidate buffer: every element ties.
    s, L = workloads.random_rows(9, 4, 131072, [131072, 100000, 65537, 2049], dist="const")
    for K in (1, 2048):
        exp = topk_ragged_oracle(s, L, K)
        got, _ = run_gpu(s, L, K, tag=f"const auto K={K}")
        assert_same(got, exp, f"const K={K}")
        got, _ = run_gpu(s, L, K, tag=f"const single K={K}", force_path=1)
        assert_same(got, exp, f"const single K={K}")


def test_increasing_rows_refill_every_tile():
    # Every new tile beats the whole buffer: the worst case for compaction.
    s, L = workloads.random_rows(3, 3, 70000, [70000, 65536, 33333], dist="inc")
    exp = topk_ragged_oracle(s, L, 2048)
    for path in (1, 2):
        got, _ = run_gpu(s, L, 2048, tag=f"inc path={path}", force_path=path)
        assert_same(got, exp, f"inc path={path}")


def test_speculative_bound_fallback():
    """Rows whose first tiles hold their largest values: a bound taken from
    the first elements is above the K-th best of the row, so the row must be
    streamed again.  One workgroup walks all rows (grid capped at 1), so
    rows that need the second pass alternate with rows that do not."""
    rng = np.random.default_rng(41)
    stride = 65536
    rows = []
    for r in range(6):
        x = rng.standard_normal(stride, dtype=np.float32)
        if r % 2 == 0:
            x[4096 * (1 + r // 2):] -= np.float32(10.0)   # a cliff after the first tiles
        rows.append(x)
    rows.append(-np.arange(stride, dtype=np.float32))     # strictly decreasing
    rows.append(np.arange(stride, dtype=np.float32))      # strictly increasing
    s = np.ascontiguousarray(np.stack(rows))
    lens = np.array([stride, stride - 7, 40000, 33333, 20000, stride, stride, 9000], dtype=np.int32)
    for K in (129, 1000, 2048):
        exp = topk_ragged_oracle(s, lens, K)
        for grid in (1, 0):
            got, plan = run_gpu(s, lens, K, tag=f"spec-fallback K={K} grid={grid}", force_path=1,
                                max_grid=grid)
            assert plan["path"] == rrt.PATH_SINGLE
            assert_same(got, exp, f"spec fallback K={K} grid={grid}")


@pytest.mark.parametrize("offset", [0, 1, 2])
def test_wave_by_wave_rows(offset):
    """Rows long enough for each wavefront to stream its own quarter: quarter
    edges (n at and just past the speculation threshold, lengths that leave
    a short last quarter), a quarter holding all the large values (its part
    of the buffer overflows and the row is streamed again), ties, monotone
    rows, and load widths of 4, 2 and 1 elements."""
    rng = np.random.default_rng(61 + offset)
    stride = {0: 65536, 1: 65529, 2: 65530}[offset]   # load widths 4, 1, 2
    # Wave-by-wave rows start at 8192 elements (below 8704 only n = 8192,
    # where every quarter first holds the sample's two wave tiles); 8193 and
    # 8703 take the general path with a speculative bound.
    lens = [16384, 16385, 16383, 20479, 40000, stride - 1, 49153, 30001,
            8192, 8193, 8703, 8704, 8705, 10239, 12288, 9000]
    rows = []
    for i, n in enumerate(lens):
        kind = i % 4
        if kind == 0:
            x = rng.standard_normal(stride, dtype=np.float32)
        elif kind == 1:
            x = rng.standard_normal(stride, dtype=np.float32)
            x[3 * n // 4:] += np.float32(5.0)           # the last quarter holds the largest values
        elif kind == 2:
            x = rng.integers(0, 3, size=stride).astype(np.float32)   # heavy ties
        else:
            x = (np.arange(stride, dtype=np.float32) * np.float32(0.25))
            if i % 8 == 7:
                x = -x
        rows.append(x)
    s = np.ascontiguousarray(np.stack(rows))
    workloads.fill_tails(rng, s, np.array(lens))
    L = np.array(lens, dtype=np.int32)
    for K in (129, 700, 2048):
        exp = topk_ragged_oracle(s, L, K)
        for grid in (0, 1):
            got, plan = run_gpu(s, L, K, offset=offset, tag=f"waves off={offset} K={K} grid={grid}",
                                force_path=1, max_grid=grid)
            assert plan["path"] == rrt.PATH_SINGLE and plan["idx16"] == 1
            assert_same(got, exp, f"waves offset={offset} K={K} grid={grid}")


def test_many_rows_random_lengths():
    rng = np.random.default_rng(31)
    lens = rng.integers(0, 20000, size=700)
    s, L = workloads.random_rows(31, 700, 20000, lens, dist="normal")
    for K in (64, 513, 2048):
        exp = topk_ragged_oracle(s, L, K)
        got, _ = run_gpu(s, L, K, tag=f"700 rows K={K}")
        assert_same(got, exp, f"700 rows K={K}")


# ---------------------------------------------------------------------------
# Streaming-read reference (measurement kernel)
# ---------------------------------------------------------------------------

def _max_key_of_prefix(row: np.ndarray, n: int) -> int:
    if n <= 0:
        return 0
    u = row[:n].view(np.uint32).astype(np.uint64)
    u = np.where(u == 0x80000000, 0, u)
    k = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)
    return int(k.max())


@pytest.mark.parametrize("offset", [0, 1, 2])
def test_read_reference_reads_exactly_the_valid_prefix(offset):
    import torch
    # Tails hold random bit patterns (NaNs, infinities): reading past a
    # length would change the answer.
    w = workloads.make_workload("decode")
    lens = w.flat_lengths.copy()
    lens[:6] = [0, 1, 2047, 2048, 2049, 32768]
    dev = torch.device("cuda:0")
    flat = np.ascontiguousarray(w.scores.reshape(-1))
    buf = torch.empty(flat.size + offset + 4, dtype=torch.float32, device=dev)
    buf[offset:offset + flat.size].copy_(torch.from_numpy(flat))
    s = buf[offset:offset + flat.size].view(w.scores.shape)
    L = torch.from_numpy(lens).to(dev)
    got = rrt.read_reference(s, L).cpu().numpy().view(np.uint32)
    exp = [_max_key_of_prefix(w.scores[r], int(min(max(lens[r], 0), w.row_stride)))
           for r in range(w.num_rows)]
    assert got.tolist() == exp


# ---------------------------------------------------------------------------
# Errors reported by the launch path on the device
# ---------------------------------------------------------------------------

def test_missing_workspace_is_an_error():
    import torch
    dev = torch.device("cuda:0")
    s = torch.zeros(16, 131072, device=dev)
    L = torch.full((16,), 131072, dtype=torch.int32, device=dev)
    assert rrt.workspace_size(16, 131072, 2048, device=dev) > 0
    with pytest.raises(rrt.TopKError) as e:
        rrt.topk_ragged(s, L, 2048)
    assert e.value.code == -3 and "workspace" in str(e.value)
    assert rrt.workspace_size(4, 8192, 512, device=dev) == 0
    s = torch.zeros(4, 8192, device=dev)
    out = rrt.topk_ragged(s, torch.full((4,), 8192, dtype=torch.int32, device=dev), 512)
    torch.cuda.synchronize()
    assert out[0].tolist() == list(range(512))
    note("errors ok")


# ---------------------------------------------------------------------------
# Row offsets (topk_ragged_offsets): indices into a flat ragged layout
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["decode", "mtp", "long_k2048", "prefill"])
def test_row_offsets_flat_layout(name):
    from oracle import topk_ragged_offsets_oracle
    w = workloads.make_workload(name)
    n = np.clip(w.flat_lengths.astype(np.int64), 0, w.row_stride)
    starts = np.concatenate([[0], np.cumsum(n)[:-1]])
    assert starts[-1] + n[-1] <= 2**31 - 1
    exp = topk_ragged_offsets_oracle(w.scores, w.lengths, w.K, starts)
    paths = [{}, dict(force_path=1)]
    if name != "prefill":
        paths += [dict(force_path=2), dict(force_path=1, force_block=512)]
    for ov in paths:
        got, _ = run_gpu(w.scores, w.lengths, w.K, tag=f"{name} offsets {ov}", row_offsets=starts, **ov)
        assert_same(got, exp, f"{name} offsets {ov}")


def test_row_offsets_near_int32_limit():
    from oracle import topk_ragged_offsets_oracle
    rng = np.random.default_rng(77)
    lens = [0, 1, 100, 2048, 2049, 40000, 65536, 20000]
    s, L = workloads.random_rows(77, len(lens), 65536, lens, dist="levels", levels=300)
    offs = (2**31 - 1 - np.asarray(lens, dtype=np.int64)).clip(0, None) - rng.integers(0, 1000, len(lens))
    for K in (64, 2048):
        exp = topk_ragged_offsets_oracle(s, L, K, offs)
        for ov in ({}, dict(force_path=2), dict(force_path=1, max_grid=3)):
            got, _ = run_gpu(s, L, K, tag=f"offsets near 2^31 K={K} {ov}", row_offsets=offs, **ov)
            assert_same(got, exp, f"offsets near 2^31 K={K} {ov}")


# ---------------------------------------------------------------------------
# Values output (topk_ragged_values): exact score bits beside the indices
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["decode", "long_k1024", "prefill"])
def test_values_output(name):
    import torch
    from oracle import topk_ragged_values_oracle
    dev = torch.device("cuda:0")
    w = workloads.make_workload(name)
    if name == "decode":
        w.scores[1, :40] = np.float32(-0.0)   # chosen signed zeros keep their sign
        w.scores[1, 40:] = np.float32(-1.0)
    s = torch.from_numpy(w.scores).to(dev)
    L = torch.from_numpy(w.flat_lengths).to(dev)
    n = np.clip(w.flat_lengths.astype(np.int64), 0, w.row_stride)
    starts = np.concatenate([[0], np.cumsum(n)[:-1]])
    for offs in (None, starts):
        exp_i, exp_v = topk_ragged_values_oracle(w.scores, w.lengths, w.K, offs)
        ro = None if offs is None else torch.from_numpy(offs.astype(np.int32)).to(dev)
        ws = rrt.new_workspace(rrt.workspace_size(w.num_rows, w.row_stride, w.K, scores=s), dev)
        gi, gv = rrt.topk_ragged_values(s, L, w.K, workspace=ws, row_offsets=ro)
        torch.cuda.synchronize()
        assert_same(gi.cpu().numpy(), exp_i, f"{name} values idx offs={offs is not None}")
        assert np.array_equal(gv.cpu().numpy().view(np.uint32), exp_v.view(np.uint32)), name


# ---------------------------------------------------------------------------
# Column strides (topk_ragged_strided): rows packed into the workspace first
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["transposed", "every_other", "stride3"])
def test_strided_rows(layout):
    import torch
    from oracle import topk_ragged_strided_oracle, topk_ragged_values_oracle
    dev = torch.device("cuda:0")
    rng = np.random.default_rng({"transposed": 1, "every_other": 2, "stride3": 3}[layout])
    R, N = 48, 40000
    if layout == "transposed":
        flat = rng.standard_normal(N * R).astype(np.float32)
        rs, cs = 1, R
    elif layout == "every_other":
        rs, cs = 2 * N + 5, 2
        flat = rng.standard_normal(R * rs).astype(np.float32)
    else:
        rs, cs = 3 * N + 7, 3
        flat = rng.standard_normal(R * rs).astype(np.float32)
    lens = rng.integers(0, N + 1, size=R).astype(np.int32)
    lens[:6] = [0, 1, 2047, 2048, 2049, N]
    base = torch.from_numpy(flat).to(dev)
    view = torch.as_strided(base, (R, N), (rs, cs))
    L = torch.from_numpy(lens).to(dev)
    for K in (100, 2048):
        exp = topk_ragged_strided_oracle(flat, rs, cs, N, R, lens, K)
        nbytes = rrt.strided_workspace_size(R, N, K, device=dev)
        ws = rrt.new_workspace(nbytes, dev)
        got = rrt.topk_ragged_strided(view, L, K, workspace=ws)
        torch.cuda.synchronize()
        assert_same(got.cpu().numpy(), exp, f"{layout} K={K}")
        plan_bytes = rrt.workspace_size(R, N, K, device=dev)
        assert int(ws[:plan_bytes // ws.element_size()].count_nonzero().item()) == 0
        # With row offsets and values.
        dense = np.ascontiguousarray(view.cpu().numpy())
        starts = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]])
        ei, ev = topk_ragged_values_oracle(dense, lens, K, starts)
        vals = torch.empty((R, K), dtype=torch.float32, device=dev)
        gi, gv = rrt.topk_ragged_strided(view, L, K, workspace=ws, out_values=vals,
                                         row_offsets=torch.from_numpy(starts.astype(np.int32)).to(dev))
        torch.cuda.synchronize()
        assert_same(gi.cpu().numpy(), ei, f"{layout} K={K} offsets")
        assert np.array_equal(gv.cpu().numpy().view(np.uint32), ev.view(np.uint32))


# ---------------------------------------------------------------------------
# bf16 scores (topk_ragged_bf16): the same selection on the exact widening
# ---------------------------------------------------------------------------

def _to_bf16(scores: np.ndarray):
    import torch
    t = torch.from_numpy(scores).to(torch.bfloat16)   # round to nearest even
    return t, t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["small", "decode", "mtp", "long_k1024", "long_k2048", "prefill"])
def test_bf16_workloads(name):
    import torch
    from oracle import topk_ragged_bf16_oracle
    dev = torch.device("cuda:0")
    w = workloads.make_workload(name)
    tb, bits = _to_bf16(w.scores)
    # bf16 tails of random bits, as for fp32 (never read)
    rng = np.random.default_rng(9)
    for r, n in enumerate(np.clip(w.flat_lengths, 0, w.row_stride)):
        bits[r, n:] = rng.integers(0, 65536, size=w.row_stride - n, dtype=np.uint32).astype(np.uint16)
    exp = topk_ragged_bf16_oracle(bits, w.lengths, w.K)
    s = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    L = torch.from_numpy(w.flat_lengths).to(dev)
    paths = [{}, dict(force_path=1)]
    if name in ("mtp", "long_k2048"):
        paths.append(dict(force_path=2))
    for ov in paths:
        ws = rrt.new_workspace(rrt.workspace_size(w.num_rows, w.row_stride, w.K, device=dev, **ov), dev)
        got = rrt.topk_ragged_bf16(s, L, w.K, workspace=ws, next_n=w.next_n, **ov)
        torch.cuda.synchronize()
        assert_same(got.cpu().numpy(), exp, f"bf16 {name} {ov}")
        assert ws is None or int(ws.count_nonzero().item()) == 0


@pytest.mark.parametrize("offset", [0, 1])
def test_bf16_edges_values_offsets(offset):
    """Ties (bf16 keeps 8 bits of mantissa), signed zeros, lengths around K
    and the tiles, 16- and 2-byte loads (offset 1 misaligns every row),
    values and row offsets."""
    import torch
    from oracle import topk_ragged_bf16_oracle, topk_ragged_values_oracle, widen_bf16
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(13 + offset)
    stride = 40000 if offset == 0 else 40001
    lens = np.array([0, 1, 700, 2047, 2048, 2049, 16384, 16385, 30000, stride], dtype=np.int32)
    x = rng.standard_normal((len(lens), stride)).astype(np.float32)
    x[3] = np.where(rng.random(stride) < 0.5, -0.0, 0.0).astype(np.float32)
    x[8] = rng.integers(-3, 3, size=stride).astype(np.float32)
    _, bits = _to_bf16(x)
    flat = np.zeros(bits.size + offset, dtype=np.uint16)
    flat[offset:] = bits.reshape(-1)
    buf = torch.from_numpy(flat.view(np.int16)).to(dev).view(torch.bfloat16)
    s = buf[offset:].view(len(lens), stride)
    L = torch.from_numpy(lens).to(dev)
    n = np.clip(lens.astype(np.int64), 0, stride)
    starts = np.concatenate([[0], np.cumsum(n)[:-1]])
    ro = torch.from_numpy(starts.astype(np.int32)).to(dev)
    for K in (1, 129, 2048):
        exp = topk_ragged_bf16_oracle(bits, lens, K)
        ws = rrt.new_workspace(rrt.workspace_size(len(lens), stride, K, device=dev), dev)
        got = rrt.topk_ragged_bf16(s, L, K, workspace=ws)
        torch.cuda.synchronize()
        assert_same(got.cpu().numpy(), exp, f"bf16 edges offset={offset} K={K}")
        ei, ev = topk_ragged_values_oracle(widen_bf16(bits), lens, K, starts)
        vals = torch.empty((len(lens), K), dtype=torch.float32, device=dev)
        gi, gv = rrt.topk_ragged_bf16(s, L, K, workspace=ws, out_values=vals, row_offsets=ro)
        torch.cuda.synchronize()
        assert_same(gi.cpu().numpy(), ei, f"bf16 values offset={offset} K={K}")
        assert np.array_equal(gv.cpu().numpy().view(np.uint32), ev.view(np.uint32))
