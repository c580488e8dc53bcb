"""Pins of the CPU oracle against things other than itself (no GPU).

* hand-worked examples (tests/golden/hand_examples.json);
* an O(n^2) rank count of the rule on tiny rows, random and exhaustive;
* numpy's stable argsort on rows of every workload;
* closed forms (K >= n, empty, constant, increasing, decreasing rows);
* the value multiset against numpy.partition;
* invariants on every output row;
* argument handling (clamped lengths, next_n, NaN rejection).

A plausible slip in the oracle -- ">=" for ">" in the order, the tie going to
the higher index, unsorted output, a missing -1 pad, reading past the length,
an off-by-one in nth_element -- fails at least one of these.
"""

from __future__ import annotations

import itertools
import json
import os

import numpy as np
import pytest

from oracle import topk_ragged_oracle
from row_radix_top_amd import workloads
from tests.pins import argsort_row, bruteforce_row, check_invariants

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _row_from_strings(vals):
    return np.array([float(v) for v in vals], dtype=np.float32)


def test_hand_examples():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 10
    for c in cases:
        row = _row_from_strings(c["row"])
        got = topk_ragged_oracle(row[None, :], np.array([c["n"]], np.int32), c["K"])
        assert got[0].tolist() == c["expected"], c
        # The brute-force rank count agrees with the hand result too.
        assert bruteforce_row(row, c["n"], c["K"]) == c["expected"], c


def test_bruteforce_random_tiny():
    rng = np.random.default_rng(7)
    for trial in range(400):
        n_alloc = int(rng.integers(1, 65))
        alphabet = [np.float32(v) for v in (-1.5, -0.0, 0.0, 0.5, 2.0)][: int(rng.integers(2, 6))]
        row = np.array(rng.choice(alphabet, size=n_alloc), dtype=np.float32)
        n = int(rng.integers(0, n_alloc + 1))
        K = int(rng.integers(1, n_alloc + 3))
        got = topk_ragged_oracle(row[None, :], np.array([n], np.int32), K)[0]
        assert got.tolist() == bruteforce_row(row, n, K), (row, n, K)


def test_bruteforce_exhaustive_three_letters():
    # Every sequence over {a < b < c} up to length 7, every K in [1, n+2].
    # Letter b is split between -0.0 and +0.0 to exercise signed zeros.
    letters = [np.float32(-1.0), np.float32(0.0), np.float32(1.0)]
    count = 0
    for n in range(0, 8):
        for seq in itertools.product(range(3), repeat=n):
            row = np.array([letters[s] for s in seq] + [np.float32(9.0)], dtype=np.float32)
            for i, s in enumerate(seq):
                if s == 1 and i % 2 == 1:
                    row[i] = np.float32(-0.0)
            batch = []
            for K in range(1, n + 3):
                batch.append((K, bruteforce_row(row, n, K)))
            for K, exp in batch:
                got = topk_ragged_oracle(row[None, :], np.array([n], np.int32), K)[0]
                assert got.tolist() == exp, (row, n, K)
                count += 1
    assert count > 10000


@pytest.mark.parametrize("name", ["small", "decode", "mtp", "long_k1024", "long_k2048"])
def test_argsort_and_invariants_on_workloads(name):
    w = workloads.make_workload(name)
    out = topk_ragged_oracle(w.scores, w.lengths, w.K)
    flat = w.flat_lengths
    for r in range(w.num_rows):
        n = int(flat[r])
        exp = argsort_row(w.scores[r], n, w.K)
        assert np.array_equal(out[r], exp), (name, r)
        check_invariants(w.scores[r], n, w.K, out[r])


def test_argsort_prefill_sample():
    # The full prefill workload is 1 GiB; a row sample keeps the CPU suite short.
    w = workloads.make_workload("prefill")
    rows = np.array([0, 1, 2, 777, 2048, 3333, 4094, 4095])
    out = topk_ragged_oracle(w.scores[rows], w.flat_lengths[rows], w.K)
    for i, r in enumerate(rows):
        n = int(w.flat_lengths[r])
        assert n == 61440 + r
        assert np.array_equal(out[i], argsort_row(w.scores[r], n, w.K))
        check_invariants(w.scores[r], n, w.K, out[i])


def test_decode_has_short_rows():
    w = workloads.make_workload("decode")
    assert (w.flat_lengths < w.K).any()
    out = topk_ragged_oracle(w.scores, w.lengths, w.K)
    for r in np.nonzero(w.flat_lengths < w.K)[0]:
        n = int(w.flat_lengths[r])
        assert out[r, :n].tolist() == list(range(n))
        assert np.all(out[r, n:] == -1)


def test_value_multiset_matches_partition():
    w = workloads.make_workload("long_k2048")
    out = topk_ragged_oracle(w.scores, w.lengths, w.K)
    for r in range(w.num_rows):
        n = int(w.flat_lengths[r])
        x = w.scores[r, :n]
        top = np.sort(np.partition(x, n - w.K)[n - w.K:])
        assert np.array_equal(np.sort(x[out[r]]), top)


def test_closed_forms():
    K = 16
    stride = 200
    # K >= n: 0..n-1 then -1.
    s, L = workloads.random_rows(1, 3, stride, [5, 16, 0])
    out = topk_ragged_oracle(s, L, K)
    assert out[0].tolist() == list(range(5)) + [-1] * 11
    assert out[1].tolist() == list(range(16))
    assert out[2].tolist() == [-1] * 16
    # Constant row: the first K positions.
    s, L = workloads.random_rows(2, 2, stride, [stride, 100], dist="const")
    out = topk_ragged_oracle(s, L, K)
    assert out[0].tolist() == list(range(K)) and out[1].tolist() == list(range(K))
    # Strictly increasing row: the last K positions of the prefix.
    s, L = workloads.random_rows(3, 2, stride, [stride, 77], dist="inc")
    out = topk_ragged_oracle(s, L, K)
    assert out[0].tolist() == list(range(stride - K, stride))
    assert out[1].tolist() == list(range(77 - K, 77))
    # Strictly decreasing row: the first K positions.
    s, L = workloads.random_rows(4, 1, stride, [stride], dist="dec")
    out = topk_ragged_oracle(s, L, K)
    assert out[0].tolist() == list(range(K))


def test_special_values_rows():
    for dist in ("signed_zero", "denorm", "inf", "levels"):
        s, L = workloads.random_rows(11, 6, 300, [300, 299, 150, 33, 1, 0], dist=dist, levels=5)
        for K in (1, 7, 32, 64, 299, 300, 301):
            out = topk_ragged_oracle(s, L, K)
            for r in range(6):
                assert np.array_equal(out[r], argsort_row(s[r], int(L[r]), K)), (dist, K, r)
                check_invariants(s[r], int(L[r]), K, out[r])
        # Brute force on the short rows.
        for r in (3, 4, 5):
            for K in (1, 5, 40):
                got = topk_ragged_oracle(s[r:r + 1], L[r:r + 1], K)[0]
                assert got.tolist() == bruteforce_row(s[r], int(L[r]), K)


def test_lengths_are_clamped():
    s, _ = workloads.random_rows(5, 3, 50, [50, 50, 50])
    L = np.array([-7, 50, 999], dtype=np.int32)
    out = topk_ragged_oracle(s, L, 8)
    assert out[0].tolist() == [-1] * 8
    assert np.array_equal(out[1], argsort_row(s[1], 50, 8))
    assert np.array_equal(out[2], argsort_row(s[2], 50, 8))


def test_next_n_groups_rows_without_changing_selection():
    w = workloads.make_workload("mtp")
    a = topk_ragged_oracle(w.scores, w.lengths, w.K)  # 2-D lengths -> next_n = 2
    b = topk_ragged_oracle(w.scores, w.flat_lengths, w.K, next_n=1)
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        topk_ragged_oracle(w.scores[:3], w.flat_lengths[:3], w.K, next_n=2)


def test_nan_in_valid_prefix_is_rejected():
    row = np.array([[1.0, np.nan, 2.0, 3.0]], dtype=np.float32)
    with pytest.raises(ValueError):
        topk_ragged_oracle(row, np.array([3], np.int32), 2)
    # A NaN past the length is fine.
    out = topk_ragged_oracle(row, np.array([1], np.int32), 2)
    assert out[0].tolist() == [0, -1]


def test_thread_count_does_not_change_result():
    w = workloads.make_workload("mtp")
    a = topk_ragged_oracle(w.scores, w.lengths, w.K, threads=1)
    b = topk_ragged_oracle(w.scores, w.lengths, w.K, threads=7)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Row offsets (the reading of the pages' "RaggedTransform")
# ---------------------------------------------------------------------------

def test_offsets_index_a_flat_ragged_layout():
    """Lay the rows' valid prefixes end to end and give each row its start:
    the shifted indices must address that flat array, fall inside the row's
    own stretch in ascending order, and gather exactly the row's best values
    (checked against numpy's stable argsort of the row, not the oracle)."""
    from oracle import topk_ragged_offsets_oracle
    rng = np.random.default_rng(7)
    rows, stride = 40, 3000
    lens = rng.integers(0, stride + 1, size=rows).astype(np.int32)
    lens[:3] = [0, 1, 5]
    s = rng.integers(-20, 20, size=(rows, stride)).astype(np.float32)  # plenty of ties
    flat = np.concatenate([s[r, :lens[r]] for r in range(rows)])
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    for K in (1, 7, 64, 3000):
        out = topk_ragged_offsets_oracle(s, lens, K, starts)
        for r in range(rows):
            n = int(lens[r])
            m = min(K, n)
            assert np.all(out[r, m:] == -1)
            pos = out[r, :m]
            assert np.all(pos >= starts[r]) and np.all(pos < starts[r] + n)
            assert np.all(np.diff(pos) > 0)
            exp = argsort_row(s[r], n, K)[:m] + starts[r]
            assert np.array_equal(pos, exp), (K, r)
            assert np.array_equal(np.sort(flat[pos]), np.sort(s[r, exp - starts[r]]))


def test_offsets_zero_and_range():
    from oracle import topk_ragged_offsets_oracle
    s, L = workloads.random_rows(8, 6, 500, [0, 1, 499, 500, 250, 17], dist="normal")
    base = topk_ragged_oracle(s, L, 32)
    assert np.array_equal(topk_ragged_offsets_oracle(s, L, 32, np.zeros(6, np.int32)), base)
    big = np.full(6, 2**31 - 500, dtype=np.int64)
    out = topk_ragged_offsets_oracle(s, L, 32, big)
    assert np.array_equal(out, np.where(base >= 0, base + big[:, None], -1))
    with pytest.raises(ValueError):
        topk_ragged_offsets_oracle(s, L, 32, np.full(6, 2**31 - 10, dtype=np.int64))
    with pytest.raises(ValueError):
        topk_ragged_offsets_oracle(s, L, 32, np.full(6, -1, dtype=np.int64))


def test_values_are_the_best_scores_bit_for_bit():
    """The values output: each row's chosen scores, in index order, are its
    min(K, n) largest (numpy's sort of the prefix, not the oracle), the bits
    are the input's (a chosen -0.0 stays -0.0), the padding is -inf."""
    from oracle import topk_ragged_values_oracle
    rng = np.random.default_rng(11)
    rows, stride = 30, 700
    lens = rng.integers(0, stride + 1, size=rows).astype(np.int32)
    s = rng.standard_normal((rows, stride)).astype(np.float32)
    s[0, :5] = [-0.0, 0.0, -0.0, -1.0, -2.0]
    lens[0] = 5
    for K in (1, 3, 50, 700):
        idx, vals = topk_ragged_values_oracle(s, lens, K)
        for r in range(rows):
            n = int(lens[r])
            m = min(K, n)
            assert np.all(np.isneginf(vals[r, m:]))
            assert np.array_equal(vals[r, :m].view(np.uint32), s[r, idx[r, :m]].view(np.uint32))
            assert np.array_equal(np.sort(vals[r, :m]), np.sort(np.sort(s[r, :n])[::-1][:m]))
    idx, vals = topk_ragged_values_oracle(s, lens, 3)
    assert list(idx[0]) == [0, 1, 2]
    assert list(vals[0].view(np.uint32)) == [0x80000000, 0, 0x80000000]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    idx2, vals2 = topk_ragged_values_oracle(s, lens, 50, starts)
    assert np.array_equal(vals2.view(np.uint32), topk_ragged_values_oracle(s, lens, 50)[1].view(np.uint32))


def test_strided_rows_match_dense_copies():
    """Rows with a column stride: the transposed layout must select exactly
    what the oracle selects on numpy's transposed copy, every other column of
    a wider matrix what it selects on the sliced copy, and a unit column
    stride what it selects on the plain rows."""
    from oracle import topk_ragged_strided_oracle
    rng = np.random.default_rng(21)
    N, R = 900, 12
    base = rng.integers(-30, 30, size=(N, R)).astype(np.float32)   # columns become rows
    lens = rng.integers(0, N + 1, size=R).astype(np.int32)
    for K in (1, 40, 900):
        got = topk_ragged_strided_oracle(base, 1, R, N, R, lens, K)
        assert np.array_equal(got, topk_ragged_oracle(np.ascontiguousarray(base.T), lens, K))
        for r in range(R):
            check_invariants(np.ascontiguousarray(base.T)[r], lens[r], K, got[r])
    wide = rng.standard_normal((R, 2 * N + 3)).astype(np.float32)
    got = topk_ragged_strided_oracle(wide, 2 * N + 3, 2, N, R, lens, 64)
    assert np.array_equal(got, topk_ragged_oracle(np.ascontiguousarray(wide[:, :2 * N:2]), lens, 64))
    got = topk_ragged_strided_oracle(wide, 2 * N + 3, 1, 2 * N + 3, R, lens, 64)
    assert np.array_equal(got, topk_ragged_oracle(wide, lens, 64))


def test_bf16_widening_matches_torch():
    """The oracle widens bf16 by shifting its bits; torch's own bf16 -> fp32
    conversion must agree on every one of the 65536 bit patterns (NaNs
    compared by NaN-ness), and the selection on a bf16 tensor converted by
    torch must equal the oracle's."""
    import torch
    from oracle import topk_ragged_bf16_oracle, widen_bf16
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = widen_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((20, 3000)).astype(np.float32)).to(torch.bfloat16)
    b = x.view(torch.int16).numpy().view(np.uint16)
    lens = rng.integers(0, 3001, size=20).astype(np.int32)
    for K in (1, 100, 3000):
        assert np.array_equal(topk_ragged_bf16_oracle(b, lens, K), topk_ragged_oracle(x.float().numpy(), lens, K))
