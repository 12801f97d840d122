"""Host logic of the balanced block-sparse schedule (fa_sparse_schedule).

Checked against the mask by brute force: every tile row (column) is covered
by its items exactly once, in order, by runs of at most `seg` tiles; split
rows (columns) have the fewest segments, of lengths differing by at most
one, each with its own slot, the first one flagged; items are listed
longest first; causal schedules hold only tiles at or below the diagonal.
Also the validation of the balanced entry points, which returns before any
launch (no GPU needed).
"""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import exact_io_aware_09_amd._lib as _lib
from exact_io_aware_09_amd.attention import sparse_schedule

HEADER = Path(__file__).resolve().parents[1] / "include" / "fa.h"


def reach_lists(mask, causal):
    nb = mask.shape[0]
    rows = [[u for u in range(nb) if mask[r, u] and (not causal or u <= r)] for r in range(nb)]
    cols = [[u for u in range(nb) if mask[u, c] and (not causal or u >= c)] for c in range(nb)]
    return rows, cols


def check_direction(items, longs, lists, expect, seg, n_slots):
    nb = len(expect)
    counts = items[:, 2]
    assert all(counts[i] >= counts[i + 1] for i in range(len(counts) - 1)), "longest first"
    seen_slots = set()
    long_of = {int(t): (int(s0), int(ns)) for t, s0, ns, _ in longs}
    assert len(long_of) == len(longs)
    for t in range(nb):
        mine = [it for it in items if it[0] == t]
        T = len(expect[t])
        if T <= seg:
            assert len(mine) == 1 and mine[0][3] == -1 and t not in long_of
            it = mine[0]
            assert list(lists[it[1]:it[1] + it[2]]) == expect[t]
            continue
        s0, ns = long_of[t]
        assert ns == -(-T // seg) and len(mine) == ns
        by_slot = sorted(mine, key=lambda it: it[3] >> 1)
        assert [it[3] >> 1 for it in by_slot] == list(range(s0, s0 + ns))
        assert [it[3] & 1 for it in by_slot] == [1] + [0] * (ns - 1)
        lens = [int(it[2]) for it in by_slot]
        assert max(lens) - min(lens) <= 1 and max(lens) <= seg and sum(lens) == T
        got = []
        for it in by_slot:
            got += list(lists[it[1]:it[1] + it[2]])
        assert got == expect[t]
        seen_slots.update(range(s0, s0 + ns))
    assert seen_slots == set(range(n_slots))


def band_global(nb, w=1):
    i = np.arange(nb)
    m = (np.abs(i[:, None] - i[None, :]) <= w).astype(np.int32)
    m[0, :] = 1
    m[:, 0] = 1
    return m


MASKS = [
    ("band_global", lambda nb: band_global(nb)),
    ("random", lambda nb: (np.random.default_rng(nb).random((nb, nb)) < 0.4).astype(np.int32)),
    ("dense", lambda nb: np.ones((nb, nb), np.int32)),
    ("empty_rows", lambda nb: np.triu(np.ones((nb, nb), np.int32))),
    ("empty", lambda nb: np.zeros((nb, nb), np.int32)),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seg", [1, 2, 3, 8, 0])
@pytest.mark.parametrize("name,make", MASKS)
@pytest.mark.parametrize("N", [1, 300, 1000, 4096])
def test_schedule_covers_every_tile_once(N, name, make, seg, causal):
    nb = -(-N // 128)
    mask = make(nb)
    s = sparse_schedule(mask, N, causal, 2, 3, seg_tiles=seg)
    f = s.field
    assert f("MAGIC") == _lib.FA_SCHED_MAGIC_VALUE and f("HEADER_INTS") == _lib.FA_SCHED_HEADER
    assert f("NB") == nb and f("CAUSAL") == int(causal) and f("TOTAL") == s.host.size
    rows, cols = reach_lists(mask, causal)
    nnz = sum(len(r) for r in rows)
    assert f("NNZ") == nnz == sum(len(c) for c in cols)
    eff = f("SEG")
    if seg == 0:
        assert eff == min(nb, max(8, -(-2 * 3 * nnz // 1024)))
    else:
        assert eff == min(seg, nb)
    lists = s.lists()
    check_direction(s.rows(), s.long_rows(), lists, rows, eff, f("ROW_SLOTS"))
    check_direction(s.cols(), s.long_cols(), lists, cols, eff, f("COL_SLOTS"))
    # offsets keep the item sections 16-byte aligned for the device copy
    for off in ("OFF_ROWS", "OFF_COLS", "OFF_LONG_ROWS", "OFF_LONG_COLS", "OFF_LISTS"):
        assert f(off) % 4 == 0


def test_default_segment_splits_only_the_long_rows():
    # N = 65,536: a band of 3 tiles plus one global row and column, 8 heads
    nb = 512
    mask = band_global(nb)
    s = sparse_schedule(mask, nb * 128, False, 1, 8)
    seg = s.field("SEG")
    nnz = int(mask.sum())
    assert seg == max(8, -(-8 * nnz // 1024))
    assert s.field("N_LONG_ROWS") == 1 and s.field("N_LONG_COLS") == 1
    assert s.long_rows()[0][0] == 0 and s.long_cols()[0][0] == 0
    assert int(s.rows()[:, 2].max()) <= seg and int(s.cols()[:, 2].max()) <= seg
    # a dense mask is already balanced: nothing is split
    d = sparse_schedule(np.ones((nb, nb), np.int32), nb * 128, False, 1, 8)
    assert d.field("N_LONG_ROWS") == 0 and d.field("N_LONG_COLS") == 0


def test_header_constants_match_the_binding():
    text = HEADER.read_text()
    defs = dict(re.findall(r"#define FA_SCHED_(\w+)\s+(0x[0-9A-Fa-f]+|\d+)", text))
    for name, idx in _lib.FA_SCHED_FIELDS.items():
        assert int(defs[name], 0) == idx, name
    assert int(defs["HEADER"], 0) == _lib.FA_SCHED_HEADER
    assert int(defs["MAGIC_VALUE"], 0) == _lib.FA_SCHED_MAGIC_VALUE


def test_schedule_argument_errors():
    m = np.ones((2, 2), np.int32)
    need = ctypes.c_size_t(0)
    call = lambda *a: _lib.fa_sparse_schedule(*a)
    assert call(None, 200, 0, 1, 1, 0, None, 0, ctypes.addressof(need)) == _lib.FA_ERR_INVALID_ARG
    assert call(m.ctypes.data, 0, 0, 1, 1, 0, None, 0, ctypes.addressof(need)) == _lib.FA_ERR_INVALID_ARG
    assert call(m.ctypes.data, 200, 2, 1, 1, 0, None, 0, ctypes.addressof(need)) == _lib.FA_ERR_INVALID_ARG
    assert call(m.ctypes.data, 200, 0, 1, 1, -1, None, 0, ctypes.addressof(need)) == _lib.FA_ERR_INVALID_ARG
    assert call(m.ctypes.data, 200, 0, 1, 1, 0, None, 0, None) == _lib.FA_ERR_INVALID_ARG
    assert call(m.ctypes.data, 200, 0, 1, 1, 0, None, 0, ctypes.addressof(need)) == _lib.FA_OK
    assert need.value > _lib.FA_SCHED_HEADER
    small = np.zeros(need.value - 1, np.int32)
    assert call(m.ctypes.data, 200, 0, 1, 1, 0, small.ctypes.data, small.size,
                ctypes.addressof(need)) == _lib.FA_ERR_NO_WORKSPACE


def test_workspace_bytes():
    nb = 8
    s = sparse_schedule(band_global(nb), nb * 128, False, 2, 3, seg_tiles=2)
    B, H, N, d = 2, 3, nb * 128, 64
    rs, cs = s.field("ROW_SLOTS"), s.field("COL_SLOTS")
    assert rs > 0 and cs > 0
    a = lambda x: (x + 255) // 256 * 256
    tile = B * H * 128
    fwd = _lib.fa_sparse_workspace_bytes(s.host.ctypes.data, B, H, N, d, 0)
    assert fwd == a(rs * tile * d * 4) + a(rs * tile * 4)
    bwd = _lib.fa_sparse_workspace_bytes(s.host.ctypes.data, B, H, N, d, 1)
    base = _lib.fa_backward_workspace_bytes(B, H, N, d, _lib.FA_BF16)
    assert bwd == a(base) + a(rs * tile * d * 4) + 2 * a(cs * tile * d * 4)
    # wrong N (another tile count), bad d, broken header
    assert _lib.fa_sparse_workspace_bytes(s.host.ctypes.data, B, H, N + 128, d, 0) == 0
    assert _lib.fa_sparse_workspace_bytes(s.host.ctypes.data, B, H, N, 48, 0) == 0
    bad = s.host.copy()
    bad[0] ^= 1
    assert _lib.fa_sparse_workspace_bytes(bad.ctypes.data, B, H, N, d, 0) == 0
    # nothing split: the forward needs no workspace
    n = sparse_schedule(band_global(nb), nb * 128, False, 2, 3, seg_tiles=nb)
    assert _lib.fa_sparse_workspace_bytes(n.host.ctypes.data, B, H, N, d, 0) == 0


A = 1 << 20  # a 16-byte aligned fake device address; never dereferenced (validation fails first)


def test_balanced_entry_points_validate_before_launch():
    nb = 4
    N = nb * 128
    s = sparse_schedule(band_global(nb), N, False, 1, 1, seg_tiles=2)
    h = s.host.ctypes.data
    big = 1 << 40
    fwd = lambda sched, dev, ws, wsb, n=N, causal=0, d=64: _lib.fa_forward_sparse_balanced(
        A, A, A, A, A, sched, dev, ws, wsb, 1, 1, n, d, 0.125, causal, _lib.FA_BF16, None)
    bwd = lambda sched, dev, ws, wsb, n=N, causal=0: _lib.fa_backward_sparse_balanced(
        A, A, A, A, A, A, sched, dev, A, A, A, ws, wsb, 1, 1, n, 64, 0.125, causal,
        _lib.FA_BF16, None)
    for call in (fwd, bwd):
        assert call(None, A, A, big) == _lib.FA_ERR_INVALID_ARG           # no host copy
        assert call(h, None, A, big) == _lib.FA_ERR_INVALID_ARG           # no device copy
        assert call(h, A, A, big, n=N + 128) == _lib.FA_ERR_INVALID_ARG   # other tile count
        assert call(h, A, A, big, causal=1) == _lib.FA_ERR_INVALID_ARG    # other causal flag
        assert call(h, A + 4, A, big) == _lib.FA_ERR_MISALIGNED
        assert call(h, A, None, 0) == _lib.FA_ERR_NO_WORKSPACE
        assert call(h, A, A, 16) == _lib.FA_ERR_NO_WORKSPACE
        bad = s.host.copy()
        bad[_lib.FA_SCHED_FIELDS["OFF_LISTS"]] += 1                       # section off its boundary
        assert call(bad.ctypes.data, A, A, big) == _lib.FA_ERR_INVALID_ARG
    assert fwd(h, A, A, big, d=48) == _lib.FA_ERR_UNSUPPORTED
