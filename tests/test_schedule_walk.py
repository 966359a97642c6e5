"""CPU walk of the decode kernel's work partition (no GPU): the balanced schedule's tile shares,
the segment loop each worker runs, the partial slots it writes and the slots the merge reads back,
and the workgroup-id -> (worker, member) placement on the XCDs.

The HIP kernels compute these index maps on the device; here they are restated from the kernel
sources' rules and walked exhaustively on ragged batches (empty sequences included), checking that
every loop advances and ends, that every 32-token tile is computed exactly once, that no two
segments share a partial slot and that the merge finds exactly the slots that were written.  The
split itself is the exact sequence split of the feature request's "Directions under
investigation" (a context cut into parts merged by log-sum-exp)."""

import numpy as np
import pytest

TILE = 32


def tile_prefix(seq_lens):
    """tile_prefix[b] = tiles of sequences before b (tile_prefix_block)."""
    tiles = (np.asarray(seq_lens, dtype=np.int64) + TILE - 1) // TILE
    return np.concatenate([[0], np.cumsum(tiles)])


def last_seq_at_or_before(prefix, g, batch):
    """The kernel's binary search: the last b in [0, batch] with prefix[b] <= g."""
    lo, hi = 0, batch
    steps = 0
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if prefix[mid] <= g:
            lo = mid
        else:
            hi = mid - 1
        steps += 1
        assert steps <= 64, "binary search does not end"
    return lo


def walk_worker(u, workers, seq_lens):
    """Segments (b, t_begin, t_end, first tile, end tile, slot) of balanced worker u, following the
    kernel's loop; asserts that every pass advances."""
    batch = len(seq_lens)
    prefix = tile_prefix(seq_lens)
    total = int(prefix[batch])
    nw = min(workers, total)
    if u >= nw:
        return []
    g_next, g_end = u * total // nw, (u + 1) * total // nw
    segs = []
    while True:
        if g_next >= g_end:
            break
        b = last_seq_at_or_before(prefix, g_next, batch)
        assert b < batch, "a tile index past the batch"
        p0, p1 = int(prefix[b]), int(prefix[b + 1])
        seg_end = min(g_end, p1)
        assert seg_end > g_next, "the segment loop does not advance"
        t_begin = (g_next - p0) * TILE
        t_end = min(int(seq_lens[b]), (seg_end - p0) * TILE)
        assert 0 <= t_begin < t_end <= seq_lens[b], "empty or out-of-range segment"
        segs.append((b, t_begin, t_end, g_next, seg_end, b + u))
        g_next = seg_end
        assert len(segs) <= batch, "more segments than sequences"
    return segs


def merge_slots(b, workers, seq_lens):
    """The merge kernel's view: the contiguous slots b + worker_of(first tile) ..
    b + worker_of(last tile) of sequence b (none for an empty sequence)."""
    prefix = tile_prefix(seq_lens)
    total = int(prefix[-1])
    nw = min(workers, total)
    p0, p1 = int(prefix[b]), int(prefix[b + 1])
    if p1 <= p0:
        return []

    def worker_of(t):
        return ((t + 1) * nw - 1) // total

    return [b + w for w in range(worker_of(p0), worker_of(p1 - 1) + 1)]


def merge_skips(b, workers, seq_lens):
    """The merge's rule for rows the decode kernel finishes itself (prefill): the sequence's first
    and last tiles fall in the same worker's share."""
    prefix = tile_prefix(seq_lens)
    total = int(prefix[-1])
    nw = min(workers, total)
    p0, p1 = int(prefix[b]), int(prefix[b + 1])
    return p1 > p0 and ((p0 + 1) * nw - 1) // total == (p1 * nw - 1) // total


def check_partition(seq_lens, workers):
    batch = len(seq_lens)
    prefix = tile_prefix(seq_lens)
    total = int(prefix[-1])
    covered = np.zeros(total, dtype=np.int64)
    written = {}
    whole = set()  # sequences the decode kernel finishes: one segment from first to last tile
    for u in range(workers):
        for b, t0, t1, g0, g1, slot in walk_worker(u, workers, seq_lens):
            if g0 == prefix[b] and g1 == prefix[b + 1]:
                whole.add(b)
            covered[g0:g1] += 1
            assert slot not in written, "two segments write one partial slot"
            assert 0 <= slot < batch + workers, "slot outside the workspace"
            written[slot] = (b, t0, t1)
    assert np.all(covered == 1), "a tile computed twice or never"
    # token coverage per sequence: the segments of b tile [0, T_b) exactly
    for b in range(batch):
        spans = sorted((t0, t1) for slot, (bb, t0, t1) in written.items() if bb == b)
        pos = 0
        for t0, t1 in spans:
            assert t0 == pos
            pos = t1
        assert pos == seq_lens[b]
        # the merge reads exactly the slots the kernel wrote for b
        assert sorted(s for s, (bb, _, _) in written.items() if bb == b) == merge_slots(b, workers, seq_lens)
        # the kernel finishes b itself exactly when the merge skips it, and then b is one segment
        assert (b in whole) == merge_skips(b, workers, seq_lens)
        if b in whole:
            assert len(spans) == 1


RAGGED = [
    [1000, 0, 1, 4097, 33],
    [0, 0, 0, 5],
    [31, 32, 33, 64, 65, 0, 1],
    [0] * 7 + [70000],
    [5, 0, 40, 1, 0, 70],
]


@pytest.mark.parametrize("lens", RAGGED)
@pytest.mark.parametrize("workers", [1, 2, 3, 7, 64, 256, 1000])
def test_balanced_partition_covers_every_tile_once(lens, workers):
    check_partition(np.asarray(lens, dtype=np.int64), workers)


def test_balanced_partition_random_batches():
    rng = np.random.default_rng(2024)
    for _ in range(300):
        batch = int(rng.integers(1, 40))
        lens = rng.integers(0, 3000, size=batch)
        lens[rng.random(batch) < 0.3] = 0
        if lens.sum() == 0:
            lens[0] = 1
        check_partition(lens, int(rng.integers(1, 600)))


def test_all_empty_batch_has_no_work():
    # zero tiles: min(workers, 0) = 0 workers take part and the merge reads no slot
    lens = np.zeros(5, dtype=np.int64)
    for u in range(8):
        assert walk_worker(u, 8, lens) == []
    assert all(merge_slots(b, 8, lens) == [] for b in range(5))


def placement(L, xcds, members, units, prefill_blocks):
    """Workgroup id L -> (worker u, member): the decode kernel's XCD-aware map.  Consecutive ids
    go to the XCDs in turn; decode calls give the members of one unit ids `xcds` apart (same XCD,
    adjacent dispatch slots); prefill calls give each XCD a contiguous block of workers."""
    xcd, slot = L % xcds, L // xcds
    member = slot % members
    if prefill_blocks:
        u = xcd * ((units + xcds - 1) // xcds) + slot // members
    else:
        u = (slot // members) * xcds + xcd
    return u, member, xcd


@pytest.mark.parametrize("xcds", [1, 2, 4, 8])
@pytest.mark.parametrize("members", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("units", [1, 7, 8, 9, 100, 257])
@pytest.mark.parametrize("prefill_blocks", [False, True])
def test_workgroup_placement_is_a_bijection(xcds, members, units, prefill_blocks):
    blocks = (units + xcds - 1) // xcds * xcds * members
    seen = {}
    for L in range(blocks):
        u, member, xcd = placement(L, xcds, members, units, prefill_blocks)
        if u >= units:
            continue  # a padding workgroup returns at once
        assert (u, member) not in seen, "two workgroups take one (worker, member)"
        seen[(u, member)] = xcd
    assert len(seen) == units * members
    if not prefill_blocks:
        # every member of one unit runs on the same XCD (they share the unit's rows in its L2)
        for u in range(units):
            assert len({seen[(u, m)] for m in range(members)}) == 1
