"""The per-XCD chunk table of the streaming kernels: the sort takes the active
experts in rank order (descending pair count) and gives each to the XCD
with the fewest chunks so far (lowest index on ties), listing each XCD's
chunks expert by expert.  The host
sizes the table and the grid with ceil(max_chunks / 8) + ceil(T / 64) slots
per XCD, max_chunks = min(E, P) + P // 64; this checks that no XCD's list
ever needs more, over random routings and the extreme ones (every expert
equally loaded, one expert taking every token, k = E), and that the order
in which the kernels take a list's units (an expert's chunks interleaved
column tile by column tile) runs every chunk's every tile exactly once."""
import numpy as np
import pytest

XCDS, CHUNK = 8, 64


def slots_needed(counts, chunk_rows):
    m = np.sort([(c + chunk_rows - 1) // chunk_rows for c in counts if c > 0])[::-1]
    L = np.zeros(XCDS, int)
    for mr in m:
        L[int(np.argmin(L))] += mr          # argmin: the lowest index on ties
    return L


def test_greedy_lists_are_balanced_to_one_expert():
    # the point of the greedy order: no list exceeds the lightest one by more
    # than the largest expert's chunk count
    rng = np.random.default_rng(9)
    for _ in range(200):
        counts = rng.integers(0, 300, size=int(rng.integers(1, 512)))
        L = slots_needed(counts, CHUNK)
        m = [(c + CHUNK - 1) // CHUNK for c in counts if c > 0]
        assert L.max() - L.min() <= (max(m) if m else 0)


def bound(T, E, k):
    P = T * k
    max_chunks = min(E, P) + P // CHUNK
    return -(-max_chunks // XCDS) + -(-min(T, P) // CHUNK)


def routing_counts(rng, T, E, k, skew):
    logits = rng.standard_normal((T, E)) + skew * np.log1p(np.arange(E))[::-1]
    ids = np.argsort(-logits, axis=1)[:, :k]
    return np.bincount(ids.ravel(), minlength=E)


@pytest.mark.parametrize("chunk_rows", [64, 128])
def test_random_routings_fit_the_slot_bound(chunk_rows):
    rng = np.random.default_rng(5)
    for _ in range(300):
        E = int(rng.choice([1, 2, 4, 8, 16, 64, 128, 300, 512]))
        k = int(rng.integers(1, min(E, 32) + 1))
        T = int(rng.choice([1, 7, 64, 65, 200, 512, 4096, 8192]))
        counts = routing_counts(rng, T, E, k, float(rng.choice([0.0, 1.0, 4.0])))
        assert counts.sum() == T * k
        L = slots_needed(counts, chunk_rows)
        assert L.max() <= bound(T, E, k), (T, E, k)
        # the lists hold every chunk once
        assert L.sum() == sum((c + chunk_rows - 1) // chunk_rows for c in counts)


@pytest.mark.parametrize("T,E,k", [(8192, 8, 8), (8192, 16, 8), (4096, 32, 32), (513, 512, 32), (1, 512, 32),
                                   (64, 64, 1), (8191, 9, 8)])
def test_extreme_routings_fit_the_slot_bound(T, E, k):
    # every expert equally loaded, and the hottest possible experts (all T
    # tokens on the first k experts) next to a long tail of single pairs
    even = np.full(E, T * k // E)
    even[: T * k - even.sum()] += 1
    hot = np.zeros(E, int)
    hot[:k] = T
    # k - 1 experts on every token, each token's last pick spread one pair
    # per expert over the rest, the leftover on the first of them
    tail = hot.copy()
    if E > k:
        tail[k - 1] = 0
        n = min(T, E - k + 1)
        tail[k - 1:k - 1 + n] += 1
        tail[k - 1] += T - n
    for counts in (even, hot, tail):
        assert counts.sum() == T * k and counts.max() <= T
        assert slots_needed(counts, CHUNK).max() <= bound(T, E, k), (T, E, k)


def unit_of(u, nt_per, group_pos, group_m):
    """Work unit u of one XCD's list -> (slot, column tile), as the kernels
    map it: slot q = u // nt_per carries its chunk's index among its
    expert's chunks (pos) and their number (m); an expert's m chunks run
    column tile by column tile."""
    q = u // nt_per
    pos, m = group_pos[q], group_m[q]
    if m == 1:
        return q, u - q * nt_per
    v = u - (q - pos) * nt_per
    nt = v // m
    return q - pos + v % m, nt


@pytest.mark.parametrize("nt_per", [1, 12, 16, 24])
def test_unit_order_covers_every_chunk_and_tile_once(nt_per):
    # every (slot, column tile) of a list is one unit, and the m chunks of an
    # expert take adjacent units for each column tile
    rng = np.random.default_rng(nt_per)
    for _ in range(50):
        ms = [int(x) for x in rng.choice([1, 1, 1, 2, 3, 5], size=int(rng.integers(1, 12)))]
        pos = [p for m in ms for p in range(m)]
        gm = [m for m in ms for _ in range(m)]
        n = len(pos)
        seen = [unit_of(u, nt_per, pos, gm) for u in range(n * nt_per)]
        assert sorted(seen) == [(q, t) for q in range(n) for t in range(nt_per)]
        first = 0
        for m in ms:
            units = seen[first * nt_per:(first + m) * nt_per]
            for t in range(nt_per):
                assert units[t * m:(t + 1) * m] == [(first + c, t) for c in range(m)]
            first += m


def rounds_placement(mv):
    """The sort's placement of ranked experts (chunk counts mv, non-increasing)
    by one 64-lane wave: per round, the XCDs at the lowest load take one
    expert each from the current run of equal counts, in index order, or,
    when all eight are at the lowest load, whole levels of the run at once.
    Returns (XCD, first slot) per rank."""
    load, asg = [0] * XCDS, [None] * len(mv)
    for r0 in range(0, len(mv), 64):
        blk = mv[r0:r0 + 64]
        pos = 0
        while pos < len(blk):
            m = blk[pos]
            nrun = sum(1 for v in blk[pos:] if v == m)
            lo = min(load)
            takers = [x for x in range(XCDS) if load[x] == lo]
            if len(takers) == XCDS and nrun >= XCDS:
                lv = nrun // XCDS
                for p in range(lv * XCDS):
                    asg[r0 + pos + p] = (p % XCDS, lo + (p // XCDS) * m)
                load = [v + lv * m for v in load]
                pos += lv * XCDS
                continue
            cnt = min(len(takers), nrun)
            for b, x in enumerate(takers[:cnt]):
                asg[r0 + pos + b] = (x, load[x])
                load[x] += m
            pos += cnt
    return asg


def test_round_placement_is_sequential_greedy():
    # each expert, in rank order, to the XCD with the fewest chunks so far
    # (lowest index on ties), at that XCD's current load as its first slot
    rng = np.random.default_rng(21)
    for _ in range(2000):
        n = int(rng.integers(1, 400))
        mv = sorted((int(v) for v in rng.choice([1, 1, 1, 1, 2, 2, 3, 5, 8, 17], size=n)), reverse=True)
        load, want = [0] * XCDS, []
        for m in mv:
            x = int(np.argmin(load))
            want.append((x, load[x]))
            load[x] += m
        assert rounds_placement(mv) == want
