"""The stream-K division of the decode (host-side mirror of its arithmetic,
no GPU): workgroup w of N takes global chunks [floor(w T / N), floor((w+1) T
/ N)), N = min(grid, T); a pair cut between ranges keeps part 0 in slot 2 w0
(+1 when the pair starts inside w0's range) and part k > 0 in slot 2 (w0 + k).
The kernel relies on: every chunk of every pair decoded exactly once, the
parts of a pair numbered 0..n-1 by consecutive workgroups, the owner of a
chunk found in closed form, and no two parts sharing a slot below 2 * grid."""

from __future__ import annotations

import random


def group_of(x: int, T: int, N: int) -> int:
    return min(((x + 1) * N - 1) // T, N - 1)


def partition(counts: list, grid: int):
    pre = [0]
    for c in counts:
        pre.append(pre[-1] + c)
    T = pre[-1]
    N = min(grid, T)
    lo_of = lambda w: w * T // N  # noqa: E731
    parts = {q: [] for q in range(len(counts))}
    slots = {}
    for wg in range(N):
        lo, hi = lo_of(wg), lo_of(wg + 1)
        assert lo < hi  # no empty range once N <= T
        q = 0
        z = len(counts) - 1
        while q < z:  # first pair ending past lo
            m = (q + z) // 2
            if pre[m + 1] > lo:
                z = m
            else:
                q = m + 1
        while q < len(counts) and pre[q] < hi:
            base, cnt = pre[q], counts[q]
            if cnt:
                w0 = group_of(base, T, N)
                nparts = group_of(base + cnt - 1, T, N) - w0 + 1
                slot0 = 2 * w0 + (0 if base == lo_of(w0) else 1)
                mine = slot0 if wg == w0 else 2 * wg
                k = wg - w0
                assert mine == (slot0 if k == 0 else 2 * (w0 + 1) + 2 * (k - 1))
                if nparts > 1:
                    assert mine not in slots and mine < 2 * grid
                    slots[mine] = (wg, q)
                parts[q].append((k, max(lo, base) - base, min(hi, base + cnt) - base, nparts))
            q += 1
    return T, N, parts


def test_group_of_inverts_the_ranges():
    for T in range(1, 60):
        for N in range(1, T + 1):
            for x in range(T):
                w = group_of(x, T, N)
                assert w * T // N <= x < (w + 1) * T // N


def test_every_chunk_once_parts_contiguous_slots_distinct():
    rng = random.Random(7)
    cases = 0
    for _ in range(4000):
        P = rng.randint(1, 40)
        counts = [rng.choice([0, 0, rng.randint(1, 5), rng.randint(1, 300)]) for _ in range(P)]
        if sum(counts) == 0:
            continue
        T, N, parts = partition(counts, rng.randint(1, 3 * P + 5))
        for q, cnt in enumerate(counts):
            segs = sorted(parts[q])
            if cnt == 0:
                assert not segs  # written by the separate zero pass
                continue
            assert [s[0] for s in segs] == list(range(len(segs)))
            assert all(s[3] == len(segs) for s in segs)
            assert segs[0][1] == 0 and segs[-1][2] == cnt
            assert all(a[2] == b[1] for a, b in zip(segs, segs[1:]))
        cases += 1
    assert cases > 3000


def test_one_long_pair_is_cut_into_many_parts():
    """The shape the batched merge exists for: one pair over almost the
    whole grid, more parts than the 128 the merge holds in LDS."""
    _, _, parts = partition([1500 * 1, 1], 256)
    assert len(parts[0]) > 128 and len(parts[1]) == 1
