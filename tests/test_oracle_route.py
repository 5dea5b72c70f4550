"""Pins of the oracle's routing and index build against brute force.

The routing groups token-expert pairs into contiguous per-expert ranges
(HPC-Ops x SGLang blog, section "MoE", routing & index build); the order
inside a range is fixed to ascending pair index, and dropped pairs (ids
outside [0, E)) follow all experts.  A plain comparison sort on the key
(expert id, or E for a dropped pair) with the pair index as tie breaker
must give the same permutation.
"""
import itertools

import numpy as np
import pytest

import oracle


def brute_route(ids, E, BM):
    ids = [int(v) for v in np.asarray(ids).reshape(-1)]
    P = len(ids)
    key = [v if 0 <= v < E else E for v in ids]
    order = sorted(range(P), key=lambda p: (key[p], p))
    pos = [0] * P
    for r, p in enumerate(order):
        pos[p] = r
    counts = [sum(1 for v in key if v == e) for e in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    tasks = []
    for e in range(E):
        m0 = 0
        while m0 < counts[e]:
            tasks.append([e, offsets[e] + m0, min(BM, counts[e] - m0), 0])
            m0 += BM
    return order, pos, offsets, tasks, P - offsets[E]


def check_against_brute(ids, E, BM):
    got = oracle.route(np.asarray(ids, dtype=np.int32), E, BM)
    order, pos, offsets, tasks, nd = brute_route(ids, E, BM)
    assert got["sorted"].tolist() == order
    assert got["pos"].tolist() == pos
    assert got["offsets"].tolist() == offsets
    assert got["tasks"].tolist() == tasks
    assert got["num_tasks"] == len(tasks)
    assert got["num_dropped"] == nd
    return got


def test_exhaustive_tiny():
    # every id vector over {-1, 0, .., E} for P <= 5, E <= 3, several tile heights
    for E in (1, 2, 3):
        for P in range(0, 6):
            for ids in itertools.product(range(-1, E + 1), repeat=P):
                for BM in (1, 2, 3):
                    check_against_brute(list(ids), E, BM)


@pytest.mark.parametrize("P,E,BM,p_drop,seed", [
    (2, 8, 16, 0.0, 1), (8, 128, 16, 0.0, 2), (512, 128, 32, 0.0, 3), (4096, 64, 64, 0.1, 4),
    (32768, 256, 128, 0.0, 5), (1000, 7, 5, 0.3, 6), (65536, 256, 64, 0.05, 7),
])
def test_random_against_brute(P, E, BM, p_drop, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=P).astype(np.int32)
    drop = rng.random(P) < p_drop
    ids[drop] = rng.choice([-1, E, E + 3, -(2 ** 31)], size=int(drop.sum()))
    check_against_brute(ids, E, BM)


def test_invariants_skewed():
    rng = np.random.default_rng(11)
    E, BM = 64, 16
    ids = np.where(rng.random(5000) < 0.5, 0, rng.integers(1, E, 5000)).astype(np.int32)
    ids[::97] = -1
    g = oracle.route(ids, E, BM)
    off, srt, pos = g["offsets"], g["sorted"], g["pos"]
    P = ids.size
    assert np.all(np.diff(off) >= 0)
    assert off[-1] + g["num_dropped"] == P
    assert np.array_equal(srt[pos], np.arange(P))          # inverse permutations
    assert np.array_equal(np.sort(srt), np.arange(P))
    for e in range(E):
        seg = srt[off[e]:off[e + 1]]
        assert np.all(ids[seg] == e) and np.all(np.diff(seg) > 0)
    tail = srt[off[-1]:]
    assert np.all((ids[tail] < 0) | (ids[tail] >= E)) and np.all(np.diff(tail) > 0)
    # tasks tile every expert range exactly once, in order, with <= BM rows
    covered = np.zeros(P, dtype=np.int32)
    prev = (-1, -1)
    for e, r0, rows, z in g["tasks"]:
        assert z == 0 and 1 <= rows <= BM
        assert off[e] <= r0 and r0 + rows <= off[e + 1]
        assert (e, r0) > prev
        prev = (e, r0)
        covered[r0:r0 + rows] += 1
    assert np.all(covered[:off[-1]] == 1) and np.all(covered[off[-1]:] == 0)
    assert g["num_tasks"] <= oracle.max_tasks(P, E, BM)


def test_task_count_bound():
    # sum_e ceil(c_e/BM) <= (P - A)//BM + A <= P//BM + min(E, P), A = active experts;
    # the middle bound is reached when every expert holds 1 + a multiple of BM pairs
    E, BM = 4, 4
    ids = np.array([0] * 5 + [1] * 5 + [2] * 5 + [3] * 1, dtype=np.int32)
    g = oracle.route(ids, E, BM)
    assert g["num_tasks"] == 2 + 2 + 2 + 1 == (ids.size - 4) // BM + 4
    assert g["num_tasks"] <= oracle.max_tasks(ids.size, E, BM)


def test_duplicates_within_token_are_separate_pairs():
    ids = np.array([[3, 3], [1, 3]], dtype=np.int32)
    g = check_against_brute(ids, 4, 8)
    assert g["offsets"].tolist() == [0, 0, 1, 1, 4]
    assert g["sorted"].tolist() == [2, 0, 1, 3]
