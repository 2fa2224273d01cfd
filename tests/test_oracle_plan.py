"""Pins of the split-plan re-derivation by its invariants (CPU only)."""
import numpy as np
import pytest

from oracle import plan as PL


def _check(seq_lens, Sq, N, C):
    p = PL.split_plan(seq_lens, Sq, N, C)
    hg = PL.head_groups(Sq, N)
    budget = max(1, C // hg)
    assert 1 <= p["num_parts"] <= budget
    items = p["items"]
    # parts are numbered 0..num_parts-1 in order, each non-empty
    parts = [it[0] for it in items]
    assert parts == sorted(parts) and set(parts) == set(range(p["num_parts"]))
    # every request's key range is covered exactly once, in order, by its segments
    by_req = {}
    for (_, b, ks, ke, pidx) in items:
        by_req.setdefault(b, []).append((ks, ke, pidx))
    assert sorted(by_req) == list(range(len(seq_lens)))
    nxt = 0
    red = {b: (base, n) for (b, base, n) in p["reduce"]}
    for b, segs in sorted(by_req.items()):
        L = int(seq_lens[b])
        pos = 0
        for (ks, ke, _) in segs:
            assert ks == pos and ke >= ks
            pos = ke
        assert pos == L
        if len(segs) > 1:
            assert all(ke > ks for (ks, ke, _) in segs)
            base, n = red[b]
            assert n == len(segs) and base == nxt
            assert [s[2] for s in segs] == list(range(base, base + n))
            nxt += n
            # splits start on granule boundaries
            assert all(ks % PL.GRANULE == 0 for (ks, _, _) in segs)
        else:
            assert b not in red and segs[0][2] == -1
    assert nxt == p["num_partials"]
    # load of each part stays within the target used
    load = {}
    for (pt, b, ks, ke, _) in items:
        g = -(-ke // PL.GRANULE) - ks // PL.GRANULE
        load[pt] = load.get(pt, 0) + PL.SEG_COST + g
    assert max(load.values()) <= p["target"]
    return p


@pytest.mark.parametrize("seed", range(40))
def test_plan_invariants_random(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 300))
    special = [0, 1, 63, 64, 65, 255, 256, 257, 32768]
    L = rng.integers(0, 20000, size=B)
    k = int(rng.integers(0, B + 1))
    L[:k] = rng.choice(special, size=k)
    Sq = int(rng.integers(1, 9))
    N = int(rng.integers(1, 129))
    C = int(rng.choice([1, 7, 64, 256, 304]))
    _check(L, Sq, N, C)


def test_plan_workload_shapes():
    # a single short request fits one segment; long uniform requests split evenly
    p = _check([256], 1, 16, 256)
    assert p["items"] == [(0, 0, 0, 256, -1)] and p["reduce"] == []
    # 4 tokens x 128 heads = 4 head groups of 128 rows, so 64 parts for 256 CUs: each
    # request (64 granules + 1 of segment cost) is cut in two near-equal halves
    p = _check([4096] * 32, 4, 128, 256)
    assert PL.head_groups(4, 128) == 4 and p["num_parts"] == 64
    assert p["reduce"] == [(b, 2 * b, 2) for b in range(32)]
    # 128 heads fit one group: 256 parts, the minimum chunk (4 granules) sets the cut
    p = _check([4096] * 8, 1, 128, 256)
    assert PL.head_groups(1, 128) == 1 and all(n == 16 for (_, _, n) in p["reduce"])
    p = _check([0, 0, 5], 1, 128, 256)
    assert [it[1:] for it in p["items"]] == [(0, 0, 0, -1), (1, 0, 0, -1), (2, 0, 5, -1)]


def test_plan_is_independent_of_head_count_when_groups_match():
    L = np.random.default_rng(9).integers(1, 9000, size=50)
    a = PL.split_plan(L, 1, 16, 256)
    b = PL.split_plan(L, 1, 64, 256)
    assert a["items"] == b["items"] and a["reduce"] == b["reduce"]


def test_workspace_bytes():
    assert PL.workspace_bytes(3, 1, 16) == 3 * (32 * 512 * 2 + 16 * 8)  # 16 rows -> one 32-row block
    assert PL.workspace_bytes(2, 1, 128) == 2 * 128 * (512 * 2 + 8)
    assert PL.workspace_bytes(1, 4, 40) == 160 * 512 * 2 + 160 * 8


def test_gather_rows_all_matches_golden():
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_expansion.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert PL.gather_rows_all(c["block_table"], c["seq_lens"], c["page_size"]) == c["rows"]
