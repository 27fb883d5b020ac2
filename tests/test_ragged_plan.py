"""Ragged-batch planning (host logic, no GPU): the model of the prep kernel's
records covers every (request, row block, key) exactly once, stays within the
launch bounds the host sizes, and numbers slots and merged blocks the way the
merge pass reads them."""
import numpy as np
import pytest

import ragged_plan_model as RP

MFMA = dict(rpb=128, target=256)      # bf16 cache, one-term queries
Q2 = dict(rpb=64, target=256)         # bf16 cache, two-term queries (the default)
F32 = dict(rpb=64, target=256, cost=RP.COST_F32)
VALU = dict(rpb=16, target=512)


def _merge_slots(rec, mb):
    """Rows and slots of merged block mb, as attn_merge_ragged_kernel reads
    them from the merge table."""
    slot0, n, row0, rows = RP.merge_table(rec)[mb]
    return row0, rows, [slot0 + s for s in range(n)]


def check(prefix, q_len, H, max_q, kv_stride, rpb, target, cost=RP.COST_DEFAULT, n_nodes=None):
    rec = RP.plan(prefix, q_len, H, max_q, kv_stride, rpb, target, cost, n_nodes=n_nodes)
    bound_units, bound_slots, bound_merges = RP.launch_bounds(len(q_len), H, max_q, rpb, target)
    assert rec["units"] <= bound_units and rec["merges"] <= bound_merges
    covered = {}
    slots = {}
    for x in range(bound_units):
        d = RP.decode(rec, x, H)
        if x >= rec["units"]:
            assert d is None
            continue
        b, rb, piece, k0, k1, slot = d
        r = rec["req"][b]
        assert r["q_len"] > 0 and 0 <= rb < r["n_blk"] and 0 <= k0 < k1 <= r["prefix"] + r["q_len"], d
        covered.setdefault((b, rb), []).append((k0, k1))
        if slot >= 0:
            assert 0 <= slot < bound_slots and slot not in slots, d
            slots[slot] = (b, rb, piece)
    q_start = 0
    for b, r in enumerate(rec["req"]):
        q = min(max(q_len[b], 0), max_q)
        if n_nodes is not None:
            q = min(q, max(0, n_nodes - q_start))
        assert r["q_len"] == q and r["q_start"] == q_start
        q_start += q
        if n_nodes is not None:
            assert q_start <= n_nodes
        assert r["n_blk"] == -(-(q * H) // rpb)
        kv = r["prefix"] + q
        for rb in range(r["n_blk"]):
            pieces = sorted(covered.get((b, rb), []))
            assert pieces and pieces[0][0] == 0 and pieces[-1][1] == kv, (b, rb, pieces)
            assert all(pieces[i][1] == pieces[i + 1][0] for i in range(len(pieces) - 1)), (b, rb)
            if len(pieces) == 1:
                assert all(v[:2] != (b, rb) for v in slots.values())
    # merged blocks: exactly the split row blocks, each reading its own slots
    # and writing its own rows
    seen = set()
    for mb in range(rec["merges"]):
        row0, rows, sl = _merge_slots(rec, mb)
        b = max(i for i, r in enumerate(rec["req"]) if r["n_blk"] and r["q_start"] * H <= row0)
        r = rec["req"][b]
        rb, off = divmod(row0 - r["q_start"] * H, rpb)
        assert off == 0 and rb < r["n_blk"] and rows == min(rpb, r["q_len"] * H - rb * rpb), (mb, b, rb)
        assert (b, rb) not in seen and len(sl) > 1
        seen.add((b, rb))
        assert sorted(sl) == sorted(s for s, v in slots.items() if v[:2] == (b, rb)), (b, rb)
    assert len(seen) == len({v[:2] for v in slots.values()})
    return rec


def _families(rng):
    yield [int(x) for x in rng.choice([9, 17, 33], 32)], [int(x) for x in rng.integers(2048, 16384, 32)], 64, 33
    yield [33] * 32, [8192] * 32, 64, 33
    B = int(rng.integers(2, 12))
    yield [int(x) for x in rng.integers(1, 65, B)], [int(x) for x in rng.integers(10000, 200000, B)], 64, 64
    B = int(rng.integers(64, 200))
    yield [int(x) for x in rng.integers(0, 34, B)], [int(x) for x in rng.integers(0, 4000, B)], 16, 33
    yield [33] * 32, [int(min(200000, x)) for x in rng.lognormal(8.5, 1.0, 32)], 64, 33


@pytest.mark.parametrize("seed", range(4))
def test_plan_covers_and_bounds(seed):
    rng = np.random.default_rng(seed)
    for q_len, prefix, H, max_q in _families(rng):
        kv_stride = max(p + q for p, q in zip(prefix, q_len)) + 3
        for kern in (MFMA, Q2, F32, VALU):
            check(prefix, q_len, H, max_q, kv_stride, **kern)


def test_plan_edge_cases():
    # empty requests, no prefix, one node, lengths clamped into the bounds
    check([0, 5, 100, 7], [0, 1, 0, 3], 8, 4, 120, **MFMA)
    check([50, -4, 10**9, 3], [9, 300, 2, -1], 8, 16, 100, **MFMA)
    check([0], [1], 1, 1, 1, **MFMA)
    check([0] * 5, [0] * 5, 4, 8, 64, **VALU)
    check([200000], [64], 128, 64, 200064, **MFMA)   # one request, many row blocks, long prefix
    check([300, 40000], [256, 1], 2, 256, 40256, **VALU)
    check([300, 40000, 0], [256, 1, 7], 2, 256, 40256, **F32)


def test_plan_unsorted_large_batch():
    """More classes than the prep kernel sorts in LDS: request order, still a
    cover."""
    rng = np.random.default_rng(3)
    B = 2100
    q_len = [int(x) for x in rng.integers(0, 9, B)]
    prefix = [int(x) for x in rng.integers(0, 700, B)]
    rec = check(prefix, q_len, 4, 8, 720, **MFMA)
    assert rec["cls_id"] == list(range(2 * B))


def test_plan_orders_longest_first():
    """Each XCD's queue (blocks x = k, k + 8, ...) takes units longest first."""
    rng = np.random.default_rng(5)
    q_len = [int(x) for x in rng.choice([9, 17, 33], 32)]
    prefix = [int(x) for x in rng.integers(2048, 16384, 32)]
    rec = RP.plan(prefix, q_len, 64, 33, 16500, **MFMA)
    lens = []
    for x in range(rec["units"]):
        b, rb, piece, k0, k1, slot = RP.decode(rec, x, 64)
        r = rec["req"][b]
        lens.append(r["t_chunk"] if rb == r["n_blk"] - 1 else r["b_chunk"])
    whole = rec["units"] // (8 * RP.DEAL) * (8 * RP.DEAL)
    for k in range(8):
        q = lens[k:whole:8]
        assert q == sorted(q, reverse=True), k
    assert rec["choice"] != 0  # a batch this uneven is cut


def test_plan_uniform_batch_keeps_whole_blocks():
    """Equal requests: the blocks before the last stay whole and the last
    blocks are cut into pieces that fill the last round, the uniform plan's
    choice."""
    rec = RP.plan([8192] * 32, [33] * 32, 64, 33, 8225, **MFMA)
    for r in rec["req"]:
        assert r["b_split"] == 1 and r["t_split"] > 1


def test_plan_node_bound():
    """Device lengths that sum past the caller's n_nodes rows: the request
    crossing the bound keeps its nodes below it, later ones none, and no unit,
    slot or merged row reaches past n_nodes."""
    rng = np.random.default_rng(11)
    for q_len, prefix, H, max_q in _families(rng):
        kv_stride = max(p + q for p, q in zip(prefix, q_len)) + 3
        tot = sum(min(max(q, 0), max_q) for q in q_len)
        for N in (0, 1, tot // 3, tot - 1, tot, tot + 5):
            for kern in (MFMA, Q2, F32, VALU):
                rec = check(prefix, q_len, H, max_q, kv_stride, n_nodes=N, **kern)
                assert sum(r["q_len"] for r in rec["req"]) == min(N, tot)
                for mb in range(rec["merges"]):
                    _, _, row0, rows = RP.merge_table(rec)[mb]
                    assert row0 + rows <= N * H
    # the crossing request is cut inside itself
    rec = RP.plan([10, 10, 10], [5, 5, 5], 4, 8, 40, n_nodes=7, **MFMA)
    assert [r["q_len"] for r in rec["req"]] == [5, 2, 0]
    assert [r["q_start"] for r in rec["req"]] == [0, 5, 7]
