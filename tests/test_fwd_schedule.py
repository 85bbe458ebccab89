"""CPU model of the forward kernel's static schedule (host logic; no GPU).

The persistent forward deals (head, query-block pair) items to workgroups and runs each
workgroup's items as one stream of K/V tiles through a 4-stage LDS ring, requesting stream
position t + 2 at step t.  This model replays that schedule for a launch shape -- the grid policy
of the host launcher, then per workgroup the item sequence, the tile requests and the tile reads
-- and checks that every read finds, in its ring stage, the tile of the item being computed.

It mirrors fa_fwd_kernel.hip's describe / following / request logic and its launch() grid choice;
a change to either must be made here as well.
"""
import math

import pytest

BM, BN, STAGES = 256, 64, 4


def grid_policy(BH, Tq, Tk, cus, single_tile_rule=True):
    """(grid, groups) as the host launcher picks them."""
    nqb = -(-Tq // BM)
    pairs = BH * ((nqb + 1) // 2)
    if single_tile_rule and Tk <= BN:
        return pairs, 1
    if pairs > cus and cus >= 8:
        return cus - cus % 8, 8
    return min(pairs, max(cus, 1)), 1


def simulate(BH, Tq, Tk, causal, cus=256, single_tile_rule=True):
    """Replay the schedule; returns (bad_reads, items_run, item_count_per_head_block)."""
    grid, X = grid_policy(BH, Tq, Tk, cus, single_tile_rule)
    nqb = -(-Tq // BM)
    npairs = (nqb + 1) // 2
    off = Tk - Tq
    bad = 0
    seen = {}

    for n in range(grid):
        x, c = n % X, n // X
        C = -(-(grid - x) // X)
        PX = -(-(BH - x) // X) * npairs

        def describe(pp, half):
            hl, j = divmod(pp, npairs)
            bh = x + X * hl
            i0 = (nqb - 1 - j if half == 0 else j) * BM
            kend = Tk
            if causal:
                kend = min(Tk, min(i0 + BM, Tq) + off)
            return {"pp": pp, "half": half, "bh": bh, "i0": i0, "ntiles": -(-kend // BN)}

        def following(it):
            j = it["pp"] % npairs
            if it["half"] == 0 and nqb - 1 - j != j:
                return describe(it["pp"], 1)
            return describe(it["pp"] + C, 0)

        stage = [None] * STAGES

        def load(pos, item, tile):
            stage[pos % STAGES] = (item["bh"], item["i0"], tile)

        def read(pos, item, tile):
            nonlocal bad
            if stage[pos % STAGES] != (item["bh"], item["i0"], tile):
                bad += 1

        cur = describe(c, 0)
        if cur["pp"] < PX:   # prologue: stream positions 0 and 1
            load(0, cur, 0)
            if cur["ntiles"] > 1:
                load(1, cur, 1)
            else:
                nx = following(cur)
                if nx["pp"] < PX:
                    load(1, nx, 0)
        g0 = 0
        while cur["pp"] < PX:
            nxt = following(cur)
            has_nxt = nxt["pp"] < PX
            nt = cur["ntiles"]
            key = (cur["bh"], cur["i0"])
            seen[key] = seen.get(key, 0) + 1
            for t in range(nt):
                xt = t + 2   # request(t + 2) at the start of matrix section t
                if xt < nt:
                    load(g0 + xt, cur, xt)
                elif has_nxt and xt - nt < nxt["ntiles"]:
                    load(g0 + xt, nxt, xt - nt)
                if t > 0:
                    read(g0 + t - 1, cur, t - 1)   # V^T of the previous tile
                read(g0 + t, cur, t)               # K of this tile; its V^T is read ahead
            read(g0 + nt - 1, cur, nt - 1)         # last step: the last tile's V^T
            g0 += nt
            cur = nxt
    return bad, seen, nqb


SHAPES = [
    # (BH, Tq, Tk, causal)
    (256, 4096, 4096, True),      # the prefill workload (B=8, h=32)
    (256, 1024, 1024, True),      # B=8, h=32, T=1024
    (64, 16384, 16384, True),     # B=2, h=32, T=16384
    (111, 1100, 1100, True), (111, 1100, 1500, True), (90, 1300, 1300, False),
    (130, 1024, 1024, True),
    (256, 4096, 64, False),       # one key tile per item, many items per head
    (1024, 64, 64, True),         # B=32, h=32, T=64
    (300, 300, 40, False), (700, 1, 1, True), (256, 4096, 65, False), (256, 129, 64, True),
]


@pytest.mark.parametrize("BH,Tq,Tk,causal", SHAPES)
def test_every_tile_read_finds_its_tile(BH, Tq, Tk, causal):
    bad, seen, nqb = simulate(BH, Tq, Tk, causal)
    assert bad == 0, f"{bad} tile reads find another tile in their ring stage"
    # every (head, query block) item runs exactly once
    assert len(seen) == BH * nqb and all(v == 1 for v in seen.values())


@pytest.mark.parametrize("BH,Tq,Tk,causal", [(256, 4096, 64, False), (1024, 64, 64, True)])
def test_model_sees_the_lookahead_gap_without_the_single_tile_rule(BH, Tq, Tk, causal):
    """Without the launcher's rule for one-tile items, a workgroup with three or more such items
    reads a ring stage whose tile was never requested: the model must detect it."""
    bad, _, _ = simulate(BH, Tq, Tk, causal, single_tile_rule=False)
    assert bad > 0


def test_grid_policy_matches_the_launcher_cases():
    assert grid_policy(256, 4096, 4096, 256) == (256, 8)
    assert grid_policy(2, 128, 128, 256) == (2, 1)
    assert grid_policy(256, 4096, 64, 256) == (256 * 8, 1)
    assert math.ceil(4096 / BM) == 16
