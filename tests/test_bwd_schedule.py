"""CPU model of the backward dK/dV kernel's persistent schedule (host logic; no GPU).

It mirrors for_each_block in fa_bwd_kernel.hip and the dK/dV launch's grid choice: every (head,
key block) item must be run exactly once, and under the causal mask every workgroup must get the
same amount of work when the pairs divide evenly.  A change to either must be made here as well.
"""
import pytest

OWN_K = 128


def grid_policy(BH, nblk, cus):
    pairs = BH * ((nblk + 1) // 2)
    if pairs > cus and cus >= 8:
        return cus - cus % 8, 8
    return min(pairs, max(cus, 1)), 1


def schedule(BH, nblk, cus=256):
    """{workgroup: [(bh, blk), ...]} as the kernel runs them."""
    G, X = grid_policy(BH, nblk, cus)
    out = {}
    for n in range(G):
        x, c = n % X, n // X
        C = -(-(G - x) // X)
        np_ = (nblk + 1) // 2
        PX = -(-(BH - x) // X) * np_
        items = []
        u = 0
        while True:
            pp = c + (u >> 1) * C
            if pp >= PX:
                break
            hl, j = divmod(pp, np_)
            blk = j if (u & 1) else nblk - 1 - j
            if (u & 1) and blk == nblk - 1 - j:
                u += 1
                continue
            items.append((x + X * hl, blk))
            u += 1
        out[n] = items
    return out


SHAPES = [
    # (BH, Tk)
    (256, 4096), (256, 1024), (64, 16384), (111, 1100), (90, 1300), (130, 1024), (2, 200),
    (1, 1), (8, 256), (3, 129), (256, 4097), (7, 70000),
]


@pytest.mark.parametrize("BH,Tk", SHAPES)
def test_every_block_runs_once(BH, Tk):
    nblk = -(-Tk // OWN_K)
    sched = schedule(BH, nblk)
    seen = [it for items in sched.values() for it in items]
    assert sorted(seen) == sorted((bh, b) for bh in range(BH) for b in range(nblk))


@pytest.mark.parametrize("BH,Tk", [(256, 4096), (256, 1024), (64, 16384)])
def test_causal_work_is_balanced(BH, Tk):
    """Block j sees Tq - 128 j queries (Tq = Tk): every workgroup's total is the same."""
    nblk = Tk // OWN_K
    sched = schedule(BH, nblk)
    totals = {sum(Tk - OWN_K * b for _, b in items) for items in sched.values()}
    assert len(totals) == 1


def test_xcd_groups_keep_heads_together():
    """With 8 groups, workgroup n only runs heads congruent to n mod 8."""
    sched = schedule(256, 32)
    assert all(bh % 8 == n % 8 for n, items in sched.items() for bh, _ in items)
