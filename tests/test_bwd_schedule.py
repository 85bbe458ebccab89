"""CPU models of the backward kernels' persistent schedules (host logic; no GPU).

The dK/dV part mirrors for_each_block in fa_bwd_kernel.hip and the dK/dV launch's grid choice:
every (head, key block) item must be run exactly once, and under the causal mask every workgroup
must get the same amount of work when the pairs divide evenly.  The dQ part mirrors take_item /
for_each_item (XCD-local item queues with stealing) under random interleavings of the
workgroups: every (head, query block) item is taken exactly once, queues hand out only their own
heads, head by head and longest block first, and a workgroup leaves its own queue only when it
is empty.  A change to the kernels' schedules must be made here as well.
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


# ---- the dQ kernel's item queues (take_item / for_each_item in fa_bwd_kernel.hip) ----------

OWN_Q = 256


def dq_grid_policy(BH, nblk, cus):
    items = BH * nblk
    if items > cus and cus >= 8:
        return cus - cus % 8, 8
    return min(items, max(cus, 1)), 1


def queue_items(BH, nblk, X, x):
    return -(-(BH - x) // X) * nblk


def simulate_queues(BH, nblk, cus, rev, seed):
    """Runs the workgroups' take loop in a random interleaving (one take at a time, as the
    counters' atomics serialise them) -> ({workgroup: [(bh, blk, queue), ...]}, counters)."""
    import random
    rng = random.Random(seed)
    G, X = dq_grid_policy(BH, nblk, cus)
    ctr = [0] * X
    done = {n: False for n in range(G)}
    taken = {n: [] for n in range(G)}
    while not all(done.values()):
        n = rng.choice([m for m in range(G) if not done[m]])
        x0 = n % X
        got = None
        for q in range(X):
            x = (x0 + q) % X
            k = ctr[x]
            ctr[x] += 1
            if k < queue_items(BH, nblk, X, x):
                got = (x, k)
                break
        if got is None:
            done[n] = True
            continue
        x, k = got
        hl, r = divmod(k, nblk)
        taken[n].append((x + X * hl, nblk - 1 - r if rev else r, x))
    return taken, ctr, X


DQ_SHAPES = [(256, 4096), (256, 1024), (64, 16384), (111, 1100), (2, 200), (1, 1), (9, 300),
             (3, 70000), (130, 256)]


@pytest.mark.parametrize("BH,Tq", DQ_SHAPES)
@pytest.mark.parametrize("seed", [0, 1])
def test_dq_queues_take_every_item_once(BH, Tq, seed):
    nblk = -(-Tq // OWN_Q)
    taken, ctr, X = simulate_queues(BH, nblk, 256, True, seed)
    seen = sorted((bh, b) for items in taken.values() for bh, b, _ in items)
    assert seen == sorted((bh, b) for bh in range(BH) for b in range(nblk))
    # a queue only ever hands out heads of its residue class
    assert all(bh % X == x for items in taken.values() for bh, _, x in items)
    # counters end past their queues (each workgroup's last, failed, round) and never wrap
    assert all(c >= queue_items(BH, nblk, X, x) for x, c in enumerate(ctr))


def test_dq_queue_order_is_head_major_longest_first():
    """Items leave a queue head by head, and within a head from the last query block (under the
    causal mask the one with the most keys) down."""
    nblk, X, x = 16, 8, 5
    seq = []
    for k in range(queue_items(64, nblk, X, x)):
        hl, r = divmod(k, nblk)
        seq.append((x + X * hl, nblk - 1 - r))
    assert seq[:nblk] == [(5, b) for b in range(nblk - 1, -1, -1)]
    assert [bh for bh, _ in seq] == sorted(bh for bh, _ in seq)


def test_dq_own_queue_first():
    """A workgroup takes from another queue only once its own is empty."""
    taken, _, X = simulate_queues(256, 16, 256, True, 7)
    for n, items in taken.items():
        own = [i for i, (_, _, x) in enumerate(items) if x == n % X]
        other = [i for i, (_, _, x) in enumerate(items) if x != n % X]
        if own and other:
            assert max(own) < min(other)
