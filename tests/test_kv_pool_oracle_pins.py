"""Pins for the paged KV pool model (HPD-Parsing notes, "KV cache and
shared-prefix reuse", Algorithm 1): a hand-worked sequence of operations, and
invariants on random operation sequences (every block's reference count is
the number of live sequences that hold it; releasing everything frees every
block; slots of live tokens never collide unless one sequence views the
other's block)."""
import os

import numpy as np
import pytest

from oracle.kv_pool_oracle import KVPool, PoolError

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def parse_ops(name):
    ops = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("pool"):
                pool = tuple(int(x) for x in line.split()[1:])
                continue
            lhs, rhs = line.split("->")
            res, refs = rhs.split(";")
            ops.append((lhs.split(), res.strip(), [int(x) for x in refs.split()[1:]]))
    return pool, ops


def test_golden_pool_sequence():
    (nb, bs), ops = parse_ops("kv_pool_worked.txt")
    pool = KVPool(nb, bs)
    for args, want, refs in ops:
        op, a = args[0], [int(x) for x in args[1:]]
        if op == "new":
            got = str(pool.new_seq())
        elif op == "append":
            try:
                got = " ".join(str(s) for s in pool.append(*a))
            except PoolError:
                got = "error"
        elif op == "fork":
            got = str(pool.fork(*a))
        elif op == "release":
            pool.release(*a)
            got = "ok"
        elif op == "table":
            v, vl, o, ol = pool.table(*a)
            got = f"view {' '.join(map(str, v))} / {vl} own {' '.join(map(str, o))} / {ol}"
        assert got == want, (args, got, want)
        assert pool.ref == refs, (args, pool.ref, refs)


def check_invariants(pool):
    held = [0] * pool.n_blocks
    for s in pool.seqs.values():
        for b in s["view"] + s["own"]:
            held[b] += 1
        assert len(s["own"]) == (s["own_len"] + pool.bs - 1) // pool.bs
        assert len(s["view"]) == (s["view_len"] + pool.bs - 1) // pool.bs
    assert held == pool.ref
    # own blocks are never shared between two sequences' own lists
    owners = {}
    for sid, s in pool.seqs.items():
        for b in s["own"]:
            assert b not in owners
            owners[b] = sid
    # a view only holds blocks of some root's own list (or of a released root)
    for s in pool.seqs.values():
        for b in s["view"]:
            assert pool.ref[b] >= 1


@pytest.mark.parametrize("seed", range(5))
def test_pool_invariants_random(seed):
    rng = np.random.default_rng(seed)
    pool = KVPool(int(rng.integers(4, 40)), int(rng.choice([1, 2, 4, 64])))
    roots = []
    for step in range(400):
        live = list(pool.seqs)
        op = rng.integers(0, 4)
        if op == 0 or not live:
            roots.append(pool.new_seq())
        elif op == 1:
            sid = live[int(rng.integers(len(live)))]
            before = (list(pool.ref), pool.table(sid))
            try:
                slots = pool.append(sid, int(rng.integers(0, 3 * pool.bs)))
                assert len(set(slots)) == len(slots)
            except PoolError:
                assert (pool.ref, pool.table(sid)) == before  # failed appends change nothing
        elif op == 2:
            rs = [r for r in roots if r in pool.seqs]
            if rs:
                r = rs[int(rng.integers(len(rs)))]
                n = int(rng.integers(0, pool.seqs[r]["own_len"] + 1))
                pool.fork(r, n)
        else:
            pool.release(live[int(rng.integers(len(live)))])
        check_invariants(pool)
    for sid in list(pool.seqs):
        pool.release(sid)
    assert pool.free_blocks() == pool.n_blocks


def test_pool_rejects():
    pool = KVPool(2, 4)
    r = pool.new_seq()
    pool.append(r, 4)
    c = pool.fork(r, 3)
    with pytest.raises(PoolError):
        pool.fork(c, 1)          # forks come from roots
    with pytest.raises(PoolError):
        pool.fork(r, 5)          # past the parent's tokens
    with pytest.raises(PoolError):
        pool.append(r, 5)        # 9 tokens need 3 blocks
    pool.release(r)
    assert pool.ref == [1, 0]    # the fork still views block 0
    with pytest.raises(PoolError):
        pool.release(r)


def test_gather_reads_what_append_slots_wrote():
    """Tokens written at the slots append hands out read back in logical
    order through the block table (views included)."""
    import numpy as np
    from oracle import gather_paged
    pool = KVPool(10, 4)
    cache = np.full((40, 2), -1.0)
    r = pool.new_seq()
    cache[pool.append(r, 7)] = np.arange(7)[:, None]
    c = pool.fork(r, 5)
    cache[pool.append(c, 6)] = 100 + np.arange(6)[:, None]
    cache[pool.append(r, 3)] = 7 + np.arange(3)[:, None]
    v, vl, o, ol = pool.table(c)
    assert gather_paged(cache, v, vl, 4)[:, 0].tolist() == list(range(5))
    assert gather_paged(cache, o, ol, 4)[:, 0].tolist() == list(range(100, 106))
    v, vl, o, ol = pool.table(r)
    assert gather_paged(cache, o, ol, 4)[:, 0].tolist() == list(range(10))
