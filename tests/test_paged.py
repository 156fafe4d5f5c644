"""CPU tests of the paged KV pieces: the host block pool against the oracle's
pool model (same slots, tables, reference counts and errors on random
operation sequences and on the hand-worked one), and paged decode / verify
plans (semantic fields equal to the unpaged plan's, tile tables equal to the
block-table definition, work items covering every visible pair once,
validation errors)."""
import os

import numpy as np
import pytest

import oracle
from oracle.kv_pool_oracle import KVPool as PoolModel, PoolError
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth
from test_plan_abi import check_decode_items

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_pool_golden_sequence():
    from test_kv_pool_oracle_pins import parse_ops
    (nb, bs), ops = parse_ops("kv_pool_worked.txt")
    pool = ta.KVPool(nb, bs)
    for args, want, refs in ops:
        op, a = args[0], [int(x) for x in args[1:]]
        if op == "new":
            got = str(pool.new_seq())
        elif op == "append":
            try:
                got = " ".join(str(s) for s in pool.append(*a))
            except ta.TreeAttnError as e:
                assert e.code == ta.TA_ERR_CAPACITY
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
        assert pool.refs()[0].tolist() == refs, args


@pytest.mark.parametrize("seed", range(4))
def test_pool_matches_model_random(seed):
    rng = np.random.default_rng(50 + seed)
    nb, bs = int(rng.integers(1, 30)), int(rng.choice([1, 3, 64]))
    lib_pool, model = ta.KVPool(nb, bs), PoolModel(nb, bs)
    for step in range(500):
        live = sorted(model.seqs)
        op = int(rng.integers(0, 5))
        if op == 0 or not live:
            assert lib_pool.new_seq() == model.new_seq()
        elif op == 1:
            sid = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, 3 * bs + 2))
            try:
                want = model.append(sid, n)
            except PoolError:
                with pytest.raises(ta.TreeAttnError):
                    lib_pool.append(sid, n)
            else:
                assert lib_pool.append(sid, n).tolist() == want
        elif op == 2:
            sid = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, model.seqs[sid]["own_len"] + 2))
            try:
                want = model.fork(sid, n)
            except PoolError:
                with pytest.raises(ta.TreeAttnError):
                    lib_pool.fork(sid, n)
            else:
                assert lib_pool.fork(sid, n) == want
        elif op == 3:
            sid = live[int(rng.integers(len(live)))]
            model.release(sid)
            lib_pool.release(sid)
            with pytest.raises(ta.TreeAttnError):
                lib_pool.table(sid)
        else:
            sid = live[int(rng.integers(len(live)))]
            v, vl, o, ol = lib_pool.table(sid)
            assert (v.tolist(), vl, o.tolist(), ol) == model.table(sid)
        r, free = lib_pool.refs()
        assert r.tolist() == model.ref and free == model.free_blocks()


def paged_decode_setup(desc, bs, rng, spare=0):
    """Lay a decode description out in a pool: per page a root holding its
    main stream, per branch a fork at the branch's bound holding its suffix
    (s_k + K_b tokens).  Other sequences are created and released first so
    that blocks come back in a scrambled order."""
    main = desc.main_tokens()
    kq = desc.queries()
    suf = desc.suffix_len.astype(np.int64) + kq
    need = sum((int(m) + bs - 1) // bs for m in main) + sum((int(s) + bs - 1) // bs for s in suf)
    nb = need + spare + 8
    pool = ta.KVPool(nb, bs)
    junk = [pool.new_seq() for _ in range(4)]
    for j in junk:
        pool.append(j, int(rng.integers(0, 2 * bs)))
    for j in junk[::2]:
        pool.release(j)
    roots, main_slots = [], []
    for p in range(desc.n_pages):
        r = pool.new_seq()
        roots.append(r)
        main_slots.append(pool.append(r, int(main[p])))
    reg_off = np.concatenate([[0], np.cumsum(desc.n_regions.astype(np.int64))])
    suffix_slots, suffix_tables = [], []
    for b in range(desc.n_branches):
        p = int(desc.br_page[b])
        k = int(desc.br_region[b]) or int(desc.n_regions[p])
        bound = int(desc.prefix_len[p]) + int(desc.layout_len[reg_off[p]:reg_off[p] + k].sum())
        c = pool.fork(roots[p], bound)
        suffix_slots.append(pool.append(c, int(suf[b])))
        suffix_tables.append(pool.table(c)[2])
    main_tables = [pool.table(r)[2] for r in roots]
    return pool, nb, main_tables, suffix_tables, main_slots, suffix_slots


def decode_descs():
    out = [synth.decode_multi(with_tensors=False, n_pages=2).desc, synth.config4(with_tensors=False, n_pages=2).desc]
    rng = np.random.default_rng(8)
    for trial in range(4):
        n_pages = int(rng.integers(1, 4))
        N = rng.integers(0, 4, n_pages)
        L = rng.integers(0, 70, int(N.sum()))
        bp, br, s, kq = [], [], [], []
        for p in range(n_pages):
            for _ in range(int(rng.integers(0, 5))):
                bp.append(p)
                br.append(int(rng.integers(0, int(N[p]) + 1)))
                s.append(int(rng.integers(0, 2500)))
                kq.append(int(rng.integers(1, 80)))
        out.append(synth.DecodeDesc(rng.integers(0, 3000, n_pages).astype(np.int32), N.astype(np.int32),
                                    L.astype(np.int32), np.array(bp, np.int32), np.array(br, np.int32),
                                    np.array(s, np.int32), np.array(kq, np.int32)))
    return out


@pytest.mark.parametrize("bs", [64, 128, 256])
def test_paged_decode_plan(bs):
    rng = np.random.default_rng(bs)
    for desc in decode_descs():
        pool, nb, mt, st, _, _ = paged_decode_setup(desc, bs, rng)
        plan = ta.plan_decode_paged(desc.prefix_len, desc.n_regions, desc.layout_len, desc.br_page,
                                    desc.br_region, desc.suffix_len, desc.queries(), bs, nb, mt, st)
        ref = oracle.plan_decode(desc)["rows"]
        rows = plan.export("decode_rows")
        # lengths and positions are the unpaged plan's; starts are virtual, on tile boundaries
        assert np.array_equal(rows[:, [1, 3, 4]], ref[:, [1, 3, 4]])
        assert (rows[:, 0] % 64 == 0).all() and (rows[:, 2] % 64 == 0).all()
        info = plan.info
        assert info["n_keys_a"] == nb * bs and info["n_keys_b"] == nb * bs
        assert info["visible_pairs"] == int((ref[:, 1] + ref[:, 3]).sum())
        check_decode_items(plan, desc)
        # tile tables: the cache row of every tile's first token
        tiles = plan.export("paged_tiles")
        n_a = int(max([0] + [r[0] + ((r[1] + 63) // 64) * 64 for r in rows])) // 64
        ta_tab, tb_tab = tiles[:n_a], tiles[n_a:]
        # main: each page with live rows, at the virtual start its rows report
        row0 = np.concatenate([[0], np.cumsum(desc.queries())])
        for b in range(desc.n_branches):
            p = int(desc.br_page[b])
            ms = int(rows[row0[b], 0])
            for t in range(0, int(desc.main_tokens()[p]), 64):
                assert ta_tab[(ms + t) // 64] == mt[p][t // bs] * bs + t % bs
        suf = desc.suffix_len.astype(np.int64) + desc.queries()
        for b in range(desc.n_branches):
            ss = int(rows[row0[b], 2])
            for t in range(0, int(suf[b]), 64):
                assert tb_tab[(ss + t) // 64] == st[b][t // bs] * bs + t % bs


def test_paged_plan_errors():
    d = synth.config4(with_tensors=False, n_pages=1).desc
    rng = np.random.default_rng(1)
    pool, nb, mt, st, _, _ = paged_decode_setup(d, 64, rng)

    def mk(bs=64, n=nb, m=mt, s=st):
        return ta.plan_decode_paged(d.prefix_len, d.n_regions, d.layout_len, d.br_page, d.br_region,
                                    d.suffix_len, None, bs, n, m, s)
    mk()
    for bad in (dict(bs=32), dict(bs=96), dict(bs=0), dict(n=int(mt[0].max())),
                dict(m=[mt[0][:-1]]), dict(s=[t[:0] if i == 3 else t for i, t in enumerate(st)])):
        with pytest.raises(ta.TreeAttnError) as e:
            mk(**bad)
        assert e.value.code == ta.TA_ERR_INVALID_ARG, bad
    with pytest.raises(ta.TreeAttnError) as e:
        mk(n=1 << 26)
    assert e.value.code == ta.TA_ERR_CAPACITY


def test_paged_verify_plan():
    w = synth.config5(with_tensors=False, n_pages=3)
    desc = w.desc
    bs = 128
    pool = ta.KVPool(2000, bs)
    tables = []
    for p in range(desc.n_pages):
        r = pool.new_seq()
        pool.append(r, int(desc.ctx_len[p]))
        tables.append(pool.table(r)[2])
    plan = ta.plan_verify_paged(desc.ctx_len, desc.br_page, desc.n_nodes, desc.parent, bs, 2000, tables)
    ref = ta.plan_for(desc)
    for f in ("verify_mask",):
        assert np.array_equal(plan.export(f), ref.export(f))
    rows, rrows = plan.export("verify_rows"), ref.export("verify_rows")
    assert np.array_equal(rows[:, 1:], rrows[:, 1:])
    assert (rows[:, 0] % 64 == 0).all()
    tiles = plan.export("paged_tiles")
    starts = sorted(set(int(x) for x in rows[:, 0]))
    for p, cs in enumerate(starts):
        for t in range(0, int(desc.ctx_len[p]), 64):
            assert tiles[(cs + t) // 64] == tables[p][t // bs] * bs + t % bs
    assert plan.info["visible_pairs"] == ref.info["visible_pairs"]
