"""CPU tests of the C-ABI library: it loads, exports every declared entry
point, builds plans whose integer fields equal the oracle's plan reference
exactly, and rejects malformed calls on the host with the documented status
(nothing is launched, so no GPU is needed)."""
import ctypes

import numpy as np
import pytest

import oracle
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth


def test_library_exports_every_declared_symbol():
    L = ta.lib()
    declared = ta.header_symbols()
    assert len(declared) == 34
    for name in declared:
        assert hasattr(L, name), name
    assert L.tree_attn_version().decode().startswith("tree_attn")


# --------------------------------------------------------------------------
# plan bit-exactness
# --------------------------------------------------------------------------

def check_prefill_plan(desc):
    plan = ta.plan_for(desc)
    ref = oracle.plan_prefill(desc)
    for f in ("position", "main_end", "branch_start", "pages", "branches"):
        got = plan.export(f)
        assert np.array_equal(got, ref[f].reshape(got.shape)), f
    info = plan.info
    assert info["n_rows"] == desc.total_tokens()
    assert info["visible_pairs"] == int((ref["position"] + 1).sum())
    assert info["max_depth"] == (int(ref["pages"][:, 3].max()) if len(ref["pages"]) else 0)
    # the work list covers every row exactly once
    work = plan.export("work")
    cover = np.zeros(desc.total_tokens(), np.int64)
    for w in work:
        cover[w[0]:w[0] + w[1]] += 1
    assert (cover == 1).all()
    check_backward_items(desc, plan)
    return plan


def check_backward_items(desc, plan):
    """Key-major items of the backward: every key lies in exactly one key
    tile, inside one page region (main stream or branch area), and every row
    that can see a key lies in one of its tile's row segments.  A tile whose
    walk is long comes as pieces with the same segments whose row-tile ranges
    partition the walk, each with its own partial slot (slots of a tile are
    consecutive); an unsplit tile has slot -1."""
    items = plan.export("bwd_work")
    T = desc.total_tokens()
    tiles = {}
    for w in items:
        tiles.setdefault((int(w[0]), int(w[1])), []).append(w)
    owner = np.full(T, -1, np.int64)
    first = {}
    slots = []
    for n, ((k0, nk), pieces) in enumerate(sorted(tiles.items())):
        assert 0 < nk <= 64
        assert (owner[k0:k0 + nk] == -1).all()
        owner[k0:k0 + nk] = n
        w0 = pieces[0]
        for w in pieces:
            assert np.array_equal(w[:9], w0[:9])
        n_rt = -(-(int(w0[4]) - int(w0[2])) // 64) + -(-(int(w0[6]) - int(w0[5])) // 64)
        pieces = sorted(pieces, key=lambda w: int(w[9]))
        assert [int(w[9]) for w in pieces] == [0] + [int(w[10]) for w in pieces[:-1]]
        assert int(pieces[-1][10]) == n_rt
        assert all(int(w[10]) - int(w[9]) <= 100 for w in pieces)
        if len(pieces) == 1:
            assert int(pieces[0][11]) == -1
        else:
            sl = [int(w[11]) for w in pieces]
            assert sl == list(range(sl[0], sl[0] + len(sl)))
            slots += sl
        first[n] = w0
    assert sorted(slots) == list(range(len(slots)))
    assert (owner >= 0).all()
    base = 0
    for p, sl in desc.page_slices():
        P = int(desc.prefix_len[p])
        L, C = desc.layout_len[sl], desc.content_len[sl]
        M, t = P + int(L.sum()), P + int(L.sum()) + int(C.sum())
        mask = oracle.ancestor_mask_page(P, L, C)
        keys = range(t) if t <= 2048 else range(0, t, 37)  # every key of small pages, a sample of large ones
        for j in keys:
            w = first[owner[base + j]]
            k0, nk, flags = int(w[0]), int(w[1]), int(w[8])
            in_branch = base + j >= base + M
            assert bool(flags & 2) == in_branch
            assert (k0 >= base + M) == in_branch and (k0 + nk <= base + M or in_branch)
            rows = base + np.nonzero(mask[:, j])[0]
            seg = ((rows >= w[2]) & (rows < w[4])) | ((rows >= w[5]) & (rows < w[6]))
            assert seg.all(), (p, j)
            # rows declared fully visible see this key
            full = np.r_[np.arange(w[3], w[4]), np.arange(w[7], w[6])]
            assert mask[full - base, j].all(), (p, j)
        base += t


def test_backward_long_walks_are_split():
    """The one-page workload's early main-stream key tiles are seen by more
    than 100 row tiles: their walks come as pieces with partial slots."""
    plan = ta.plan_for(synth.config2(with_tensors=False).desc)
    items = plan.export("bwd_work")
    split = items[items[:, 11] >= 0]
    assert len(split) > 0 and (split[:, 10] - split[:, 9] <= 100).all()
    assert ta.backward_scratch_bytes(plan, 16) >= 2 * 16 * 8772 * 4 + len(split) * 16 * 2 * 64 * 128 * 4


def test_prefill_plan_configs_exact():
    for cfg in (1, 2, 3):
        check_prefill_plan(synth.config(cfg, with_tensors=False).desc)


def test_config1_golden_depth_through_library():
    plan = ta.plan_for(synth.config1(with_tensors=False).desc)
    pages = plan.export("pages")
    assert pages.tolist() == [[0, 64 + 18, 128, 31, 64]]


@pytest.mark.parametrize("seed", range(12))
def test_prefill_plan_random_exact(seed):
    rng = np.random.default_rng(1000 + seed)
    n_pages = int(rng.integers(1, 4))
    P = rng.integers(0, 70, n_pages)
    N = rng.integers(0, 6, n_pages)
    L = [rng.integers(0, 5, n) for n in N]
    C = [rng.integers(0, 90, n) for n in N]
    desc = synth.make_prefill_desc(P, L, C)
    check_prefill_plan(desc)


def test_prefill_plan_edge_descriptions():
    for P, L, C in [(0, [0], [1]), (1, [], []), (0, [3, 0], [0, 0]), (64, [0, 0, 0], [64, 128, 1]),
                    (63, [1], [65])]:
        check_prefill_plan(synth.make_prefill_desc([P], [np.array(L)], [np.array(C)]))


def test_decode_plan_exact():
    for w in (synth.config4(with_tensors=False), synth.config4(with_tensors=False, n_pages=3, seed=9)):
        plan = ta.plan_for(w.desc)
        ref = oracle.plan_decode(w.desc)
        assert np.array_equal(plan.export("decode_rows"), ref["rows"])
        info = plan.info
        assert info["n_keys_a"] == int(w.desc.main_tokens().sum())
        assert info["n_keys_b"] == w.desc.suffix_tokens()


def check_decode_items(plan, desc):
    """Every visible (row, key) pair is covered by exactly one work item: main
    keys through segment A (key < row_a), suffix keys through segment B
    (key < row_b); no item reaches a key outside the row's stream."""
    rows = plan.export("decode_rows")
    work = plan.export("work")
    n = rows.shape[0]
    main_cov = [dict() for _ in range(n)]
    suf_cov = [dict() for _ in range(n)]
    for w in work:
        r0, nr, a_lo, a_full, a_hi, b_lo, b_hi = (int(x) for x in w[:7])
        for r in range(r0, r0 + nr):
            ms, ml, ss, sl = (int(x) for x in rows[r, :4])
            for key in range(a_lo, a_hi):
                if key < ms + ml:
                    assert key >= ms
                    main_cov[r][key] = main_cov[r].get(key, 0) + 1
                elif key < a_full:
                    raise AssertionError("a key past a row's bound is marked fully visible")
            for key in range(b_lo, min(b_hi, ss + sl)):
                assert key >= ss
                suf_cov[r][key] = suf_cov[r].get(key, 0) + 1
    for r in range(n):
        ms, ml, ss, sl = (int(x) for x in rows[r, :4])
        assert main_cov[r] == {k: 1 for k in range(ms, ms + ml)}, r
        assert suf_cov[r] == {k: 1 for k in range(ss, ss + sl)}, r


def test_decode_multi_plan_exact_and_covering():
    w = synth.decode_multi(with_tensors=False, n_pages=2)
    descs = [w.desc]
    rng = np.random.default_rng(4)
    for trial in range(6):
        n_pages = int(rng.integers(1, 4))
        N = rng.integers(0, 4, n_pages)
        L = rng.integers(0, 5, int(N.sum()))
        bp, br, s, kq = [], [], [], []
        for p in range(n_pages):
            for _ in range(int(rng.integers(0, 5))):
                bp.append(p)
                br.append(int(rng.integers(0, int(N[p]) + 1)))
                s.append(int(rng.integers(0, 3000 if trial % 2 else 40)))
                kq.append(int(rng.integers(1, 150 if trial == 3 else 10)))
        descs.append(synth.DecodeDesc(rng.integers(0, 1500, n_pages).astype(np.int32), N.astype(np.int32),
                                      L.astype(np.int32), np.array(bp, np.int32), np.array(br, np.int32),
                                      np.array(s, np.int32), np.array(kq, np.int32)))
    for desc in descs:
        plan = ta.plan_for(desc)
        ref = oracle.plan_decode(desc)
        assert np.array_equal(plan.export("decode_rows"), ref["rows"])
        info = plan.info
        assert info["n_rows"] == desc.n_rows()
        assert info["n_keys_b"] == desc.suffix_tokens()
        assert info["visible_pairs"] == int((ref["rows"][:, 1] + ref["rows"][:, 3]).sum())
        if desc is not descs[0]:
            check_decode_items(plan, desc)
    # a single-token multi plan is the plain decode plan
    w4 = synth.config4(with_tensors=False, n_pages=2)
    d = w4.desc
    a = ta.plan_decode(d.prefix_len, d.n_regions, d.layout_len, d.br_page, d.br_region, d.suffix_len)
    b = ta.plan_decode(d.prefix_len, d.n_regions, d.layout_len, d.br_page, d.br_region, d.suffix_len,
                       np.ones(d.n_branches, np.int32))
    for f in ("decode_rows", "work"):
        assert np.array_equal(a.export(f), b.export(f))


def test_verify_plan_exact():
    for w in (synth.config5(with_tensors=False), synth.config5(with_tensors=False, n_pages=3, seed=5)):
        plan = ta.plan_for(w.desc)
        ref = oracle.plan_verify(w.desc)
        assert np.array_equal(plan.export("verify_mask").astype(np.uint64), ref["mask"])
        assert np.array_equal(plan.export("verify_rows"), ref["rows"])
    # depth bound of the generator: no node deeper than 8 below the context
    assert plan.info["max_depth"] <= 8


def test_verify_plan_64_node_tree_uses_top_bit():
    parent = np.arange(-1, 63, dtype=np.int32)  # a chain of 64 nodes
    desc = synth.VerifyDesc(np.array([5], np.int32), np.array([0], np.int32), np.array([64], np.int32), parent)
    plan = ta.plan_for(desc)
    m = plan.export("verify_mask").astype(np.uint64)
    assert int(m[-1]) == (1 << 64) - 1
    assert np.array_equal(m, oracle.plan_verify(desc)["mask"])


# --------------------------------------------------------------------------
# host-side error paths
# --------------------------------------------------------------------------

def expect(code, fn, *a, **k):
    with pytest.raises(ta.TreeAttnError) as e:
        fn(*a, **k)
    assert e.value.code == code, str(e.value)


def test_plan_errors():
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_prefill, [-1], [0], [], [])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_prefill, [4], [1], [-2], [3])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_prefill, [4], [1], [2], [-3])
    expect(ta.TA_ERR_CAPACITY, ta.plan_prefill, [2**30, 2**30], [0, 0], [], [])
    # decode: region out of range, pages not grouped, negative suffix
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_decode, [4], [2], [1, 1], [0], [3], [0])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_decode, [4, 4], [1, 1], [1, 1], [1, 0], [1, 1], [0, 0])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_decode, [4], [1], [1], [0], [1], [-1])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_decode, [4], [1], [1], [1], [1], [0])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_decode, [4], [1], [1], [0], [-1], [0])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_decode, [4], [1], [1], [0], [1], [0], [0])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_decode, [4], [1], [1], [0, 0], [1, 0], [0, 0], [2, -1])
    # verify: parent not earlier, too many nodes, bad page
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_verify, [5], [0], [3], [-1, 2, 0])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_verify, [5], [0], [2], [-1, 1])
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_verify, [5], [0], [2], [-2, 0])
    expect(ta.TA_ERR_CAPACITY, ta.plan_verify, [5], [0], [65], [-1] * 65)
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_verify, [5], [1], [1], [-1])


class FakeArgs:
    """Aligned host addresses standing in for device pointers: every call
    below fails validation before anything dereferences them."""

    def __init__(self):
        self.buf = (ctypes.c_uint8 * 4096)()
        base = ctypes.addressof(self.buf)
        self.p = ctypes.c_void_p((base + 255) & ~255)
        self.odd = ctypes.c_void_p(((base + 255) & ~255) + 8)


def test_launch_errors_before_any_device_work():
    L = ta.lib()
    fa = FakeArgs()
    p = fa.p
    plan = ta.plan_prefill([8], [1], [2], [3])
    h = plan.handle
    bf, f32 = ta.TA_DTYPE_BF16, ta.TA_DTYPE_F32
    # (dtype, hq, hkv, d, scale) -> status
    cases = [
        ((7, 2, 1, 32, 0.2), ta.TA_ERR_UNSUPPORTED),
        ((bf, 3, 2, 32, 0.2), ta.TA_ERR_INVALID_ARG),
        ((bf, 0, 1, 32, 0.2), ta.TA_ERR_INVALID_ARG),
        ((bf, 6, 1, 32, 0.2), ta.TA_ERR_UNSUPPORTED),   # group 6 does not divide 32
        ((bf, 2, 1, 96, 0.2), ta.TA_ERR_UNSUPPORTED),
        ((bf, 2, 1, 32, 0.0), ta.TA_ERR_INVALID_ARG),
        ((bf, 2, 1, 32, float("nan")), ta.TA_ERR_INVALID_ARG),
        ((f32, 2, 1, 32, 0.2), ta.TA_ERR_STATE),        # valid, but never uploaded
    ]
    for (dt, hq, hkv, d, sc), code in cases:
        rc = L.tree_attn_prefill(h, dt, hq, hkv, d, sc, p, p, p, p, None, None, 0, None)
        assert rc == code, (dt, hq, hkv, d, sc, rc, ta.last_error())
    # NULL and misaligned tensors
    assert L.tree_attn_prefill(h, bf, 2, 1, 32, 0.2, None, p, p, p, None, None, 0, None) == ta.TA_ERR_INVALID_ARG
    assert L.tree_attn_prefill(h, bf, 2, 1, 32, 0.2, fa.odd, p, p, p, None, None, 0, None) == ta.TA_ERR_INVALID_ARG
    # wrong plan kind for the entry point
    assert L.tree_attn_verify(h, bf, 2, 1, 32, 0.2, p, p, p, p, p, p, None, None, 0, None) == ta.TA_ERR_STATE
    # workspace checks of upload happen before any copy
    assert L.tree_attn_plan_upload(h, None, 1 << 20, None) == ta.TA_ERR_WORKSPACE
    assert L.tree_attn_plan_upload(h, fa.odd, 1 << 20, None) == ta.TA_ERR_INVALID_ARG
    assert L.tree_attn_plan_upload(h, p, 16, None) == ta.TA_ERR_WORKSPACE


def test_decode_scratch_errors():
    L = ta.lib()
    fa = FakeArgs()
    p = fa.p
    plan = ta.plan_decode([10], [2], [1, 1], [0, 0], [1, 2], [3, 0])
    need = ta.scratch_bytes(plan, 4, 32)
    assert need > 0
    bf = ta.TA_DTYPE_BF16
    rc = L.tree_attn_decode(plan.handle, bf, 4, 2, 32, 0.2, p, p, p, p, p, p, None, None, need, None)
    assert rc == ta.TA_ERR_WORKSPACE
    rc = L.tree_attn_decode(plan.handle, bf, 4, 2, 32, 0.2, p, p, p, p, p, p, None, p, need - 1, None)
    assert rc == ta.TA_ERR_WORKSPACE
    rc = L.tree_attn_decode(plan.handle, bf, 4, 2, 32, 0.2, p, p, p, p, p, p, None, p, need, None)
    assert rc == ta.TA_ERR_STATE


def test_export_errors():
    plan = ta.plan_prefill([8], [1], [2], [3])
    with pytest.raises(ta.TreeAttnError) as e:
        ta.plan_export(plan, "verify_mask")
    assert e.value.code == ta.TA_ERR_INVALID_ARG


# --------------------------------------------------------------------------
# load balancing by key-range splits
# --------------------------------------------------------------------------

def _pieces_cover(plan, desc_rows):
    """Every row tile's key tiles are covered exactly once by its pieces, and
    split pieces own disjoint partial slots that the merge table lists."""
    work = plan.export("work")
    by_tile = {}
    for w in work:
        by_tile.setdefault((int(w[0]), int(w[1])), []).append(w)
    rows_split = 0
    slots = set()
    for (row0, nrows), pieces in by_tile.items():
        pieces.sort(key=lambda w: w[8])
        assert pieces[0][8] == 0
        for a, b in zip(pieces, pieces[1:]):
            assert a[9] == b[8]
        na = (pieces[0][4] - pieces[0][2] + 63) // 64
        nb = (pieces[0][6] - pieces[0][5] + 63) // 64
        assert pieces[-1][9] == na + nb
        if len(pieces) > 1:
            rows_split += nrows
            for w in pieces:
                assert w[7] >= 0
                for t in range(nrows):
                    assert w[7] + t not in slots
                    slots.add(int(w[7] + t))
        else:
            assert pieces[0][7] == -1
    return rows_split, len(slots)


def test_balance_splits_the_one_page_prefill():
    w = synth.config2(with_tensors=False)
    plan = ta.plan_for(w.desc)
    before = plan.export("work").shape[0]
    plan.balance(8, 512)
    info = plan.info
    assert plan.export("work").shape[0] > before
    rows_split, n_slots = _pieces_cover(plan, w.desc.total_tokens())
    assert rows_split > 0 and info["n_partials"] == n_slots
    assert ta.scratch_bytes(plan, 16, 128) > 0
    # the integer contract is unchanged by balancing
    ref = oracle.plan_prefill(w.desc)
    assert np.array_equal(plan.export("main_end"), ref["main_end"])


def test_balance_leaves_balanced_plans_alone():
    w = synth.config3(with_tensors=False)
    plan = ta.plan_for(w.desc)
    before = plan.export("work")
    plan.balance(8, 512)
    assert plan.info["n_partials"] == 0
    assert np.array_equal(plan.export("work"), before)


def test_balance_errors():
    plan = ta.plan_for(synth.config2(with_tensors=False).desc)
    expect(ta.TA_ERR_INVALID_ARG, ta.plan_balance, plan, 0, 512)
    plan.balance(8, 512)
    assert plan.info["n_partials"] > 0
    expect(ta.TA_ERR_STATE, ta.plan_balance, plan, 8, 512)
    d = ta.plan_decode([10], [1], [1], [0], [1], [3])
    d.balance(8, 512)           # no-op for decode


def test_decode_items_mark_segments_that_several_row_groups_read():
    """Decode copies stream past the caches unless other items read the same
    keys: a page with more than one row group marks its main chunks (flag 4),
    a branch with more than one group of new tokens its suffix chunks (8)."""
    # page 0: 3 branches x 30 new tokens = 90 rows (two row groups);
    # page 1: branch 3 has 70 new tokens (two groups of rows and of suffix keys);
    # page 2: two single-token branches (one group, nothing shared)
    desc = synth.DecodeDesc(np.array([500, 300, 200], np.int32), np.array([2, 2, 1], np.int32),
                            np.array([20, 30, 10, 10, 7], np.int32),
                            np.array([0, 0, 0, 1, 1, 2, 2], np.int32), np.array([0, 1, 2, 1, 2, 0, 1], np.int32),
                            np.array([40, 50, 0, 90, 5, 3, 9], np.int32),
                            n_query=np.array([30, 30, 30, 70, 1, 1, 1], np.int32))
    plan = ta.plan_for(desc)
    check_decode_items(plan, desc)
    work = plan.export("work")
    row_page = np.repeat(desc.br_page, desc.n_query)
    row_branch = np.repeat(np.arange(len(desc.br_page)), desc.n_query)
    seen = set()
    for w in work:
        r0, nr, a_lo, a_hi, b_lo, b_hi, flags = (int(w[i]) for i in (0, 1, 2, 4, 5, 6, 10))
        if a_hi > a_lo:
            page = int(row_page[r0])
            assert bool(flags & 4) == (page < 2), (page, flags)
            seen.add(("main", page))
        else:
            assert b_hi > b_lo
            br = int(row_branch[r0])
            assert bool(flags & 8) == (br == 3), (br, flags)
            seen.add(("suffix", br))
        assert not flags & ~(1 | 4 | 8)
    assert {("main", 0), ("main", 1), ("main", 2), ("suffix", 3), ("suffix", 4), ("suffix", 6)} <= seen
    # the single-token decode workload: nothing is marked
    w1 = synth.config4(with_tensors=False)
    for w in ta.plan_for(w1.desc).export("work"):
        assert int(w[10]) & (4 | 8) == 0


def test_backward_scratch_checks_with_split_key_walks():
    """The backward needs two fp32 values per (query head, row) plus the fp32
    partial dK, dV of every piece of a split key walk; one byte less is a
    WORKSPACE error, checked before the plan's upload state."""
    L = ta.lib()
    fa = FakeArgs()
    p = fa.p
    plan = ta.plan_for(synth.config2(with_tensors=False).desc)
    rows = plan.info["n_rows"]
    n_kpart = int((plan.export("bwd_work")[:, 11] >= 0).sum())
    assert n_kpart > 0
    hq, hkv, d = 16, 8, 128
    half = -(-rows * hq * 4 // 256) * 256
    need = 2 * half + n_kpart * hkv * 2 * 64 * d * 4
    assert ta.backward_scratch_bytes(plan, hq) >= need
    bf = ta.TA_DTYPE_BF16

    def call(nbytes):
        return L.tree_attn_prefill_backward(plan.handle, bf, hq, hkv, d, 0.088, p, p, p, p, p, p, p, p, p, p,
                                            nbytes, None)

    assert call(need - 1) == ta.TA_ERR_WORKSPACE
    assert call(need) == ta.TA_ERR_STATE  # valid, but never uploaded


@pytest.mark.parametrize("which", ["prefill", "prefill_balanced", "decode", "decode_multi", "verify"])
def test_device_image_tables_equal_the_oracle_plan(which):
    """The packed image that tree_attn_plan_upload copies holds, per row, the
    bounds the oracle's plan defines, and the exported work list."""
    import plan_image
    if which.startswith("prefill"):
        desc = synth.make_prefill_desc([200, 0, 65], [np.array([3, 0, 5, 2, 1]), np.array([4]), np.array([])],
                                       [np.array([70, 0, 9, 130, 1]), np.array([3]), np.array([])])
        plan = ta.plan_for(desc)
        if which == "prefill_balanced":
            plan.balance(8, 64)
    elif which == "decode":
        desc = synth.config4(with_tensors=False, n_pages=3).desc
        plan = ta.plan_for(desc)
    elif which == "decode_multi":
        desc = synth.decode_multi(with_tensors=False, n_pages=2).desc
        plan = ta.plan_for(desc)
    else:
        desc = synth.config5(with_tensors=False, n_pages=4).desc
        plan = ta.plan_for(desc)
    image = plan.export("device_image").view(np.uint8)
    plan_image.check_against_oracle(plan, desc, image)
