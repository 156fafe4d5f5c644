"""Pins for the fp64 oracle: checks against things the pages and mathematics
fix, not against the oracle's own formulas.

* closed form: one branch with an empty layout is plain causal attention,
  and every branch equals causal attention over its own virtual sequence
  [X, B_<=k, Y_k] assembled by concatenation (PaDoc paper summary, "Training
  paradigm"); checked with torch's SDPA routine in float64;
* library routine: dense masked SDPA with a mask built here by slicing;
* invariant: perturbing non-ancestor tokens leaves a row bit-identical;
* brute force: every tiny page description against a per-pair Python loop
  over ancestor sets written as label sets;
* hand-worked golden fixtures (tests/golden);
* depth formulas (same page, "Formal assumptions and factorization");
* closed forms: q = 0 gives lse = ln |Anc(i)|, constant V gives O = V;
* LSE merge of disjoint key sets equals attention over their union;
* cross-entry identities: decode == prefill row, chain verify == causal.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tree_structured_attention_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def sdpa64(q, k, v, *, causal=False, mask=None, scale=None):
    """torch SDPA in float64 with GQA by repetition; q [T,Hq,d], k/v [S,Hkv,d]."""
    q = torch.as_tensor(np.asarray(q, np.float64))
    k = torch.as_tensor(np.asarray(k, np.float64))
    v = torch.as_tensor(np.asarray(v, np.float64))
    g = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    am = None if mask is None else torch.as_tensor(mask)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                       attn_mask=am, is_causal=causal, scale=scale)
    return o.transpose(0, 1).numpy()


def rand(rng, *shape):
    return rng.standard_normal(shape)


def virtual_index_lists(P, L, C):
    """Packed indices of each branch's virtual sequence [X, B_<=k, Y_k], built
    by slicing the packed order [X | B_1..B_N | Y_1..Y_N]."""
    M = P + sum(L)
    out = []
    lay_end = P
    con_start = M
    for lk, ck in zip(L, C):
        lay_end += lk
        idx = list(range(0, lay_end)) + list(range(con_start, con_start + ck))
        out.append((idx, ck))
        con_start += ck
    return out


def mask_by_slicing(P, L, C):
    M = P + sum(L)
    T = M + sum(C)
    m = np.zeros((T, T), bool)
    for i in range(M):
        m[i, : i + 1] = True
    for idx, ck in virtual_index_lists(P, L, C):
        head = idx[: len(idx) - ck]
        for t in range(ck):
            row = idx[len(idx) - ck + t]
            m[row, head] = True
            m[row, idx[len(idx) - ck: len(idx) - ck + t + 1]] = True
    return m


def one_page(P, L, C):
    return synth.make_prefill_desc([P], [np.array(L)], [np.array(C)])


# --------------------------------------------------------------------------
# closed forms vs. library causal attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("P,C", [(7, 5), (0, 9), (13, 1), (1, 0)])
def test_single_branch_empty_layout_is_causal(P, C):
    rng = np.random.default_rng(P * 31 + C)
    T = P + C
    q, k, v = rand(rng, T, 4, 8), rand(rng, T, 2, 8), rand(rng, T, 2, 8)
    o, _ = oracle.prefill(one_page(P, [0], [C]), q, k, v, 0.37)
    ref = sdpa64(q, k, v, causal=True, scale=0.37)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_no_regions_is_causal_over_prefix():
    rng = np.random.default_rng(5)
    q, k, v = rand(rng, 11, 2, 4), rand(rng, 11, 1, 4), rand(rng, 11, 1, 4)
    o, _ = oracle.prefill(synth.make_prefill_desc([11], [np.array([])], [np.array([])]), q, k, v, 0.5)
    assert np.max(np.abs(o - sdpa64(q, k, v, causal=True, scale=0.5))) < 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_every_branch_is_causal_over_its_virtual_sequence(seed):
    rng = np.random.default_rng(100 + seed)
    P = int(rng.integers(0, 9))
    N = int(rng.integers(1, 5))
    L = [int(x) for x in rng.integers(0, 4, N)]
    C = [int(x) for x in rng.integers(0, 7, N)]
    T = P + sum(L) + sum(C)
    q, k, v = rand(rng, T, 4, 8), rand(rng, T, 2, 8), rand(rng, T, 2, 8)
    o, _ = oracle.prefill(one_page(P, L, C), q, k, v, 0.3)
    M = P + sum(L)
    # main stream: plain causal attention over [X | B]
    ref_main = sdpa64(q[:M], k[:M], v[:M], causal=True, scale=0.3)
    assert np.max(np.abs(o[:M] - ref_main)) < 1e-12 if M else True
    for idx, ck in virtual_index_lists(P, L, C):
        if ck == 0:
            continue
        ref = sdpa64(q[idx], k[idx], v[idx], causal=True, scale=0.3)
        assert np.max(np.abs(o[idx[-ck:]] - ref[-ck:])) < 1e-12


def test_matches_dense_masked_sdpa_multi_page():
    rng = np.random.default_rng(7)
    pages = [(5, [2, 0, 3], [4, 0, 2]), (0, [1], [3]), (3, [], [])]
    desc = synth.make_prefill_desc([p[0] for p in pages], [np.array(p[1]) for p in pages],
                                   [np.array(p[2]) for p in pages])
    T = desc.total_tokens()
    q, k, v = rand(rng, T, 6, 16), rand(rng, T, 3, 16), rand(rng, T, 3, 16)
    o, lse = oracle.prefill(desc, q, k, v, 0.25)
    base = 0
    for P, L, C in pages:
        t = P + sum(L) + sum(C)
        sl = slice(base, base + t)
        m = mask_by_slicing(P, L, C)
        ref = sdpa64(q[sl], k[sl], v[sl], mask=m, scale=0.25)
        assert np.max(np.abs(o[sl] - ref)) < 1e-12
        base += t


# --------------------------------------------------------------------------
# hand-worked fixtures
# --------------------------------------------------------------------------

def read_fixture(name):
    rows = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows.setdefault(key, []).append(vals)
    return rows


def test_golden_tiny_page_mask():
    fx = read_fixture("tiny_page_mask.txt")
    P = int(fx["prefix"][0][0])
    L = [int(x) for x in fx["layout"][0]]
    C = [int(x) for x in fx["content"][0]]
    want = np.array([[c == "1" for c in r[0]] for r in fx["mask"]])
    assert (oracle.ancestor_mask_page(P, L, C) == want).all()
    plan = oracle.plan_prefill(one_page(P, L, C))
    assert plan["position"].tolist() == [int(x) for x in fx["position"][0]]
    assert oracle.depth(P, L, C) == (int(fx["depth"][0][0]), int(fx["depth_seq"][0][0]))


def test_golden_tiny_tree_mask():
    fx = read_fixture("tiny_tree_mask.txt")
    parent = [int(x) for x in fx["parent"][0]]
    want = [int(x) for x in fx["mask"][0]]
    a = oracle.tree_ancestor_mask(parent)
    got = [sum(1 << j for j in range(len(parent)) if a[i, j]) for i in range(len(parent))]
    assert got == want
    desc = synth.VerifyDesc(np.array([10], np.int32), np.array([0], np.int32),
                            np.array([len(parent)], np.int32), np.array(parent, np.int32))
    plan = oracle.plan_verify(desc)
    assert plan["mask"].astype(np.int64).tolist() == want
    assert plan["rows"][:, 3].tolist() == [10 + int(d) for d in fx["depth"][0]]


# --------------------------------------------------------------------------
# depth formulas
# --------------------------------------------------------------------------

def test_depth_golden_config1():
    # synth config 1 seed 0 draws C = [18, 15, 13]; L = 6 each.
    w = synth.config1(with_tensors=False)
    assert w.desc.content_len.tolist() == [18, 15, 13]
    # by hand: D = max(6+18, 12+15, 18+13) = 31; D_seq = 18 + 46 = 64
    assert oracle.depth(64, [6, 6, 6], [18, 15, 13]) == (31, 64)


def test_depth_special_cases():
    assert oracle.depth(5, [], []) == (0, 0)
    assert oracle.depth(0, [4], [0]) == (4, 4)          # empty branch still counts its layout
    assert oracle.depth(9, [1, 1, 1], [10, 0, 0]) == (11, 13)
    # a single region: the parallel depth equals the sequential one
    assert oracle.depth(3, [5], [7]) == (12, 12)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_nonancestor_perturbation_bit_identical():
    rng = np.random.default_rng(11)
    pages = [(6, [2, 3, 1], [5, 4, 6]), (4, [1, 2], [3, 3])]
    desc = synth.make_prefill_desc([p[0] for p in pages], [np.array(p[1]) for p in pages],
                                   [np.array(p[2]) for p in pages])
    T = desc.total_tokens()
    q, k, v = rand(rng, T, 4, 8), rand(rng, T, 2, 8), rand(rng, T, 2, 8)
    o0, l0 = oracle.prefill(desc, q, k, v, 0.4)
    masks = [mask_by_slicing(*p) for p in pages]
    base = 0
    for (P, L, C), m in zip(pages, masks):
        t = P + sum(L) + sum(C)
        for r in rng.choice(t, 6, replace=False):
            r = int(r)
            anc = np.zeros(T, bool)
            anc[base:base + t] = m[r]
            non = ~anc
            for fill_v in (1e30, None):
                q2, k2, v2 = q.copy(), k.copy(), v.copy()
                others = np.flatnonzero(non)
                others = others[others != base + r]
                q2[others] = np.nan
                k2[non] = np.nan
                v2[non] = rand(rng, int(non.sum()), 2, 8) if fill_v is None else fill_v
                o1, l1 = oracle.prefill(desc, q2, k2, v2, 0.4)
                assert np.array_equal(o1[base + r], o0[base + r])
                assert np.array_equal(l1[:, base + r], l0[:, base + r])
        base += t


def test_zero_query_lse_counts_ancestors():
    # q = 0 makes every visible score 0, so lse_i = ln |Anc(i)| exactly, and
    # |Anc(i)| = i + 1 (main) or P + L_<=k + t + 1 (content token Y_k[t]).
    P, L, C = 9, [3, 0, 2, 4], [5, 2, 0, 7]
    rng = np.random.default_rng(3)
    T = P + sum(L) + sum(C)
    q = np.zeros((T, 2, 4))
    k, v = rand(rng, T, 1, 4), rand(rng, T, 1, 4)
    _, lse = oracle.prefill(one_page(P, L, C), q, k, v, 1.0)
    M = P + sum(L)
    want = list(range(1, M + 1))
    acc = P
    for lk, ck in zip(L, C):
        acc += lk
        want += [acc + t + 1 for t in range(ck)]
    assert np.allclose(np.exp(lse[0]), want, rtol=1e-13, atol=0)
    assert np.allclose(np.exp(lse[1]), want, rtol=1e-13, atol=0)


def test_constant_v_gives_v():
    P, L, C = 5, [2, 2], [3, 4]
    rng = np.random.default_rng(4)
    T = P + sum(L) + sum(C)
    q, k = rand(rng, T, 2, 4), rand(rng, T, 2, 4)
    v = np.broadcast_to(np.array([1.5, -2.0, 0.25, 7.0]), (T, 2, 4)).copy()
    o, _ = oracle.prefill(one_page(P, L, C), q, k, v, 0.9)
    assert np.allclose(o, v, rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# brute force over every tiny description
# --------------------------------------------------------------------------

def _brute_page(P, L, C, q, k, v, scale):
    """Per-pair loop; ancestor sets as sets of labels ('X', i) / ('B', k, u) /
    ('Y', k, u), in packed order."""
    labels = [("X", i) for i in range(P)]
    for kk, lk in enumerate(L, 1):
        labels += [("B", kk, u) for u in range(lk)]
    for kk, ck in enumerate(C, 1):
        labels += [("Y", kk, u) for u in range(ck)]
    T = len(labels)
    main_order = [i for i, lab in enumerate(labels) if lab[0] != "Y"]

    def anc(i):
        lab = labels[i]
        if lab[0] != "Y":
            return set(main_order[: main_order.index(i) + 1])
        _, kk, t = lab
        s = {j for j, b in enumerate(labels) if b[0] == "X" or (b[0] == "B" and b[1] <= kk)}
        s |= {j for j, b in enumerate(labels) if b[0] == "Y" and b[1] == kk and b[2] <= t}
        return s

    hq, hkv, d = q.shape[1], k.shape[1], q.shape[2]
    o = np.zeros((T, hq, d))
    for i in range(T):
        a = sorted(anc(i))
        for h in range(hq):
            g = h // (hq // hkv)
            sc = [scale * sum(q[i, h, x] * k[j, g, x] for x in range(d)) for j in a]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            z = sum(w)
            for x in range(d):
                o[i, h, x] = sum(wj * v[j, g, x] for wj, j in zip(w, a)) / z
    return o


def test_brute_force_all_tiny_descriptions():
    rng = np.random.default_rng(21)
    cases = 0
    for P in range(0, 3):
        for N in range(0, 3):
            for L in itertools.product(range(0, 3), repeat=N):
                for C in itertools.product(range(0, 3), repeat=N):
                    T = P + sum(L) + sum(C)
                    if T == 0:
                        continue
                    q, k, v = rand(rng, T, 2, 3), rand(rng, T, 1, 3), rand(rng, T, 1, 3)
                    o, _ = oracle.prefill(one_page(P, list(L), list(C)), q, k, v, 0.7)
                    ref = _brute_page(P, list(L), list(C), q, k, v, 0.7)
                    assert np.max(np.abs(o - ref)) < 1e-12, (P, L, C)
                    cases += 1
    assert cases > 100


# --------------------------------------------------------------------------
# plan fields vs. the visibility definition
# --------------------------------------------------------------------------

def test_plan_prefill_fields_reproduce_mask():
    pages = [(4, [1, 0, 2], [3, 2, 0]), (0, [2], [4]), (5, [], [])]
    desc = synth.make_prefill_desc([p[0] for p in pages], [np.array(p[1]) for p in pages],
                                   [np.array(p[2]) for p in pages])
    plan = oracle.plan_prefill(desc)
    base = 0
    for pi, (P, L, C) in enumerate(pages):
        t = P + sum(L) + sum(C)
        m = mask_by_slicing(P, L, C)
        for r in range(t):
            row = base + r
            vis = np.zeros(t, bool)
            vis[: plan["main_end"][row] - base] = True
            vis[plan["branch_start"][row] - base: r + 1] = True
            assert (vis == m[r]).all()
            assert plan["position"][row] == m[r].sum() - 1
        assert plan["pages"][pi, :3].tolist() == [base, P + sum(L), t]
        assert tuple(plan["pages"][pi, 3:]) == oracle.depth(P, L, C)
        base += t


# --------------------------------------------------------------------------
# cascade decomposition and cross-entry identities
# --------------------------------------------------------------------------

def test_lse_merge_of_disjoint_key_sets():
    rng = np.random.default_rng(8)
    q, k, v = rand(rng, 3, 4, 8), rand(rng, 40, 2, 8), rand(rng, 40, 2, 8)
    full = oracle.masked_attention(q, k, v, np.ones((3, 40), bool), 0.3)
    parts = [oracle.masked_attention(q, k[a:b], v[a:b], np.ones((3, b - a), bool), 0.3)
             for a, b in [(0, 7), (7, 31), (31, 40)]]
    o, lse = oracle.lse_merge(parts)
    assert np.max(np.abs(o - full[0])) < 1e-13
    assert np.max(np.abs(lse - full[1])) < 1e-13


def test_decode_equals_prefill_row():
    """A branch row served as a request over [shared main | own suffix] equals
    the packed prefill row of the same token (PaDoc summary, "Inference")."""
    rng = np.random.default_rng(9)
    P, L = 6, [2, 3, 1]
    s = [4, 0, 2]          # tokens already in each branch
    C = [x + 1 for x in s]  # the current token is the last of each branch
    T = P + sum(L) + sum(C)
    M = P + sum(L)
    q, k, v = rand(rng, T, 4, 8), rand(rng, T, 2, 8), rand(rng, T, 2, 8)
    o_pf, l_pf = oracle.prefill(one_page(P, L, C), q, k, v, 0.35)
    ddesc = synth.DecodeDesc(np.array([P], np.int32), np.array([3], np.int32), np.array(L, np.int32),
                             np.zeros(3, np.int32), np.array([1, 2, 3], np.int32), np.array(s, np.int32))
    rows = [M + sum(C[:i]) + s[i] for i in range(3)]
    o_dc, l_dc = oracle.decode(ddesc, q[rows], k[:M], v[:M], k[M:], v[M:], 0.35)
    assert np.max(np.abs(o_dc - o_pf[rows])) < 1e-12
    assert np.max(np.abs(l_dc - l_pf[:, rows])) < 1e-12
    plan = oracle.plan_decode(ddesc)
    assert plan["rows"][:, 4].tolist() == oracle.plan_prefill(one_page(P, L, C))["position"][rows].tolist()


def test_multi_token_decode_equals_prefill_rows():
    """K new tokens per branch (a P-MTP window, or a branch's first tokens
    prefilled over the cached prefix) served over [shared main | own suffix]
    equal the packed prefill rows of the same tokens; a layout-stream row
    (region 0) over a page whose last layout region is still being written
    equals the prefill rows of that region (PaDoc summary, "Inference": the
    layout stream and the content streams are separate requests over the
    shared prefix)."""
    rng = np.random.default_rng(19)
    P, L = 5, [2, 3, 4]
    C = [6, 1, 5]
    s = [2, 0, 1]                       # tokens already in each branch
    K = [C[i] - s[i] for i in range(3)]  # the rest of each branch is new
    T = P + sum(L) + sum(C)
    M = P + sum(L)
    q, k, v = rand(rng, T, 4, 8), rand(rng, T, 2, 8), rand(rng, T, 2, 8)
    o_pf, l_pf = oracle.prefill(one_page(P, L, C), q, k, v, 0.35)
    pos_pf = oracle.plan_prefill(one_page(P, L, C))["position"]
    # content branches: decode rows are prefill rows [start_k + s_k, end_k)
    ddesc = synth.DecodeDesc(np.array([P], np.int32), np.array([3], np.int32), np.array(L, np.int32),
                             np.zeros(3, np.int32), np.array([1, 2, 3], np.int32), np.array(s, np.int32),
                             np.array(K, np.int32))
    rows = [M + sum(C[:i]) + s[i] + j for i in range(3) for j in range(K[i])]
    o_dc, l_dc = oracle.decode(ddesc, q[rows], k[:M], v[:M], k[M:], v[M:], 0.35)
    assert np.max(np.abs(o_dc - o_pf[rows])) < 1e-12
    assert np.max(np.abs(l_dc - l_pf[:, rows])) < 1e-12
    assert oracle.plan_decode(ddesc)["rows"][:, 4].tolist() == pos_pf[rows].tolist()
    # layout stream: main = X, B_1, B_2; B_3 is its private suffix, 1 token
    # already written and 3 new ones
    M2 = P + L[0] + L[1]
    ldesc = synth.DecodeDesc(np.array([P], np.int32), np.array([2], np.int32), np.array(L[:2], np.int32),
                             np.zeros(1, np.int32), np.zeros(1, np.int32), np.array([1], np.int32),
                             np.array([3], np.int32))
    rows = [M2 + 1 + j for j in range(3)]
    o_ly, l_ly = oracle.decode(ldesc, q[rows], k[:M2], v[:M2], k[M2:M], v[M2:M], 0.35)
    assert np.max(np.abs(o_ly - o_pf[rows])) < 1e-12
    assert np.max(np.abs(l_ly - l_pf[:, rows])) < 1e-12
    assert oracle.plan_decode(ldesc)["rows"][:, 4].tolist() == pos_pf[rows].tolist()


def test_chain_verify_is_causal():
    """A chain tree (parent = previous node) under the tree ancestor mask is
    causal attention over [context | nodes] (HSD notes, key design 3 (b))."""
    rng = np.random.default_rng(10)
    ctx, n = 13, 6
    desc = synth.VerifyDesc(np.array([ctx], np.int32), np.array([0], np.int32), np.array([n], np.int32),
                            np.arange(-1, n - 1, dtype=np.int32))
    q = rand(rng, n, 4, 8)
    kc, vc = rand(rng, ctx, 2, 8), rand(rng, ctx, 2, 8)
    kt, vt = rand(rng, n, 2, 8), rand(rng, n, 2, 8)
    o, _ = oracle.verify(desc, q, kc, vc, kt, vt, 0.3)
    qq = np.concatenate([np.zeros((ctx, 4, 8)), q])
    ref = sdpa64(qq, np.concatenate([kc, kt]), np.concatenate([vc, vt]), causal=True, scale=0.3)
    assert np.max(np.abs(o - ref[ctx:])) < 1e-12


def test_verify_branches_are_isolated_and_match_sdpa():
    rng = np.random.default_rng(12)
    parents = [np.array([-1, 0, 0, 1, 2, 2, 4]), np.array([-1, 0, 1]), np.array([-1])]
    desc = synth.VerifyDesc(np.array([9, 5], np.int32), np.array([0, 0, 1], np.int32),
                            np.array([7, 3, 1], np.int32), np.concatenate(parents).astype(np.int32))
    n = 11
    q = rand(rng, n, 2, 8)
    kc, vc = rand(rng, 14, 1, 8), rand(rng, 14, 1, 8)
    kt, vt = rand(rng, n, 1, 8), rand(rng, n, 1, 8)
    o, _ = oracle.verify(desc, q, kc, vc, kt, vt, 0.5)
    # node by node: visible keys = own page context + ancestor path (itself included)
    node_off = [0, 7, 10, 11]
    ctx_off = [0, 9, 14]
    for b, par in enumerate(parents):
        p = int(desc.br_page[b])
        for i in range(len(par)):
            path = []
            j = i
            while j >= 0:
                path.append(node_off[b] + j)
                j = int(par[j])
            kk = np.concatenate([kc[ctx_off[p]:ctx_off[p + 1]], kt[path]])
            vv = np.concatenate([vc[ctx_off[p]:ctx_off[p + 1]], vt[path]])
            ref = sdpa64(q[node_off[b] + i:node_off[b] + i + 1], kk, vv, scale=0.5)
            assert np.max(np.abs(o[node_off[b] + i] - ref[0])) < 1e-12


# --------------------------------------------------------------------------
# backward of the packed forward (the training path)
# --------------------------------------------------------------------------

def test_backward_matches_central_differences():
    """Gradients of loss = sum(o * w) by central differences of the forward
    (a property of the forward alone: no formula of the backward is used)."""
    rng = np.random.default_rng(11)
    desc = one_page(3, [2, 1], [3, 2])  # 11 tokens, two branches
    T = desc.total_tokens()
    q, k, v = rand(rng, T, 2, 4), rand(rng, T, 1, 4), rand(rng, T, 1, 4)
    w = rand(rng, T, 2, 4)
    scale = 0.7
    dq, dk, dv = oracle.prefill_backward(desc, q, k, v, w, scale)

    def loss(qq, kk, vv):
        return float((oracle.prefill(desc, qq, kk, vv, scale)[0] * w).sum())

    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{"qq": args_p["q"], "kk": args_p["k"], "vv": args_p["v"]})
                        - loss(**{"qq": args_m["q"], "kk": args_m["k"], "vv": args_m["v"]})) / (2 * eps)
        assert np.max(np.abs(num - g)) < 1e-7, name


def test_backward_matches_autograd_of_dense_masked_sdpa():
    """torch autograd through the library SDPA routine (float64, mask built
    by slicing, GQA by repeating KV heads) gives the same gradients."""
    rng = np.random.default_rng(12)
    pages = [(5, [2, 0, 3], [4, 0, 2]), (0, [1], [3]), (3, [], [])]
    desc = synth.make_prefill_desc([p[0] for p in pages], [np.array(p[1]) for p in pages],
                                   [np.array(p[2]) for p in pages])
    T = desc.total_tokens()
    q, k, v, do = rand(rng, T, 4, 8), rand(rng, T, 2, 8), rand(rng, T, 2, 8), rand(rng, T, 4, 8)
    dq, dk, dv = oracle.prefill_backward(desc, q, k, v, do, 0.3)
    base = 0
    for P, L, C in pages:
        t = P + sum(L) + sum(C)
        sl = slice(base, base + t)
        qt = torch.tensor(q[sl], requires_grad=True)
        kt = torch.tensor(k[sl], requires_grad=True)
        vt = torch.tensor(v[sl], requires_grad=True)
        o = F.scaled_dot_product_attention(qt.transpose(0, 1), kt.repeat_interleave(2, dim=1).transpose(0, 1),
                                           vt.repeat_interleave(2, dim=1).transpose(0, 1),
                                           attn_mask=torch.as_tensor(mask_by_slicing(P, L, C)), scale=0.3)
        o.transpose(0, 1).backward(torch.tensor(do[sl]))
        assert np.max(np.abs(qt.grad.numpy() - dq[sl])) < 1e-11
        assert np.max(np.abs(kt.grad.numpy() - dk[sl])) < 1e-11
        assert np.max(np.abs(vt.grad.numpy() - dv[sl])) < 1e-11
        base += t


def test_backward_pages_and_unseen_keys_get_no_gradient():
    """An output gradient on one page moves nothing on another page, and a
    key no row with a non-zero output gradient can see gets exactly zero."""
    rng = np.random.default_rng(13)
    desc = synth.make_prefill_desc([4, 6], [np.array([2, 2]), np.array([1])], [np.array([3, 1]), np.array([5])])
    T = desc.total_tokens()
    t0 = 4 + 4 + 4  # tokens of page 0
    q, k, v = rand(rng, T, 2, 8), rand(rng, T, 2, 8), rand(rng, T, 2, 8)
    do = rand(rng, T, 2, 8)
    do[t0:] = 0.0
    # only the first branch's rows of page 0 carry a gradient: rows 8..10
    # (branch 1 content); they see X (0..3), B_1 (4..5) and themselves
    do[:8] = 0.0
    do[11] = 0.0
    dq, dk, dv = oracle.prefill_backward(desc, q, k, v, do, 0.5)
    assert np.all(dq[t0:] == 0) and np.all(dk[t0:] == 0) and np.all(dv[t0:] == 0)
    unseen = [6, 7, 11]  # B_2 and the second branch's content
    assert np.all(dk[unseen] == 0) and np.all(dv[unseen] == 0)
    assert np.all(np.abs(dv[[0, 1, 2, 3, 4, 5, 8, 9, 10]]).sum(axis=(1, 2)) > 0)


def test_sampled_backward_equals_full_backward():
    """The row/column-at-a-time oracle used on large pages equals the dense
    one on pages small enough for both."""
    rng = np.random.default_rng(14)
    pages = [(9, [2, 0, 3], [5, 0, 4]), (4, [1], [6])]
    desc = synth.make_prefill_desc([p[0] for p in pages], [np.array(p[1]) for p in pages],
                                   [np.array(p[2]) for p in pages])
    T = desc.total_tokens()
    q, k, v, do = rand(rng, T, 4, 8), rand(rng, T, 2, 8), rand(rng, T, 2, 8), rand(rng, T, 4, 8)
    dq, dk, dv = oracle.prefill_backward(desc, q, k, v, do, 0.4)
    rows = [0, 5, 13, 20, 23, T - 1]
    keys = [1, 9, 14, 18, 27, T - 2]
    sq, sk, sv = oracle.prefill_backward_sampled(desc, q, k, v, do, 0.4, rows, keys)
    assert np.max(np.abs(sq - dq[rows])) < 1e-12
    assert np.max(np.abs(sk - dk[keys])) < 1e-12
    assert np.max(np.abs(sv - dv[keys])) < 1e-12
