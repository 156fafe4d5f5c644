"""GPU invariant: a row's output depends only on its ancestors.

Every query row keeps bit-identical outputs (o and lse) when every token
outside its ancestor set changes, for all three entry points:
  prefill  Anc(B_k) = {X, B_<k} (causal main stream) and
           Anc(Y_k) = {X, B_<=k} plus Y_k causally ("PaDoc: Layout-Grounded
           Parallel Decoding for Document Parsing", paper summary, "Training
           paradigm");
  decode   the page's main stream up to the branch's bound plus the
           branch's own suffix (PaDoc summary, "Inference": request-level
           serving gives the same visibility);
  verify   the page's context plus the node's own ancestor path ("HSD"
           notes, key design 3 (b), tree ancestor mask).
Ancestor sets come from the oracle's plan functions (the library's own plan
is not consulted).

What changes: q of every other row and k of every non-ancestor key become
NaN, +-1e30 or large fresh noise (40 N(0,1), scores far beyond the range a
row's softmax base tracks); v of non-ancestor keys that may share a 64-key
tile with keys another row of the same work item needs becomes +-1e30 or
fresh noise, and every other v (other pages, other branches' suffixes,
other pages' trees) becomes NaN.  A NaN v of a key in a tile another row
needs would reach this row through 0 * NaN in the PV product, the one
documented exception.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth

pytestmark = pytest.mark.gpu

FILLS = ("nan", "huge", "noise")
HEADS = {torch.bfloat16: (16, 8, 128), torch.float32: (4, 2, 128)}


def say(msg):
    print(msg, flush=True)


def fill_rows(t, sel, how, rng):
    """Replace the rows `sel` (bool over dim 0) of t in place."""
    n = int(sel.sum())
    if n == 0:
        return
    shape = (n,) + tuple(t.shape[1:])
    if how == "nan":
        val = np.full(shape, np.nan, np.float32)
    elif how == "huge":
        val = rng.choice(np.array([-1e30, 1e30], np.float32), size=shape)
    else:
        val = (40.0 * rng.standard_normal(shape)).astype(np.float32)
    t[torch.from_numpy(sel)] = torch.from_numpy(val).to(t.dtype)


def v_fill(how):
    """Non-ancestor v that may share a tile with other rows' keys: finite."""
    return "huge" if how == "huge" else "noise"


def same_bits(o1, o0, l1, l0, r, what):
    assert np.array_equal(o1[r].view(np.uint32), o0[r].view(np.uint32)), f"{what}: o of row {r} changed"
    assert np.array_equal(l1[:, r].view(np.uint32), l0[:, r].view(np.uint32)), f"{what}: lse of row {r} changed"


def run_prefill(desc, t, hq, hkv, d, plan):
    g = {k: v.to("cuda").contiguous() for k, v in t.items()}
    o, lse = ta.prefill(plan, g["q"], g["k"], g["v"], scale=d ** -0.5)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_nonancestor_perturbation_bit_identical(dtype):
    hq, hkv, d = HEADS[dtype]
    # two pages; short branches share 64-token tiles with their neighbours,
    # an empty branch, a branch over one tile, several layout units
    desc = synth.make_prefill_desc([100, 30], [np.array([3, 2, 4, 1]), np.array([2, 2])],
                                   [np.array([80, 5, 0, 70]), np.array([10, 66])])
    rng = np.random.default_rng(5)
    t0 = synth.prefill_tensors(rng, desc, hq, hkv, d, dtype)
    plan = ta.plan_for(desc).upload()
    o0, l0 = run_prefill(desc, t0, hq, hkv, d, plan)
    ref = oracle.plan_prefill(desc)
    pages = ref["pages"]
    T = desc.total_tokens()
    # main rows early and at the main end, a row of the 5-token branch (its
    # tile holds the neighbouring branches), rows of long branches, page 2
    M0 = int(pages[0, 1])
    rows = [3, M0 - 1, M0 + 80 + 2, M0 + 85 + 40, T - 1, int(pages[1, 0]) + 20, int(pages[1, 0]) + 35]
    for r in rows:
        pg = int(np.searchsorted(pages[:, 0], r, side="right") - 1)
        base, _, tp = (int(x) for x in pages[pg, :3])
        anc = np.zeros(T, bool)
        anc[base:int(ref["main_end"][r])] = True
        anc[int(ref["branch_start"][r]):r + 1] = True
        non = ~anc
        page = np.zeros(T, bool)
        page[base:base + tp] = True
        q_other = np.ones(T, bool)
        q_other[r] = False
        for how in FILLS:
            frng = np.random.default_rng(1000 * r + FILLS.index(how))
            t = {k: v.clone() for k, v in t0.items()}
            fill_rows(t["q"], q_other, how, frng)
            fill_rows(t["k"], non, how, frng)
            fill_rows(t["v"], non & page, v_fill(how), frng)
            fill_rows(t["v"], ~page, "nan", frng)
            o1, l1 = run_prefill(desc, t, hq, hkv, d, plan)
            same_bits(o1, o0, l1, l0, r, f"prefill {dtype} {how}")
        say(f"[invariant] prefill {dtype} row {r}: {anc.sum()} ancestors, bit-identical under {FILLS}")


def decode_desc():
    # three pages; content branches, multi-token windows and layout-stream
    # rows (region 0) sharing a page's main stream; suffixes over one tile
    return synth.DecodeDesc(np.array([300, 50, 7], np.int32), np.array([3, 2, 1], np.int32),
                            np.array([12, 12, 12, 5, 5, 3], np.int32),
                            np.array([0, 0, 0, 0, 1, 1, 2], np.int32),
                            np.array([1, 2, 3, 0, 1, 2, 1], np.int32),
                            np.array([0, 40, 130, 4, 7, 0, 65], np.int32),
                            np.array([1, 3, 2, 2, 1, 5, 1], np.int32))


def run_decode(plan, t, d):
    g = {k: v.to("cuda").contiguous() for k, v in t.items()}
    o, lse = ta.decode(plan, g["q"], g["k_main"], g["v_main"], g["k_suffix"], g["v_suffix"], scale=d ** -0.5)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_nonancestor_perturbation_bit_identical(dtype):
    hq, hkv, d = HEADS[dtype]
    desc = decode_desc()
    rng = np.random.default_rng(9)
    t0 = synth.decode_tensors(rng, desc, hq, hkv, d, dtype)
    plan = ta.plan_for(desc).upload()
    o0, l0 = run_decode(plan, t0, d)
    rows5 = oracle.plan_decode(desc)["rows"]
    n_rows = desc.n_rows()
    n_main = t0["k_main"].shape[0]
    n_suf = t0["k_suffix"].shape[0]
    main_off = np.concatenate([[0], np.cumsum(desc.main_tokens())])
    kq = desc.queries()
    suf_off = np.concatenate([[0], np.cumsum(desc.suffix_len.astype(np.int64) + kq)])
    row_branch = np.repeat(np.arange(desc.n_branches), kq)
    for r in range(n_rows):
        ms, ml, ss, vs, _ = (int(x) for x in rows5[r])
        b = int(row_branch[r])
        p = int(desc.br_page[b])
        anc_m = np.zeros(n_main, bool)
        anc_m[ms:ms + ml] = True
        anc_s = np.zeros(n_suf, bool)
        anc_s[ss:ss + vs] = True
        page_m = np.zeros(n_main, bool)
        page_m[main_off[p]:main_off[p + 1]] = True
        own_s = np.zeros(n_suf, bool)
        own_s[suf_off[b]:suf_off[b + 1]] = True
        q_other = np.ones(n_rows, bool)
        q_other[r] = False
        for how in FILLS:
            frng = np.random.default_rng(1000 * r + FILLS.index(how))
            t = {k: v.clone() for k, v in t0.items()}
            fill_rows(t["q"], q_other, how, frng)
            fill_rows(t["k_main"], ~anc_m, how, frng)
            fill_rows(t["k_suffix"], ~anc_s, how, frng)
            # main keys past the row's bound share tiles with longer-bound
            # rows of the page, later tokens of the row's own window share
            # its suffix tiles: finite there, NaN everywhere else
            fill_rows(t["v_main"], page_m & ~anc_m, v_fill(how), frng)
            fill_rows(t["v_main"], ~page_m, "nan", frng)
            fill_rows(t["v_suffix"], own_s & ~anc_s, v_fill(how), frng)
            fill_rows(t["v_suffix"], ~own_s, "nan", frng)
            o1, l1 = run_decode(plan, t, d)
            same_bits(o1, o0, l1, l0, r, f"decode {dtype} {how}")
    say(f"[invariant] decode {dtype}: all {n_rows} rows bit-identical under {FILLS}")


def run_verify(plan, t, d):
    g = {k: v.to("cuda").contiguous() for k, v in t.items()}
    o, lse = ta.verify(plan, g["q"], g["k_ctx"], g["v_ctx"], g["k_tree"], g["v_tree"], scale=d ** -0.5)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_verify_nonancestor_perturbation_bit_identical(dtype):
    hq, hkv, d = HEADS[dtype]
    rng = np.random.default_rng(13)
    trees = [(0, synth.random_tree_parents(rng, 32)), (0, synth.random_tree_parents(rng, 32)),
             (0, np.array([-1, 0, 0, 1])), (1, np.arange(-1, 19)), (1, synth.random_tree_parents(rng, 17)),
             (2, np.array([-1, -1, 1]))]
    desc = synth.VerifyDesc(np.array([300, 70, 0], np.int32), np.array([t[0] for t in trees], np.int32),
                            np.array([len(t[1]) for t in trees], np.int32),
                            np.concatenate([np.asarray(t[1], np.int32) for t in trees]))
    t0 = synth.verify_tensors(rng, desc, hq, hkv, d, dtype)
    plan = ta.plan_for(desc).upload()
    o0, l0 = run_verify(plan, t0, d)
    n = desc.total_nodes()
    ctx_off = np.concatenate([[0], np.cumsum(desc.ctx_len.astype(np.int64))])
    node_off = np.concatenate([[0], np.cumsum(desc.n_nodes.astype(np.int64))])
    n_ctx = int(ctx_off[-1])
    # every node of trees 0, 2, 3 and 5, a few of the others
    rows = (list(range(node_off[0], node_off[1])) + [int(node_off[1]) + 5, int(node_off[1]) + 31]
            + list(range(node_off[2], node_off[4])) + [int(node_off[4]) + 16] + list(range(node_off[5], n)))
    for r in rows:
        b = int(np.searchsorted(node_off, r, side="right") - 1)
        p = int(desc.br_page[b])
        i = r - int(node_off[b])
        a = oracle.tree_ancestor_mask(desc.parent[node_off[b]:node_off[b + 1]])
        anc_c = np.zeros(n_ctx, bool)
        anc_c[ctx_off[p]:ctx_off[p + 1]] = True
        anc_t = np.zeros(n, bool)
        anc_t[node_off[b]:node_off[b + 1]] = a[i]
        page_t = np.isin(np.repeat(desc.br_page, desc.n_nodes), [p])
        q_other = np.ones(n, bool)
        q_other[r] = False
        for how in FILLS:
            frng = np.random.default_rng(1000 * r + FILLS.index(how))
            t = {k: v.clone() for k, v in t0.items()}
            fill_rows(t["q"], q_other, how, frng)
            fill_rows(t["k_ctx"], ~anc_c, how, frng)
            fill_rows(t["k_tree"], ~anc_t, how, frng)
            fill_rows(t["v_ctx"], ~anc_c, "nan", frng)
            # nodes of the page's trees share the row tile's tree tiles
            fill_rows(t["v_tree"], page_t & ~anc_t, v_fill(how), frng)
            fill_rows(t["v_tree"], ~page_t, "nan", frng)
            o1, l1 = run_verify(plan, t, d)
            same_bits(o1, o0, l1, l0, r, f"verify {dtype} {how}")
    say(f"[invariant] verify {dtype}: {len(rows)} nodes bit-identical under {FILLS}")
