"""CPU tests of the draft-tree entry points: tree_attn_draft_tree against the
oracle (bit-exact, on the hand-worked round and on seeded random drafts of
page-like shape), its output feeding tree_attn_plan_verify, and the host-side
validation of tree_attn_draft_tree and tree_attn_accept (nothing launched)."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def read_fixture(name):
    rows = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, *vals = line.split()
                rows.setdefault(key, []).append([int(float(x)) if "." not in x else float(x) for x in vals])
    return rows


def same_tree(got, want):
    tok, par = got
    return tok.tolist() == list(want[0]) and par.tolist() == list(want[1])


def test_draft_tree_golden_round():
    fx = read_fixture("draft_tree_worked.txt")
    acc, n, drafts = fx["accepted"][0], fx["window"][0][0], fx["draft"]
    got = ta.draft_tree(acc, drafts, n, max_nodes=64)
    assert got[0].tolist() == fx["tokens"][0] and got[1].tolist() == fx["parent"][0]
    got = ta.draft_tree(acc, drafts, n, max_nodes=5)
    assert got[0].tolist() == fx["tokens_cap5"][0] and got[1].tolist() == fx["parent_cap5"][0]
    got = ta.draft_tree(acc, drafts, n, max_nodes=64, max_depth=2)
    assert got[0].tolist() == fx["tokens_depth2"][0] and got[1].tolist() == fx["parent_depth2"][0]


@pytest.mark.parametrize("seed", range(6))
def test_draft_tree_matches_oracle_random(seed):
    rng = np.random.default_rng(100 + seed)
    for trial in range(150):
        alpha = int(rng.integers(2, 6))
        n = int(rng.integers(1, 5))
        acc = rng.integers(0, alpha, int(rng.integers(0, 10))).tolist()
        drafts = [rng.integers(0, alpha, int(rng.integers(0, 40))).tolist() for _ in range(int(rng.integers(0, 5)))]
        cap = int(rng.integers(0, 70))
        depth = int(rng.integers(0, 9))
        want = oracle.draft_tree(acc, drafts, n, cap, depth if depth > 0 else None)
        assert same_tree(ta.draft_tree(acc, drafts, n, cap, depth), want), (seed, trial)


def test_draft_tree_page_shaped_drafts():
    """Region drafts of a page (hundreds of tokens each over a large
    vocabulary, with repeated structural runs such as table separators) and
    an accepted sequence that ends inside one of them."""
    rng = np.random.default_rng(7)
    for trial in range(5):
        drafts = []
        for r in range(6):
            d = rng.integers(0, 151936, int(rng.integers(100, 800))).tolist()
            sep = [101, 102, 103]  # a separator run repeated through the draft
            for j in range(0, len(d) - 3, int(rng.integers(20, 60))):
                d[j:j + 3] = sep
            drafts.append(d)
        src = drafts[int(rng.integers(0, 6))]
        cut = int(rng.integers(3, len(src)))
        acc = list(rng.integers(0, 151936, 20)) + src[:cut]
        for cap, depth in ((64, 8), (32, 8), (64, 0), (5, 3)):
            want = oracle.draft_tree(acc, drafts, 3, cap, depth if depth else None)
            got = ta.draft_tree(acc, drafts, 3, cap, depth)
            assert same_tree(got, want), (trial, cap, depth)
        acc = list(acc[:-3]) + [101, 102, 103]
        want = oracle.draft_tree(acc, drafts, 3, 64, 8)
        got = ta.draft_tree(acc, drafts, 3, 64, 8)
        assert same_tree(got, want) and len(got[0]) > 1


def test_draft_tree_feeds_the_verify_plan():
    rng = np.random.default_rng(9)
    trees = []
    for b in range(4):
        drafts = [rng.integers(0, 4, 60).tolist() for _ in range(3)]
        acc = drafts[0][:10]
        trees.append(ta.draft_tree(acc, drafts, 3, max_nodes=32, max_depth=8))
    n_nodes = [len(t[0]) for t in trees]
    parent = np.concatenate([t[1] for t in trees])
    plan = ta.plan_verify([100, 50], [0, 0, 1, 1], n_nodes, parent)
    mask = plan.export("verify_mask")
    off = 0
    for tok, par in trees:
        a = oracle.tree_ancestor_mask(par) if len(par) else np.zeros((0, 0), bool)
        want = [sum(1 << j for j in range(len(par)) if a[i, j]) for i in range(len(par))]
        assert mask[off:off + len(par)].tolist() == want
        off += len(par)


def test_draft_tree_errors():
    L = ta.lib()
    n = ctypes.c_int32(-7)
    tok = (ctypes.c_int32 * 4)()
    par = (ctypes.c_int32 * 4)()
    acc = (ctypes.c_int32 * 3)(1, 2, 3)
    lens = (ctypes.c_int32 * 1)(3)
    I = ctypes.cast
    P = ctypes.POINTER(ctypes.c_int32)
    args_ok = [I(acc, P), 3, I(acc, P), I(lens, P), 1, 3, 4, 0, I(tok, P), I(par, P), ctypes.byref(n)]
    assert L.tree_attn_draft_tree(*args_ok) == ta.TA_OK and n.value == 0  # match at the draft's end only
    for i, bad in ((5, 0), (6, -1), (7, -1), (1, -1), (4, -2)):
        a = list(args_ok)
        a[i] = bad
        n.value = -7
        assert L.tree_attn_draft_tree(*a) == ta.TA_ERR_INVALID_ARG, (i, bad)
        assert n.value == -7
    a = list(args_ok)
    a[8] = None
    assert L.tree_attn_draft_tree(*a) == ta.TA_ERR_INVALID_ARG
    a = list(args_ok)
    a[10] = None
    assert L.tree_attn_draft_tree(*a) == ta.TA_ERR_INVALID_ARG
    neg = (ctypes.c_int32 * 1)(-1)
    a = list(args_ok)
    a[3] = I(neg, P)
    assert L.tree_attn_draft_tree(*a) == ta.TA_ERR_INVALID_ARG


def test_accept_errors_before_any_device_work():
    L = ta.lib()
    buf = (ctypes.c_uint8 * 8192)()
    base = (ctypes.addressof(buf) + 255) & ~255
    p = ctypes.c_void_p(base)
    odd = ctypes.c_void_p(base + 1)
    vplan = ta.plan_verify([10], [0, 0], [3, 2], [-1, 0, 0, -1, 0])
    need = ta.accept_scratch_bytes(vplan, 1000)
    assert 0 < need <= 8192 - 256
    bf, f32 = ta.TA_DTYPE_BF16, ta.TA_DTYPE_F32
    TAU, EXACT = ta.TA_ACCEPT_TAU, ta.TA_ACCEPT_EXACT

    def call(plan=vplan, dtype=bf, logits=p, vocab=1000, ld=1000, tokens=p, tau=0.75, mode=TAU, path=p,
             n_path=p, nxt=p, scratch=p, nbytes=need):
        return L.tree_attn_accept(plan.handle, dtype, logits, vocab, ld, tokens, tau, mode, path, n_path, nxt,
                                  scratch, nbytes, None)

    assert call() == ta.TA_ERR_STATE  # valid, but the plan was never uploaded
    assert call(mode=EXACT, tau=float("nan")) == ta.TA_ERR_STATE  # tau is ignored in exact mode
    assert call(plan=ta.plan_prefill([8], [1], [2], [3])) == ta.TA_ERR_STATE
    assert call(dtype=7) == ta.TA_ERR_UNSUPPORTED
    assert call(mode=2) == ta.TA_ERR_INVALID_ARG
    for tau in (0.0, -1.0, float("inf"), float("nan")):
        assert call(tau=tau) == ta.TA_ERR_INVALID_ARG
    assert call(vocab=0) == ta.TA_ERR_INVALID_ARG
    assert call(vocab=1 << 31, ld=1 << 31) == ta.TA_ERR_INVALID_ARG
    assert call(ld=999) == ta.TA_ERR_INVALID_ARG
    assert call(logits=None) == ta.TA_ERR_INVALID_ARG
    assert call(logits=odd) == ta.TA_ERR_INVALID_ARG
    assert call(dtype=f32, logits=ctypes.c_void_p(base + 2)) == ta.TA_ERR_INVALID_ARG
    assert call(tokens=None) == ta.TA_ERR_INVALID_ARG
    assert call(path=None) == ta.TA_ERR_INVALID_ARG
    assert call(n_path=None) == ta.TA_ERR_INVALID_ARG
    assert call(nxt=None) == ta.TA_ERR_INVALID_ARG
    assert call(scratch=None) == ta.TA_ERR_WORKSPACE
    assert call(nbytes=need - 1) == ta.TA_ERR_WORKSPACE
    assert call(scratch=ctypes.c_void_p(base + 16)) == ta.TA_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert L.tree_attn_accept_scratch_bytes(ta.plan_prefill([8], [1], [2], [3]).handle, 10,
                                            ctypes.byref(n)) == ta.TA_ERR_STATE
    assert L.tree_attn_accept_scratch_bytes(vplan.handle, 0, ctypes.byref(n)) == ta.TA_ERR_INVALID_ARG
