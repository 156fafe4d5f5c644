"""Pins for the draft-tree oracle (HSD paper notes, key design 3; HPD-Parsing
notes, Algorithm 1), checked against things fixed outside its own code:

* a hand-worked round (tests/golden/draft_tree_worked.txt);
* window matching against a byte-string search (a different mechanism);
* the prefix tree against its definition as the set of distinct candidate
  prefixes, each node's parent being its prefix minus the last token, and the
  tree ancestor mask against the prefix relation;
* acceptance: invariance under a per-row shift (log-probabilities versus
  logits), the limits tau -> 0 (walk to a leaf along the best children) and
  tau > 1 (nothing accepted), and exact mode on a chain equal to the
  acceptance-length definition written as a set maximum.
"""
import os

import numpy as np

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


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


def ints(vals):
    return [int(x) for x in vals]


def test_golden_draft_tree_round():
    fx = read_fixture("draft_tree_worked.txt")
    accepted = ints(fx["accepted"][0])
    n = int(fx["window"][0][0])
    drafts = [ints(d) for d in fx["draft"]]
    assert oracle.draft_candidates(accepted, drafts, n) == [ints(c) for c in fx["candidate"]]
    tok, par = oracle.draft_tree(accepted, drafts, n, max_nodes=64)
    assert tok == ints(fx["tokens"][0]) and par == ints(fx["parent"][0])
    tok5, par5 = oracle.draft_tree(accepted, drafts, n, max_nodes=5)
    assert tok5 == ints(fx["tokens_cap5"][0]) and par5 == ints(fx["parent_cap5"][0])
    tok2, par2 = oracle.draft_tree(accepted, drafts, n, max_nodes=64, max_depth=2)
    assert tok2 == ints(fx["tokens_depth2"][0]) and par2 == ints(fx["parent_depth2"][0])

    V = int(fx["vocab"][0][0])
    logp = np.full((len(tok) + 1, V), -10.0)
    for r, t, s in fx["score"]:
        logp[int(r), int(t)] = float(s)
    path, free = oracle.tree_accept(tok, par, logp, float(fx["tau"][0][0]))
    assert path == ints(fx["path"][0]) and free == int(fx["free"][0][0])
    path, free = oracle.tree_accept(tok, par, logp, float(fx["tau2"][0][0]))
    assert path == ints(fx["path2"][0]) and free == int(fx["free2"][0][0])
    path, free = oracle.tree_accept(tok, par, logp, exact=True)
    assert path == ints(fx["path_exact"][0]) and free == int(fx["free_exact"][0][0])



def oov_case():
    fx = read_fixture("draft_tree_worked.txt")
    V = int(fx["vocab"][0][0])
    tok, par = ints(fx["oov_tokens"][0]), ints(fx["oov_parent"][0])
    logp = np.full((len(tok) + 1, V), -10.0)
    for r, t, s in fx["oov_score"]:
        logp[int(r), int(t)] = float(s)
    return fx, V, tok, par, logp


def test_golden_out_of_vocabulary_tokens_are_never_accepted():
    """A drafted token outside [0, V) (negative, or >= V) has no score, so
    the walk skips its node; the hand-worked case puts the top score of a
    row on the last column, where a negative token index would wrap."""
    fx, V, tok, par, logp = oov_case()
    path, free = oracle.tree_accept(tok, par, logp, float(fx["oov_tau"][0][0]))
    assert path == ints(fx["oov_path"][0]) and free == int(fx["oov_free"][0][0])
    path, free = oracle.tree_accept(tok, par, logp, exact=True)
    assert path == ints(fx["oov_path_exact"][0]) and free == int(fx["oov_free_exact"][0][0])


def _matches_by_bytes(w, d):
    """Match positions of w in d through bytes.find on a 4-byte encoding."""
    enc = lambda xs: b"".join(int(x).to_bytes(4, "little", signed=True) for x in xs)
    hay, needle, out, start = enc(d), enc(w), [], 0
    while True:
        i = hay.find(needle, start)
        if i < 0:
            return out
        if i % 4 == 0:
            out.append(i // 4)
        start = i + 1


def test_window_match_against_byte_search():
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 5))
        alpha = int(rng.integers(2, 5))
        accepted = rng.integers(0, alpha, int(rng.integers(0, 8))).tolist()
        drafts = [rng.integers(0, alpha, int(rng.integers(0, 30))).tolist()
                  for _ in range(int(rng.integers(0, 4)))]
        want = []
        if len(accepted) >= n:
            w = accepted[-n:]
            for d in drafts:
                for j in _matches_by_bytes(w, d):
                    if j + n < len(d):
                        want.append(d[j + n:])
        assert oracle.draft_candidates(accepted, drafts, n) == want, trial


def _distinct_prefixes(cands):
    seen, order = set(), []
    for c in cands:
        for i in range(1, len(c) + 1):
            p = tuple(c[:i])
            if p not in seen:
                seen.add(p)
                order.append(p)
    return order


def _prefix_of(tok, par, i):
    out = []
    while i >= 0:
        out.append(tok[i])
        i = par[i]
    return tuple(reversed(out))


def test_prefix_tree_is_the_set_of_distinct_prefixes():
    rng = np.random.default_rng(5)
    for trial in range(200):
        cands = [rng.integers(0, 3, int(rng.integers(1, 7))).tolist()
                 for _ in range(int(rng.integers(0, 6)))]
        cap = int(rng.integers(0, 40))
        depth = int(rng.integers(1, 8)) if trial % 2 else None
        tok, par = oracle.prefix_tree(cands, cap, depth)
        pref = [_prefix_of(tok, par, i) for i in range(len(tok))]
        # nodes are the first `cap` distinct prefixes of length <= depth, in
        # enumeration order
        want = [p for p in _distinct_prefixes(cands) if depth is None or len(p) <= depth]
        assert pref == want[:cap], trial
        assert all(-1 <= par[i] < i for i in range(len(par)))
        # the tree ancestor mask is the prefix relation
        a = oracle.tree_ancestor_mask(par) if tok else np.zeros((0, 0), bool)
        for i in range(len(tok)):
            for j in range(len(tok)):
                assert bool(a[i, j]) == (pref[i][:len(pref[j])] == pref[j])


def _random_tree(rng, n):
    par = [-1]
    for i in range(1, n):
        par.append(int(rng.integers(-1, i)))
    return par[:n]


def test_accept_depends_on_score_differences_only():
    rng = np.random.default_rng(7)
    for trial in range(100):
        n, V = int(rng.integers(0, 12)), int(rng.integers(2, 30))
        par = _random_tree(rng, n)
        tok = rng.integers(0, V, n).tolist()
        # dyadic scores and shifts keep every difference exact in fp64
        z = rng.integers(-64, 64, (n + 1, V)) / 8.0
        shift = rng.integers(-1000, 1000, (n + 1, 1)) / 4.0
        tau = float(rng.choice([0.75, 0.5, 0.9, 1.0]))
        assert oracle.tree_accept(tok, par, z, tau) == oracle.tree_accept(tok, par, z + shift, tau)
        assert (oracle.tree_accept(tok, par, z, exact=True)
                == oracle.tree_accept(tok, par, z + shift, exact=True))


def test_accept_limits_of_tau():
    rng = np.random.default_rng(11)
    for trial in range(100):
        n, V = int(rng.integers(0, 12)), int(rng.integers(2, 30))
        par = _random_tree(rng, n)
        tok = rng.integers(0, V, n).tolist()
        z = rng.standard_normal((n + 1, V))
        # tau > 1: the difference is never positive, nothing is accepted
        assert oracle.tree_accept(tok, par, z, 1.5) == ([], int(np.argmax(z[0])))
        # tau -> 0: walk along the best child down to a leaf
        path, free = oracle.tree_accept(tok, par, z, 1e-300)
        cur, row = -1, 0
        for node in path:
            kids = [c for c in range(n) if par[c] == cur]
            assert node in kids
            assert z[row, tok[node]] == max(z[row, tok[c]] for c in kids)
            cur, row = node, 1 + node
        assert not any(par[c] == cur for c in range(n))
        assert free == int(np.argmax(z[row]))


def test_exact_mode_on_chains_is_the_acceptance_length():
    rng = np.random.default_rng(13)
    for trial in range(200):
        K, V = int(rng.integers(0, 10)), int(rng.integers(2, 6))
        draft = rng.integers(0, V, K).tolist()
        z = rng.standard_normal((K + 1, V))
        target = [int(np.argmax(z[i])) for i in range(K + 1)]
        # n_acc = max{k : target_i == draft_i for all i <= k}, as a set maximum
        n_acc = max(k for k in range(K + 1) if all(target[i] == draft[i] for i in range(k)))
        assert oracle.chain_accept(draft, target) == (n_acc, target[n_acc])
        path, free = oracle.tree_accept(draft, list(range(-1, K - 1)), z, exact=True)
        assert path == list(range(n_acc)) and free == target[n_acc]
        # with tau = 1 a chain accepts exactly where the drafted token reaches
        # the row maximum (here unique with probability one)
        path1, _ = oracle.tree_accept(draft, list(range(-1, K - 1)), z, 1.0)
        assert path1 == path

