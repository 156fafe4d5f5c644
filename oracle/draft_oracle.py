"""Reference draft-tree utilities for tree verification (plain Python).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the library never
imports it and it imports nothing from the library.

Source: [HSD] "HSD: Training-Free Acceleration for Document Parsing
Vision-Language Models with Hierarchical Speculative Decoding" (paper notes),
key design 3, decoupled speculative verification:
  (a) draft-target matching: the last n accepted tokens form a reference
      window w (n = 3 by default); every position j where a draft holds w
      (draft[j : j + n] == w) yields the candidate continuation
      draft[j + n :];
  (b) prefix-tree batching: the candidates become a prefix tree (shared
      prefixes merged, each node one distinct prefix, its children the
      possible next tokens), linearised into a packed sequence that the
      target verifies in one forward under the tree ancestor mask;
  verification walks the tree greedily from the root: among the children of
  the current node it takes the token u* the model rates highest and accepts
  it if log p(u*) - log p(u_hat) >= log tau, u_hat being the model's top token
  over the whole vocabulary (tau = 0.75 by default); the walk stops at the
  first rejection, and one freely generated token u_hat follows the accepted
  path.
The HPD-Parsing notes ("P-MTP") verify drafted chains of future tokens per
branch; a chain is the special case of a tree whose nodes have one child.

Readings where the notes are silent (listed in the design notes):
  * a window needs n accepted tokens; with fewer there is no candidate;
  * empty continuations (a match at a draft's end) are dropped;
  * candidates are taken draft by draft, matches in position order, and
    inserted in that order; the linearised order is node creation order, so
    every parent precedes its children; top-level nodes have parent -1 (they
    hang off the accepted sequence);
  * a node budget caps the tree: insertion stops at the first token that
    would create a node beyond it (earlier candidates keep their nodes);
    an optional depth budget first cuts every candidate to that many tokens;
  * ties in "highest" go to the lowest node index (children) and the lowest
    token id (vocabulary);
  * a node whose token lies outside the vocabulary is never accepted.
"""
from __future__ import annotations

import math

import numpy as np


def draft_candidates(accepted, drafts, window: int = 3):
    """Continuations of every match of the last `window` accepted tokens."""
    acc = [int(x) for x in accepted]
    if window <= 0 or len(acc) < window:
        return []
    w = acc[len(acc) - window:]
    out = []
    for d in drafts:
        d = [int(x) for x in d]
        for j in range(0, len(d) - window + 1):
            if d[j:j + window] == w and j + window < len(d):
                out.append(d[j + window:])
    return out


def prefix_tree(candidates, max_nodes: int, max_depth=None):
    """Linearised prefix tree of the candidates: (tokens, parent) lists.

    max_depth (optional) keeps only the first max_depth tokens of each
    candidate."""
    tokens, parent = [], []
    children = {-1: {}}  # node -> {token: child node}
    for cand in candidates:
        cur = -1
        if max_depth is not None:
            cand = cand[:max_depth]
        for t in cand:
            t = int(t)
            nxt = children[cur].get(t)
            if nxt is None:
                if len(tokens) >= max_nodes:
                    break
                nxt = len(tokens)
                tokens.append(t)
                parent.append(cur)
                children[cur][t] = nxt
                children[nxt] = {}
            cur = nxt
        else:
            continue
        break
    return tokens, parent


def draft_tree(accepted, drafts, window: int = 3, max_nodes: int = 64, max_depth=None):
    """Window match, then prefix tree ([HSD] key design 3 (a) + (b))."""
    return prefix_tree(draft_candidates(accepted, drafts, window), max_nodes, max_depth)


def tree_accept(tokens, parent, logp, tau: float = 0.75, exact: bool = False):
    """Greedy walk over a verified tree ([HSD] key design 3, verification).

    logp: [n_nodes + 1, V] log-probabilities (or logits: only differences
    within a row matter); row 0 is the model's next-token distribution after
    the accepted sequence, row 1 + i the one after node i.
    tau mode: at each node take the child u* the model rates highest and
    accept it iff log p(u*) - log p(u_hat) >= log tau, computed in fp64.
    exact mode (HPD-Parsing's acceptance, y* = u_hat): accept the child whose
    token is u_hat.
    Returns (accepted node path, free token u_hat of the row after the path).
    """
    logp = np.asarray(logp)
    n, V = len(tokens), logp.shape[1]
    kids = {-1: []}
    for i in range(n):
        kids.setdefault(i, [])
        if 0 <= int(tokens[i]) < V:  # a token outside the vocabulary is never a candidate
            kids[int(parent[i])].append(i)
    log_tau = math.log(tau)
    path, cur, row = [], -1, 0
    while kids.get(cur):
        top = int(np.argmax(logp[row]))  # first maximum: lowest token id
        if exact:
            hit = [c for c in kids[cur] if int(tokens[c]) == top]
            if not hit:
                break
            best = hit[0]
        else:
            best = None
            for c in kids[cur]:  # ascending node index: ties keep the first
                if best is None or logp[row, tokens[c]] > logp[row, tokens[best]]:
                    best = c
            diff = float(logp[row, tokens[best]]) - float(logp[row, top])
            if not diff >= log_tau:
                break
        path.append(best)
        cur, row = best, 1 + best
    return path, int(np.argmax(logp[row]))


def chain_accept(draft, target):
    """HPD-Parsing acceptance length of a drafted chain (Algorithm 1).

    draft: the K drafted tokens t_1..t_K; target: the target model's own
    greedy tokens y*_1..y*_{K+1} at the same positions.  n_acc is the largest
    k with y*_i = t_i for every i <= k; the token that follows the accepted
    drafts is the target's y*_{n_acc + 1}.
    """
    k = 0
    while k < len(draft) and int(target[k]) == int(draft[k]):
        k += 1
    return k, int(target[k])
