"""Seeded synthetic workloads for layout-grounded tree attention.

This module only draws input *structure* (page/branch/tree sizes and
topologies) and input *values* (q/k/v).  It holds none of the attention
arithmetic, so the oracle and the HIP path can both be fed from it without
sharing any code of the method.

Workload shapes follow the pages:
  * page prefix of 4096 visual tokens, 16,384-token packed cap and bf16
    training (PaDoc summary page, "Training recipe");
  * 16 query / 8 KV heads, head_dim 128 (HPD-Parsing notes: the
    InternVL3.5-1B decoder with GQA);
  * a 4,809-token page prefix for decode (HPD-Parsing blog, Table 2 input
    tokens per page);
  * verify trees are linearised draft prefix trees (HSD notes, key design 3,
    prefix-tree batching).

Draw order per config (numpy ``default_rng(seed)``):
  1  C = integers(5, 21, N=3)
  2  z = standard_normal(24)
  3  per page: N = integers(12, 41), then z = standard_normal(N)
  4  per page: s = integers(0, 1025, 24)
  5  P = integers(4096, 16385, 64); then per branch (page-major) and per
     node i = 1..31 one integers(len(eligible)) with eligible ascending
then the tensors, ``standard_normal(dtype=float32)`` in argument order.
Lognormal content lengths: C = clip(rint(exp(5 + 0.8 z)), 8, 1024).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

PACKED_CAP = 16384


@dataclass
class PrefillDesc:
    """Per-page description of a packed page [X | B_1..B_N | Y_1..Y_N]."""
    prefix_len: np.ndarray   # [n_pages] int32  (P)
    n_regions: np.ndarray    # [n_pages] int32  (N)
    layout_len: np.ndarray   # [sum N]  int32   (L_k), page-major
    content_len: np.ndarray  # [sum N]  int32   (C_k), page-major

    @property
    def n_pages(self) -> int:
        return int(self.prefix_len.shape[0])

    def page_slices(self):
        off = 0
        for p in range(self.n_pages):
            n = int(self.n_regions[p])
            yield p, slice(off, off + n)
            off += n

    def page_tokens(self) -> np.ndarray:
        """Packed length of each page (a size, needed to shape tensors)."""
        out = np.zeros(self.n_pages, dtype=np.int64)
        for p, sl in self.page_slices():
            out[p] = int(self.prefix_len[p]) + int(self.layout_len[sl].sum()) + int(self.content_len[sl].sum())
        return out

    def total_tokens(self) -> int:
        return int(self.page_tokens().sum())


@dataclass
class DecodeDesc:
    """Pages' main streams [X | B_1..B_N] plus live rows (page, region k, s_k):
    content branches (k = 1..N) and layout-stream rows (k = 0, seeing the whole
    main stream).  Each holds s_k earlier private tokens and n_query new ones
    (1 unless given), the last n_query of its suffix."""
    prefix_len: np.ndarray   # [n_pages]
    n_regions: np.ndarray    # [n_pages]
    layout_len: np.ndarray   # [sum N]
    br_page: np.ndarray      # [n_branches], non-decreasing
    br_region: np.ndarray    # [n_branches], 0 (layout stream) or 1..N of its page
    suffix_len: np.ndarray   # [n_branches], s_k = tokens already in the branch
    n_query: Optional[np.ndarray] = None  # [n_branches] new tokens (query rows) per branch, >= 1

    def queries(self) -> np.ndarray:
        if self.n_query is None:
            return np.ones(self.n_branches, dtype=np.int64)
        return self.n_query.astype(np.int64)

    def n_rows(self) -> int:
        return int(self.queries().sum())

    @property
    def n_pages(self) -> int:
        return int(self.prefix_len.shape[0])

    @property
    def n_branches(self) -> int:
        return int(self.br_page.shape[0])

    def main_tokens(self) -> np.ndarray:
        out = np.zeros(self.n_pages, dtype=np.int64)
        off = 0
        for p in range(self.n_pages):
            n = int(self.n_regions[p])
            out[p] = int(self.prefix_len[p]) + int(self.layout_len[off:off + n].sum())
            off += n
        return out

    def suffix_tokens(self) -> int:
        # every branch stores s_k previous tokens plus its new ones
        return int((self.suffix_len.astype(np.int64) + self.queries()).sum())


@dataclass
class VerifyDesc:
    """Per-page context plus per-branch draft trees given as parent arrays."""
    ctx_len: np.ndarray      # [n_pages]
    br_page: np.ndarray      # [n_branches], non-decreasing
    n_nodes: np.ndarray      # [n_branches]
    parent: np.ndarray       # [sum n_nodes]; -1 = hangs off the context, else < own index

    @property
    def n_pages(self) -> int:
        return int(self.ctx_len.shape[0])

    @property
    def n_branches(self) -> int:
        return int(self.br_page.shape[0])

    def total_nodes(self) -> int:
        return int(self.n_nodes.sum())


@dataclass
class Workload:
    name: str
    kind: str                 # "prefill" | "decode" | "verify"
    desc: object
    hq: int
    hkv: int
    head_dim: int
    dtype: torch.dtype
    tensors: dict = field(default_factory=dict)   # CPU tensors in `dtype`
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


def lognormal_lengths(z: np.ndarray) -> np.ndarray:
    return np.clip(np.rint(np.exp(5.0 + 0.8 * z)), 8, 1024).astype(np.int32)


def cap_page(prefix: int, layout: np.ndarray, content: np.ndarray, cap: int = PACKED_CAP) -> np.ndarray:
    """Truncate in packed order: shorten the last branches (to zero if needed)."""
    content = content.copy()
    excess = prefix + int(layout.sum()) + int(content.sum()) - cap
    k = len(content) - 1
    while excess > 0 and k >= 0:
        cut = min(excess, int(content[k]))
        content[k] -= cut
        excess -= cut
        k -= 1
    if excess > 0:
        raise ValueError("prefix plus layout alone exceed the packed cap")
    return content


def _normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


def prefill_tensors(rng, desc: PrefillDesc, hq, hkv, d, dtype):
    t = desc.total_tokens()
    return {
        "q": _normal(rng, (t, hq, d), dtype),
        "k": _normal(rng, (t, hkv, d), dtype),
        "v": _normal(rng, (t, hkv, d), dtype),
    }


def make_prefill_desc(prefixes, layouts, contents) -> PrefillDesc:
    return PrefillDesc(
        prefix_len=np.asarray(prefixes, dtype=np.int32),
        n_regions=np.asarray([len(c) for c in contents], dtype=np.int32),
        layout_len=np.concatenate([np.asarray(l, dtype=np.int32) for l in layouts]) if layouts else np.zeros(0, np.int32),
        content_len=np.concatenate([np.asarray(c, dtype=np.int32) for c in contents]) if contents else np.zeros(0, np.int32),
    )


def config1(seed: int = 0, with_tensors: bool = True) -> Workload:
    """Tiny fp32 tree: 1 page, P=64, 3 regions of 6 layout tokens, C ~ U{5..20}."""
    rng = np.random.default_rng(seed)
    c = rng.integers(5, 21, 3).astype(np.int32)
    desc = make_prefill_desc([64], [np.full(3, 6)], [c])
    w = Workload("tiny_fp32_tree_P64_N3", "prefill", desc, 2, 1, 32, torch.float32, seed=seed)
    if with_tensors:
        w.tensors = prefill_tensors(rng, desc, 2, 1, 32, torch.float32)
    return w


def config2(seed: int = 1, with_tensors: bool = True) -> Workload:
    """One page: P=4096, 24 regions of 12 layout tokens, lognormal content."""
    rng = np.random.default_rng(seed)
    c = lognormal_lengths(rng.standard_normal(24))
    lay = np.full(24, 12, dtype=np.int32)
    c = cap_page(4096, lay, c)
    desc = make_prefill_desc([4096], [lay], [c])
    w = Workload("prefill_1page_P4096_N24", "prefill", desc, 16, 8, 128, torch.bfloat16, seed=seed)
    if with_tensors:
        w.tensors = prefill_tensors(rng, desc, 16, 8, 128, torch.bfloat16)
    return w


def config3(seed: int = 2, with_tensors: bool = True) -> Workload:
    """Eight pages: P=4096, N ~ U{12..40}, otherwise as the one-page case."""
    rng = np.random.default_rng(seed)
    lays, cons = [], []
    for _ in range(8):
        n = int(rng.integers(12, 41))
        c = lognormal_lengths(rng.standard_normal(n))
        lay = np.full(n, 12, dtype=np.int32)
        lays.append(lay)
        cons.append(cap_page(4096, lay, c))
    desc = make_prefill_desc([4096] * 8, lays, cons)
    w = Workload("prefill_8pages_P4096_N12to40", "prefill", desc, 16, 8, 128, torch.bfloat16, seed=seed)
    if with_tensors:
        w.tensors = prefill_tensors(rng, desc, 16, 8, 128, torch.bfloat16)
    return w


def decode_tensors(rng, desc: DecodeDesc, hq, hkv, d, dtype):
    m = int(desc.main_tokens().sum())
    s = desc.suffix_tokens()
    return {
        "q": _normal(rng, (desc.n_rows(), hq, d), dtype),
        "k_main": _normal(rng, (m, hkv, d), dtype),
        "v_main": _normal(rng, (m, hkv, d), dtype),
        "k_suffix": _normal(rng, (s, hkv, d), dtype),
        "v_suffix": _normal(rng, (s, hkv, d), dtype),
    }


def config4(seed: int = 3, with_tensors: bool = True, n_pages: int = 16) -> Workload:
    """16 pages x 24 live branches; P=4809, L_k=12, s_k ~ U{0..1024}."""
    rng = np.random.default_rng(seed)
    s = np.concatenate([rng.integers(0, 1025, 24) for _ in range(n_pages)]).astype(np.int32)
    desc = DecodeDesc(
        prefix_len=np.full(n_pages, 4809, dtype=np.int32),
        n_regions=np.full(n_pages, 24, dtype=np.int32),
        layout_len=np.full(24 * n_pages, 12, dtype=np.int32),
        br_page=np.repeat(np.arange(n_pages, dtype=np.int32), 24),
        br_region=np.tile(np.arange(1, 25, dtype=np.int32), n_pages),
        suffix_len=s,
    )
    w = Workload(f"decode_{n_pages}pages_x24branches_P4809", "decode", desc, 16, 8, 128, torch.bfloat16, seed=seed)
    if with_tensors:
        w.tensors = decode_tensors(rng, desc, 16, 8, 128, torch.bfloat16)
    return w


def decode_multi(seed: int = 6, with_tensors: bool = True, n_pages: int = 16, window: int = 8) -> Workload:
    """The decode workload's pages with a drafted window of `window` new tokens
    per live row: per page one layout-stream row (region 0, 0..11 layout
    tokens of its current region already written) followed by 24 content
    branches with s_k ~ U{0..1024}."""
    rng = np.random.default_rng(seed)
    s_lay = rng.integers(0, 12, n_pages)
    s_br = rng.integers(0, 1025, (n_pages, 24))
    suffix = np.concatenate([[s_lay[p]] + list(s_br[p]) for p in range(n_pages)]).astype(np.int32)
    desc = DecodeDesc(
        prefix_len=np.full(n_pages, 4809, dtype=np.int32),
        n_regions=np.full(n_pages, 24, dtype=np.int32),
        layout_len=np.full(24 * n_pages, 12, dtype=np.int32),
        br_page=np.repeat(np.arange(n_pages, dtype=np.int32), 25),
        br_region=np.tile(np.arange(0, 25, dtype=np.int32), n_pages),
        suffix_len=suffix,
        n_query=np.full(25 * n_pages, window, dtype=np.int32),
    )
    w = Workload(f"decode_multi_{n_pages}pages_x(1+24)rows_x{window}tokens_P4809", "decode", desc, 16, 8, 128,
                 torch.bfloat16, seed=seed)
    if with_tensors:
        w.tensors = decode_tensors(rng, desc, 16, 8, 128, torch.bfloat16)
    return w


def random_tree_parents(rng, n_nodes: int, max_children: int = 3, max_depth: int = 8) -> np.ndarray:
    """Node 0 is the root (depth 0, hangs off the context); node i picks its
    parent uniformly among earlier nodes with < max_children children and
    depth < max_depth, so every node has depth <= max_depth."""
    parent = np.full(n_nodes, -1, dtype=np.int32)
    children = np.zeros(n_nodes, dtype=np.int64)
    depth = np.zeros(n_nodes, dtype=np.int64)
    for i in range(1, n_nodes):
        eligible = [j for j in range(i) if children[j] < max_children and depth[j] < max_depth]
        j = eligible[int(rng.integers(len(eligible)))]
        parent[i] = j
        children[j] += 1
        depth[i] = depth[j] + 1
    return parent


def verify_tensors(rng, desc: VerifyDesc, hq, hkv, d, dtype):
    c = int(desc.ctx_len.astype(np.int64).sum())
    n = desc.total_nodes()
    return {
        "q": _normal(rng, (n, hq, d), dtype),
        "k_ctx": _normal(rng, (c, hkv, d), dtype),
        "v_ctx": _normal(rng, (c, hkv, d), dtype),
        "k_tree": _normal(rng, (n, hkv, d), dtype),
        "v_tree": _normal(rng, (n, hkv, d), dtype),
    }


def config5(seed: int = 4, with_tensors: bool = True, n_pages: int = 64,
            branches_per_page: int = 8, nodes: int = 32) -> Workload:
    """64 pages x 8 branches; P_p ~ U{4096..16384}; 32-node random draft trees."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(4096, 16385, n_pages).astype(np.int32)
    parents = [random_tree_parents(rng, nodes) for _ in range(n_pages * branches_per_page)]
    desc = VerifyDesc(
        ctx_len=ctx,
        br_page=np.repeat(np.arange(n_pages, dtype=np.int32), branches_per_page),
        n_nodes=np.full(n_pages * branches_per_page, nodes, dtype=np.int32),
        parent=np.concatenate(parents).astype(np.int32),
    )
    w = Workload(f"verify_{n_pages}pages_x{branches_per_page}branches_x{nodes}nodes", "verify",
                 desc, 16, 8, 128, torch.bfloat16, seed=seed)
    if with_tensors:
        w.tensors = verify_tensors(rng, desc, 16, 8, 128, torch.bfloat16)
    return w


def config5_unshared(seed: int = 4, nodes: int = 32) -> Workload:
    """The verify workload's 512 draft trees, each over a prefix of its own
    (P ~ U{4096..16384} per tree, no sharing between trees): 512 pages of one
    branch each, about 5.2 M context tokens (21.7 GB of bf16 K/V).  Tensors
    are drawn on the GPU (``verify_tensors_device``): the host would need
    minutes for them."""
    w = config5(seed, with_tensors=False, n_pages=512, branches_per_page=1, nodes=nodes)
    w.name = f"verify_512_unshared_prefixes_x{nodes}nodes"
    return w


def verify_tensors_device(seed: int, desc: VerifyDesc, hq, hkv, d, dtype, device="cuda"):
    """q, k_ctx, v_ctx, k_tree, v_tree ~ N(0, 1) drawn in that order by
    torch's generator on `device` seeded with `seed` (for workloads too large
    to draw on the host)."""
    g = torch.Generator(device=device).manual_seed(seed)
    c = int(desc.ctx_len.astype(np.int64).sum())
    n = desc.total_nodes()
    shapes = {"q": (n, hq, d), "k_ctx": (c, hkv, d), "v_ctx": (c, hkv, d), "k_tree": (n, hkv, d),
              "v_tree": (n, hkv, d)}
    return {k: torch.randn(sh, generator=g, device=device, dtype=torch.float32).to(dtype)
            for k, sh in shapes.items()}


# Vocabulary size of the Qwen-family decoders the pages build on; the pages
# do not print it, so this is a stand-in for the logits width.
VOCAB = 151936


def draft_tokens(rng, desc: VerifyDesc, vocab: int) -> np.ndarray:
    """Drafted token of every node, uniform over the vocabulary."""
    return rng.integers(0, vocab, desc.total_nodes()).astype(np.int32)


def accept_logits(seed: int, desc: VerifyDesc, tokens: np.ndarray, vocab: int, ld: int = None,
                  dtype: torch.dtype = torch.bfloat16, device="cuda", p_plant: float = 0.9) -> torch.Tensor:
    """Logits rows for the acceptance walk, tree-major: per tree one row for
    the position after the accepted sequence, then one per node.

    Background scores ~ 1.5 N(0, 1) clipped to [-10, 3]; every row has one
    top token at 4.0.  In a fraction p_plant of the rows that have children,
    one child's drafted token is made the top token (70%) or is set to
    4.0 - gap with gap ~ U(0, 0.6), which straddles log(0.75), so walks of
    a few accepted nodes occur, as in the acceptance lengths of 2.5 to 4.6
    tokens per step the HSD notes report.  Columns
    [vocab, ld) hold 100.0, which the walk must never read."""
    ld = vocab if ld is None else ld
    rng = np.random.default_rng(seed)
    n_trees = desc.n_branches
    rows = desc.total_nodes() + n_trees
    g = torch.Generator(device=device).manual_seed(seed)
    z = torch.randn(rows, ld, generator=g, device=device, dtype=dtype)
    z.mul_(1.5).clamp_(-10.0, 3.0)
    top = rng.integers(0, vocab, rows)
    p_rows, p_tok, p_val = [], [], []
    off = 0
    for b in range(n_trees):
        n = int(desc.n_nodes[b])
        par = desc.parent[off:off + n]
        row0 = off + b
        for r in range(n + 1):
            kids = np.nonzero(par == r - 1)[0]
            if len(kids) == 0 or rng.random() >= p_plant:
                continue
            c = int(kids[int(rng.integers(len(kids)))])
            t = int(tokens[off + c])
            if rng.random() < 0.7:
                top[row0 + r] = t
            elif t != top[row0 + r]:
                p_rows.append(row0 + r)
                p_tok.append(t)
                p_val.append(4.0 - rng.uniform(0.0, 0.6))
        off += n
    rix = torch.arange(rows, device=device)
    z[rix, torch.as_tensor(top, device=device)] = 4.0
    if p_rows:
        z[torch.as_tensor(p_rows, device=device), torch.as_tensor(p_tok, device=device)] = torch.as_tensor(
            p_val, device=device, dtype=torch.float32).to(dtype)
    if ld > vocab:
        z[:, vocab:] = 100.0
    return z


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def config(i: int, **kw) -> Workload:
    return CONFIGS[i](**kw)
