"""fp64 CPU oracle: plain masked-softmax attention over an explicit ancestor mask.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the library
imports this file, and this file imports nothing from the library.  It is
deliberately slow and direct: the visibility rule is written out as a dense
boolean mask, and attention is softmax(scale * q k^T, masked by selection) v,
all in float64.  Inputs of any dtype are upcast exactly to float64.

Sources (page titles and sections):
  [PaDoc] "PaDoc: Layout-Grounded Parallel Decoding for Document Parsing"
      (paper summary page), sections "Formal assumptions and factorization"
      (depth formulas D_seq and D_PaDoc), "Training paradigm" (ancestor sets
      Anc(B_k) = {X, B_<k}, Anc(Y_k) = {X, B_<=k}; the layout stream is one
      causal sequence; branch Y_k queries attend the virtual key/value
      sequence [X, B_<=k, Y_k]), "Inference" (request-level serving with
      shared-prefix KV reuse gives the same visibility as the fused mask).
  [HPD] "HPD-Parsing: Hierarchical Parallel Document Parsing" (paper notes),
      section "Prerequisites: KV cache and shared-prefix reuse" (forked
      branches reference the parent's prefix KV, zero-copy).
  [HSD] "HSD: Training-Free Acceleration for Document Parsing Vision-Language
      Models with Hierarchical Speculative Decoding" (paper notes), key design
      3 (b) "prefix-tree batching": a linearised draft prefix tree under the
      tree ancestor mask, each token seeing the accepted sequence plus its own
      ancestor path.

Readings taken where the pages are silent (listed again in the design notes):
  * packed order per page is [X | B_1..B_N | Y_1..Y_N], pages concatenated;
  * X is the causal head of the layout stream;
  * every token sees itself (diagonal included), for main, branch and tree;
  * GQA query head h reads KV head h // (Hq / Hkv);
  * decode: the current token's K/V is already appended to its branch, so a
    branch row with s_k earlier tokens sees main[0 : P + L_<=k] plus its own
    s_k + 1 suffix tokens;
  * verify: node i sees its page's whole context plus anc*(i) (ancestors and
    itself) inside its own branch's tree;
  * LSE is the natural-log log-sum-exp of the scaled, masked scores.
"""
from __future__ import annotations

import numpy as np

_ROW_BLOCK = 1024


def _f64(x) -> np.ndarray:
    """Exact upcast to float64 (bf16 and fp32 values are representable)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Visibility, written as sets ([PaDoc] "Training paradigm")
# ---------------------------------------------------------------------------

def _page_labels(P: int, L, C):
    """Label every packed token of one page.

    Returns (is_main, region, index):
      main tokens (X then B_1..B_N): is_main=True, index = position in the
        layout stream, region = 0 for X and k for tokens of B_k;
      content tokens of Y_k: is_main=False, region = k, index = t (0-based
        position inside Y_k).
    """
    L = [int(x) for x in L]
    C = [int(x) for x in C]
    is_main, region, index = [], [], []
    for i in range(P):
        is_main.append(True); region.append(0); index.append(i)
    pos = P
    for k, lk in enumerate(L, start=1):
        for _ in range(lk):
            is_main.append(True); region.append(k); index.append(pos); pos += 1
    for k, ck in enumerate(C, start=1):
        for t in range(ck):
            is_main.append(False); region.append(k); index.append(t)
    return np.array(is_main, bool), np.array(region, np.int64), np.array(index, np.int64)


def ancestor_mask_page(P: int, L, C) -> np.ndarray:
    """Dense boolean mask A[i, j] = token i may attend to token j, one page.

    * main query i, main key j: the layout stream (with X at its head) is one
      causal sequence, so j <= i in the stream.
    * content query Y_k[t], main key j: j is in X or in B_m with m <= k
      (Anc(Y_k) = {X, B_<=k}).
    * content query Y_k[t], content key Y_m[u]: same branch (m = k) and
      u <= t (causal inside the branch); never another branch.
    """
    is_main, region, index = _page_labels(P, L, C)
    qm, km = is_main[:, None], is_main[None, :]
    qr, kr = region[:, None], region[None, :]
    qi, ki = index[:, None], index[None, :]
    main_main = qm & km & (ki <= qi)
    cont_main = (~qm) & km & (kr <= qr)
    cont_cont = (~qm) & (~km) & (kr == qr) & (ki <= qi)
    return main_main | cont_main | cont_cont


def tree_ancestor_mask(parent) -> np.ndarray:
    """A[i, j] = node j is node i itself or one of its ancestors ([HSD] 3(b))."""
    parent = [int(p) for p in parent]
    n = len(parent)
    a = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        while j >= 0:
            a[i, j] = True
            j = parent[j]
    return a


# ---------------------------------------------------------------------------
# Attention by definition
# ---------------------------------------------------------------------------

def masked_attention(q, k, v, mask, scale: float):
    """softmax(scale * q k^T with non-visible scores replaced by -inf) @ v.

    q: [Tq, Hq, d]; k, v: [Tk, Hkv, d]; mask: [Tq, Tk] bool (shared by heads).
    Returns o [Tq, Hq, d] float64 and lse [Hq, Tq] float64 (natural log).
    Scores are masked by selection, so non-visible keys never contribute.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    o = np.zeros((tq, hq, d))
    lse = np.zeros((hq, tq))
    for h in range(hq):
        kh, vh = k[:, h // g, :], v[:, h // g, :]
        for r0 in range(0, tq, _ROW_BLOCK):
            r1 = min(tq, r0 + _ROW_BLOCK)
            s = scale * (q[r0:r1, h, :] @ kh.T)
            s = np.where(mask[r0:r1], s, -np.inf)
            m = s.max(axis=1)
            p = np.exp(s - m[:, None])
            l = p.sum(axis=1)
            o[r0:r1, h, :] = (p @ vh) / l[:, None]
            lse[h, r0:r1] = m + np.log(l)
    return o, lse


def masked_attention_backward(q, k, v, do, mask, scale: float):
    """Gradients of o = masked_attention(q, k, v, mask, scale) for the output
    gradient do, written out from the definition in float64.

    With S = scale q k^T (non-visible entries -inf), P = row softmax of S and
    o = P v:
      dv = P^T do,  dP = do v^T,  dS_ij = P_ij (dP_ij - sum_l P_il dP_il),
      dq = scale dS k,  dk = scale dS^T q.
    A KV head's gradients sum over the query heads that read it (GQA).
    Returns dq [Tq, Hq, d], dk and dv [Tk, Hkv, d].
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        kh, vh = k[:, h // g, :], v[:, h // g, :]
        for r0 in range(0, tq, _ROW_BLOCK):
            r1 = min(tq, r0 + _ROW_BLOCK)
            s = scale * (q[r0:r1, h, :] @ kh.T)
            s = np.where(mask[r0:r1], s, -np.inf)
            m = s.max(axis=1)
            p = np.exp(s - m[:, None])
            p /= p.sum(axis=1)[:, None]
            dp = do[r0:r1, h, :] @ vh.T
            ds = p * (dp - (p * dp).sum(axis=1)[:, None])
            dv[:, h // g, :] += p.T @ do[r0:r1, h, :]
            dq[r0:r1, h, :] = scale * (ds @ kh)
            dk[:, h // g, :] += scale * (ds.T @ q[r0:r1, h, :])
    return dq, dk, dv


def lse_merge(parts):
    """Combine attention results over disjoint key sets from (o, lse) pairs.

    o = sum_i exp(lse_i - lse) o_i with lse = log sum_i exp(lse_i); this is
    the identity behind serving a branch as a request whose KV is the shared
    prefix plus its own suffix ([PaDoc] "Inference").
    """
    lses = np.stack([p[1] for p in parts])          # [n, Hq, T]
    top = lses.max(axis=0)
    w = np.exp(lses - top)
    tot = w.sum(axis=0)
    lse = top + np.log(tot)
    o = sum(np.transpose(w[i] / tot)[:, :, None] * parts[i][0] for i in range(len(parts)))
    return o, lse


def _page_offsets(prefix_len, n_regions, layout_len, content_len):
    off_r, off_t = 0, 0
    for p in range(len(prefix_len)):
        n = int(n_regions[p])
        P = int(prefix_len[p])
        L = [int(x) for x in layout_len[off_r:off_r + n]]
        C = [int(x) for x in content_len[off_r:off_r + n]] if content_len is not None else None
        yield p, P, L, C, off_t
        off_r += n
        if C is not None:
            off_t += P + sum(L) + sum(C)


def prefill(desc, q, k, v, scale: float):
    """Packed tree-varlen forward over every page ([PaDoc] "Training paradigm").

    q: [T, Hq, d], k/v: [T, Hkv, d] in packed order.  Returns o [T, Hq, d] and
    lse [Hq, T] in float64.  Pages never see each other.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, hq, d = q.shape
    o = np.zeros((T, hq, d))
    lse = np.zeros((hq, T))
    for p, P, L, C, base in _page_offsets(desc.prefix_len, desc.n_regions, desc.layout_len, desc.content_len):
        tp = P + sum(L) + sum(C)
        if tp == 0:
            continue
        sl = slice(base, base + tp)
        mask = ancestor_mask_page(P, L, C)
        o[sl], lse[:, sl] = masked_attention(q[sl], k[sl], v[sl], mask, scale)
    return o, lse


def prefill_backward(desc, q, k, v, do, scale: float):
    """Gradients of the packed tree-varlen forward (``prefill``) with respect
    to q, k and v for the output gradient do, page by page under the same
    ancestor mask.  The training path the PaDoc summary describes
    ("Training paradigm") differentiates exactly this forward.
    Returns dq [T, Hq, d], dk and dv [T, Hkv, d] in float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for p, P, L, C, base in _page_offsets(desc.prefix_len, desc.n_regions, desc.layout_len, desc.content_len):
        tp = P + sum(L) + sum(C)
        if tp == 0:
            continue
        sl = slice(base, base + tp)
        mask = ancestor_mask_page(P, L, C)
        dq[sl], dk[sl], dv[sl] = masked_attention_backward(q[sl], k[sl], v[sl], do[sl], mask, scale)
    return dq, dk, dv


def prefill_backward_sampled(desc, q, k, v, do, scale: float, rows, keys):
    """dq of the packed rows ``rows`` and dk, dv of the packed tokens
    ``keys``, from the same definition as ``prefill_backward`` but one row or
    one key column at a time (for pages too large for the dense gradient).
    Uses the fp64 forward (o, lse) of every page.  Returns dq [len(rows), Hq,
    d], dk and dv [len(keys), Hkv, d]."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    T, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    o, lse = prefill(desc, q, k, v, scale)
    dd = (do * o).sum(axis=2)  # [T, Hq]
    rows, keys = [int(r) for r in rows], [int(j) for j in keys]
    dq = np.zeros((len(rows), hq, d))
    dk = np.zeros((len(keys), hkv, d))
    dv = np.zeros((len(keys), hkv, d))
    for p, P, L, C, base in _page_offsets(desc.prefix_len, desc.n_regions, desc.layout_len, desc.content_len):
        tp = P + sum(L) + sum(C)
        mine_r = [(n, r - base) for n, r in enumerate(rows) if base <= r < base + tp]
        mine_k = [(n, j - base) for n, j in enumerate(keys) if base <= j < base + tp]
        if not mine_r and not mine_k:
            continue
        sl = slice(base, base + tp)
        mask = ancestor_mask_page(P, L, C)
        qp, kp, vp, dop = q[sl], k[sl], v[sl], do[sl]
        for h in range(hq):
            kh, vh = kp[:, h // g, :], vp[:, h // g, :]
            for n, i in mine_r:
                s = np.where(mask[i], scale * (kh @ qp[i, h]), -np.inf)
                pr = np.exp(s - lse[h, base + i])
                ds = pr * (vh @ dop[i, h] - dd[base + i, h])
                dq[n, h] = scale * (ds @ kh)
            for n, j in mine_k:
                s = np.where(mask[:, j], scale * (qp[:, h, :] @ kh[j]), -np.inf)
                pr = np.exp(s - lse[h, sl])
                ds = pr * (dop[:, h, :] @ vh[j] - dd[sl, h])
                dk[n, h // g] += scale * (ds @ qp[:, h, :])
                dv[n, h // g] += pr @ dop[:, h, :]
    return dq, dk, dv


def decode(desc, q, k_main, v_main, k_suffix, v_suffix, scale: float, rows=None):
    """Branch decode over the shared main stream ([PaDoc] "Inference"; [HPD]
    shared prefix), one or more new tokens per live branch.

    Branch b (page p, region k, s_k earlier tokens, K_b new tokens) owns the
    suffix rows suffix_b[0 : s_k + K_b]; its query row j (0 <= j < K_b) is
    suffix token s_k + j and attends to main_p[0 : P + L_<=k] ++
    suffix_b[0 : s_k + j + 1] (causal among the new tokens).  Region k = 0 is
    the page's layout stream, which sees the whole main stream.  Rows are
    branch-major.  ``rows`` optionally restricts the computation to some rows
    (others are returned as zeros).
    """
    q = _f64(q)
    nr, hq, d = q.shape
    main_off = np.zeros(desc.n_pages + 1, dtype=np.int64)
    reg_off = np.zeros(desc.n_pages + 1, dtype=np.int64)
    for p in range(desc.n_pages):
        n = int(desc.n_regions[p])
        reg_off[p + 1] = reg_off[p] + n
        main_off[p + 1] = main_off[p] + int(desc.prefix_len[p]) + int(desc.layout_len[reg_off[p]:reg_off[p + 1]].sum())
    kq = desc.queries()
    suf_off = np.concatenate([[0], np.cumsum(desc.suffix_len.astype(np.int64) + kq)])
    row_off = np.concatenate([[0], np.cumsum(kq)])
    o = np.zeros((nr, hq, d))
    lse = np.zeros((hq, nr))
    todo = set(range(nr)) if rows is None else set(int(r) for r in rows)
    for b in range(desc.n_branches):
        p = int(desc.br_page[b])
        kreg = int(desc.br_region[b])
        n_reg = kreg if kreg > 0 else int(desc.n_regions[p])  # layout stream: all of B
        lay = desc.layout_len[reg_off[p]:reg_off[p] + n_reg]
        visible_main = int(desc.prefix_len[p]) + int(lay.sum())
        m0 = int(main_off[p])
        s0 = int(suf_off[b])
        s = int(desc.suffix_len[b])
        for j in range(int(kq[b])):
            r = int(row_off[b]) + j
            if r not in todo:
                continue
            kk = np.concatenate([_f64(k_main[m0:m0 + visible_main]), _f64(k_suffix[s0:s0 + s + j + 1])])
            vv = np.concatenate([_f64(v_main[m0:m0 + visible_main]), _f64(v_suffix[s0:s0 + s + j + 1])])
            mask = np.ones((1, kk.shape[0]), dtype=bool)
            ob, lb = masked_attention(q[r:r + 1], kk, vv, mask, scale)
            o[r] = ob[0]
            lse[:, r] = lb[:, 0]
    return o, lse


def verify(desc, q, k_ctx, v_ctx, k_tree, v_tree, scale: float, pages=None):
    """Draft-tree verification ([HSD] key design 3 (b)).

    Node i of branch b sees its page's whole context and the tree nodes of its
    own branch that are i itself or its ancestors.  Rows are nodes,
    branch-major.  ``pages`` optionally restricts the computation.
    """
    q = _f64(q)
    n, hq, d = q.shape
    ctx_off = np.concatenate([[0], np.cumsum(desc.ctx_len.astype(np.int64))])
    node_off = np.concatenate([[0], np.cumsum(desc.n_nodes.astype(np.int64))])
    o = np.zeros((n, hq, d))
    lse = np.zeros((hq, n))
    todo = range(desc.n_pages) if pages is None else pages
    for p in todo:
        brs = [b for b in range(desc.n_branches) if int(desc.br_page[b]) == p]
        if not brs:
            continue
        rows = np.concatenate([np.arange(node_off[b], node_off[b + 1]) for b in brs])
        if rows.size == 0:
            continue
        c0, c1 = int(ctx_off[p]), int(ctx_off[p + 1])
        nr = rows.size
        mask = np.zeros((nr, (c1 - c0) + nr), dtype=bool)
        mask[:, : c1 - c0] = True
        r = 0
        for b in brs:
            nb = int(desc.n_nodes[b])
            a = tree_ancestor_mask(desc.parent[node_off[b]:node_off[b + 1]])
            mask[r:r + nb, (c1 - c0) + r:(c1 - c0) + r + nb] = a
            r += nb
        kk = np.concatenate([_f64(k_ctx[c0:c1]), _f64(k_tree[rows])])
        vv = np.concatenate([_f64(v_ctx[c0:c1]), _f64(v_tree[rows])])
        op, lp = masked_attention(q[rows], kk, vv, mask, scale)
        o[rows] = op
        lse[:, rows] = lp
    return o, lse


# ---------------------------------------------------------------------------
# Integer plan reference
# ---------------------------------------------------------------------------

def depth(P: int, L, C):
    """Critical-path depths ([PaDoc] "Formal assumptions and factorization").

    D_seq = l(B_1:N) + sum_k l(Y_k); D_PaDoc = max_k [l(B_<=k) + l(Y_k)]
    (0 for a page without regions).  The prefix X is given, not decoded.
    """
    L = [int(x) for x in L]
    C = [int(x) for x in C]
    d_seq = sum(L) + sum(C)
    d_par = 0
    acc = 0
    for lk, ck in zip(L, C):
        acc += lk
        d_par = max(d_par, acc + ck)
    return d_par, d_seq


def plan_prefill(desc):
    """Integer fields of the prefill plan, from the visibility definition.

    Per packed token (absolute indices):
      position      index in its virtual sequence (main stream, or
                    [X, B_<=k, Y_k] for a content token)
      main_end      visible main keys are [page_base, main_end)
      branch_start  visible branch keys are [branch_start, token] (empty,
                    i.e. token + 1, for main tokens)
    Per page: base, main length M, packed length T, D, D_seq.
    Per branch (page-major): main_bound, branch_start, branch_len.
    """
    pos, mend, bstart = [], [], []
    pages, branches = [], []
    for p, P, L, C, base in _page_offsets(desc.prefix_len, desc.n_regions, desc.layout_len, desc.content_len):
        M = P + sum(L)
        T = M + sum(C)
        for i in range(M):
            pos.append(i); mend.append(base + i + 1); bstart.append(base + i + 1)
        acc_l, acc_c = 0, 0
        for lk, ck in zip(L, C):
            acc_l += lk
            b0 = base + M + acc_c
            branches.append((base + P + acc_l, b0, ck))
            for t in range(ck):
                pos.append(P + acc_l + t); mend.append(base + P + acc_l); bstart.append(b0)
            acc_c += ck
        dp, ds = depth(P, L, C)
        pages.append((base, M, T, dp, ds))
    return {
        "position": np.array(pos, np.int64),
        "main_end": np.array(mend, np.int64),
        "branch_start": np.array(bstart, np.int64),
        "pages": np.array(pages, np.int64).reshape(-1, 5),
        "branches": np.array(branches, np.int64).reshape(-1, 3),
    }


def plan_decode(desc):
    """Per query row (branch-major): main_start, main_len (= P + L_<=k, the
    whole main stream for a layout row), suffix_start, visible suffix length
    (= s_k + j + 1 for new token j), position (= main_len + s_k + j)."""
    rows = []
    main_off = 0
    reg_off = 0
    starts, regs = [], []
    for p in range(desc.n_pages):
        n = int(desc.n_regions[p])
        starts.append(main_off)
        regs.append(reg_off)
        main_off += int(desc.prefix_len[p]) + int(desc.layout_len[reg_off:reg_off + n].sum())
        reg_off += n
    suf = 0
    kq = desc.queries()
    for b in range(desc.n_branches):
        p = int(desc.br_page[b])
        k = int(desc.br_region[b])
        if k == 0:
            k = int(desc.n_regions[p])
        lay = int(desc.layout_len[regs[p]:regs[p] + k].sum())
        mlen = int(desc.prefix_len[p]) + lay
        s = int(desc.suffix_len[b])
        for j in range(int(kq[b])):
            rows.append((starts[p], mlen, suf, s + j + 1, mlen + s + j))
        suf += s + int(kq[b])
    return {"rows": np.array(rows, np.int64).reshape(-1, 5)}


def plan_verify(desc):
    """Per node (branch-major): ancestor bitmask (bit j = node j of the same
    branch is the node itself or an ancestor), ctx_start, ctx_len, tree_base
    (absolute index of the branch's node 0), position (= ctx_len + depth)."""
    ctx_off = np.concatenate([[0], np.cumsum(desc.ctx_len.astype(np.int64))])
    node_off = np.concatenate([[0], np.cumsum(desc.n_nodes.astype(np.int64))])
    rows, masks = [], []
    for b in range(desc.n_branches):
        p = int(desc.br_page[b])
        par = desc.parent[node_off[b]:node_off[b + 1]]
        a = tree_ancestor_mask(par)
        for i in range(a.shape[0]):
            bits = 0
            for j in range(a.shape[1]):
                if a[i, j]:
                    bits |= 1 << j
            masks.append(bits)
            rows.append((int(ctx_off[p]), int(desc.ctx_len[p]), int(node_off[b]),
                         int(desc.ctx_len[p]) + int(a[i].sum()) - 1))
    return {"mask": np.array(masks, dtype=np.uint64), "rows": np.array(rows, np.int64).reshape(-1, 4)}
