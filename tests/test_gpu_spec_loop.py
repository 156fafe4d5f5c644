"""Three rounds of the speculative loop that the draft-tree, paged-verify,
acceptance and pool entry points make up together, on the GPU, with random
K/V and logits standing in for a model: per page, build the draft tree from
the accepted tokens and the drafts (host), verify it over the page's context
read through its block table, walk it with the logits, and append the
accepted nodes' K/V plus the free token's to the page's pooled context.
Every round is checked against the oracle (attention on the gathered
context, the greedy walk) and the pooled context against the K/V the loop
appended."""
import numpy as np
import pytest
import torch

import oracle
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth

pytestmark = pytest.mark.gpu


def test_speculative_rounds():
    rng = np.random.default_rng(77)
    dev = "cuda"
    hq, hkv, d, bs, vocab = 8, 2, 64, 64, 500
    n_pages = 2
    pool = ta.KVPool(64, bs)
    ck = torch.zeros((64 * bs, hkv, d), dtype=torch.bfloat16, device=dev)
    cv = torch.zeros_like(ck)
    roots, ctx_k, ctx_v, accepted, drafts = [], [], [], [], []
    for p in range(n_pages):
        n0 = int(rng.integers(100, 300))
        r = pool.new_seq()
        k = torch.randn((n0, hkv, d)).to(torch.bfloat16)
        v = torch.randn((n0, hkv, d)).to(torch.bfloat16)
        s = torch.as_tensor(pool.append(r, n0), device=dev)
        ck[s], cv[s] = k.to(dev), v.to(dev)
        roots.append(r)
        ctx_k.append(k)
        ctx_v.append(v)
        accepted.append(rng.integers(0, vocab, 6).tolist())
    for rnd in range(3):
        # drafts that hold the accepted tail (so candidates exist) and noise
        for p in range(n_pages):
            tail = accepted[p][-3:]
            drafts_p = [tail + rng.integers(0, vocab, 8).tolist(),
                        rng.integers(0, vocab, 5).tolist() + tail + rng.integers(0, vocab, 4).tolist(),
                        tail + rng.integers(0, vocab, 3).tolist()]
            drafts = drafts[:p] + [drafts_p] + drafts[p + 1:]
        trees = [ta.draft_tree(accepted[p], drafts[p], 3, 16, 4) for p in range(n_pages)]
        n_nodes = [len(t[0]) for t in trees]
        assert min(n_nodes) > 0, "the drafts hold the window, so every tree has nodes"
        parent = np.concatenate([t[1] for t in trees])
        ctx_len = [pool.table(r)[3] for r in roots]
        tables = [pool.table(r)[2] for r in roots]
        plan = ta.plan_verify_paged(ctx_len, list(range(n_pages)), n_nodes, parent, bs, pool.n_blocks, tables)
        plan.upload()
        n = int(sum(n_nodes))
        q = torch.randn((n, hq, d)).to(torch.bfloat16)
        kt = torch.randn((n, hkv, d)).to(torch.bfloat16)
        vt = torch.randn((n, hkv, d)).to(torch.bfloat16)
        o, lse = ta.verify(plan, q.to(dev), ck, cv, kt.to(dev), vt.to(dev), scale=d ** -0.5)
        torch.cuda.synchronize()
        # oracle on the context gathered back through the block tables
        desc = synth.VerifyDesc(np.array(ctx_len, np.int32), np.arange(n_pages, dtype=np.int32),
                                np.array(n_nodes, np.int32), parent.astype(np.int32))
        kc = torch.cat([oracle.gather_paged(ck.cpu(), tables[p], ctx_len[p], bs) for p in range(n_pages)])
        vc = torch.cat([oracle.gather_paged(cv.cpu(), tables[p], ctx_len[p], bs) for p in range(n_pages)])
        assert torch.equal(kc, torch.cat(ctx_k)) and torch.equal(vc, torch.cat(ctx_v))
        ro, rl = oracle.verify(desc, q, kc, vc, kt, vt, d ** -0.5)
        err = np.abs(o.float().cpu().numpy() - ro)
        assert (err <= 2e-2 + 1e-2 * np.abs(ro)).all(), (rnd, err.max())
        # the walk over logits for each tree
        toks = np.concatenate([t[0] for t in trees]).astype(np.int32)
        logits = synth.accept_logits(100 + rnd, desc, toks, vocab, vocab, torch.float32, dev)
        path, n_path, nxt = ta.accept(plan, logits, torch.as_tensor(toks, device=dev))
        torch.cuda.synchronize()
        z = logits.cpu().numpy()
        off = 0
        for p in range(n_pages):
            m = n_nodes[p]
            got = (path[off:off + int(n_path[p])].tolist(), int(nxt[p]))
            want = oracle.tree_accept(toks[off:off + m], parent[off:off + m], z[off + p:off + p + m + 1], 0.75)
            assert got == want, (rnd, p, got, want)
            # append the accepted nodes' K/V and a new K/V for the free token
            nodes = [off + i for i in got[0]]
            k_new = torch.cat([kt[nodes], torch.randn((1, hkv, d)).to(torch.bfloat16)])
            v_new = torch.cat([vt[nodes], torch.randn((1, hkv, d)).to(torch.bfloat16)])
            s = torch.as_tensor(pool.append(roots[p], len(nodes) + 1), device=dev)
            ck[s], cv[s] = k_new.to(dev), v_new.to(dev)
            ctx_k[p] = torch.cat([ctx_k[p], k_new])
            ctx_v[p] = torch.cat([ctx_v[p], v_new])
            accepted[p] += [int(toks[i]) for i in nodes] + [got[1]]
            off += m
    for p in range(n_pages):
        v, vl, own, ol = pool.table(roots[p])
        assert ol == ctx_k[p].shape[0]
        assert torch.equal(oracle.gather_paged(ck.cpu(), own, ol, bs), ctx_k[p])
