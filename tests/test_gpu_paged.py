"""GPU tests of the paged KV path: decode and verify through block tables
(blocks handed out by the host pool, shared prefix blocks viewed by forked
branches, scrambled physical order) give bit-identical results to the same
launches on contiguous buffers, which the parity tests check against the
oracle; one case is also checked against the oracle directly."""
import numpy as np
import pytest
import torch

import oracle
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth
from test_paged import paged_decode_setup

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def to_cache(nb, bs, pieces, like):
    """A [nb * bs, Hkv, d] cache holding each (slots, rows) piece."""
    cache = torch.zeros((nb * bs,) + tuple(like.shape[1:]), dtype=like.dtype, device="cuda")
    for slots, rows in pieces:
        if len(slots):
            cache[torch.as_tensor(slots, device="cuda")] = rows.cuda()
    return cache


def run_paged_decode(w, bs, seed):
    desc, t = w.desc, w.tensors
    rng = np.random.default_rng(seed)
    pool, nb, mt, st, main_slots, suf_slots = paged_decode_setup(desc, bs, rng)
    main = desc.main_tokens()
    m_off = np.concatenate([[0], np.cumsum(main)])
    suf = desc.suffix_len.astype(np.int64) + desc.queries()
    s_off = np.concatenate([[0], np.cumsum(suf)])
    pieces_k = [(main_slots[p], t["k_main"][m_off[p]:m_off[p + 1]]) for p in range(desc.n_pages)]
    pieces_k += [(suf_slots[b], t["k_suffix"][s_off[b]:s_off[b + 1]]) for b in range(desc.n_branches)]
    pieces_v = [(main_slots[p], t["v_main"][m_off[p]:m_off[p + 1]]) for p in range(desc.n_pages)]
    pieces_v += [(suf_slots[b], t["v_suffix"][s_off[b]:s_off[b + 1]]) for b in range(desc.n_branches)]
    ck, cv = to_cache(nb, bs, pieces_k, t["k_main"]), to_cache(nb, bs, pieces_v, t["v_main"])
    plan = ta.plan_decode_paged(desc.prefix_len, desc.n_regions, desc.layout_len, desc.br_page, desc.br_region,
                                desc.suffix_len, desc.queries(), bs, nb, mt, st).upload()
    q = t["q"].cuda()
    o, lse = ta.decode(plan, q, ck, cv, ck, cv, scale=w.scale)
    plan_c = ta.plan_for(desc).upload()
    o_c, lse_c = ta.decode(plan_c, q, t["k_main"].cuda(), t["v_main"].cuda(), t["k_suffix"].cuda(),
                           t["v_suffix"].cuda(), scale=w.scale)
    torch.cuda.synchronize()
    return o, lse, o_c, lse_c


def small_multi(dtype, seed):
    rng = np.random.default_rng(seed)
    desc = synth.DecodeDesc(np.array([1500, 0, 7, 40], np.int32), np.array([3, 2, 1, 0], np.int32),
                            np.array([5, 0, 1200, 3, 4, 2], np.int32), np.array([0, 0, 0, 0, 1, 1, 1, 2, 3], np.int32),
                            np.array([0, 1, 3, 2, 0, 2, 1, 1, 0], np.int32),
                            np.array([5, 0, 2100, 70, 0, 1, 0, 2047, 3], np.int32),
                            np.array([8, 3, 65, 1, 130, 64, 8, 2, 5], np.int32))
    w = synth.Workload("paged", "decode", desc, 8, 2, 64, dtype, seed=seed)
    w.tensors = synth.decode_tensors(rng, desc, 8, 2, 64, dtype)
    return w


@pytest.mark.parametrize("bs", [64, 128, 1024])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_paged_decode_bit_identical_small(bs, dtype):
    w = small_multi(dtype, 3)
    say(f"[paged decode] small bs={bs} {dtype}")
    o, lse, o_c, lse_c = run_paged_decode(w, bs, bs)
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)


def test_paged_decode_matches_oracle():
    w = small_multi(torch.bfloat16, 4)
    o, lse, _, _ = run_paged_decode(w, 64, 1)
    t = w.tensors
    ro, rl = oracle.decode(w.desc, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], w.scale)
    err = np.abs(o.float().cpu().numpy() - ro)
    assert (err <= 2e-2 + 1e-2 * np.abs(ro)).all(), err.max()
    assert np.abs(lse.cpu().numpy() - rl).max() < 2e-3 + 1e-3 * np.abs(rl).max()


@pytest.mark.parametrize("which,bs", [("config4", 256), ("multi", 64)])
def test_paged_decode_bit_identical_full_size(which, bs):
    w = synth.config4() if which == "config4" else synth.decode_multi()
    say(f"[paged decode] {w.name} bs={bs}")
    o, lse, o_c, lse_c = run_paged_decode(w, bs, 7)
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)


@pytest.mark.parametrize("bs", [64, 512])
def test_paged_verify_bit_identical(bs):
    w = synth.config5(n_pages=6)
    desc, t = w.desc, w.tensors
    say(f"[paged verify] 6 pages bs={bs}")
    pool = ta.KVPool(sum((int(c) + bs - 1) // bs for c in desc.ctx_len) + 20, bs)
    junk = pool.new_seq()
    pool.append(junk, 3 * bs)
    roots, slots = [], []
    for p in range(desc.n_pages):
        r = pool.new_seq()
        slots.append(pool.append(r, int(desc.ctx_len[p])))
        roots.append(r)
        if p == 1:
            pool.release(junk)
    tables = [pool.table(r)[2] for r in roots]
    c_off = np.concatenate([[0], np.cumsum(desc.ctx_len.astype(np.int64))])
    nb = pool.n_blocks
    ck = to_cache(nb, bs, [(slots[p], t["k_ctx"][c_off[p]:c_off[p + 1]]) for p in range(desc.n_pages)], t["k_ctx"])
    cv = to_cache(nb, bs, [(slots[p], t["v_ctx"][c_off[p]:c_off[p + 1]]) for p in range(desc.n_pages)], t["v_ctx"])
    plan = ta.plan_verify_paged(desc.ctx_len, desc.br_page, desc.n_nodes, desc.parent, bs, nb, tables).upload()
    q, kt, vt = t["q"].cuda(), t["k_tree"].cuda(), t["v_tree"].cuda()
    o, lse = ta.verify(plan, q, ck, cv, kt, vt, scale=w.scale)
    plan_c = ta.plan_for(desc).upload()
    o_c, lse_c = ta.verify(plan_c, q, t["k_ctx"].cuda(), t["v_ctx"].cuda(), kt, vt, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)


def test_paged_verify_balanced_bit_identical():
    """A paged verify plan balanced into split row tiles (pieces start on tile
    boundaries of the paged context) equals the contiguous plan balanced the
    same way."""
    w = synth.config5(n_pages=3)
    desc, t = w.desc, w.tensors
    bs = 128
    pool = ta.KVPool(sum((int(c) + bs - 1) // bs for c in desc.ctx_len) + 4, bs)
    junk = pool.new_seq()
    pool.append(junk, 2 * bs)
    roots, slots = [], []
    for p in range(desc.n_pages):
        r = pool.new_seq()
        slots.append(pool.append(r, int(desc.ctx_len[p])))
        roots.append(r)
    pool.release(junk)
    tables = [pool.table(r)[2] for r in roots]
    c_off = np.concatenate([[0], np.cumsum(desc.ctx_len.astype(np.int64))])
    nb = pool.n_blocks
    ck = to_cache(nb, bs, [(slots[p], t["k_ctx"][c_off[p]:c_off[p + 1]]) for p in range(desc.n_pages)], t["k_ctx"])
    cv = to_cache(nb, bs, [(slots[p], t["v_ctx"][c_off[p]:c_off[p + 1]]) for p in range(desc.n_pages)], t["v_ctx"])
    plan = ta.plan_verify_paged(desc.ctx_len, desc.br_page, desc.n_nodes, desc.parent, bs, nb, tables)
    plan.balance(w.hkv, 256)
    plan_c = ta.plan_for(desc).balance(w.hkv, 256)
    assert plan.info["n_partials"] > 0 and plan.info["n_partials"] == plan_c.info["n_partials"]
    plan.upload()
    plan_c.upload()
    q, kt, vt = t["q"].cuda(), t["k_tree"].cuda(), t["v_tree"].cuda()
    o, lse = ta.verify(plan, q, ck, cv, kt, vt, scale=w.scale)
    o_c, lse_c = ta.verify(plan_c, q, t["k_ctx"].cuda(), t["v_ctx"].cuda(), kt, vt, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)
