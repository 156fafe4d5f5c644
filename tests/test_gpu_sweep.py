"""Seeded random sweep of small descriptions through prefill, decode and
verify, every row against the oracle (the same tolerances as the parity
tests: bf16 2e-2 / 1e-2, fp32 1e-5, lse 2e-3 / 1e-3 in bf16).

Lengths are drawn from sets that sit on and around the 64-token tile
(0, 1, 63, 64, 65, 128) and from small random values, so prefix, layout
and content boundaries fall inside, at the start and at the end of tiles;
trees are chains, random trees of depth <= 8, single nodes and 64-node
chains.  Each case prints its description first, so a failure names it.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth

pytestmark = pytest.mark.gpu

EDGE = [0, 1, 63, 64, 65, 128]
HEADS = [(16, 8, 128, torch.bfloat16), (8, 2, 64, torch.bfloat16), (4, 4, 32, torch.bfloat16),
         (4, 1, 128, torch.bfloat16), (4, 2, 64, torch.float32), (2, 1, 32, torch.float32)]
TOL = {torch.bfloat16: ((2e-2, 1e-2), (2e-3, 1e-3)), torch.float32: ((1e-5, 1e-5), (1e-5, 1e-5))}


def pick_len(rng, hi=300):
    return int(rng.choice(EDGE)) if rng.random() < 0.6 else int(rng.integers(0, hi))


def close(got, ref, tol, what):
    atol, rtol = tol
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside; max_abs={err.max():.3g}"


def heads_for(seed):
    return HEADS[seed % len(HEADS)]


@pytest.mark.parametrize("seed", range(24))
def test_prefill_random_description(seed):
    rng = np.random.default_rng(1000 + seed)
    hq, hkv, d, dtype = heads_for(seed)
    pages = []
    for _ in range(int(rng.integers(1, 4))):
        n = int(rng.integers(0, 7))
        P = pick_len(rng, 400)
        L = [int(rng.choice([0, 1, 3, 12, 64, 65])) for _ in range(n)]
        C = [pick_len(rng, 250) for _ in range(n)]
        pages.append((P, L, C))
    if sum(P + sum(L) + sum(C) for P, L, C in pages) == 0:
        pages.append((5, [1], [3]))
    print(f"[sweep] prefill seed={seed} heads={(hq, hkv, d)} {dtype} pages={pages}", flush=True)
    desc = synth.make_prefill_desc([p[0] for p in pages], [np.array(p[1], np.int32) for p in pages],
                                   [np.array(p[2], np.int32) for p in pages])
    t = synth.prefill_tensors(rng, desc, hq, hkv, d, dtype)
    plan = ta.plan_for(desc)
    if seed % 3 == 2:
        plan.balance(hkv, 32)  # split row tiles: fp32 partials and the merge
    plan.upload()
    g = {k: v.cuda() for k, v in t.items()}
    o, lse = ta.prefill(plan, g["q"], g["k"], g["v"], scale=d ** -0.5)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(desc, t["q"], t["k"], t["v"], d ** -0.5)
    close(o.float().cpu().numpy(), ro, TOL[dtype][0], "o")
    close(lse.cpu().numpy(), rl, TOL[dtype][1], "lse")


@pytest.mark.parametrize("seed", range(16))
def test_decode_random_description(seed):
    rng = np.random.default_rng(2000 + seed)
    hq, hkv, d, dtype = heads_for(seed)
    n_pages = int(rng.integers(1, 4))
    P, N, L, bp, br, s, kq = [], [], [], [], [], [], []
    for p in range(n_pages):
        n = int(rng.integers(0, 5))
        P.append(pick_len(rng, 600))
        N.append(n)
        L += [int(rng.choice([0, 1, 12, 64])) for _ in range(n)]
        for _ in range(int(rng.integers(0, 5))):
            bp.append(p)
            br.append(int(rng.integers(0, n + 1)))  # 0: the page's layout stream
            s.append(pick_len(rng, 300))
            kq.append(int(rng.choice([1, 1, 2, 8, 64, 65])))
    if not bp:
        bp, br, s, kq = [0], [0], [3], [1]
    desc = synth.DecodeDesc(np.array(P, np.int32), np.array(N, np.int32), np.array(L, np.int32),
                            np.array(bp, np.int32), np.array(br, np.int32), np.array(s, np.int32),
                            np.array(kq, np.int32))
    print(f"[sweep] decode seed={seed} heads={(hq, hkv, d)} {dtype} P={P} N={N} L={L} rows="
          f"{list(zip(bp, br, s, kq))}", flush=True)
    if desc.main_tokens().sum() + desc.suffix_tokens() == 0:
        pytest.skip("empty")
    t = synth.decode_tensors(rng, desc, hq, hkv, d, dtype)
    plan = ta.plan_for(desc).upload()
    g = {k: v.cuda() for k, v in t.items()}
    o, lse = ta.decode(plan, g["q"], g["k_main"], g["v_main"], g["k_suffix"], g["v_suffix"], scale=d ** -0.5)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(desc, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], d ** -0.5)
    close(o.float().cpu().numpy(), ro, TOL[dtype][0], "o")
    close(lse.cpu().numpy(), rl, TOL[dtype][1], "lse")


@pytest.mark.parametrize("seed", range(16))
def test_verify_random_description(seed):
    rng = np.random.default_rng(3000 + seed)
    hq, hkv, d, dtype = heads_for(seed)
    n_pages = int(rng.integers(1, 4))
    ctx = [pick_len(rng, 700) for _ in range(n_pages)]
    trees = []
    for p in range(n_pages):
        for _ in range(int(rng.integers(0, 5))):
            kind = int(rng.integers(0, 4))
            if kind == 0:
                par = np.arange(-1, int(rng.integers(1, 65)) - 1)  # a chain, up to 64 nodes
            elif kind == 1:
                par = synth.random_tree_parents(rng, int(rng.integers(1, 65)))  # depth <= 8
            elif kind == 2:
                par = np.array([-1])
            else:  # several roots hanging off the context
                n = int(rng.integers(2, 20))
                par = np.array([-1 if rng.random() < 0.3 or i == 0 else int(rng.integers(0, i)) for i in range(n)])
            trees.append((p, par.astype(np.int32)))
    if not trees:
        trees = [(0, np.array([-1], np.int32))]
    desc = synth.VerifyDesc(np.array(ctx, np.int32), np.array([t[0] for t in trees], np.int32),
                            np.array([len(t[1]) for t in trees], np.int32),
                            np.concatenate([t[1] for t in trees]).astype(np.int32))
    print(f"[sweep] verify seed={seed} heads={(hq, hkv, d)} {dtype} ctx={ctx} trees="
          f"{[(p, len(x)) for p, x in trees]}", flush=True)
    t = synth.verify_tensors(rng, desc, hq, hkv, d, dtype)
    plan = ta.plan_for(desc)
    if seed % 3 == 2:
        plan.balance(hkv, 32)
    plan.upload()
    g = {k: v.cuda() for k, v in t.items()}
    o, lse = ta.verify(plan, g["q"], g["k_ctx"], g["v_ctx"], g["k_tree"], g["v_tree"], scale=d ** -0.5)
    torch.cuda.synchronize()
    ro, rl = oracle.verify(desc, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], d ** -0.5)
    close(o.float().cpu().numpy(), ro, TOL[dtype][0], "o")
    close(lse.cpu().numpy(), rl, TOL[dtype][1], "lse")


@pytest.mark.parametrize("entry", ["prefill", "decode", "verify"])
def test_largest_head_group(entry):
    """32 query heads on one KV head (the largest group the library takes):
    sixteen head pairs per KV head, every entry point against the oracle."""
    hq, hkv, d, dtype = 32, 1, 64, torch.bfloat16
    rng = np.random.default_rng(4242)
    print(f"[sweep] group 32 {entry}", flush=True)
    if entry == "prefill":
        desc = synth.make_prefill_desc([130, 7], [np.array([2, 1]), np.array([1])], [np.array([65, 3]), np.array([64])])
        t = synth.prefill_tensors(rng, desc, hq, hkv, d, dtype)
        plan = ta.plan_for(desc).upload()
        g = {k: v.cuda() for k, v in t.items()}
        o, lse = ta.prefill(plan, g["q"], g["k"], g["v"], scale=d ** -0.5)
        torch.cuda.synchronize()
        ro, rl = oracle.prefill(desc, t["q"], t["k"], t["v"], d ** -0.5)
    elif entry == "decode":
        desc = synth.DecodeDesc(np.array([150, 64], np.int32), np.array([2, 1], np.int32),
                                np.array([4, 12, 0], np.int32), np.array([0, 0, 1], np.int32),
                                np.array([1, 2, 0], np.int32), np.array([3, 70, 0], np.int32),
                                np.array([1, 8, 2], np.int32))
        t = synth.decode_tensors(rng, desc, hq, hkv, d, dtype)
        plan = ta.plan_for(desc).upload()
        g = {k: v.cuda() for k, v in t.items()}
        o, lse = ta.decode(plan, g["q"], g["k_main"], g["v_main"], g["k_suffix"], g["v_suffix"], scale=d ** -0.5)
        torch.cuda.synchronize()
        ro, rl = oracle.decode(desc, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], d ** -0.5)
    else:
        par = synth.random_tree_parents(rng, 20).astype(np.int32)
        desc = synth.VerifyDesc(np.array([100, 65], np.int32), np.array([0, 1, 1], np.int32),
                                np.array([20, 1, 3], np.int32),
                                np.concatenate([par, np.array([-1, -1, 0, 1], np.int32)]))
        t = synth.verify_tensors(rng, desc, hq, hkv, d, dtype)
        plan = ta.plan_for(desc).upload()
        g = {k: v.cuda() for k, v in t.items()}
        o, lse = ta.verify(plan, g["q"], g["k_ctx"], g["v_ctx"], g["k_tree"], g["v_tree"], scale=d ** -0.5)
        torch.cuda.synchronize()
        ro, rl = oracle.verify(desc, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], d ** -0.5)
    close(o.float().cpu().numpy(), ro, TOL[dtype][0], "o")
    close(lse.cpu().numpy(), rl, TOL[dtype][1], "lse")
