"""GPU parity: the HIP library against the fp64 oracle, element by element.

Tolerances (elementwise |gpu - ref| <= atol + rtol * |ref|): bf16 inputs
atol 2e-2 / rtol 1e-2; fp32 inputs 1e-5 / 1e-5.  Full-size workloads are
checked on sampled rows that the oracle computes one by one; small ones on
every row.  Every call goes through the C ABI via the ctypes binding.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (2e-2, 1e-2), torch.float32: (1e-5, 1e-5)}
LSE_TOL = {torch.bfloat16: (2e-3, 1e-3), torch.float32: (1e-5, 1e-5)}


def say(msg):
    print(msg, flush=True)


def close(got, ref, tol, what):
    atol, rtol = tol
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu={got[i]!r} ref={ref[i]!r} max_abs={err.max():.3g}")
    return float(err.max())


def cuda(t):
    return t.to("cuda").contiguous()


def gpu_prefill(w, plan=None, **kw):
    plan = plan or ta.plan_for(w.desc).upload()
    t = {k: cuda(v) for k, v in w.tensors.items()}
    o, lse = ta.prefill(plan, t["q"], t["k"], t["v"], scale=w.scale, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), (None if lse is None else lse.cpu().numpy())


def prefill_workload(P, L, C, hq=16, hkv=8, d=128, dtype=torch.bfloat16, seed=0, pages=None):
    rng = np.random.default_rng(seed)
    if pages is None:
        pages = [(P, L, C)]
    desc = synth.make_prefill_desc([p[0] for p in pages], [np.array(p[1]) for p in pages],
                                   [np.array(p[2]) for p in pages])
    w = synth.Workload("test", "prefill", desc, hq, hkv, d, dtype, seed=seed)
    w.tensors = synth.prefill_tensors(rng, desc, hq, hkv, d, dtype)
    return w


def check_prefill_full(w, tag):
    say(f"[prefill] {tag}: rows={w.desc.total_tokens()} hq={w.hq} hkv={w.hkv} d={w.head_dim} {w.dtype}")
    o, lse = gpu_prefill(w)
    ro, rl = oracle.prefill(w.desc, w.tensors["q"], w.tensors["k"], w.tensors["v"], w.scale)
    e1 = close(o, ro, TOL[w.dtype], f"{tag} o")
    e2 = close(lse, rl, LSE_TOL[w.dtype], f"{tag} lse")
    say(f"    max_abs o={e1:.3g} lse={e2:.3g}")


def test_prefill_config1_fp32_exactness():
    check_prefill_full(synth.config1(), "tiny fp32 tree (P=64, N=3)")


@pytest.mark.parametrize("case", [
    # ragged: several row tiles, empty layout units/branches, branches shorter
    # and longer than one 64-token tile, a tile spanning many short branches
    dict(pages=[(200, [3, 0, 5, 2, 1], [70, 0, 9, 130, 1]), (0, [4], [3]), (65, [], [])]),
    dict(pages=[(37, [1] * 12, [5, 6, 7, 1, 2, 3, 4, 5, 6, 7, 8, 9])]),
    dict(pages=[(1, [0], [200])]),
])
@pytest.mark.parametrize("heads", [(16, 8, 128), (8, 8, 64), (8, 2, 32), (4, 1, 128)])
def test_prefill_small_bf16(case, heads):
    hq, hkv, d = heads
    w = prefill_workload(None, None, None, hq=hq, hkv=hkv, d=d, pages=case["pages"], seed=hq * 7 + d)
    check_prefill_full(w, f"bf16 {case['pages'][0][:1]} heads={heads}")


@pytest.mark.parametrize("heads", [(4, 2, 128), (2, 2, 64)])
def test_prefill_small_fp32(heads):
    hq, hkv, d = heads
    w = prefill_workload(None, None, None, hq=hq, hkv=hkv, d=d, dtype=torch.float32,
                         pages=[(70, [2, 3, 0], [66, 0, 40]), (5, [1], [2])], seed=3)
    check_prefill_full(w, f"fp32 heads={heads}")


def sampled_prefill_check(w, n_per_page, seed):
    say(f"[prefill] {w.name}: rows={w.desc.total_tokens()} (sampled {n_per_page}/page)")
    o, lse = gpu_prefill(w)
    rng = np.random.default_rng(seed)
    q, k, v = w.tensors["q"], w.tensors["k"], w.tensors["v"]
    base = 0
    off = 0
    worst = 0.0
    for p in range(w.desc.n_pages):
        n = int(w.desc.n_regions[p])
        P = int(w.desc.prefix_len[p])
        L = w.desc.layout_len[off:off + n]
        C = w.desc.content_len[off:off + n]
        off += n
        T = P + int(L.sum()) + int(C.sum())
        M = P + int(L.sum())
        # always include the edges: first/last main row, first/last branch row
        rows = set(rng.choice(T, n_per_page, replace=False).tolist()) | {0, M - 1, M, T - 1}
        rows = np.array(sorted(r for r in rows if 0 <= r < T))
        mask = oracle.ancestor_mask_page(P, L, C)[rows]
        sl = slice(base, base + T)
        ro, rl = oracle.masked_attention(q[sl][rows], k[sl], v[sl], mask, w.scale)
        worst = max(worst, close(o[base + rows], ro, TOL[w.dtype], f"{w.name} page {p} o"))
        close(lse[:, base + rows], rl, LSE_TOL[w.dtype], f"{w.name} page {p} lse")
        base += T
    say(f"    max_abs o={worst:.3g}")


def test_prefill_config2_full_size_sampled():
    sampled_prefill_check(synth.config2(), 160, 1)


def test_prefill_config3_full_size_sampled():
    sampled_prefill_check(synth.config3(), 40, 2)


def test_prefill_deterministic():
    w = synth.config2()
    plan = ta.plan_for(w.desc).upload()
    a = gpu_prefill(w, plan)
    b = gpu_prefill(w, plan)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_prefill_without_lse():
    w = prefill_workload(None, None, None, pages=[(50, [2], [40])])
    o, _ = gpu_prefill(w, want_lse=False)
    ro, _ = oracle.prefill(w.desc, w.tensors["q"], w.tensors["k"], w.tensors["v"], w.scale)
    close(o, ro, TOL[w.dtype], "no-lse o")


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def gpu_decode(w, plan=None):
    plan = plan or ta.plan_for(w.desc).upload()
    t = {k: cuda(v) for k, v in w.tensors.items()}
    o, lse = ta.decode(plan, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], scale=w.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def decode_workload(P, N, L, branches, hq=16, hkv=8, d=128, dtype=torch.bfloat16, seed=0):
    """branches: list of (page, region, s) or (page, region, s, new tokens)."""
    rng = np.random.default_rng(seed)
    multi = any(len(b) > 3 for b in branches)
    desc = synth.DecodeDesc(np.array(P, np.int32), np.array(N, np.int32), np.array(L, np.int32),
                            np.array([b[0] for b in branches], np.int32),
                            np.array([b[1] for b in branches], np.int32),
                            np.array([b[2] for b in branches], np.int32),
                            np.array([b[3] if len(b) > 3 else 1 for b in branches], np.int32) if multi else None)
    w = synth.Workload("dec", "decode", desc, hq, hkv, d, dtype, seed=seed)
    w.tensors = synth.decode_tensors(rng, desc, hq, hkv, d, dtype)
    return w


def check_decode(w, rows=None, tag=""):
    say(f"[decode] {tag}: branches={w.desc.n_branches} rows={w.desc.n_rows()} hq={w.hq} d={w.head_dim} {w.dtype}")
    o, lse = gpu_decode(w)
    t = w.tensors
    ro, rl = oracle.decode(w.desc, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], w.scale,
                           rows=rows)
    rows = np.arange(w.desc.n_rows()) if rows is None else np.array(rows)
    e = close(o[rows], ro[rows], TOL[w.dtype], f"{tag} o")
    close(lse[:, rows], rl[:, rows], LSE_TOL[w.dtype], f"{tag} lse")
    say(f"    max_abs o={e:.3g}")


@pytest.mark.parametrize("heads,dtype", [((16, 8, 128), torch.bfloat16), ((4, 4, 64), torch.bfloat16),
                                         ((8, 2, 32), torch.bfloat16), ((4, 2, 128), torch.float32)])
def test_decode_small(heads, dtype):
    hq, hkv, d = heads
    # main streams longer than one decode chunk, empty suffixes (s = 0),
    # suffixes over one chunk, a page with no live branch, P = 0
    w = decode_workload([1500, 0, 7], [3, 2, 1], [5, 0, 1200, 3, 4, 2],
                        [(0, 1, 0), (0, 3, 2100), (0, 2, 70), (1, 2, 1), (1, 1, 0)],
                        hq=hq, hkv=hkv, d=d, dtype=dtype, seed=d)
    check_decode(w, tag=f"small heads={heads}")


def test_decode_config4_full_size_sampled():
    w = synth.config4()
    rng = np.random.default_rng(3)
    rows = sorted(set(rng.choice(w.desc.n_branches, 40, replace=False).tolist()) | {0, 23, 383})
    check_decode(w, rows=rows, tag="config4 16 pages x 24 branches")


@pytest.mark.parametrize("heads,dtype", [((16, 8, 128), torch.bfloat16), ((4, 4, 64), torch.bfloat16),
                                         ((8, 2, 32), torch.bfloat16), ((4, 2, 128), torch.float32)])
def test_decode_multi_small(heads, dtype):
    hq, hkv, d = heads
    # several new tokens per branch (1, 3, 8, 64, 65, 130), layout-stream
    # rows (region 0), suffixes over one chunk with a window, empty s, a page
    # with no regions, P = 0
    w = decode_workload([1500, 0, 7, 40], [3, 2, 1, 0], [5, 0, 1200, 3, 4, 2],
                        [(0, 0, 5, 8), (0, 1, 0, 3), (0, 3, 2100, 65), (0, 2, 70, 1), (1, 0, 0, 130),
                         (1, 2, 1, 64), (1, 1, 0, 8), (2, 1, 2047, 2), (3, 0, 3, 5)],
                        hq=hq, hkv=hkv, d=d, dtype=dtype, seed=d + 1)
    check_decode(w, tag=f"multi small heads={heads}")


def test_decode_multi_full_size_sampled():
    w = synth.decode_multi()
    rng = np.random.default_rng(5)
    n = w.desc.n_rows()
    rows = sorted(set(rng.choice(n, 60, replace=False).tolist()) | {0, 7, 8, 199, n - 1})
    check_decode(w, rows=rows, tag="16 pages x 25 rows x 8 tokens")


def test_decode_multi_equals_prefill_rows():
    """A branch's new tokens (a window, or its first tokens prefilled over the
    cached prefix) and a layout-stream window equal the packed prefill rows
    of the same tokens (both on the GPU, same K/V values)."""
    P, L, C = 90, [4, 70, 3], [40, 1, 130]
    s = [0, 0, 100]
    K = [C[i] - s[i] for i in range(3)]
    w = prefill_workload(P, L, C, seed=12)
    o_pf, l_pf = gpu_prefill(w)
    M = P + sum(L)
    t = w.tensors
    ddesc = synth.DecodeDesc(np.array([P], np.int32), np.array([3], np.int32), np.array(L, np.int32),
                             np.zeros(3, np.int32), np.array([1, 2, 3], np.int32), np.array(s, np.int32),
                             np.array(K, np.int32))
    rows = [M + sum(C[:i]) + s[i] + j for i in range(3) for j in range(K[i])]
    wd = synth.Workload("d", "decode", ddesc, 16, 8, 128, torch.bfloat16,
                        {"q": t["q"][rows], "k_main": t["k"][:M], "v_main": t["v"][:M],
                         "k_suffix": t["k"][M:], "v_suffix": t["v"][M:]})
    o_dc, l_dc = gpu_decode(wd)
    close(o_dc, o_pf[rows], (2e-2, 1e-2), "multi decode vs prefill o")
    close(l_dc, l_pf[:, rows], (2e-3, 1e-3), "multi decode vs prefill lse")
    # layout stream writing B_3: main = X, B_1, B_2; B_3's first token is
    # already in its suffix, the other two are new
    M2 = P + L[0] + L[1]
    ldesc = synth.DecodeDesc(np.array([P], np.int32), np.array([2], np.int32), np.array(L[:2], np.int32),
                             np.zeros(1, np.int32), np.zeros(1, np.int32), np.array([1], np.int32),
                             np.array([2], np.int32))
    rows = [M2 + 1, M2 + 2]
    wl = synth.Workload("l", "decode", ldesc, 16, 8, 128, torch.bfloat16,
                        {"q": t["q"][rows], "k_main": t["k"][:M2], "v_main": t["v"][:M2],
                         "k_suffix": t["k"][M2:M], "v_suffix": t["v"][M2:M]})
    o_ly, l_ly = gpu_decode(wl)
    close(o_ly, o_pf[rows], (2e-2, 1e-2), "layout rows vs prefill o")
    close(l_ly, l_pf[:, rows], (2e-3, 1e-3), "layout rows vs prefill lse")


def test_decode_equals_prefill_row():
    """decode(branch k, s) on the shared main + own suffix equals the packed
    prefill row of the same token (both on the GPU, same K/V values)."""
    P, L, s = 90, [4, 70, 3], [5, 0, 130]
    C = [x + 1 for x in s]
    w = prefill_workload(P, L, C, seed=11)
    o_pf, l_pf = gpu_prefill(w)
    M = P + sum(L)
    t = w.tensors
    ddesc = synth.DecodeDesc(np.array([P], np.int32), np.array([3], np.int32), np.array(L, np.int32),
                             np.zeros(3, np.int32), np.array([1, 2, 3], np.int32), np.array(s, np.int32))
    rows = [M + sum(C[:i]) + s[i] for i in range(3)]
    wd = synth.Workload("d", "decode", ddesc, 16, 8, 128, torch.bfloat16,
                        {"q": t["q"][rows], "k_main": t["k"][:M], "v_main": t["v"][:M],
                         "k_suffix": t["k"][M:], "v_suffix": t["v"][M:]})
    o_dc, l_dc = gpu_decode(wd)
    close(o_dc, o_pf[rows], (2e-2, 1e-2), "decode vs prefill o")
    close(l_dc, l_pf[:, rows], (2e-3, 1e-3), "decode vs prefill lse")


# --------------------------------------------------------------------------
# verify
# --------------------------------------------------------------------------

def gpu_verify(w, plan=None):
    plan = plan or ta.plan_for(w.desc).upload()
    t = {k: cuda(v) for k, v in w.tensors.items()}
    o, lse = ta.verify(plan, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], scale=w.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def verify_workload(ctx, trees, hq=16, hkv=8, d=128, dtype=torch.bfloat16, seed=0):
    """trees: list of (page, parent array)."""
    rng = np.random.default_rng(seed)
    desc = synth.VerifyDesc(np.array(ctx, np.int32), np.array([t[0] for t in trees], np.int32),
                            np.array([len(t[1]) for t in trees], np.int32),
                            np.concatenate([np.array(t[1], np.int32) for t in trees]) if trees else
                            np.zeros(0, np.int32))
    w = synth.Workload("ver", "verify", desc, hq, hkv, d, dtype, seed=seed)
    w.tensors = synth.verify_tensors(rng, desc, hq, hkv, d, dtype)
    return w


def check_verify(w, pages=None, tag=""):
    say(f"[verify] {tag}: nodes={w.desc.total_nodes()} hq={w.hq} d={w.head_dim} {w.dtype}")
    o, lse = gpu_verify(w)
    t = w.tensors
    ro, rl = oracle.verify(w.desc, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], w.scale, pages=pages)
    if pages is None:
        rows = np.arange(w.desc.total_nodes())
    else:
        node_off = np.concatenate([[0], np.cumsum(w.desc.n_nodes)])
        rows = np.concatenate([np.arange(node_off[b], node_off[b + 1]) for b in range(w.desc.n_branches)
                               if int(w.desc.br_page[b]) in pages])
    e = close(o[rows], ro[rows], TOL[w.dtype], f"{tag} o")
    close(lse[:, rows], rl[:, rows], LSE_TOL[w.dtype], f"{tag} lse")
    say(f"    max_abs o={e:.3g}")


@pytest.mark.parametrize("heads,dtype", [((16, 8, 128), torch.bfloat16), ((8, 4, 64), torch.bfloat16),
                                         ((4, 2, 32), torch.float32)])
def test_verify_small(heads, dtype):
    hq, hkv, d = heads
    rng = np.random.default_rng(d)
    trees = [(0, synth.random_tree_parents(rng, 32)), (0, synth.random_tree_parents(rng, 32)),
             (0, [-1]), (1, list(range(-1, 63))), (1, [-1, -1, 0, 1]), (2, synth.random_tree_parents(rng, 17))]
    w = verify_workload([300, 70, 0], trees, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=1)
    check_verify(w, tag=f"small heads={heads}")


def test_verify_config5_full_size_sampled():
    w = synth.config5()
    check_verify(w, pages=[0, 37, 63], tag="config5 64 pages x 8 trees x 32 nodes")


def test_verify_chain_equals_prefill_rows():
    """A chain draft tree over a context equals causal prefill rows of a page
    whose prefix is the context and whose single branch is the chain."""
    ctx, n = 150, 40
    w = prefill_workload(ctx, [0], [n], seed=12)
    o_pf, l_pf = gpu_prefill(w)
    t = w.tensors
    vdesc = synth.VerifyDesc(np.array([ctx], np.int32), np.array([0], np.int32), np.array([n], np.int32),
                             np.arange(-1, n - 1, dtype=np.int32))
    wv = synth.Workload("v", "verify", vdesc, 16, 8, 128, torch.bfloat16,
                        {"q": t["q"][ctx:], "k_ctx": t["k"][:ctx], "v_ctx": t["v"][:ctx],
                         "k_tree": t["k"][ctx:], "v_tree": t["v"][ctx:]})
    o_v, l_v = gpu_verify(wv)
    close(o_v, o_pf[ctx:], (2e-2, 1e-2), "chain verify vs prefill o")
    close(l_v, l_pf[:, ctx:], (2e-3, 1e-3), "chain verify vs prefill lse")


# --------------------------------------------------------------------------
# plans balanced by key-range splits (fp32 partials + fixed-order merge)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,heads", [(torch.bfloat16, (16, 8, 128)), (torch.float32, (4, 2, 32))])
def test_prefill_split_tiles_match_oracle(dtype, heads):
    hq, hkv, d = heads
    w = prefill_workload(None, None, None, hq=hq, hkv=hkv, d=d, dtype=dtype,
                         pages=[(1500, [4, 0, 9], [300, 5, 700]), (700, [2], [90])], seed=21)
    plan = ta.plan_for(w.desc).balance(hkv, 256)  # long tiles vs many slots: split
    assert plan.info["n_partials"] > 0
    plan.upload()
    say(f"[prefill split] pieces={plan.info['n_work']} partial slots={plan.info['n_partials']}")
    o, lse = gpu_prefill(w, plan)
    ro, rl = oracle.prefill(w.desc, w.tensors["q"], w.tensors["k"], w.tensors["v"], w.scale)
    close(o, ro, TOL[dtype], "split prefill o")
    close(lse, rl, LSE_TOL[dtype], "split prefill lse")


def test_prefill_config2_balanced_sampled_and_deterministic():
    w = synth.config2()
    plan = ta.plan_for(w.desc).balance(w.hkv).upload()
    say(f"[prefill balanced] pieces={plan.info['n_work']} partial slots={plan.info['n_partials']}")
    a = gpu_prefill(w, plan)
    b = gpu_prefill(w, plan)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # same values as the unsplit plan, within the merge's fp32 rounding
    c = gpu_prefill(w)
    close(a[0], c[0], (2e-2, 1e-2), "balanced vs unsplit o")
    rng = np.random.default_rng(31)
    T = w.desc.total_tokens()
    P = int(w.desc.prefix_len[0])
    rows = np.array(sorted(set(rng.choice(T, 120, replace=False).tolist()) | {0, T - 1}))
    mask = oracle.ancestor_mask_page(P, w.desc.layout_len, w.desc.content_len)[rows]
    ro, rl = oracle.masked_attention(w.tensors["q"][rows], w.tensors["k"], w.tensors["v"], mask, w.scale)
    close(a[0][rows], ro, TOL[w.dtype], "balanced config2 o")
    close(a[1][:, rows], rl, LSE_TOL[w.dtype], "balanced config2 lse")


def test_verify_split_tiles_match_oracle():
    rng = np.random.default_rng(41)
    trees = [(0, synth.random_tree_parents(rng, 32)), (0, synth.random_tree_parents(rng, 32)),
             (1, synth.random_tree_parents(rng, 20))]
    w = verify_workload([2500, 900], trees, seed=2)
    plan = ta.plan_for(w.desc).balance(w.hkv, 256)
    assert plan.info["n_partials"] > 0
    plan.upload()
    o, lse = gpu_verify(w, plan)
    t = w.tensors
    ro, rl = oracle.verify(w.desc, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], w.scale)
    close(o, ro, TOL[w.dtype], "split verify o")
    close(lse, rl, LSE_TOL[w.dtype], "split verify lse")


# --------------------------------------------------------------------------
# score range: a row's exp2 base may lag its running maximum; tiles whose
# scores rise far above it (up to overflowing exp2) must move it, tiles far
# below it must not lose it
# --------------------------------------------------------------------------

def scale_keys(k, kind):
    """Key rows times a factor of their position: 'rise' (scores grow along
    the stream, the last tiles some hundred binary orders above the first),
    'fall' (the reverse) or 'spike' (one stretch of keys 40 times larger)."""
    n = k.shape[0]
    pos = torch.arange(n, dtype=torch.float32)
    if kind == "rise":
        f = 1 + pos / 8
    elif kind == "fall":
        f = 1 + (n - 1 - pos) / 8
    else:
        f = torch.ones(n)
        f[n // 3:n // 3 + 20] = 40.0
    return (k.float() * f[:, None, None]).to(k.dtype)


def fp32_score_tol(q, k, v, scale):
    """fp32 inputs: the kernel's scores carry fp32 rounding of about
    sqrt(d) * 2^-24 * scale * sum|q_i k_i| (a property of fp32 dot products,
    not of the kernel), which perturbs every softmax weight by that relative
    amount and the output by up to twice it times max|v|.  At scores of a few
    hundred this passes the fixed 1e-5, so these cases widen the absolute
    term by that bound."""
    qa, ka = q.abs().double(), k.abs().double()
    g = qa.shape[1] // ka.shape[1]
    s_abs = max(float((qa[:, h] @ ka[:, h // g].T).max()) for h in range(qa.shape[1])) * scale
    d = q.shape[-1]
    return (1e-5 + 2 * np.sqrt(d) * 2.0 ** -24 * s_abs * float(v.abs().max()), 1e-5)


@pytest.mark.parametrize("kind", ["rise", "fall", "spike"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_score_range(kind, dtype):
    w = prefill_workload(None, None, None, hq=4, hkv=2, d=128, dtype=dtype,
                         pages=[(300, [3, 2, 0], [100, 80, 5])], seed=5)
    t = w.tensors
    t["k"] = scale_keys(t["k"], kind)
    say(f"[prefill] score range {kind} {dtype}")
    o, lse = gpu_prefill(w)
    ro, rl = oracle.prefill(w.desc, t["q"], t["k"], t["v"], w.scale)
    tol = TOL[dtype] if dtype == torch.bfloat16 else fp32_score_tol(t["q"], t["k"], t["v"], w.scale)
    e = close(o, ro, tol, f"{kind} o")
    close(lse, rl, LSE_TOL[dtype] if dtype == torch.bfloat16 else (tol[0], 1e-5), f"{kind} lse")
    say(f"    max_abs o={e:.3g} (atol {tol[0]:.3g})")


@pytest.mark.parametrize("kind", ["rise", "spike"])
def test_decode_score_range(kind):
    w = decode_workload([1500, 7], [3, 1], [5, 0, 1200, 3],
                        [(0, 1, 0), (0, 3, 2100), (0, 2, 70), (1, 1, 5)], hq=4, hkv=2, d=128, seed=6)
    w.tensors["k_main"] = scale_keys(w.tensors["k_main"], kind)
    w.tensors["k_suffix"] = scale_keys(w.tensors["k_suffix"], kind)
    check_decode(w, tag=f"score range {kind}")


@pytest.mark.parametrize("kind", ["rise", "spike"])
def test_verify_score_range(kind):
    rng = np.random.default_rng(8)
    trees = [(0, synth.random_tree_parents(rng, 32)), (0, list(range(-1, 63))), (1, [-1, 0, 0, 1])]
    w = verify_workload([700, 70], trees, hq=4, hkv=2, d=128, seed=9)
    w.tensors["k_ctx"] = scale_keys(w.tensors["k_ctx"], kind)
    w.tensors["k_tree"] = scale_keys(w.tensors["k_tree"], kind)
    check_verify(w, tag=f"score range {kind}")


def test_verify_unshared_full_size_sampled():
    """Verify with 512 independent prefixes (one 32-node tree per context,
    contexts ~ U{4096..16384}, 21.7 GB of K/V drawn on the GPU) in the launch
    configuration the bench times (balanced plan); the trees of pages 0, 255
    and 511 against the oracle."""
    w = synth.config5_unshared()
    t = synth.verify_tensors_device(41, w.desc, w.hq, w.hkv, w.head_dim, w.dtype)
    plan = ta.plan_for(w.desc).balance(w.hkv).upload()
    say(f"[verify] unshared: {w.desc.n_pages} contexts, {int(w.desc.ctx_len.sum())} context tokens")
    o, lse = ta.verify(plan, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], scale=w.scale)
    torch.cuda.synchronize()
    ctx_off = np.concatenate([[0], np.cumsum(w.desc.ctx_len.astype(np.int64))])
    node_off = np.concatenate([[0], np.cumsum(w.desc.n_nodes.astype(np.int64))])
    for p in (0, 255, 511):  # page p holds tree p
        c0, c1, n0, n1 = int(ctx_off[p]), int(ctx_off[p + 1]), int(node_off[p]), int(node_off[p + 1])
        sub = synth.VerifyDesc(w.desc.ctx_len[p:p + 1], np.zeros(1, np.int32), w.desc.n_nodes[p:p + 1],
                               w.desc.parent[n0:n1])
        ro, rl = oracle.verify(sub, t["q"][n0:n1].cpu(), t["k_ctx"][c0:c1].cpu(), t["v_ctx"][c0:c1].cpu(),
                               t["k_tree"][n0:n1].cpu(), t["v_tree"][n0:n1].cpu(), w.scale)
        e = close(o[n0:n1].float().cpu().numpy(), ro, TOL[w.dtype], f"unshared page {p} o")
        close(lse[:, n0:n1].cpu().numpy(), rl, LSE_TOL[w.dtype], f"unshared page {p} lse")
        say(f"    page {p}: ctx {c1 - c0}, max_abs o={e:.3g}")
