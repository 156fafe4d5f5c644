"""Benchmark of the tree attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of every forward entry point over resident synthetic
inputs:
  prefill  the packed batch of eight pages: P = 4096, N ~ U{12..40} regions
           of 12 layout tokens, lognormal content, 77,400 tokens (seed 2),
           16q/8kv heads, d = 128, bf16 -- the headline `value`
  decode   16 pages x 24 live branches, P = 4809, s_k ~ U{0..1024}
  verify   64 pages x 8 draft trees of 32 nodes, contexts ~ U{4096..16384}
           shared by the trees of a page
Timed in the same loop and reported under `entries`, outside the step: the
one-page prefill (8,772 tokens, seed 1), verify with 512 independent
prefixes (one tree per context), the prefill backward (dq, dk, dv of the
one-page workload), the greedy acceptance walk over the verify trees (bf16
logits, 151,936-entry vocabulary), a multi-token decode (8-token windows for
the decode pages' 24 branches plus one layout-stream row per page) and the
decode workload read from a paged cache of 64-token blocks.

Each entry point is bracketed by HIP events on the stream it is launched on
(torch's current stream).  Every entry reports both roofline components --
algorithmic FLOPs (4 d Hq per visible pair; 8 d Hq in the backward) and
algorithmic bytes (every distinct input byte read once, every output byte
written once) over the average launch time -- against MI355X's published
peaks (2.5 PFLOP/s dense bf16, 8 TB/s) and against the peaks two
calibration loops reach on this GPU (an MFMA loop and a streaming read).
The fp64 CPU oracle is timed on bounded samples of the prefill, decode and
verify workloads on this host's cores.  One JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from tree_structured_attention_amd import binding as ta  # noqa: E402
from tree_structured_attention_amd import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "tree-attn prefill tokens/s + %MFMA peak; branch-decode tokens/s + %HBM BW"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def elt(dtype):
    return 2 if dtype == torch.bfloat16 else 4


def scratch_for(plan, w):
    n = ta.scratch_bytes(plan, w.hq, w.head_dim)
    return torch.empty(n + 256, dtype=torch.uint8, device="cuda") if n else None


# --zero-inputs (diagnostic): the prefill entries run on all-zero q / k / v
ZERO_INPUTS = False


def prefill_case(w=None, name="prefill", in_step=True):
    """Packed prefill over a balanced plan (row tiles split so the launch
    fills the chip); the host plan's steady-state cost is timed on a second
    build."""
    w = w or synth.config3()
    ta.plan_for(w.desc).balance(w.hkv)
    t0 = time.perf_counter()
    plan = ta.plan_for(w.desc).balance(w.hkv)
    plan_us = (time.perf_counter() - t0) * 1e6
    plan.upload()
    t = {k: v.cuda() for k, v in w.tensors.items()}
    if ZERO_INPUTS:
        for x in t.values():
            x.zero_()
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.hq, t["q"].shape[0]), dtype=torch.float32, device="cuda")
    scratch = scratch_for(plan, w)
    info = plan.info

    def run():
        ta.prefill(plan, t["q"], t["k"], t["v"], scale=w.scale, out=o, lse=lse, scratch=scratch)

    e = elt(w.dtype)
    rows = info["n_rows"]
    # q, k, v read once, o and lse written once
    bytes_ = rows * (2 * w.hq + 2 * w.hkv) * w.head_dim * e + rows * w.hq * 4
    flops = 4.0 * w.head_dim * w.hq * info["visible_pairs"]
    return dict(name=name, w=w, plan=plan, run=run, unit_count=rows, unit="packed tokens", flops=flops,
                bytes=bytes_, bound="mfma", plan_us=plan_us, in_step=in_step,
                kernel="attn_kernel<bf16,128,2,prefill> (+ merge_kernel for split tiles)")


def prefill_1page_case():
    """The one-page prefill (P = 4096, 24 regions, 8,772 tokens)."""
    return prefill_case(synth.config2(), "prefill_1page", in_step=False)


def decode_case(w=None, name="decode"):
    w = w or synth.config4()
    ta.plan_for(w.desc)
    t0 = time.perf_counter()
    plan = ta.plan_for(w.desc)
    plan_us = (time.perf_counter() - t0) * 1e6
    plan.upload()
    t = {k: v.cuda() for k, v in w.tensors.items()}
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.hq, t["q"].shape[0]), dtype=torch.float32, device="cuda")
    scratch = scratch_for(plan, w)
    info = plan.info
    rows = plan.export("decode_rows")  # main_start, main_len, suffix_start, visible suffix, position

    def run():
        ta.decode(plan, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], scale=w.scale,
                  out=o, lse=lse, scratch=scratch)

    # distinct keys any row reads: per page the longest visible main prefix, plus every suffix token
    main_keys = 0
    for start in np.unique(rows[:, 0]):
        main_keys += int(rows[rows[:, 0] == start, 1].max())
    suffix_keys = w.desc.suffix_tokens()
    e = elt(w.dtype)
    kv_bytes = (main_keys + suffix_keys) * w.hkv * w.head_dim * 2 * e
    qo_bytes = info["n_rows"] * w.hq * w.head_dim * 2 * e + info["n_rows"] * w.hq * 4
    flops = 4.0 * w.head_dim * w.hq * info["visible_pairs"]
    return dict(name=name, w=w, plan=plan, run=run, unit_count=info["n_rows"], unit="query tokens",
                flops=flops, bytes=kv_bytes + qo_bytes, bound="hbm", plan_us=plan_us, in_step=name == "decode",
                kernel="attn_kernel<bf16,128,2,decode> + merge_kernel")


def decode_paged_case():
    """The decode workload with every main stream and suffix in a paged cache
    of 64-token blocks from the host pool (branches fork their page's main
    stream without copying it): timed beside the step."""
    w = synth.config4()
    desc, t = w.desc, w.tensors
    bs = 64
    main = desc.main_tokens()
    suf = desc.suffix_len.astype(np.int64) + desc.queries()
    nb = int(sum((int(m) + bs - 1) // bs for m in main) + sum((int(s) + bs - 1) // bs for s in suf)) + 64
    pool = ta.KVPool(nb, bs)
    reg_off = np.concatenate([[0], np.cumsum(desc.n_regions.astype(np.int64))])
    m_off = np.concatenate([[0], np.cumsum(main)])
    s_off = np.concatenate([[0], np.cumsum(suf)])
    roots, slots_k = [], []
    ck = torch.zeros((nb * bs,) + tuple(t["k_main"].shape[1:]), dtype=t["k_main"].dtype, device="cuda")
    cv = torch.zeros_like(ck)
    for p in range(desc.n_pages):
        r = pool.new_seq()
        s = torch.as_tensor(pool.append(r, int(main[p])), device="cuda")
        ck[s] = t["k_main"][m_off[p]:m_off[p + 1]].cuda()
        cv[s] = t["v_main"][m_off[p]:m_off[p + 1]].cuda()
        roots.append(r)
    # host cost of a step's bookkeeping: fork every branch, give it room for
    # its suffix, build the paged plan
    st, suffix_slots = [], []
    t0 = time.perf_counter()
    for b in range(desc.n_branches):
        p = int(desc.br_page[b])
        k = int(desc.br_region[b]) or int(desc.n_regions[p])
        bound = int(desc.prefix_len[p]) + int(desc.layout_len[reg_off[p]:reg_off[p] + k].sum())
        c = pool.fork(roots[p], bound)
        suffix_slots.append(pool.append(c, int(suf[b])))
        st.append(pool.table(c)[2])
    mt = [pool.table(r)[2] for r in roots]
    plan = ta.plan_decode_paged(desc.prefix_len, desc.n_regions, desc.layout_len, desc.br_page, desc.br_region,
                                desc.suffix_len, None, bs, nb, mt, st)
    plan_us = (time.perf_counter() - t0) * 1e6
    for b in range(desc.n_branches):
        s = torch.as_tensor(suffix_slots[b], device="cuda")
        ck[s] = t["k_suffix"][s_off[b]:s_off[b + 1]].cuda()
        cv[s] = t["v_suffix"][s_off[b]:s_off[b + 1]].cuda()
    plan.upload()
    q = t["q"].cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, q.shape[0]), dtype=torch.float32, device="cuda")
    scratch = scratch_for(plan, w)
    info = plan.info

    def run():
        ta.decode(plan, q, ck, cv, ck, cv, scale=w.scale, out=o, lse=lse, scratch=scratch)

    e = elt(w.dtype)
    kv_bytes = (int(main.sum()) + int(suf.sum())) * w.hkv * w.head_dim * 2 * e
    qo_bytes = info["n_rows"] * w.hq * w.head_dim * 2 * e + info["n_rows"] * w.hq * 4
    return dict(name="decode_paged", w=w, plan=plan, run=run, unit_count=info["n_rows"], unit="query tokens",
                flops=4.0 * w.head_dim * w.hq * info["visible_pairs"], bytes=kv_bytes + qo_bytes, bound="hbm",
                plan_us=plan_us, in_step=False, kernel="attn_kernel<bf16,128,2,decode> + merge_kernel (paged)")


def decode_multi_case():
    """Drafted windows of 8 new tokens for every live row of the decode pages,
    plus one layout-stream row per page: timed beside the step."""
    return decode_case(synth.decode_multi(), "decode_multi")


def verify_case(w=None, name="verify", in_step=True, tensors=None):
    w = w or synth.config5()
    ta.plan_for(w.desc).balance(w.hkv)
    t0 = time.perf_counter()
    plan = ta.plan_for(w.desc).balance(w.hkv)
    plan_us = (time.perf_counter() - t0) * 1e6
    plan.upload()
    t = tensors if tensors is not None else {k: v.cuda() for k, v in w.tensors.items()}
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.hq, t["q"].shape[0]), dtype=torch.float32, device="cuda")
    scratch = scratch_for(plan, w)
    info = plan.info

    def run():
        ta.verify(plan, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], scale=w.scale, out=o, lse=lse,
                  scratch=scratch)

    e = elt(w.dtype)
    flops = 4.0 * w.head_dim * w.hq * info["visible_pairs"]
    bytes_ = ((info["n_keys_a"] + info["n_keys_b"]) * w.hkv * w.head_dim * 2 * e
              + info["n_rows"] * w.hq * w.head_dim * 2 * e + info["n_rows"] * w.hq * 4)
    bound = "mfma" if flops / (PEAK_BF16_TFLOPS * 1e12) >= bytes_ / (PEAK_HBM_GBS * 1e9) else "hbm"
    return dict(name=name, w=w, plan=plan, run=run, unit_count=info["n_rows"], unit="draft nodes",
                flops=flops, bytes=bytes_, bound=bound, plan_us=plan_us, in_step=in_step,
                kernel="attn_kernel<bf16,128,2,verify> (+ merge_kernel for split tiles)")


def verify_unshared_case():
    """The 512 draft trees of the verify workload, each over a prefix of its
    own (512 contexts ~ U{4096..16384}, 21.7 GB of K/V): the HBM-bound
    reading of the verify workload.  Inputs drawn on the GPU."""
    w = synth.config5_unshared()
    t = synth.verify_tensors_device(41, w.desc, w.hq, w.hkv, w.head_dim, w.dtype)
    return verify_case(w, "verify_unshared", in_step=False, tensors=t)


def backward_case():
    """Prefill backward (dq, dk, dv) of the one-page workload: timed beside the
    step, not inside it (the step is the forward hot path)."""
    w = synth.config2()
    plan = ta.plan_for(w.desc)  # the backward walks an unbalanced plan
    plan.upload()
    t = {k: v.cuda() for k, v in w.tensors.items()}
    rng = np.random.default_rng(101)
    g = torch.from_numpy(rng.standard_normal(tuple(t["q"].shape), dtype=np.float32)).to(torch.bfloat16).cuda()
    o, lse = ta.prefill(plan, t["q"], t["k"], t["v"], scale=w.scale)
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    need = ta.backward_scratch_bytes(plan, w.hq)
    scratch = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    info = plan.info

    def run():
        ta.prefill_backward(plan, t["q"], t["k"], t["v"], o, lse, g, scale=w.scale, dq=dq, dk=dk, dv=dv,
                            scratch=scratch)

    # dv = P^T dO, dP = dO V^T, dq = dS K, dk = dS^T Q: 4 products of 2 d flops
    # per visible pair and query head (the recomputed S is not counted)
    flops = 8.0 * w.head_dim * w.hq * info["visible_pairs"]
    # q, o, dO (Hq heads), k, v (Hkv) and lse read once; dq, dk, dv written once
    rows = info["n_rows"]
    bytes_ = rows * (4 * w.hq + 4 * w.hkv) * w.head_dim * 2 + rows * w.hq * 4
    return dict(name="backward", w=w, plan=plan, run=run, unit_count=rows, unit="packed tokens",
                flops=flops, bytes=bytes_, bound="mfma", plan_us=0.0, in_step=False,
                kernel="bwd_prep_kernel<128> + bwd_fused_kernel<128> (row tiles, then key tiles) + bwd_kmerge_kernel<128>")


def accept_case():
    """Greedy acceptance over the verify workload's draft trees (64 pages x 8
    branches x 32 nodes) from bf16 logits over a 151,936-entry vocabulary:
    timed beside the step, not inside it.  The host part (window match and
    prefix-tree build from page-shaped drafts, then the verify plan) is timed
    on the CPU and reported as its plan time."""
    w = synth.config5(with_tensors=False)
    desc = w.desc
    vocab = synth.VOCAB
    rng = np.random.default_rng(21)
    # host: one tree per branch from 6 region drafts of 100-800 tokens whose
    # last accepted tokens occur in them
    drafts = [[rng.integers(0, vocab, int(rng.integers(100, 800))).astype(np.int32) for _ in range(6)]
              for _ in range(8)]
    t0 = time.perf_counter()
    for b in range(desc.n_branches):
        ds = drafts[b % 8]
        src = ds[b % 6]
        cut = 3 + (b * 37) % (len(src) - 3)
        ta.draft_tree(src[:cut], ds, 3, 32, 8)
    plan = ta.plan_for(desc)
    plan_us = (time.perf_counter() - t0) * 1e6
    plan.upload()
    tokens = torch.as_tensor(synth.draft_tokens(rng, desc, vocab), device="cuda")
    logits = synth.accept_logits(22, desc, tokens.cpu().numpy(), vocab, vocab, torch.bfloat16, "cuda")
    n_trees = desc.n_branches
    path = torch.empty(desc.total_nodes(), dtype=torch.int32, device="cuda")
    n_path = torch.empty(n_trees, dtype=torch.int32, device="cuda")
    nxt = torch.empty(n_trees, dtype=torch.int32, device="cuda")
    scratch = torch.empty(ta.accept_scratch_bytes(plan, vocab) + 256, dtype=torch.uint8, device="cuda")

    def run():
        ta.accept(plan, logits, tokens, tau=0.75, path=path, n_path=n_path, next_token=nxt, scratch=scratch)

    # every logits row is read once; the tree tables, tokens and results are
    # a few hundred KB and left out
    bytes_ = float(logits.numel() * 2)
    return dict(name="accept", w=w, plan=plan, run=run, unit_count=n_trees, unit="draft trees",
                flops=0.0, bytes=bytes_, bound="hbm", plan_us=plan_us, in_step=False,
                kernel="row_argmax_kernel<bf16> + tree_walk_kernel<bf16>")


def traffic_for(entry):
    """HBM bytes per launch of an entry point's kernels, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it was taken on the current
    kernel sources (else None)."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)["entries"][entry]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, "tree_structured_attention_amd", "csrc", src), "rb") as f:
                h.update(f.read())
    except (OSError, ValueError, KeyError):
        return None
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec.get("bytes_per_launch")


def host_cpu():
    """The host's cores as the oracle sees them: os.cpu_count(), the cores
    this process may run on, the BLAS thread count and the CPU model."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"cpu_count": os.cpu_count(), "usable_cores": affinity, "blas_threads": int(threads), "cpu_model": model}


def _baseline(done, elapsed, unit, cpu, sample):
    return {"value": done / elapsed, "unit": unit, "cores": cpu["blas_threads"], "kind": "oracle",
            "sample": sample, "seconds": elapsed, **cpu}


def cpu_prefill(w, budget_s, cpu):
    """The fp64 oracle on the packed prefill batch: pages in a random order,
    each page's dense ancestor mask built (and timed), then its rows in a
    random order in blocks of 256, until the budget is spent."""
    import oracle  # test infrastructure: used only for this reported baseline
    desc, t = w.desc, w.tensors
    rng = np.random.default_rng(0)
    reg = np.concatenate([[0], np.cumsum(desc.n_regions.astype(np.int64))])
    tok = np.concatenate([[0], np.cumsum(desc.page_tokens())])
    done, pages_seen = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for p in rng.permutation(desc.n_pages):
            L = desc.layout_len[reg[p]:reg[p + 1]]
            C = desc.content_len[reg[p]:reg[p + 1]]
            base, T = int(tok[p]), int(tok[p + 1] - tok[p])
            mask = oracle.ancestor_mask_page(int(desc.prefix_len[p]), L, C)
            pages_seen += 1
            order = rng.permutation(T)
            for i in range(0, T, 256):
                rows = np.sort(order[i:i + 256])
                oracle.masked_attention(t["q"][base + rows], t["k"][base:base + T], t["v"][base:base + T],
                                        mask[rows], w.scale)
                done += len(rows)
                if time.perf_counter() - t0 >= budget_s:
                    break
            if time.perf_counter() - t0 >= budget_s:
                break
    el = time.perf_counter() - t0
    return _baseline(done, el, "packed tokens/s", cpu,
                     f"{done} rows of the {desc.total_tokens()}-token {desc.n_pages}-page prefill batch "
                     f"({pages_seen} page masks built), random rows in blocks of 256, all {w.hq} heads, fp64 numpy "
                     f"with the dense ancestor mask, {el:.1f} s")


def cpu_decode(w, budget_s, cpu):
    """The fp64 decode oracle on rows in a random order, 16 at a time."""
    import oracle
    t = w.tensors
    n = w.desc.n_rows()
    order = np.random.default_rng(0).permutation(n)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        start = done % n
        rows = order[start:min(n, start + 16)]
        oracle.decode(w.desc, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], w.scale, rows=rows)
        done += len(rows)
    el = time.perf_counter() - t0
    return _baseline(done, el, "query tokens/s", cpu,
                     f"{done} of the {n} branch rows (16 per call, random order), all {w.hq} heads, fp64 numpy, "
                     f"{el:.1f} s")


def cpu_verify(w, budget_s, cpu):
    """The fp64 verify oracle page by page (a page's 8 trees together, its
    context and tree mask explicit), pages in a random order."""
    import oracle
    t = w.tensors
    desc = w.desc
    per_page = np.bincount(desc.br_page, weights=desc.n_nodes, minlength=desc.n_pages).astype(np.int64)
    done, pages = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for p in np.random.default_rng(pages).permutation(desc.n_pages):
            oracle.verify(desc, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], w.scale, pages=[int(p)])
            done += int(per_page[p])
            pages += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    el = time.perf_counter() - t0
    return _baseline(done, el, "draft nodes/s", cpu,
                     f"{pages} of the {desc.n_pages} pages ({done} draft nodes), all {w.hq} heads, fp64 numpy with "
                     f"the explicit tree mask, {el:.1f} s")


def calibrate():
    """Attainable peaks on this GPU: the best rate of the MFMA loop and of
    the streaming read over a few launch shapes, three launches each."""
    def timed(fn, reps=3):
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            work = fn()
            b.record()
            torch.cuda.synchronize()
            sec = a.elapsed_time(b) / 1e3
            best = work / sec if best is None else max(best, work / sec)
        return best

    sink = torch.empty(4 * 4096, dtype=torch.float32, device="cuda")
    # matrix-core loops twice: pseudo-random operands that differ from one
    # instruction to the next (as the attention kernels' operands do on
    # N(0,1) data), then one fixed operand pattern; the chip lowers its clock
    # under the power limit on the first kind
    seed = 0x5EED
    mfma = {blocks: timed(lambda: ta.calib_mfma(blocks, 4000, sink, seed=seed)) / 1e12 for blocks in (1024, 2048, 4096)}
    mfma_fixed = {blocks: timed(lambda: ta.calib_mfma(blocks, 4000, sink)) / 1e12 for blocks in (1024, 2048, 4096)}
    src = torch.ones(1 << 32, dtype=torch.uint8, device="cuda")  # 4 GiB
    rsink = torch.empty(32768, dtype=torch.int32, device="cuda")
    read = {blocks: timed(lambda: ta.calib_read(src, blocks, rsink)) / 1e9 for blocks in (2048, 4096, 8192, 16384, 32768)}
    del src
    # the attention tile loop's own instruction mix (a model of the forward's
    # 64-key tile: 32 MFMAs and the softmax per wave and iteration): with
    # register operands, LDS operands, and LDS operands plus the per-tile
    # copy; random Q / K / V (N(0,1) bf16 copy source), then fixed patterns
    gen = torch.Generator(device="cuda").manual_seed(seed)
    tsrc = torch.randn(8 << 20, dtype=torch.bfloat16, device="cuda", generator=gen)  # 16 MiB
    tsrc_fixed = torch.ones(16 << 20, dtype=torch.uint8, device="cuda")
    names = ("registers", "lds_operands", "lds_operands_and_copy")
    tile = {names[v]: max(timed(lambda: ta.calib_tile(v, blocks, 2000, sink, tsrc, seed=seed)) / 1e12
                          for blocks in (512, 1024)) for v in (0, 1, 2)}
    tile_fixed = {names[v]: max(timed(lambda: ta.calib_tile(v, blocks, 2000, sink, tsrc_fixed)) / 1e12
                                for blocks in (512, 1024)) for v in (0, 1, 2)}
    del tsrc, tsrc_fixed
    return {"mfma_bf16_tflops": max(mfma.values()), "hbm_read_gbs": max(read.values()),
            "tile_loop_tflops": tile,
            "fixed_operands": {"mfma_bf16_tflops": max(mfma_fixed.values()), "tile_loop_tflops": tile_fixed},
            "tile_loop": "tree_attn_calib_tile: the forward's 64-key tile loop at bf16 / head_dim 128 (16 S "
                         "MFMAs, the softmax of 32 scores and its 2^16 test, 16 PV MFMAs, a barrier per "
                         "iteration), 2,000 iterations, best of 512/1024 workgroups of 4 waves; operands from "
                         "registers / from an LDS tile in the kernel's layout / the same plus the kernel's "
                         "copy of the next tile per iteration (16 MiB source, L2-resident per KV head); "
                         "pseudo-random Q, K, V (N(0,1) bf16 source); 'fixed_operands': the same loops on fixed "
                         "operand patterns",
            "mfma_loop": "tree_attn_calib_mfma: waves issuing back-to-back bf16 32x32x16 MFMAs on 8 accumulators, "
                         "4,000 rounds; best of 1024/2048/4096 workgroups of 4 waves; pseudo-random operands, a "
                         "different pair per accumulator: "
                         + ", ".join(f"{k}: {v:.0f}" for k, v in mfma.items()) + " TFLOP/s; one fixed operand "
                         "pair ('fixed_operands'): " + ", ".join(f"{k}: {v:.0f}" for k, v in mfma_fixed.items())
                         + " TFLOP/s",
            "read_loop": "tree_attn_calib_read: 4 GiB streamed with 16-byte non-temporal loads; best of "
                         "2048-32768 workgroups of 256 threads: "
                         + ", ".join(f"{k}: {v:.0f}" for k, v in read.items()) + " GB/s"}


ENTRIES = {
    "prefill": prefill_case, "decode": decode_case, "verify": verify_case, "prefill_1page": prefill_1page_case,
    "verify_unshared": verify_unshared_case, "backward": backward_case, "accept": accept_case,
    "decode_multi": decode_multi_case, "decode_paged": decode_paged_case,
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for each CPU baseline (prefill, decode, verify)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calib", action="store_true", help="skip the attainable-peak loops")
    ap.add_argument("--only", choices=sorted(ENTRIES), default=None,
                    help="time one entry point only (profiling runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before timing, run a plain device copy of this many MiB three times "
                         "(reference for scaling HBM byte counters)")
    ap.add_argument("--zero-inputs", action="store_true",
                    help="diagnostic: run the prefill entry chosen by --only on all-zero q, k, v (the same "
                         "instructions with no bit activity in the data; compare with the default run)")
    args = ap.parse_args()
    if args.zero_inputs:
        if args.only not in ("prefill", "prefill_1page"):
            print("--zero-inputs needs --only prefill or --only prefill_1page", file=sys.stderr)
            sys.exit(2)
        global ZERO_INPUTS
        ZERO_INPUTS = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the tree attention path has no multi-GPU mode "
              "(pages shard across GPUs with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.calib_copy_mib > 0:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")
        del src, dst
    attainable = None
    if not args.no_calib and args.only is None:
        attainable = calibrate()
        log(f"[bench] attainable: {attainable['mfma_bf16_tflops']:.0f} TFLOP/s bf16 "
            f"({attainable['fixed_operands']['mfma_bf16_tflops']:.0f} on fixed operands), "
            f"{attainable['hbm_read_gbs']:.0f} GB/s read; tile-loop model "
            + " / ".join(f"{v:.0f}" for v in attainable["tile_loop_tflops"].values())
            + " (fixed operands: "
            + " / ".join(f"{v:.0f}" for v in attainable["fixed_operands"]["tile_loop_tflops"].values()) + ")"
            + " TFLOP/s (registers / LDS operands / LDS operands + copy)")
    log("[bench] generating inputs")
    cases = []
    for name, fn in ENTRIES.items():
        if args.only is None or args.only == name:
            cases.append(fn())
            log(f"[bench] {name}: {cases[-1]['w'].name} ready")
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for c in cases:
            c["run"]()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(cases) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        for i, c in enumerate(cases):
            c["run"]()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"[bench] timed {args.steps} steps in {wall * 1e3:.1f} ms")

    per_case = {}
    for i, c in enumerate(cases):
        ms = [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]
        avg = float(np.mean(ms))
        sec = avg / 1e3
        tflops = c["flops"] / sec / 1e12
        gbs = c["bytes"] / sec / 1e9
        r = {"workload": c["w"].name, "kernel": c["kernel"], "ms_avg": avg, "ms_min": float(np.min(ms)),
             "ms_median": float(np.median(ms)), f"{c['unit'].replace(' ', '_')}_per_s": c["unit_count"] / sec,
             "flops_per_launch": c["flops"], "bytes_per_launch": c["bytes"], "tflops": tflops, "gbs": gbs,
             "flop_frac": tflops / PEAK_BF16_TFLOPS, "byte_frac": gbs / PEAK_HBM_GBS,
             "plan_build_us": c["plan_us"]}
        if attainable:
            r["flop_frac_attainable"] = tflops / attainable["mfma_bf16_tflops"]
            r["byte_frac_attainable"] = gbs / attainable["hbm_read_gbs"]
            if c["name"] in ("prefill", "verify", "prefill_1page"):
                # against the model of the forward's own tile loop with its copies
                r["flop_frac_tile_model"] = tflops / attainable["tile_loop_tflops"]["lds_operands_and_copy"]
        if c["bound"] == "mfma":
            r["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic_for(c["name"])}
        else:
            r["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": gbs / PEAK_HBM_GBS, "traffic": traffic_for(c["name"])}
        per_case[c["name"]] = r
        log(f"[bench] {c['name']}: {avg * 1e3:.1f} us  flop_frac={r['flop_frac']:.3f} byte_frac={r['byte_frac']:.3f}")

    step_names = [c["name"] for c in cases if c.get("in_step", True)] or [c["name"] for c in cases]
    step_ms = sum(per_case[n]["ms_avg"] for n in step_names)
    dominant = max(step_names, key=lambda k: per_case[k]["ms_avg"])
    head = per_case.get("prefill") or per_case[dominant]
    value = head.get("packed_tokens_per_s") or next(v for k, v in head.items() if k.endswith("_per_s"))
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "packed tokens/s" if "prefill" in per_case else "units/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "zeros (diagnostic)" if ZERO_INPUTS else "synthetic",
        "config": {"workload": "packed tree-varlen prefill, batch of 8 pages (seed 2): P=4096, N~U{12..40} regions, "
                               "L=12, lognormal content clipped to [8,1024], cap 16,384 per page, 77,400 packed "
                               "tokens; 16q/8kv heads, d=128, bf16. Step also runs decode (16 pages x 24 branches, "
                               "P=4809) and verify (64 pages x 8 trees x 32 nodes)",
                   "prefill_tokens": per_case.get("prefill", {}).get("workload"),
                   "step_entries": step_names,
                   "parallelism": "single GPU"},
        "roofline": dict(per_case[dominant]["roofline"], kernel=per_case[dominant]["kernel"], entry=dominant),
        "attainable": attainable,
        "entries": per_case,
        "wall_ms_timed_region": wall * 1e3,
    }
    for name, key in (("prefill", "prefill_mfma_frac"), ("prefill_1page", "prefill_1page_mfma_frac"),
                      ("verify", "verify_mfma_frac"), ("verify_unshared", "verify_unshared_hbm_frac"),
                      ("decode", "decode_hbm_frac"), ("backward", "backward_mfma_frac"),
                      ("accept", "accept_hbm_frac"), ("decode_multi", "decode_multi_hbm_frac"),
                      ("decode_paged", "decode_paged_hbm_frac")):
        if name in per_case:
            out[key] = per_case[name]["roofline"]["frac"]
    if "decode" in per_case:
        out["decode_query_tokens_per_s"] = per_case["decode"]["query_tokens_per_s"]
    if not args.no_cpu_baseline and args.only is None:
        log("[bench] timing the CPU oracle baselines")
        cpu = host_cpu()
        byname = {c["name"]: c for c in cases}
        per_case["prefill"]["cpu_baseline"] = cpu_prefill(byname["prefill"]["w"], args.cpu_budget, cpu)
        per_case["decode"]["cpu_baseline"] = cpu_decode(byname["decode"]["w"], args.cpu_budget / 2, cpu)
        per_case["verify"]["cpu_baseline"] = cpu_verify(byname["verify"]["w"], args.cpu_budget, cpu)
        out["cpu_baseline"] = per_case["prefill"]["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
