"""HIP graph capture of the compute entry points.

Every compute entry point only launches kernels on the caller's stream (no
allocation, copy, memset or synchronisation inside), so a serving loop can
capture a step once and replay it.  Each case captures one call into a
torch.cuda.CUDAGraph with preallocated outputs and scratch, replays it three
times with eager work and synchronisations between the replays (the outputs
are overwritten with NaN before each), and requires every replay to equal
the eager call bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def replay_matches(call, outs, tag):
    """call() launches into the preallocated `outs`; compare eager vs graph."""
    call()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as torch asks before capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, want)):
            assert torch.equal(a, b), f"{tag}: output {i} differs on replay {rep}"
        del junk
    say(f"[graph] {tag}: 3 replays equal the eager call")


def scratch_for(plan, hq, d):
    return torch.empty(ta.scratch_bytes(plan, hq, d) + 256, dtype=torch.uint8, device=DEV)


def test_graph_prefill_balanced():
    w = synth.config2()
    plan = ta.plan_for(w.desc).balance(w.hkv).upload(DEV)  # split tiles: attention + merge launches
    t = {k: v.to(DEV) for k, v in w.tensors.items()}
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.hq, t["q"].shape[0]), dtype=torch.float32, device=DEV)
    s = scratch_for(plan, w.hq, w.head_dim)
    replay_matches(lambda: ta.prefill(plan, t["q"], t["k"], t["v"], scale=w.scale, out=o, lse=lse, scratch=s),
                   [o, lse], "prefill (balanced, 1 page)")


def test_graph_decode_and_multi():
    for w in (synth.config4(), synth.decode_multi()):
        plan = ta.plan_for(w.desc).upload(DEV)
        t = {k: v.to(DEV) for k, v in w.tensors.items()}
        o = torch.empty_like(t["q"])
        lse = torch.empty((w.hq, t["q"].shape[0]), dtype=torch.float32, device=DEV)
        s = scratch_for(plan, w.hq, w.head_dim)
        replay_matches(lambda: ta.decode(plan, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"],
                                         scale=w.scale, out=o, lse=lse, scratch=s),
                       [o, lse], f"decode {w.name}")


def test_graph_verify():
    w = synth.config5()
    plan = ta.plan_for(w.desc).balance(w.hkv).upload(DEV)
    t = {k: v.to(DEV) for k, v in w.tensors.items()}
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.hq, t["q"].shape[0]), dtype=torch.float32, device=DEV)
    s = scratch_for(plan, w.hq, w.head_dim)
    replay_matches(lambda: ta.verify(plan, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"],
                                     scale=w.scale, out=o, lse=lse, scratch=s),
                   [o, lse], "verify 64 pages x 8 trees")


def test_graph_backward():
    w = synth.config2()
    plan = ta.plan_for(w.desc).upload(DEV)
    t = {k: v.to(DEV) for k, v in w.tensors.items()}
    rng = np.random.default_rng(3)
    g = torch.from_numpy(rng.standard_normal(tuple(t["q"].shape), dtype=np.float32)).to(torch.bfloat16).to(DEV)
    o, lse = ta.prefill(plan, t["q"], t["k"], t["v"], scale=w.scale)
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    s = torch.empty(ta.backward_scratch_bytes(plan, w.hq) + 256, dtype=torch.uint8, device=DEV)
    replay_matches(lambda: ta.prefill_backward(plan, t["q"], t["k"], t["v"], o, lse, g, scale=w.scale,
                                               dq=dq, dk=dk, dv=dv, scratch=s),
                   [dq, dk, dv], "prefill backward (1 page)")


def test_graph_accept():
    w = synth.config5(with_tensors=False)
    desc = w.desc
    vocab = 32000
    rng = np.random.default_rng(4)
    tokens = synth.draft_tokens(rng, desc, vocab)
    logits = synth.accept_logits(5, desc, tokens, vocab, vocab, torch.bfloat16, DEV)
    plan = ta.plan_for(desc).upload(DEV)
    tok = torch.as_tensor(tokens, device=DEV)
    path = torch.empty(desc.total_nodes(), dtype=torch.int32, device=DEV)
    n_path = torch.empty(desc.n_branches, dtype=torch.int32, device=DEV)
    nxt = torch.empty(desc.n_branches, dtype=torch.int32, device=DEV)
    s = torch.empty(ta.accept_scratch_bytes(plan, vocab) + 256, dtype=torch.uint8, device=DEV)

    def call():
        path.fill_(-1)  # entries past the accepted path are left as they were
        ta.accept(plan, logits, tok, vocab=vocab, path=path, n_path=n_path, next_token=nxt, scratch=s)

    replay_matches(call, [path, n_path, nxt], "greedy acceptance 512 trees")
