"""GPU edge cases through the C ABI: empty plans (no rows, no keys) launch
nothing and leave the outputs untouched; the widest GQA group (32 query heads
per KV head); draft trees of 0 and 1 nodes beside full ones; a decode row that
sees no main-stream key.  Compared with the fp64 oracle at the bf16 tolerance
of the parity tests."""
import numpy as np
import pytest
import torch

import oracle
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth
from test_gpu_parity import (TOL, LSE_TOL, close, decode_workload, gpu_decode, gpu_verify, prefill_workload,
                             check_prefill_full, verify_workload, check_decode)

pytestmark = pytest.mark.gpu


def test_empty_plans_launch_nothing():
    dev = "cuda"
    bf = torch.bfloat16
    sentinel = torch.full((4, 2, 64), 7.0, dtype=bf, device=dev)
    empty = torch.empty((0, 2, 64), dtype=bf, device=dev)
    # prefill: no pages, and a page with no tokens
    for desc in (synth.make_prefill_desc([], [], []), synth.make_prefill_desc([0], [np.array([])], [np.array([])])):
        plan = ta.plan_for(desc).upload()
        o, lse = ta.prefill(plan, empty, empty[:, :1], empty[:, :1], scale=0.1)
        assert o.shape[0] == 0 and lse.shape[1] == 0
    # decode with no live branch
    d = synth.DecodeDesc(np.array([100], np.int32), np.array([1], np.int32), np.array([5], np.int32),
                         np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32))
    plan = ta.plan_for(d).upload()
    kv = torch.randn((105, 1, 64), device=dev).to(bf)
    o, _ = ta.decode(plan, empty, kv, kv, kv[:0], kv[:0], scale=0.1)
    assert o.shape[0] == 0
    # verify with trees of no nodes
    v = synth.VerifyDesc(np.array([10], np.int32), np.zeros(2, np.int32), np.zeros(2, np.int32),
                         np.zeros(0, np.int32))
    plan = ta.plan_for(v).upload()
    kc = torch.randn((10, 1, 64), device=dev).to(bf)
    o, _ = ta.verify(plan, empty, kc, kc, kc[:0], kc[:0], scale=0.1)
    assert o.shape[0] == 0
    # backward of an empty prefill
    plan = ta.plan_for(synth.make_prefill_desc([], [], [])).upload()
    lse = torch.empty((2, 0), device=dev)
    dq, dk, dv = ta.prefill_backward(plan, empty, empty[:, :1], empty[:, :1], empty, lse, empty, scale=0.1)
    assert dq.shape[0] == 0
    torch.cuda.synchronize()
    assert (sentinel == 7.0).all()


def test_widest_gqa_group_prefill():
    w = prefill_workload(None, None, None, hq=32, hkv=1, d=64,
                         pages=[(90, [3, 5], [70, 9]), (10, [1], [1])], seed=31)
    check_prefill_full(w, "group 32")


def test_widest_gqa_group_decode():
    w = decode_workload([300, 20], [2, 1], [4, 6, 3], [(0, 1, 5, 3), (0, 0, 2, 4), (1, 1, 0, 1)],
                        hq=32, hkv=1, d=64, seed=32)
    check_decode(w, tag="group 32")


def test_verify_empty_and_single_node_trees_beside_full_ones():
    rng = np.random.default_rng(33)
    trees = [(0, []), (0, [-1]), (0, list(synth.random_tree_parents(rng, 64))), (1, []), (1, [-1, -1, 0]),
             (1, [-1])]
    for hq, hkv, d in ((16, 8, 128), (32, 1, 64)):
        w = verify_workload([70, 200], trees, hq=hq, hkv=hkv, d=d, seed=hq)
        o, lse = gpu_verify(w)
        t = w.tensors
        ro, rl = oracle.verify(w.desc, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], w.scale)
        close(o, ro, TOL[w.dtype], f"verify edge trees heads={hq}/{hkv} o")
        close(lse, rl, LSE_TOL[w.dtype], f"verify edge trees heads={hq}/{hkv} lse")


def test_calibration_loops_do_their_work():
    """The roofline calibration loops: the streaming read folds every 4-byte
    word of the buffer exactly once (the XOR over the workgroups' words
    equals the buffer's XOR, for sizes with and without a ragged tail), and
    the MFMA loop reports 32,768 FLOP per instruction."""
    rng = np.random.default_rng(3)
    for n_words in (1 << 20, (1 << 20) + 4 * 37):
        words = rng.integers(-2**31, 2**31, n_words, dtype=np.int64).astype(np.int32)
        src = torch.from_numpy(words).cuda()
        sink = torch.zeros(300, dtype=torch.int32, device="cuda")
        assert ta.calib_read(src, 300, sink) == 4 * n_words
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(words.view(np.uint32)), n_words
    for seed in (0, 7):  # fixed operands, then pseudo-random ones
        fsink = torch.zeros(4 * 8, dtype=torch.float32, device="cuda")
        assert ta.calib_mfma(8, 10, fsink, seed=seed) == 8 * 4 * 10 * 8 * 32768
        torch.cuda.synchronize()
        assert torch.isfinite(fsink).all() and (fsink != 0).all(), seed
    with pytest.raises(ta.TreeAttnError):
        ta.calib_read(src[:3], 4, sink)  # 12 bytes: not a multiple of 16
    # the tile-loop model, each variant: 32 MFMAs of 32,768 FLOP per wave and
    # iteration, every wave writes a finite word
    tile_src = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    for variant in (0, 1, 2):
        for seed in (0, 7):
            fsink = torch.full((4 * 8,), float("nan"), dtype=torch.float32, device="cuda")
            src = tile_src if variant == 2 else None
            assert ta.calib_tile(variant, 8, 5, fsink, src, seed=seed) == 8 * 4 * 5 * 32 * 32768
            torch.cuda.synchronize()
            assert torch.isfinite(fsink).all(), (variant, seed)
