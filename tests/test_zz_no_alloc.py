"""tree_attn_decode_noalloc (partials in the library's file-scope device
scratch) against tree_attn_decode (caller scratch) through the C ABI: the
same kernels on the same inputs, so outputs must be bit-identical (and so
within the bf16 tolerance), on consecutive calls of decreasing size that
reuse the array with the previous call's contents still in it."""

import numpy as np
import pytest
import torch

from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth

pytestmark = pytest.mark.gpu


def run_both(w, plan):
    t = {k: v.cuda() for k, v in w.tensors.items()}
    o_ref, l_ref = ta.decode(plan, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], scale=w.scale)
    o = torch.full_like(t["q"], float("nan"))
    lse = torch.full((w.hq, t["q"].shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    ta.decode_noalloc(plan, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], o, lse, scale=w.scale)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), lse.cpu().numpy()), (o_ref.float().cpu().numpy(), l_ref.cpu().numpy())


def small_multi():
    rng = np.random.default_rng(12)
    desc = synth.DecodeDesc(np.array([300, 70], np.int32), np.array([3, 1], np.int32),
                            np.array([12, 12, 12, 5], np.int32), np.array([0, 0, 0, 1], np.int32),
                            np.array([1, 0, 3, 1], np.int32), np.array([5, 2, 140, 0], np.int32),
                            np.array([1, 3, 8, 2], np.int32))
    w = synth.Workload("small_multi", "decode", desc, 16, 8, 128, torch.bfloat16, seed=12)
    w.tensors = synth.decode_tensors(rng, desc, 16, 8, 128, torch.bfloat16)
    return w


def test_decode_noalloc_equals_decode_on_calls_of_decreasing_size():
    # 50.8 MiB of partials, then 6.1 MiB, then a few KB: each later call
    # finds the earlier call's partials in the shared array
    for w in (synth.decode_multi(), synth.config4(), small_multi()):
        plan = ta.plan_for(w.desc).upload()
        need = ta.scratch_bytes(plan, w.hq, w.head_dim)
        assert 0 < need <= ta.TA_STATIC_SCRATCH_BYTES
        (o, l), (o_ref, l_ref) = run_both(w, plan)
        print(f"[noalloc] {w.name}: rows={w.desc.n_rows()} scratch={need / 2**20:.2f} MiB", flush=True)
        assert np.array_equal(o.view(np.uint32), o_ref.view(np.uint32)), w.name
        assert np.array_equal(l.view(np.uint32), l_ref.view(np.uint32)), w.name
        err = np.abs(o - o_ref)
        assert (err <= 2e-2 + 1e-2 * np.abs(o_ref)).all()


def test_decode_noalloc_rejects_plans_beyond_its_scratch():
    # 16 pages x 25 rows x 40 new tokens: more partials than 64 MiB hold
    w = synth.decode_multi(with_tensors=False, window=40)
    plan = ta.plan_for(w.desc).upload()
    need = ta.scratch_bytes(plan, w.hq, w.head_dim)
    assert need > ta.TA_STATIC_SCRATCH_BYTES
    rows = w.desc.n_rows()
    q = torch.zeros(rows, w.hq, w.head_dim, dtype=torch.bfloat16, device="cuda")
    km = torch.zeros(int(w.desc.main_tokens().sum()), w.hkv, w.head_dim, dtype=torch.bfloat16, device="cuda")
    ks = torch.zeros(w.desc.suffix_tokens(), w.hkv, w.head_dim, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    with pytest.raises(ta.TreeAttnError) as e:
        ta.decode_noalloc(plan, q, km, km, ks, ks, o)
    assert e.value.code == ta.TA_ERR_CAPACITY and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not o.any()  # nothing was enqueued
