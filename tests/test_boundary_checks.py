"""CPU tests of the boundary's own checks: nothing here launches a kernel.

The binding validates every tensor argument before it takes a device
pointer (dtype agreement, head counts and head_dim, v shaped like k, outputs
shaped like q, lse fp32 [Hq, rows]); CPU tensors drive those checks, and a
call that passes them stops at the device check instead.  The C ABI maps a
host allocation failure inside any exported call to TA_ERR_CAPACITY instead
of letting the exception cross the ABI (tested in a subprocess whose address
space is capped).
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest
import torch

from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth

BF, F32 = torch.bfloat16, torch.float32


def prefill_setup(hq=4, hkv=2, d=64):
    desc = synth.make_prefill_desc([40], [np.array([3, 2])], [np.array([20, 9])])
    T = desc.total_tokens()
    plan = ta.plan_for(desc)
    q = torch.zeros(T, hq, d, dtype=BF)
    k = torch.zeros(T, hkv, d, dtype=BF)
    return plan, q, k, k.clone(), T


def expect_invalid(fn, *args, match=None, **kw):
    with pytest.raises(ta.TreeAttnError) as e:
        fn(*args, **kw)
    assert e.value.code == ta.TA_ERR_INVALID_ARG, str(e.value)
    if match:
        assert match in str(e.value), str(e.value)


def test_prefill_valid_cpu_args_reach_the_device_check():
    plan, q, k, v, _ = prefill_setup()
    expect_invalid(ta.prefill, plan, q, k, v, match="GPU")


@pytest.mark.parametrize("bad", ["k_dtype", "v_dtype", "v_shape", "head_dim", "out_shape", "out_dtype",
                                 "lse_dtype", "lse_shape", "q_rank", "k_noncontig", "scratch_dtype"])
def test_prefill_argument_mismatch_is_rejected_before_launch(bad):
    plan, q, k, v, T = prefill_setup()
    kw = {}
    if bad == "k_dtype":
        k = k.float()
    elif bad == "v_dtype":
        v = v.float()
    elif bad == "v_shape":
        v = torch.zeros(T, 1, 64, dtype=BF)
    elif bad == "head_dim":
        k = torch.zeros(T, 2, 32, dtype=BF)
        v = k.clone()
    elif bad == "out_shape":
        kw["out"] = torch.zeros(T - 1, 4, 64, dtype=BF)
    elif bad == "out_dtype":
        kw["out"] = torch.zeros(T, 4, 64, dtype=F32)
    elif bad == "lse_dtype":
        kw["lse"] = torch.zeros(4, T, dtype=BF)
    elif bad == "lse_shape":
        kw["lse"] = torch.zeros(T, 4, dtype=F32)
    elif bad == "q_rank":
        q = q.reshape(T, -1)
    elif bad == "k_noncontig":
        k = torch.zeros(2, 64, T, dtype=BF).permute(2, 0, 1)
        v = k.clone()
    elif bad == "scratch_dtype":
        kw["scratch"] = torch.zeros(1024, dtype=F32)
    expect_invalid(ta.prefill, plan, q, k, v, **kw)


def decode_setup():
    desc = synth.DecodeDesc(np.array([50], np.int32), np.array([2], np.int32), np.array([4, 4], np.int32),
                            np.zeros(2, np.int32), np.array([1, 2], np.int32), np.array([3, 5], np.int32))
    plan = ta.plan_for(desc)
    t = synth.decode_tensors(np.random.default_rng(0), desc, 4, 2, 64, BF)
    return plan, t


def test_decode_valid_cpu_args_reach_the_device_check():
    plan, t = decode_setup()
    expect_invalid(ta.decode, plan, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"], match="GPU")


@pytest.mark.parametrize("bad", ["suffix_heads", "suffix_dtype", "main_v_shape", "suffix_head_dim"])
def test_decode_argument_mismatch_is_rejected_before_launch(bad):
    plan, t = decode_setup()
    if bad == "suffix_heads":
        t["k_suffix"] = torch.zeros(t["k_suffix"].shape[0], 1, 64, dtype=BF)
        t["v_suffix"] = t["k_suffix"].clone()
    elif bad == "suffix_dtype":
        t["v_suffix"] = t["v_suffix"].float()
    elif bad == "main_v_shape":
        t["v_main"] = t["v_main"][:-1].contiguous()
    elif bad == "suffix_head_dim":
        t["k_suffix"] = torch.zeros(t["k_suffix"].shape[0], 2, 32, dtype=BF)
        t["v_suffix"] = t["k_suffix"].clone()
    expect_invalid(ta.decode, plan, t["q"], t["k_main"], t["v_main"], t["k_suffix"], t["v_suffix"])


def test_verify_argument_mismatch_is_rejected_before_launch():
    desc = synth.VerifyDesc(np.array([30], np.int32), np.array([0], np.int32), np.array([3], np.int32),
                            np.array([-1, 0, 0], np.int32))
    plan = ta.plan_for(desc)
    t = synth.verify_tensors(np.random.default_rng(0), desc, 4, 2, 64, BF)
    expect_invalid(ta.verify, plan, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"], match="GPU")
    expect_invalid(ta.verify, plan, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"], t["v_tree"].float())
    expect_invalid(ta.verify, plan, t["q"], t["k_ctx"], t["v_ctx"], t["k_tree"][:, :1].contiguous(),
                   t["v_tree"][:, :1].contiguous())


@pytest.mark.parametrize("bad", ["dk_shape", "dv_dtype", "o_shape", "d_o_dtype", "lse_dtype", "dq_shape",
                                 "lse_missing"])
def test_backward_argument_mismatch_is_rejected_before_launch(bad):
    plan, q, k, v, T = prefill_setup()
    args = dict(o=q.clone(), lse=torch.zeros(4, T, dtype=F32), d_o=q.clone())
    kw = {}
    if bad == "dk_shape":
        kw["dk"] = torch.zeros(T, 4, 64, dtype=BF)
    elif bad == "dv_dtype":
        kw["dv"] = v.float()
    elif bad == "o_shape":
        args["o"] = q[:-1].clone()
    elif bad == "d_o_dtype":
        args["d_o"] = q.float()
    elif bad == "lse_dtype":
        args["lse"] = torch.zeros(4, T, dtype=BF)
    elif bad == "dq_shape":
        kw["dq"] = torch.zeros(T, 2, 64, dtype=BF)
    elif bad == "lse_missing":
        args["lse"] = None
    expect_invalid(ta.prefill_backward, plan, q, k, v, args["o"], args["lse"], args["d_o"], **kw)


def test_backward_valid_cpu_args_reach_the_device_check():
    plan, q, k, v, T = prefill_setup()
    expect_invalid(ta.prefill_backward, plan, q, k, v, q.clone(), torch.zeros(4, T, dtype=F32), q.clone(),
                   match="GPU")


# ---------------------------------------------------------------------------
# host allocation failure inside an exported call
# ---------------------------------------------------------------------------

OOM_SCRIPT = textwrap.dedent("""
    import ctypes, resource, sys
    L = ctypes.CDLL(sys.argv[1])
    L.tree_attn_last_error.restype = ctypes.c_char_p
    vm = 0
    for line in open("/proc/self/status"):
        if line.startswith("VmSize:"):
            vm = int(line.split()[1]) * 1024
    cap = vm + (1 << 30)
    resource.setrlimit(resource.RLIMIT_AS, (cap, cap))
    I32 = ctypes.c_int32
    out = ctypes.c_void_p()
    # one page of 2^30 - 1 prefix tokens: valid, but its per-token host
    # tables need tens of GB
    P = (I32 * 1)((1 << 30) - 1)
    N = (I32 * 1)(0)
    rc = L.tree_attn_plan_prefill(P, N, None, None, I32(1), ctypes.byref(out))
    print("prefill", rc, L.tree_attn_last_error().decode(), flush=True)
    assert rc == -3 and not out.value, rc
    # a pool of 2^30 - 1 one-token blocks: 4 GB of reference counts
    rc = L.tree_attn_pool_create(I32((1 << 30) - 1), I32(1), ctypes.byref(out))
    print("pool", rc, L.tree_attn_last_error().decode(), flush=True)
    assert rc == -3 and not out.value, rc
    # the library still works afterwards
    P = (I32 * 1)(10)
    rc = L.tree_attn_plan_prefill(P, N, None, None, I32(1), ctypes.byref(out))
    assert rc == 0 and out.value
    L.tree_attn_plan_destroy(out)
    print("ok", flush=True)
""")


def test_host_allocation_failure_returns_capacity_status():
    if not os.path.exists(ta.LIB_PATH):
        pytest.skip("library not built")
    r = subprocess.run([sys.executable, "-c", OOM_SCRIPT, ta.LIB_PATH], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "out of host memory" in r.stdout and r.stdout.strip().endswith("ok"), r.stdout


def test_decode_noalloc_host_checks():
    """tree_attn_decode_noalloc checks on the host, before any device work: a
    plan whose partials exceed TA_STATIC_SCRATCH_BYTES gets CAPACITY, a
    plan that fits but is not uploaded gets STATE (fake, never dereferenced
    16-byte aligned pointers stand in for the tensors)."""
    import ctypes
    L = ta.lib()
    fake = ctypes.c_void_p(1 << 20)
    big = ta.plan_for(synth.decode_multi(with_tensors=False, window=40).desc)
    assert ta.scratch_bytes(big, 16, 128) > ta.TA_STATIC_SCRATCH_BYTES
    rc = L.tree_attn_decode_noalloc(big.handle, ta.TA_DTYPE_BF16, 16, 8, 128, 0.088, fake, fake, fake, fake, fake,
                                    fake, None, None)
    assert rc == ta.TA_ERR_CAPACITY and "static scratch" in ta.last_error()
    small = ta.plan_for(synth.config4(with_tensors=False, n_pages=2).desc)
    rc = L.tree_attn_decode_noalloc(small.handle, ta.TA_DTYPE_BF16, 16, 8, 128, 0.088, fake, fake, fake, fake,
                                    fake, fake, None, None)
    assert rc == ta.TA_ERR_STATE


def test_calib_tile_host_checks():
    """tree_attn_calib_tile rejects a bad variant, a missing or short copy
    source (variant 2) and out-of-range sizes on the host, before any launch
    (a fake, never dereferenced pointer stands in for the sink)."""
    import ctypes
    L = ta.lib()
    fake = ctypes.c_void_p(1 << 20)
    flops = ctypes.c_int64()
    for args in ((3, 8, 5, 0, None, 0), (-1, 8, 5, 7, None, 0), (2, 8, 5, 0, None, 0), (2, 8, 5, 7, fake, 4096),
                 (0, 0, 5, 0, None, 0), (0, 8, 0, 7, None, 0)):
        rc = L.tree_attn_calib_tile(*args, fake, ctypes.byref(flops), None)
        assert rc == ta.TA_ERR_INVALID_ARG, (args, rc)
        assert "calib_tile" in ta.last_error()
    for args in ((0, 5, 0), (8, 0, 7), (1 << 21, 5, 0)):
        rc = L.tree_attn_calib_mfma(*args, fake, ctypes.byref(flops), None)
        assert rc == ta.TA_ERR_INVALID_ARG, (args, rc)
        assert "calib_mfma" in ta.last_error()
