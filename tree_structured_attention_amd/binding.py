"""Thin ctypes binding over libtree_attn's C ABI (argument marshalling only).

Every step of the attention path runs in the HIP library; this module only
turns torch tensors into pointers and streams, allocates the caller-owned
device workspace/scratch with torch, and raises on a non-zero status.  It
fails loudly if the library has not been built: there is no fallback.

Names mirror the C entry points without the ``tree_attn_`` prefix:
``plan_prefill``, ``plan_decode``, ``plan_verify``, ``plan_balance``,
``plan_info``, ``plan_export``, ``plan_upload``, ``plan_destroy``,
``scratch_bytes``, ``prefill``, ``decode``, ``verify``.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import re
from typing import Optional

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtree_attn.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tree_attn.h")

TA_OK = 0
TA_ERR_INVALID_ARG = -1
TA_ERR_UNSUPPORTED = -2
TA_ERR_CAPACITY = -3
TA_ERR_WORKSPACE = -4
TA_ERR_HIP = -5
TA_ERR_STATE = -6

TA_DTYPE_F32 = 0
TA_DTYPE_BF16 = 1

TA_PLAN_PREFILL = 1
TA_PLAN_DECODE = 2
TA_PLAN_VERIFY = 3

FIELD = {
    "position": 1,
    "main_end": 2,
    "branch_start": 3,
    "pages": 4,
    "branches": 5,
    "decode_rows": 6,
    "verify_mask": 7,
    "verify_rows": 8,
    "work": 9,
    "bwd_work": 10,
    "paged_tiles": 11,
    "device_layout": 12,
    "device_image": 13,
}
FIELD_WIDTH = {"pages": 5, "branches": 3, "decode_rows": 5, "verify_rows": 4, "work": 11, "bwd_work": 12}


class TreeAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"tree_attn error {code}: {msg}")
        self.code = code


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("n_pages", ctypes.c_int32),
        ("n_branches", ctypes.c_int32),
        ("n_work", ctypes.c_int32),
        ("n_rows", ctypes.c_int64),
        ("n_keys_a", ctypes.c_int64),
        ("n_keys_b", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("n_partials", ctypes.c_int64),
        ("visible_pairs", ctypes.c_int64),
        ("max_depth", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)


def lib() -> ctypes.CDLL:
    """Load libtree_attn.so (built by tree_structured_attention_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m tree_structured_attention_amd.build` "
                "(the tree attention path has no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        pp = ctypes.POINTER(ctypes.c_void_p)
        sig = {
            "tree_attn_plan_prefill": ([_I32P, _I32P, _I32P, _I32P, i32, pp], ctypes.c_int),
            "tree_attn_plan_decode": ([_I32P, _I32P, _I32P, i32, _I32P, _I32P, _I32P, i32, pp], ctypes.c_int),
            "tree_attn_plan_decode_multi": ([_I32P, _I32P, _I32P, i32, _I32P, _I32P, _I32P, _I32P, i32, pp],
                                            ctypes.c_int),
            "tree_attn_plan_verify": ([_I32P, i32, _I32P, _I32P, _I32P, i32, pp], ctypes.c_int),
            "tree_attn_plan_decode_paged": ([_I32P, _I32P, _I32P, i32, _I32P, _I32P, _I32P, _I32P, i32, i32, i32,
                                             _I32P, _I64P, _I32P, _I64P, pp], ctypes.c_int),
            "tree_attn_plan_verify_paged": ([_I32P, i32, _I32P, _I32P, _I32P, i32, i32, i32, _I32P, _I64P, pp],
                                            ctypes.c_int),
            "tree_attn_pool_create": ([i32, i32, pp], ctypes.c_int),
            "tree_attn_pool_destroy": ([_P], None),
            "tree_attn_pool_new_seq": ([_P, _I32P], ctypes.c_int),
            "tree_attn_pool_fork": ([_P, i32, i32, _I32P], ctypes.c_int),
            "tree_attn_pool_append": ([_P, i32, i32, _I64P], ctypes.c_int),
            "tree_attn_pool_release": ([_P, i32], ctypes.c_int),
            "tree_attn_pool_table": ([_P, i32, _I32P, i32, _I32P, _I32P, i32, _I32P], ctypes.c_int),
            "tree_attn_pool_refs": ([_P, _I32P, i32, _I32P], ctypes.c_int),
            "tree_attn_plan_info": ([_P, ctypes.POINTER(PlanInfo)], ctypes.c_int),
            "tree_attn_plan_export": ([_P, i32, ctypes.POINTER(i64), i64, ctypes.POINTER(i64)], ctypes.c_int),
            "tree_attn_plan_upload": ([_P, _P, sz, _P], ctypes.c_int),
            "tree_attn_plan_destroy": ([_P], None),
            "tree_attn_plan_balance": ([_P, i32, i32], ctypes.c_int),
            "tree_attn_scratch_bytes": ([_P, i32, i32, ctypes.POINTER(sz)], ctypes.c_int),
            "tree_attn_prefill": ([_P, i32, i32, i32, i32, f32, _P, _P, _P, _P, _P, _P, sz, _P], ctypes.c_int),
            "tree_attn_decode": ([_P, i32, i32, i32, i32, f32, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P],
                                 ctypes.c_int),
            "tree_attn_verify": ([_P, i32, i32, i32, i32, f32, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P],
                                 ctypes.c_int),
            "tree_attn_backward_scratch_bytes": ([_P, i32, ctypes.POINTER(sz)], ctypes.c_int),
            "tree_attn_prefill_backward": ([_P, i32, i32, i32, i32, f32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz,
                                            _P], ctypes.c_int),
            "tree_attn_draft_tree": ([_I32P, i32, _I32P, _I32P, i32, i32, i32, i32, _I32P, _I32P, _I32P],
                                     ctypes.c_int),
            "tree_attn_accept_scratch_bytes": ([_P, i64, ctypes.POINTER(sz)], ctypes.c_int),
            "tree_attn_accept": ([_P, i32, _P, i64, i64, _P, ctypes.c_double, i32, _P, _P, _P, _P, sz, _P],
                                 ctypes.c_int),
            "tree_attn_decode_noalloc": ([_P, i32, i32, i32, i32, f32, _P, _P, _P, _P, _P, _P, _P, _P],
                                         ctypes.c_int),
            "tree_attn_calib_mfma": ([i32, i32, ctypes.c_uint32, _P, _I64P, _P], ctypes.c_int),
            "tree_attn_calib_read": ([_P, i64, i32, _P, _P], ctypes.c_int),
            "tree_attn_calib_tile": ([i32, i32, i32, ctypes.c_uint32, _P, i64, _P, _I64P, _P], ctypes.c_int),
            "tree_attn_last_error": ([], ctypes.c_char_p),
            "tree_attn_version": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Entry points declared in include/tree_attn.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(tree_attn_\w+)\s*\(", text)))


def last_error() -> str:
    return lib().tree_attn_last_error().decode()


def _check(rc: int):
    if rc != TA_OK:
        raise TreeAttnError(rc, last_error())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_I32P) if a.size else None


# ---------------------------------------------------------------------------
# plans
# ---------------------------------------------------------------------------

class Plan:
    """Owns a host plan (and, once uploaded, its device workspace tensor)."""

    def __init__(self, handle: int, kind: int):
        self.handle = ctypes.c_void_p(handle)
        self.kind = kind
        self.workspace: Optional[torch.Tensor] = None
        self._keep = []

    @property
    def info(self) -> dict:
        return plan_info(self)

    def export(self, field: str) -> np.ndarray:
        return plan_export(self, field)

    def upload(self, device=None, stream=None) -> "Plan":
        return plan_upload(self, device, stream)

    def balance(self, n_kv_heads: int, n_slots: int = None) -> "Plan":
        return plan_balance(self, n_kv_heads, n_slots)

    def close(self):
        if self.handle is not None and self.handle.value:
            lib().tree_attn_plan_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass


def plan_prefill(prefix_len, n_regions, layout_len, content_len) -> Plan:
    P, N, L, C = _i32(prefix_len), _i32(n_regions), _i32(layout_len), _i32(content_len)
    out = ctypes.c_void_p()
    _check(lib().tree_attn_plan_prefill(_ptr(P), _ptr(N), _ptr(L), _ptr(C), int(P.size), ctypes.byref(out)))
    return Plan(out.value, TA_PLAN_PREFILL)


def plan_decode(prefix_len, n_regions, layout_len, br_page, br_region, suffix_len, n_query=None) -> Plan:
    """Decode plan; n_query (new tokens per branch) selects the multi-token
    form.  br_region 0 is a page's layout stream."""
    P, N, L = _i32(prefix_len), _i32(n_regions), _i32(layout_len)
    bp, br, s = _i32(br_page), _i32(br_region), _i32(suffix_len)
    out = ctypes.c_void_p()
    if n_query is None:
        _check(lib().tree_attn_plan_decode(_ptr(P), _ptr(N), _ptr(L), int(P.size), _ptr(bp), _ptr(br), _ptr(s),
                                           int(bp.size), ctypes.byref(out)))
    else:
        kq = _i32(n_query)
        if kq.size != bp.size:
            raise TreeAttnError(TA_ERR_INVALID_ARG, "n_query needs one entry per branch")
        _check(lib().tree_attn_plan_decode_multi(_ptr(P), _ptr(N), _ptr(L), int(P.size), _ptr(bp), _ptr(br),
                                                 _ptr(s), _ptr(kq), int(bp.size), ctypes.byref(out)))
    return Plan(out.value, TA_PLAN_DECODE)


def plan_verify(ctx_len, br_page, n_nodes, parent) -> Plan:
    c, bp, nn, pa = _i32(ctx_len), _i32(br_page), _i32(n_nodes), _i32(parent)
    out = ctypes.c_void_p()
    _check(lib().tree_attn_plan_verify(_ptr(c), int(c.size), _ptr(bp), _ptr(nn), _ptr(pa), int(bp.size),
                                       ctypes.byref(out)))
    return Plan(out.value, TA_PLAN_VERIFY)


def plan_for(desc) -> Plan:
    """Plan from a synth description object (PrefillDesc / DecodeDesc / VerifyDesc)."""
    name = type(desc).__name__
    if name == "PrefillDesc":
        return plan_prefill(desc.prefix_len, desc.n_regions, desc.layout_len, desc.content_len)
    if name == "DecodeDesc":
        return plan_decode(desc.prefix_len, desc.n_regions, desc.layout_len, desc.br_page, desc.br_region,
                           desc.suffix_len, getattr(desc, "n_query", None))
    if name == "VerifyDesc":
        return plan_verify(desc.ctx_len, desc.br_page, desc.n_nodes, desc.parent)
    raise TypeError(f"no plan for {name}")


def default_slots() -> int:
    """Concurrent workgroups of the attention kernel on the current GPU
    (2 per compute unit; 512 on MI355X)."""
    try:
        return 2 * torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    except Exception:
        return 512


def plan_balance(plan: Plan, n_kv_heads: int, n_slots: int = None) -> Plan:
    _check(lib().tree_attn_plan_balance(plan.handle, int(n_kv_heads), int(n_slots or default_slots())))
    return plan


def plan_info(plan: Plan) -> dict:
    info = PlanInfo()
    _check(lib().tree_attn_plan_info(plan.handle, ctypes.byref(info)))
    return info.as_dict()


def plan_export(plan: Plan, field: str) -> np.ndarray:
    n = ctypes.c_int64()
    rc = lib().tree_attn_plan_export(plan.handle, FIELD[field], None, 0, ctypes.byref(n))
    if rc not in (TA_OK, TA_ERR_WORKSPACE):
        _check(rc)
    buf = np.zeros(max(n.value, 1), dtype=np.int64)
    _check(lib().tree_attn_plan_export(plan.handle, FIELD[field], buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                       buf.size, ctypes.byref(n)))
    buf = buf[: n.value]
    w = FIELD_WIDTH.get(field)
    return buf.reshape(-1, w) if w else buf


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def plan_upload(plan: Plan, device=None, stream=None) -> Plan:
    """Allocate the device workspace with torch and enqueue the plan copy."""
    nbytes = plan_info(plan)["workspace_bytes"]
    dev = torch.device("cuda" if device is None else device)
    with _on(stream):
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    off = (-ws.data_ptr()) % 256
    ws_view = ws[off: off + nbytes]
    _check(lib().tree_attn_plan_upload(plan.handle, ctypes.c_void_p(ws_view.data_ptr()), nbytes,
                                       _stream_handle(stream)))
    plan.workspace = ws
    plan.workspace_view = ws_view
    return plan


def plan_destroy(plan: Plan):
    plan.close()


def scratch_bytes(plan: Plan, hq: int, head_dim: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().tree_attn_scratch_bytes(plan.handle, hq, head_dim, ctypes.byref(n)))
    return int(n.value)


def _scratch(plan, hq, d, device, scratch):
    """Caller-provided scratch (uint8 tensor) or a fresh one; returns the
    256-byte aligned pointer, its usable bytes and the tensor to keep alive
    across the call."""
    need = scratch_bytes(plan, hq, d)
    if need == 0:
        return None, 0, None
    if scratch is None:
        scratch = torch.empty(need + 256, dtype=torch.uint8, device=device)
    off = (-scratch.data_ptr()) % 256
    view = scratch[off:]
    return ctypes.c_void_p(view.data_ptr()), view.numel(), scratch


# ---------------------------------------------------------------------------
# launches
# ---------------------------------------------------------------------------

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TA_DTYPE_BF16
    if t.dtype == torch.float32:
        return TA_DTYPE_F32
    raise TreeAttnError(TA_ERR_UNSUPPORTED, f"dtype {t.dtype} is not supported (bf16 or fp32)")


def _dev_ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise TreeAttnError(TA_ERR_INVALID_ARG, "tensors must live on the GPU")
    if not t.is_contiguous():
        raise TreeAttnError(TA_ERR_INVALID_ARG, "tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _bad(msg):
    return TreeAttnError(TA_ERR_INVALID_ARG, msg)


def _check_args(q, kv_pairs, out=None, lse=None, like_q=(), like_kv=()):
    """Host-side checks of every tensor argument before any pointer is taken.

    The C ABI receives raw pointers and sizes (hq, hkv, head_dim) derived
    from q and the first key tensor, so a tensor of another dtype, head
    count, head_dim or an undersized output would be read or written out of
    bounds on the device.  Checked here: q is [rows, Hq, d]; each (k, v)
    pair is [tokens, Hkv, d] with v shaped like k; every tensor has q's
    dtype and device and is contiguous; `out` and the tensors in `like_q`
    are shaped like q, those in `like_kv` like the first key tensor; `lse`
    is fp32 [Hq, rows].  Returns (hq, hkv, d)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise _bad("q is [rows, Hq, d]")
    _dtype_code(q)
    rows, hq, d = q.shape
    named = [("q", q)]
    hkv = kshape = None
    for (kn, k), (vn, v) in kv_pairs:
        if k is None or v is None:
            raise _bad(f"{kn} and {vn} are required")
        if k.dim() != 3:
            raise _bad(f"{kn} is [tokens, Hkv, d]")
        if tuple(v.shape) != tuple(k.shape):
            raise _bad(f"{vn} {tuple(v.shape)} must have the shape of {kn} {tuple(k.shape)}")
        if k.shape[2] != d:
            raise _bad(f"{kn} has head_dim {k.shape[2]}; q has {d}")
        if hkv is None:
            hkv, kshape = k.shape[1], tuple(k.shape)
        elif k.shape[1] != hkv:
            raise _bad(f"{kn} has {k.shape[1]} KV heads; the first key tensor has {hkv}")
        named += [(kn, k), (vn, v)]
    for name, t in like_q:
        if t is not None and tuple(t.shape) != tuple(q.shape):
            raise _bad(f"{name} {tuple(t.shape)} must have the shape of q {tuple(q.shape)}")
        named.append((name, t))
    for name, t in like_kv:
        if t is not None and tuple(t.shape) != kshape:
            raise _bad(f"{name} {tuple(t.shape)} must have the shape of the key tensor {kshape}")
        named.append((name, t))
    if out is not None:
        if tuple(out.shape) != tuple(q.shape):
            raise _bad(f"out {tuple(out.shape)} must have the shape of q {tuple(q.shape)}")
        named.append(("out", out))
    for name, t in named:
        if t is None:
            continue
        if t.dtype != q.dtype:
            raise _bad(f"{name} is {t.dtype}; q is {q.dtype} (all tensors share one dtype)")
        if t.device != q.device:
            raise _bad(f"{name} is on {t.device}; q is on {q.device}")
        if not t.is_contiguous():
            raise _bad(f"{name} must be contiguous")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (hq, rows):
            raise _bad(f"lse must be float32 [Hq, rows] = [{hq}, {rows}]; got {lse.dtype} {tuple(lse.shape)}")
        if lse.device != q.device or not lse.is_contiguous():
            raise _bad("lse must be contiguous on q's device")
    return hq, hkv, d


def _check_scratch_tensor(scratch, device):
    if scratch is None:
        return
    if scratch.dtype != torch.uint8 or scratch.dim() != 1 or not scratch.is_contiguous():
        raise _bad("scratch is a contiguous 1-D uint8 tensor")
    if scratch.device != device:
        raise _bad(f"scratch is on {scratch.device}; the inputs are on {device}")


def _rows(plan: Plan, q, seg_a=(), seg_b=()):
    """Host-side shape checks against the plan: the kernels index rows and
    keys from the plan's tables, so short tensors would be read out of
    bounds."""
    info = plan_info(plan)
    if q.shape[0] != info["n_rows"]:
        raise TreeAttnError(TA_ERR_INVALID_ARG, f"q has {q.shape[0]} rows; the plan has {info['n_rows']}")
    for t in seg_a:
        if t is not None and t.shape[0] < info["n_keys_a"]:
            raise TreeAttnError(TA_ERR_INVALID_ARG, f"a key/value tensor has {t.shape[0]} tokens; the plan needs "
                                                    f"{info['n_keys_a']}")
    for t in seg_b:
        if t is not None and t.shape[0] < info["n_keys_b"]:
            raise TreeAttnError(TA_ERR_INVALID_ARG, f"a key/value tensor has {t.shape[0]} tokens; the plan needs "
                                                    f"{info['n_keys_b']}")


def _on(stream):
    """Allocate temporaries on the stream the launch uses, so torch's caching
    allocator does not hand their memory to other work while the kernels
    still run there."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _outputs(q, want_lse, out=None, lse=None):
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    return out, (lse if want_lse else None)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def prefill(plan: Plan, q, k, v, scale=None, want_lse=True, out=None, lse=None,
            scratch: Optional[torch.Tensor] = None, stream=None):
    hq, hkv, d = _check_args(q, [(("k", k), ("v", v))], out=out, lse=lse)
    _check_scratch_tensor(scratch, q.device)
    _rows(plan, q, (k, v), (k, v))
    with _on(stream):
        o, l = _outputs(q, want_lse, out, lse)
        sp, sn, keep = _scratch(plan, hq, d, q.device, scratch)
    _check(lib().tree_attn_prefill(plan.handle, _dtype_code(q), hq, hkv, d, _scale(scale, d), _dev_ptr(q),
                                   _dev_ptr(k), _dev_ptr(v), _dev_ptr(o), _dev_ptr(l), sp, sn,
                                   _stream_handle(stream)))
    return o, l


def decode(plan: Plan, q, k_main, v_main, k_suffix, v_suffix, scale=None, want_lse=True, out=None, lse=None,
           scratch: Optional[torch.Tensor] = None, stream=None):
    hq, hkv, d = _check_args(q, [(("k_main", k_main), ("v_main", v_main)),
                                 (("k_suffix", k_suffix), ("v_suffix", v_suffix))], out=out, lse=lse)
    _check_scratch_tensor(scratch, q.device)
    _rows(plan, q, (k_main, v_main), (k_suffix, v_suffix))
    with _on(stream):
        o, l = _outputs(q, want_lse, out, lse)
        sp, sn, keep = _scratch(plan, hq, d, q.device, scratch)
    _check(lib().tree_attn_decode(plan.handle, _dtype_code(q), hq, hkv, d, _scale(scale, d), _dev_ptr(q),
                                  _dev_ptr(k_main), _dev_ptr(v_main), _dev_ptr(k_suffix), _dev_ptr(v_suffix),
                                  _dev_ptr(o), _dev_ptr(l), sp, sn, _stream_handle(stream)))
    return o, l


TA_STATIC_SCRATCH_BYTES = 64 << 20


def decode_noalloc(plan: Plan, q, k_main, v_main, k_suffix, v_suffix, out, lse=None, scale=None, stream=None):
    """tree_attn_decode_noalloc: decode whose partials live in the library's
    file-scope device scratch (the C call allocates nothing).  The caller
    passes the outputs: out like q, lse fp32 [Hq, rows] or None."""
    if out is None:
        raise _bad("decode_noalloc writes into caller-provided outputs: pass out")
    hq, hkv, d = _check_args(q, [(("k_main", k_main), ("v_main", v_main)),
                                 (("k_suffix", k_suffix), ("v_suffix", v_suffix))], out=out, lse=lse)
    _rows(plan, q, (k_main, v_main), (k_suffix, v_suffix))
    _check(lib().tree_attn_decode_noalloc(plan.handle, _dtype_code(q), hq, hkv, d, _scale(scale, d), _dev_ptr(q),
                                          _dev_ptr(k_main), _dev_ptr(v_main), _dev_ptr(k_suffix),
                                          _dev_ptr(v_suffix), _dev_ptr(out), _dev_ptr(lse), _stream_handle(stream)))
    return out, lse


def verify(plan: Plan, q, k_ctx, v_ctx, k_tree, v_tree, scale=None, want_lse=True, out=None, lse=None,
           scratch: Optional[torch.Tensor] = None, stream=None):
    hq, hkv, d = _check_args(q, [(("k_ctx", k_ctx), ("v_ctx", v_ctx)), (("k_tree", k_tree), ("v_tree", v_tree))],
                             out=out, lse=lse)
    _check_scratch_tensor(scratch, q.device)
    _rows(plan, q, (k_ctx, v_ctx), (k_tree, v_tree))
    with _on(stream):
        o, l = _outputs(q, want_lse, out, lse)
        sp, sn, keep = _scratch(plan, hq, d, q.device, scratch)
    _check(lib().tree_attn_verify(plan.handle, _dtype_code(q), hq, hkv, d, _scale(scale, d), _dev_ptr(q),
                                  _dev_ptr(k_ctx), _dev_ptr(v_ctx), _dev_ptr(k_tree), _dev_ptr(v_tree),
                                  _dev_ptr(o), _dev_ptr(l), sp, sn, _stream_handle(stream)))
    return o, l


def backward_scratch_bytes(plan: Plan, hq: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().tree_attn_backward_scratch_bytes(plan.handle, hq, ctypes.byref(n)))
    return int(n.value)


def prefill_backward(plan: Plan, q, k, v, o, lse, d_o, scale=None, dq=None, dk=None, dv=None,
                     scratch: Optional[torch.Tensor] = None, stream=None):
    """Gradients (dq, dk, dv) of the packed forward for output gradient d_o;
    o and lse are the forward's outputs for the same q, k, v."""
    if o is None or d_o is None or lse is None:
        raise _bad("o, lse and d_o are required")
    hq, hkv, d = _check_args(q, [(("k", k), ("v", v))], lse=lse,
                             like_q=(("o", o), ("d_o", d_o), ("dq", dq)), like_kv=(("dk", dk), ("dv", dv)))
    if k.shape[0] != q.shape[0]:
        raise _bad(f"k has {k.shape[0]} tokens; the packed prefill has one key per query row ({q.shape[0]})")
    _check_scratch_tensor(scratch, q.device)
    _rows(plan, q, (k, v), (k, v))
    need = backward_scratch_bytes(plan, hq)
    with _on(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        if scratch is None and need:
            scratch = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    sp, sn = None, 0
    if need:
        off = (-scratch.data_ptr()) % 256
        view = scratch[off:]
        sp, sn = ctypes.c_void_p(view.data_ptr()), view.numel()
    _check(lib().tree_attn_prefill_backward(plan.handle, _dtype_code(q), hq, hkv, d, _scale(scale, d), _dev_ptr(q),
                                            _dev_ptr(k), _dev_ptr(v), _dev_ptr(o), _dev_ptr(lse), _dev_ptr(d_o),
                                            _dev_ptr(dq), _dev_ptr(dk), _dev_ptr(dv), sp, sn,
                                            _stream_handle(stream)))
    return dq, dk, dv


# ---------------------------------------------------------------------------
# draft trees
# ---------------------------------------------------------------------------

TA_ACCEPT_TAU = 0
TA_ACCEPT_EXACT = 1


def draft_tree(accepted, drafts, window: int = 3, max_nodes: int = 64, max_depth: int = 0):
    """Prefix tree of the draft continuations that follow the last `window`
    accepted tokens.  Returns (tokens, parent) int32 arrays; parent -1 marks
    nodes that follow the accepted sequence."""
    acc = _i32(accepted)
    ds = [_i32(d) for d in drafts]
    lens = _i32([len(d) for d in ds])
    cat = np.concatenate(ds) if ds else np.zeros(0, np.int32)
    cat = _i32(cat)
    tok = np.zeros(max(max_nodes, 0), np.int32)
    par = np.zeros(max(max_nodes, 0), np.int32)
    n = ctypes.c_int32()
    _check(lib().tree_attn_draft_tree(_ptr(acc), acc.size, _ptr(cat), _ptr(lens), lens.size, window, max_nodes,
                                      max_depth, _ptr(tok), _ptr(par), ctypes.byref(n)))
    return tok[:n.value].copy(), par[:n.value].copy()


def accept_scratch_bytes(plan: Plan, vocab: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().tree_attn_accept_scratch_bytes(plan.handle, vocab, ctypes.byref(n)))
    return int(n.value)


def accept(plan: Plan, logits, tokens, tau: float = 0.75, exact: bool = False, vocab: int = None,
           path=None, n_path=None, next_token=None, scratch: Optional[torch.Tensor] = None, stream=None):
    """Greedy acceptance over the trees of a verify plan.

    logits: [n_nodes + n_trees, ld] bf16/fp32 on the GPU, tree-major (row 0 of
    a tree scores the token after the accepted sequence, row 1 + i the token
    after node i); tokens: int32 [n_nodes].  Returns (path, n_path,
    next_token) int32 tensors: tree b's accepted nodes are
    path[node_off[b] : node_off[b] + n_path[b]]."""
    if logits.dim() != 2:
        raise TreeAttnError(TA_ERR_INVALID_ARG, "logits is [rows, ld]")
    ld = logits.shape[1]
    vocab = ld if vocab is None else int(vocab)
    info = plan_info(plan)
    n_nodes, n_trees = info["n_rows"], info["n_branches"]
    if logits.shape[0] < n_nodes + n_trees:
        raise TreeAttnError(TA_ERR_INVALID_ARG, "logits needs n_nodes + n_trees rows")
    if tokens.dtype != torch.int32 or tokens.numel() < n_nodes:
        raise TreeAttnError(TA_ERR_INVALID_ARG, "tokens must be int32 with one entry per node")
    for name, t, n in (("path", path, n_nodes), ("n_path", n_path, n_trees), ("next_token", next_token, n_trees)):
        if t is not None and (t.dtype != torch.int32 or t.numel() < n):
            raise TreeAttnError(TA_ERR_INVALID_ARG, f"{name} must be int32 with at least {n} entries")
    dev = logits.device
    for name, t in (("logits", logits), ("tokens", tokens), ("path", path), ("n_path", n_path),
                    ("next_token", next_token)):
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise _bad(f"{name} must be contiguous on the logits' device")
    _check_scratch_tensor(scratch, dev)
    need = accept_scratch_bytes(plan, vocab)
    with _on(stream):
        path = torch.zeros(max(n_nodes, 1), dtype=torch.int32, device=dev) if path is None else path
        n_path = torch.empty(max(n_trees, 1), dtype=torch.int32, device=dev) if n_path is None else n_path
        next_token = torch.empty(max(n_trees, 1), dtype=torch.int32, device=dev) if next_token is None else next_token
        if scratch is None:
            scratch = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    off = (-scratch.data_ptr()) % 256
    view = scratch[off:]
    _check(lib().tree_attn_accept(plan.handle, _dtype_code(logits), _dev_ptr(logits), vocab, ld, _dev_ptr(tokens),
                                  float(tau), TA_ACCEPT_EXACT if exact else TA_ACCEPT_TAU, _dev_ptr(path),
                                  _dev_ptr(n_path), _dev_ptr(next_token), ctypes.c_void_p(view.data_ptr()),
                                  view.numel(), _stream_handle(stream)))
    return path[:n_nodes], n_path[:n_trees], next_token[:n_trees]


# ---------------------------------------------------------------------------
# paged KV: plans over block tables, and the host block pool
# ---------------------------------------------------------------------------

def _tables(tables):
    """List of per-sequence block lists -> (concatenated int32, int64 offsets)."""
    off = np.zeros(len(tables) + 1, np.int64)
    for i, tb in enumerate(tables):
        off[i + 1] = off[i] + len(tb)
    cat = np.ascontiguousarray(np.concatenate([np.asarray(tb, np.int32) for tb in tables])
                               if tables and off[-1] else np.zeros(0, np.int32), dtype=np.int32)
    return cat, off


def _p64(a: np.ndarray):
    return a.ctypes.data_as(_I64P) if a.size else None


def plan_decode_paged(prefix_len, n_regions, layout_len, br_page, br_region, suffix_len, n_query,
                      block_size: int, n_cache_blocks: int, main_tables, suffix_tables) -> Plan:
    """Decode plan whose main streams and suffixes live in a paged cache:
    main_tables[p] / suffix_tables[b] are block-id lists."""
    P, N, L = _i32(prefix_len), _i32(n_regions), _i32(layout_len)
    bp, br, s = _i32(br_page), _i32(br_region), _i32(suffix_len)
    kq = None if n_query is None else _i32(n_query)
    mb, mo = _tables(main_tables)
    sb, so = _tables(suffix_tables)
    out = ctypes.c_void_p()
    _check(lib().tree_attn_plan_decode_paged(_ptr(P), _ptr(N), _ptr(L), int(P.size), _ptr(bp), _ptr(br), _ptr(s),
                                             None if kq is None else _ptr(kq), int(bp.size), block_size,
                                             n_cache_blocks, _ptr(mb), _p64(mo), _ptr(sb), _p64(so),
                                             ctypes.byref(out)))
    return Plan(out.value, TA_PLAN_DECODE)


def plan_verify_paged(ctx_len, br_page, n_nodes, parent, block_size: int, n_cache_blocks: int, ctx_tables) -> Plan:
    c, bp, nn, pa = _i32(ctx_len), _i32(br_page), _i32(n_nodes), _i32(parent)
    cb, co = _tables(ctx_tables)
    out = ctypes.c_void_p()
    _check(lib().tree_attn_plan_verify_paged(_ptr(c), int(c.size), _ptr(bp), _ptr(nn), _ptr(pa), int(bp.size),
                                             block_size, n_cache_blocks, _ptr(cb), _p64(co), ctypes.byref(out)))
    return Plan(out.value, TA_PLAN_VERIFY)


class KVPool:
    """Host block pool of a paged KV cache (see tree_attn_pool_* in the header)."""

    def __init__(self, n_blocks: int, block_size: int):
        h = ctypes.c_void_p()
        _check(lib().tree_attn_pool_create(n_blocks, block_size, ctypes.byref(h)))
        self.handle, self.n_blocks, self.block_size = h, n_blocks, block_size

    def new_seq(self) -> int:
        s = ctypes.c_int32()
        _check(lib().tree_attn_pool_new_seq(self.handle, ctypes.byref(s)))
        return s.value

    def fork(self, parent: int, n_tokens: int) -> int:
        s = ctypes.c_int32()
        _check(lib().tree_attn_pool_fork(self.handle, parent, n_tokens, ctypes.byref(s)))
        return s.value

    def append(self, seq: int, n_tokens: int) -> np.ndarray:
        slots = np.zeros(max(n_tokens, 0), np.int64)
        _check(lib().tree_attn_pool_append(self.handle, seq, n_tokens, _p64(slots)))
        return slots

    def release(self, seq: int):
        _check(lib().tree_attn_pool_release(self.handle, seq))

    def table(self, seq: int):
        """(view blocks, view tokens, own blocks, own tokens)."""
        vt, ot = ctypes.c_int32(), ctypes.c_int32()
        rc = lib().tree_attn_pool_table(self.handle, seq, None, 0, ctypes.byref(vt), None, 0, ctypes.byref(ot))
        if rc not in (TA_OK, TA_ERR_WORKSPACE):
            _check(rc)
        bs = self.block_size
        v = np.zeros((vt.value + bs - 1) // bs, np.int32)
        o = np.zeros((ot.value + bs - 1) // bs, np.int32)
        _check(lib().tree_attn_pool_table(self.handle, seq, _ptr(v), v.size, ctypes.byref(vt), _ptr(o), o.size,
                                          ctypes.byref(ot)))
        return v, vt.value, o, ot.value

    def refs(self):
        r = np.zeros(self.n_blocks, np.int32)
        f = ctypes.c_int32()
        _check(lib().tree_attn_pool_refs(self.handle, _ptr(r) if r.size else None, self.n_blocks, ctypes.byref(f)))
        return r, f.value

    def close(self):
        if self.handle:
            lib().tree_attn_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# roofline calibration (measurement only)
# ---------------------------------------------------------------------------

def calib_mfma(blocks: int, iters: int, sink: torch.Tensor, seed: int = 0, stream=None) -> int:
    """Enqueue the bf16 MFMA loop (seed 0: one fixed operand pair; otherwise
    pseudo-random operands that differ between instructions); returns its
    FLOP count.  sink: float32 tensor of >= 4 * blocks entries on the GPU."""
    if sink.dtype != torch.float32 or sink.numel() < 4 * blocks:
        raise _bad("sink must be float32 with at least 4 * blocks entries")
    flops = ctypes.c_int64()
    _check(lib().tree_attn_calib_mfma(int(blocks), int(iters), int(seed) & 0xFFFFFFFF, _dev_ptr(sink),
                                      ctypes.byref(flops),
                                      _stream_handle(stream)))
    return int(flops.value)


def calib_read(src: torch.Tensor, blocks: int, sink: torch.Tensor, stream=None) -> int:
    """Enqueue the streaming read of the whole of src; returns its bytes.
    sink: int32 tensor of >= blocks entries on the GPU."""
    if sink.dtype != torch.int32 or sink.numel() < blocks:
        raise _bad("sink must be int32 with at least `blocks` entries")
    nbytes = src.numel() * src.element_size()
    _check(lib().tree_attn_calib_read(_dev_ptr(src), nbytes, int(blocks), _dev_ptr(sink), _stream_handle(stream)))
    return nbytes


def calib_tile(variant: int, blocks: int, iters: int, sink: torch.Tensor, src: torch.Tensor = None,
               seed: int = 0, stream=None) -> int:
    """Enqueue the tile-loop model (variant 0: register operands, 1: LDS
    operands, 2: LDS operands and a copy per iteration from src; seed 0:
    fixed operand patterns, otherwise pseudo-random ones); returns its MFMA
    FLOP count.  sink: float32 tensor of >= 4 * blocks entries on the GPU;
    src (variant 2): a GPU tensor of >= 262,144 bytes."""
    if sink.dtype != torch.float32 or sink.numel() < 4 * blocks:
        raise _bad("sink must be float32 with at least 4 * blocks entries")
    sp, nbytes = None, 0
    if src is not None:
        sp, nbytes = _dev_ptr(src), src.numel() * src.element_size()
    flops = ctypes.c_int64()
    _check(lib().tree_attn_calib_tile(int(variant), int(blocks), int(iters), int(seed) & 0xFFFFFFFF, sp, nbytes,
                                      _dev_ptr(sink), ctypes.byref(flops), _stream_handle(stream)))
    return int(flops.value)
