"""Helpers (no tests): decode a plan's device image into its tables and
compare them with the oracle's plan of the same description.

The image is what tree_attn_plan_upload copies to the device workspace; its
section offsets come from TA_FIELD_DEVICE_LAYOUT.  Per row, row_a and row_b
hold the visibility bounds the kernels test (prefill: main_end and
branch_start; decode: the absolute ends of the row's main keys and suffix
keys; verify: the end of the page's context and the tree's first node),
which the oracle's plan functions define independently of the library.
"""
import numpy as np

import oracle

SECTIONS = ("work", "row_a", "row_b", "mask", "merge", "kwork", "kmerge", "trees", "tile_a", "tile_b", "total")


def image_tables(plan, image: np.ndarray):
    """Split a device image (uint8) into its tables."""
    lay = dict(zip(SECTIONS, (int(x) for x in plan.export("device_layout"))))
    info = plan.info
    assert image.size == lay["total"] == info["workspace_bytes"]
    rows, n_work = info["n_rows"], info["n_work"]

    def sec(name, count, dtype):
        nbytes = count * np.dtype(dtype).itemsize
        return image[lay[name]:lay[name] + nbytes].view(dtype)

    return {
        "work": sec("work", n_work * 12, np.int32).reshape(n_work, 12),
        "row_a": sec("row_a", rows, np.int32),
        "row_b": sec("row_b", rows, np.int32),
        "mask": sec("mask", rows if plan.kind == 3 else 0, np.uint64),
        "layout": lay,
    }


def check_against_oracle(plan, desc, image: np.ndarray):
    """The image's per-row bounds equal the oracle plan's; its work list
    equals the host work list the plan exports (WorkItem field order:
    row0, nrows, a_lo, a_full, a_hi, b_lo, b_hi, out, flags, tile_lo,
    tile_hi, b_full)."""
    t = image_tables(plan, image)
    kind = plan.kind
    if kind == 1:
        ref = oracle.plan_prefill(desc)
        assert np.array_equal(t["row_a"], ref["main_end"]), "row_a != main_end"
        assert np.array_equal(t["row_b"], ref["branch_start"]), "row_b != branch_start"
    elif kind == 2:
        r = oracle.plan_decode(desc)["rows"]
        assert np.array_equal(t["row_a"], r[:, 0] + r[:, 1]), "row_a != main end"
        assert np.array_equal(t["row_b"], r[:, 2] + r[:, 3]), "row_b != suffix end"
    else:
        ref = oracle.plan_verify(desc)
        r = ref["rows"]
        assert np.array_equal(t["row_a"], r[:, 0] + r[:, 1]), "row_a != context end"
        assert np.array_equal(t["row_b"], r[:, 2]), "row_b != tree base"
        assert np.array_equal(t["mask"], ref["mask"]), "row_mask != ancestor bitmask"
    w = plan.export("work")  # row0, nrows, a_lo, a_full, a_hi, b_lo, b_hi, out, tile_lo, tile_hi, flags
    img = t["work"]
    assert np.array_equal(img[:, :8], w[:, :8]) and np.array_equal(img[:, 9:11], w[:, 8:10]) \
        and np.array_equal(img[:, 8], w[:, 10]), "work list differs from the exported one"
    return t
