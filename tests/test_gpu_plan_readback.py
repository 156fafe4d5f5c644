"""Plan parity on the device: the workspace tree_attn_plan_upload fills is
read back and compared byte for byte with the plan's host image, and its
per-row bounds and ancestor bitmasks with the oracle's plan of the same
description (bit-exact integers)."""
import numpy as np
import pytest
import torch

import plan_image
from tree_structured_attention_amd import binding as ta
from tree_structured_attention_amd import synth

pytestmark = pytest.mark.gpu


def readback(plan):
    torch.cuda.synchronize()
    return plan.workspace_view.cpu().numpy()


@pytest.mark.parametrize("which", ["prefill_config2", "prefill_config3_balanced", "decode_config4",
                                   "decode_multi", "verify_config5", "prefill_edges"])
def test_uploaded_workspace_equals_host_image_and_oracle(which):
    if which == "prefill_config2":
        desc = synth.config2(with_tensors=False).desc
        plan = ta.plan_for(desc)
    elif which == "prefill_config3_balanced":
        desc = synth.config3(with_tensors=False).desc
        plan = ta.plan_for(desc).balance(8)
    elif which == "decode_config4":
        desc = synth.config4(with_tensors=False).desc
        plan = ta.plan_for(desc)
    elif which == "decode_multi":
        desc = synth.decode_multi(with_tensors=False).desc
        plan = ta.plan_for(desc)
    elif which == "verify_config5":
        desc = synth.config5(with_tensors=False).desc
        plan = ta.plan_for(desc)
    else:
        desc = synth.make_prefill_desc([200, 0, 65, 1], [np.array([3, 0, 5, 2, 1]), np.array([4]), np.array([]),
                                                         np.array([0])],
                                       [np.array([70, 0, 9, 130, 1]), np.array([3]), np.array([]),
                                        np.array([200])])
        plan = ta.plan_for(desc)
    host = plan.export("device_image").view(np.uint8)
    plan.upload()
    dev = readback(plan)
    assert dev.size == host.size
    assert np.array_equal(dev, host), f"{which}: {int((dev != host).sum())} bytes differ"
    t = plan_image.check_against_oracle(plan, desc, dev)
    print(f"[readback] {which}: {dev.size} bytes, {t['work'].shape[0]} work items, "
          f"{t['row_a'].size} rows equal to the oracle plan", flush=True)
