"""The GPU's replica tree against the hand-derived cases of
tests/golden/reduction_order.json (the pages' averaging formula and their
point that the reduction order changes the bits; the derivations are in the
file).  The cases hold the same values in different orders and expect
different g_bar, so they are also the negative control: a tree with another
order, or with a wider intermediate precision, fails them.  Checked in the
three ways the library forms g_bar: from incoming partials, from the
accumulators, and with the last micro-step fused into the tree."""
import json
import os

import numpy as np
import pytest
import torch

import gradient_reduce_adam_amd as dp

from gpu_common import log

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "reduction_order.json")
P = 1000  # three full pieces and a ragged tail


@pytest.mark.parametrize("mode", ["partials", "accumulators", "fused"])
def test_tree_matches_hand_derived_cases(mode):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    s = torch.cuda.current_stream().cuda_stream
    for case in cases:
        vals = case["replicas"]
        n = len(vals)
        plan = dp.Plan((P,), n, "bf16", "bf16")
        grads = [torch.full((P,), v, dtype=torch.bfloat16, device="cuda") for v in vals]
        zeros = torch.zeros(P, dtype=torch.bfloat16, device="cuda")
        acc = torch.zeros((n, P), dtype=torch.float32, device="cuda")
        gbar = torch.full((P,), -1.0, dtype=torch.float32, device="cuda")
        try:
            plan.bind("gbar", gbar)
            for r in range(n):
                plan.bind("acc", acc[r], r)
            plan.state_init(0.9, 0.999, stream=s)
            if mode == "partials":
                for r in range(n):
                    plan.bind("grad", grads[r], r)
                plan.reduce_replicas("grad", stream=s)
            elif mode == "accumulators":
                for r in range(n):
                    plan.bind("grad", grads[r], r)
                plan.accumulate_all(first=True, stream=s)  # acc_r = the exact binary32 value
                plan.reduce_replicas("acc", stream=s)
            else:
                for r in range(n):
                    plan.bind("grad", zeros, r)
                plan.accumulate_all(first=True, stream=s)  # acc_r = 0
                for r in range(n):
                    plan.bind("grad", grads[r], r)
                plan.accumulate_reduce(stream=s)  # tree of (0 + g_r) = tree of g_r
            torch.cuda.synchronize()
            got = gbar.cpu().numpy()
        finally:
            plan.close()
        want = np.float32(case["gbar"])
        log(f"{mode} {vals}: gpu {got[0]!r} want {want!r}")
        assert np.all(got.view(np.uint32) == want.view(np.uint32)), (mode, vals, np.unique(got), want)
