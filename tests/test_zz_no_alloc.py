"""m3_layer_prefill_noalloc, the entry point that allocates nothing (its sequence split uses the
library's own device scratch array), against m3_layer_prefill with a caller workspace: two calls
in a row, the second with a smaller input, each split into segments, so the second call runs on
scratch that still holds the first call's values.  Both calls run the same kernels on the same
plan, so their outputs must be identical; sampled heads are also checked against the fp64 oracle
at the bf16 bar (2e-2).  Every call goes through the C ABI."""
from __future__ import annotations

import pytest
import torch

import oracle
from gpu_util import TOL, angle_err, rel_err
from state_space_sequence_m3_amd import inputs, m3scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _slice_head(inp, hi):
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
        elif k in ("x", "B", "C", "dt", "lam", "theta"):
            out[k] = v[:, :, hi:hi + 1].cpu()
        elif k in ("A", "bias_B", "bias_C", "w_out", "normw_B", "normw_C"):
            out[k] = v[hi:hi + 1].cpu()
        else:
            out[k] = v[:, hi:hi + 1].cpu()
    return out


def _args(d, w):
    return (d["x"], d["B"], d["C"], d["dt"], d["theta"], d["A"], d["lam"], d.get("normw_B"), d.get("normw_C"),
            d.get("bias_B"), d.get("bias_C"), d["w_out"] if w.mix else None, d.get("phi_in"), d.get("h_in"),
            d.get("Bbar_prev"), d.get("x_prev"))


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_the_workspace_call(order):
    calls = [
        # the long-context workload (b1 L16384 H64 R4: 64 (b, h) pairs, split into 8 segments)
        (inputs.WORKLOADS["long_mimo4_b1_l16384"], [3, 58], 8),
        # smaller: 4 pairs of 3000 steps, 2 segments, SISO, its own carried state and angle
        (inputs.Workload("noalloc_small", 1, 3000, 4, 64, 128, 1, 32, "bf16", True, True, False, 1.0), [1, 3], 32),
    ]
    for w, heads, chunk in calls:
        print("noalloc call", w.name, flush=True)
        dims = m3scan.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, chunk, m3scan.M3_BF16)
        need = m3scan.layer_prefill_workspace_bytes(dims)
        assert 0 < need <= m3scan.NOALLOC_SCRATCH_BYTES, need
        carry = w.name == "noalloc_small"
        inp = inputs.make_prefill_inputs(w, seed=91, device=DEV, normw=True, carry=carry)
        ya, ha, pa = m3scan.m3_layer_prefill(*_args(inp, w), chunk=chunk)
        yb, hb, pb = m3scan.m3_layer_prefill_noalloc(*_args(inp, w), chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb) and torch.equal(ha, hb) and torch.equal(pa, pb)
        for hi in heads:
            ref = oracle.layer(_slice_head(inp, hi), bcnorm=True, mix=w.mix)
            assert rel_err(yb[:, :, hi:hi + 1], ref["y"]) <= TOL["bf16"], hi
            assert rel_err(hb[:, hi:hi + 1], ref["h_out"]) <= TOL["bf16"], hi
            assert angle_err(pb[:, hi:hi + 1], ref["phi_out"]) <= 1e-3, hi
        del inp, ya, yb
        torch.cuda.empty_cache()


def test_noalloc_without_a_split_uses_no_scratch():
    """A call whose pairs fill the GPU runs in one pass, exactly as m3_layer_prefill does."""
    w = inputs.Workload("noalloc_dense", 8, 256, 64, 64, 128, 1, 32, "bf16", True, True, False, 1.0)
    dims = m3scan.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, 32, m3scan.M3_BF16)
    assert m3scan.layer_prefill_workspace_bytes(dims) == 0
    inp = inputs.make_prefill_inputs(w, seed=92, device=DEV)
    ya, ha, pa = m3scan.m3_layer_prefill(*_args(inp, w), chunk=32)
    yb, hb, pb = m3scan.m3_layer_prefill_noalloc(*_args(inp, w), chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb) and torch.equal(ha, hb) and torch.equal(pa, pb)
