"""Parity at the full workload sizes, in the launch configuration bench.py times.

The GPU runs the whole batch; the fp64 oracle recomputes a few sampled (batch, head) pairs from
the same inputs (every (batch, head) is independent, so a sampled pair is checked exactly, not
approximately).  Inputs are drawn on the device with a seeded generator; the sampled slices are
copied to the host for the oracle.

Errors are normwise per output tensor, max|gpu - ref| / max|ref|; for decode the output tensor is
y over all decode steps of the run, and each step's y is also judged on its own: its error
against its own largest value, or against a floor of the run's largest where the step's y is
smaller than that (a single step's y can be far below its typical size when the sum over the
state rows nearly cancels; its absolute error is then the usual one).  The floor is 1% for
m3_layer_decode_step and 10% for m3_bcnorm_rope + m3_decode_step, whose rotated Bbar and Cbar are
rounded to bf16 between the two calls: that rounding (2^-9 of each element) reaches y_t through a
sum over the N state rows and the state built from the rounded Bbar, and leaves an absolute error
of about 1e-3 of the run's largest y in a cancelling step (1.1e-3 at worst over the sampled
pairs), so 1% would judge rounding as failure.  A step that is wrong (a stale or missing carry, a
skipped update) is off by the order of its own size and fails either bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, angle_err, per_step_rel_err, rel_err, to_np
from state_space_sequence_m3_amd import inputs, m3scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

SEQ_KEYS = ("x", "B", "C", "dt", "lam", "theta")


def _slice_pair(inp, bi, hi):
    """Host copy of one (batch, head) pair's prefill inputs, with per-head constants."""
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
        elif k in SEQ_KEYS:
            out[k] = v[bi:bi + 1, :, hi:hi + 1].cpu()
        elif k == "A":
            out[k] = v[hi:hi + 1].cpu()
        elif k in ("bias_B", "bias_C", "w_out", "normw_B", "normw_C"):
            out[k] = v[hi:hi + 1].cpu()
        else:  # carried state [b, H, ...]
            out[k] = v[bi:bi + 1, hi:hi + 1].cpu()
    return out


def _layer(d, w):
    Bb, Cb, phi = m3scan.m3_bcnorm_rope(d["B"], d["C"], d["dt"], d["theta"], d["normw_B"],
                                        d["normw_C"], d["bias_B"], d["bias_C"], d.get("phi_in"),
                                        bcnorm=w.bcnorm)
    y, h = m3scan.m3_prefill(d["x"], Bb, Cb, d["dt"], d["A"], d["lam"], d["w_out"] if w.mix else None,
                             d.get("h_in"), d.get("Bbar_prev"), d.get("x_prev"), chunk=w.chunk)
    return Bb, Cb, y, h, phi


def _fused_layer(d, w):
    """m3_layer_prefill in the launch configuration bench.py times (chunk * R = 32)."""
    return m3scan.m3_layer_prefill(d["x"], d["B"], d["C"], d["dt"], d["theta"], d["A"], d["lam"],
                                   d["normw_B"], d["normw_C"], d["bias_B"], d["bias_C"],
                                   d["w_out"] if w.mix else None, d.get("phi_in"), d.get("h_in"),
                                   d.get("Bbar_prev"), d.get("x_prev"), chunk=32 // w.rank,
                                   bcnorm=w.bcnorm)


@pytest.mark.parametrize("name,pairs", [
    ("siso_b8_l2048", [(0, 0), (1, 31), (2, 46), (3, 17), (5, 8), (7, 63)]),
    ("mimo4_b8_l2048", [(0, 5), (2, 62), (4, 23), (6, 40)]),
    ("mamba2_siso_b8_l2048", [(1, 2), (7, 60)]),
    ("siso_n64_b8_l2048", [(2, 9), (5, 33)]),
    # the rest of the comparison grid (Mamba-2 mode / SISO / MIMO R = 4 x fp32 / bf16 x N 64 / 128)
    ("mimo4_n64_b8_l2048", [(1, 7)]),
    ("mamba2_siso_n64_b8_l2048", [(6, 21)]),
    ("siso_f32_b8_l2048", [(2, 11)]),
    ("siso_n64_f32_b8_l2048", [(7, 0)]),
    ("mimo4_f32_b8_l2048", [(4, 50)]),
    ("mimo4_n64_f32_b8_l2048", [(3, 63)]),
    ("mamba2_siso_f32_b8_l2048", [(0, 30)]),
    ("mamba2_siso_n64_f32_b8_l2048", [(5, 44)]),
])
@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
def test_prefill_workload_sampled(name, pairs, fused):
    w = inputs.WORKLOADS[name]
    print("workload", name, "fused" if fused else "two calls", flush=True)
    inp = inputs.make_prefill_inputs(w, seed=1, device=DEV)
    if fused:
        y, h, phi = _fused_layer(inp, w)
    else:
        _, _, y, h, phi = _layer(inp, w)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(h).all()
    for bi, hi in pairs:
        ref = oracle.layer(_slice_pair(inp, bi, hi), bcnorm=w.bcnorm, mix=w.mix)
        ys = y[bi:bi + 1, :, hi:hi + 1]
        assert rel_err(ys, ref["y"]) <= TOL[w.io], (bi, hi)
        assert rel_err(h[bi:bi + 1, hi:hi + 1], ref["h_out"]) <= TOL[w.io], (bi, hi)
        assert angle_err(phi[bi:bi + 1, hi:hi + 1], ref["phi_out"]) <= 1e-3



@pytest.mark.parametrize("name,pairs", [
    ("siso_b8_l2048", [(0, 3), (4, 27), (6, 58)]),
    ("mimo4_b8_l2048", [(1, 12), (5, 49), (7, 33)]),
    ("long_mimo4_b1_l16384", [(0, 17)]),
])
def test_two_calls_bench_chunk_sampled(name, pairs):
    """m3_bcnorm_rope + m3_prefill on chunks of 32 rows (chunk * R = 32), the launch configuration
    bench.py times for the two-call path (the long-context workload: its sequence split)."""
    w = inputs.WORKLOADS[name]
    wc = w.with_(chunk=32 // w.rank)
    print("workload", name, "two calls, chunk", wc.chunk, flush=True)
    inp = inputs.make_prefill_inputs(w, seed=2, device=DEV, carry=True)
    _, _, y, h, phi = _layer(inp, wc)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(h).all()
    for bi, hi in pairs:
        ref = oracle.layer(_slice_pair(inp, bi, hi), bcnorm=w.bcnorm, mix=w.mix)
        assert rel_err(y[bi:bi + 1, :, hi:hi + 1], ref["y"]) <= TOL[w.io], (bi, hi)
        assert rel_err(h[bi:bi + 1, hi:hi + 1], ref["h_out"]) <= TOL[w.io], (bi, hi)
        assert angle_err(phi[bi:bi + 1, hi:hi + 1], ref["phi_out"]) <= 1e-3

def _decode_steps(w, dinp, steps, mix, h, phi, Bprev, xprev, consts_dev, toks, fused=False):
    """`steps` tokens, each m3_bcnorm_rope (L = 1) + m3_decode_step, or with `fused` one
    m3_layer_decode_step; the rotated-B buffers are swapped between steps."""
    Bcur = torch.empty_like(Bprev)
    Ccur = torch.empty_like(Bprev)
    ys = []
    for s in range(steps):
        if fused:
            y, _ = m3scan.m3_layer_decode_step(h, phi, Bprev, xprev, toks["x"][s], toks["B"][s],
                                               toks["C"][s], toks["dt"][s], toks["theta"][s],
                                               consts_dev["A"], toks["lam"][s], None, None,
                                               consts_dev["bias_B"], consts_dev["bias_C"],
                                               consts_dev["w_out"] if mix else None, Bbar_out=Bcur)
        else:
            m3scan.m3_bcnorm_rope(toks["B"][s].unsqueeze(1), toks["C"][s].unsqueeze(1),
                                  toks["dt"][s].unsqueeze(1), toks["theta"][s].unsqueeze(1), None, None,
                                  consts_dev["bias_B"], consts_dev["bias_C"], phi,
                                  Bbar=Bcur.unsqueeze(1), Cbar=Ccur.unsqueeze(1), phi_out=phi)
            y = m3scan.m3_decode_step(h, Bprev, xprev, toks["x"][s], Bcur, Ccur, toks["dt"][s],
                                      consts_dev["A"], toks["lam"][s],
                                      consts_dev["w_out"] if mix else None)
        ys.append(y)
        Bprev, Bcur = Bcur, Bprev
        xprev = toks["x"][s]
    return ys, Bprev, xprev


@pytest.mark.parametrize("name,pairs", [
    ("decode_b128_r1", [(0, 0), (40, 50), (77, 31), (127, 63)]),
    ("decode_b128_r4", [(5, 2), (64, 33), (99, 9), (120, 60)]),
    # a state four times the Infinity Cache (the DRAM-bound decode lines of the benchmark)
    ("decode_b512_r1", [(0, 0), (255, 12), (511, 63)]),
    ("decode_b512_r4", [(100, 44), (300, 7), (511, 0)]),
])
@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
def test_decode_workload_sampled(name, pairs, fused):
    w = inputs.WORKLOADS[name]
    print("workload", name, "fused" if fused else "two calls", flush=True)
    steps = w.decode_steps
    dinp = inputs.make_decode_inputs(w, seed=3, steps=steps, device=DEV)
    st = dinp["state"]
    h = st["h"].clone()
    phi = st["phi"].clone()
    ys, _, _ = _decode_steps(w, dinp, steps, w.mix, h, phi, st["Bbar_prev"].clone(),
                             st["x_prev"].clone(), dinp, dinp["tokens"], fused=fused)
    torch.cuda.synchronize()
    floor = 1e-2 if fused else 1e-1
    step_errs = []
    for bi, hi in pairs:
        consts = {"A": dinp["A"][hi:hi + 1].cpu(), "bias_B": dinp["bias_B"][hi:hi + 1].cpu(),
                  "bias_C": dinp["bias_C"][hi:hi + 1].cpu(),
                  "w_out": dinp["w_out"][hi:hi + 1].cpu() if w.mix else None}
        state = {k: st[k][bi:bi + 1, hi:hi + 1].cpu() for k in ("phi", "Bbar_prev", "x_prev")}
        state["h"] = st["h"][bi:bi + 1, hi:hi + 1].cpu()
        rys = []
        for s in range(steps):
            tok = {k: dinp["tokens"][k][s, bi:bi + 1, hi:hi + 1].cpu() for k in SEQ_KEYS}
            ry, state = oracle.decode_step(state, tok, consts, mix=w.mix)
            rys.append(ry)
        # y over all decode steps is one output tensor: normwise error over the whole of it, and
        # step by step
        yg = torch.stack([y[bi:bi + 1, hi:hi + 1] for y in ys], 0)
        err = rel_err(yg, np.stack(rys, 0))
        assert err <= TOL[w.io], (bi, hi, err)
        step_errs.append((bi, hi, per_step_rel_err(yg, np.stack(rys, 0), 0, floor)))
        assert rel_err(h[bi:bi + 1, hi:hi + 1], state["h"]) <= TOL[w.io]
        assert angle_err(phi[bi:bi + 1, hi:hi + 1], state["phi"]) <= 1e-3
    assert max(e for _, _, e in step_errs) <= TOL[w.io], step_errs


def test_long_context_prefill_then_decode_sampled():
    """b=1, L=16384, MIMO R=4, theta ~ N(0, pi^2); then 512 decode steps from the final state."""
    w = inputs.WORKLOADS["long_mimo4_b1_l16384"]
    print("workload", w.name, flush=True)
    inp = inputs.make_prefill_inputs(w, seed=4, device=DEV)
    b, H, R, N, P = w.batch, w.nheads, w.rank, w.dstate, w.headdim
    Bb, Cb, phi = m3scan.m3_bcnorm_rope(inp["B"], inp["C"], inp["dt"], inp["theta"], None, None,
                                        inp["bias_B"], inp["bias_C"])
    Bl = torch.empty((b, H, R, N), dtype=torch.bfloat16, device=DEV)
    xl = torch.empty((b, H, R, P), dtype=torch.bfloat16, device=DEV)
    y, h = m3scan.m3_prefill(inp["x"], Bb, Cb, inp["dt"], inp["A"], inp["lam"], inp["w_out"],
                             Bbar_last=Bl, x_last=xl, chunk=w.chunk)
    torch.cuda.synchronize()
    dsteps = w.decode_steps
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    toks = inputs.make_sequence(w, g, DEV, (dsteps, b))
    ys, _, _ = _decode_steps(w, None, dsteps, True, h, phi, Bl, xl, inp, toks)
    torch.cuda.synchronize()
    for hi in (0, 41):
        pair = _slice_pair(inp, 0, hi)
        ref = oracle.layer(pair, mix=True)
        assert rel_err(y[:, :, hi:hi + 1], ref["y"]) <= TOL["bf16"], hi
        state = {"h": ref["h_out"], "phi": ref["phi_out"], "Bbar_prev": ref["Bbar_last"],
                 "x_prev": ref["x_last"]}
        consts = {"A": pair["A"], "bias_B": pair["bias_B"], "bias_C": pair["bias_C"],
                  "w_out": pair["w_out"]}
        rys = []
        for s in range(dsteps):
            tok = {k: toks[k][s, 0:1, hi:hi + 1].cpu() for k in SEQ_KEYS}
            ry, state = oracle.decode_step(state, tok, consts, mix=True)
            rys.append(ry)
        yg = torch.stack([y[:, hi:hi + 1] for y in ys], 0)
        err = rel_err(yg, np.stack(rys, 0))
        assert err <= TOL["bf16"], (hi, err)
        serr = per_step_rel_err(yg, np.stack(rys, 0), 0)
        assert serr <= TOL["bf16"], (hi, serr)
        assert rel_err(h[:, hi:hi + 1], state["h"]) <= TOL["bf16"]
        assert angle_err(phi[:, hi:hi + 1], state["phi"]) <= 1e-3


def test_long_context_layer_prefill_sampled():
    """m3_layer_prefill on b=1, L=16384, MIMO R=4 (64 (b, h) pairs: the call splits each sequence
    into segments that run in parallel), sampled heads against the oracle."""
    w = inputs.WORKLOADS["long_mimo4_b1_l16384"]
    print("workload", w.name, "fused", flush=True)
    inp = inputs.make_prefill_inputs(w, seed=6, device=DEV)
    dims = m3scan.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, 0, m3scan.M3_BF16)
    assert m3scan.layer_prefill_workspace_bytes(dims) > 0
    y, h, phi = m3scan.m3_layer_prefill(inp["x"], inp["B"], inp["C"], inp["dt"], inp["theta"], inp["A"],
                                        inp["lam"], None, None, inp["bias_B"], inp["bias_C"], inp["w_out"])
    torch.cuda.synchronize()
    for hi in (3, 20, 47, 58):
        ref = oracle.layer(_slice_pair(inp, 0, hi), mix=True)
        assert rel_err(y[:, :, hi:hi + 1], ref["y"]) <= TOL["bf16"], hi
        assert rel_err(h[:, hi:hi + 1], ref["h_out"]) <= TOL["bf16"], hi
        assert angle_err(phi[:, hi:hi + 1], ref["phi_out"]) <= 1e-3, hi


@pytest.mark.parametrize("name,head", [("siso_b8_l2048", 17), ("mimo4_b8_l2048", 40)])
def test_backward_workload_sampled(name, head):
    """m3_layer_backward over the whole b8 L2048 batch (the configuration bench.py times); the
    oracle recomputes every batch element of one head, which gives that head's per-sequence
    gradients and its batch-summed parameter gradients exactly."""
    w = inputs.WORKLOADS[name]
    print("backward workload", name, "head", head, flush=True)
    inp = inputs.make_prefill_inputs(w, seed=5, device=DEV)
    cot = inputs.make_cotangents(w, seed=6, device=DEV)
    g = m3scan.m3_layer_backward(inp["x"], inp["B"], inp["C"], inp["dt"], inp["theta"], inp["A"],
                                 inp["lam"], cot["dy"], inp["normw_B"], inp["normw_C"], inp["bias_B"],
                                 inp["bias_C"], inp["w_out"] if w.mix else None, bcnorm=w.bcnorm)
    torch.cuda.synchronize()
    hs = slice(head, head + 1)
    pair = {}
    for k, v in inp.items():
        if v is None:
            pair[k] = None
        elif k in SEQ_KEYS:
            pair[k] = v[:, :, hs].cpu()
        else:   # per-head constants
            pair[k] = v[hs].cpu()
    c = {"dy": cot["dy"][:, :, hs].cpu(), "dh_out": None, "dphi_out": None}
    ref = oracle.layer_backward(pair, c["dy"], bcnorm=w.bcnorm, mix=w.mix)
    for k in ("x", "B", "C", "dt", "lam", "h_in"):
        got = g[k][:, :, hs] if k in SEQ_KEYS else g[k][:, hs]
        assert rel_err(got, ref[k]) <= TOL[w.io], k
    for k in ("A", "bias_B", "bias_C", "normw_B", "normw_C") + (("w_out",) if w.mix else ()):
        assert rel_err(g[k][hs], ref[k]) <= TOL[w.io], k
    # dtheta and dphi_in sum cancelling terms: error against the size of the terms summed
    dt = to_np(pair["dt"])[..., None]
    S = ref["theta"] / dt
    nxt = np.concatenate([S[:, 1:], np.zeros_like(S[:, :1])], axis=1)
    A = np.flip(np.cumsum(np.flip(np.abs(S - nxt), 1), 1), 1)
    assert np.abs(to_np(g["theta"][:, :, hs]) - ref["theta"]).max() <= TOL[w.io] * (dt * A).max()
    assert np.abs(to_np(g["phi_in"][:, hs]) - ref["phi_in"]).max() <= TOL[w.io] * A[:, 0].max()
