"""GPU parity of head groups: raw B and C in G < H head slots, slot s shared by the H / G
consecutive heads s H/G .. (s+1) H/G - 1, in every call that takes raw B and C
(m3_bcnorm_rope, m3_layer_prefill with and without the sequence split, m3_layer_prefill_varlen,
m3_layer_decode_step, m3_layer_chunk_states + m3_layer_backward).

The oracle defines the grouped layout as its expansion (each head reads its slot's rows) and the
gradient of a shared row as the sum over the heads that read it (oracle.heads_from_groups /
groups_from_heads, pinned by one-head calls and central differences in pins.check_head_groups).
Every call goes through the C ABI; tolerances are gpu_util.TOL, normwise per tensor.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, angle_err, rel_err, to_dev, to_np
from state_space_sequence_m3_amd import inputs, m3scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _wl(io, b, L, H, G, P, N, R, Q, mix=False, bcnorm=True, bias=True):
    return inputs.Workload("groups", b, L, H, P, N, R, Q, io, bcnorm, bias, mix, groups=G)


def _ang_tol(io):
    return 1e-3 if io == "bf16" else 1e-4


LAYER_CASES = [
    # io, b, L, H, G, P, N, R, chunk, mix, carry
    ("bf16", 2, 333, 4, 2, 64, 128, 1, 32, False, True),    # two groups of two, ragged tail
    ("bf16", 1, 200, 4, 1, 64, 128, 4, 8, True, True),      # every head shares one slot, MIMO
    ("bf16", 2, 150, 8, 2, 64, 64, 2, 16, True, False),     # N = 64, groups of four
    ("f32", 2, 75, 4, 2, 16, 16, 2, 8, True, True),         # fp32
    ("bf16", 1, 130, 6, 3, 64, 128, 1, 64, False, True),    # odd group count, 64-row chunks
]


def _ids(c):
    return "%s-b%d-L%d-H%d-G%d-P%d-N%d-R%d-Q%d" % c[:9]


def _layer(d, w, chunk, mix, **kw):
    return m3scan.m3_layer_prefill(d["x"], d["B"], d["C"], d["dt"], d["theta"], d["A"], d["lam"],
                                   d.get("normw_B"), d.get("normw_C"), d.get("bias_B"), d.get("bias_C"),
                                   d["w_out"] if mix else None, d.get("phi_in"), d.get("h_in"),
                                   d.get("Bbar_prev"), d.get("x_prev"), chunk=chunk, **kw)


@pytest.mark.parametrize("case", LAYER_CASES, ids=_ids)
def test_grouped_layer_prefill(case):
    io, b, L, H, G, P, N, R, Q, mix, carry = case
    print("grouped layer", _ids(case), flush=True)
    w = _wl(io, b, L, H, G, P, N, R, Q, mix)
    inp = inputs.make_prefill_inputs(w, seed=91, normw=True, carry=carry)
    assert tuple(inp["B"].shape) == (b, L, G, R, N)
    d = to_dev(inp, DEV)
    Blast = torch.empty((b, H, R, N), dtype=w.torch_io, device=DEV)
    xlast = torch.empty((b, H, R, P), dtype=w.torch_io, device=DEV)
    y, h, phi = _layer(d, w, Q, mix, Bbar_last=Blast, x_last=xlast)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=mix)
    tol = TOL[io]
    assert rel_err(y, ref["y"]) <= tol
    assert rel_err(h, ref["h_out"]) <= tol
    assert angle_err(phi, ref["phi_out"]) <= _ang_tol(io)
    assert rel_err(Blast, ref["Bbar_last"]) <= tol
    assert rel_err(xlast, ref["x_last"]) == 0.0


@pytest.mark.parametrize("case", LAYER_CASES[:4], ids=_ids)
def test_grouped_bcnorm_rope_then_prefill(case):
    """The two-call path: m3_bcnorm_rope reads the grouped raw rows and writes per-head Bbar and
    Cbar, which m3_prefill (per head only) scans."""
    io, b, L, H, G, P, N, R, Q, mix, carry = case
    w = _wl(io, b, L, H, G, P, N, R, Q, mix)
    inp = inputs.make_prefill_inputs(w, seed=92, normw=True, carry=carry)
    d = to_dev(inp, DEV)
    Bb, Cb, phi = m3scan.m3_bcnorm_rope(d["B"], d["C"], d["dt"], d["theta"], d.get("normw_B"),
                                        d.get("normw_C"), d.get("bias_B"), d.get("bias_C"), d.get("phi_in"))
    y, h = m3scan.m3_prefill(d["x"], Bb, Cb, d["dt"], d["A"], d["lam"], d["w_out"] if mix else None,
                             d.get("h_in"), d.get("Bbar_prev"), d.get("x_prev"), chunk=Q)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=mix)
    tol = TOL[io]
    assert tuple(Bb.shape) == (b, L, H, R, N)
    assert rel_err(Bb, ref["Bbar"]) <= tol
    assert rel_err(Cb, ref["Cbar"]) <= tol
    assert angle_err(phi, ref["phi_out"]) <= _ang_tol(io)
    assert rel_err(y, ref["y"]) <= tol
    assert rel_err(h, ref["h_out"]) <= tol


@pytest.mark.parametrize("io,b,L,H,G,R,Q,mix", [("bf16", 1, 3000, 2, 1, 1, 32, False),
                                                 ("bf16", 1, 5000, 4, 2, 4, 8, True),
                                                 ("f32", 1, 4100, 2, 1, 2, 8, True)])
def test_grouped_split_layer_prefill(io, b, L, H, G, R, Q, mix):
    """Few (b, h) pairs and long sequences: the sequence split (two passes and the chaining
    kernel) with grouped raw rows."""
    P, N = (16, 16) if io == "f32" else (64, 128)
    w = _wl(io, b, L, H, G, P, N, R, Q, mix)
    dims = m3scan.make_dims(b, L, H, P, N, R, Q, m3scan.M3_BF16 if io == "bf16" else m3scan.M3_F32,
                            groups=G)
    assert m3scan.layer_prefill_workspace_bytes(dims) > 0, "the split is not used"
    inp = inputs.make_prefill_inputs(w, seed=94, normw=True, carry=True)
    d = to_dev(inp, DEV)
    Blast = torch.empty((b, H, R, N), dtype=w.torch_io, device=DEV)
    y, h, phi = _layer(d, w, Q, mix, Bbar_last=Blast)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=mix)
    tol = TOL[io]
    assert rel_err(y, ref["y"]) <= tol
    assert rel_err(h, ref["h_out"]) <= tol
    assert angle_err(phi, ref["phi_out"]) <= _ang_tol(io)
    assert rel_err(Blast, ref["Bbar_last"]) <= tol


def test_grouped_layer_prefill_varlen():
    lens = [100, 1, 0, 257, 33]
    T = sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    nseq, H, G, P, N, R, Q = len(lens), 4, 2, 64, 128, 2, 16
    w = _wl("bf16", 1, T, H, G, P, N, R, Q, mix=True)
    inp = inputs.make_prefill_inputs(w, seed=95, normw=True)
    carry = inputs.make_decode_state(w.with_(batch=nseq), inputs._gen(96, "cpu"), "cpu")
    d = to_dev(inp, DEV)
    dc = to_dev(carry, DEV)
    packed = {k: d[k][0] for k in ("x", "B", "C", "dt", "lam", "theta")}
    y, h, phi = m3scan.m3_layer_prefill_varlen(
        cu, packed["x"], packed["B"], packed["C"], packed["dt"], packed["theta"], d["A"], packed["lam"],
        d["normw_B"], d["normw_C"], d["bias_B"], d["bias_C"], d["w_out"], phi_in=dc["phi"], h_in=dc["h"],
        Bbar_prev=dc["Bbar_prev"], x_prev=dc["x_prev"], chunk=Q)
    torch.cuda.synchronize()
    off = 0
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(h[s], dc["h"][s])
            continue
        seq = {k: inp[k][:, off:off + n] for k in ("x", "B", "C", "dt", "lam", "theta")}
        seq.update({k: inp[k] for k in ("A", "bias_B", "bias_C", "w_out", "normw_B", "normw_C")})
        seq.update(h_in=carry["h"][s:s + 1], phi_in=carry["phi"][s:s + 1],
                   Bbar_prev=carry["Bbar_prev"][s:s + 1], x_prev=carry["x_prev"][s:s + 1])
        ref = oracle.layer(seq, bcnorm=True, mix=True)
        assert rel_err(y[off:off + n].unsqueeze(0), ref["y"]) <= TOL["bf16"], s
        assert rel_err(h[s:s + 1], ref["h_out"]) <= TOL["bf16"], s
        assert angle_err(phi[s:s + 1], ref["phi_out"]) <= 1e-3, s
        off += n


@pytest.mark.parametrize("R,io,b,H,G", [(1, "bf16", 3, 4, 2), (4, "bf16", 3, 8, 1), (2, "f32", 2, 4, 2),
                                        (4, "bf16", 300, 8, 2)])
def test_grouped_layer_decode(R, io, b, H, G):
    """m3_layer_decode_step with grouped raw rows, several steps in a row (the last case holds
    more pairs than the GPU runs decode workgroups at once)."""
    base = inputs.WORKLOADS["decode_b128_r4" if R > 1 else "decode_b128_r1"]
    w = base.with_(batch=b, nheads=H, rank=R, io=io, groups=G)
    steps = 6 if b < 100 else 2
    dinp = inputs.make_decode_inputs(w, 97, steps, normw=True)
    d = to_dev({k: v for k, v in dinp.items() if k not in ("tokens", "state")}, DEV)
    toks = to_dev(dinp["tokens"], DEV)
    st = to_dev(dinp["state"], DEV)
    assert tuple(toks["B"].shape[1:]) == (b, G, R, w.dstate)
    h, phi = st["h"].clone(), st["phi"].clone()
    Bprev, xprev = st["Bbar_prev"].clone(), st["x_prev"].clone()
    Bcur = torch.empty_like(Bprev)
    ys = []
    for s in range(steps):
        x = toks["x"][s]
        y, _ = m3scan.m3_layer_decode_step(h, phi, Bprev, xprev, x, toks["B"][s], toks["C"][s],
                                           toks["dt"][s], toks["theta"][s], d["A"], toks["lam"][s],
                                           d["normw_B"], d["normw_C"], d["bias_B"], d["bias_C"],
                                           d["w_out"] if w.mix else None, Bbar_out=Bcur)
        ys.append(y)
        Bprev, Bcur = Bcur, Bprev
        xprev = x
    torch.cuda.synchronize()
    consts = {k: dinp.get(k) for k in ("A", "bias_B", "bias_C", "w_out", "normw_B", "normw_C")}
    state = dict(dinp["state"])
    rys = []
    for s in range(steps):
        tok = {k: dinp["tokens"][k][s] for k in ("x", "B", "C", "dt", "lam", "theta")}
        ry, state = oracle.decode_step(state, tok, consts, mix=w.mix)
        rys.append(ry)
    assert rel_err(torch.stack(ys, 0), np.stack(rys, 0)) <= TOL[io]
    assert rel_err(h, state["h"]) <= TOL[io]
    assert angle_err(phi, state["phi"]) <= _ang_tol(io)
    assert rel_err(Bprev, state["Bbar_prev"]) <= TOL[io]


BWD_CASES = [
    # io, b, L, H, G, P, N, R, mix
    ("bf16", 2, 333, 4, 2, 64, 128, 1, False),
    ("bf16", 1, 150, 4, 1, 64, 128, 4, True),
    ("f32", 2, 75, 4, 2, 16, 16, 2, True),
    ("bf16", 1, 200, 6, 3, 64, 64, 1, False),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "%s-b%d-L%d-H%d-G%d-P%d-N%d-R%d" % c[:8])
def test_grouped_backward(case):
    io, b, L, H, G, P, N, R, mix = case
    print("grouped backward", case, flush=True)
    w = _wl(io, b, L, H, G, P, N, R, 0, mix)
    inp = inputs.make_prefill_inputs(w, seed=98, normw=True, carry=True)
    cot = inputs.make_cotangents(w, seed=99)
    d, c = to_dev(inp, DEV), to_dev(cot, DEV)
    grads = m3scan.m3_layer_backward(d["x"], d["B"], d["C"], d["dt"], d["theta"], d["A"], d["lam"], c["dy"],
                                     d["normw_B"], d["normw_C"], d["bias_B"], d["bias_C"],
                                     d["w_out"] if mix else None, d["phi_in"], d["h_in"], d["Bbar_prev"],
                                     d["x_prev"], c["dh_out"], c["dphi_out"])
    torch.cuda.synchronize()
    ref = oracle.layer_backward(inp, cot["dy"], cot["dh_out"], cot["dphi_out"], mix=mix)
    assert tuple(grads["B"].shape) == (b, L, G, R, N)
    tol = TOL[io]
    errs = {k: rel_err(grads[k], ref[k]) for k in ("x", "B", "C", "dt", "lam", "A", "normw_B", "normw_C",
                                                     "bias_B", "bias_C", "h_in", "Bbar_prev", "x_prev")}
    if mix:
        errs["w_out"] = rel_err(grads["w_out"], ref["w_out"])
    print("normwise", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


@pytest.mark.parametrize("name,pairs", [("siso_g1_b8_l2048", [(0, 0), (7, 63)]),
                                        ("mimo4_g1_b8_l2048", [(0, 5), (6, 40)]),
                                        ("mimo4_g8_b8_l2048", [(3, 9), (5, 62)])])
def test_grouped_workload_sampled(name, pairs):
    """Full sizes, in the launch configuration bench.py times (m3_layer_prefill, chunk * R = 32):
    sampled (batch, head) pairs recomputed by the oracle from the pair's inputs and its slot's
    raw rows."""
    w = inputs.WORKLOADS[name]
    print("workload", name, flush=True)
    inp = inputs.make_prefill_inputs(w, seed=1, device=DEV)
    y, h, phi = m3scan.m3_layer_prefill(inp["x"], inp["B"], inp["C"], inp["dt"], inp["theta"], inp["A"],
                                        inp["lam"], inp["normw_B"], inp["normw_C"], inp["bias_B"],
                                        inp["bias_C"], inp["w_out"] if w.mix else None, chunk=32 // w.rank)
    torch.cuda.synchronize()
    H, G = w.nheads, w.bc_heads
    for bi, hi in pairs:
        slot = hi * G // H
        one = {}
        for k, v in inp.items():
            if v is None:
                one[k] = None
            elif k in ("B", "C"):
                one[k] = v[bi:bi + 1, :, slot:slot + 1].cpu()
            elif k in ("x", "dt", "lam", "theta"):
                one[k] = v[bi:bi + 1, :, hi:hi + 1].cpu()
            else:   # per-head constants
                one[k] = v[hi:hi + 1].cpu()
        ref = oracle.layer(one, bcnorm=w.bcnorm, mix=w.mix)
        ys = y[bi:bi + 1, :, hi:hi + 1]
        assert rel_err(ys, ref["y"]) <= TOL[w.io], (bi, hi)
        assert rel_err(h[bi:bi + 1, hi:hi + 1], ref["h_out"]) <= TOL[w.io], (bi, hi)
        assert angle_err(phi[bi:bi + 1, hi:hi + 1], ref["phi_out"]) <= 1e-3, (bi, hi)
