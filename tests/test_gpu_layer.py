"""GPU parity of m3_layer_prefill (BCNorm, bias and rotation applied while each chunk is staged,
then the chunked scan) against the fp64 oracle's layer core (oracle.layer = bcnorm_rope then
scan), on seeded inputs that span several chunks and end in a ragged tail.  Every call goes
through the C ABI (via the ctypes binding).  Tolerances are those of gpu_util.TOL."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, angle_err, per_head_rel_err, rel_err, to_dev
from state_space_sequence_m3_amd import inputs, m3scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _wl(io, b, L, H, P, N, R, Q, bcnorm=True, bias=True, mix=False, theta_std=1.0):
    return inputs.Workload("case", b, L, H, P, N, R, Q, io, bcnorm, bias, mix, theta_std)


def _run(d, w, chunk, mix, **kw):
    return m3scan.m3_layer_prefill(d["x"], d["B"], d["C"], d["dt"], d["theta"], d["A"], d["lam"],
                                   d.get("normw_B"), d.get("normw_C"), d.get("bias_B"), d.get("bias_C"),
                                   d["w_out"] if mix else None, d.get("phi_in"), d.get("h_in"),
                                   d.get("Bbar_prev"), d.get("x_prev"), chunk=chunk, bcnorm=w.bcnorm,
                                   **kw)


LAYER_CASES = [
    # io, b, L, H, P, N, R, chunk, bcnorm, normw, bias, mix, carry, theta_std
    ("f32", 1, 64, 1, 16, 16, 1, 16, False, False, False, False, False, 1.0),  # tiny SISO fp32
    ("f32", 2, 75, 2, 16, 16, 2, 8, True, True, True, True, True, 1.0),
    ("bf16", 2, 333, 3, 64, 128, 1, 32, True, True, True, False, True, 1.0),
    ("bf16", 2, 200, 3, 64, 128, 1, 16, True, False, True, False, True, 1.0),
    ("bf16", 1, 333, 3, 64, 128, 1, 64, True, True, True, False, True, 1.0),
    ("bf16", 1, 150, 3, 64, 128, 4, 8, True, True, True, True, True, 1.0),
    ("bf16", 1, 150, 2, 64, 128, 4, 16, True, True, True, True, False, 1.0),
    ("bf16", 1, 90, 2, 64, 128, 2, 16, True, False, True, False, True, 1.0),
    ("f32", 1, 70, 2, 64, 64, 1, 32, True, True, True, False, True, 1.0),
    ("bf16", 1, 70, 2, 64, 64, 8, 2, True, True, True, True, True, 1.0),
    ("bf16", 1, 100, 2, 64, 128, 16, 2, True, True, True, True, True, 1.0),
    ("bf16", 1, 257, 2, 64, 128, 1, 32, True, True, True, False, True, math.pi),
    ("bf16", 2, 129, 2, 64, 128, 1, 32, False, False, False, False, False, 1.0),
    ("f32", 1, 45, 2, 64, 128, 4, 8, True, True, True, True, True, 1.0),
    ("bf16", 1, 70, 2, 64, 128, 8, 8, True, True, True, True, True, 1.0),    # 64 rows, R = 8
]


@pytest.mark.parametrize("case", LAYER_CASES,
                         ids=lambda c: "%s-b%d-L%d-H%d-P%d-N%d-R%d-Q%d" % c[:8])
def test_layer_parity(case):
    io, b, L, H, P, N, R, Q, bcnorm, normw, bias, mix, carry, tstd = case
    w = _wl(io, b, L, H, P, N, R, Q, bcnorm, bias, mix, tstd)
    inp = inputs.make_prefill_inputs(w, seed=31, normw=normw, carry=carry)
    d = to_dev(inp, DEV)
    Blast = torch.empty((b, H, R, N), dtype=w.torch_io, device=DEV)
    xlast = torch.empty((b, H, R, P), dtype=w.torch_io, device=DEV)
    y, h, phi = _run(d, w, Q, mix, Bbar_last=Blast, x_last=xlast)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=bcnorm, mix=mix)
    tol = TOL[io]
    assert rel_err(y, ref["y"]) <= tol
    ph = per_head_rel_err(y, ref["y"], 2 if mix else 3)
    assert ph <= tol, ph
    assert rel_err(h, ref["h_out"]) <= tol
    assert angle_err(phi, ref["phi_out"]) <= (1e-3 if io == "bf16" else 1e-4)
    assert rel_err(Blast, ref["Bbar_last"]) <= tol
    assert rel_err(xlast, ref["x_last"]) == 0.0


def test_layer_default_chunk():
    w = _wl("bf16", 1, 100, 2, 64, 128, 4, 0, mix=True)
    inp = inputs.make_prefill_inputs(w, seed=32, carry=True)
    d = to_dev(inp, DEV)
    y, h, phi = _run(d, w, 0, True)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=True)
    assert rel_err(y, ref["y"]) <= TOL["bf16"]
    assert rel_err(h, ref["h_out"]) <= TOL["bf16"]


def test_layer_split_carry():
    """layer(0..t1) then layer(t1..L) with every carry passed on equals the oracle over 0..L."""
    w = _wl("bf16", 2, 300, 2, 64, 128, 2, 16, mix=True)
    inp = inputs.make_prefill_inputs(w, seed=33, normw=True, carry=True)
    d = to_dev(inp, DEV)
    t1 = 113
    first = {k: (v[:, :t1] if k in ("x", "B", "C", "dt", "lam", "theta") else v) for k, v in d.items()}
    second = {k: (v[:, t1:] if k in ("x", "B", "C", "dt", "lam", "theta") else v) for k, v in d.items()}
    b, H, R, N, P = 2, 2, 2, 128, 64
    Blast = torch.empty((b, H, R, N), dtype=torch.bfloat16, device=DEV)
    xlast = torch.empty((b, H, R, P), dtype=torch.bfloat16, device=DEV)
    y1, h1, phi1 = _run({k: v.contiguous() for k, v in first.items()}, w, 16, True,
                        Bbar_last=Blast, x_last=xlast)
    second = {k: v.contiguous() for k, v in second.items()}
    second.update(h_in=h1, phi_in=phi1, Bbar_prev=Blast, x_prev=xlast)
    y2, h2, phi2 = _run(second, w, 16, True)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=True)
    y = torch.cat([y1, y2], dim=1)
    assert rel_err(y, ref["y"]) <= TOL["bf16"]
    assert rel_err(h2, ref["h_out"]) <= TOL["bf16"]
    assert angle_err(phi2, ref["phi_out"]) <= 1e-3


def test_layer_in_place_state_and_angle():
    w = _wl("bf16", 1, 97, 2, 64, 128, 1, 32)
    inp = inputs.make_prefill_inputs(w, seed=34, carry=True)
    d = to_dev(inp, DEV)
    h = d["h_in"].clone()
    phi = d["phi_in"].clone()
    d2 = dict(d, h_in=h, phi_in=phi)
    _run(d2, w, 32, False, h_out=h, phi_out=phi)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=False)
    assert rel_err(h, ref["h_out"]) <= TOL["bf16"]
    assert angle_err(phi, ref["phi_out"]) <= 1e-3


def test_layer_empty_sequence_passes_the_carry_through():
    w = _wl("bf16", 2, 0, 2, 64, 128, 1, 32)
    inp = inputs.make_prefill_inputs(w, seed=35, carry=True)
    d = to_dev(inp, DEV)
    Blast = torch.full_like(d["Bbar_prev"], 7.0)
    xlast = torch.full_like(d["x_prev"], 7.0)
    y, h, phi = _run(d, w, 32, False, Bbar_last=Blast, x_last=xlast)
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(h, d["h_in"])
    assert torch.equal(Blast, d["Bbar_prev"])
    assert torch.equal(xlast, d["x_prev"])
    assert angle_err(phi, inp["phi_in"].double().numpy()) <= 1e-6


def test_layer_unsupported_chunk_is_rejected():
    w = _wl("bf16", 1, 48, 1, 64, 128, 1, 48)
    d = to_dev(inputs.make_prefill_inputs(w, seed=36), DEV)
    with pytest.raises(m3scan.M3Error) as e:
        _run(d, w, 48, False)
    assert e.value.status == m3scan.M3_E_UNSUPPORTED
    w = _wl("bf16", 1, 48, 1, 32, 128, 1, 32)      # no kernel for P = 32
    d = to_dev(inputs.make_prefill_inputs(w, seed=36), DEV)
    with pytest.raises(m3scan.M3Error) as e:
        _run(d, w, 32, False)
    assert e.value.status == m3scan.M3_E_UNSUPPORTED


# ---------------------------------------------------------------------------------------------
# m3_layer_decode_step: rotation + decode in one launch
# ---------------------------------------------------------------------------------------------
def _fused_decode_run(w, steps, seed, mix, normw):
    dinp = inputs.make_decode_inputs(w, seed, steps, normw=normw)
    d = to_dev({k: v for k, v in dinp.items() if k not in ("tokens", "state")}, DEV)
    toks = to_dev(dinp["tokens"], DEV)
    st = to_dev(dinp["state"], DEV)
    h, phi = st["h"].clone(), st["phi"].clone()
    Bprev, xprev = st["Bbar_prev"].clone(), st["x_prev"].clone()
    Bcur = torch.empty_like(Bprev)
    ys = []
    for s in range(steps):
        x = toks["x"][s]
        y, _ = m3scan.m3_layer_decode_step(h, phi, Bprev, xprev, x, toks["B"][s], toks["C"][s],
                                           toks["dt"][s], toks["theta"][s], d["A"], toks["lam"][s],
                                           d.get("normw_B"), d.get("normw_C"), d["bias_B"], d["bias_C"],
                                           d["w_out"] if mix else None, Bbar_out=Bcur)
        ys.append(y)
        Bprev, Bcur = Bcur, Bprev
        xprev = x
    torch.cuda.synchronize()
    consts = {k: dinp.get(k) for k in ("A", "bias_B", "bias_C", "w_out", "normw_B", "normw_C")}
    state = dict(dinp["state"])
    rys = []
    for s in range(steps):
        tok = {k: dinp["tokens"][k][s] for k in ("x", "B", "C", "dt", "lam", "theta")}
        ry, state = oracle.decode_step(state, tok, consts, mix=mix)
        rys.append(ry)
    return ys, h, phi, Bprev, rys, state


@pytest.mark.parametrize("R,io,normw", [(1, "bf16", False), (4, "bf16", True), (2, "f32", True),
                                        (8, "bf16", False)])
def test_layer_decode_parity(R, io, normw):
    base = inputs.WORKLOADS["decode_b128_r4" if R > 1 else "decode_b128_r1"]
    w = base.with_(batch=3, nheads=5, rank=R, io=io)
    ys, h, phi, Blast, rys, state = _fused_decode_run(w, 12, seed=51 + R, mix=w.mix, normw=normw)
    assert rel_err(torch.stack(ys, 0), np.stack(rys, 0)) <= TOL[io]
    assert rel_err(h, state["h"]) <= TOL[io]
    assert angle_err(phi, state["phi"]) <= (1e-4 if io == "f32" else 1e-3)
    assert rel_err(Blast, state["Bbar_prev"]) <= TOL[io]


@pytest.mark.parametrize("R,io,dstate", [(1, "bf16", 128), (4, "bf16", 128), (2, "f32", 64)])
def test_layer_decode_many_pairs_per_workgroup(R, io, dstate):
    """More (batch, head) pairs than the GPU holds decode workgroups at once, with an odd head
    count: the grid is then a multiple of H below the pair count and every workgroup serves
    several pairs of one head in turn, loading the next pair while it updates the current one."""
    base = inputs.WORKLOADS["decode_b128_r4" if R > 1 else "decode_b128_r1"]
    w = base.with_(batch=300, nheads=7, rank=R, io=io, dstate=dstate)
    ys, h, phi, Blast, rys, state = _fused_decode_run(w, 3, seed=61 + R, mix=w.mix, normw=True)
    assert rel_err(torch.stack(ys, 0), np.stack(rys, 0)) <= TOL[io]
    assert rel_err(h, state["h"]) <= TOL[io]
    assert angle_err(phi, state["phi"]) <= (1e-4 if io == "f32" else 1e-3)
    assert rel_err(Blast, state["Bbar_prev"]) <= TOL[io]


def test_layer_prefill_then_layer_decode_continue_the_sequence():
    """m3_layer_prefill over 0..L-k then k m3_layer_decode_step calls equal the oracle's layer
    core over 0..L, token by token."""
    w = _wl("bf16", 2, 150, 3, 64, 128, 4, 8, mix=True)
    inp = inputs.make_prefill_inputs(w, seed=52, normw=True)
    d = to_dev(inp, DEV)
    k = 6
    L0 = w.seqlen - k
    head = {kk: (v[:, :L0].contiguous() if kk in ("x", "B", "C", "dt", "lam", "theta") else v)
            for kk, v in d.items()}
    Blast = torch.empty((2, 3, 4, 128), dtype=torch.bfloat16, device=DEV)
    xlast = torch.empty((2, 3, 4, 64), dtype=torch.bfloat16, device=DEV)
    y0, h, phi = _run(head, w, 8, True, Bbar_last=Blast, x_last=xlast)
    Bprev, xprev, Bcur = Blast, xlast, torch.empty_like(Blast)
    ys = [y0]
    for t in range(L0, w.seqlen):
        x = d["x"][:, t].contiguous()
        y, _ = m3scan.m3_layer_decode_step(h, phi, Bprev, xprev, x, d["B"][:, t].contiguous(),
                                           d["C"][:, t].contiguous(), d["dt"][:, t].contiguous(),
                                           d["theta"][:, t].contiguous(), d["A"], d["lam"][:, t].contiguous(),
                                           d["normw_B"], d["normw_C"], d["bias_B"], d["bias_C"], d["w_out"],
                                           Bbar_out=Bcur)
        ys.append(y.unsqueeze(1))
        Bprev, Bcur = Bcur, Bprev
        xprev = x
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=True)
    assert rel_err(torch.cat(ys, 1), ref["y"]) <= TOL["bf16"]
    assert rel_err(h, ref["h_out"]) <= TOL["bf16"]
    assert angle_err(phi, ref["phi_out"]) <= 1e-3


def test_layer_decode_rejects_aliased_rotated_b():
    w = inputs.WORKLOADS["decode_b128_r1"].with_(batch=1, nheads=2)
    dinp = inputs.make_decode_inputs(w, 53, 1, device=DEV)
    st, tk = dinp["state"], dinp["tokens"]
    with pytest.raises(m3scan.M3Error) as e:
        m3scan.m3_layer_decode_step(st["h"], st["phi"], st["Bbar_prev"], st["x_prev"], tk["x"][0], tk["B"][0],
                                    tk["C"][0], tk["dt"][0], tk["theta"][0], dinp["A"], tk["lam"][0],
                                    Bbar_out=st["Bbar_prev"])
    assert e.value.status == m3scan.M3_E_ALIAS


# ---------------------------------------------------------------------------------------------
# Mamba-2 mode (lambda = 1, theta = 0, no BCNorm or bias) on the same kernels
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("N,R,chunk", [(128, 1, 64), (128, 1, 32), (64, 1, 32), (128, 4, 8)])
def test_mamba2_mode_parity(N, R, chunk):
    w = inputs.Workload("m2", 2, 150, 3, 64, N, R, chunk, "bf16", False, False, R > 1, mamba2=True)
    inp = inputs.make_prefill_inputs(w, seed=61, carry=True)
    d = to_dev(inp, DEV)
    ref = oracle.layer(inp, bcnorm=False, mix=w.mix)
    # fused call, with a carried-in state and angle (theta = 0 keeps the angle where it was)
    y, h, phi = _run(d, w, chunk, w.mix)
    # the plain scan straight on the raw B and C: with theta = 0, no BCNorm and no bias they are
    # Bbar and Cbar (up to the carried angle, so this call starts from zero)
    y2, h2 = m3scan.m3_prefill(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"],
                               d["w_out"] if w.mix else None, chunk=chunk)
    torch.cuda.synchronize()
    assert rel_err(y, ref["y"]) <= TOL["bf16"]
    assert rel_err(h, ref["h_out"]) <= TOL["bf16"]
    assert angle_err(phi, ref["phi_out"]) <= 1e-3
    ref2 = oracle.layer({k: v for k, v in inp.items() if k not in ("h_in", "phi_in", "Bbar_prev", "x_prev")},
                        bcnorm=False, mix=w.mix)
    assert rel_err(y2, ref2["y"]) <= TOL["bf16"]
    assert rel_err(h2, ref2["h_out"]) <= TOL["bf16"]


# ---------------------------------------------------------------------------------------------
# decode captured in a HIP graph (small-batch serving: launches, not bytes, bound the step)
# ---------------------------------------------------------------------------------------------
def test_layer_decode_graph_replays_match_eager():
    """K fused decode steps captured once and replayed three times, with eager work and
    synchronisation between replays, give exactly the eager steps' y, state, angle and rotated
    B every time (and the eager steps match the oracle)."""
    K = 8
    w = inputs.WORKLOADS["decode_b128_r4"].with_(batch=1, nheads=8)
    dinp = inputs.make_decode_inputs(w, 71, K, device=DEV)
    toks, st = dinp["tokens"], dinp["state"]
    b, H, R, N, P = w.batch, w.nheads, w.rank, w.dstate, w.headdim
    bufs = [torch.empty_like(st["Bbar_prev"]) for _ in range(2)]
    ys = torch.empty((K, b, H, P), dtype=torch.bfloat16, device=DEV)
    h = torch.empty_like(st["h"])
    phi = torch.empty_like(st["phi"])
    x0 = st["x_prev"].clone()

    def reset():
        h.copy_(st["h"])
        phi.copy_(st["phi"])
        bufs[0].copy_(st["Bbar_prev"])

    def steps():
        xprev = x0
        for s in range(K):
            m3scan.m3_layer_decode_step(h, phi, bufs[s % 2], xprev, toks["x"][s], toks["B"][s], toks["C"][s],
                                        toks["dt"][s], toks["theta"][s], dinp["A"], toks["lam"][s], None, None,
                                        dinp["bias_B"], dinp["bias_C"], dinp["w_out"], y=ys[s],
                                        Bbar_out=bufs[(s + 1) % 2])
            xprev = toks["x"][s]

    reset()
    steps()
    torch.cuda.synchronize()
    eager = [ys.clone(), h.clone(), phi.clone(), bufs[K % 2].clone()]
    # oracle on the eager run
    consts = {k: dinp.get(k) for k in ("A", "bias_B", "bias_C", "w_out")}
    state = {k: v.cpu() for k, v in st.items()}
    rys = []
    for s in range(K):
        tok = {k: toks[k][s].cpu() for k in ("x", "B", "C", "dt", "lam", "theta")}
        ry, state = oracle.decode_step(state, tok, {k: (v.cpu() if v is not None else None)
                                                    for k, v in consts.items()}, mix=True)
        rys.append(ry)
    assert rel_err(eager[0], np.stack(rys, 0)) <= TOL["bf16"]
    assert rel_err(eager[1], state["h"]) <= TOL["bf16"]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # one warm run on the capture stream
        reset()
        steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        steps()
    for rep in range(3):
        ys.fill_(float("nan"))
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, eager[0]), rep
        assert torch.equal(h, eager[1]), rep
        assert torch.equal(phi, eager[2]), rep
        assert torch.equal(bufs[K % 2], eager[3]), rep


# ---------------------------------------------------------------------------------------------
# packed variable-length batch (serving: prompts of mixed lengths, no padding)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("R,chunk,io", [(1, 32, "bf16"), (4, 8, "bf16"), (2, 8, "f32")])
def test_layer_prefill_varlen_matches_each_sequence(R, chunk, io):
    lens = [100, 1, 0, 257, 33]
    T = sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    nseq, H, P, N = len(lens), 3, 64, 128
    w = _wl(io, 1, T, H, P, N, R, chunk, mix=R > 1)
    inp = inputs.make_prefill_inputs(w, seed=81, normw=True)
    # per-sequence carries drawn like the decode state
    carry = inputs.make_decode_state(w.with_(batch=nseq), inputs._gen(82, "cpu"), "cpu")
    d = to_dev(inp, DEV)
    dc = to_dev(carry, DEV)
    packed = {k: d[k][0] for k in ("x", "B", "C", "dt", "lam", "theta")}
    Blast = torch.full((nseq, H, R, N), 7.0, dtype=w.torch_io, device=DEV)
    xlast = torch.full((nseq, H, R, P), 7.0, dtype=w.torch_io, device=DEV)
    y, h, phi = m3scan.m3_layer_prefill_varlen(
        cu, packed["x"], packed["B"], packed["C"], packed["dt"], packed["theta"], d["A"], packed["lam"],
        d["normw_B"], d["normw_C"], d["bias_B"], d["bias_C"], d["w_out"] if w.mix else None,
        phi_in=dc["phi"], h_in=dc["h"], Bbar_prev=dc["Bbar_prev"], x_prev=dc["x_prev"],
        Bbar_last=Blast, x_last=xlast, chunk=chunk)
    torch.cuda.synchronize()
    off = 0
    for s, n in enumerate(lens):
        if n == 0:   # the carry passes through
            assert torch.equal(h[s], dc["h"][s])
            assert torch.equal(Blast[s], dc["Bbar_prev"][s])
            assert torch.equal(xlast[s], dc["x_prev"][s])
            assert angle_err(phi[s], carry["phi"][s].double().numpy()) <= 1e-6
            continue
        seq = {k: inp[k][:, off:off + n] for k in ("x", "B", "C", "dt", "lam", "theta")}
        seq.update({k: inp[k] for k in ("A", "bias_B", "bias_C", "w_out", "normw_B", "normw_C")})
        seq.update(h_in=carry["h"][s:s + 1], phi_in=carry["phi"][s:s + 1],
                   Bbar_prev=carry["Bbar_prev"][s:s + 1], x_prev=carry["x_prev"][s:s + 1])
        ref = oracle.layer(seq, bcnorm=True, mix=w.mix)
        assert rel_err(y[off:off + n].unsqueeze(0), ref["y"]) <= TOL[io], s
        assert rel_err(h[s:s + 1], ref["h_out"]) <= TOL[io], s
        assert angle_err(phi[s:s + 1], ref["phi_out"]) <= (1e-3 if io == "bf16" else 1e-4), s
        assert rel_err(Blast[s:s + 1], ref["Bbar_last"]) <= TOL[io], s
        assert rel_err(xlast[s:s + 1], ref["x_last"]) == 0.0, s
        off += n
