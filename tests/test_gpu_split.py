"""GPU parity of the sequence split of m3_prefill and m3_layer_prefill: with few (b, h) pairs and
long sequences, and a workspace, each sequence runs as segments in parallel: pass 1 (every
segment, y included, the later ones from zero carries), a chaining kernel, pass 2 (each later
segment's first steps again from its true carry, until the carry's share of y has decayed by
2^-48).  Checked against the fp64 oracle's
layer core over the whole sequence, with carries in, ragged last segments and 2-4 segments (so
that the chaining runs); the same call run in one pass is checked against the oracle too.
Every call goes through the C ABI (via the ctypes binding).  Tolerances are those of
gpu_util.TOL."""
from __future__ import annotations

import pytest
import torch

import oracle
from gpu_util import TOL, angle_err, rel_err, to_dev
from state_space_sequence_m3_amd import inputs, m3scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

SPLIT_CASES = [
    # io, b, L, H, P, N, R, chunk (fused), chunk (m3_prefill), mix, carry
    ("bf16", 1, 3000, 2, 64, 128, 1, 32, 64, False, True),   # 2 segments, ragged tail
    ("bf16", 1, 5000, 2, 64, 128, 4, 8, 16, True, True),     # 4 segments: chaining runs twice
    ("f32", 1, 4100, 1, 16, 16, 2, 8, 16, True, True),       # 3 segments, fp32
    ("bf16", 1, 4096, 2, 64, 64, 1, 32, 32, False, False),   # N = 64, segments of 1024
    ("bf16", 2, 3500, 1, 64, 128, 2, 8, 32, True, True),     # b = 2, 16-row fused chunks
    ("bf16", 3, 2100, 1, 64, 128, 1, 16, 16, False, True),   # b = 3, chunk 16 in both calls
    ("bf16", 1, 12288, 1, 64, 128, 1, 32, 64, False, True),  # 12 segments: the chaining runs
                                                              # two blocks of segments
    ("bf16", 1, 3000, 2, 64, 64, 8, 4, 8, True, True),       # R = 8: 4- and 8-step chunks
]


def _wl(io, b, L, H, P, N, R, Q, mix):
    return inputs.Workload("split", b, L, H, P, N, R, Q, io, True, True, mix, 1.0)


def _layer(d, w, chunk, mix, **kw):
    return m3scan.m3_layer_prefill(d["x"], d["B"], d["C"], d["dt"], d["theta"], d["A"], d["lam"],
                                   d.get("normw_B"), d.get("normw_C"), d.get("bias_B"), d.get("bias_C"),
                                   d["w_out"] if mix else None, d.get("phi_in"), d.get("h_in"),
                                   d.get("Bbar_prev"), d.get("x_prev"), chunk=chunk, **kw)


def _dims(w, chunk):
    return m3scan.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, chunk,
                            m3scan.M3_BF16 if w.io == "bf16" else m3scan.M3_F32)


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "%s-b%d-L%d-H%d-P%d-N%d-R%d" % c[:7])
def test_split_layer_prefill(case):
    io, b, L, H, P, N, R, Qf, Qp, mix, carry = case
    w = _wl(io, b, L, H, P, N, R, Qf, mix)
    assert m3scan.layer_prefill_workspace_bytes(_dims(w, Qf)) > 0, "the split is not used"
    inp = inputs.make_prefill_inputs(w, seed=81, normw=True, carry=carry)
    d = to_dev(inp, DEV)
    Blast = torch.empty((b, H, R, N), dtype=w.torch_io, device=DEV)
    xlast = torch.empty((b, H, R, P), dtype=w.torch_io, device=DEV)
    y, h, phi = _layer(d, w, Qf, mix, Bbar_last=Blast, x_last=xlast)
    y1, h1, phi1 = _layer(d, w, Qf, mix, workspace=False)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=mix)
    tol = TOL[io]
    assert rel_err(y, ref["y"]) <= tol
    assert rel_err(h, ref["h_out"]) <= tol
    assert angle_err(phi, ref["phi_out"]) <= (1e-3 if io == "bf16" else 1e-4)
    assert rel_err(Blast, ref["Bbar_last"]) <= tol
    assert rel_err(xlast, ref["x_last"]) == 0.0
    # the same call in one pass (no workspace) meets the same bar
    assert rel_err(y1, ref["y"]) <= tol
    assert rel_err(h1, ref["h_out"]) <= tol
    assert angle_err(phi1, ref["phi_out"]) <= (1e-3 if io == "bf16" else 1e-4)


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "%s-b%d-L%d-H%d-P%d-N%d-R%d" % c[:7])
def test_split_prefill_two_calls(case):
    io, b, L, H, P, N, R, Qf, Qp, mix, carry = case
    w = _wl(io, b, L, H, P, N, R, Qp, mix)
    assert m3scan.prefill_workspace_bytes(_dims(w, Qp)) > 0, "the split is not used"
    inp = inputs.make_prefill_inputs(w, seed=82, normw=True, carry=carry)
    d = to_dev(inp, DEV)
    Bb, Cb, phi = m3scan.m3_bcnorm_rope(d["B"], d["C"], d["dt"], d["theta"], d.get("normw_B"),
                                        d.get("normw_C"), d.get("bias_B"), d.get("bias_C"), d.get("phi_in"))
    Blast = torch.empty((b, H, R, N), dtype=w.torch_io, device=DEV)
    xlast = torch.empty((b, H, R, P), dtype=w.torch_io, device=DEV)
    y, h = m3scan.m3_prefill(d["x"], Bb, Cb, d["dt"], d["A"], d["lam"], d["w_out"] if mix else None,
                             d.get("h_in"), d.get("Bbar_prev"), d.get("x_prev"), Bbar_last=Blast,
                             x_last=xlast, chunk=Qp)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=mix)
    tol = TOL[io]
    assert rel_err(y, ref["y"]) <= tol
    assert rel_err(h, ref["h_out"]) <= tol
    assert rel_err(Blast, ref["Bbar_last"]) <= tol
    assert rel_err(xlast, ref["x_last"]) == 0.0


def test_split_layer_prefill_in_place_carry():
    """h_out = h_in and phi_out = phi_in on the split path (the angle pass must not clobber the
    carried angle before segment 0 reads it)."""
    w = _wl("bf16", 1, 4500, 2, 64, 128, 2, 16, True)
    inp = inputs.make_prefill_inputs(w, seed=83, normw=True, carry=True)
    d = to_dev(inp, DEV)
    h = d["h_in"].clone()
    phi = d["phi_in"].clone()
    y, _, _ = _layer(dict(d, h_in=h, phi_in=phi), w, 16, True, h_out=h, phi_out=phi)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=True)
    assert rel_err(y, ref["y"]) <= TOL["bf16"]
    assert rel_err(h, ref["h_out"]) <= TOL["bf16"]
    assert angle_err(phi, ref["phi_out"]) <= 1e-3


def test_split_rerun_lengths():
    """Pass 2's rerun length per segment, from the log2 decay l2(t) = log2(e) A sum_{s <= t} dt_s
    counted from the segment's start: whole 16-step chunks up to the last chunk whose first step
    still has l2 >= -48 (the decay is monotone here, so that step is the chunk's largest).  Three
    heads at the extremes: A = -1e-4 (the carry never decays: every segment is rerun whole),
    A = -40 (gone within a chunk) and A = -16 with dt = 4 at each segment's first step (gone at
    that step: nothing is rerun).  The recorded lengths are read back from the workspace, and y,
    h_out and phi_out checked against the oracle, through m3_layer_prefill and m3_prefill."""
    L, H, P, N, R, Q = 4100, 3, 64, 128, 2, 16
    w = _wl("bf16", 1, L, H, P, N, R, Q, True)
    inp = inputs.make_prefill_inputs(w, seed=86, normw=True, carry=True)
    inp["A"] = torch.tensor([-1e-4, -40.0, -16.0], dtype=torch.float32)
    # 3 pairs on 256 compute units: 4100 steps in segments of 1536 (a multiple of 512, at least
    # 1024 steps each): 1536, 1536, 1028
    seglen, nseg = 1536, 3
    for s in range(1, nseg):
        inp["dt"][0, s * seglen, 2] = 4.0
    r = lambda n: (n + 255) // 256 * 256
    off_fix = r(H * nseg * N * P * 4) + r(H * nseg * R * N * 2) + r(H * nseg * 4)
    need = m3scan.layer_prefill_workspace_bytes(_dims(w, Q))
    assert need == off_fix + r(H * nseg * 4) + 2 * r(H * nseg * (N // 2) * 4), \
        "the split plan differs from the one this test assumes"
    d = to_dev(inp, DEV)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y, h, phi = _layer(d, w, Q, True, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, bcnorm=True, mix=True)
    assert rel_err(y, ref["y"]) <= TOL["bf16"]
    assert rel_err(h, ref["h_out"]) <= TOL["bf16"]
    assert angle_err(phi, ref["phi_out"]) <= 1e-3
    fix = ws[off_fix:off_fix + H * nseg * 4].view(torch.int32).view(H, nseg).cpu()
    # the same split through m3_prefill (its workspace ends after the rerun lengths)
    Bb, Cb, _ = m3scan.m3_bcnorm_rope(d["B"], d["C"], d["dt"], d["theta"], d["normw_B"], d["normw_C"],
                                      d["bias_B"], d["bias_C"], d["phi_in"])
    need2 = m3scan.prefill_workspace_bytes(_dims(w, Q))
    assert need2 == off_fix + r(H * nseg * 4)
    ws2 = torch.empty(need2, dtype=torch.uint8, device=DEV)
    y2, h2 = m3scan.m3_prefill(d["x"], Bb, Cb, d["dt"], d["A"], d["lam"], d["w_out"], d["h_in"],
                               d["Bbar_prev"], d["x_prev"], chunk=Q, workspace=ws2)
    torch.cuda.synchronize()
    assert rel_err(y2, ref["y"]) <= TOL["bf16"]
    assert rel_err(h2, ref["h_out"]) <= TOL["bf16"]
    fix2 = ws2[off_fix:off_fix + H * nseg * 4].view(torch.int32).view(H, nseg).cpu()
    dt = inp["dt"][0].double()
    for f in (fix, fix2):
        for hh in range(H):
            for s in range(nseg):
                t0, t1 = s * seglen, min((s + 1) * seglen, L)
                l2 = torch.cumsum(dt[t0:t1, hh] * float(inp["A"][hh]) * 1.4426950408889634, 0)
                firsts = l2[::Q]
                # a chunk whose first step sits within 1e-3 of the threshold may go either way in fp32
                lo = [c + 1 for c in range(len(firsts)) if firsts[c] >= -48 + 1e-3]
                hi = [c + 1 for c in range(len(firsts)) if firsts[c] >= -48 - 1e-3]
                lo = min(max(lo, default=0) * Q, t1 - t0)
                hi = min(max(hi, default=0) * Q, t1 - t0)
                assert lo <= int(f[hh, s]) <= hi, (hh, s, int(f[hh, s]), lo, hi)
        assert f[0].tolist() == [1536, 1536, 1028]
        assert f[1].tolist() == [Q, Q, Q]
        assert f[2, 1:].tolist() == [0, 0]


def test_split_workspace_too_small_is_rejected():
    w = _wl("bf16", 1, 3000, 2, 64, 128, 1, 32, False)
    inp = inputs.make_prefill_inputs(w, seed=84)
    d = to_dev(inp, DEV)
    need = m3scan.layer_prefill_workspace_bytes(_dims(w, 32))
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(m3scan.M3Error) as e:
        _layer(d, w, 32, False, workspace=small)
    assert e.value.status == m3scan.M3_E_WORKSPACE


_HEAD_AXIS = {"x": 2, "dt": 2, "lam": 2, "theta": 2, "A": 0, "h_in": 1, "Bbar_prev": 1,
              "x_prev": 1, "phi_in": 1, "bias_B": 0, "bias_C": 0, "normw_B": 0, "normw_C": 0,
              "w_out": 0}


def _oracle_heads(inp, heads, G, H, mix):
    """oracle.layer on the listed heads only: each head with its own inputs and its group's raw B
    and C rows (slot h // (H / G))."""
    sub = {k: v.index_select(_HEAD_AXIS[k], torch.tensor(heads)) for k, v in inp.items()
           if k in _HEAD_AXIS and v is not None}
    slots = torch.tensor([h // (H // G) for h in heads])
    sub["B"] = inp["B"].index_select(2, slots)
    sub["C"] = inp["C"].index_select(2, slots)
    return oracle.layer(sub, bcnorm=True, mix=mix)


def test_split_in_place_carry_with_reordered_segments():
    """The in-place carry (h_out = h_in, phi_out = phi_in) on a split whose segments run out of
    order: 100 (b, h) pairs in 6 segments (pass 1: 600 workgroups, more than the 512 the GPU holds
    at once; 6 does not divide 600 / 8 = 75), heads in 25 groups of 4, so the grouped launch
    reorders its workgroups XCD by XCD and some pairs' segment 0 starts after their last segment
    has finished (a pass that wrote h_out or phi_out would have overwritten the carry before
    segment 0 read it).  Sampled heads (among them 12, whose segment 0 runs in block 576 and last
    segment in block 17) against the oracle; then m3_prefill with its state in place, on the same
    shape per head."""
    H, G, L = 100, 25, 6144
    w = inputs.Workload("split_inplace", 1, L, H, 64, 128, 1, 32, "bf16", True, True, False, 1.0, groups=G)
    dims = m3scan.make_dims(1, L, H, 64, 128, 1, 32, m3scan.M3_BF16, groups=G)
    need = m3scan.layer_prefill_workspace_bytes(dims)
    assert need > 0, "the split is not used"
    inp = inputs.make_prefill_inputs(w, seed=85, normw=True, carry=True)
    d = to_dev(inp, DEV)
    h = d["h_in"].clone()
    phi = d["phi_in"].clone()
    y, _, _ = _layer(dict(d, h_in=h, phi_in=phi), w, 32, False, h_out=h, phi_out=phi)
    torch.cuda.synchronize()
    heads = [0, 12, 13, 50, 87, 99]
    ref = _oracle_heads(inp, heads, G, H, False)
    hs = torch.tensor(heads, device=DEV)
    assert rel_err(y.index_select(2, hs), ref["y"]) <= TOL["bf16"]
    assert rel_err(h.index_select(1, hs), ref["h_out"]) <= TOL["bf16"]
    assert angle_err(phi.index_select(1, hs), ref["phi_out"]) <= 1e-3
    # m3_prefill (per-head rotated B and C), state in place, 64-step chunks: 600 workgroups again
    Bb, Cb, _ = m3scan.m3_bcnorm_rope(d["B"], d["C"], d["dt"], d["theta"], d["normw_B"], d["normw_C"],
                                      d["bias_B"], d["bias_C"], d["phi_in"])
    pd = m3scan.make_dims(1, L, H, 64, 128, 1, 64, m3scan.M3_BF16)
    assert m3scan.prefill_workspace_bytes(pd) > 0, "the split is not used"
    h2 = d["h_in"].clone()
    y2, _ = m3scan.m3_prefill(d["x"], Bb, Cb, d["dt"], d["A"], d["lam"], None, h2, d["Bbar_prev"],
                              d["x_prev"], h_out=h2, chunk=64)
    torch.cuda.synchronize()
    assert rel_err(y2.index_select(2, hs), ref["y"]) <= TOL["bf16"]
    assert rel_err(h2.index_select(1, hs), ref["h_out"]) <= TOL["bf16"]
