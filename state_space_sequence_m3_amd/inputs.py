"""Seeded synthetic inputs for the Mamba-3 SSM layer core.

This module only draws random tensors; it holds none of the method's arithmetic.  Both the GPU
library's callers and the fp64 oracle take their inputs from here, so both see the same rounded
values (bf16 draws are rounded once, to nearest-even, and the oracle upcasts them exactly).

The five workloads are the layer-level shapes of the Mamba-3 paper's latency study (1.5B model,
batch 128, 512-16384 tokens, described on the bud-325 notes page, "Benchmarking Latencies"),
with no trained weights or activations: every tensor is drawn from the distribution below.

  x, B, C         ~ N(0, 1)
  dt              = softplus(N(0, 1) - 1)              per (batch, step, head)
  A               = -exp(U(0, ln 16))                  per head
  lam             = sigmoid(N(0, 1))                   per (batch, step, head)
  theta           ~ N(0, s^2), s = 1 (pi for the long-context workload), per rotation pair
  bias_B, bias_C  ~ N(0, 0.1^2)                        per (head, rank, state index)
  w_out           ~ N(0, 1) / sqrt(R)                  per (head, rank, head-dim index)
  decode state    h ~ N(0, 1), phi ~ U(-pi, pi), Bbar_prev, x_prev ~ N(0, 1)

Draw order (fixed, so a seed names one input set): A, bias_B, bias_C, w_out, x, B, C, dt, lam,
theta, then the decode-state tensors.

Mamba-2 mode (the ``mamba2`` workloads) sets lam = 1 and theta = 0 after the draws, with BCNorm
and biases off: the same kernels then run the exponential-Euler recurrence without rotation.

Head-group workloads (``groups`` = G > 0) draw raw B and C with G head slots instead of H (same
distribution); every other tensor stays per head.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int      # P
    dstate: int       # N
    rank: int         # R (1 = SISO)
    chunk: int        # Q
    io: str           # "f32" or "bf16"
    bcnorm: bool
    bias: bool
    mix: bool         # per-head output mixing over the R ranks
    theta_std: float = 1.0
    decode_steps: int = 0
    mamba2: bool = False  # Mamba-2 mode: lambda = 1 (exponential-Euler step) and theta = 0
    groups: int = 0       # head slots of raw B and C, shared by groups of H / G heads (0: per head)
    note: str = field(default="", compare=False)

    @property
    def bc_heads(self) -> int:
        """Head slots of raw B and C: G, or H when every head has its own."""
        return self.groups if self.groups else self.nheads

    @property
    def torch_io(self):
        return torch.float32 if self.io == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_siso_f32": Workload("tiny_siso_f32", 1, 64, 1, 16, 16, 1, 16, "f32", False, False, False,
                              note="b1 L64 H1 P16 N16 R1 Q16, fp32, rotation on, BCNorm off"),
    "siso_b8_l2048": Workload("siso_b8_l2048", 8, 2048, 64, 64, 128, 1, 64, "bf16", True, True,
                              False, note="b8 L2048 H64 P64 N128 R1 Q64, bf16 io, fp32 state"),
    "mimo4_b8_l2048": Workload("mimo4_b8_l2048", 8, 2048, 64, 64, 128, 4, 16, "bf16", True, True,
                               True, note="b8 L2048 H64 P64 N128 R4 Q16, bf16 io, mixing on"),
    "mamba2_siso_b8_l2048": Workload("mamba2_siso_b8_l2048", 8, 2048, 64, 64, 128, 1, 64, "bf16", False,
                                     False, False, mamba2=True,
                                     note="Mamba-2 mode: lambda = 1, theta = 0, no BCNorm/bias; b8 L2048 N128"),
    "siso_n64_b8_l2048": Workload("siso_n64_b8_l2048", 8, 2048, 64, 64, 64, 1, 64, "bf16", True, True,
                                  False, note="b8 L2048 H64 P64 N64 R1: the d_state = 64 variant"),
    "decode_b128_r1": Workload("decode_b128_r1", 128, 1, 64, 64, 128, 1, 1, "bf16", True, True,
                               False, decode_steps=256, note="b128 H64 P64 N128 R1, 256 steps"),
    "decode_b128_r4": Workload("decode_b128_r4", 128, 1, 64, 64, 128, 4, 1, "bf16", True, True,
                               True, decode_steps=256, note="b128 H64 P64 N128 R4, 256 steps"),
    "siso_g1_b8_l2048": Workload("siso_g1_b8_l2048", 8, 2048, 64, 64, 128, 1, 64, "bf16", True, True,
                                 False, groups=1,
                                 note="SISO b8 L2048 with raw B and C shared by all 64 heads (G = 1)"),
    "mimo4_g1_b8_l2048": Workload("mimo4_g1_b8_l2048", 8, 2048, 64, 64, 128, 4, 16, "bf16", True, True,
                                  True, groups=1,
                                  note="MIMO R4 b8 L2048 with raw B and C shared by all 64 heads (G = 1)"),
    "mimo4_g8_b8_l2048": Workload("mimo4_g8_b8_l2048", 8, 2048, 64, 64, 128, 4, 16, "bf16", True, True,
                                  True, groups=8,
                                  note="MIMO R4 b8 L2048 with raw B and C shared by groups of 8 heads"),
    # decode with a state of 1.07 GB, four times the 256 MB Infinity Cache: every step streams the
    # state from DRAM (the b128 state, 268 MB, can be partly served by that cache)
    "decode_b512_r1": Workload("decode_b512_r1", 512, 1, 64, 64, 128, 1, 1, "bf16", True, True,
                               False, decode_steps=256, note="b512 H64 P64 N128 R1, 256 steps"),
    "decode_b512_r4": Workload("decode_b512_r4", 512, 1, 64, 64, 128, 4, 1, "bf16", True, True,
                               True, decode_steps=256, note="b512 H64 P64 N128 R4, 256 steps"),
    "long_mimo4_b1_l16384": Workload("long_mimo4_b1_l16384", 1, 16384, 64, 64, 128, 4, 16, "bf16",
                                     True, True, True, theta_std=math.pi, decode_steps=512,
                                     note="b1 L16384 H64 R4 Q16, theta std pi, then 512 decode steps"),
}

# The comparison grid of the kernel-time table on the aipaper.cc summary (section 6.2, Table 3):
# Mamba-2 mode, SISO and MIMO R = 4, each with fp32 and bf16 io and d_state 64 and 128, on the b8
# L2048 H64 P64 layer shape.  Keyed by (mode, io, N).
def _grid():
    base = {"mamba2": WORKLOADS["mamba2_siso_b8_l2048"], "siso": WORKLOADS["siso_b8_l2048"],
            "mimo4": WORKLOADS["mimo4_b8_l2048"]}
    grid = {}
    for mode, w0 in base.items():
        for io in ("f32", "bf16"):
            for n in (64, 128):
                suffix = ("" if n == 128 else "_n64") + ("" if io == "bf16" else "_f32")
                name = w0.name.replace("_b8", suffix + "_b8") if suffix else w0.name
                if name not in WORKLOADS:
                    WORKLOADS[name] = w0.with_(name=name, io=io, dstate=n,
                                               note="%s, %s io, d_state %d (comparison grid)" % (mode, io, n))
                grid[(mode, io, n)] = name
    return grid


TABLE3_GRID = _grid()


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(g, shape, device, std=1.0, mean=0.0):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std + mean


def _uniform(g, shape, device, lo, hi):
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def make_params(w: Workload, g, device, normw: bool = False) -> dict:
    """Per-head constants: A [H], bias_B/bias_C [H,R,N], w_out [H,R,P], optional normw [H,N]."""
    H, R, N, P = w.nheads, w.rank, w.dstate, w.headdim
    out = {"A": -torch.exp(_uniform(g, (H,), device, 0.0, math.log(16.0)))}
    out["bias_B"] = _normal(g, (H, R, N), device, 0.1) if w.bias else None
    out["bias_C"] = _normal(g, (H, R, N), device, 0.1) if w.bias else None
    out["w_out"] = _normal(g, (H, R, P), device) / math.sqrt(R) if w.mix else None
    if normw:
        out["normw_B"] = 1.0 + _normal(g, (H, N), device, 0.1)
        out["normw_C"] = 1.0 + _normal(g, (H, N), device, 0.1)
    else:
        out["normw_B"] = None
        out["normw_C"] = None
    return out


def make_sequence(w: Workload, g, device, lead: tuple) -> dict:
    """Per-step tensors with leading dims ``lead`` (e.g. (b, L) for prefill, (steps, b) for decode).

    x [*lead, H, R, P], B, C [*lead, G, R, N] (G = H unless the workload shares them across head
    groups), dt, lam [*lead, H], theta [*lead, H, N/2], all in the workload's io dtype.
    """
    H, R, N, P = w.nheads, w.rank, w.dstate, w.headdim
    io = w.torch_io
    out = {}
    out["x"] = _normal(g, (*lead, H, R, P), device).to(io)
    out["B"] = _normal(g, (*lead, w.bc_heads, R, N), device).to(io)
    out["C"] = _normal(g, (*lead, w.bc_heads, R, N), device).to(io)
    out["dt"] = torch.nn.functional.softplus(_normal(g, (*lead, H), device) - 1.0).to(io)
    out["lam"] = torch.sigmoid(_normal(g, (*lead, H), device)).to(io)
    out["theta"] = _normal(g, (*lead, H, N // 2), device, w.theta_std).to(io)
    if w.mamba2:   # drawn first, so the other tensors of a seed are the same in both modes
        out["lam"] = torch.ones_like(out["lam"])
        out["theta"] = torch.zeros_like(out["theta"])
    return out


def make_decode_state(w: Workload, g, device) -> dict:
    """Resident decode state: h [b,H,N,P] f32, phi [b,H,N/2] f32, Bbar_prev, x_prev (io)."""
    b, H, R, N, P = w.batch, w.nheads, w.rank, w.dstate, w.headdim
    return {
        "h": _normal(g, (b, H, N, P), device),
        "phi": _uniform(g, (b, H, N // 2), device, -math.pi, math.pi),
        "Bbar_prev": _normal(g, (b, H, R, N), device).to(w.torch_io),
        "x_prev": _normal(g, (b, H, R, P), device).to(w.torch_io),
    }


def make_prefill_inputs(w: Workload, seed: int, device="cpu", normw: bool = False,
                        carry: bool = False) -> dict:
    """All inputs of one prefill call of workload ``w``.

    With ``carry`` the call also receives a carried-in state (h_in, phi_in, Bbar_prev, x_prev)
    drawn like the decode state, as a continuation of an earlier call would.
    """
    g = _gen(seed, device)
    out = make_params(w, g, device, normw=normw)
    out.update(make_sequence(w, g, device, (w.batch, w.seqlen)))
    if carry:
        st = make_decode_state(w, g, device)
        out["h_in"] = st["h"]
        out["phi_in"] = st["phi"]
        out["Bbar_prev"] = st["Bbar_prev"]
        out["x_prev"] = st["x_prev"]
    return out


def make_cotangents(w: Workload, seed: int, device="cpu") -> dict:
    """Seeded cotangents for a backward call of workload ``w``: dy with y's shape ([b, L, H, P]
    with output mixing, else [b, L, H, R, P]) in the io dtype, dh_out [b, H, N, P] and
    dphi_out [b, H, N/2] in fp32, all ~ N(0, 1)."""
    g = _gen(seed, device)
    b, L, H, R, N, P = w.batch, w.seqlen, w.nheads, w.rank, w.dstate, w.headdim
    yshape = (b, L, H, P) if w.mix else (b, L, H, R, P)
    return {"dy": _normal(g, yshape, device).to(w.torch_io),
            "dh_out": _normal(g, (b, H, N, P), device),
            "dphi_out": _normal(g, (b, H, N // 2), device)}


def make_decode_inputs(w: Workload, seed: int, steps: int, device="cpu",
                       normw: bool = False) -> dict:
    """Constants, a starting state and ``steps`` tokens laid out step-major ([steps, b, H, ...])."""
    g = _gen(seed, device)
    out = make_params(w, g, device, normw=normw)
    out["tokens"] = make_sequence(w, g, device, (steps, w.batch))
    out["state"] = make_decode_state(w, g, device)
    return out
