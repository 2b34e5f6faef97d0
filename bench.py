#!/usr/bin/env python3
"""Benchmark of the Mamba-3 SSM layer core on one MI355X.

One step = one pass of the layer core (BCNorm + bias + rotation, then the chunked scan) over one
batch of the SISO workload (b=8, L=2048, H=64, P=64, N=128, R=1, bf16 io, fp32 state) through
m3_layer_prefill, which does both in one kernel (chunk 32).  `value` is prefill tokens/s (b * L
tokens per step).  The same line carries:
  * the two-call path (m3_bcnorm_rope then m3_prefill, chunk 64) and the MIMO R=4 workload
    through both paths;
  * the comparison grid of the kernel-time table (Mamba-2 mode / SISO / MIMO R=4, fp32 / bf16,
    d_state 64 / 128) through the fused call;
  * decode steps/s on the B=128 workloads (state 268 MB) and on B=512 (state 1.07 GB, four times
    the 256 MB Infinity Cache, so every step streams its state from DRAM), R=1 and R=4, through
    m3_layer_decode_step and through the two calls (m3_bcnorm_rope L=1 + m3_decode_step);
  * head groups, packed variable-length prefill, the long-context split, small-batch decode from
    HIP graphs, and the backward pass;
  * the roofline of the step's kernel measured live with HIP events on the launch stream, a plain
    1 GiB copy timed in the same run, and the fp64 oracle's throughput on bounded samples of the
    workloads on the host cores.
Every timed loop runs its warm-up steps and then at least WARM_S seconds of the same work before
the timed steps (the GPU's clocks ramp over the first tens of milliseconds of work).

    python bench.py [--gpus 1] [--steps 20] [--warmup 20] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from state_space_sequence_m3_amd import inputs, m3scan  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 MFMA, TFLOP/s
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X fp32 (matrix and vector), TFLOP/s


KERNEL_SOURCES = {
    "prefill_kernel<bf16,128,64,4>": ("prefill.hip", "m3_device.h", "m3_mapping.h", "m3_launch.h", "m3_mma.h"),
    "prefill_kernel<bf16,128,64,2,fused>": ("prefill.hip", "m3_device.h", "m3_mapping.h", "m3_launch.h", "m3_mma.h"),
}
LAYER_CHUNK_ROWS = 32   # chunk * R rows per tile of the fused kernel
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "layer_core_siso_b8_l2048_hbm_traffic.md")


def source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "state_space_sequence_m3_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE record of this kernel, or
    None if there is none or the kernel's sources changed since the counters were taken."""
    if kernel not in KERNEL_SOURCES or not os.path.exists(TRAFFIC_FILE):
        return None
    want = source_digest(KERNEL_SOURCES[kernel])
    with open(TRAFFIC_FILE) as f:
        for line in f:
            line = line.strip()
            if not line.startswith("traffic-record "):
                continue
            kv = dict(item.split("=", 1) for item in line.split()[1:])
            if kv.get("kernel") == kernel and kv.get("workload") == workload and kv.get("digest") == want:
                return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


def prefill_bytes_per_token_head(w) -> int:
    """Compulsory HBM bytes of m3_prefill per (token, head): x, Bbar, Cbar, dt, lam read once,
    y written once (the final state is added per (b, h) separately)."""
    es = 2 if w.io == "bf16" else 4
    R, N, P = w.rank, w.dstate, w.headdim
    y = P if w.mix else R * P
    return es * (R * P + 2 * R * N + 2 + y)


def bcnorm_bytes_per_token_head(w) -> int:
    """m3_bcnorm_rope: B, C, theta, dt read once; Bbar, Cbar written once."""
    es = 2 if w.io == "bf16" else 4
    R, N = w.rank, w.dstate
    return es * (4 * R * N + N // 2 + 1)


def layer_bytes_per_token_head(w) -> float:
    """m3_layer_prefill: x, raw B and C, theta, dt, lam read once, y written once.  Raw B and C
    shared by groups of heads are read once per group: a share G / H of them per head."""
    es = 2 if w.io == "bf16" else 4
    R, N, P = w.rank, w.dstate, w.headdim
    y = P if w.mix else R * P
    return es * (R * P + 2 * R * N * w.bc_heads / w.nheads + N // 2 + 2 + y)


def prefill_flops_per_token_head(w) -> int:
    """Chunked form with full Q x Q blocks: 2 Q R^2 (N + P) + 4 R N P."""
    Q, R, N, P = w.chunk, w.rank, w.dstate, w.headdim
    return 2 * Q * R * R * (N + P) + 4 * R * N * P


def decode_bytes_per_head(w) -> int:
    """m3_decode_step per (b, h): fp32 state read + written, Bbar_prev, x_prev, x, Bbar, Cbar,
    dt, lam read, y written."""
    es = 2 if w.io == "bf16" else 4
    R, N, P = w.rank, w.dstate, w.headdim
    y = P if w.mix else R * P
    return 2 * N * P * 4 + es * (3 * R * N + 2 * R * P + 2 + y)


def layer_decode_bytes_per_head(w) -> int:
    """m3_layer_decode_step per (b, h): fp32 state read + written, angle read + written, Bbar_prev,
    x_prev, x, raw B and C, dt, lam, theta read, the rotated B and y written."""
    es = 2 if w.io == "bf16" else 4
    R, N, P = w.rank, w.dstate, w.headdim
    y = P if w.mix else R * P
    return 2 * N * P * 4 + 2 * (N // 2) * 4 + es * (4 * R * N + 2 * R * P + 2 + N // 2 + y)


# The GPU reaches its steady clocks only after some tens of milliseconds of sustained work: every
# timed loop below first runs its `warmup` steps, then keeps running the same step until at least
# WARM_S seconds of work have passed since the warm-up began (untimed), then times its steps.
WARM_S = float(os.environ.get("M3_BENCH_WARM_S", "0.25"))


def warm_up(step, warmup):
    t_start = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    while time.perf_counter() - t_start < WARM_S:
        for _ in range(4):
            step()
        torch.cuda.synchronize()


def time_prefill(w, steps, warmup, dev, inp=None, scan_only=False):
    """The two-call path: m3_bcnorm_rope then m3_prefill (chunk w.chunk).  With scan_only the
    rotation call is left out and m3_prefill reads the raw B and C (Mamba-2 mode)."""
    if inp is None:
        inp = inputs.make_prefill_inputs(w, seed=0, device=dev)
    b, L, H, R, N, P = w.batch, w.seqlen, w.nheads, w.rank, w.dstate, w.headdim
    io = w.torch_io
    Bb = torch.empty((b, L, H, R, N), dtype=io, device=dev)
    Cb = torch.empty_like(Bb)
    phi = torch.empty((b, H, N // 2), dtype=torch.float32, device=dev)
    y = torch.empty((b, L, H, P) if w.mix else (b, L, H, R, P), dtype=io, device=dev)
    h = torch.empty((b, H, N, P), dtype=torch.float32, device=dev)
    dims = m3scan.make_dims(b, L, H, P, N, R, w.chunk, m3scan.M3_BF16 if w.io == "bf16" else m3scan.M3_F32)
    wsb = m3scan.bcnorm_rope_workspace_bytes(dims)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    pneed = m3scan.prefill_workspace_bytes(dims)
    pws = torch.empty(pneed, dtype=torch.uint8, device=dev) if pneed else False
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if not scan_only:
            m3scan.m3_bcnorm_rope(inp["B"], inp["C"], inp["dt"], inp["theta"], inp["normw_B"],
                                  inp["normw_C"], inp["bias_B"], inp["bias_C"], None, Bbar=Bb, Cbar=Cb,
                                  phi_out=phi, bcnorm=w.bcnorm, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        m3scan.m3_prefill(inp["x"], inp["B"] if scan_only else Bb, inp["C"] if scan_only else Cb,
                          inp["dt"], inp["A"], inp["lam"],
                          inp["w_out"] if w.mix else None, y=y, h_out=h, chunk=w.chunk, workspace=pws)
        if ev is not None:
            ev[2].record(stream)

    warm_up(step, warmup)
    # whole-step timing: K steps between two events
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    # per-kernel timing on the same stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    ms_bc = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    ms_pf = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    return inp, ms_step, ms_bc, ms_pf


def time_layer(w, inp, chunk, steps, warmup, dev):
    """`steps` fused layer passes (m3_layer_prefill) between two HIP events on the launch stream."""
    b, L, H, R, N, P = w.batch, w.seqlen, w.nheads, w.rank, w.dstate, w.headdim
    y = torch.empty((b, L, H, P) if w.mix else (b, L, H, R, P), dtype=w.torch_io, device=dev)
    h = torch.empty((b, H, N, P), dtype=torch.float32, device=dev)
    phi = torch.empty((b, H, N // 2), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # the sequence-split workspace (few long sequences), allocated once outside the timed region
    dims = m3scan.make_dims(b, L, H, P, N, R, chunk, m3scan.M3_BF16 if w.io == "bf16" else m3scan.M3_F32,
                            w.bcnorm, groups=w.groups)
    need = m3scan.layer_prefill_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else False

    def step():
        m3scan.m3_layer_prefill(inp["x"], inp["B"], inp["C"], inp["dt"], inp["theta"], inp["A"],
                                inp["lam"], inp["normw_B"], inp["normw_C"], inp["bias_B"],
                                inp["bias_C"], inp["w_out"] if w.mix else None, y=y, h_out=h,
                                phi_out=phi, chunk=chunk, bcnorm=w.bcnorm, workspace=ws)

    warm_up(step, warmup)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


# Decode tokens come from a ring of this many distinct seeded tokens (step s uses token s mod
# TOKEN_RING): the state, read and written every step, is what the step moves; the tokens only
# need to be distinct and realistic, not 256 + warm-up different ones.
TOKEN_RING = 32


def time_layer_decode(w, steps, warmup, dev):
    """`steps` consecutive decode tokens through m3_layer_decode_step (rotation + decode in one
    launch), HIP-event timed on the launch stream."""
    dinp = inputs.make_decode_inputs(w, seed=0, steps=TOKEN_RING, device=dev)
    toks, st = dinp["tokens"], dinp["state"]
    b, H, R, N, P = w.batch, w.nheads, w.rank, w.dstate, w.headdim
    h, phi = st["h"], st["phi"]
    bufs = [st["Bbar_prev"], torch.empty_like(st["Bbar_prev"])]
    y = torch.empty((b, H, P) if w.mix else (b, H, R, P), dtype=w.torch_io, device=dev)
    stream = torch.cuda.current_stream()
    xprev = st["x_prev"]
    count = 0

    def tok():
        nonlocal xprev, count
        s = count % TOKEN_RING
        Bprev, Bcur = bufs[count % 2], bufs[(count + 1) % 2]
        m3scan.m3_layer_decode_step(h, phi, Bprev, xprev, toks["x"][s], toks["B"][s], toks["C"][s],
                                    toks["dt"][s], toks["theta"][s], dinp["A"], toks["lam"][s], None,
                                    None, dinp["bias_B"], dinp["bias_C"],
                                    dinp["w_out"] if w.mix else None, y=y, Bbar_out=Bcur)
        xprev = toks["x"][s]
        count += 1

    warm_up(tok, warmup)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        tok()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


VARLEN_LENGTHS = (512, 1024, 2048, 3072, 4096, 1536, 2560, 1536)   # 16384 tokens, 8 prompts


def time_varlen(w, steps, warmup, dev):
    """m3_layer_prefill_varlen on a packed batch of prompts of mixed lengths (the SISO layer's
    shapes, as many tokens as its b * L), HIP-event timed."""
    T = sum(VARLEN_LENGTHS)
    wp = w.with_(batch=1, seqlen=T)
    inp = inputs.make_prefill_inputs(wp, seed=0, device=dev)
    offs = [0]
    for n in VARLEN_LENGTHS:
        offs.append(offs[-1] + n)
    cu = torch.tensor(offs, dtype=torch.int32, device=dev)
    packed = {k: inp[k][0] for k in ("x", "B", "C", "dt", "lam", "theta")}
    y = torch.empty((T, w.nheads, w.headdim), dtype=w.torch_io, device=dev)

    def step():
        m3scan.m3_layer_prefill_varlen(cu, packed["x"], packed["B"], packed["C"], packed["dt"], packed["theta"],
                                       inp["A"], packed["lam"], inp["normw_B"], inp["normw_C"], inp["bias_B"],
                                       inp["bias_C"], None, y=y.view(T, w.nheads, w.rank, w.headdim),
                                       chunk=LAYER_CHUNK_ROWS // w.rank)

    warm_up(step, warmup)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    return {"ms": ms, "tokens/s": T / (ms / 1e3), "lengths": list(VARLEN_LENGTHS),
            "how": "m3_layer_prefill_varlen, one packed batch, chunk %d" % (LAYER_CHUNK_ROWS // w.rank)}


def time_small_batch_decode(w, steps, dev, graph_steps=16):
    """Decode at small batch, where launches rather than bytes bound a step: `steps` tokens of
    m3_layer_decode_step launched one by one, and the same tokens replayed from HIP graphs that
    each hold `graph_steps` steps.  Returns (eager ms/step, graph ms/step)."""
    dinp = inputs.make_decode_inputs(w, seed=0, steps=graph_steps, device=dev)
    toks, st = dinp["tokens"], dinp["state"]
    b, H, R, N, P = w.batch, w.nheads, w.rank, w.dstate, w.headdim
    h, phi = st["h"].clone(), st["phi"].clone()
    bufs = [st["Bbar_prev"].clone(), torch.empty_like(st["Bbar_prev"])]
    ys = torch.empty((graph_steps, b, H, P) if w.mix else (graph_steps, b, H, R, P), dtype=w.torch_io,
                     device=dev)
    x0 = st["x_prev"]

    def run():
        xprev = x0
        for s in range(graph_steps):
            m3scan.m3_layer_decode_step(h, phi, bufs[s % 2], xprev, toks["x"][s], toks["B"][s], toks["C"][s],
                                        toks["dt"][s], toks["theta"][s], dinp["A"], toks["lam"][s], None,
                                        None, dinp["bias_B"], dinp["bias_C"],
                                        dinp["w_out"] if w.mix else None, y=ys[s],
                                        Bbar_out=bufs[(s + 1) % 2])
            xprev = toks["x"][s]

    reps = max(1, steps // graph_steps)
    run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        run()
    t1.record()
    torch.cuda.synchronize()
    ms_eager = t0.elapsed_time(t1) / (reps * graph_steps)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    graph.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_graph = t0.elapsed_time(t1) / (reps * graph_steps)
    return ms_eager, ms_graph


def time_decode(w, steps, warmup, dev):
    """`steps` consecutive decode tokens (bcnorm_rope L=1 + decode_step each), HIP-event timed."""
    dinp = inputs.make_decode_inputs(w, seed=0, steps=TOKEN_RING, device=dev)
    toks, st = dinp["tokens"], dinp["state"]
    b, H, R, N, P = w.batch, w.nheads, w.rank, w.dstate, w.headdim
    h, phi = st["h"], st["phi"]
    bufs = [st["Bbar_prev"], torch.empty_like(st["Bbar_prev"])]
    Cc = torch.empty_like(bufs[0])
    y = torch.empty((b, H, P) if w.mix else (b, H, R, P), dtype=w.torch_io, device=dev)
    stream = torch.cuda.current_stream()
    xprev = st["x_prev"]

    def tok(c, ev=None):
        nonlocal xprev
        s = c % TOKEN_RING
        Bprev, Bcur = bufs[c % 2], bufs[(c + 1) % 2]
        if ev is not None:
            ev[0].record(stream)
        m3scan.m3_bcnorm_rope(toks["B"][s].unsqueeze(1), toks["C"][s].unsqueeze(1),
                              toks["dt"][s].unsqueeze(1), toks["theta"][s].unsqueeze(1), None, None,
                              dinp["bias_B"], dinp["bias_C"], phi, Bbar=Bcur.unsqueeze(1),
                              Cbar=Cc.unsqueeze(1), phi_out=phi)
        if ev is not None:
            ev[1].record(stream)
        m3scan.m3_decode_step(h, Bprev, xprev, toks["x"][s], Bcur, Cc, toks["dt"][s], dinp["A"],
                              toks["lam"][s], dinp["w_out"] if w.mix else None, y=y)
        if ev is not None:
            ev[2].record(stream)
        xprev = toks["x"][s]

    count = 0

    def next_tok():
        nonlocal count
        tok(count)
        count += 1

    warm_up(next_tok, warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for k in range(steps):
        tok(count + k, evs[k])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_tok = t0.elapsed_time(t1) / steps
    ms_bc = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    ms_dec = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    return ms_tok, ms_bc, ms_dec


def backward_bytes_per_token_head(w) -> int:
    """Compulsory HBM bytes of m3_layer_backward per (token, head): the forward inputs x, B, C, dt,
    lam, theta and the cotangent dy read once, the gradients dx, dB, dC, ddt, dlam, dtheta written
    once.  The chunk states the call saves and reads back are its own intermediates (excluded).
    Raw B and C shared by groups of heads (and their gradients) count G / H per head."""
    es = 2 if w.io == "bf16" else 4
    R, N, P = w.rank, w.dstate, w.headdim
    io = R * P + 2 * R * N * w.bc_heads / w.nheads + 2 + N // 2
    return es * (2 * io + (P if w.mix else R * P))


def backward_flops_per_token_head(w, chunk_rows) -> int:
    """MFMA flops of m3_layer_backward per (token, head), counting full chunk-square blocks: per
    chunk of QR rows, S and dP (QR^2 N, QR^2 P), dX, dBbar, dCbar (QR^2 P, 2 QR^2 N plus three
    QR N P state products), the state cotangent and the saved-state recompute (2 QR N P), the
    recomputed Y for the mixing gradient (QR N P + QR^2 P), 2 flops per multiply-add."""
    R, N, P, QR = w.rank, w.dstate, w.headdim, chunk_rows
    per_chunk = 2 * (QR * QR * (3 * N + 2 * P) + 5 * QR * N * P)
    if w.mix:
        per_chunk += 2 * (QR * N * P + QR * QR * P)
    return per_chunk * R // QR


def time_backward(w, steps, warmup, dev):
    """m3_layer_backward on workload w (inputs, cotangents, gradients and workspace allocated
    once), HIP-event timed on the launch stream; also m3_layer_chunk_states alone (the first of the
    call's kernels) for the split."""
    inp = inputs.make_prefill_inputs(w, seed=0, device=dev)
    cot = inputs.make_cotangents(w, seed=1, device=dev)
    mixw = inp["w_out"] if w.mix else None
    grads = m3scan.m3_layer_backward(inp["x"], inp["B"], inp["C"], inp["dt"], inp["theta"], inp["A"],
                                     inp["lam"], cot["dy"], inp["normw_B"], inp["normw_C"], inp["bias_B"],
                                     inp["bias_C"], mixw, bcnorm=w.bcnorm)
    dims = m3scan.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, 0,
                            m3scan._io_code(w.torch_io), w.bcnorm, groups=w.groups)
    ws = torch.empty(m3scan.layer_backward_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        m3scan.m3_layer_backward(inp["x"], inp["B"], inp["C"], inp["dt"], inp["theta"], inp["A"], inp["lam"],
                                 cot["dy"], inp["normw_B"], inp["normw_C"], inp["bias_B"], inp["bias_C"], mixw,
                                 grads=grads, bcnorm=w.bcnorm, workspace=ws)

    def states():
        m3scan.m3_layer_chunk_states(inp["x"], inp["B"], inp["dt"], inp["theta"], inp["A"], inp["lam"],
                                     inp["normw_B"], inp["bias_B"], bcnorm=w.bcnorm)

    out = {}
    for name, fn in (("m3_layer_backward", step), ("m3_layer_chunk_states", states)):
        warm_up(fn, warmup)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        out[name] = t0.elapsed_time(t1) / steps
    del inp, cot, grads, ws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, inp, nheads: int):
    """The fp64 oracle (unchanged) on a bounded sample of the prefill workload: every batch row
    and the first `nheads` heads, i.e. batch * nheads (batch, head) pairs over the full length
    (by default all heads: the whole workload, about a second of host work)."""
    import oracle
    host = {}
    for k in ("x", "B", "C", "dt", "lam", "theta"):
        host[k] = inp[k][:, :, :nheads].cpu()
    host["A"] = inp["A"][:nheads].cpu()
    for k in ("bias_B", "bias_C", "normw_B", "normw_C", "w_out"):
        host[k] = None if inp[k] is None else inp[k][:nheads].cpu()
    t_start = time.perf_counter()
    oracle.layer(host, bcnorm=w.bcnorm, mix=w.mix)
    secs = time.perf_counter() - t_start
    pairs = w.batch * nheads
    tokens = pairs * w.seqlen / w.nheads   # (batch, head) pairs -> whole-layer tokens
    return {"value": tokens / secs, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d (batch, head) pairs (all %d batch rows x %d of %d heads) x %d steps of "
                      "%s, fp64 bcnorm_rope + scan, %.2f s wall; tokens = pairs * L / H"
                      % (pairs, w.batch, nheads, w.nheads, w.seqlen, w.name, secs)}


def copy_probe(nbytes: int, steps: int, warmup: int, dev):
    """A plain device-to-device copy of known size: the practical HBM ceiling on this machine, and
    the reference against which the FETCH_SIZE / WRITE_SIZE counters are scaled."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).normal_()
    dst = torch.empty_like(src)
    warm_up(lambda: dst.copy_(src), warmup)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    moved = 2 * src.numel() * 4
    return {"copy_bytes_read": src.numel() * 4, "copy_bytes_written": src.numel() * 4,
            "ms": ms, "GB/s": moved / ms / 1e6, "hbm_frac": moved / ms / 1e6 / HBM_PEAK_GBS}


def grid_entry(wv, inpv, steps, warmup, dev):
    """One cell of the comparison grid: m3_layer_prefill (and, in Mamba-2 mode, m3_prefill on
    the raw B and C, which are already the scan's inputs there)."""
    thv = wv.batch * wv.seqlen * wv.nheads
    rows = LAYER_CHUNK_ROWS
    ms_l = time_layer(wv, inpv, rows // wv.rank, steps, warmup, dev)
    wl = wv.with_(chunk=rows // wv.rank)
    lb = thv * layer_bytes_per_token_head(wv) + wv.batch * wv.nheads * wv.dstate * (wv.headdim + 1) * 4
    lf = thv * prefill_flops_per_token_head(wl)
    peak = BF16_MFMA_PEAK_TFLOPS if wv.io == "bf16" else FP32_MFMA_PEAK_TFLOPS
    entry = {"workload": wv.name, "m3_layer_prefill": {
        "ms": ms_l, "tokens/s": wv.batch * wv.seqlen / (ms_l / 1e3), "chunk": wl.chunk,
        "GB/s": lb / ms_l / 1e6, "hbm_frac": lb / ms_l / 1e6 / HBM_PEAK_GBS,
        "TFLOP/s": lf / ms_l / 1e9, "mfma_frac": lf / ms_l / 1e9 / peak}}
    if wv.mamba2:
        _, _, _, ms_p = time_prefill(wv, steps, warmup, dev, inpv, scan_only=True)
        pb = thv * prefill_bytes_per_token_head(wv) + wv.batch * wv.nheads * wv.dstate * wv.headdim * 4
        entry["m3_prefill"] = {"ms": ms_p, "tokens/s": wv.batch * wv.seqlen / (ms_p / 1e3), "chunk": wv.chunk,
                               "GB/s": pb / ms_p / 1e6, "hbm_frac": pb / ms_p / 1e6 / HBM_PEAK_GBS}
    return entry


def time_grid(steps, warmup, dev):
    """The kernel-time comparison grid of the aipaper.cc summary (section 6.2, Table 3): Mamba-2
    mode, SISO and MIMO R = 4, each in fp32 and bf16 io at d_state 64 and 128, on the b8 L2048
    H64 P64 layer, all through the same fused kernel."""
    out = {}
    for (mode, io, n), name in inputs.TABLE3_GRID.items():
        wv = inputs.WORKLOADS[name]
        inpv = inputs.make_prefill_inputs(wv, seed=0, device=dev)
        out["%s/%s/N%d" % (mode, io, n)] = grid_entry(wv, inpv, steps, warmup, dev)
        del inpv
        torch.cuda.empty_cache()
    return out


def more_cpu_baselines(w, inp):
    """The unchanged oracle on bounded samples of the other workloads (on the host's OpenMP
    threads), and on one thread for the SISO workload: MIMO prefill (one head of every batch
    row), one decode step of the whole b128 batch (R = 1 and R = 4), and the long-context prefill
    on two heads (the full 16384 steps)."""
    import oracle
    out = {}

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    threads = oracle.num_threads()
    # SISO on one thread: 4 (batch, head) pairs, full length
    host = {k: (None if v is None else (v[:1, :, :4] if k in ("x", "B", "C", "dt", "lam", "theta") else v[:4]).cpu())
            for k, v in inp.items()}
    oracle.set_num_threads(1)
    try:
        secs = timed(lambda: oracle.layer(host, bcnorm=w.bcnorm, mix=w.mix))
    finally:
        oracle.set_num_threads(threads)
    out["siso_b8_l2048_one_thread"] = {
        "value": 4 * w.seqlen / w.nheads / secs, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": "4 (batch, head) pairs x %d steps, %.2f s" % (w.seqlen, secs)}
    for name, heads in (("mimo4_b8_l2048", 1), ("long_mimo4_b1_l16384", 2)):
        wv = inputs.WORKLOADS[name]
        g = inputs.make_prefill_inputs(wv.with_(nheads=heads), seed=0)
        secs = timed(lambda: oracle.layer(g, bcnorm=wv.bcnorm, mix=wv.mix))
        out[name] = {"value": wv.batch * heads * wv.seqlen / wv.nheads / secs, "unit": "tokens/s",
                     "cores": threads, "kind": "oracle",
                     "sample": "%d (batch, head) pairs x %d steps, %.2f s; tokens = pairs * L / H"
                               % (wv.batch * heads, wv.seqlen, secs)}
    for name in ("decode_b128_r1", "decode_b128_r4"):
        wd = inputs.WORKLOADS[name]
        dinp = inputs.make_decode_inputs(wd, seed=0, steps=1)
        tok = {k: v[0] for k, v in dinp["tokens"].items()}
        consts = {"A": dinp["A"], "bias_B": dinp["bias_B"], "bias_C": dinp["bias_C"], "w_out": dinp["w_out"]}
        secs = timed(lambda: oracle.decode_step(dinp["state"], tok, consts, mix=wd.mix))
        out[name] = {"value": 1.0 / secs, "unit": "steps/s", "cores": threads, "kind": "oracle",
                     "sample": "one decode step of all %d (batch, head) pairs, %.3f s" % (wd.batch * wd.nheads, secs)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed steps before the timed ones (followed by WARM_S seconds of the same work)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--cpu-heads", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-mimo", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--copy-only", type=int, default=0, metavar="BYTES",
                    help="only time a plain device copy of BYTES bytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer core has no cross-GPU step, and its throughput "
              "is measured on a single MI355X (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_only:
        print(json.dumps({"copy_probe": copy_probe(args.copy_only, args.steps, args.warmup, dev)}))
        return
    m3scan.load()

    def path_stats(w, inp, chunk_rows):
        """Both paths on workload w: the fused call (the step) and the two calls."""
        th = w.batch * w.seqlen * w.nheads
        tokens = w.batch * w.seqlen
        state = w.batch * w.nheads * w.dstate * w.headdim * 4
        angle = w.batch * w.nheads * (w.dstate // 2) * 4
        ms_layer = time_layer(w, inp, chunk_rows // w.rank, args.steps, args.warmup, dev)
        wl = w.with_(chunk=chunk_rows // w.rank)
        ly_bytes = th * layer_bytes_per_token_head(w) + state + angle
        ly_flops = th * prefill_flops_per_token_head(wl)
        # the two calls run m3_prefill on chunks of the same 32 rows as the fused call (measured
        # faster than the 64-row chunk of the workload's statement: SISO 2%, MIMO 8.5%)
        _, ms_two, ms_bc, ms_pf = time_prefill(wl, args.steps, args.warmup, dev, inp)
        pf_bytes = th * prefill_bytes_per_token_head(w) + state
        bc_bytes = th * bcnorm_bytes_per_token_head(w) + angle
        pf_flops = th * prefill_flops_per_token_head(wl)
        return {
            "m3_layer_prefill": {"ms": ms_layer, "tokens/s": tokens / (ms_layer / 1e3), "chunk": wl.chunk,
                                 "bytes": ly_bytes, "GB/s": ly_bytes / ms_layer / 1e6,
                                 "TFLOP/s": ly_flops / ms_layer / 1e9,
                                 "hbm_frac": ly_bytes / ms_layer / 1e6 / HBM_PEAK_GBS,
                                 "mfma_frac": ly_flops / ms_layer / 1e9 / BF16_MFMA_PEAK_TFLOPS},
            "two_calls": {"ms": ms_two, "tokens/s": tokens / (ms_two / 1e3), "chunk": wl.chunk},
            "m3_prefill": {"ms": ms_pf, "bytes": pf_bytes, "GB/s": pf_bytes / ms_pf / 1e6,
                           "TFLOP/s": pf_flops / ms_pf / 1e9,
                           "hbm_frac": pf_bytes / ms_pf / 1e6 / HBM_PEAK_GBS,
                           "mfma_frac": pf_flops / ms_pf / 1e9 / BF16_MFMA_PEAK_TFLOPS},
            "m3_bcnorm_rope": {"ms": ms_bc, "bytes": bc_bytes, "GB/s": bc_bytes / ms_bc / 1e6,
                               "hbm_frac": bc_bytes / ms_bc / 1e6 / HBM_PEAK_GBS},
        }

    w = inputs.WORKLOADS["siso_b8_l2048"]
    inp = inputs.make_prefill_inputs(w, seed=0, device=dev)
    kernels = path_stats(w, inp, LAYER_CHUNK_ROWS)
    # the practical ceiling of this GPU's memory system in the same run: a plain 1 GiB device copy
    copy = copy_probe(1 << 30, 10, 10, dev)
    torch.cuda.empty_cache()
    ms_step = kernels["m3_layer_prefill"]["ms"]
    tokens = w.batch * w.seqlen
    mimo = None
    if not args.no_mimo:
        wm = inputs.WORKLOADS["mimo4_b8_l2048"]
        inpm = inputs.make_prefill_inputs(wm, seed=0, device=dev)
        mimo = path_stats(wm, inpm, LAYER_CHUNK_ROWS)
        del inpm
        torch.cuda.empty_cache()
    # Mamba-2 mode (lambda = 1, theta = 0, no BCNorm/bias) and the d_state = 64 variant, on the
    # same kernels: the fused call (chunk 32) and the plain scan (chunk 64; in Mamba-2 mode the raw
    # B and C are already Bbar and Cbar, so the scan alone is the whole layer core)
    variants = None
    table3 = None
    if not args.no_mimo:
        table3 = time_grid(args.steps, args.warmup, dev)
        variants = {}
        # raw B and C shared by groups of heads (G = 1: all 64 heads; G = 8: groups of 8)
        for vname in ("siso_g1_b8_l2048", "mimo4_g1_b8_l2048", "mimo4_g8_b8_l2048"):
            wv = inputs.WORKLOADS[vname]
            inpv = inputs.make_prefill_inputs(wv, seed=0, device=dev)
            thv = wv.batch * wv.seqlen * wv.nheads
            ms_l = time_layer(wv, inpv, LAYER_CHUNK_ROWS // wv.rank, args.steps, args.warmup, dev)
            lb = thv * layer_bytes_per_token_head(wv) + wv.batch * wv.nheads * wv.dstate * (wv.headdim + 1) * 4
            lf = thv * prefill_flops_per_token_head(wv.with_(chunk=LAYER_CHUNK_ROWS // wv.rank))
            variants[vname] = {"m3_layer_prefill": {
                "ms": ms_l, "tokens/s": wv.batch * wv.seqlen / (ms_l / 1e3), "groups": wv.groups,
                "GB/s": lb / ms_l / 1e6, "hbm_frac": lb / ms_l / 1e6 / HBM_PEAK_GBS,
                "TFLOP/s": lf / ms_l / 1e9, "mfma_frac": lf / ms_l / 1e9 / BF16_MFMA_PEAK_TFLOPS}}
            del inpv
            torch.cuda.empty_cache()
        variants["siso_varlen_packed"] = time_varlen(w, args.steps, args.warmup, dev)
        # the long-context workload's prefill: b = 1, L = 16384, MIMO R = 4, i.e. 64 (b, h) pairs,
        # so both paths split each sequence into segments that run in parallel
        wl4 = inputs.WORKLOADS["long_mimo4_b1_l16384"]
        inp4 = inputs.make_prefill_inputs(wl4, seed=0, device=dev)
        th4 = wl4.batch * wl4.seqlen * wl4.nheads
        ms_l4 = time_layer(wl4, inp4, LAYER_CHUNK_ROWS // wl4.rank, args.steps, args.warmup, dev)
        lb4 = th4 * layer_bytes_per_token_head(wl4) + wl4.batch * wl4.nheads * wl4.dstate * (wl4.headdim + 1) * 4
        wl4c = wl4.with_(chunk=LAYER_CHUNK_ROWS // wl4.rank)   # 32-row chunks, as above
        _, ms_s4, ms_b4, ms_p4 = time_prefill(wl4c, args.steps, args.warmup, dev, inp4)
        pb4 = th4 * prefill_bytes_per_token_head(wl4) + wl4.batch * wl4.nheads * wl4.dstate * wl4.headdim * 4
        toks4 = wl4.batch * wl4.seqlen
        variants["long_mimo4_b1_l16384"] = {
            "m3_layer_prefill": {"ms": ms_l4, "tokens/s": toks4 / (ms_l4 / 1e3), "GB/s": lb4 / ms_l4 / 1e6,
                                 "hbm_frac": lb4 / ms_l4 / 1e6 / HBM_PEAK_GBS,
                                 "chunk": LAYER_CHUNK_ROWS // wl4.rank},
            "two_calls": {"ms": ms_s4, "tokens/s": toks4 / (ms_s4 / 1e3), "bcnorm_rope_ms": ms_b4,
                          "chunk": wl4c.chunk},
            "m3_prefill": {"ms": ms_p4, "GB/s": pb4 / ms_p4 / 1e6, "hbm_frac": pb4 / ms_p4 / 1e6 / HBM_PEAK_GBS},
            "how": "sequence split into segments run in parallel (64 (b, h) pairs): every segment once, "
                   "the end states (and, fused, angles) chained, then each later segment's first steps "
                   "again from its true carry"}
        del inp4
        torch.cuda.empty_cache()
    # the step is one kernel: the fused layer kernel
    kd = kernels["m3_layer_prefill"]
    kname = "prefill_kernel<bf16,128,64,2,fused>"
    roofline = {"kernel": "m3_layer_prefill (%s)" % kname, "bound": "hbm", "achieved": round(kd["GB/s"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kd["GB/s"] / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(kname, w.name),
                "algorithmic_bytes_per_launch": kd["bytes"], "avg_launch_ms": round(kd["ms"], 5),
                "mfma_tflops": round(kd["TFLOP/s"], 1), "mfma_frac_of_bf16_peak": round(kd["mfma_frac"], 4),
                "copy_GB/s": round(copy["GB/s"], 1), "frac_of_copy": round(kd["GB/s"] / copy["GB/s"], 4)}

    decode = None
    if not args.no_decode:
        decode = {}
        for name in ("decode_b128_r1", "decode_b128_r4", "decode_b512_r1", "decode_b512_r4"):
            wd = inputs.WORKLOADS[name]
            ms_fused = time_layer_decode(wd, args.decode_steps, args.warmup, dev)
            ms_tok, ms_dbc, ms_dec = time_decode(wd, args.decode_steps, args.warmup, dev)
            dbytes = wd.batch * wd.nheads * decode_bytes_per_head(wd)
            fbytes = wd.batch * wd.nheads * layer_decode_bytes_per_head(wd)
            decode[name] = {"steps_per_s": 1e3 / ms_fused, "ms_per_step": ms_fused,
                            "layer_decode_step_GB/s": fbytes / ms_fused / 1e6,
                            "layer_decode_step_hbm_frac": fbytes / ms_fused / 1e6 / HBM_PEAK_GBS,
                            "layer_decode_step_bytes": fbytes,
                            "layer_decode_step_frac_of_copy": fbytes / ms_fused / 1e6 / copy["GB/s"],
                            "state_bytes": wd.batch * wd.nheads * wd.dstate * wd.headdim * 4,
                            "two_calls": {"steps_per_s": 1e3 / ms_tok, "ms_per_step": ms_tok,
                                          "decode_step_ms": ms_dec, "bcnorm_rope_ms": ms_dbc,
                                          "decode_step_GB/s": dbytes / ms_dec / 1e6,
                                          "decode_step_hbm_frac": dbytes / ms_dec / 1e6 / HBM_PEAK_GBS,
                                          "decode_step_bytes": dbytes}}
            torch.cuda.empty_cache()
        # small batch (the long-context workload's decode tail: b = 1, H = 64, R = 4)
        wl = inputs.WORKLOADS["long_mimo4_b1_l16384"]
        ms_e, ms_g = time_small_batch_decode(wl, args.decode_steps, dev)
        decode["decode_b1_r4"] = {"steps_per_s": 1e3 / ms_g, "ms_per_step": ms_g,
                                  "how": "m3_layer_decode_step, 16 steps per HIP graph replay",
                                  "eager": {"steps_per_s": 1e3 / ms_e, "ms_per_step": ms_e}}

    # backward pass of the layer core (gradients of every input), SISO and MIMO workloads
    backward = None
    if not args.no_backward:
        backward = {}
        # the last: raw B and C shared by all heads (dB, dC summed over the heads by a second kernel)
        for bname in ("siso_b8_l2048",) + (() if args.no_mimo else ("mimo4_b8_l2048", "siso_g1_b8_l2048")):
            wb = inputs.WORKLOADS[bname]
            t = time_backward(wb, args.steps, args.warmup, dev)
            thb = wb.batch * wb.seqlen * wb.nheads
            rows = 64 if wb.io == "bf16" else 32
            bb = thb * backward_bytes_per_token_head(wb) + 3 * wb.batch * wb.nheads * wb.dstate * wb.headdim * 4
            bf = thb * backward_flops_per_token_head(wb, rows)
            ms = t["m3_layer_backward"]
            backward[bname] = {"ms": ms, "tokens/s": wb.batch * wb.seqlen / (ms / 1e3),
                               "chunk_states_ms": t["m3_layer_chunk_states"],
                               "bytes": bb, "GB/s": bb / ms / 1e6, "hbm_frac": bb / ms / 1e6 / HBM_PEAK_GBS,
                               "TFLOP/s": bf / ms / 1e9, "mfma_frac": bf / ms / 1e9 / BF16_MFMA_PEAK_TFLOPS,
                               "chunk_rows": rows}

    cpu = None
    cpu_more = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, args.cpu_heads)
        cpu_more = more_cpu_baselines(w, inp)

    line = {
        "metric": "prefill tokens/s and B=128 decode steps/s per Mamba-3 layer; % of roofline",
        "value": tokens / (ms_step / 1e3),
        "warm_s": WARM_S,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the SISO b8 L2048 layer workload)",
        "config": {"workload": "siso_b8_l2048: m3_layer_prefill (BCNorm + bias + rotation + chunked "
                               "scan in one kernel), b=8 L=2048 H=64 P=64 N=128 R=1 chunk=%d, bf16 io, "
                               "fp32 state" % kernels["m3_layer_prefill"]["chunk"],
                   "batch": w.batch, "seq_len": w.seqlen, "nheads": w.nheads, "headdim": w.headdim,
                   "dstate": w.dstate, "rank": w.rank, "chunk": kernels["m3_layer_prefill"]["chunk"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "cpu_baselines": cpu_more,
        "mimo4_b8_l2048": mimo,
        "table3_grid": table3,
        "variants": variants,
        "decode": decode,
        "backward": backward,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
