"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function that
include/m3scan.h declares, and each validation error is reported with its status and message.
Validation runs before any device access, so every call here returns before touching a GPU."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from state_space_sequence_m3_amd import m3scan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m3scan.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(m3_[a-z_]+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("m3_bcnorm_rope", "m3_prefill", "m3_decode_step", "m3_last_error",
              "m3_bcnorm_rope_workspace_bytes", "m3_prefill_workspace_bytes", "m3_version"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = m3scan.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", m3scan.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(m3_[a-z_]+)\b", out))
    assert set(declared_functions()) <= exported
    assert set(m3scan.EXPORTED) == set(declared_functions())


def test_version():
    assert "gfx950" in m3scan.version()


def _dims(**kw):
    d = dict(batch=2, seqlen=8, nheads=3, headdim=64, dstate=128, rank=1, chunk=0, io=m3scan.M3_BF16,
             bcnorm=True, eps=1e-5)
    d.update(kw)
    return m3scan.make_dims(**d)


P = ctypes.c_void_p
ALIGNED = 0x10000        # fake, aligned device addresses: validation never dereferences them


def _ptrs(n, base=ALIGNED, stride=1 << 24):
    return [P(base + i * stride) for i in range(n)]


def _prefill(dims, ptrs):
    lib = m3scan.load()
    return lib.m3_prefill(ctypes.byref(dims), *ptrs, 0, None)


def _prefill_args():
    # x, Bbar, Cbar, dt, A, lam, w_out, h_in, Bbar_prev, x_prev, y, h_out, Bbar_last, x_last, ws
    p = _ptrs(15)
    for i in (6, 7, 8, 9, 12, 13, 14):
        p[i] = None
    return p


def test_prefill_null_pointer():
    p = _prefill_args()
    p[0] = None
    assert _prefill(_dims(), p) == m3scan.M3_E_NULL
    assert "x is NULL" in m3scan.last_error()


def test_prefill_bad_dims():
    assert _prefill(_dims(dstate=127), _prefill_args()) == m3scan.M3_E_DIMS
    assert _prefill(_dims(batch=-1), _prefill_args()) == m3scan.M3_E_DIMS
    assert _prefill(_dims(rank=0), _prefill_args()) == m3scan.M3_E_DIMS


def test_prefill_bad_dtype():
    assert _prefill(_dims(io=7), _prefill_args()) == m3scan.M3_E_DTYPE


def test_prefill_unsupported_shape():
    assert _prefill(_dims(headdim=32), _prefill_args()) == m3scan.M3_E_UNSUPPORTED
    assert _prefill(_dims(rank=3, chunk=16), _prefill_args()) == m3scan.M3_E_UNSUPPORTED
    assert _prefill(_dims(chunk=128), _prefill_args()) == m3scan.M3_E_UNSUPPORTED
    assert "no kernel" in m3scan.last_error()


def test_prefill_sequence_span_limit():
    """A sequence whose rows span 2^31 bytes or more per tensor is rejected (32-bit offsets)."""
    # 2^31 / (64 heads * 128 * 2 bytes) = 131072 steps; the 3 chunks of margin push it over
    assert _prefill(_dims(seqlen=131072 - 64, nheads=64), _prefill_args()) == m3scan.M3_E_DIMS
    assert "2^31" in m3scan.last_error()


def test_prefill_misaligned():
    p = _prefill_args()
    p[1] = P(ALIGNED + (1 << 24) + 8)
    assert _prefill(_dims(), p) == m3scan.M3_E_ALIGN


def test_fp32_pointers_need_four_byte_alignment():
    """A and w_out are fp32 in every call: a 2-byte-aligned pointer is refused even when the io
    type is bf16 (2-byte elements)."""
    p = _prefill_args()
    p[4] = P(ALIGNED + 4 * (1 << 24) + 2)            # A
    assert _prefill(_dims(), p) == m3scan.M3_E_ALIGN and "A" in m3scan.last_error()
    p = _prefill_args()
    p[6] = P(ALIGNED + 6 * (1 << 24) + 2)            # w_out
    assert _prefill(_dims(), p) == m3scan.M3_E_ALIGN and "w_out" in m3scan.last_error()
    lib = m3scan.load()
    q = _ptrs(11)                                     # h, Bbar_prev, x_prev, x, Bbar, Cbar, dt, A, lam, w_out, y
    call = lambda qq: lib.m3_decode_step(ctypes.byref(_dims(seqlen=1)), *qq, None)
    r = list(q)
    r[7] = P(q[7].value + 2)
    assert call(r) == m3scan.M3_E_ALIGN and "A" in m3scan.last_error()
    r = list(q)
    r[9] = P(q[9].value + 2)
    assert call(r) == m3scan.M3_E_ALIGN and "w_out" in m3scan.last_error()


def test_prefill_output_overlapping_input():
    p = _prefill_args()
    p[10] = p[0]    # y on top of x
    assert _prefill(_dims(), p) == m3scan.M3_E_ALIAS


def test_prefill_valid_call_without_gpu_reports_no_device():
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU driver is present; this checks the no-device path")
    assert _prefill(_dims(), _prefill_args()) == m3scan.M3_E_NODEVICE


def test_bcnorm_rope_errors():
    lib = m3scan.load()
    # B, C, dt, theta, normw_B, normw_C, bias_B, bias_C, phi_in, Bbar, Cbar, phi_out, ws
    p = _ptrs(13)
    for i in (4, 5, 6, 7, 8, 12):
        p[i] = None
    d = _dims()
    call = lambda dims, q, wsb=0: lib.m3_bcnorm_rope(ctypes.byref(dims), *q, wsb, None)
    q = list(p)
    q[3] = None
    assert call(d, q) == m3scan.M3_E_NULL
    assert call(_dims(dstate=96), p) == m3scan.M3_E_UNSUPPORTED
    long = _dims(seqlen=4096)
    # one angle row of N/2 floats per quarter of each 512-step segment
    assert m3scan.bcnorm_rope_workspace_bytes(long) == 2 * 3 * 8 * 4 * 64 * 4
    assert call(long, p) == m3scan.M3_E_WORKSPACE
    q = list(p)
    q[9] = q[0]
    assert call(d, q) == m3scan.M3_E_ALIAS
    # phi_out may be the phi_in buffer (angle carried in place) but not partly overlap it.  The
    # call without its workspace stops at the workspace check, after the alias check, so it
    # never reaches a device.
    q = list(p)
    q[8] = q[11]
    assert call(long, q) == m3scan.M3_E_WORKSPACE
    q[8] = P(q[11].value + 8)
    assert call(long, q) == m3scan.M3_E_ALIAS


def test_decode_errors():
    lib = m3scan.load()
    # h, Bbar_prev, x_prev, x, Bbar, Cbar, dt, A, lam, w_out, y
    p = _ptrs(11)
    p[9] = None
    call = lambda dims, q: lib.m3_decode_step(ctypes.byref(dims), *q, None)
    assert call(_dims(seqlen=2), p) == m3scan.M3_E_DIMS
    assert call(_dims(seqlen=1, headdim=48), p) == m3scan.M3_E_UNSUPPORTED
    q = list(p)
    q[0] = P(ALIGNED + 4)
    assert call(_dims(seqlen=1), q) == m3scan.M3_E_ALIGN
    q = list(p)
    q[10] = q[0]
    assert call(_dims(seqlen=1), q) == m3scan.M3_E_ALIAS


def test_workspace_sizes():
    assert m3scan.prefill_workspace_bytes(_dims()) == 0
    assert m3scan.bcnorm_rope_workspace_bytes(_dims(seqlen=512)) == 0
    assert m3scan.bcnorm_rope_workspace_bytes(_dims(seqlen=513)) == 2 * 3 * 2 * 4 * 64 * 4


def test_sequence_split_workspace_sizes():
    """The split plan of m3_prefill / m3_layer_prefill (this host has no GPU: 256 compute units
    are assumed, so the split aims at 512 workgroups)."""
    kw = dict(batch=1, seqlen=16384, nheads=64, rank=4, chunk=16)
    # 64 pairs -> 8 segments of 2048 steps: end states [64, 8, 128, 64] f32, last Bbar rows
    # [64, 8, 4, 128] bf16, log2 decays [64, 8] f32, steps of each segment to rerun [64, 8] int32
    state, bbar, decay, fix = 64 * 8 * 128 * 64 * 4, 64 * 8 * 4 * 128 * 2, 64 * 8 * 4, 64 * 8 * 4
    assert m3scan.prefill_workspace_bytes(_dims(**kw)) == state + bbar + decay + fix
    # fused, chunk 8 (32 rows): plus each segment's end angle from the first pass and its true
    # start angle (64 angles each)
    fused = dict(kw, chunk=8)
    assert m3scan.layer_prefill_workspace_bytes(_dims(**fused)) == \
        state + bbar + decay + fix + 2 * 64 * 8 * 64 * 4
    # enough pairs, too short a sequence, or a chunk that does not divide 512: no split
    assert m3scan.prefill_workspace_bytes(_dims(batch=8, seqlen=2048, nheads=64)) == 0
    assert m3scan.prefill_workspace_bytes(_dims(batch=1, seqlen=2047, nheads=64)) == 0
    assert m3scan.prefill_workspace_bytes(_dims(batch=1, seqlen=16384, nheads=64, chunk=48)) == 0
    assert m3scan.layer_prefill_workspace_bytes(_dims(batch=8, seqlen=16384, nheads=64)) == 0
    # a ragged tail: 3000 steps over 2 pairs -> at most 2 segments (1024 steps each at least), of
    # 1536 steps (a multiple of 512); workspace sections are padded to 256 bytes
    r = lambda n: (n + 255) // 256 * 256
    assert m3scan.prefill_workspace_bytes(_dims(batch=1, seqlen=3000, nheads=2, rank=1, chunk=32)) == \
        r(2 * 2 * 128 * 64 * 4) + r(2 * 2 * 1 * 128 * 2) + r(2 * 2 * 4) + r(2 * 2 * 4)


def test_binding_raises_without_the_library(tmp_path, monkeypatch):
    monkeypatch.setattr(m3scan, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        m3scan.load(str(tmp_path / "missing.so"))


def test_layer_prefill_errors():
    lib = m3scan.load()
    # x, B, C, dt, theta, normw_B, normw_C, bias_B, bias_C, A, lam, w_out, phi_in, h_in,
    # Bbar_prev, x_prev, y, h_out, phi_out, Bbar_last, x_last, ws
    p = _ptrs(22)
    for i in (5, 6, 7, 8, 11, 12, 13, 14, 15, 19, 20, 21):
        p[i] = None
    call = lambda dims, q: lib.m3_layer_prefill(ctypes.byref(dims), *q, 0, None)
    q = list(p)
    q[4] = None                                   # theta is required
    assert call(_dims(chunk=32), q) == m3scan.M3_E_NULL
    assert "theta is NULL" in m3scan.last_error()
    assert call(_dims(chunk=48), p) == m3scan.M3_E_UNSUPPORTED   # 48-row tiles are two-call only
    assert call(_dims(headdim=32), p) == m3scan.M3_E_UNSUPPORTED
    q = list(p)
    q[18] = q[4]                                  # phi_out on top of theta
    assert call(_dims(chunk=32), q) == m3scan.M3_E_ALIAS
    q = list(p)
    q[12], q[18] = P(q[18].value + 4), q[18]      # phi_in partly overlapping phi_out
    assert call(_dims(chunk=32), q) == m3scan.M3_E_ALIAS


def test_layer_decode_step_errors():
    lib = m3scan.load()
    # h, phi, Bbar_prev, x_prev, x, B, C, dt, theta, normw_B, normw_C, bias_B, bias_C, A, lam,
    # w_out, y, Bbar_out
    p = _ptrs(18)
    for i in (9, 10, 11, 12, 15):
        p[i] = None
    call = lambda dims, q: lib.m3_layer_decode_step(ctypes.byref(dims), *q, None)
    assert call(_dims(seqlen=3), p) == m3scan.M3_E_DIMS
    q = list(p)
    q[17] = None
    assert call(_dims(seqlen=1), q) == m3scan.M3_E_NULL
    q = list(p)
    q[17] = q[2]                                  # rotated B written over Bbar_prev
    assert call(_dims(seqlen=1), q) == m3scan.M3_E_ALIAS
    assert call(_dims(seqlen=1, rank=16), p) == m3scan.M3_E_UNSUPPORTED


def test_layer_prefill_varlen_needs_offsets():
    lib = m3scan.load()
    # cu_seqlens, then the m3_layer_prefill pointers without the workspace
    p = _ptrs(22)
    for i in (6, 7, 8, 9, 12, 13, 14, 15, 16, 20, 21):
        p[i] = None
    call = lambda dims, q: lib.m3_layer_prefill_varlen(ctypes.byref(dims), *q, None)
    q = list(p)
    q[0] = None
    assert call(_dims(chunk=32), q) == m3scan.M3_E_NULL
    assert "cu_seqlens" in m3scan.last_error()
    q = list(p)
    q[0] = P(ALIGNED + 2)
    assert call(_dims(chunk=32), q) == m3scan.M3_E_ALIGN
    q = list(p)
    q[0] = q[17]                                  # offsets inside y
    assert call(_dims(chunk=32), q) == m3scan.M3_E_ALIAS


def _bwd_args(ws_bytes_ok=True):
    # x B C dt theta normw_B normw_C bias_B bias_C A lam w_out phi_in h_in Bbar_prev x_prev
    # dy dh_out dphi_out | dx dB dC ddt dtheta dA dlam dnormw_B dnormw_C dbias_B dbias_C dw_out
    # dphi_in dh_in dBbar_prev dx_prev | workspace
    p = _ptrs(36)
    for i in (5, 6, 7, 8, 11, 12, 13, 14, 15, 17, 18, 26, 27, 28, 29, 30, 33, 34):
        p[i] = None
    return p


def _bwd(dims, p, ws_bytes):
    return m3scan.load().m3_layer_backward(ctypes.byref(dims), *p, ws_bytes, None)


def test_layer_backward_sizes():
    d = _dims(seqlen=130)
    assert m3scan.layer_backward_chunk(d) == 64
    assert m3scan.layer_backward_chunk(_dims(rank=4)) == 16
    assert m3scan.layer_backward_chunk(_dims(io=m3scan.M3_F32)) == 32
    assert m3scan.layer_backward_chunk(_dims(rank=8)) == 0
    # states (3 chunks) + angles + per-(b, h) partial sums + per-chunk step sums (5 per step and
    # 3 per chunk), each rounded up to 256 bytes
    st = 2 * 3 * 3 * 64 * 128 * 2
    ph = 2 * 3 * 3 * 64 * 4
    part = 2 * 3 * (1 + 64 + 2 * 128 + 2 * 128) * 4
    steps = 2 * 3 * 3 * (5 * 64 + 3) * 4
    r = lambda n: (n + 255) // 256 * 256
    assert m3scan.layer_backward_workspace_bytes(d) == r(st) + r(ph) + r(part) + r(steps)
    assert m3scan.layer_backward_workspace_bytes(_dims(rank=8)) == 0


def test_layer_backward_errors():
    d = _dims()
    need = m3scan.layer_backward_workspace_bytes(d)
    assert _bwd(d, _bwd_args(), need) == m3scan.M3_E_NODEVICE   # valid: stops at the device check
    p = _bwd_args()
    p[0] = None
    assert _bwd(d, p, need) == m3scan.M3_E_NULL and "x is NULL" in m3scan.last_error()
    p = _bwd_args()
    p[16] = None
    assert _bwd(d, p, need) == m3scan.M3_E_NULL and "dy is NULL" in m3scan.last_error()
    assert _bwd(d, _bwd_args(), need - 1) == m3scan.M3_E_WORKSPACE
    p = _bwd_args()
    p[35] = None
    assert _bwd(d, p, need) == m3scan.M3_E_WORKSPACE
    assert _bwd(_dims(rank=8), _bwd_args(), 1 << 30) == m3scan.M3_E_UNSUPPORTED
    assert _bwd(_dims(chunk=5), _bwd_args(), need) == m3scan.M3_E_UNSUPPORTED
    assert _bwd(_dims(chunk=64), _bwd_args(), need) == m3scan.M3_E_NODEVICE
    p = _bwd_args()
    p[19] = P(p[19].value + 2)
    assert _bwd(d, p, need) == m3scan.M3_E_ALIGN and "dx" in m3scan.last_error()
    p = _bwd_args()
    p[19] = p[0]
    assert _bwd(d, p, need) == m3scan.M3_E_ALIAS
    p = _bwd_args()
    p[20] = p[35]
    assert _bwd(d, p, need) == m3scan.M3_E_ALIAS and "workspace" in m3scan.last_error()


def test_layer_chunk_states_errors():
    lib = m3scan.load()
    d = _dims()
    # x B dt theta normw_B bias_B A lam phi_in h_in Bbar_prev x_prev states phis
    p = _ptrs(14)
    for i in (4, 5, 8, 9, 10, 11):
        p[i] = None
    assert lib.m3_layer_chunk_states(ctypes.byref(d), *p, None) == m3scan.M3_E_NODEVICE
    q = list(p)
    q[12] = None
    assert lib.m3_layer_chunk_states(ctypes.byref(d), *q, None) == m3scan.M3_E_NULL
    assert lib.m3_layer_chunk_states(ctypes.byref(_dims(headdim=32)), *p, None) == m3scan.M3_E_UNSUPPORTED
    q = list(p)
    q[12] = q[0]
    assert lib.m3_layer_chunk_states(ctypes.byref(d), *q, None) == m3scan.M3_E_ALIAS


def test_head_groups_validation():
    """dims->ngroups: 0 or a divisor of nheads; only the calls that take raw B and C accept G < H
    (m3_prefill and m3_decode_step take per-head Bbar and Cbar)."""
    lib = m3scan.load()
    assert ctypes.sizeof(m3scan.M3Dims) == 80
    p = _ptrs(22)
    for i in (5, 6, 7, 8, 11, 12, 13, 14, 15, 19, 20, 21):
        p[i] = None
    layer = lambda dims: lib.m3_layer_prefill(ctypes.byref(dims), *p, 0, None)
    base = dict(nheads=4, chunk=32)
    assert layer(_dims(groups=3, **base)) == m3scan.M3_E_DIMS            # 3 does not divide 4
    assert "ngroups" in m3scan.last_error()
    assert layer(_dims(groups=8, **base)) == m3scan.M3_E_DIMS            # more slots than heads
    assert layer(_dims(groups=-1, **base)) == m3scan.M3_E_DIMS
    for g in (0, 1, 2, 4):                                               # valid: stops at the device
        assert layer(_dims(groups=g, **base)) == m3scan.M3_E_NODEVICE
    assert _prefill(_dims(groups=2, nheads=4), _prefill_args()) == m3scan.M3_E_DIMS
    assert "per-head" in m3scan.last_error()
    assert _prefill(_dims(groups=4, nheads=4), _prefill_args()) == m3scan.M3_E_NODEVICE
    dec = _ptrs(11)
    dec[9] = None
    assert lib.m3_decode_step(ctypes.byref(_dims(seqlen=1, nheads=4, groups=1)), *dec, None) == m3scan.M3_E_DIMS
    # raw B, C of G slots are smaller than per-head ones: an output right after a G-slot B is legal
    dims = _dims(groups=1, **base)
    q = list(p)
    nB = 2 * 8 * 1 * 1 * 128 * 2                                         # b L G R N bf16
    q[16] = P(q[1].value + nB)                                           # y just past B
    assert layer(dims) == m3scan.M3_E_NODEVICE
    assert lib.m3_layer_prefill(ctypes.byref(dims), *q, 0, None) == m3scan.M3_E_NODEVICE
    q[16] = P(q[1].value + nB - 16)                                      # y overlapping B's end
    assert lib.m3_layer_prefill(ctypes.byref(dims), *q, 0, None) == m3scan.M3_E_ALIAS


def test_head_groups_backward_workspace():
    """With G < H the backward workspace adds per-head dB and dC rows (b L H R N io each)."""
    d = _dims(seqlen=130, nheads=4)
    g = _dims(seqlen=130, nheads=4, groups=2)
    r = lambda n: (n + 255) // 256 * 256
    per_head = 2 * 130 * 4 * 1 * 128 * 2
    assert m3scan.layer_backward_workspace_bytes(g) == m3scan.layer_backward_workspace_bytes(d) + 2 * r(per_head)
    assert m3scan.layer_backward_workspace_bytes(_dims(seqlen=130, nheads=4, groups=4)) == \
        m3scan.layer_backward_workspace_bytes(d)
    assert m3scan.layer_backward_workspace_bytes(_dims(nheads=4, groups=3)) == 0


def test_noalloc_rejects_a_split_beyond_its_scratch():
    """m3_layer_prefill_noalloc: dims whose sequence split needs more than the library's scratch
    array are refused before any device work (the split plan assumes 256 compute units when no
    device answers)."""
    lib = m3scan.load()
    # 500 (b, h) pairs, 2 segments of 1024 steps: 32.8 MB of states + rotated B + angles > 32 MiB
    d = _dims(batch=2, seqlen=2048, nheads=250, rank=4, chunk=8)
    assert m3scan.layer_prefill_workspace_bytes(d) > m3scan.NOALLOC_SCRATCH_BYTES
    # x, B, C, dt, theta, normw_B, normw_C, bias_B, bias_C, A, lam, w_out, phi_in, h_in, Bbar_prev,
    # x_prev, y, h_out, phi_out, Bbar_last, x_last
    p = _ptrs(21)
    for i in (5, 6, 7, 8, 11, 12, 13, 14, 15, 19, 20):   # optional pointers
        p[i] = None
    st = lib.m3_layer_prefill_noalloc(ctypes.byref(d), *p, None)
    assert st == m3scan.M3_E_WORKSPACE and "scratch" in m3scan.last_error()
    # a call that does not split needs no scratch: it gets past the size check (and then stops at
    # the device check here)
    small = _dims(batch=8, seqlen=64, nheads=64, rank=1, chunk=32)
    assert m3scan.layer_prefill_workspace_bytes(small) == 0
    st = lib.m3_layer_prefill_noalloc(ctypes.byref(small), *p, None)
    if not os.path.exists("/dev/kfd"):
        assert st == m3scan.M3_E_NODEVICE
