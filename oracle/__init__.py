"""fp64 CPU oracle for the Mamba-3 SSM layer core.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the HIP library and it is
never fed a value that the HIP library produced.

The arithmetic lives in ``m3_oracle.c`` (plain C, double precision, one time step after another);
this module only converts arrays to contiguous float64, calls the C functions through ctypes, and
composes them.  Every function cites the passage it follows:

* ``bcnorm_rope``   BCNorm + head bias (papernotes.org, key design item 4) and the cumulative
                    rotation of B and C (aipaper.cc section 4.2, Proposition 3; rotation matrix
                    of metaphor-xennon section 2.2).
* ``scan``          exponential-trapezoidal recurrence (aipaper.cc section 4.1, Proposition 1)
                    with the MIMO rank-R update (aipaper.cc section 4.3).
* ``layer``         the two composed: the layer core from raw B and C to y and the final state.
* ``decode_step``   the same composition for one new token, with the state, the angle and the
                    previous-token factors carried in.
* ``scan_backward``, ``bcnorm_rope_backward``, ``layer_backward``
                    exact gradients of the three forward functions above (reverse-mode through
                    the same steps in reverse order; the pages define no backward pass, so the
                    gradient of the forward definition is the definition followed).
* ``heads_from_groups``, ``groups_from_heads``
                    raw B and C with G < H head slots, shared by groups of H / G consecutive
                    heads.  The pages define B and C per head; the shared layout is defined here
                    as its expansion (head h reads slot h // (H / G)), and the gradient of a
                    shared row is the sum of the gradients of the heads that read it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB = os.path.join(_HERE, "libm3oracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (strict IEEE double, no fast-math).  Returns the .so path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-fno-fast-math",
             "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    lib.m3o_bcnorm_rope.restype = None
    lib.m3o_bcnorm_rope.argtypes = [_I64] * 5 + [ctypes.c_int, ctypes.c_double] + [_D] * 12
    lib.m3o_scan.restype = None
    lib.m3o_scan.argtypes = [_I64] * 6 + [_D] * 12
    lib.m3o_scan_backward.restype = None
    lib.m3o_scan_backward.argtypes = [_I64] * 6 + [_D] * 22
    lib.m3o_bcnorm_rope_backward.restype = None
    lib.m3o_bcnorm_rope_backward.argtypes = [_I64] * 5 + [ctypes.c_int, ctypes.c_double] + [_D] * 21
    lib.m3o_num_threads.restype = ctypes.c_int
    lib.m3o_num_threads.argtypes = []
    lib.m3o_set_num_threads.restype = None
    lib.m3o_set_num_threads.argtypes = [ctypes.c_int]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(_LIB)
    return _lib


def _f64(a):
    """Contiguous float64 copy of an array-like (torch CPU tensors included), or None."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: exact upcast of bf16 / fp32 values
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_D)


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else the cores it may run on)."""
    return int(_load().m3o_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for the oracle's later calls (the arithmetic does not depend on it)."""
    _load().m3o_set_num_threads(int(n))


def heads_from_groups(v, H):
    """Raw B or C [b, L, G, R, N] with G head slots -> [b, L, H, R, N]: head h reads slot
    h // (H // G), so each slot serves the H / G consecutive heads of its group."""
    v = _f64(v)
    G = v.shape[2]
    assert G >= 1 and H % G == 0
    return np.repeat(v, H // G, axis=2)


def groups_from_heads(g, G):
    """Gradient of ``heads_from_groups``: [b, L, H, R, N] -> [b, L, G, R, N], each slot's
    gradient the sum over the heads of its group."""
    b, L, H, R, N = g.shape
    return g.reshape(b, L, G, H // G, R, N).sum(axis=3)


def bcnorm_rope(B, C, dt, theta, normw_B=None, normw_C=None, bias_B=None, bias_C=None,
                phi_in=None, bcnorm=True, eps=1e-5, lib=None):
    """BCNorm, bias and cumulative rotation for B, C of shape [b, L, H, R, N] (or [b, L, G, R, N]
    with head slots shared by groups of heads: expanded by ``heads_from_groups``).

    dt is [b, L, H], theta is [b, L, H, N/2], normw_* are [H, N], bias_* are [H, R, N] and phi_in
    is [b, H, N/2] (each optional except B, C, dt, theta).  Returns (Bbar, Cbar, phi_out) with
    Bbar, Cbar [b, L, H, R, N] and phi_out the final cumulative angle, not reduced modulo 2*pi.
    """
    B, C, dt, theta = _f64(B), _f64(C), _f64(dt), _f64(theta)
    if B.shape[2] != dt.shape[2]:
        B, C = heads_from_groups(B, dt.shape[2]), heads_from_groups(C, dt.shape[2])
    nb, L, H, R, N = B.shape
    assert C.shape == B.shape and dt.shape == (nb, L, H) and theta.shape == (nb, L, H, N // 2)
    assert N % 2 == 0
    normw_B, normw_C, bias_B, bias_C, phi_in = map(_f64, (normw_B, normw_C, bias_B, bias_C, phi_in))
    for w in (normw_B, normw_C):
        assert w is None or w.shape == (H, N)
    for bb in (bias_B, bias_C):
        assert bb is None or bb.shape == (H, R, N)
    assert phi_in is None or phi_in.shape == (nb, H, N // 2)
    Bbar = np.empty_like(B)
    Cbar = np.empty_like(C)
    phi_out = np.empty((nb, H, N // 2), dtype=np.float64)
    (lib or _load()).m3o_bcnorm_rope(nb, L, H, R, N, int(bool(bcnorm)), float(eps),
                            _ptr(B), _ptr(C), _ptr(dt), _ptr(theta),
                            _ptr(normw_B), _ptr(normw_C), _ptr(bias_B), _ptr(bias_C),
                            _ptr(phi_in), _ptr(Bbar), _ptr(Cbar), _ptr(phi_out))
    return Bbar, Cbar, phi_out


def scan(x, Bbar, Cbar, dt, A, lam, w_out=None, h_in=None, Bbar_prev=None, x_prev=None,
         lib=None):
    """Exponential-trapezoidal MIMO recurrence on rotated B, C.

    x is [b, L, H, R, P]; Bbar, Cbar are [b, L, H, R, N]; dt, lam are [b, L, H]; A is [H];
    w_out is [H, R, P] or None; h_in is [b, H, N, P]; Bbar_prev is [b, H, R, N]; x_prev is
    [b, H, R, P].  Returns (y, h_out): y is [b, L, H, P] with w_out, else [b, L, H, R, P].
    """
    x, Bbar, Cbar, dt, A, lam = map(_f64, (x, Bbar, Cbar, dt, A, lam))
    nb, L, H, R, P = x.shape
    N = Bbar.shape[-1]
    assert Bbar.shape == (nb, L, H, R, N) and Cbar.shape == Bbar.shape
    assert dt.shape == (nb, L, H) and lam.shape == (nb, L, H) and A.shape == (H,)
    w_out, h_in, Bbar_prev, x_prev = map(_f64, (w_out, h_in, Bbar_prev, x_prev))
    assert w_out is None or w_out.shape == (H, R, P)
    assert h_in is None or h_in.shape == (nb, H, N, P)
    assert Bbar_prev is None or Bbar_prev.shape == (nb, H, R, N)
    assert x_prev is None or x_prev.shape == (nb, H, R, P)
    y = np.empty((nb, L, H, P) if w_out is not None else (nb, L, H, R, P), dtype=np.float64)
    h_out = np.empty((nb, H, N, P), dtype=np.float64)
    (lib or _load()).m3o_scan(nb, L, H, R, P, N, _ptr(x), _ptr(Bbar), _ptr(Cbar), _ptr(dt), _ptr(A),
                     _ptr(lam), _ptr(w_out), _ptr(h_in), _ptr(Bbar_prev), _ptr(x_prev),
                     _ptr(y), _ptr(h_out))
    return y, h_out


def layer(inp: dict, bcnorm=True, eps=1e-5, mix=True, lib=None):
    """Layer core from raw inputs: ``bcnorm_rope`` then ``scan``.

    ``inp`` holds arrays under the names x, B, C, dt, A, lam, theta and optionally normw_B,
    normw_C, bias_B, bias_C, w_out, phi_in, h_in, Bbar_prev, x_prev.  Returns a dict with y,
    h_out, phi_out, Bbar, Cbar, Bbar_last (= Bbar[:, -1]) and x_last (= x[:, -1]).
    """
    g = inp.get
    Bbar, Cbar, phi_out = bcnorm_rope(g("B"), g("C"), g("dt"), g("theta"), g("normw_B"),
                                      g("normw_C"), g("bias_B"), g("bias_C"), g("phi_in"),
                                      bcnorm=bcnorm, eps=eps, lib=lib)
    y, h_out = scan(g("x"), Bbar, Cbar, g("dt"), g("A"), g("lam"),
                    g("w_out") if mix else None, g("h_in"), g("Bbar_prev"), g("x_prev"), lib=lib)
    x = _f64(g("x"))
    return {"y": y, "h_out": h_out, "phi_out": phi_out, "Bbar": Bbar, "Cbar": Cbar,
            "Bbar_last": Bbar[:, -1].copy(), "x_last": x[:, -1].copy()}


def decode_step(state: dict, tok: dict, consts: dict, bcnorm=True, eps=1e-5, mix=True,
                lib=None):
    """One decode step = the layer core with L = 1 and everything carried.

    ``state`` holds h [b, H, N, P], phi [b, H, N/2], Bbar_prev [b, H, R, N], x_prev [b, H, R, P];
    ``tok`` holds the new token's x [b, H, R, P], B, C [b, H, R, N] (or [b, G, R, N]), dt, lam [b, H] and
    theta [b, H, N/2]; ``consts`` holds A and optionally normw_B, normw_C, bias_B, bias_C, w_out.
    Returns (y, new_state) with y [b, H, P] (mixed) or [b, H, R, P].
    """
    inp = dict(consts)
    for k in ("x", "B", "C", "dt", "lam", "theta"):
        inp[k] = _f64(tok[k])[:, None]
    inp["h_in"] = state["h"]
    inp["phi_in"] = state["phi"]
    inp["Bbar_prev"] = state["Bbar_prev"]
    inp["x_prev"] = state["x_prev"]
    out = layer(inp, bcnorm=bcnorm, eps=eps, mix=mix, lib=lib)
    new_state = {"h": out["h_out"], "phi": out["phi_out"], "Bbar_prev": out["Bbar_last"],
                 "x_prev": out["x_last"]}
    return out["y"][:, 0], new_state


def scan_backward(x, Bbar, Cbar, dt, A, lam, dy, w_out=None, h_in=None, Bbar_prev=None,
                  x_prev=None, dh_out=None, lib=None):
    """Gradients of ``scan`` for the cotangents dy (layout of y) and dh_out (layout of h_out,
    None = 0).  Returns a dict: x, Bbar, Cbar, dt, lam (layouts of those inputs), A [H], w_out
    [H, R, P] (None without mixing), h_in [b, H, N, P], and Bbar_prev, x_prev (None unless both
    were given).  Gradients of per-head parameters are summed over the batch."""
    x, Bbar, Cbar, dt, A, lam, dy = map(_f64, (x, Bbar, Cbar, dt, A, lam, dy))
    nb, L, H, R, P = x.shape
    N = Bbar.shape[-1]
    w_out, h_in, Bbar_prev, x_prev, dh_out = map(_f64, (w_out, h_in, Bbar_prev, x_prev, dh_out))
    assert dy.shape == ((nb, L, H, P) if w_out is not None else (nb, L, H, R, P))
    assert dh_out is None or dh_out.shape == (nb, H, N, P)
    carry = Bbar_prev is not None and x_prev is not None
    g = {"x": np.empty_like(x), "Bbar": np.empty_like(Bbar), "Cbar": np.empty_like(Cbar),
         "dt": np.empty_like(dt), "lam": np.empty_like(lam), "A": np.empty_like(A),
         "w_out": np.empty_like(w_out) if w_out is not None else None,
         "h_in": np.empty((nb, H, N, P)),
         "Bbar_prev": np.empty((nb, H, R, N)) if carry else None,
         "x_prev": np.empty((nb, H, R, P)) if carry else None}
    (lib or _load()).m3o_scan_backward(
        nb, L, H, R, P, N, _ptr(x), _ptr(Bbar), _ptr(Cbar), _ptr(dt), _ptr(A), _ptr(lam),
        _ptr(w_out), _ptr(h_in), _ptr(Bbar_prev), _ptr(x_prev), _ptr(dy), _ptr(dh_out),
        _ptr(g["x"]), _ptr(g["Bbar"]), _ptr(g["Cbar"]), _ptr(g["dt"]), _ptr(g["A"]),
        _ptr(g["lam"]), _ptr(g["w_out"]), _ptr(g["h_in"]), _ptr(g["Bbar_prev"]),
        _ptr(g["x_prev"]))
    return g


def bcnorm_rope_backward(B, C, dt, theta, dBbar, dCbar, normw_B=None, normw_C=None, bias_B=None,
                         bias_C=None, phi_in=None, dphi_out=None, bcnorm=True, eps=1e-5, lib=None):
    """Gradients of ``bcnorm_rope`` for the cotangents dBbar, dCbar (layout of Bbar) and dphi_out
    ([b, H, N/2], None = 0).  Returns a dict: B, C, dt (the rotation's share only), theta,
    phi_in, and normw_B, normw_C [H, N], bias_B, bias_C [H, R, N] summed over the batch (zero
    for normw without BCNorm)."""
    B, C, dt, theta, dBbar, dCbar = map(_f64, (B, C, dt, theta, dBbar, dCbar))
    nb, L, H, R, N = B.shape
    normw_B, normw_C, bias_B, bias_C, phi_in, dphi_out = map(
        _f64, (normw_B, normw_C, bias_B, bias_C, phi_in, dphi_out))
    assert dBbar.shape == B.shape and dCbar.shape == B.shape
    assert dphi_out is None or dphi_out.shape == (nb, H, N // 2)
    g = {"B": np.empty_like(B), "C": np.empty_like(C), "dt": np.empty_like(dt),
         "theta": np.empty_like(theta), "phi_in": np.empty((nb, H, N // 2)),
         "normw_B": np.empty((H, N)), "normw_C": np.empty((H, N)),
         "bias_B": np.empty((H, R, N)), "bias_C": np.empty((H, R, N))}
    (lib or _load()).m3o_bcnorm_rope_backward(
        nb, L, H, R, N, int(bool(bcnorm)), float(eps), _ptr(B), _ptr(C), _ptr(dt), _ptr(theta),
        _ptr(normw_B), _ptr(normw_C), _ptr(bias_B), _ptr(bias_C), _ptr(phi_in), _ptr(dBbar),
        _ptr(dCbar), _ptr(dphi_out), _ptr(g["B"]), _ptr(g["C"]), _ptr(g["dt"]), _ptr(g["theta"]),
        _ptr(g["phi_in"]), _ptr(g["normw_B"]), _ptr(g["normw_C"]), _ptr(g["bias_B"]),
        _ptr(g["bias_C"]))
    return g


def layer_backward(inp: dict, dy, dh_out=None, dphi_out=None, bcnorm=True, eps=1e-5, mix=True,
                   lib=None):
    """Gradients of ``layer`` for the cotangents dy, dh_out and dphi_out (None = 0): the forward
    rotation is recomputed, ``scan_backward`` gives the gradients of the rotated B and C, and
    ``bcnorm_rope_backward`` carries them back to the raw inputs.  dt reaches both the scan and
    the rotation angle, so its gradient is the sum of the two shares.  Returns a dict keyed by
    input name (x, B, C, dt, A, lam, theta, normw_B, normw_C, bias_B, bias_C, w_out, phi_in, h_in,
    Bbar_prev, x_prev).  With raw B and C in G < H head slots, their gradients are summed over
    each group's heads (``groups_from_heads``)."""
    g = inp.get
    H = _f64(g("dt")).shape[2]
    B, C = _f64(g("B")), _f64(g("C"))
    G = B.shape[2]
    if G != H:
        B, C = heads_from_groups(B, H), heads_from_groups(C, H)
    Bbar, Cbar, _ = bcnorm_rope(B, C, g("dt"), g("theta"), g("normw_B"), g("normw_C"),
                                g("bias_B"), g("bias_C"), g("phi_in"), bcnorm=bcnorm, eps=eps,
                                lib=lib)
    gs = scan_backward(g("x"), Bbar, Cbar, g("dt"), g("A"), g("lam"), dy,
                       g("w_out") if mix else None, g("h_in"), g("Bbar_prev"), g("x_prev"),
                       dh_out, lib=lib)
    gr = bcnorm_rope_backward(B, C, g("dt"), g("theta"), gs["Bbar"], gs["Cbar"],
                              g("normw_B"), g("normw_C"), g("bias_B"), g("bias_C"), g("phi_in"),
                              dphi_out, bcnorm=bcnorm, eps=eps, lib=lib)
    dB, dC = gr["B"], gr["C"]
    if G != H:
        dB, dC = groups_from_heads(dB, G), groups_from_heads(dC, G)
    return {"x": gs["x"], "B": dB, "C": dC, "dt": gs["dt"] + gr["dt"], "A": gs["A"],
            "lam": gs["lam"], "theta": gr["theta"], "normw_B": gr["normw_B"],
            "normw_C": gr["normw_C"], "bias_B": gr["bias_B"], "bias_C": gr["bias_C"],
            "w_out": gs["w_out"], "phi_in": gr["phi_in"], "h_in": gs["h_in"],
            "Bbar_prev": gs["Bbar_prev"], "x_prev": gs["x_prev"]}


def build_variant(src_text: str, out_path: str):
    """Compile C source text (a modified copy of the oracle, used by the tests that check the
    pins catch planted mistakes) and return its bound library handle."""
    cpath = out_path + ".c"
    with open(cpath, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           "-ffp-contract=off", cpath, "-o", out_path, "-lm"])
    return _bind(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()
