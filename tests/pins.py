"""Checks that pin the fp64 oracle to results fixed by the pages and by mathematics.

None of these re-types the oracle's own step-by-step recurrence.  Each reaches the expected value
by a different route: a materialised structured-mask matrix, a complex-valued state, explicit 2x2
rotation matrices acting on the unrotated state, a closed form, an ODE with a known solution, a
superposition identity, or an invariant.  Every check takes ``lib`` (None = the built oracle) so
the same checks can be run against deliberately broken builds of the oracle.

Pages cited (titles of the web pages on the Mamba-3 paper):
  * aipaper.cc summary: section 4.1 Proposition 1 (trapezoidal recurrence, alpha/beta/gamma,
    lambda = 1 gives Euler); section 4.2 Propositions 2 and 3 (complex diagonal transition,
    block-diagonal rotations, cumulative rotation of B and C); section 4.3 (MIMO update).
  * papernotes.org summary: key design 1 (second-order accuracy; structured mask = 1-semiseparable
    times 2-band; lambda = 1/2 is the classical trapezoid), key design 2 (parity as the rotation
    R(pi x_t)), key design 3 (MIMO as R^2 SISO calls), key design 4 (BCNorm = RMSNorm on B, C).
  * metaphor-xennon SSM family comparison: section 2.2 (rotation matrix R_t), section 1.3 / 6.3
    (SSD form Y = (L o C B^T) X).
"""
from __future__ import annotations

import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_case(seed, L=12, R=2, N=6, P=3, H=1, b=1, carry=True):
    r = _rng(seed)
    c = {
        "x": r.standard_normal((b, L, H, R, P)),
        "B": r.standard_normal((b, L, H, R, N)),
        "C": r.standard_normal((b, L, H, R, N)),
        "dt": np.log1p(np.exp(r.standard_normal((b, L, H)) - 1.0)),
        "lam": 1.0 / (1.0 + np.exp(-r.standard_normal((b, L, H)))),
        "theta": r.standard_normal((b, L, H, N // 2)),
        "A": -np.exp(r.uniform(0, math.log(16.0), H)),
    }
    if carry:
        c["h_in"] = r.standard_normal((b, H, N, P))
        c["Bbar_prev"] = r.standard_normal((b, H, R, N))
        c["x_prev"] = r.standard_normal((b, H, R, P))
        c["phi_in"] = r.uniform(-math.pi, math.pi, (b, H, N // 2))
    return c


# ---------------------------------------------------------------------------------------------
# 1. Structured-mask matrix form (papernotes key design 1: L = 1-semiseparable x 2-band;
#    metaphor-xennon section 1.3: Y = (L o C B^T) X; aipaper section 4.3: MIMO B_t X_t^T).
# ---------------------------------------------------------------------------------------------
def brute_force_masked(x, Bb, Cb, dt, A, lam, h_in=None, Bp=None, xp=None):
    """One (batch, head): materialise D (decay, explicit products), W (2-band), L = D W, the
    (L R x L R) matrix M = (L kron 1_RxR) o (Cbar Bbar^T) and Y = M X, plus the carried-in terms."""
    L, R, P = x.shape
    alpha = np.exp(dt * A)
    beta = (1.0 - lam) * dt * alpha
    gamma = lam * dt
    D = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            D[t, s] = np.prod(alpha[s + 1:t + 1])      # decay from s to t (empty product = 1)
    W = np.zeros((L, L))
    for s in range(L):
        W[s, s] = gamma[s]
        if s + 1 < L:
            W[s + 1, s] = beta[s + 1]
    Lm = D @ W
    G = np.einsum("tan,sbn->tasb", Cb, Bb)             # Cbar_t[a] . Bbar_s[b]
    M = (Lm[:, None, :, None] * G).reshape(L * R, L * R)
    Y = (M @ x.reshape(L * R, P)).reshape(L, R, P)
    if h_in is not None:
        for t in range(L):
            Y[t] += np.prod(alpha[:t + 1]) * (Cb[t] @ h_in)
    if Bp is not None:
        u_prev = Bp.T @ xp
        for t in range(L):
            Y[t] += np.prod(alpha[1:t + 1]) * beta[0] * (Cb[t] @ u_prev)
    return Y


def check_masked_matrix_form(lib=None):
    for seed, R in ((1, 1), (2, 2), (3, 3)):
        c = _rand_case(seed, L=13, R=R, N=6, P=3)
        y, _ = oracle.scan(c["x"], c["B"], c["C"], c["dt"], c["A"], c["lam"], None, c["h_in"],
                           c["Bbar_prev"], c["x_prev"], lib=lib)
        ref = brute_force_masked(c["x"][0, :, 0], c["B"][0, :, 0], c["C"][0, :, 0], c["dt"][0, :, 0],
                                 c["A"][0], c["lam"][0, :, 0], c["h_in"][0, 0],
                                 c["Bbar_prev"][0, 0], c["x_prev"][0, 0])
        err = np.abs(y[0, :, 0] - ref).max() / np.abs(ref).max()
        assert err < 1e-12, ("masked-matrix form", R, err)


# ---------------------------------------------------------------------------------------------
# 2. lambda = 1 reduces to Mamba-2's exponential-Euler step (aipaper section 4.1; papernotes
#    key design 1).  The reference below is the Euler recurrence h = e^{dt A} h + dt B x.
# ---------------------------------------------------------------------------------------------
def check_lambda_one_is_euler(lib=None):
    c = _rand_case(11, L=20, R=2, N=4, P=5)
    lam = np.ones_like(c["lam"])
    y, h = oracle.scan(c["x"], c["B"], c["C"], c["dt"], c["A"], lam, None, c["h_in"],
                       c["Bbar_prev"], c["x_prev"], lib=lib)
    hh = c["h_in"][0, 0].copy()
    for t in range(20):
        d = c["dt"][0, t, 0]
        hh = math.exp(d * c["A"][0]) * hh + d * (c["B"][0, t, 0].T @ c["x"][0, t, 0])
        yt = c["C"][0, t, 0] @ hh
        assert np.abs(y[0, t, 0] - yt).max() <= 1e-12 * max(1.0, np.abs(yt).max())
    assert np.abs(h[0, 0] - hh).max() <= 1e-12 * max(1.0, np.abs(hh).max())


# ---------------------------------------------------------------------------------------------
# 3. Constant inputs without rotation: g_t = u [gamma a^t + (beta + gamma)(1 - a^t)/(1 - a)]
#    (a closed form of the recurrence of aipaper section 4.1 for constant dt, A, lambda, B, x).
# ---------------------------------------------------------------------------------------------
def check_constant_input_closed_form(lib=None):
    L, N, P = 40, 4, 3
    r = _rng(21)
    bvec, cvec, xvec = r.standard_normal(N), r.standard_normal(N), r.standard_normal(P)
    for d, A, lm in ((0.3, -1.7, 0.35), (0.9, -0.2, 0.8), (0.5, 0.0, 0.5)):
        x = np.broadcast_to(xvec, (1, L, 1, 1, P)).copy()
        B = np.broadcast_to(bvec, (1, L, 1, 1, N)).copy()
        C = np.broadcast_to(cvec, (1, L, 1, 1, N)).copy()
        dt = np.full((1, L, 1), d)
        lam = np.full((1, L, 1), lm)
        y, _ = oracle.scan(x, B, C, dt, np.array([A]), lam, lib=lib)
        a = math.exp(d * A)
        beta, gamma = (1 - lm) * d * a, lm * d
        u = np.outer(bvec, xvec)
        for t in range(L):
            if a == 1.0:
                coef = gamma + (beta + gamma) * t
            else:
                coef = gamma * a ** t + (beta + gamma) * (1 - a ** t) / (1 - a)
            ref = cvec @ (coef * u)
            assert np.abs(y[0, t, 0, 0] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


# ---------------------------------------------------------------------------------------------
# 4. Constant inputs with a constant rotation, solved in the complex frame of aipaper section 4.2
#    (transition e^{dt (A + i theta)} per pair).  With rho = a e^{i phi}:
#    z_t = rho^t gamma v + (beta e^{i phi} + gamma) v (1 - rho^t) / (1 - rho),  y_t = Re(conj(c) z_t)
# ---------------------------------------------------------------------------------------------
def check_rotating_constant_closed_form(lib=None):
    L, N, P = 30, 6, 2
    K = N // 2
    r = _rng(31)
    bvec, cvec, xvec = r.standard_normal(N), r.standard_normal(N), r.standard_normal(P)
    th = r.standard_normal(K) * 2.0
    d, A, lm = 0.4, -0.6, 0.3
    x = np.broadcast_to(xvec, (1, L, 1, 1, P)).copy()
    B = np.broadcast_to(bvec, (1, L, 1, 1, N)).copy()
    C = np.broadcast_to(cvec, (1, L, 1, 1, N)).copy()
    dt = np.full((1, L, 1), d)
    lam = np.full((1, L, 1), lm)
    theta = np.broadcast_to(th, (1, L, 1, K)).copy()
    Bb, Cb, _ = oracle.bcnorm_rope(B, C, dt, theta, bcnorm=False, lib=lib)
    y, _ = oracle.scan(x, Bb, Cb, dt, np.array([A]), lam, lib=lib)
    a = math.exp(d * A)
    beta, gamma = (1 - lm) * d * a, lm * d
    phi = d * th
    rho = a * np.exp(1j * phi)                          # [K]
    bz = bvec[0::2] + 1j * bvec[1::2]
    cz = cvec[0::2] + 1j * cvec[1::2]
    v = bz[:, None] * xvec[None, :]                     # [K, P]
    for t in range(L):
        z = (rho ** t * gamma)[:, None] * v + ((beta * np.exp(1j * phi) + gamma)
                                              * (1 - rho ** t) / (1 - rho))[:, None] * v
        ref = np.real(np.conj(cz)[:, None] * z).sum(0)
        assert np.abs(y[0, t, 0, 0] - ref).max() <= 1e-11 * max(1.0, np.abs(ref).max()), t


# ---------------------------------------------------------------------------------------------
# 5. Parity through rotations by pi (papernotes key design 2: parity is R(pi x_t)).  Hand-built
#    sequence in tests/golden/parity_flip.txt: one unit impulse at t = 0, then zero input and a
#    rotation angle of pi on each '1' bit.  Expected y_t = a^t (-1)^{sum of bits 1..t}.
# ---------------------------------------------------------------------------------------------
def load_parity_golden():
    bits, signs = [], []
    with open(os.path.join(GOLDEN, "parity_flip.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            t, bit, sign = line.split()
            bits.append(int(bit))
            signs.append(int(sign))
    return np.array(bits), np.array(signs)


def check_parity_flip(lib=None):
    bits, signs = load_parity_golden()
    L = len(bits)
    for A, lm, y0 in ((0.0, 1.0, 1.0), (-0.05, 1.0, 1.0), (-0.05, 0.5, 0.5)):
        x = np.zeros((1, L, 1, 1, 1))
        x[0, 0] = 1.0
        B = np.zeros((1, L, 1, 1, 2))
        B[0, :, 0, 0, 0] = 1.0
        C = B.copy()
        dt = np.ones((1, L, 1))
        lam = np.full((1, L, 1), lm)
        theta = (math.pi * bits).reshape(1, L, 1, 1)
        Bb, Cb, _ = oracle.bcnorm_rope(B, C, dt, theta, bcnorm=False, lib=lib)
        y, _ = oracle.scan(x, Bb, Cb, dt, np.array([A]), lam, lib=lib)
        a = math.exp(A)
        expect = signs * a ** np.arange(L)
        expect[0] = y0
        assert np.abs(y[0, :, 0, 0, 0] - expect).max() < 1e-13, (A, lm)


# ---------------------------------------------------------------------------------------------
# 6. Complex-valued SSM == real SSM with cumulative rotation of B and C (aipaper section 4.2,
#    Propositions 2-3).  Reference: complex state per pair, transition a_t e^{i dt_t theta_t},
#    previous-input term carried by the full complex transition, output Re(conj(c) h).
#    The oracle's returned state is the rotated frame: h_final = e^{i Phi} g_final.
# ---------------------------------------------------------------------------------------------
def _complex_reference(c, bcnorm_vecs):
    """One (batch, head); bcnorm_vecs = (Btilde, Ctilde) after norm and bias, unrotated."""
    Bt, Ct = bcnorm_vecs
    x = c["x"][0, :, 0]
    L, R, P = x.shape
    K = Bt.shape[-1] // 2
    bz = Bt[..., 0::2] + 1j * Bt[..., 1::2]          # [L, R, K]
    cz = Ct[..., 0::2] + 1j * Ct[..., 1::2]
    phi0 = c["phi_in"][0, 0]
    g0 = c["h_in"][0, 0]
    h = np.exp(1j * phi0)[:, None] * (g0[0::2] + 1j * g0[1::2])       # [K, P], unrotated frame
    bp = c["Bbar_prev"][0, 0]
    v_prev = np.exp(1j * phi0)[:, None] * ((bp[:, 0::2] + 1j * bp[:, 1::2]).T @ c["x_prev"][0, 0])
    Phi = phi0.copy()
    ys = []
    for t in range(L):
        d, lm = c["dt"][0, t, 0], c["lam"][0, t, 0]
        a = math.exp(d * c["A"][0])
        step = np.exp(1j * d * c["theta"][0, t, 0])     # [K]
        v = bz[t].T @ x[t]                              # [K, P]
        h = (a * step)[:, None] * h + ((1 - lm) * d * a * step)[:, None] * v_prev + lm * d * v
        ys.append(np.real(np.conj(cz[t]) @ h))         # [R, P]
        v_prev = v
        Phi = Phi + d * c["theta"][0, t, 0]
    return np.array(ys), h, Phi


def check_complex_frame(lib=None):
    c = _rand_case(41, L=17, R=2, N=8, P=3)
    Bb, Cb, phi = oracle.bcnorm_rope(c["B"], c["C"], c["dt"], c["theta"], phi_in=c["phi_in"],
                                     bcnorm=False, lib=lib)
    y, g = oracle.scan(c["x"], Bb, Cb, c["dt"], c["A"], c["lam"], None, c["h_in"],
                       c["Bbar_prev"], c["x_prev"], lib=lib)
    ys, hz, Phi = _complex_reference(c, (c["B"][0, :, 0], c["C"][0, :, 0]))
    assert np.abs(y[0, :, 0] - ys).max() < 1e-12 * np.abs(ys).max()
    gz = g[0, 0, 0::2] + 1j * g[0, 0, 1::2]
    assert np.abs(np.exp(1j * Phi)[:, None] * gz - hz).max() < 1e-12 * np.abs(hz).max()
    assert np.abs(phi[0, 0] - Phi).max() < 1e-12


# ---------------------------------------------------------------------------------------------
# 7. The same with explicit real 2x2 rotation matrices R_t = [[cos, -sin], [sin, cos]] of angle
#    dt_t theta_t acting on the unrotated real state (metaphor-xennon section 2.2; aipaper
#    Proposition 2: real state of doubled size with block-diagonal rotations).
# ---------------------------------------------------------------------------------------------
def check_real_rotation_matrices(lib=None):
    c = _rand_case(51, L=15, R=1, N=4, P=2)
    c["h_in"][:] = 0.0
    c["Bbar_prev"][:] = 0.0
    c["phi_in"][:] = 0.0
    Bb, Cb, _ = oracle.bcnorm_rope(c["B"], c["C"], c["dt"], c["theta"], bcnorm=False, lib=lib)
    y, _ = oracle.scan(c["x"], Bb, Cb, c["dt"], c["A"], c["lam"], lib=lib)
    N, P, L = 4, 2, 15
    h = np.zeros((N, P))
    u_prev = np.zeros((N, P))
    for t in range(L):
        d, lm = c["dt"][0, t, 0], c["lam"][0, t, 0]
        a = math.exp(d * c["A"][0])
        Rt = np.zeros((N, N))
        for k in range(N // 2):
            ang = d * c["theta"][0, t, 0, k]
            Rt[2 * k:2 * k + 2, 2 * k:2 * k + 2] = [[math.cos(ang), -math.sin(ang)],
                                                     [math.sin(ang), math.cos(ang)]]
        u = np.outer(c["B"][0, t, 0, 0], c["x"][0, t, 0, 0])
        h = a * (Rt @ h) + (1 - lm) * d * a * (Rt @ u_prev) + lm * d * u
        yt = c["C"][0, t, 0, 0] @ h
        assert np.abs(y[0, t, 0, 0] - yt).max() < 1e-12 * max(1.0, np.abs(yt).max()), t
        u_prev = u


# ---------------------------------------------------------------------------------------------
# 8. Order of accuracy on h' = a h + cos(w t) (papernotes key design 1: Euler local error
#    O(dt^2), exponential-trapezoid O(dt^3); lambda = 1/2 is the classical trapezoid).  Halving dt
#    divides the global error by 4 for lambda = 1/2 and by 2 for lambda = 1 or 0.
# ---------------------------------------------------------------------------------------------
def _ode_final_error(lm, steps, a=-0.7, w=2.0, T=4.0, h0=0.3, lib=None):
    d = T / steps
    ts = d * np.arange(1, steps + 1)
    x = np.cos(w * ts).reshape(1, steps, 1, 1, 1)
    B = np.zeros((1, steps, 1, 1, 2))
    B[..., 0] = 1.0
    dt = np.full((1, steps, 1), d)
    lam = np.full((1, steps, 1), lm)
    h_in = np.array([[[[h0], [0.0]]]])
    Bp = np.array([[[[1.0, 0.0]]]])
    xp = np.array([[[[1.0]]]])                          # x(0) = cos(0)
    _, h = oracle.scan(x, B, B, dt, np.array([a]), lam, None, h_in, Bp, xp, lib=lib)
    hp = lambda t: (-a * math.cos(w * t) + w * math.sin(w * t)) / (a * a + w * w)
    exact = hp(T) + math.exp(a * T) * (h0 - hp(0.0))
    return abs(h[0, 0, 0, 0] - exact)


def check_order_of_accuracy(lib=None):
    for lm, lo, hi in ((0.5, 3.8, 4.2), (1.0, 1.85, 2.15), (0.0, 1.85, 2.15)):
        e1 = _ode_final_error(lm, 400, lib=lib)
        e2 = _ode_final_error(lm, 800, lib=lib)
        ratio = e1 / e2
        assert lo < ratio < hi, (lm, ratio)


def check_trapezoid_exact_on_linear_input(lib=None):
    """With A = 0 and lambda = 1/2 the update is the classical trapezoid rule, exact for a linear
    input: h(T) = h0 + integral_0^T (c0 + c1 t) dt."""
    steps, T, c0, c1, h0 = 37, 3.0, 0.4, -1.3, 0.25
    d = T / steps
    ts = d * np.arange(1, steps + 1)
    x = (c0 + c1 * ts).reshape(1, steps, 1, 1, 1)
    B = np.zeros((1, steps, 1, 1, 2))
    B[..., 0] = 1.0
    _, h = oracle.scan(x, B, B, np.full((1, steps, 1), d), np.array([0.0]),
                       np.full((1, steps, 1), 0.5), None, np.array([[[[h0], [0.0]]]]),
                       np.array([[[[1.0, 0.0]]]]), np.array([[[[c0]]]]), lib=lib)
    assert abs(h[0, 0, 0, 0] - (h0 + c0 * T + 0.5 * c1 * T * T)) < 1e-12


# ---------------------------------------------------------------------------------------------
# 9. MIMO = sum of R^2 SISO runs (papernotes key design 3): Y[r_out] = sum_{r_in}
#    SISO(x[r_in], Bbar[r_in], Cbar[r_out]); the state is the sum over r_in.
# ---------------------------------------------------------------------------------------------
def check_mimo_is_sum_of_siso(lib=None):
    R = 3
    c = _rand_case(61, L=11, R=R, N=4, P=3)
    y, h = oracle.scan(c["x"], c["B"], c["C"], c["dt"], c["A"], c["lam"], None, c["h_in"],
                       c["Bbar_prev"], c["x_prev"], lib=lib)
    for ro in range(R):
        acc = 0.0
        hacc = 0.0
        for ri in range(R):
            ys, hs = oracle.scan(c["x"][:, :, :, ri:ri + 1], c["B"][:, :, :, ri:ri + 1],
                                 c["C"][:, :, :, ro:ro + 1], c["dt"], c["A"], c["lam"], None,
                                 c["h_in"] if ri == 0 else None, c["Bbar_prev"][:, :, ri:ri + 1],
                                 c["x_prev"][:, :, ri:ri + 1], lib=lib)
            acc = acc + ys[:, :, :, 0]
            hacc = hacc + hs
        assert np.abs(y[:, :, :, ro] - acc).max() < 1e-12 * np.abs(acc).max()
        assert np.abs(h - hacc).max() < 1e-12 * np.abs(hacc).max()


# ---------------------------------------------------------------------------------------------
# 10. BCNorm invariants (papernotes key design 4: RMSNorm on B and C; head-specific bias):
#     unit RMS per vector (eps -> 0, no weight), RMS = weight for a constant weight, the bias is
#     added after the norm, and the rotation preserves the norm of every pair.
# ---------------------------------------------------------------------------------------------
def check_bcnorm_invariants(lib=None):
    r = _rng(71)
    b, L, H, R, N = 2, 5, 3, 2, 8
    B = r.standard_normal((b, L, H, R, N)) * 3.0
    C = r.standard_normal((b, L, H, R, N)) * 0.2
    dt = np.abs(r.standard_normal((b, L, H)))
    th0 = np.zeros((b, L, H, N // 2))
    th = r.standard_normal((b, L, H, N // 2))
    Bb, Cb, _ = oracle.bcnorm_rope(B, C, dt, th0, eps=1e-300, lib=lib)
    for X in (Bb, Cb):
        assert np.abs(np.sqrt((X ** 2).mean(-1)) - 1.0).max() < 1e-12
    w = np.full((H, N), 2.5)
    Bw, _, _ = oracle.bcnorm_rope(B, C, dt, th0, normw_B=w, normw_C=w, eps=1e-300, lib=lib)
    assert np.abs(np.sqrt((Bw ** 2).mean(-1)) - 2.5).max() < 1e-12
    bias = r.standard_normal((H, R, N))
    Bbias, Cbias, _ = oracle.bcnorm_rope(B, C, dt, th0, bias_B=bias, bias_C=-bias, eps=1e-300,
                                         lib=lib)
    assert np.abs(Bbias - Bb - bias).max() < 1e-12
    assert np.abs(Cbias - Cb + bias).max() < 1e-12
    Br, Cr, _ = oracle.bcnorm_rope(B, C, dt, th, bias_B=bias, eps=1e-300, lib=lib)
    pn = lambda X: X[..., 0::2] ** 2 + X[..., 1::2] ** 2
    assert np.abs(pn(Br) - pn(Bbias)).max() < 1e-11
    assert np.abs(pn(Cr) - pn(Cb)).max() < 1e-11


# ---------------------------------------------------------------------------------------------
# 11. Carry: a sequence split in two calls, the second given the first's final state, angle and
#     last (Bbar, x), equals one call over the whole sequence.
# ---------------------------------------------------------------------------------------------
def check_split_carry(lib=None):
    c = _rand_case(81, L=19, R=2, N=6, P=3, H=2, b=2)
    full = oracle.layer(c, mix=False, lib=lib)
    t1 = 7
    first = {k: (v[:, :t1] if k in ("x", "B", "C", "dt", "lam", "theta") else v)
             for k, v in c.items()}
    o1 = oracle.layer(first, mix=False, lib=lib)
    second = {k: (v[:, t1:] if k in ("x", "B", "C", "dt", "lam", "theta") else v)
              for k, v in c.items()}
    second.update(h_in=o1["h_out"], phi_in=o1["phi_out"], Bbar_prev=o1["Bbar_last"],
                  x_prev=o1["x_last"])
    o2 = oracle.layer(second, mix=False, lib=lib)
    y = np.concatenate([o1["y"], o2["y"]], axis=1)
    assert np.abs(y - full["y"]).max() < 1e-12 * np.abs(full["y"]).max()
    assert np.abs(o2["h_out"] - full["h_out"]).max() < 1e-12 * np.abs(full["h_out"]).max()
    assert np.abs(o2["phi_out"] - full["phi_out"]).max() < 1e-12


# ---------------------------------------------------------------------------------------------
# 11. Gradients: central finite differences of the forward oracle.  The pages define no backward
#     pass; the gradient of the forward definition is what the backward computes, and a central
#     difference of the forward (O(h^2) truncation, h = 1e-5) reaches it by another route.
# ---------------------------------------------------------------------------------------------
def _grad_case(seed, R, mix, bcnorm, carry, weights, groups=0):
    c = _rand_case(seed, L=6, R=R, N=4, P=3, H=2, b=2, carry=carry)
    if groups:   # raw B and C shared by the heads: the first `groups` head slots are kept
        c["B"] = c["B"][:, :, :groups].copy()
        c["C"] = c["C"][:, :, :groups].copy()
    r = _rng(seed + 1000)
    H, N, P = 2, 4, 3
    if weights:
        c["normw_B"] = 1.0 + 0.3 * r.standard_normal((H, N))
        c["normw_C"] = 1.0 + 0.3 * r.standard_normal((H, N))
    c["bias_B"] = 0.5 * r.standard_normal((H, R, N))
    c["bias_C"] = 0.5 * r.standard_normal((H, R, N))
    if mix:
        c["w_out"] = r.standard_normal((H, R, P))
    return c


def _objective(c, cot, mix, bcnorm, lib):
    out = oracle.layer(c, bcnorm=bcnorm, mix=mix, lib=lib)
    return (float(np.sum(cot["y"] * out["y"])) + float(np.sum(cot["h"] * out["h_out"]))
            + float(np.sum(cot["phi"] * out["phi_out"])))


def check_layer_gradients_fd(lib=None):
    step = 1e-5
    for seed, R, mix, bcnorm, carry, weights, groups in [(91, 2, True, True, True, True, 0),
                                                         (92, 1, False, False, False, False, 0),
                                                         (93, 3, False, True, True, False, 0),
                                                         (94, 2, True, True, True, True, 1)]:
        c = _grad_case(seed, R, mix, bcnorm, carry, weights, groups)
        b, L, H, _, P = c["x"].shape
        N = c["B"].shape[-1]
        r = _rng(seed + 2000)
        cot = {"y": r.standard_normal((b, L, H, P) if mix else (b, L, H, R, P)),
               "h": r.standard_normal((b, H, N, P)), "phi": r.standard_normal((b, H, N // 2))}
        grads = oracle.layer_backward(c, cot["y"], cot["h"], cot["phi"], bcnorm=bcnorm, mix=mix,
                                      lib=lib)
        for name, val in c.items():
            if name == "w_out" and not mix:
                continue
            got = grads[name]
            assert got is not None and got.shape == val.shape, name
            fd = np.empty_like(val)
            flat = val.reshape(-1)
            for i in range(flat.size):
                keep = flat[i]
                flat[i] = keep + step
                fp = _objective(c, cot, mix, bcnorm, lib)
                flat[i] = keep - step
                fm = _objective(c, cot, mix, bcnorm, lib)
                flat[i] = keep
                fd.reshape(-1)[i] = (fp - fm) / (2 * step)
            scale = max(1.0, float(np.abs(fd).max()))
            err = float(np.abs(got - fd).max())
            assert err <= 1e-6 * scale, (seed, name, err, scale)


# ---------------------------------------------------------------------------------------------
# 12. Head groups: raw B and C in G < H slots, slot s shared by heads s H/G .. (s+1) H/G - 1.  The
#     pages define B and C per head, so each head of a group must get exactly what a one-head
#     call with its slot's rows gives.  Reached here by slicing every per-head input at h and the
#     B, C slot at h G / H for a separate one-head call.
# ---------------------------------------------------------------------------------------------
_HEAD_AXIS = {"x": 2, "dt": 2, "lam": 2, "theta": 2, "A": 0, "h_in": 1, "Bbar_prev": 1,
              "x_prev": 1, "phi_in": 1, "bias_B": 0, "bias_C": 0, "normw_B": 0, "normw_C": 0,
              "w_out": 0}


def check_head_groups(lib=None):
    b, L, H, G, R, N, P = 2, 9, 4, 2, 2, 6, 3
    c = _rand_case(101, L=L, R=R, N=N, P=P, H=H, b=b)
    r = _rng(1101)
    c["B"] = r.standard_normal((b, L, G, R, N))
    c["C"] = r.standard_normal((b, L, G, R, N))
    c["bias_B"] = 0.5 * r.standard_normal((H, R, N))
    c["bias_C"] = 0.5 * r.standard_normal((H, R, N))
    c["normw_B"] = 1.0 + 0.3 * r.standard_normal((H, N))
    c["normw_C"] = 1.0 + 0.3 * r.standard_normal((H, N))
    c["w_out"] = r.standard_normal((H, R, P))
    out = oracle.layer(c, mix=True, lib=lib)
    assert out["y"].shape == (b, L, H, P) and out["Bbar"].shape == (b, L, H, R, N)
    for h in range(H):
        slot = (h * G) // H
        one = {k: np.take(v, [h], axis=_HEAD_AXIS[k]) for k, v in c.items() if k in _HEAD_AXIS}
        one["B"] = c["B"][:, :, slot:slot + 1]
        one["C"] = c["C"][:, :, slot:slot + 1]
        ref = oracle.layer(one, mix=True, lib=lib)
        assert np.abs(out["y"][:, :, h:h + 1] - ref["y"]).max() <= 1e-13 * np.abs(ref["y"]).max()
        assert np.abs(out["h_out"][:, h:h + 1] - ref["h_out"]).max() <= 1e-13 * np.abs(ref["h_out"]).max()
        assert np.abs(out["Bbar_last"][:, h:h + 1] - ref["Bbar_last"]).max() <= 1e-13
    # gradients of the shared rows: central differences of the forward (two groups of two heads,
    # so a sum over the wrong heads shows)
    d = _rand_case(102, L=4, R=1, N=4, P=2, H=H, b=1)
    r = _rng(1102)
    d["B"] = r.standard_normal((1, 4, G, 1, 4))
    d["C"] = r.standard_normal((1, 4, G, 1, 4))
    d["bias_B"] = 0.5 * r.standard_normal((H, 1, 4))
    d["bias_C"] = 0.5 * r.standard_normal((H, 1, 4))
    cot = {"y": r.standard_normal((1, 4, H, 1, 2)), "h": r.standard_normal((1, H, 4, 2)),
           "phi": r.standard_normal((1, H, 2))}
    grads = oracle.layer_backward(d, cot["y"], cot["h"], cot["phi"], mix=False, lib=lib)
    step = 1e-5
    for name in ("B", "C"):
        flat = d[name].reshape(-1)
        fd = np.empty(flat.size)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + step
            fp = _objective(d, cot, False, True, lib)
            flat[i] = keep - step
            fm = _objective(d, cot, False, True, lib)
            flat[i] = keep
            fd[i] = (fp - fm) / (2 * step)
        got = grads[name].reshape(-1)
        assert grads[name].shape == d[name].shape
        assert np.abs(got - fd).max() <= 1e-6 * max(1.0, float(np.abs(fd).max())), name


# ---------------------------------------------------------------------------------------------
# 13. Two readings written out (the pages leave them open): the MIMO output mixing
#     y[p] = sum_r w_out[h, r, p] Y[r, p] (papernotes key design 3 gives x_t as P x R; the mixing
#     back to P is the reading) and BCNorm's eps, added to the mean square under the square root.
#     Each is checked against its definition by another route: the unmixed outputs weighted and
#     summed here, and the closed form of a constant vector, c w / sqrt(c^2 + eps).
# ---------------------------------------------------------------------------------------------
def check_output_mixing(lib=None):
    c = _rand_case(111, L=7, R=3, N=4, P=5, H=2, b=2)
    r = _rng(1111)
    w_out = r.standard_normal((2, 3, 5))
    c["w_out"] = w_out
    mixed = oracle.layer(c, mix=True, lib=lib)["y"]                  # [b, L, H, P]
    ranks = oracle.layer(c, mix=False, lib=lib)["y"]                 # [b, L, H, R, P]
    ref = np.zeros_like(mixed)
    for h in range(2):
        for rr in range(3):
            ref[:, :, h, :] += w_out[h, rr, :] * ranks[:, :, h, rr, :]
    assert np.abs(mixed - ref).max() <= 1e-13 * np.abs(ref).max()


def check_bcnorm_eps(lib=None):
    L, N = 3, 8
    dt = np.full((1, L, 1), 0.3)
    th0 = np.zeros((1, L, 1, N // 2))
    w = np.linspace(0.5, 1.5, N).reshape(1, N)
    for cval, eps in ((0.7, 1e-5), (0.7, 0.49), (-2.0, 3.0), (1e-3, 1e-5)):
        B = np.full((1, L, 1, 1, N), cval)
        Bb, Cb, _ = oracle.bcnorm_rope(B, -B, dt, th0, normw_B=w, normw_C=w, eps=eps, lib=lib)
        want = cval * w[0] / math.sqrt(cval * cval + eps)
        assert np.abs(Bb[0, :, 0, 0] - want).max() <= 1e-14
        assert np.abs(Cb[0, :, 0, 0] + want).max() <= 1e-14


# ---------------------------------------------------------------------------------------------
# 14. Decode = the layer core one token at a time (aipaper section 4.1 Proposition 1 is a step
#     recurrence; decode carries its state, angle and previous-token factors from step to step).
#     k chained ``oracle.decode_step`` calls must give the outputs of one ``oracle.layer`` call
#     over the same k steps, and leave behind its final state, angle, last rotated B and last x.
#     Without BCNorm or bias the chained outputs must also equal the complex-frame reference of
#     check 6 (aipaper Propositions 2-3), a route that does not go through ``oracle.layer``.
# ---------------------------------------------------------------------------------------------
def _decode_chain(c, mix, bcnorm, lib):
    """Run c's L steps through oracle.decode_step one token at a time; returns (ys, state)."""
    L = c["x"].shape[1]
    consts = {k: c[k] for k in ("A", "normw_B", "normw_C", "bias_B", "bias_C", "w_out") if k in c}
    state = {"h": c["h_in"], "phi": c["phi_in"], "Bbar_prev": c["Bbar_prev"], "x_prev": c["x_prev"]}
    ys = []
    for t in range(L):
        tok = {k: c[k][:, t] for k in ("x", "B", "C", "dt", "lam", "theta")}
        y, state = oracle.decode_step(state, tok, consts, bcnorm=bcnorm, mix=mix, lib=lib)
        ys.append(y)
    return np.stack(ys, axis=1), state


def check_decode_chain(lib=None):
    c = _rand_case(121, L=9, R=2, N=6, P=3, H=2, b=2)
    r = _rng(1121)
    c["normw_B"] = 1.0 + 0.3 * r.standard_normal((2, 6))
    c["normw_C"] = 1.0 + 0.3 * r.standard_normal((2, 6))
    c["bias_B"] = 0.5 * r.standard_normal((2, 2, 6))
    c["bias_C"] = 0.5 * r.standard_normal((2, 2, 6))
    c["w_out"] = r.standard_normal((2, 2, 3))
    full = oracle.layer(c, mix=True, lib=lib)
    ys, st = _decode_chain(c, True, True, lib)
    tol = lambda ref: 1e-12 * max(1.0, float(np.abs(ref).max()))
    assert np.abs(ys - full["y"]).max() <= tol(full["y"]), "decode outputs"
    assert np.abs(st["h"] - full["h_out"]).max() <= tol(full["h_out"]), "decode state"
    assert np.abs(st["phi"] - full["phi_out"]).max() <= 1e-12, "decode angle"
    assert np.abs(st["Bbar_prev"] - full["Bbar_last"]).max() <= tol(full["Bbar_last"]), "decode last Bbar"
    assert np.abs(st["x_prev"] - full["x_last"]).max() == 0.0, "decode last x"
    # no BCNorm, no bias, unmixed: against the complex-valued recurrence
    d = _rand_case(122, L=11, R=2, N=8, P=3)
    ys, st = _decode_chain(d, False, False, lib)
    ref, hz, Phi = _complex_reference(d, (d["B"][0, :, 0], d["C"][0, :, 0]))
    assert np.abs(ys[0, :, 0] - ref).max() <= 1e-12 * np.abs(ref).max(), "decode vs complex frame"
    gz = st["h"][0, 0, 0::2] + 1j * st["h"][0, 0, 1::2]
    assert np.abs(np.exp(1j * Phi)[:, None] * gz - hz).max() <= 1e-12 * np.abs(hz).max()
    assert np.abs(st["phi"][0, 0] - Phi).max() <= 1e-12


ALL_CHECKS = [
    check_masked_matrix_form,
    check_lambda_one_is_euler,
    check_constant_input_closed_form,
    check_rotating_constant_closed_form,
    check_parity_flip,
    check_complex_frame,
    check_real_rotation_matrices,
    check_order_of_accuracy,
    check_trapezoid_exact_on_linear_input,
    check_mimo_is_sum_of_siso,
    check_bcnorm_invariants,
    check_split_carry,
    check_layer_gradients_fd,
    check_head_groups,
    check_output_mixing,
    check_bcnorm_eps,
    check_decode_chain,
]
