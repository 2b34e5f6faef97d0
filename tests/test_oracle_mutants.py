"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of the oracle's C source with one plausible mistake (a dropped term, a
wrong sign, a wrong index or operand), built on the CPU into a temporary library.  The pins in
``pins.py`` are run against it; the test passes only if some pin rejects the mutant.  This shows
the pins are sharp enough to catch each kind of mistake, not that the oracle is right (that is
what ``test_oracle_pins.py`` checks).
"""
import numpy as np
import pytest

import oracle
import pins

GRAD_MARKER = "/*\n * Gradients of m3o_scan"

# (name, text in m3_oracle.c, replacement)
MUTANTS = [
    ("beta_without_decay", "const double beta = (1.0 - lm) * d * alpha;",
     "const double beta = (1.0 - lm) * d;"),
    ("gamma_uses_one_minus_lambda", "const double gamma = lm * d;",
     "const double gamma = (1.0 - lm) * d;"),
    ("alpha_missing_dt", "const double alpha = exp(d * A[h]);", "const double alpha = exp(A[h]);"),
    ("previous_input_not_kept", "uprev = u;\n            u = tmp;", "(void)tmp;"),
    ("output_reads_B", "const double *ct = Cbar + (row * R + r) * N;",
     "const double *ct = Bbar + (row * R + r) * N;"),
    ("rotation_transposed",
     "out[2 * k] = c * v[2 * k] + s * v[2 * k + 1];\n                        out[2 * k + 1] = -s * v[2 * k] + c * v[2 * k + 1];",
     "out[2 * k] = c * v[2 * k] - s * v[2 * k + 1];\n                        out[2 * k + 1] = s * v[2 * k] + c * v[2 * k + 1];"),
    ("angle_without_dt", "phi[k] += d * theta[row * K + k];", "phi[k] += theta[row * K + k];"),
    ("angle_skips_current_step",
     "for (int64_t k = 0; k < K; ++k)\n                phi[k] += d * theta[row * K + k];",
     "for (int64_t k = 0; k < K && t > 0; ++k)\n                phi[k] += dt[row - H] * theta[(row - H) * K + k];"),
    ("rms_not_mean", "ms /= (double)N;", ""),
    ("bias_dropped", "v[n] += bias[(h * R + r) * N + n];", "(void)bias;"),
    ("h_in_ignored", "g[i] = h_in ? h_in[(ib * H + h) * NP + i] : 0.0;", "g[i] = 0.0;"),
    ("carried_input_ignored", "if (Bbar_prev && x_prev) {", "if (0) {"),
    ("rank_sum_dropped", "u[n * P + p] += bt[n] * xt[p];", "u[n * P + p] = bt[n] * xt[p];"),
    ("mix_weight_of_rank_zero", "acc += w_out[(h * R + r) * P + p] * Y[r * P + p];",
     "acc += w_out[(h * R) * P + p] * Y[r * P + p];"),
    ("eps_outside_sqrt", "const double inv = 1.0 / sqrt(ms + eps);",
     "const double inv = 1.0 / (sqrt(ms) + eps);"),
    ("pair_swapped_in_rotation", "out[2 * k + 1] = -s * v[2 * k] + c * v[2 * k + 1];",
     "out[2 * k + 1] = -s * v[2 * k + 1] + c * v[2 * k];"),
    # gradients
    ("grad_beta_carry_dropped", "dU[i] = gamma * dg[i] + dcarry[i];", "dU[i] = gamma * dg[i];"),
    ("grad_alpha_uses_current_state", "dal += dg[i] * gp[i];", "dal += dg[i] * gt[i];"),
    ("grad_A_beta_term_dropped",
     "dA_part[bh] += dal * d * alpha + dbe * (1.0 - lm) * d * d * alpha;",
     "dA_part[bh] += dal * d * alpha;"),
    ("grad_mix_weight_dropped", "dw_part[(bh * R + r) * P + p] += acc * dyp;", "(void)acc;"),
    ("grad_angle_sign", "dphi[k] += dout[2 * k] * o1 - dout[2 * k + 1] * o0;",
     "dphi[k] += dout[2 * k + 1] * o0 - dout[2 * k] * o1;"),
    ("grad_rotation_not_inverted", "dvb[2 * k] = c * dout[2 * k] - s * dout[2 * k + 1];",
     "dvb[2 * k] = c * dout[2 * k] + s * dout[2 * k + 1];"),
    ("grad_rms_projection_dropped",
     "dsrc[n] = wn * inv * dvb[n] - inv * inv * inv * v[n] / (double)N * sdot;",
     "dsrc[n] = wn * inv * dvb[n];"),
    ("grad_angle_suffix_skips_current_step",
     "S[k] += dphi[k];\n                dtheta[row * K + k] = S[k] * dt[row];",
     "dtheta[row * K + k] = S[k] * dt[row];\n                S[k] += dphi[k];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    # forward mutants edit the forward functions, gradient mutants the backward ones (the
    # backward recomputes the forward, so some statements appear in both)
    cut = src.index(GRAD_MARKER)
    fwd, bwd = src[:cut], src[cut:]
    if name.startswith("grad_"):
        assert bwd.count(old) == 1, "mutation site not found exactly once: " + name
        src = fwd + bwd.replace(old, new)
    else:
        assert fwd.count(old) == 1, "mutation site not found exactly once: " + name
        src = fwd.replace(old, new) + bwd
    lib = oracle.build_variant(src, str(tmp_path / ("m_" + name + ".so")))
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(lib=lib)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, "no pin caught mutant " + name


# Planted mistakes in the oracle's head-group layer (Python): expanding the slots in the wrong
# order (slot h mod G instead of h // (H / G)) and summing the gradients over the wrong heads.
def _tiled_expansion(v, H):
    v = oracle._f64(v)
    return np.tile(v, (1, 1, H // v.shape[2], 1, 1))


def _strided_fold(g, G):
    b, L, H, R, N = g.shape
    return g.reshape(b, L, H // G, G, R, N).sum(axis=2)


@pytest.mark.parametrize("name,fn", [("heads_from_groups", _tiled_expansion),
                                     ("groups_from_heads", _strided_fold)])
def test_group_mutant_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(oracle, name, fn)
    with pytest.raises(AssertionError):
        pins.check_head_groups()


# Planted wiring mistakes in the oracle's decode step (Python): the carry it hands to the next
# token.  Each wraps the real step and then corrupts one carried field, as a mistake in mapping
# the layer's outputs back into the state would.
_REAL_DECODE = oracle.decode_step


def _stale_bbar(state, tok, consts, **kw):
    y, new = _REAL_DECODE(state, tok, consts, **kw)
    return y, dict(new, Bbar_prev=state["Bbar_prev"])


def _unadvanced_phi(state, tok, consts, **kw):
    y, new = _REAL_DECODE(state, tok, consts, **kw)
    return y, dict(new, phi=state["phi"])


def _stale_x(state, tok, consts, **kw):
    y, new = _REAL_DECODE(state, tok, consts, **kw)
    return y, dict(new, x_prev=state["x_prev"])


def _unrotated_bbar(state, tok, consts, **kw):
    # the raw B (normalised and biased, not rotated) carried instead of the rotated one
    y, new = _REAL_DECODE(state, tok, consts, **kw)
    return y, dict(new, Bbar_prev=oracle._f64(tok["B"]))


@pytest.mark.parametrize("fn", [_stale_bbar, _unadvanced_phi, _stale_x, _unrotated_bbar],
                         ids=lambda f: f.__name__.lstrip("_"))
def test_decode_wiring_mutant_is_caught(monkeypatch, fn):
    monkeypatch.setattr(oracle, "decode_step", fn)
    with pytest.raises(AssertionError):
        pins.check_decode_chain()
