"""Host pins of the exp2 polynomial behind attn_fwd_exp2_poly (no GPU).

The constants in csrc/exp2_poly.h must be what csrc/exp2_poly_fit.py
computes, and that fit must be the minimax one: by Chebyshev's alternation
theorem a polynomial of the fitted form is the best approximation in the
maximum norm exactly when its error takes its largest magnitude with
alternating signs at one more point than it has free coefficients.  The
error bound the header states is checked against numpy's exp2 through the
whole range reduction, in float32 arithmetic as the kernel does it.
"""
import importlib.util
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_attention_transformer_amd", "csrc")


def _fit_module():
    spec = importlib.util.spec_from_file_location("exp2_poly_fit",
                                                  os.path.join(CSRC, "exp2_poly_fit.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.fixture(scope="module")
def fitmod():
    return _fit_module()


def header_constants():
    text = open(os.path.join(CSRC, "exp2_poly.h")).read()
    vals = {}
    for name, lit in re.findall(r"constexpr float (kExp2P\d) = ([0-9a-fA-Fx.p+-]+)f;", text):
        vals[name] = float.fromhex(lit)
    return [vals["kExp2P1"], vals["kExp2P2"], vals["kExp2P3"]]


def test_header_constants_are_the_fit(fitmod):
    hdr = header_constants()
    fit = fitmod.coefficients_f32()
    assert hdr == fit
    # float32 values, held exactly by the hex literals
    assert all(float(np.float32(c)) == c for c in hdr)


def test_fit_equioscillates(fitmod):
    """Four alternation points (three coefficients + 1), equal magnitude,
    alternating signs, and no larger error anywhere on (0, 1]."""
    c, E, ref = fitmod.fit()
    assert len(ref) == 4
    e_ref = fitmod._err(c, ref)
    assert np.all(np.sign(e_ref[1:]) == -np.sign(e_ref[:-1]))
    np.testing.assert_allclose(np.abs(e_ref), E, rtol=1e-6)
    grid = np.linspace(0.0, 1.0, 1_000_001)[1:]
    assert np.abs(fitmod._err(c, grid)).max() <= E * (1 + 1e-6)
    # the relative error of the degree-3 fit of 2^f on [0, 1): ~2^-13.5
    assert 8.0e-5 < E < 9.0e-5


def test_fit_beats_the_taylor_and_interpolating_cubics(fitmod):
    """Sanity of the optimum: the minimax cubic has a smaller maximum
    relative error than the Taylor cubic at 0 and than the cubic that
    interpolates 2^f at f = 1/3, 2/3, 1 (both with p(0) = 1)."""
    c, E, _ = fitmod.fit()
    f = np.linspace(0.0, 1.0, 100_001)

    def rel(coef):
        p = 1.0 + f * np.polyval(np.asarray(coef)[::-1], f)
        return np.abs(p / np.exp2(f) - 1).max()

    ln2 = np.log(2.0)
    taylor = [ln2, ln2 ** 2 / 2, ln2 ** 3 / 6]
    nodes = np.array([1 / 3, 2 / 3, 1.0])
    A = np.stack([nodes, nodes ** 2, nodes ** 3], axis=1)
    interp = np.linalg.solve(A, np.exp2(nodes) - 1)
    assert rel(c) < rel(taylor) and rel(c) < rel(interp)
    assert abs(rel(c) - E) < 1e-9


def exp2_poly_f32(x, coef):
    """The kernel's steps in float32: clamp at -200, fract / floor, Horner in
    fused multiply-adds (each emulated exactly in float64, then rounded
    once), ldexp."""
    c1, c2, c3 = (np.float64(np.float32(v)) for v in coef)
    x = np.asarray(x, dtype=np.float32)
    xc = np.maximum(x, np.float32(-200.0))
    j = np.floor(xc.astype(np.float64))
    f = np.float32(xc.astype(np.float64) - j).astype(np.float64)    # exact in float32
    p = np.float32(c3 * f + c2).astype(np.float64)
    p = np.float32(p * f + c1).astype(np.float64)
    p = np.float32(p * f + 1.0)
    return np.ldexp(p, j.astype(np.int64)).astype(np.float32)


def test_exp2_bound_through_the_range_reduction():
    coef = header_constants()
    rng = np.random.default_rng(7)
    x = np.concatenate([np.linspace(-126.0, 8.0, 2_000_001), rng.uniform(-30, 8, 1_000_000)])
    x = x.astype(np.float32)
    got = exp2_poly_f32(x, coef).astype(np.float64)
    want = np.exp2(x.astype(np.float64))
    rel = np.abs(got / want - 1)
    # the fit's 8.56e-5 plus a few float32 roundings
    assert rel.max() < 8.6e-5 + 4 * 2.0 ** -24


def test_exp2_special_values():
    coef = header_constants()
    # masked scores give exactly zero, as the hardware exponential does
    assert exp2_poly_f32(np.float32(-np.inf), coef) == 0.0
    assert exp2_poly_f32(np.float32(-200.0), coef) == 0.0
    # integers give exact powers of two (p(0) = 1): the row maximum's weight is 1
    for k in range(-100, 9):
        assert exp2_poly_f32(np.float32(k), coef) == np.float32(2.0 ** k)
    # monotone across the integer steps, where the pieces join
    x = np.float32(np.arange(-20, 8)) + np.float32(0.0)
    below = np.nextafter(x, np.float32(-np.inf))
    assert np.all(exp2_poly_f32(below, coef) <= exp2_poly_f32(x, coef))
