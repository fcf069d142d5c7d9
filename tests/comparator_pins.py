"""Pins of the GEMM comparators (oracle.gemm_check, oracle.gemm_check_f8), which decide every
non-integer GEMM and convolution parity test on the GPU.

Each pin takes the module that holds the comparators (the committed ``oracle`` package, or a
deliberately broken copy of it) and plants results whose verdict the contract fixes: the rule
"finite and |g − r| ≤ max(1e-2·|r|, 1e-3)" (1e-2 relative error; 1e-3 absolute on entries below
0.1, where 1e-2·|r| is the smaller of the two), and for 8-bit inputs that bound plus
F8_DOT_BOUND · Σ_k |a_k·b_k|.  Values at the bound are built in binary64 so that the error the
comparator computes is exactly at, or one unit in the last place beyond, its bound.
"""
import numpy as np
import pytest


def _at_and_past(r: float, bound: float):
    """(g at the bound, g just past it) above r: g - r <= bound, then the next double has g - r > bound."""
    g = r + bound
    while g - r > bound:
        g = np.nextafter(g, -np.inf)
    while True:
        nxt = np.nextafter(g, np.inf)
        if nxt - r > bound:
            return g, nxt
        g = nxt


def _verdict(m, got, ref, **kw):
    return m.gemm_check(np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64), **kw)["pass"]


def pin_exact_passes(m):
    r = np.linspace(-3.0, 3.0, 64).reshape(8, 8)
    assert _verdict(m, r, r)
    assert m.gemm_check(r, r)["n_fail"] == 0


def pin_non_finite_fails(m):
    r = np.full((4, 4), 0.5)
    for bad in (np.nan, np.inf, -np.inf):
        g = r.copy()
        g[2, 3] = bad
        res = m.gemm_check(g, r)
        assert not res["pass"], f"{bad} passed"
        assert res["n_fail"] == 1


def pin_relative_branch_at_and_past_the_bound(m):
    for r in (0.5, -0.5, 3.25, -1000.0, 0.125):
        bound = max(1e-2 * abs(r), 1e-3)
        at, past = _at_and_past(r, bound)
        assert _verdict(m, [[at]], [[r]]), f"error at the bound fails for r={r}"
        assert not _verdict(m, [[past]], [[r]]), f"error past the bound passes for r={r}"
        # the same on the other side of r
        at_lo, past_lo = 2 * r - at, 2 * r - past
        if abs(at_lo - r) <= bound:
            assert _verdict(m, [[at_lo]], [[r]])
        if abs(past_lo - r) > bound:
            assert not _verdict(m, [[past_lo]], [[r]]), f"error below r past the bound passes for r={r}"


def pin_absolute_branch_at_and_past_the_bound(m):
    # below 0.1 the bound is 1e-3, not 1e-2·|r|
    for r in (0.0, 0.05, -0.05, 0.0999, 1e-6):
        at, past = _at_and_past(r, 1e-3)
        assert _verdict(m, [[at]], [[r]]), f"error at 1e-3 fails for r={r}"
        assert not _verdict(m, [[past]], [[r]]), f"error past 1e-3 passes for r={r}"
    # an error between 1e-2·|r| and 1e-3 passes only because of the absolute branch
    assert _verdict(m, [[0.05 + 8e-4]], [[0.05]])
    assert _verdict(m, [[-0.05 - 8e-4]], [[-0.05]])


def pin_branch_switch_at_a_tenth(m):
    # just above |r| = 0.1 the relative branch takes over: 1.5e-3 passes at r = 0.2, and only
    # there (an absolute-only rule would fail it)
    assert _verdict(m, [[0.2 + 1.5e-3]], [[0.2]])
    assert not _verdict(m, [[0.05 + 1.5e-3]], [[0.05]])
    # at r = 0.1 the two branches meet: an error of 0.99e-3 passes, 1.01e-3 does not
    assert _verdict(m, [[0.1 + 0.99e-3]], [[0.1]])
    assert not _verdict(m, [[0.1 + 1.01e-3]], [[0.1]])
    res = m.gemm_check(np.array([0.05, 0.0999, 0.1, 0.2, -0.05]), np.array([0.05, 0.0999, 0.1, 0.2, -0.05]))
    assert res["n_abs_branch"] == 3


def pin_sign_and_scale_slips_fail(m):
    r = np.linspace(0.5, 2.0, 16).reshape(4, 4)
    assert not _verdict(m, -r, r), "a sign slip passes"
    assert not _verdict(m, r * 1.02, r), "a 2 % scale slip passes"
    assert not _verdict(m, r - 0.03 * np.abs(r), r), "an error below r passes"


def pin_one_bad_entry_among_good_fails(m):
    r = np.random.default_rng(3).standard_normal((32, 32))
    g = r.copy()
    g[31, 0] += 0.5
    res = m.gemm_check(g, r)
    assert not res["pass"] and res["n_fail"] == 1


def pin_shape_slip_fails(m):
    r = np.arange(12.0).reshape(3, 4)
    for g in (np.arange(4.0).reshape(1, 4), r.T.copy(), r.reshape(-1)):
        try:
            verdict = _verdict(m, g, r)
        except ValueError:
            continue
        assert not verdict, f"result of shape {g.shape} against reference of shape {r.shape} passes"
    # a reference that broadcasts against the result must not pass either
    try:
        verdict = _verdict(m, np.tile(np.arange(4.0), (3, 1)), np.arange(4.0).reshape(1, 4))
    except ValueError:
        verdict = False
    assert not verdict, "a broadcast reference passes"


def pin_f8_dot_term(m):
    """gemm_check_f8: the bound widens by F8_DOT_BOUND · Σ|a_k||b_k| per entry (B stored N×K)."""
    rng = np.random.default_rng(8)
    M, N, K = 6, 5, 128
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((N, K))
    ref = a @ b.T
    absum = np.abs(a) @ np.abs(b).T
    assert abs(m.F8_DOT_BOUND - 2.0 ** -13) == 0.0
    assert m.gemm_check_f8(ref, ref, a, b)["pass"]
    # an error just inside the widened bound passes, just outside fails
    base = np.maximum(1e-2 * np.abs(ref), 1e-3)
    widened = base + m.F8_DOT_BOUND * absum
    g = ref + 0.999 * widened
    assert m.gemm_check_f8(g, ref, a, b)["pass"]
    g = ref + 1.001 * widened
    res = m.gemm_check_f8(g, ref, a, b)
    assert not res["pass"] and res["n_fail"] == M * N
    # the widening is per entry: a row of A with larger magnitudes gets a wider bound
    a2 = a.copy()
    a2[0] *= 64.0
    ref2 = a2 @ b.T
    absum2 = np.abs(a2) @ np.abs(b).T
    g = ref2 + np.maximum(1e-2 * np.abs(ref2), 1e-3) + 0.5 * m.F8_DOT_BOUND * absum2
    assert m.gemm_check_f8(g, ref2, a2, b)["pass"]
    g[1, 0] = ref2[1, 0] + np.maximum(1e-2 * abs(ref2[1, 0]), 1e-3) + 2.0 * m.F8_DOT_BOUND * absum[1, 0]
    assert not m.gemm_check_f8(g, ref2, a2, b)["pass"]
    # magnitudes, not signed sums: with cancelling products Σ a·b is small but Σ|a·b| is not
    a3 = np.ones((1, K))
    b3 = np.tile(np.array([1.0, -1.0]), K // 2).reshape(1, K)
    ref3 = a3 @ b3.T  # 0
    g3 = ref3 + 1e-3 + 0.9 * m.F8_DOT_BOUND * K
    assert m.gemm_check_f8(g3, ref3, a3, b3)["pass"]
    # NaN fails however wide the bound
    g = ref.copy()
    g[0, 0] = np.nan
    assert not m.gemm_check_f8(g, ref, a * 1e6, b * 1e6)["pass"]
    # operands that are not M×K and N×K are refused or fail
    try:
        verdict = m.gemm_check_f8(ref, ref, a, b.T.copy())["pass"]
    except ValueError:
        verdict = False
    assert not verdict


ALL_PINS = [pin_exact_passes, pin_non_finite_fails, pin_relative_branch_at_and_past_the_bound,
            pin_absolute_branch_at_and_past_the_bound, pin_branch_switch_at_a_tenth, pin_sign_and_scale_slips_fail,
            pin_one_bad_entry_among_good_fails, pin_shape_slip_fails, pin_f8_dot_term]
