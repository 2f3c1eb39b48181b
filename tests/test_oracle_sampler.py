"""Pins for the oracle's sampler primitives: fix, the inverse-CDF sampler,
argmax_low and the exact accept predicate, plus the pages' worked example of
the accept/reject rule, enumerated exactly over the 2^24 uniform grid."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import golden

GRID = 1 << 24


def F(x) -> Fraction:
    """Exact rational value of an fp32 number."""
    return Fraction(float(np.float32(x)))


# ------------------------------------------------------------------ fix --
@pytest.mark.parametrize("x,want", [
    (0.0, 0), (-0.0, 0), (1.0, 1 << 40), (0.5, 1 << 39), (2.0**-40, 1), (2.0**-41, 0),
    (0.1, int(Fraction(float(np.float32(0.1))) * (1 << 40))),
    (np.float32(1) - np.float32(2**-24), (1 << 40) - (1 << 16)),
])
def test_fix_exact(x, want):
    assert oracle.fix(x) == want


@pytest.mark.parametrize("x", [np.nan, np.inf, -np.inf, -1e-30, 1.0000001, 2.0])
def test_fix_rejects_invalid(x):
    with pytest.raises(ValueError):
        oracle.fix(x)


# ---------------------------------------------------------- sample_icdf --
def closed_form_counts(q):
    """#{u in [0,2^24) : C_{v-1} <= floor(u Z / 2^24) < C_v}
       = ceil(C_v 2^24 / Z) - ceil(C_{v-1} 2^24 / Z), in exact integers."""
    Z = sum(q)
    C = np.cumsum([0] + list(q)).tolist()

    def ceil_div(a, b):
        return -((-a) // b)

    return [ceil_div(C[v + 1] * GRID, Z) - ceil_div(C[v] * GRID, Z) for v in range(len(q))]


@pytest.mark.parametrize("q", [
    [1, 1, 1],
    [3, 0, 5, 0, 1],
    [0, 0, 7],
    [(1 << 40), 0, 1],
    [123456789012, 987654321, 5, 0, 77777777777, 1, 2, 3],
    [(1 << 40) - 1, (1 << 40) - 3, (1 << 39) + 17],
])
def test_icdf_brute_force_matches_closed_form(q):
    counts = oracle.icdf_histogram(q).tolist()
    assert counts == closed_form_counts(q)
    assert sum(counts) == GRID
    Z = sum(q)
    for v, cnt in enumerate(counts):
        assert abs(Fraction(cnt, GRID) - Fraction(q[v], Z)) <= Fraction(1, GRID)
        if q[v] == 0:
            assert cnt == 0  # zero-mass tokens are never drawn


def test_icdf_empty_is_none():
    assert oracle.sample_icdf([0, 0, 0], 12345) == -1


def test_icdf_extreme_needles():
    q = [5, 0, 3]
    assert oracle.sample_icdf(q, 0) == 0
    assert oracle.sample_icdf(q, GRID - 1) == 2


# ---------------------------------------------------------------- argmax --
def test_argmax_low_matches_numpy_first_occurrence():
    rng = np.random.default_rng(3)
    for _ in range(500):
        V = int(rng.integers(1, 40))
        x = rng.integers(0, 4, size=V).astype(np.float32) / 4  # many ties
        assert oracle.argmax_low(x) == int(np.argmax(x))


def test_argmax_low_nan_is_error():
    assert oracle.argmax_low(np.array([0.1, np.nan, 0.2], np.float32)) == -2


# ---------------------------------------------------------------- accept --
def exact_accept(r, T, D):
    return F(r) * F(D) < F(T)


def test_accept_predicate_exact_random():
    rng = np.random.default_rng(11)
    for _ in range(20000):
        r = np.float32(rng.integers(0, GRID) / GRID)
        T = np.float32(rng.random() ** rng.integers(1, 8))
        D = np.float32(rng.random() ** rng.integers(1, 8))
        if rng.random() < 0.2:
            D = T  # ties
        assert oracle.accept(r, T, D) == exact_accept(r, T, D)


@pytest.mark.parametrize("r,T,D,want", [
    (0.0, 0.0, 0.0, False),            # T = D = 0 rejects
    (0.0, 1e-30, 0.0, True),           # D = 0, T > 0 accepts (T/D -> inf)
    (0.999, 1e-38, 0.0, True),
    (0.0, 0.0, 0.5, False),            # T = 0 never accepts
    (0.0, 0.25, 0.25, True),           # T = D always passes
    (1 - 2**-24, 0.25, 0.25, True),
    (1 - 2**-24, 1e-45, 1e-45, True),  # subnormal tie
    (0.5, 0.25, 0.5, False),           # r = T/D exactly is not "<"
    (0.5 - 2**-24, 0.25, 0.5, True),
])
def test_accept_edges(r, T, D, want):
    assert oracle.accept(r, T, D) == want == exact_accept(r, T, D)


def test_quiz_floor5_accept_probability_one():
    g = golden("floor5_quiz.json")
    n = oracle.accept_count(g["target_p"], g["draft_q"])
    assert Fraction(n, GRID) == Fraction(g["accept_probability"]).limit_denominator(1)


# ------------------------------------------------- worked example (exact) --
def test_floor5_worked_example_exact():
    g = golden("floor5_worked_example.json")
    T = np.array(g["target_p"], np.float32)
    D = np.array(g["draft_q"], np.float32)
    V = 3
    # P(draft = v): the draft spins its own wheel on fix(D)
    qD = [oracle.fix(x) for x in D]
    pd = [Fraction(int(c), GRID) for c in oracle.icdf_histogram(qD)]
    # P(accept | v): exact count of u24 with r * D < T
    pacc = [Fraction(oracle.accept_count(T[v], D[v]), GRID) for v in range(V)]
    # closed form of the same count from the exact rationals
    for v in range(V):
        want = min(GRID, -((-F(T[v]) * GRID) // F(D[v])))
        assert oracle.accept_count(T[v], D[v]) == want
    # residual wheel fix(T) - fix(D), saturating, then the sampler
    q_res = [max(0, oracle.fix(T[v]) - oracle.fix(D[v])) for v in range(V)]
    pres = [Fraction(int(c), GRID) for c in oracle.icdf_histogram(q_res)]

    tol = Fraction(3, GRID) + Fraction(V, 1 << 40) + Fraction(1, 10**7)
    branch_accept = [pd[v] * pacc[v] for v in range(V)]
    rejected = sum(pd[v] * (1 - pacc[v]) for v in range(V))
    assert abs(branch_accept[0] - Fraction(g["branch_accept_round"])) < tol
    assert abs(branch_accept[1] - Fraction(g["branch_accept_bright"])) < tol
    assert abs(branch_accept[2] - Fraction(g["branch_accept_lovely"])) < tol
    assert abs(rejected - Fraction(g["branch_reject_after_round"])) < tol
    assert abs(pacc[0] - Fraction(g["accept_prob_round"])) < tol
    for v in range(V):
        assert abs(pres[v] - Fraction(g["residual_normalized"][v])) < tol
    final = [branch_accept[v] + rejected * pres[v] for v in range(V)]
    for v in range(V):
        assert abs(final[v] - Fraction(g["final_distribution"][v])) < tol
    # rejected mass equals the residual area (over-bet = under-bet)
    area = Fraction(sum(q_res), 1 << 40)
    assert abs(area - Fraction(g["rejected_mass_equals_residual_area"])) < tol


def test_worked_example_through_verify_sample_u():
    """The same example through the full rule with explicit uniforms: every
    accept/reject/residual branch lands where the enumeration says."""
    g = golden("floor5_worked_example.json")
    T = np.array([g["target_p"], g["target_p"]], np.float32)  # row 2 = bonus row
    D = np.array([g["draft_q"]], np.float32)
    # draft "round" with r just below / at 0.625 -> accept / reject
    below = int(0.625 * GRID) - 1
    rc, n, out = oracle.verify_sample_u(T, D, [0], [below], 0)
    assert rc == 0 and n == 1 and out[0] == 0
    rc, n, out = oracle.verify_sample_u(T, D, [0], [int(0.625 * GRID)], 0)
    assert rc == 0 and n == 0 and out[0] == 1          # residual needle 0 -> "bright"
    rc, n, out = oracle.verify_sample_u(T, D, [0], [GRID - 1], GRID - 1)
    assert rc == 0 and n == 0 and out[0] == 2          # residual needle at top -> "lovely"
    # "bright" and "lovely" always pass
    for d in (1, 2):
        rc, n, out = oracle.verify_sample_u(T, D, [d], [GRID - 1], 0)
        assert rc == 0 and n == 1 and out[0] == d


# ----------------------------------------------------------- mass balance --
def test_mass_balance_random_pairs():
    """sum_v (T-D)+ = 1 - sum_v min(T, D) on the 2^-40 grid, up to one grid
    step per entry from the floors."""
    rng = np.random.default_rng(5)
    for V in (2, 3, 17, 1000):
        for _ in range(20):
            T = rng.dirichlet(np.ones(V)).astype(np.float32)
            D = rng.dirichlet(np.ones(V)).astype(np.float32)
            fT = np.array([oracle.fix(x) for x in T], dtype=object)
            fD = np.array([oracle.fix(x) for x in D], dtype=object)
            res = sum(max(0, a - b) for a, b in zip(fT, fD))
            mins = sum(min(F(a), F(b)) for a, b in zip(T, D))
            tot = sum(F(a) for a in T)  # fp32 rows sum to 1 only approximately
            exact = (tot - mins) * (1 << 40)
            assert abs(Fraction(res) - exact) <= V
