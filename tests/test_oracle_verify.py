"""Pins for the oracle's accept/reject rule (sampling and greedy variants)
against what the pages fix: the greedy quiz and the two Boss-level rounds,
the 1..K+1 tokens-per-round bound, distribution preservation (chi-square),
per-position acceptance sum_v min(T, D), and the Floor-6 tokens-per-round
formula."""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
import synth
from conftest import golden


def one_hot_rows(ids, V):
    T = np.zeros((len(ids), V), np.float32)
    T[np.arange(len(ids)), ids] = 1.0
    return T


# ------------------------------------------------------------ greedy pins --
def test_level4_greedy_quiz():
    g = golden("level4_greedy_quiz.json")
    vocab = g["vocab"]
    ix = {w: i for i, w in enumerate(vocab)}
    T = one_hot_rows([ix[w] for w in g["target_top"]], len(vocab))
    d = [ix[w] for w in g["draft"]]
    rc, n, out = oracle.verify_greedy(T, d)
    assert rc == 0
    assert n == g["n_accepted"]
    assert [vocab[i] for i in out[: n + 1]] == g["committed"]


def test_boss_level_two_rounds():
    g = golden("boss_two_rounds.json")
    vocab = g["vocab"]
    ix = {w: i for i, w in enumerate(vocab)}
    total, passes = 0, 0
    for rnd in g["rounds"]:
        T = one_hot_rows([ix[w] for w in rnd["target_top"]], len(vocab))
        d = [ix[w] for w in rnd["draft"]]
        rc, n, out = oracle.verify_greedy(T, d)
        passes += 1
        assert rc == 0 and n == rnd["n_accepted"]
        assert [vocab[i] for i in out[: n + 1]] == rnd["emitted"]
        total += n + 1
        # the sampling rule on one-hot rows reaches the same decision
        for u in (0, (1 << 24) - 1):
            rc2, n2, out2 = oracle.verify_sample_u(T, T[:-1], d, [u] * len(d), u)
            assert rc2 == 0 and n2 == n and list(out2[: n + 1]) == list(out[: n + 1])
    assert total == g["total_tokens"] and passes == g["target_passes"]


def test_one_hot_sampling_equals_greedy():
    rng = np.random.default_rng(9)
    V = 12
    for _ in range(300):
        K = int(rng.integers(1, 8))
        top = rng.integers(0, V, size=K + 1)
        d = rng.integers(0, V, size=K)
        # make prefixes of matches common
        m = int(rng.integers(0, K + 1))
        d[:m] = top[:m]
        T = one_hot_rows(top, V)
        D = one_hot_rows(d, V)
        rg, ng, og = oracle.verify_greedy(T, d)
        rs, ns, os_ = oracle.verify_sample(T, D, d, 1003, 0, int(rng.integers(0, 1 << 30)), 40)
        assert rg == rs == 0 and ng == ns and list(og[: ng + 1]) == list(os_[: ns + 1])


# -------------------------------------------------------- bounds & errors --
def test_tokens_per_round_between_1_and_K_plus_1():
    for sigma in (0.1, 0.5, 2.0):
        T, D = synth.logit_pair(16, 6, 500, sigma)
        d = np.stack([oracle.draft_sample_batch(D[:, i, :], 1003, 100 + i) for i in range(6)], 1)
        for greedy in (False, True):
            out, n = oracle.accept_reject_batch(T, D, d, 1003, np.full(16, 100), 0, greedy)
            assert np.all(n >= 0) and np.all(n <= 6)
            for b in range(16):
                emitted = out[b, : n[b] + 1]
                assert np.all(emitted >= 0) and np.all(emitted < 500)
                assert np.all(out[b, n[b] + 1:] == -1)
                # accepted prefix equals the drafts
                assert list(emitted[: n[b]]) == list(d[b, : n[b]])


def test_invalid_inputs_are_errors():
    T = np.full((2, 4), 0.25, np.float32)
    D = np.full((1, 4), 0.25, np.float32)
    rc, n, out = oracle.verify_sample(T, D, [7], 1, 0, 0, 0)  # draft out of range
    assert rc != 0 and n == -1 and list(out) == [-1, -1]
    Tn = T.copy(); Tn[0, 2] = np.nan
    rc, n, _ = oracle.verify_sample(Tn, D, [2], 1, 0, 0, 0)   # gathered NaN
    assert rc == oracle.EBADPROB and n == -1
    rc, n, _ = oracle.verify_greedy(Tn, [0])                   # greedy reads every row
    assert rc == oracle.EBADPROB
    Tb = T.copy(); Tb[1, 0] = 1.5                                 # invalid value in bonus row
    rc, n, _ = oracle.verify_sample(Tb, D, [1], 1, 0, 0, 0)
    assert rc == oracle.EBADPROB


def test_empty_residual_falls_back_to_target_row():
    # T == D exactly: a reject leaves no residual mass; the replacement is drawn
    # from T itself.  Force a reject with D(d) > T(d) impossible here, so use a
    # row where T(d) = 0 = D(d) (T = D = 0 rejects) and T == D elsewhere.
    T = np.array([[0.0, 0.5, 0.5], [1 / 3, 1 / 3, 1 / 3]], np.float32)
    D = np.array([[0.0, 0.5, 0.5]], np.float32)
    rc, n, out = oracle.verify_sample_u(T, D, [0], [0], 0)
    assert rc == 0 and n == 0 and out[0] == 1
    rc, n, out = oracle.verify_sample_u(T, D, [0], [0], (1 << 24) - 1)
    assert rc == 0 and n == 0 and out[0] == 2


# ------------------------------------------- distribution preservation ----
def _pipeline_first_token(T, D, K, trials, seed=1003, c=0):
    """Full sampling procedure: drafts from D rows via the draft sampler, then
    the rule.  Every trial is a separate sequence s = trial."""
    V = T.shape[-1]
    B = trials
    Tb = np.broadcast_to(T, (B, K + 1, V))
    Db = np.broadcast_to(D, (B, K, V))
    pos = np.full(B, 50, np.uint64)
    d = np.stack([oracle.draft_sample_batch(np.broadcast_to(D[i], (B, V)), seed, 50 + i, c)
                  for i in range(K)], 1)
    out, n = oracle.accept_reject_batch(Tb, Db, d, seed, pos, c, False)
    return out, n, d


@pytest.mark.slow
@pytest.mark.parametrize("which", ["dirichlet", "reversed", "uniform"])
def test_vocab8_output_distribution_equals_target(which):
    """Vocab 8, T and D ~ Dirichlet(1), 1e6 trials: the emitted token follows
    T (chi-square, p > 0.01).  A poor drafter (T reversed, or uniform) changes
    only the acceptance rate, never the output law."""
    T, D = synth.dirichlet_pair(8)
    if which == "reversed":
        D = T[::-1].copy()
    elif which == "uniform":
        D = np.full(8, 1 / 8, np.float32)
    Tk = np.stack([T, T])
    Dk = D[None, :]
    out, n, _ = _pipeline_first_token(Tk, Dk, 1, 1_000_000)
    counts = np.bincount(out[:, 0], minlength=8)
    expected = T.astype(np.float64) / T.astype(np.float64).sum() * counts.sum()
    chi2, p = stats.chisquare(counts, expected)
    assert p > 0.01, (which, chi2, p)


@pytest.mark.slow
def test_per_position_acceptance_matches_sum_min():
    """Acceptance of draft i given it is reached equals
    beta_i = sum_v min(T_i(v), D_i(v)) (binomial z-test)."""
    V, K, trials = 50, 4, 200_000
    rng = np.random.default_rng(21)
    T = rng.dirichlet(np.ones(V), size=K + 1).astype(np.float32)
    D = rng.dirichlet(np.ones(V) * 0.7, size=K).astype(np.float32)
    beta = np.minimum(T[:K].astype(np.float64), D.astype(np.float64)).sum(1)
    out, n, d = _pipeline_first_token(T, D, K, trials)
    for i in range(K):
        reached = n >= i
        acc = n[reached] > i
        k, m = int(acc.sum()), int(reached.sum())
        z = (k - m * beta[i]) / math.sqrt(m * beta[i] * (1 - beta[i]))
        assert abs(z) < 4.5, (i, k / m, beta[i], z)
    # E[n_acc] = sum_j prod_{i<=j} beta_i
    mean = n.mean()
    want = oracle.expected_accepted(beta)
    sd = n.std() / math.sqrt(trials)
    assert abs(mean - want) < 5 * sd


def test_floor6_tokens_per_round_formula():
    g = golden("floor6_tokens_per_round.json")
    for case in g["cases"]:
        v = oracle.expected_tokens_per_round(case["alpha"], case["k"])
        assert round(v, g["printed_decimals"]) == case["printed"]
        # the product form reduces to it when every beta_i = alpha
        assert abs(oracle.expected_accepted([case["alpha"]] * case["k"]) + 1 - v) < 1e-12


@pytest.mark.slow
def test_iid_acceptance_mean_tokens_per_round():
    """Rows built so every position has beta = alpha: the mean number of
    emitted tokens per round is (1 - alpha^(K+1)) / (1 - alpha)."""
    K, V, trials = 4, 4, 200_000
    for alpha in (0.8, 0.5):
        # T = (alpha, 1-alpha, 0, 0), D = (1, 0, 0, 0): sum min = alpha
        T = np.tile(np.array([alpha, 1 - alpha, 0, 0], np.float32), (K + 1, 1))
        D = np.tile(np.array([1, 0, 0, 0], np.float32), (K, 1))
        out, n, _ = _pipeline_first_token(T, D, K, trials)
        emitted = n + 1
        want = oracle.expected_tokens_per_round(alpha, K)
        assert abs(emitted.mean() - want) < 5 * emitted.std() / math.sqrt(trials)
