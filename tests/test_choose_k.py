"""Choosing K from the measured acceptance rate: the oracle's helpers pinned
to the pages, and the library's host-side helpers (spec_expected_tokens,
spec_alpha_from_tokens, spec_choose_k) checked against the oracle's.  No GPU
is touched: these are plain host functions of libspec.

[en] Floor 6 gives the mean tokens per round under iid acceptance; [int]
"speedup" gives the round cost, K draft steps plus one target pass."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "floor6_tokens_per_round.json")


def _lib():
    sd = pytest.importorskip("speculative_decoding_02_amd")
    try:
        sd.binding.lib()
    except ImportError as e:
        pytest.skip(str(e))
    return sd


def test_oracle_expected_tokens_matches_floor6_table():
    g = json.load(open(GOLDEN))
    for c in g["cases"]:
        assert round(oracle.expected_tokens(c["alpha"], c["k"]), g["printed_decimals"]) == c["printed"]
    assert oracle.expected_tokens(1.0, 5) == 6.0
    assert oracle.expected_tokens(0.0, 5) == 1.0


def test_oracle_choose_k_special_cases():
    # nothing is ever accepted: every K yields one token, the cheapest round wins
    assert oracle.choose_k(0.0, 0.5, 3.0, 7) == 1
    # everything is accepted and drafting is free: as many as allowed
    assert oracle.choose_k(1.0, 0.0, 3.0, 7) == 7
    # everything accepted: (K+1)/(K t_d + t_v) grows with K iff t_v > t_d
    assert oracle.choose_k(1.0, 1.0, 3.0, 6) == 6
    assert oracle.choose_k(1.0, 3.0, 1.0, 6) == 1
    assert oracle.choose_k(1.0, 2.0, 2.0, 6) == 1  # flat: ties go to the smaller K


def test_oracle_choose_k_monotone():
    rng = np.random.default_rng(3)
    for _ in range(300):
        td, tv, km = float(rng.uniform(0.01, 2)), float(rng.uniform(0.5, 5)), int(rng.integers(1, 9))
        ks = [oracle.choose_k(a, td, tv, km) for a in np.linspace(0, 1, 41)]
        assert all(x <= y for x, y in zip(ks, ks[1:]))  # more acceptance, longer drafts
        a = float(rng.uniform(0, 1))
        ks = [oracle.choose_k(a, t, tv, km) for t in np.linspace(0.01, 3, 41)]
        assert all(x >= y for x, y in zip(ks, ks[1:]))  # dearer drafts, shorter drafts


def test_library_matches_oracle():
    sd = _lib()
    rng = np.random.default_rng(4)
    for _ in range(2000):
        a, K = float(rng.uniform(0, 1)), int(rng.integers(1, 16))
        assert sd.spec_expected_tokens(a, K) == oracle.expected_tokens(a, K)
        td, tv, km = float(rng.uniform(0, 2)), float(rng.uniform(0.1, 5)), int(rng.integers(1, 9))
        assert sd.spec_choose_k(a, td, tv, km) == oracle.choose_k(a, td, tv, km)


def test_library_alpha_from_tokens_round_trip():
    sd = _lib()
    for K in (1, 2, 4, 7):
        for a in np.linspace(0.01, 0.99, 25):
            t = oracle.expected_tokens(float(a), K)
            assert abs(sd.spec_alpha_from_tokens(t, K) - a) < 1e-9
        assert sd.spec_alpha_from_tokens(1.0, K) == 0.0
        assert sd.spec_alpha_from_tokens(0.5, K) == 0.0
        assert sd.spec_alpha_from_tokens(K + 1.0, K) == 1.0


def test_library_choose_k_errors():
    sd = _lib()
    for args in ((-0.1, 1, 1, 4), (1.1, 1, 1, 4), (0.5, -1, 1, 4), (0.5, 0, 0, 4), (0.5, 1, 1, 0)):
        with pytest.raises(sd.SpecError) as e:
            sd.spec_choose_k(*args)
        assert e.value.code == sd.SPEC_ERR_ARG
    with pytest.raises(ValueError):
        oracle.choose_k(0.5, 1.0, 1.0, 0)
