"""Pins of the oracle's prompt-lookup (n-gram) drafter, orc_ngram_draft.

The pages ([en] Floor 6, [zh] Level 6) describe n-gram drafting such as prompt
lookup as searching the preceding text for a chunk that is likely to repeat
and proposing what followed it, with the verification rule unchanged.  The
readings fixed here (longest key first, latest occurrence, the followed text
repeated with its period when it is shorter than K, the pending token when
nothing matches) are checked two ways: hand-worked cases, and an independent
search with Python's bytes.rfind on random small-alphabet histories."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("hist,L,K,n_max,want,want_n", [
    # suffix [5,1] last seen ending at 1; followed by 2,3,5,1 (period 4)
    ([5, 1, 2, 3, 5, 1], 5, 6, 3, [2, 3, 5, 1, 2, 3], 2),
    # nothing repeats: the pending token is proposed
    ([1, 2, 3, 4], 3, 3, 3, [4, 4, 4], 0),
    # key length capped at L; period 1
    ([7, 7], 1, 3, 4, [7, 7, 7], 1),
    # a longer key wins over a later, shorter one
    ([1, 2, 9, 2, 1, 2], 5, 4, 2, [9, 2, 1, 2], 2),
    # of two occurrences the latest wins
    ([1, 2, 3, 1, 2, 4, 1, 2], 7, 5, 2, [4, 1, 2, 4, 1], 2),
    # a single token of history
    ([3], 0, 2, 3, [3, 3], 0),
])
def test_worked_cases(hist, L, K, n_max, want, want_n):
    d, n = oracle.ngram_draft(hist, L, K, n_max)
    assert list(d) == want and n == want_n


def _by_rfind(hist, L, K, n_max):
    """Independent reading: bytes.rfind over the text before the pending token."""
    text = bytes(hist[:L])
    for n in range(min(n_max, L), 0, -1):
        idx = text.rfind(bytes(hist[L - n + 1: L + 1]))
        if idx >= 0:
            j = idx + n - 1
            p = L - j
            return [hist[j + 1 + i % p] for i in range(K)], n
    return [hist[L]] * K, 0


def test_matches_independent_search():
    rng = np.random.default_rng(11)
    for trial in range(3000):
        alpha = int(rng.integers(2, 6))
        L = int(rng.integers(0, 40))
        hist = [int(x) for x in rng.integers(0, alpha, L + 1)]
        K = int(rng.integers(1, 9))
        n_max = int(rng.integers(1, 6))
        d, n = oracle.ngram_draft(hist, L, K, n_max)
        wd, wn = _by_rfind(hist, L, K, n_max)
        assert (list(d), n) == (wd, wn), (hist, L, K, n_max)


def test_invariants_on_long_text():
    rng = np.random.default_rng(12)
    hist = [int(x) for x in rng.integers(0, 50, 3000)]
    for L in (100, 999, 2999):
        d, n = oracle.ngram_draft(hist, L, 7, 4)
        if n:
            suffix = hist[L - n + 1: L + 1]
            # the first draft token follows an occurrence of the key ...
            starts = [s for s in range(0, L - n + 1) if hist[s: s + n] == suffix]
            assert starts and hist[starts[-1] + n] == d[0]
            # ... and no longer key occurs
            if n < 4 and n < L:
                longer = hist[L - n: L + 1]
                assert not any(hist[s: s + n + 1] == longer for s in range(0, L - n))


def test_bad_arguments():
    with pytest.raises(ValueError):
        oracle.ngram_draft([1, 2], 2, 3, 2)
    with pytest.raises(ValueError):
        oracle.ngram_draft([1, 2], 1, 0, 2)
    with pytest.raises(ValueError):
        oracle.ngram_draft([1, 2], 1, 3, 0)
