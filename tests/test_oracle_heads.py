"""Pins for the oracle's multi-token-prediction head drafter.

The pages ("Speculative decoding internals", variants: MTP) give the idea --
the target carries extra output heads, head k predicting the token k places
ahead -- but no head architecture; the oracle's reading is
z_k = h + silu(W_k h) scored by the target's own LM head.  What is fixed
independently of that code:
  * zero head matrices reduce every head to the target's own LM head at the
    same position (silu(0) = 0), so D_k must equal the T row of the forward
    pass at that position, bit for bit;
  * W_k = a I turns the head into an elementwise map, computed here with
    numpy/scipy (expit for the sigmoid, a matrix product and a softmax);
  * head k uses matrix k only (permuting the matrices permutes the rows);
  * greedy speculative output equals plain greedy decoding whatever the
    drafts ([int] algorithm core; [en] Floor 4);
  * every round drafts from the state of the last committed position, which a
    fresh forward pass over the committed text reproduces exactly (the forward
    is row-invariant).
"""
import numpy as np
import pytest
from scipy import special

import oracle
import synth

N_HEADS = 4


@pytest.fixture(scope="module")
def toy():
    w = synth.weights_np(synth.TOY)
    return oracle.Model(synth.TOY, w), w


def last_state(model, tokens):
    """(final normed state, T row) of the last of `tokens` from a fresh forward."""
    kv = oracle.KV(model, len(tokens) + 4)
    lg, hid = oracle.forward_hidden(model, kv, tokens, 0)
    return hid[-1], oracle.softmax_f32(lg[-1])


def test_zero_heads_reproduce_the_target_head(toy):
    tgt, _ = toy
    pr = synth.prompt(synth.TOY.vocab, 20)
    h, T = last_state(tgt, pr)
    W = np.zeros((N_HEADS, 64, 64), np.uint16)
    D, d = oracle.heads_draft(tgt, W, h, N_HEADS, greedy=True, seed=synth.SEED_PHILOX, P=20)
    for k in range(N_HEADS):
        assert np.array_equal(D[k], T)
    assert np.all(d == oracle.argmax_low(T))


@pytest.mark.parametrize("a", [0.5, 2.0, -1.0, 8.0])
def test_scaled_identity_heads_closed_form(toy, a):
    tgt, w = toy
    pr = synth.prompt(synth.TOY.vocab, 12, seed=5)
    h, _ = last_state(tgt, pr)
    d_model = synth.TOY.d_model
    eye = synth.f32_to_bf16_bits(np.eye(d_model, dtype=np.float32) * np.float32(a))
    W = np.stack([eye] * 2)
    D, _ = oracle.heads_draft(tgt, W, h, 2, greedy=True, seed=1, P=12)
    z = h + special.expit(a * h) * (a * h)  # silu(a h) elementwise
    lm = synth.bf16_bits_to_f32(w["lm_head"]).astype(np.float64)
    ref = special.softmax(lm @ z)
    for k in range(2):
        np.testing.assert_allclose(D[k], ref, rtol=2e-6, atol=1e-9)


def test_head_k_uses_matrix_k(toy):
    tgt, _ = toy
    W = synth.heads_np(synth.TOY, N_HEADS)
    h, _ = last_state(tgt, synth.prompt(synth.TOY.vocab, 9, seed=3))
    D, _ = oracle.heads_draft(tgt, W, h, N_HEADS, greedy=True, seed=1, P=9)
    perm = [2, 0, 3, 1]
    Dp, _ = oracle.heads_draft(tgt, W[perm], h, N_HEADS, greedy=True, seed=1, P=9)
    for k in range(N_HEADS):
        assert np.array_equal(Dp[k], D[perm[k]])
    # fewer heads drafted: the first rows are the same
    D2, _ = oracle.heads_draft(tgt, W, h, 2, greedy=True, seed=1, P=9)
    assert np.array_equal(D2, D[:2])


def test_sampled_drafts_use_word0_at_their_positions(toy):
    tgt, _ = toy
    W = synth.heads_np(synth.TOY, N_HEADS)
    h, _ = last_state(tgt, synth.prompt(synth.TOY.vocab, 15, seed=4))
    P = 15
    D, d = oracle.heads_draft(tgt, W, h, N_HEADS, greedy=False, seed=77, P=P, c=3)
    for k in range(N_HEADS):
        assert d[k] == oracle.draft_sample(D[k], 77, P + k, 0, 3, greedy=False)


@pytest.mark.parametrize("K", [1, 2, 4])
@pytest.mark.parametrize("zero", [False, True])
def test_greedy_stream_equals_plain_greedy(toy, K, zero):
    tgt, _ = toy
    W = (np.zeros((N_HEADS, 64, 64), np.uint16) if zero else synth.heads_np(synth.TOY, N_HEADS))
    pr = synth.prompt(synth.TOY.vocab, 24)
    plain = oracle.generate(tgt, pr, 40, greedy=True)
    spec, nacc, drafts, st = oracle.spec_generate_heads(tgt, W, pr, 40, K, greedy=True)
    assert np.array_equal(plain, spec)
    assert np.all(nacc >= 0) and np.all(nacc <= K)
    assert st["target_passes"] == st["rounds"] == st["draft_passes"]
    assert drafts.shape == (st["rounds"], K)


def test_drafts_follow_the_last_committed_state(toy):
    """Each round's drafts equal heads_draft on the state of position LT-1
    recomputed from scratch over the committed text."""
    tgt, _ = toy
    W = synth.heads_np(synth.TOY, N_HEADS)
    pr = synth.prompt(synth.TOY.vocab, 16, seed=11)
    K, seed, n_new = 3, synth.SEED_PHILOX, 30
    out, nacc, drafts, st = oracle.spec_generate_heads(tgt, W, pr, n_new, K, greedy=False,
                                                       seed=seed)
    hist = np.concatenate([pr, out])
    LT = len(pr) - 1
    for r in range(st["rounds"]):
        h, _ = last_state(tgt, hist[:LT])
        _, d = oracle.heads_draft(tgt, W, h, K, greedy=False, seed=seed, P=LT + 1)
        assert np.array_equal(d, drafts[r]), r
        LT += int(nacc[r]) + 1
        if LT >= len(hist):
            break


def test_argument_errors(toy):
    tgt, _ = toy
    W = synth.heads_np(synth.TOY, 2)
    h = np.zeros(64)
    with pytest.raises(ValueError):
        oracle.heads_draft(tgt, W, h, 3, greedy=True, seed=0, P=1)  # K > heads
    with pytest.raises(ValueError):
        oracle.spec_generate_heads(tgt, W, [5], 4, 1, greedy=True)  # nothing prefilled
