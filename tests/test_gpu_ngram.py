"""GPU parity of the prompt-lookup (n-gram) drafter, spec_draft_ngram, and of
verify rounds fed by it ([en] Floor 6: drafts from repeated chunks of the
preceding text; the verification rule is the same whatever the source).

Each round is teacher-forced: the GPU's draft tokens must equal the oracle's
orc_ngram_draft on the GPU's committed history (bit-exact, integer work), its
draft rows must be exactly one-hot, and the accept/reject outcome must equal
the oracle rule on the GPU's own target rows with those one-hot rows.  In
greedy mode the whole stream must equal the oracle's plain greedy decoding,
token for token, whatever the drafts were."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Buffers, dev_weights

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _ctx(tcfg, tw, dcfg, dw, prompt, K, greedy, max_seq):
    import speculative_decoding_02_amd as sd
    tdev, ddev = dev_weights(tw, dw)
    ctx = sd.spec_init(tcfg, tdev, dcfg, ddev, prompt, k_max=K, max_seq=max_seq, greedy=greedy)
    return ctx, (tdev, ddev)


def _round(sd, ctx, K, n_max, seed, b, greedy):
    st = sd.spec_get_state(ctx)
    hist = sd.spec_get_history(ctx, st["target_len"] + 1)
    sd.spec_draft_ngram(ctx, K, n_max, b.d, None if greedy else b.D)
    sd.spec_verify(ctx, K, seed, b.d, b.D, b.out, b.nacc, b.T, b.logits)
    sd.spec_commit(ctx, b.out, b.nacc)
    sd.spec_sync(ctx)
    d = b.d.cpu().numpy()
    want, n = oracle.ngram_draft(hist, st["target_len"], K, n_max)
    np.testing.assert_array_equal(d, want)
    out = b.out.cpu().numpy()
    nacc = int(b.nacc.cpu().numpy()[0])
    T = b.T.cpu().numpy()
    if greedy:
        rc, n_o, out_o = oracle.verify_greedy(T, d)
    else:
        D = b.D.cpu().numpy()
        onehot = np.zeros_like(D)
        onehot[np.arange(K), d] = 1.0
        np.testing.assert_array_equal(D, onehot)
        rc, n_o, out_o = oracle.verify_sample(T, D, d, seed, 0, 0, st["target_len"] + 1)
    assert (nacc, list(out)) == (n_o, list(out_o))
    return nacc, n


@pytest.mark.parametrize("n_max", [1, 3])
def test_greedy_stream_equals_plain_greedy(n_max):
    import speculative_decoding_02_amd as sd
    tw = synth.weights_np(synth.TOY)
    dw = synth.self_draft_np(tw, 1)
    prompt = synth.prompt(synth.TOY.vocab, 32)
    K = 4
    ctx, keep = _ctx(synth.TOY, tw, synth.TOY_DRAFT, dw, prompt, K, True, 192)
    b = Buffers(K, synth.TOY.vocab)
    n_tok, hits = 0, 0
    while n_tok < 64:
        nacc, n = _round(sd, ctx, K, n_max, 0, b, True)
        n_tok += nacc + 1
        hits += n > 0
    st = sd.spec_get_state(ctx)
    gen = sd.spec_get_history(ctx, st["target_len"] + 1)[len(prompt):][:64]
    ref = oracle.generate(oracle.Model(synth.TOY, tw), prompt, 64, greedy=True)
    np.testing.assert_array_equal(gen, ref)
    assert hits > 0
    sd.spec_destroy(ctx)


def test_sampling_rounds_and_repeating_prompt():
    """A prompt that repeats with period 3 (< K) exercises long keys and the
    periodic continuation; sampling mode checks the one-hot rows and the rule."""
    import speculative_decoding_02_amd as sd
    tw = synth.weights_np(synth.TOY)
    dw = synth.self_draft_np(tw, 1)
    prompt = np.array([17, 4, 99] * 10 + [17, 4], np.int32)
    K = 7
    ctx, keep = _ctx(synth.TOY, tw, synth.TOY_DRAFT, dw, prompt, K, False, 192)
    b = Buffers(K, synth.TOY.vocab)
    lens = []
    for _ in range(12):
        nacc, n = _round(sd, ctx, K, 8, 1003, b, False)
        lens.append(n)
    assert lens[0] == 8  # the first key is the full 8 tokens of the repeating text
    # the draft model was never run: its cache still holds the prompt only
    st = sd.spec_get_state(ctx)
    assert st["draft_len"] == len(prompt) - 1 and st["device_error"] == 0
    # a model draft round afterwards catches the draft cache up first
    sd.spec_draft(ctx, K, 5, b.d, b.D)
    sd.spec_verify(ctx, K, 5, b.d, b.D, b.out, b.nacc)
    sd.spec_commit(ctx, b.out, b.nacc)
    st = sd.spec_get_state(ctx)
    assert st["device_error"] == 0 and st["draft_len"] >= st["target_len"] - K
    sd.spec_destroy(ctx)


def test_large_vocab_rows_and_errors():
    """One-hot rows over a 32000-token vocabulary (1.3B-shaped slice sharing
    its embedding and head), K = 6; bad n_max and missing rows are refused."""
    import speculative_decoding_02_amd as sd
    tcfg = synth.L13B.replace(name="1.3b-slice-1L", n_layers=1)
    dcfg = synth.L13B_DRAFT.replace(name="1.3b-draft-1L", n_layers=1)
    tw = synth.weights_torch(tcfg, device="cuda")
    dw = synth.weights_torch(dcfg, seed=synth.SEED_WEIGHTS + 1, device="cuda", share_from=tw,
                             share=("embed", "lm_head"))
    prompt = synth.prompt(tcfg.vocab, 40, seed=21)
    prompt[-3:] = prompt[5:8]  # a 3-token key that occurred before
    K = 6
    ctx = sd.spec_init(tcfg, tw, dcfg, dw, prompt, k_max=K, max_seq=128, greedy=False)
    b = Buffers(K, tcfg.vocab)
    for _ in range(3):
        _round(sd, ctx, K, 4, 77, b, False)
    for bad in (0, 9):
        with pytest.raises(sd.SpecError) as e:
            sd.spec_draft_ngram(ctx, K, bad, b.d, b.D)
        assert e.value.code == sd.SPEC_ERR_ARG
    with pytest.raises(sd.SpecError) as e:
        sd.spec_draft_ngram(ctx, K, 3, b.d, None)  # sampling mode needs the rows
    assert e.value.code == sd.SPEC_ERR_ARG
    sd.spec_destroy(ctx)
