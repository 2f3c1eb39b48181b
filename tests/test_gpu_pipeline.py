"""GPU parity of the whole round (draft loop, verify pass, accept/reject,
commit) against the oracle on the toy pair: 2-layer d=64 target, draft =
its first layer plus the shared LM head, vocab 256, 32-token prompt.

Teacher-forced: the oracle follows the GPU's own tokens and checks each
component (draft rows 1e-4 and samples bit-exact, target logits 2e-2 and rows
1e-4, accept/reject bit-exact on the GPU's rows, greedy tokens equal to the
oracle argmax except counted near-ties), and the committed state."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Buffers, Shadow, dev_weights, gpu_round

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def toy():
    tw = synth.weights_np(synth.TOY)
    dw = synth.self_draft_np(tw, 1)
    return tw, dw


def make_ctx(tw, dw, prompt, K, greedy, max_seq=192, graphs=True, tcfg=synth.TOY,
             dcfg=synth.TOY_DRAFT):
    import speculative_decoding_02_amd as sd
    tdev, ddev = dev_weights(tw, dw)
    ctx = sd.spec_init(tcfg, tdev, dcfg, ddev, prompt, k_max=K, max_seq=max_seq, greedy=greedy,
                       use_graphs=graphs)
    return ctx, (tdev, ddev)


@pytest.mark.parametrize("greedy", [True, False])
@pytest.mark.parametrize("K", [1, 4, 7])
def test_toy_rounds_match_oracle(toy, greedy, K):
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 32)
    seed = synth.SEED_PHILOX
    ctx, keep = make_ctx(tw, dw, prompt, K, greedy)
    sh = Shadow(synth.TOY, tw, synth.TOY_DRAFT, dw, prompt, 192, K, seed, greedy)
    b = Buffers(K, synth.TOY.vocab)
    emitted = 0
    while emitted < 64:
        g = gpu_round(sd, ctx, K, seed, b)
        n = sh.check_round(g)
        emitted += n + 1
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0
        assert st["target_len"] == sh.LT and st["draft_len"] == sh.LD
        assert st["pending"] == sh.hist[sh.LT]
    hist = sd.spec_get_history(ctx, sh.LT + 1)
    assert list(hist) == sh.hist[: sh.LT + 1]
    print(f"K={K} greedy={greedy}: logit err {sh.max_logit_err:.2e}, prob err "
          f"{sh.max_prob_err:.2e}, draft prob err {sh.max_draft_prob_err:.2e}, "
          f"near-ties {sh.near_ties}")


def test_greedy_stream_equals_plain_greedy(toy):
    """The GPU's greedy speculative stream equals the oracle's plain greedy
    decoding of the target (no near-ties expected at this size)."""
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 32)
    K = 4
    ctx, keep = make_ctx(tw, dw, prompt, K, True)
    b = Buffers(K, synth.TOY.vocab)
    n_tok = 0
    while n_tok < 64:
        g = gpu_round(sd, ctx, K, 0, b, with_rows=False)
        n_tok += g["nacc"] + 1
    st = sd.spec_get_state(ctx)
    hist = sd.spec_get_history(ctx, st["target_len"] + 1)
    gen = hist[len(prompt):][:64]
    ref = oracle.generate(oracle.Model(synth.TOY, tw), prompt, 64, greedy=True)
    np.testing.assert_array_equal(gen, ref)


def test_graph_and_eager_agree_and_repeat(toy):
    """Graph replay, plain launches and a second identical run give identical
    tokens and rows (fixed-order reductions everywhere)."""
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 20, seed=5)
    K = 4
    runs = []
    for graphs in (True, False, True):
        ctx, keep = make_ctx(tw, dw, prompt, K, False, graphs=graphs)
        b = Buffers(K, synth.TOY.vocab)
        rounds = [gpu_round(sd, ctx, K, 77, b) for _ in range(6)]
        runs.append(rounds)
        sd.spec_destroy(ctx)
    for r in runs[1:]:
        for a, c in zip(runs[0], r):
            for k in ("d", "out", "D", "T", "logits"):
                np.testing.assert_array_equal(a[k], c[k], err_msg=k)


def test_profiling_rounds_match_and_time(toy):
    """With profiling on, the graphs carry the gate/up GEMM's timestamp slots
    and the verify pass's LM-head stamps: tokens and rows are the same as
    without, every draft and verify gate/up launch and the LM head report a
    positive duration (and the LM head none without profiling)."""
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 20, seed=6)
    K = 3
    runs = []
    for prof in (False, True):
        ctx, keep = make_ctx(tw, dw, prompt, K, False)
        if prof:
            sd.spec_set_profiling(ctx, True)
        b = Buffers(K, synth.TOY.vocab)
        rounds = []
        for _ in range(4):
            rounds.append(gpu_round(sd, ctx, K, 31, b))
            h = sd.spec_head_time(ctx)
            if prof:
                t = sd.spec_kernel_times(ctx)
                assert len(t) == K * synth.TOY_DRAFT.n_layers + synth.TOY.n_layers
                assert np.all(t > 0) and np.all(t < 50.0), t
                assert 0 < h < 50.0, h
            else:
                assert h == -1.0
        runs.append(rounds)
        sd.spec_destroy(ctx)
    for a, c in zip(runs[0], runs[1]):
        for k in ("d", "out", "D", "T", "logits"):
            np.testing.assert_array_equal(a[k], c[k], err_msg=k)


def test_external_drafts_and_state_errors(toy):
    """Verify with drafts that did not come from spec_draft (one-hot D rows:
    a deterministic drafter), commit without draft, then a draft call that
    has to catch the draft cache up; and the call-order errors."""
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 16, seed=8)
    K = 3
    V = synth.TOY.vocab
    ctx, keep = make_ctx(tw, dw, prompt, K, False)
    sh = Shadow(synth.TOY, tw, synth.TOY_DRAFT, dw, prompt, 192, K, 9, False)
    b = Buffers(K, V)
    with pytest.raises(sd.SpecError) as e:
        sd.spec_commit(ctx, b.out, b.nacc)
    assert e.value.code == sd.SPEC_ERR_STATE
    with pytest.raises(sd.SpecError) as e:
        sd.spec_verify(ctx, K + 1, 9, b.d, b.D, b.out, b.nacc)
    assert e.value.code == sd.SPEC_ERR_ARG
    rng = np.random.default_rng(4)
    for _ in range(4):  # several rounds with external drafts: draft cache lags
        d = rng.integers(0, V, size=K).astype(np.int32)
        D = np.zeros((K, V), np.float32)
        D[np.arange(K), d] = 1.0
        b.d.copy_(torch.from_numpy(d)); b.D.copy_(torch.from_numpy(D))
        sd.spec_verify(ctx, K, 9, b.d, b.D, b.out, b.nacc, b.T, b.logits)
        with pytest.raises(sd.SpecError) as e:
            sd.spec_verify(ctx, K, 9, b.d, b.D, b.out, b.nacc)
        assert e.value.code == sd.SPEC_ERR_STATE
        # drafting between a verify and its commit is refused too (it would
        # re-draft the positions awaiting their decision), by every drafter
        for draft in (lambda: sd.spec_draft(ctx, K, 9, b.d, b.D),
                      lambda: sd.spec_draft_ngram(ctx, K, 3, b.d, b.D)):
            with pytest.raises(sd.SpecError) as e:
                draft()
            assert e.value.code == sd.SPEC_ERR_STATE
        sd.spec_commit(ctx, b.out, b.nacc)
        sd.spec_sync(ctx)
        T = b.T.cpu().numpy(); out = b.out.cpu().numpy(); n = int(b.nacc.cpu().numpy()[0])
        rc, n_o, out_o = oracle.verify_sample(T, D, d, 9, 0, 0, sh.LT + 1)
        assert n == n_o and list(out) == list(out_o)
        rows = [sh.hist[sh.LT]] + list(d)
        lg = oracle.forward(sh.T, sh.kvT, rows, sh.LT)
        assert np.abs(lg - b.logits.cpu().numpy()).max() < 2e-2
        sh.hist += [int(x) for x in out[: n + 1]]
        sh.LT += n + 1
    # the draft model now lags by > 7 tokens: spec_draft catches it up first
    st = sd.spec_get_state(ctx)
    assert st["draft_len"] == len(prompt) - 1 and st["target_len"] == sh.LT
    if sh.LT - sh.LD > 0:
        oracle.forward(sh.D, sh.kvD, sh.hist[sh.LD: sh.LT], sh.LD, want_logits=False)
    sh.LD = sh.LT
    for _ in range(3):
        g = gpu_round(sd, ctx, K, 9, b)
        sh.check_round(g)
    st = sd.spec_get_state(ctx)
    assert st["target_len"] == sh.LT and st["device_error"] == 0


def test_capacity_error(toy):
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 10, seed=2)
    K = 4
    ctx, keep = make_ctx(tw, dw, prompt, K, True, max_seq=24)
    b = Buffers(K, synth.TOY.vocab)
    with pytest.raises(sd.SpecError) as e:
        for _ in range(20):
            gpu_round(sd, ctx, K, 0, b, with_rows=False)
    assert e.value.code == sd.SPEC_ERR_CAPACITY
    st = sd.spec_get_state(ctx)
    assert st["device_error"] == 0 and st["target_len"] + K + 1 > 24


def test_resume_from_committed_prefix(toy):
    """Re-initialising from the committed history with the same seed
    reproduces the continuation (uniforms are keyed by position)."""
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 12, seed=6)
    K = 3
    ctx, keep = make_ctx(tw, dw, prompt, K, False)
    b = Buffers(K, synth.TOY.vocab)
    for _ in range(3):
        gpu_round(sd, ctx, K, 5, b, with_rows=False)
    st = sd.spec_get_state(ctx)
    prefix = sd.spec_get_history(ctx, st["target_len"] + 1)
    cont1 = [gpu_round(sd, ctx, K, 5, b, with_rows=False)["out"] for _ in range(4)]
    ctx2, keep2 = make_ctx(tw, dw, prefix, K, False)
    cont2 = [gpu_round(sd, ctx2, K, 5, b, with_rows=False)["out"] for _ in range(4)]
    for x, y in zip(cont1, cont2):
        np.testing.assert_array_equal(x, y)
