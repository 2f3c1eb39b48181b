"""GPU parity of the multi-token-prediction head drafter (spec_heads_init /
spec_draft_heads) against the oracle.

Teacher-forced rounds: the oracle keeps the target's final normed state of
the last committed position, drafts with the same heads and checks the GPU's
head rows (1e-4) and draft samples (bit-exact on the GPU's own rows), then
the verify pass (logits 2e-2, rows 1e-4), the rule (bit-exact on the GPU's
rows), greedy near-ties, and the state the next round starts from (row n_acc
of the pass).  Also: the greedy stream equals plain greedy decoding, also
with the head drafter and the draft model taking turns; zero heads reproduce
the target's own row; the 8B-shaped slice at full width and vocabulary; the
argument and state errors."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import LOGIT_TOL, NEAR_TIE, PROB_TOL, Buffers, dev_weights

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

N_HEADS = 4


def heads_dev(W_bits):
    return torch.from_numpy(np.ascontiguousarray(W_bits).view(np.int16)).cuda().view(torch.bfloat16)


class HeadsShadow:
    def __init__(self, tcfg, tw_bits, W_bits, prompt, max_seq, seed, greedy, c=0):
        self.T = oracle.Model(tcfg, tw_bits)
        self.W = W_bits
        self.kv = oracle.KV(self.T, max_seq)
        self.hist = [int(x) for x in prompt]
        self.LT = len(prompt) - 1
        _, hid = oracle.forward_hidden(self.T, self.kv, self.hist[: self.LT], 0, want_logits=False)
        self.h = hid[-1]
        self.seed, self.greedy, self.c = seed, greedy, c
        self.max_head_err = self.max_prob_err = self.max_logit_err = 0.0
        self.near_ties = 0

    def check_round(self, g, K):
        LT = self.LT
        Dor, _ = oracle.heads_draft(self.T, self.W, self.h, K, self.greedy, self.seed, LT + 1, self.c)
        err = float(np.abs(Dor - g["D"]).max())
        self.max_head_err = max(self.max_head_err, err)
        assert err <= PROB_TOL, ("head rows", err)
        for k in range(K):
            ref = oracle.draft_sample(g["D"][k], self.seed, LT + 1 + k, 0, self.c, self.greedy)
            assert ref == int(g["d"][k]), ("draft sample", k, ref, int(g["d"][k]))
        rows = [self.hist[LT]] + [int(x) for x in g["d"]]
        lg, hid = oracle.forward_hidden(self.T, self.kv, rows, LT)
        lerr = float(np.abs(lg - g["logits"]).max())
        self.max_logit_err = max(self.max_logit_err, lerr)
        assert lerr <= LOGIT_TOL, ("logits", lerr)
        Tor = np.stack([oracle.softmax_f32(r) for r in lg])
        perr = float(np.abs(Tor - g["T"]).max())
        self.max_prob_err = max(self.max_prob_err, perr)
        assert perr <= PROB_TOL, ("target rows", perr)
        if self.greedy:
            rc, n, out = oracle.verify_greedy(g["T"], g["d"])
        else:
            rc, n, out = oracle.verify_sample(g["T"], g["D"], g["d"], self.seed, 0, self.c, LT + 1)
        assert rc == 0 and n == g["nacc"] and list(out) == list(g["out"]), (n, out, g)
        if self.greedy:
            for j in range(n + 1):
                tok, a = int(g["out"][j]), int(np.argmax(lg[j]))
                if tok != a:
                    assert float(lg[j][a] - lg[j][tok]) < NEAR_TIE
                    self.near_ties += 1
        self.hist += [int(x) for x in g["out"][: n + 1]]
        self.h = hid[n]
        self.LT = LT + n + 1
        return n


def heads_round(sd, ctx, K, seed, b):
    sd.spec_draft_heads(ctx, K, seed, b.d, b.D)
    sd.spec_verify(ctx, K, seed, b.d, b.D, b.out, b.nacc, b.T, b.logits)
    sd.spec_commit(ctx, b.out, b.nacc)
    sd.spec_sync(ctx)
    return {"d": b.d.cpu().numpy().copy(), "D": b.D.cpu().numpy().copy(),
            "T": b.T.cpu().numpy().copy(), "logits": b.logits.cpu().numpy().copy(),
            "out": b.out.cpu().numpy().copy(), "nacc": int(b.nacc.cpu().numpy()[0])}


@pytest.fixture(scope="module")
def toy():
    tw = synth.weights_np(synth.TOY)
    dw = synth.self_draft_np(tw, 1)
    return tw, dw, synth.heads_np(synth.TOY, N_HEADS)


def toy_ctx(sd, tw, dw, prompt, K, greedy, max_seq=160):
    tdev, ddev = dev_weights(tw, dw)
    ctx = sd.spec_init(synth.TOY, tdev, synth.TOY_DRAFT, ddev, prompt, k_max=K, max_seq=max_seq,
                       greedy=greedy)
    return ctx, (tdev, ddev)


@pytest.mark.parametrize("greedy", [True, False])
@pytest.mark.parametrize("K", [1, 4])
def test_toy_head_rounds_match_oracle(toy, K, greedy):
    import speculative_decoding_02_amd as sd
    tw, dw, W = toy
    prompt = synth.prompt(synth.TOY.vocab, 24)
    seed = synth.SEED_PHILOX
    ctx, keep = toy_ctx(sd, tw, dw, prompt, K, greedy)
    sd.spec_heads_init(ctx, heads_dev(W), N_HEADS)
    sh = HeadsShadow(synth.TOY, tw, W, prompt, 160, seed, greedy)
    b = Buffers(K, synth.TOY.vocab)
    emitted = 0
    while emitted < 48:
        emitted += sh.check_round(heads_round(sd, ctx, K, seed, b), K) + 1
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0
        assert st["target_len"] == sh.LT and st["pending"] == sh.hist[sh.LT]
        # the draft model did not run: its cache stays at the prompt
        assert st["draft_len"] == len(prompt) - 1
    print(f"K={K} greedy={greedy}: head row err {sh.max_head_err:.2e}, prob err "
          f"{sh.max_prob_err:.2e}, logit err {sh.max_logit_err:.2e}, near-ties {sh.near_ties}")


def test_head_greedy_stream_equals_plain_greedy(toy):
    import speculative_decoding_02_amd as sd
    tw, dw, W = toy
    prompt = synth.prompt(synth.TOY.vocab, 32)
    K = 4
    ctx, keep = toy_ctx(sd, tw, dw, prompt, K, True)
    sd.spec_heads_init(ctx, heads_dev(W), N_HEADS)
    b = Buffers(K, synth.TOY.vocab)
    n_tok = 0
    while n_tok < 64:
        sd.spec_draft_heads(ctx, K, 0, b.d, b.D)
        sd.spec_verify(ctx, K, 0, b.d, b.D, b.out, b.nacc)
        sd.spec_commit(ctx, b.out, b.nacc)
        sd.spec_sync(ctx)
        n_tok += int(b.nacc.cpu().numpy()[0]) + 1
    st = sd.spec_get_state(ctx)
    gen = sd.spec_get_history(ctx, st["target_len"] + 1)[len(prompt):][:64]
    ref = oracle.generate(oracle.Model(synth.TOY, tw), prompt, 64, greedy=True)
    np.testing.assert_array_equal(gen, ref)


def test_heads_and_draft_model_take_turns(toy):
    """Greedy output is the target's whatever drafts it was given: rounds
    alternate between the heads and the draft model (whose cache catches up
    with the rounds it missed), plus a plain step."""
    import speculative_decoding_02_amd as sd
    tw, dw, W = toy
    prompt = synth.prompt(synth.TOY.vocab, 20, seed=8)
    K = 3
    ctx, keep = toy_ctx(sd, tw, dw, prompt, K, True)
    sd.spec_heads_init(ctx, heads_dev(W), N_HEADS)
    b = Buffers(K, synth.TOY.vocab)
    po = torch.zeros(1, dtype=torch.int32, device="cuda")
    pn = torch.zeros(1, dtype=torch.int32, device="cuda")
    for r in range(12):
        if r % 4 == 3:
            sd.spec_verify(ctx, 0, 0, None, None, po, pn)
            sd.spec_commit(ctx, po, pn)
            continue
        if r % 2 == 0:
            sd.spec_draft_heads(ctx, K, 0, b.d, b.D)
        else:
            sd.spec_draft(ctx, K, 0, b.d, b.D)
        sd.spec_verify(ctx, K, 0, b.d, b.D, b.out, b.nacc)
        sd.spec_commit(ctx, b.out, b.nacc)
    sd.spec_sync(ctx)
    st = sd.spec_get_state(ctx)
    assert st["device_error"] == 0
    n = st["target_len"] - (len(prompt) - 1)
    gen = sd.spec_get_history(ctx, st["target_len"] + 1)[len(prompt):][:n]
    ref = oracle.generate(oracle.Model(synth.TOY, tw), prompt, n, greedy=True)
    np.testing.assert_array_equal(gen, ref)


def test_heads_override_a_draft_model_pass(toy):
    """A draft-model pass whose drafts are then replaced by the heads' leaves
    the draft cache's committed length where it was (the draft model computed
    no row of what gets committed), so the next draft-model rounds catch up
    over the committed text and match the oracle."""
    import speculative_decoding_02_amd as sd
    from gpu_util import Shadow, gpu_round
    tw, dw, W = toy
    prompt = synth.prompt(synth.TOY.vocab, 20, seed=9)
    K, seed = 3, synth.SEED_PHILOX
    ctx, keep = toy_ctx(sd, tw, dw, prompt, K, False)
    sd.spec_heads_init(ctx, heads_dev(W), N_HEADS)
    sh = Shadow(synth.TOY, tw, synth.TOY_DRAFT, dw, prompt, 160, K, seed, False)
    b = Buffers(K, synth.TOY.vocab)
    for r in range(6):
        if r % 3 == 1:
            sd.spec_draft(ctx, K, seed, b.d, b.D)
            g = heads_round(sd, ctx, K, seed, b)
            n, LT = g["nacc"], sh.LT
            oracle.forward(sh.T, sh.kvT, [sh.hist[LT]] + [int(x) for x in g["d"]], LT,
                           want_logits=False)
            sh.hist += [int(x) for x in g["out"][: n + 1]]
            sh.LT = LT + n + 1
        else:
            sh.check_round(gpu_round(sd, ctx, K, seed, b))
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0
        assert (st["target_len"], st["draft_len"]) == (sh.LT, sh.LD), r


def test_zero_heads_reproduce_the_verified_row(toy):
    """With zero head matrices every head is the target's own LM head on the
    kept state, i.e. row n_acc of the last verify's T (to the pass's
    precision); re-initialising with other heads replaces them."""
    import speculative_decoding_02_amd as sd
    tw, dw, W = toy
    prompt = synth.prompt(synth.TOY.vocab, 16, seed=2)
    K = 3
    ctx, keep = toy_ctx(sd, tw, dw, prompt, K, False)
    sd.spec_heads_init(ctx, heads_dev(W), N_HEADS)
    b = Buffers(K, synth.TOY.vocab)
    heads_round(sd, ctx, K, 5, b)
    zero = torch.zeros((N_HEADS, 64, 64), dtype=torch.bfloat16, device="cuda")
    sd.spec_heads_init(ctx, zero, N_HEADS)
    for r in range(3):
        g = heads_round(sd, ctx, K, 5 + r, b)
        Trow = g["T"][g["nacc"]]
        sd.spec_draft_heads(ctx, K, 99, b.d, b.D)
        sd.spec_sync(ctx)
        D = b.D.cpu().numpy()
        for k in range(K):
            assert float(np.abs(D[k] - Trow).max()) <= PROB_TOL
        # drop the drafts: verify and commit them so the state moves on
        sd.spec_verify(ctx, K, 99, b.d, b.D, b.out, b.nacc)
        sd.spec_commit(ctx, b.out, b.nacc)
    sd.spec_sync(ctx)
    assert sd.spec_get_state(ctx)["device_error"] == 0


def test_head_state_and_argument_errors(toy):
    import speculative_decoding_02_amd as sd
    tw, dw, W = toy
    K = 2
    b = Buffers(K, synth.TOY.vocab)
    # a one-token prompt has no processed position until the first commit
    ctx, keep = toy_ctx(sd, tw, dw, synth.prompt(synth.TOY.vocab, 1), K, True)
    with pytest.raises(sd.SpecError) as e:
        sd.spec_draft_heads(ctx, K, 0, b.d, b.D)
    assert e.value.code == sd.SPEC_ERR_STATE          # no heads yet
    Wd = heads_dev(W)
    for bad in (0, sd.SPEC_K_MAX + 1):
        with pytest.raises(sd.SpecError) as e:
            sd.spec_heads_init(ctx, Wd, bad)
        assert e.value.code == sd.SPEC_ERR_ARG
    sd.spec_heads_init(ctx, Wd, 1)
    with pytest.raises(sd.SpecError) as e:
        sd.spec_draft_heads(ctx, K, 0, b.d, b.D)      # K > n_heads
    assert e.value.code == sd.SPEC_ERR_ARG
    sd.spec_heads_init(ctx, Wd, N_HEADS)
    with pytest.raises(sd.SpecError) as e:
        sd.spec_draft_heads(ctx, K, 0, b.d, b.D)      # nothing processed yet
    assert e.value.code == sd.SPEC_ERR_STATE
    po = torch.zeros(1, dtype=torch.int32, device="cuda")
    pn = torch.zeros(1, dtype=torch.int32, device="cuda")
    sd.spec_verify(ctx, 0, 0, None, None, po, pn)
    with pytest.raises(sd.SpecError) as e:
        sd.spec_draft_heads(ctx, K, 0, b.d, b.D)      # a verify is pending
    assert e.value.code == sd.SPEC_ERR_STATE
    sd.spec_commit(ctx, po, pn)
    sd.spec_draft_heads(ctx, K, 0, b.d, b.D)          # now there is a state
    with pytest.raises(sd.SpecError) as e:
        sd.spec_draft_heads(ctx, K, 0, None, b.D)
    assert e.value.code == sd.SPEC_ERR_ARG
    sd.spec_sync(ctx)
    assert sd.spec_get_state(ctx)["device_error"] == 0


@pytest.mark.parametrize("greedy", [False, True])
def test_8b_shaped_slice_heads(greedy):
    """Full width (d 4096) and vocabulary (128256), 2 target layers, four
    4096 x 4096 heads, K = 4, in the launch plans bench.py uses."""
    import speculative_decoding_02_amd as sd
    tcfg = synth.L8B.replace(name="8b-slice-2L", n_layers=2)
    dcfg = synth.L8B_DRAFT.replace(name="1b-slice-1L", n_layers=1)
    tw = synth.weights_torch(tcfg, device="cuda")
    dw = synth.weights_torch(dcfg, seed=synth.SEED_WEIGHTS + 1, device="cuda")
    Wt = synth.heads_torch(tcfg, N_HEADS)
    torch.cuda.synchronize()
    tb = synth.torch_to_bits(tw)
    Wb = Wt.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    prompt = synth.prompt(tcfg.vocab, 12, seed=17)
    K, seed, rounds = 4, 1003, 3
    max_seq = 12 + rounds * (K + 1) + 16
    ctx = sd.spec_init(tcfg, tw, dcfg, dw, prompt, k_max=K, max_seq=max_seq, greedy=greedy)
    sd.spec_heads_init(ctx, Wt, N_HEADS)
    sh = HeadsShadow(tcfg, tb, Wb, prompt, max_seq, seed, greedy)
    b = Buffers(K, tcfg.vocab)
    for _ in range(rounds):
        sh.check_round(heads_round(sd, ctx, K, seed, b), K)
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0 and st["target_len"] == sh.LT
    print(f"8B slice heads greedy={greedy}: head row err {sh.max_head_err:.2e}, prob err "
          f"{sh.max_prob_err:.2e}, logit err {sh.max_logit_err:.2e}, near-ties {sh.near_ties}")
    sd.spec_destroy(ctx)
