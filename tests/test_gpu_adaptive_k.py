"""Adaptive K on the GPU: one context runs rounds whose K changes from round
to round (each K has its own captured graphs), every round checked against
the oracle shadow (draft rows and samples, target rows and logits, the rule
bit-exact, the committed state); then K is chosen window by window from the
acceptance the GPU's own rounds showed, and every choice is checked against
the oracle's choose_k on the same estimate and costs.

"Speculative decoding internals", speedup: a round costs K draft steps plus
one target pass and too large a K loses the gain; [en] Floor 6: the mean
number of tokens a round yields, 1 + a + ... + a^K."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Buffers, Shadow, dev_weights, gpu_round

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("greedy", [False, True])
def test_k_changes_between_rounds_and_follows_choose_k(greedy):
    import speculative_decoding_02_amd as sd
    k_max = sd.SPEC_K_MAX
    tw = synth.weights_np(synth.TOY)
    dw = synth.self_draft_np(tw, 1)
    prompt = synth.prompt(synth.TOY.vocab, 32, seed=31)
    seed = synth.SEED_PHILOX
    max_seq = 400
    tdev, ddev = dev_weights(tw, dw)
    ctx = sd.spec_init(synth.TOY, tdev, synth.TOY_DRAFT, ddev, prompt, k_max=k_max,
                       max_seq=max_seq, greedy=greedy)
    sh = Shadow(synth.TOY, tw, synth.TOY_DRAFT, dw, prompt, max_seq, k_max, seed, greedy)
    bufs = {K: Buffers(K, synth.TOY.vocab) for K in range(1, k_max + 1)}
    stream = torch.cuda.ExternalStream(sd.spec_stream(ctx))

    def one(K):
        sh.K = K
        g = gpu_round(sd, ctx, K, seed, bufs[K])
        n = sh.check_round(g)
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0 and (st["target_len"], st["draft_len"]) == (sh.LT, sh.LD)
        return n

    # scripted K sequence: every K, small after large and large after small
    for K in (4, 1, 6, 2, 7, 3, 5, 1):
        one(K)

    # costs of a draft step and of a verify pass, from events on the context stream
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    b = bufs[4]
    ev[0].record(stream)
    sd.spec_draft(ctx, 4, seed, b.d, b.D)
    ev[1].record(stream)
    sd.spec_verify(ctx, 4, seed, b.d, b.D, b.out, b.nacc, b.T, b.logits)
    ev[2].record(stream)
    sd.spec_commit(ctx, b.out, b.nacc)
    sd.spec_sync(ctx)
    t_draft = ev[0].elapsed_time(ev[1]) / 4
    t_verify = ev[1].elapsed_time(ev[2])
    g = {"d": b.d.cpu().numpy(), "D": b.D.cpu().numpy(), "T": b.T.cpu().numpy(),
         "logits": b.logits.cpu().numpy(), "out": b.out.cpu().numpy(),
         "nacc": int(b.nacc.cpu().numpy()[0])}
    sh.K = 4
    sh.check_round(g)

    # adaptive windows: alpha from the tokens the window committed, smoothed
    W, K, alpha, ks = 3, 4, None, []
    for _ in range(6):
        len0 = sh.LT
        for _ in range(W):
            one(K)
        tpr = (sh.LT - len0) / W
        a = sd.spec_alpha_from_tokens(tpr, K)
        assert 0.0 <= a <= 1.0
        if 1.0 < tpr < K + 1.0:  # the estimate inverts the Floor 6 mean
            assert abs(oracle.expected_tokens(a, K) - tpr) < 1e-9
        alpha = a if alpha is None else 0.5 * alpha + 0.5 * a
        K_next = sd.spec_choose_k(alpha, t_draft, t_verify, k_max)
        assert K_next == oracle.choose_k(alpha, t_draft, t_verify, k_max), (alpha, K_next)
        ks.append(K_next)
        K = K_next
    # the same estimates under other cost ratios move K, as choose_k says
    for t_d in (0.0, t_verify * 0.05, t_verify * 0.5, t_verify * 3.0):
        assert sd.spec_choose_k(alpha, t_d, t_verify, k_max) == oracle.choose_k(alpha, t_d,
                                                                                t_verify, k_max)
    print(f"greedy={greedy}: t_draft {t_draft:.3f} ms, t_verify {t_verify:.3f} ms, alpha "
          f"{alpha:.3f}, K per window {ks}")
    sd.spec_destroy(ctx)
