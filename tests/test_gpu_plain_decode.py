"""Plain decoding through the verify entry point with K = 0: a one-row
target pass and the next token drawn from T_1.  This is the baseline the
speedup of speculative decoding is measured against ([en] Floor 3: one
weight read per emitted token), on the same kernels and the same boundary.

Checked teacher-forced against the oracle (rows within tolerance, the token
bit-exact on the GPU's own row), against the oracle's own plain greedy decode
end to end, and mixed with speculative rounds: plain steps leave the draft
cache behind, and the next draft catches it up from the committed history."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Buffers, Shadow, dev_weights, gpu_plain_step, gpu_round

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def toy():
    tw = synth.weights_np(synth.TOY)
    dw = synth.self_draft_np(tw, 1)
    return tw, dw


def make_ctx(tw, dw, prompt, K, greedy, max_seq=192):
    import speculative_decoding_02_amd as sd
    tdev, ddev = dev_weights(tw, dw)
    ctx = sd.spec_init(synth.TOY, tdev, synth.TOY_DRAFT, ddev, prompt, k_max=K, max_seq=max_seq,
                       greedy=greedy)
    return ctx, (tdev, ddev)


@pytest.mark.parametrize("greedy", [True, False])
def test_plain_steps_teacher_forced(toy, greedy):
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 24, seed=11)
    seed = synth.SEED_PHILOX
    ctx, keep = make_ctx(tw, dw, prompt, 4, greedy)
    sh = Shadow(synth.TOY, tw, synth.TOY_DRAFT, dw, prompt, 192, 4, seed, greedy)
    b = Buffers(0, synth.TOY.vocab)
    for _ in range(40):
        sh.check_plain(gpu_plain_step(sd, ctx, seed, b))
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0 and st["target_len"] == sh.LT
        assert st["draft_len"] == len(prompt) - 1  # the draft model did not run
    assert list(sd.spec_get_history(ctx, sh.LT + 1)) == sh.hist
    print(f"greedy={greedy}: logit err {sh.max_logit_err:.2e}, prob err {sh.max_prob_err:.2e}")


def test_plain_greedy_equals_oracle_generate(toy):
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 32)
    ctx, keep = make_ctx(tw, dw, prompt, 4, True)
    b = Buffers(0, synth.TOY.vocab)
    toks = [int(gpu_plain_step(sd, ctx, 0, b)["out"][0]) for _ in range(48)]
    ref = oracle.generate(oracle.Model(synth.TOY, tw), prompt, 48, greedy=True)
    np.testing.assert_array_equal(toks, ref)


@pytest.mark.parametrize("greedy", [True, False])
def test_plain_and_speculative_interleaved(toy, greedy):
    """Runs of plain steps between speculative rounds: lags of 1..12 rows,
    both below and above what one draft step carries."""
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 16, seed=12)
    seed, K = 91, 3
    ctx, keep = make_ctx(tw, dw, prompt, K, greedy)
    sh = Shadow(synth.TOY, tw, synth.TOY_DRAFT, dw, prompt, 192, K, seed, greedy)
    bp, br = Buffers(0, synth.TOY.vocab), Buffers(K, synth.TOY.vocab)
    counts = np.zeros((8, 8), np.int64)  # the acceptance record, kept alongside
    for n_plain in (1, 5, 12, 0, 8, 2):
        for _ in range(n_plain):
            sh.check_plain(gpu_plain_step(sd, ctx, seed, bp))
            counts[0, 0] += 1
        counts[K, sh.check_round(gpu_round(sd, ctx, K, seed, br))] += 1
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0
        assert st["target_len"] == sh.LT and st["draft_len"] == sh.LD
        np.testing.assert_array_equal(st["accept_counts"], counts)
    assert list(sd.spec_get_history(ctx, sh.LT + 1)) == sh.hist


def test_plain_step_arguments(toy):
    import speculative_decoding_02_amd as sd
    tw, dw = toy
    prompt = synth.prompt(synth.TOY.vocab, 8, seed=13)
    ctx, keep = make_ctx(tw, dw, prompt, 2, False)
    b = Buffers(0, synth.TOY.vocab)
    with pytest.raises(sd.SpecError):
        sd.spec_verify(ctx, -1, 0, None, None, b.out, b.nacc)
    with pytest.raises(sd.SpecError):
        sd.spec_verify(ctx, 0, 0, None, None, None, b.nacc)
    sd.spec_verify(ctx, 0, 0, None, None, b.out, b.nacc)  # rows not requested
    with pytest.raises(sd.SpecError):  # uncommitted
        sd.spec_verify(ctx, 0, 0, None, None, b.out, b.nacc)
    sd.spec_commit(ctx, b.out, b.nacc)
    sd.spec_sync(ctx)
    assert sd.spec_get_state(ctx)["target_len"] == len(prompt)


def test_read_ceiling():
    """The streaming-read helper returns a rate between a tenth of the HBM
    peak and the peak itself (8 TB/s), and rejects bad arguments."""
    import speculative_decoding_02_amd as sd
    buf = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    gbs = sd.spec_read_ceiling(buf, reps=2)
    print(f"read ceiling over 1 GiB: {gbs:.0f} GB/s")
    assert 800.0 < gbs < 8000.0
    with pytest.raises(sd.SpecError):
        sd.spec_read_ceiling(buf[:1000], reps=1)
    with pytest.raises(sd.SpecError):
        sd.spec_read_ceiling(buf, reps=0)
