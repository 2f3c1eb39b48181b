"""GPU parity at the workloads' real per-layer shapes, in the launch
configurations bench.py uses (same GEMM plans, attention tiles, vocabulary
sizes), with fewer layers so the fp64 oracle finishes in seconds:

  * the full 8B-shaped pair (32 + 16 layers) and the full 31B-shaped pair
    (60 + 34 layers) with short prompts, and an
    8B-shaped target slice (d 4096, 32/8 heads x 128, FFN 14336, vocab
    128256) with a 1B-shaped draft slice (d 2048, 32/8 x 64, tied head);
  * 31B-shaped slice (d 5376, 32/16 heads x 168, FFN 21504, vocab 262144)
    with a 4B-shaped draft slice (20/4 heads x 128: five query heads per KV
    head), K = 5;
  * 1.3B-shaped slice (MHA 16 x 128, vocab 32000) with a draft sharing the
    target's embedding and LM head;
  * a long context: 1500-token prompt through 32/8 x 128 attention;
  * a d_model-8192 target with 256-dim heads and a draft with 32-dim heads,
    a d_model-16384 target, and a d_model-10240 target whose QKV, gate/up
    and O projections run as column slices (GEMM and attention variants the
    pairs above do not reach);
  * the benchmark's own workload at full size (sampled outputs, below).

Every round is teacher-forced: draft rows (1e-4) and samples (bit-exact),
target logits (2e-2) and rows (1e-4), accept/reject on the GPU's own rows
(bit-exact), greedy tokens equal to the oracle's argmax or counted
near-ties, and the committed state."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Buffers, Shadow

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def run_case(tcfg, dcfg, prompt_len, K, rounds, greedy, share=(), seed=1003, max_extra=64):
    import speculative_decoding_02_amd as sd
    from gpu_util import gpu_round
    tw = synth.weights_torch(tcfg, device="cuda")
    dw = synth.weights_torch(dcfg, seed=synth.SEED_WEIGHTS + 1, device="cuda", share_from=tw,
                             share=share)
    torch.cuda.synchronize()
    tb, db = synth.torch_to_bits(tw), synth.torch_to_bits(dw)
    if share:
        for k in share:  # the oracle sees the very same arrays
            db[k] = tb[k]
    prompt = synth.prompt(tcfg.vocab, prompt_len, seed=17)
    max_seq = prompt_len + rounds * (K + 1) + max_extra
    ctx = sd.spec_init(tcfg, tw, dcfg, dw, prompt, k_max=K, max_seq=max_seq, greedy=greedy)
    sh = Shadow(tcfg, tb, dcfg, db, prompt, max_seq, K, seed, greedy)
    b = Buffers(K, tcfg.vocab)
    for _ in range(rounds):
        sh.check_round(gpu_round(sd, ctx, K, seed, b))
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0
        assert (st["target_len"], st["draft_len"]) == (sh.LT, sh.LD)
    print(f"{tcfg.name}: logit err {sh.max_logit_err:.2e}, prob err {sh.max_prob_err:.2e}, "
          f"draft prob err {sh.max_draft_prob_err:.2e}, near-ties {sh.near_ties}")
    sd.spec_destroy(ctx)


@pytest.mark.parametrize("greedy", [False, True])
def test_8b_full_depth(greedy):
    """The whole 8B-shaped target (32 layers) and 1B-shaped draft (16 layers),
    K = 4, exactly as bench.py builds them, with a short prompt so the fp64
    oracle keeps up: two teacher-forced rounds."""
    run_case(synth.L8B, synth.L8B_DRAFT, prompt_len=16, K=4, rounds=2, greedy=greedy, max_extra=16)


def test_31b_full_depth():
    """The whole 31B-shaped target (60 layers, ~55 GB of bf16 weights) and
    4B-shaped draft (34 layers), K = 5, one teacher-forced round."""
    run_case(synth.G31B, synth.G31B_DRAFT, prompt_len=8, K=5, rounds=1, greedy=False, max_extra=16)


@pytest.mark.parametrize("greedy", [False, True])
def test_8b_shaped_slice(greedy):
    run_case(synth.L8B.replace(name="8b-slice-2L", n_layers=2),
             synth.L8B_DRAFT.replace(name="1b-slice-1L", n_layers=1),
             prompt_len=12, K=4, rounds=3, greedy=greedy)


def test_31b_shaped_slice():
    run_case(synth.G31B.replace(name="31b-slice-1L", n_layers=1),
             synth.G31B_DRAFT.replace(name="4b-slice-1L", n_layers=1),
             prompt_len=7, K=5, rounds=2, greedy=False)


def test_13b_shaped_slice_shared_head():
    run_case(synth.L13B.replace(name="1.3b-slice-2L", n_layers=2),
             synth.L13B_DRAFT.replace(name="1.3b-draft-slice-1L", n_layers=1),
             prompt_len=20, K=4, rounds=3, greedy=False, share=("embed", "lm_head"))


def test_long_context_attention():
    t = synth.ModelConfig("long-ctx-1L", 1, 256, 32, 8, 128, 512, 1024)
    d = t.replace(name="long-ctx-draft")
    run_case(t, d, prompt_len=1500, K=4, rounds=3, greedy=False)


def test_wide_model_and_narrow_heads():
    """Launch variants the workload pairs do not reach: a d_model-8192 target
    whose O and down projections take two column blocks per workgroup (each
    residual row spans two 16-lane groups, whose sums of squares meet in LDS),
    with 256-dim heads (eight 32-dim steps in the attention partial, 32 lanes
    per chunk group in the merge) and a QKV projection in column slices of
    24 columns, two workgroups per CU; and a draft with 32-dim heads (one
    step, 4 lanes per chunk group).  The 200-token prompt gives every head
    seven chunks to merge."""
    t = synth.ModelConfig("wide-d8192-hd256-1L", 1, 8192, 32, 8, 256, 1024, 1024)
    d = synth.ModelConfig("hd32-draft-1L", 1, 512, 16, 4, 32, 1024, 1024)
    run_case(t, d, prompt_len=200, K=4, rounds=2, greedy=False)


def test_very_wide_residual():
    """d_model 16384: the O and down projections take four column blocks per
    workgroup, so each thread of the residual epilogue handles two items and
    a row's sums of squares meet from four 16-lane groups."""
    t = synth.ModelConfig("wide-d16384-1L", 1, 16384, 16, 4, 64, 512, 1024)
    d = synth.ModelConfig("small-draft-1L", 1, 256, 8, 2, 32, 512, 1024)
    run_case(t, d, prompt_len=40, K=3, rounds=2, greedy=False)


def test_column_slice_shapes():
    """Column-slice plans the workload pairs do not reach (the 31B-shaped
    pair covers slices of two and three blocks for QKV, two for O and down,
    four for gate/up; its 4B-shaped draft one for down): a d_model-10240
    target whose QKV projection (3584 columns) runs as 14-column slices --
    seven RoPE pairs in the partial block, none whole -- its gate/up (3072
    columns) as 12-column slices (six gate/up pairs), and its O projection
    as 40-column slices (two whole blocks and 8 columns), each at >= 200 KB
    per CU."""
    t = synth.ModelConfig("slices-d10240-1L", 1, 10240, 20, 4, 128, 1536, 1024)
    d = synth.ModelConfig("small-draft-1L", 1, 256, 8, 2, 32, 512, 1024)
    run_case(t, d, prompt_len=40, K=4, rounds=2, greedy=False)


def test_column_slices_two_per_cu_residual():
    """d_model 17408: the O and down projections (residual epilogue, >= 200 KB
    per CU) take column slices of 34 columns, two workgroups per CU (512):
    two whole blocks and a partial block of 2 live columns each, 512 partial
    sums of squares for the next RMSNorm (the most a four-wave consumer
    folds); the QKV projection runs as 24-column pair slices."""
    t = synth.ModelConfig("slices-d17408-1L", 1, 17408, 32, 8, 128, 2048, 1024)
    d = synth.ModelConfig("small-draft-1L", 1, 256, 8, 2, 32, 512, 1024)
    run_case(t, d, prompt_len=24, K=3, rounds=2, greedy=False)


def test_8b_bench_workload_sampled():
    """The benchmark's workload at full size: the 8B-shaped target and
    1B-shaped draft at full depth, bench.py's 1024-token prompt, K = 4,
    sampling, in its launch plans.  The fp64 oracle cannot run this forward
    in test time, so what is checked is what it computes output by output:
    every draft token is the oracle sampler's draw from the GPU's own draft
    row (word 0 at its position), every decision is the oracle rule on the
    GPU's own target and draft rows (bit-exact), every row is a probability
    distribution, the state advances by n_acc + 1; and row 0 of the first
    five-row verify equals, bit for bit, a one-row verify (K = 0) of the same
    context in a second context (the launch plans depend on the shapes only,
    and no row's arithmetic depends on the other rows)."""
    import speculative_decoding_02_amd as sd
    from gpu_util import gpu_round
    tcfg, dcfg = synth.L8B, synth.L8B_DRAFT
    tw = synth.weights_torch(tcfg, device="cuda")
    dw = synth.weights_torch(dcfg, seed=synth.SEED_WEIGHTS + 1, device="cuda")
    torch.cuda.synchronize()
    plen, K, seed, rounds = 1024, 4, synth.SEED_PHILOX, 4
    prompt = synth.prompt(tcfg.vocab, plen)
    max_seq = plen + rounds * (K + 1) + 24
    ctx = sd.spec_init(tcfg, tw, dcfg, dw, prompt, k_max=K, max_seq=max_seq, greedy=False)
    ref = sd.spec_init(tcfg, tw, dcfg, dw, prompt, k_max=K, max_seq=max_seq, greedy=False)
    b, b1 = Buffers(K, tcfg.vocab), Buffers(K, tcfg.vocab)
    LT = plen - 1
    for r in range(rounds):
        g = gpu_round(sd, ctx, K, seed, b)
        for i in range(K):
            assert oracle.draft_sample(g["D"][i], seed, LT + 1 + i, 0, 0, False) == int(g["d"][i])
        for rows in (g["D"], g["T"]):
            assert np.all(rows >= 0.0) and np.abs(rows.sum(axis=-1) - 1.0).max() < 1e-4
        rc, n, out = oracle.verify_sample(g["T"], g["D"], g["d"], seed, 0, 0, LT + 1)
        assert rc == 0 and n == g["nacc"] and list(out[: n + 1]) == list(g["out"][: n + 1])
        if r == 0:
            sd.spec_verify(ref, 0, seed, None, None, b1.out, b1.nacc, b1.T, b1.logits)
            sd.spec_sync(ref)
            lerr = float(np.abs(b1.logits.cpu().numpy()[0] - g["logits"][0]).max())
            perr = float(np.abs(b1.T.cpu().numpy()[0] - g["T"][0]).max())
            print(f"row 0, five-row vs one-row pass: logits {lerr:.2e}, probabilities {perr:.2e}")
            assert lerr == 0.0 and perr == 0.0  # same plans and per-row arithmetic
            sd.spec_destroy(ref)
        LT += n + 1
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0 and st["target_len"] == LT
    sd.spec_destroy(ctx)


def test_8b_bench_workload_other_drafters_sampled():
    """The drafters without a draft model at the benchmark's size (full
    8B-shaped target, 1024-token prompt, K = 4, sampling), alternating:
    multi-token heads (four random 4096 x 4096 heads) -- every draft the
    oracle sampler's draw from the GPU's own head row, word 0 at its
    position -- and prompt lookup -- drafts equal to the oracle's search over
    the GPU's history, one-hot rows exact; the rule bit-exact on the GPU's
    rows after either, and the committed state."""
    import speculative_decoding_02_amd as sd
    from gpu_util import Buffers
    tcfg, dcfg = synth.L8B, synth.L8B_DRAFT
    tw = synth.weights_torch(tcfg, device="cuda")
    dw = synth.weights_torch(dcfg, seed=synth.SEED_WEIGHTS + 1, device="cuda")
    W = synth.heads_torch(tcfg, 4)
    torch.cuda.synchronize()
    plen, K, seed, rounds = 1024, 4, synth.SEED_PHILOX, 4
    prompt = synth.prompt(tcfg.vocab, plen)
    ctx = sd.spec_init(tcfg, tw, dcfg, dw, prompt, k_max=K, max_seq=plen + rounds * (K + 1) + 24,
                       greedy=False)
    sd.spec_heads_init(ctx, W, 4)
    b = Buffers(K, tcfg.vocab)
    LT = plen - 1
    for r in range(rounds):
        heads = r % 2 == 0
        if heads:
            sd.spec_draft_heads(ctx, K, seed, b.d, b.D)
        else:
            sd.spec_draft_ngram(ctx, K, 3, b.d, b.D)
        sd.spec_verify(ctx, K, seed, b.d, b.D, b.out, b.nacc, b.T, b.logits)
        sd.spec_commit(ctx, b.out, b.nacc)
        sd.spec_sync(ctx)
        d, D, T = b.d.cpu().numpy(), b.D.cpu().numpy(), b.T.cpu().numpy()
        out, n_acc = b.out.cpu().numpy(), int(b.nacc.cpu().numpy()[0])
        if heads:
            assert np.all(D >= 0.0) and np.abs(D.sum(axis=-1) - 1.0).max() < 1e-4
            for i in range(K):
                assert oracle.draft_sample(D[i], seed, LT + 1 + i, 0, 0, False) == int(d[i])
        else:
            hist = sd.spec_get_history(ctx, LT + 1)
            ref, _ = oracle.ngram_draft(hist, LT, K, 3)
            assert list(d) == list(ref)
            onehot = np.zeros_like(D)
            onehot[np.arange(K), ref] = 1.0
            assert np.array_equal(D, onehot)
        rc, n, o = oracle.verify_sample(T, D, d, seed, 0, 0, LT + 1)
        assert rc == 0 and n == n_acc and list(o[: n + 1]) == list(out[: n + 1])
        LT += n + 1
        st = sd.spec_get_state(ctx)
        assert st["device_error"] == 0 and st["target_len"] == LT
    sd.spec_destroy(ctx)
