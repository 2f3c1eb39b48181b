"""GPU parity of the batched verify (spec_batch_*) against the oracle,
sequence by sequence.

The oracle of a batch is the single-sequence oracle run once per sequence:
each sequence has its own history and cache, and sequence b draws its
Philox words with sequence index s = b.  Teacher-forced rounds: drafts come
from the oracle's self-draft model run over each sequence's committed text
(so some are accepted), the GPU verifies all sequences in one pass, and the
oracle checks every sequence's logits (2e-2) and target rows (1e-4), the
rule bit-exact on the GPU's own rows, greedy near-ties, and the committed
lengths.  Also: greedy streams equal plain greedy decoding per sequence with
the batched n-gram drafter, those drafts equal the oracle's search on each
history, the 8B-shaped slice at full width and vocabulary, the largest batch
(128 activation rows), and the argument, state and capacity errors."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import LOGIT_TOL, NEAR_TIE, PROB_TOL, dev_weights

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


class BatchBuffers:
    def __init__(self, B: int, K: int, V: int):
        z = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt, device="cuda")  # noqa: E731
        self.d = z(B, K, dt=torch.int32)
        self.D = z(B, K, V)
        self.T = z(B, K + 1, V)
        self.logits = z(B, K + 1, V)
        self.out = z(B, K + 1, dt=torch.int32)
        self.nacc = z(B, dt=torch.int32)


def self_drafts(Dm, hist, K, seed, s, greedy, c=0):
    """K drafts of the oracle's draft model over the committed text hist
    (pending token last), from a fresh cache: rows D_1..D_K and tokens drawn
    with Philox word 0 at positions len(hist)..len(hist)+K-1, sequence s."""
    kv = oracle.KV(Dm, len(hist) + K + 1)
    lg = oracle.forward(Dm, kv, list(hist), 0)[-1]
    P = len(hist)
    rows, toks = [], []
    for i in range(K):
        p = oracle.softmax_f32(lg)
        t = oracle.draft_sample(p, seed, P + i, s, c, greedy)
        rows.append(p)
        toks.append(t)
        if i + 1 < K:
            lg = oracle.forward(Dm, kv, [t], P + i)[-1]
    return np.array(toks, np.int32), np.stack(rows).astype(np.float32)


class SeqShadow:
    """Oracle state of one sequence of the batch."""

    def __init__(self, Tm, prompt, max_seq):
        self.T = Tm
        self.kv = oracle.KV(Tm, max_seq)
        self.hist = [int(x) for x in prompt]
        self.LT = len(prompt) - 1
        if self.LT > 0:
            oracle.forward(Tm, self.kv, self.hist[: self.LT], 0, want_logits=False)

    def check(self, b, g, d, D, K, seed, greedy, c=0, stats=None):
        LT = self.LT
        rows = [self.hist[LT]] + [int(x) for x in d]
        lg = oracle.forward(self.T, self.kv, rows, LT)
        lerr = float(np.abs(lg - g["logits"][b]).max())
        assert lerr <= LOGIT_TOL, ("logits", b, lerr)
        Tor = np.stack([oracle.softmax_f32(r) for r in lg])
        perr = float(np.abs(Tor - g["T"][b]).max())
        assert perr <= PROB_TOL, ("target rows", b, perr)
        if stats is not None:
            stats["logit"] = max(stats.get("logit", 0.0), lerr)
            stats["prob"] = max(stats.get("prob", 0.0), perr)
        if greedy:
            rc, n, out = oracle.verify_greedy(g["T"][b], d)
        else:
            rc, n, out = oracle.verify_sample(g["T"][b], D, d, seed, b, c, LT + 1)
        assert rc == 0 and n == g["nacc"][b] and list(out[: n + 1]) == list(g["out"][b][: n + 1]), \
            (b, n, out, g["nacc"][b], g["out"][b])
        if greedy:
            for j in range(n + 1):
                tok, a = int(g["out"][b][j]), int(np.argmax(lg[j]))
                if tok != a:
                    assert float(lg[j][a] - lg[j][tok]) < NEAR_TIE
                    if stats is not None:
                        stats["near_ties"] = stats.get("near_ties", 0) + 1
        self.hist += [int(x) for x in g["out"][b][: n + 1]]
        self.LT = LT + n + 1
        return n


def gpu_batch_round(sd, bc, K, seed, buf, d_np, D_np):
    buf.d.copy_(torch.from_numpy(d_np))
    buf.D.copy_(torch.from_numpy(D_np))
    torch.cuda.synchronize()  # the library runs on its own stream
    sd.spec_batch_verify(bc, K, seed, buf.d, buf.D, buf.out, buf.nacc, buf.T, buf.logits)
    sd.spec_batch_commit(bc, buf.out, buf.nacc)
    sd.spec_batch_sync(bc)
    return {"T": buf.T.cpu().numpy(), "logits": buf.logits.cpu().numpy(),
            "out": buf.out.cpu().numpy(), "nacc": buf.nacc.cpu().numpy()}


def batch_prompts(vocab, B, n):
    return np.stack([synth.prompt(vocab, n, seed=100 + b) for b in range(B)])


def run_teacher_forced(sd, tcfg, tw, B, K, greedy, rounds, prompt_len, seed=synth.SEED_PHILOX):
    tdev, = dev_weights(tw)
    dw = synth.self_draft_np(tw, 1)
    Dm = oracle.Model(synth.TOY_DRAFT if tcfg is synth.TOY else tcfg.replace(n_layers=1), dw)
    Tm = oracle.Model(tcfg, tw)
    prompts = batch_prompts(tcfg.vocab, B, prompt_len)
    max_seq = prompt_len + rounds * (K + 1) + 8
    bc = sd.spec_batch_init(tcfg, tdev, prompts, k_max=K, max_seq=max_seq, greedy=greedy)
    shadows = [SeqShadow(Tm, prompts[b], max_seq) for b in range(B)]
    buf = BatchBuffers(B, K, tcfg.vocab)
    stats = {}
    accepted = 0
    for _ in range(rounds):
        ds, Ds = zip(*[self_drafts(Dm, sh.hist[: sh.LT + 1], K, seed, b, greedy)
                       for b, sh in enumerate(shadows)])
        d_np, D_np = np.stack(ds), np.stack(Ds)
        g = gpu_batch_round(sd, bc, K, seed, buf, d_np, D_np)
        for b, sh in enumerate(shadows):
            accepted += sh.check(b, g, d_np[b], D_np[b], K, seed, greedy, stats=stats)
        st = sd.spec_batch_get_state(bc)
        assert np.all(st["device_error"] == 0)
        assert list(st["len"]) == [sh.LT for sh in shadows]
    for b, sh in enumerate(shadows):
        h = sd.spec_batch_get_history(bc, b, sh.LT + 1)
        assert list(h) == sh.hist[: sh.LT + 1]
    print(f"B={B} K={K} greedy={greedy}: {accepted} drafts accepted over {rounds} rounds; "
          f"logit err {stats.get('logit', 0):.2e}, prob err {stats.get('prob', 0):.2e}, "
          f"near-ties {stats.get('near_ties', 0)}")
    sd.spec_batch_destroy(bc)
    return accepted


@pytest.fixture(scope="module")
def toy_w():
    return synth.weights_np(synth.TOY)


@pytest.mark.parametrize("B,K,greedy", [(1, 4, False), (3, 3, False), (5, 4, False), (2, 1, True),
                                        (4, 4, True)])
def test_toy_batch_rounds_match_oracle(toy_w, B, K, greedy):
    """B (K+1) = 5, 12, 25, 4, 20 rows: one to four row tiles, sequences
    straddling tile boundaries."""
    import speculative_decoding_02_amd as sd
    run_teacher_forced(sd, synth.TOY, toy_w, B, K, greedy, rounds=5, prompt_len=20)


@pytest.mark.parametrize("B,K", [(16, 7), (32, 3)])
def test_toy_largest_batch(toy_w, B, K):
    """128 activation rows (the rows GEMM's limit): 16 sequences x 8 rows, and
    the most sequences a context takes, 32 x 4 rows."""
    import speculative_decoding_02_amd as sd
    acc = run_teacher_forced(sd, synth.TOY, toy_w, B, K, False, rounds=3, prompt_len=12)
    assert acc > 0


# every matrix a multiple of 128 columns: passes over more than 8 rows take
# the wide GEMM (LDS-shared activation tiles, split K for the narrow ones)
MID = synth.ModelConfig("mid-2L-d256", 2, 256, 4, 2, 64, 512, 1024)


@pytest.mark.parametrize("B,K", [(5, 4), (16, 7)])
def test_mid_batch_wide_gemm_rounds_match_oracle(B, K):
    """25 and 128 rows through the wide GEMM (QKV 512, O 256, gate/up 1024,
    down 256, LM head 1024 columns: every matrix with K split two to four
    ways)."""
    import speculative_decoding_02_amd as sd
    w = synth.weights_np(MID)
    acc = run_teacher_forced(sd, MID, w, B, K, False, rounds=3, prompt_len=14)
    assert acc > 0


HD168 = synth.ModelConfig("hd168-g5-1L", 1, 512, 20, 4, 168, 512, 1024)


def test_batch_hd168_five_query_heads():
    """168-dim heads (the merge's general chunk-group fold: 21 lanes to a
    group, three groups) with five query heads per KV head, four sequences
    (one wave scores both 16-query tiles of a chunk), 80-token prompts
    (three key chunks per head), through the rows GEMM (QKV 4704 columns)."""
    import speculative_decoding_02_amd as sd
    w = synth.weights_np(HD168)
    acc = run_teacher_forced(sd, HD168, w, 4, 4, False, rounds=3, prompt_len=80)
    assert acc > 0


def test_greedy_streams_equal_plain_greedy_with_ngram_drafts(toy_w):
    """Greedy speculative output is the target's own greedy text whatever the
    drafts; here the batched prompt-lookup drafter, on prompts that repeat so
    that some drafts are right.  The drafts equal the oracle's search over
    each sequence's history."""
    import speculative_decoding_02_amd as sd
    tdev, = dev_weights(toy_w)
    B, K, n_max, n_new = 4, 4, 3, 40
    base = batch_prompts(synth.TOY.vocab, B, 6)
    prompts = np.concatenate([base, base, base[:, :4]], axis=1)  # period-6 text
    bc = sd.spec_batch_init(synth.TOY, tdev, prompts, k_max=K, max_seq=prompts.shape[1] + 64,
                            greedy=True)
    buf = BatchBuffers(B, K, synth.TOY.vocab)
    done = np.zeros(B, np.int64)
    accepted = 0
    while done.min() < n_new:
        st = sd.spec_batch_get_state(bc)
        sd.spec_batch_draft_ngram(bc, K, n_max, buf.d, buf.D)
        sd.spec_batch_sync(bc)
        d = buf.d.cpu().numpy()
        Dn = buf.D.cpu().numpy()
        for b in range(B):
            L = int(st["len"][b])
            hist = sd.spec_batch_get_history(bc, b, L + 1)
            ref, _ = oracle.ngram_draft(hist, L, K, n_max)
            assert list(d[b]) == list(ref), (b, d[b], ref)
            onehot = np.zeros((K, synth.TOY.vocab), np.float32)
            onehot[np.arange(K), ref] = 1.0
            assert np.array_equal(Dn[b], onehot)
        sd.spec_batch_verify(bc, K, 0, buf.d, buf.D, buf.out, buf.nacc)
        sd.spec_batch_commit(bc, buf.out, buf.nacc)
        sd.spec_batch_sync(bc)
        n = buf.nacc.cpu().numpy()
        accepted += int(n.sum())
        done += n + 1
    st = sd.spec_batch_get_state(bc)
    assert np.all(st["device_error"] == 0)
    Tm = oracle.Model(synth.TOY, toy_w)
    for b in range(B):
        gen = sd.spec_batch_get_history(bc, b, int(st["len"][b]) + 1)[prompts.shape[1]:]
        ref = oracle.generate(Tm, prompts[b], len(gen), greedy=True)
        np.testing.assert_array_equal(gen, ref)
    print(f"greedy n-gram batch: {accepted} drafts accepted")
    sd.spec_batch_destroy(bc)


@pytest.mark.parametrize("greedy", [False, True])
def test_8b_shaped_slice_batch(greedy):
    """Full width (d 4096) and vocabulary (128256), 2 layers, B = 3, K = 4
    (15 rows, two row tiles)."""
    import speculative_decoding_02_amd as sd
    tcfg = synth.L8B.replace(name="8b-slice-2L", n_layers=2)
    tw = synth.weights_torch(tcfg, device="cuda")
    torch.cuda.synchronize()
    tb = synth.torch_to_bits(tw)
    B, K, seed, rounds, plen = 3, 4, 1003, 2, 10
    prompts = batch_prompts(tcfg.vocab, B, plen)
    max_seq = plen + rounds * (K + 1) + 8
    bc = sd.spec_batch_init(tcfg, tw, prompts, k_max=K, max_seq=max_seq, greedy=greedy)
    Tm = oracle.Model(tcfg, tb)
    shadows = [SeqShadow(Tm, prompts[b], max_seq) for b in range(B)]
    buf = BatchBuffers(B, K, tcfg.vocab)
    rng = np.random.default_rng(7)
    stats = {}
    for _ in range(rounds):
        # drafts drawn from sparse random rows: what is checked is the pass
        # and the rule on them
        D_np = rng.dirichlet(np.full(tcfg.vocab, 0.05), size=(B, K)).astype(np.float32)
        D_np /= D_np.sum(axis=-1, keepdims=True)
        d_np = np.stack([[oracle.draft_sample(D_np[b, i], seed, shadows[b].LT + 1 + i, b, 0, greedy)
                          for i in range(K)] for b in range(B)]).astype(np.int32)
        g = gpu_batch_round(sd, bc, K, seed, buf, d_np, D_np)
        for b, sh in enumerate(shadows):
            sh.check(b, g, d_np[b], D_np[b], K, seed, greedy, stats=stats)
        st = sd.spec_batch_get_state(bc)
        assert np.all(st["device_error"] == 0)
        assert list(st["len"]) == [sh.LT for sh in shadows]
    print(f"8B slice batch greedy={greedy}: logit err {stats['logit']:.2e}, prob err "
          f"{stats['prob']:.2e}, near-ties {stats.get('near_ties', 0)}")
    sd.spec_batch_destroy(bc)


def test_graph_replays_equal_eager_launches():
    """The captured verify pass, replayed round after round (with host work
    and synchronisation between replays), gives bit-identical rows, logits
    and decisions to the same pass launched without a graph."""
    import speculative_decoding_02_amd as sd
    w = synth.weights_np(MID)
    tdev, = dev_weights(w)
    B, K, V = 5, 3, MID.vocab
    prompts = batch_prompts(V, B, 10)
    ctxs = [sd.spec_batch_init(MID, tdev, prompts, k_max=K, max_seq=40, greedy=False,
                               use_graphs=g) for g in (True, False)]
    bufs = [BatchBuffers(B, K, V) for _ in ctxs]
    rng = np.random.default_rng(3)
    for r in range(5):
        D_np = rng.dirichlet(np.full(V, 0.3), size=(B, K)).astype(np.float32)
        d_np = D_np.argmax(axis=-1).astype(np.int32)
        got = [gpu_batch_round(sd, bc, K, 11, buf, d_np, D_np) for bc, buf in zip(ctxs, bufs)]
        for key in ("T", "logits", "out", "nacc"):
            assert np.array_equal(got[0][key], got[1][key]), (r, key)
    lens = [sd.spec_batch_get_state(bc)["len"] for bc in ctxs]
    assert np.array_equal(lens[0], lens[1])
    for bc in ctxs:
        sd.spec_batch_destroy(bc)


def test_8b_full_size_batch_sampled():
    """The batched verify at the benchmark's size: the full 8B-shaped target
    (32 layers), 1024-token prompts, K = 4.  What the oracle computes output
    by output: each sequence's decision on the GPU's own rows (bit-exact,
    sequence index b), every row a distribution.  And batch invariance: a
    3-sequence batch and a 4-sequence batch holding the same three (both
    through the wide GEMM) give those three bit-identical rows, logits and
    decisions -- no row's arithmetic depends on the other sequences."""
    import speculative_decoding_02_amd as sd
    tcfg = synth.L8B
    tw = synth.weights_torch(tcfg, device="cuda")
    torch.cuda.synchronize()
    K, seed, rounds, plen = 4, 1003, 2, 1024
    V = tcfg.vocab
    prompts = batch_prompts(V, 4, plen)
    max_seq = plen + rounds * (K + 1) + 8
    big = sd.spec_batch_init(tcfg, tw, prompts, k_max=K, max_seq=max_seq, greedy=False)
    small = sd.spec_batch_init(tcfg, tw, prompts[:3], k_max=K, max_seq=max_seq, greedy=False)
    bb, bs = BatchBuffers(4, K, V), BatchBuffers(3, K, V)
    rng = np.random.default_rng(5)
    LT = np.full(4, plen - 1)
    for _ in range(rounds):
        D_np = rng.dirichlet(np.full(V, 0.05), size=(4, K)).astype(np.float32)
        D_np /= D_np.sum(axis=-1, keepdims=True)
        d_np = np.stack([[oracle.draft_sample(D_np[b, i], seed, int(LT[b]) + 1 + i, b, 0, False)
                          for i in range(K)] for b in range(4)]).astype(np.int32)
        g = gpu_batch_round(sd, big, K, seed, bb, d_np, D_np)
        h = gpu_batch_round(sd, small, K, seed, bs, d_np[:3], D_np[:3])
        for key in ("T", "logits", "out", "nacc"):
            assert np.array_equal(g[key][:3], h[key]), key
        for b in range(4):
            rows = g["T"][b]
            assert np.all(rows >= 0.0) and np.abs(rows.sum(axis=-1) - 1.0).max() < 1e-4
            rc, n, out = oracle.verify_sample(rows, D_np[b], d_np[b], seed, b, 0, int(LT[b]) + 1)
            assert rc == 0 and n == g["nacc"][b] and list(out[: n + 1]) == list(g["out"][b][: n + 1])
            LT[b] += n + 1
        assert list(sd.spec_batch_get_state(big)["len"]) == list(LT)
    sd.spec_batch_destroy(big)
    sd.spec_batch_destroy(small)


def test_batch_errors(toy_w):
    import speculative_decoding_02_amd as sd
    tdev, = dev_weights(toy_w)
    V = synth.TOY.vocab
    pr = batch_prompts(V, 2, 8)
    with pytest.raises(sd.SpecError) as e:  # 17 sequences x 8 rows > 128
        sd.spec_batch_init(synth.TOY, tdev, batch_prompts(V, 17, 8), k_max=7, max_seq=64,
                           greedy=False)
    assert e.value.code == sd.SPEC_ERR_ARG
    with pytest.raises(sd.SpecError) as e:
        sd.spec_batch_init(synth.TOY, tdev, batch_prompts(V, 33, 8), k_max=1, max_seq=64,
                           greedy=False)
    assert e.value.code == sd.SPEC_ERR_ARG
    bad = pr.copy()
    bad[1, 3] = V
    with pytest.raises(sd.SpecError) as e:
        sd.spec_batch_init(synth.TOY, tdev, bad, k_max=2, max_seq=64, greedy=False)
    assert e.value.code == sd.SPEC_ERR_ARG
    with pytest.raises(sd.SpecError) as e:
        sd.spec_batch_init(synth.TOY, tdev, pr, k_max=2, max_seq=10, greedy=False)
    assert e.value.code == sd.SPEC_ERR_CAPACITY

    K = 2
    max_seq = 8 + 3 * (K + 1)
    bc = sd.spec_batch_init(synth.TOY, tdev, pr, k_max=K, max_seq=max_seq, greedy=False)
    buf = BatchBuffers(2, K, V)
    with pytest.raises(sd.SpecError) as e:
        sd.spec_batch_verify(bc, K + 1, 0, buf.d, buf.D, buf.out, buf.nacc)
    assert e.value.code == sd.SPEC_ERR_ARG
    with pytest.raises(sd.SpecError) as e:
        sd.spec_batch_verify(bc, K, 0, buf.d, None, buf.out, buf.nacc)  # sampling needs D
    assert e.value.code == sd.SPEC_ERR_ARG
    with pytest.raises(sd.SpecError) as e:
        sd.spec_batch_commit(bc, buf.out, buf.nacc)
    assert e.value.code == sd.SPEC_ERR_STATE
    with pytest.raises(sd.SpecError) as e:
        sd.spec_batch_draft_ngram(bc, K, 9, buf.d, buf.D)
    assert e.value.code == sd.SPEC_ERR_ARG
    # rounds until a sequence's positions would pass max_seq
    buf.D.fill_(1.0 / V)
    torch.cuda.synchronize()
    raised = False
    for _ in range(max_seq):
        sd.spec_batch_draft_ngram(bc, K, 2, buf.d, buf.D)
        try:
            sd.spec_batch_verify(bc, K, 0, buf.d, buf.D, buf.out, buf.nacc)
        except sd.SpecError as err:
            assert err.code == sd.SPEC_ERR_CAPACITY
            raised = True
            break
        with pytest.raises(sd.SpecError) as e:  # one verify at a time
            sd.spec_batch_verify(bc, K, 0, buf.d, buf.D, buf.out, buf.nacc)
        assert e.value.code == sd.SPEC_ERR_STATE
        sd.spec_batch_commit(bc, buf.out, buf.nacc)
    assert raised
    st = sd.spec_batch_get_state(bc)
    assert np.all(st["device_error"] == 0)
    assert np.any(st["len"] + K >= max_seq) and np.all(st["len"] < max_seq)
    with pytest.raises(sd.SpecError) as e:
        sd.spec_batch_get_history(bc, 2, 4)
    assert e.value.code == sd.SPEC_ERR_ARG
    sd.spec_batch_destroy(bc)
