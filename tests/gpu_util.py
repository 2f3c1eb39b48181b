"""Helpers for the GPU parity tests: device copies of synthetic weights, a
round driver over the C ABI, and an oracle shadow that follows the GPU
pipeline teacher-forced on the GPU's own tokens and checks every component:
draft rows and draft samples, target logits and rows, the accept/reject
decision (bit-exact), near-ties in greedy mode, and the committed state."""
from __future__ import annotations

import numpy as np

import oracle
import synth

LOGIT_TOL = 2e-2     # max-abs logit difference, bf16 weights / fp32 accumulation
PROB_TOL = 1e-4      # max-abs probability difference
NEAR_TIE = 1e-3      # oracle logit gap under which a greedy mismatch is a near-tie


def dev_weights(*dicts):
    """numpy bf16-bit dicts -> torch bf16 device dicts; arrays shared between
    the dicts (same object) map to one device tensor, so the library sees a
    shared embedding / LM head."""
    import torch
    cache = {}

    def conv(a):
        if id(a) not in cache:
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
            cache[id(a)] = (a, t.view(torch.bfloat16))
        return cache[id(a)][1]

    return [{k: conv(v) for k, v in d.items()} for d in dicts]


class Buffers:
    def __init__(self, K: int, V: int):
        import torch
        self.d = torch.zeros(K, dtype=torch.int32, device="cuda")
        self.D = torch.zeros(K, V, dtype=torch.float32, device="cuda")
        self.T = torch.zeros(K + 1, V, dtype=torch.float32, device="cuda")
        self.logits = torch.zeros(K + 1, V, dtype=torch.float32, device="cuda")
        self.out = torch.zeros(K + 1, dtype=torch.int32, device="cuda")
        self.nacc = torch.zeros(1, dtype=torch.int32, device="cuda")


def gpu_plain_step(sd, ctx, seed, b: Buffers):
    """One plain decode step through the same boundary: verify with K = 0
    (no drafts) and commit."""
    sd.spec_verify(ctx, 0, seed, None, None, b.out, b.nacc, b.T, b.logits)
    sd.spec_commit(ctx, b.out, b.nacc)
    sd.spec_sync(ctx)
    return {"out": b.out.cpu().numpy().copy(), "nacc": int(b.nacc.cpu().numpy()[0]),
            "T": b.T.cpu().numpy().copy(), "logits": b.logits.cpu().numpy().copy()}


def gpu_round(sd, ctx, K, seed, b: Buffers, with_rows=True):
    sd.spec_draft(ctx, K, seed, b.d, b.D)
    sd.spec_verify(ctx, K, seed, b.d, b.D, b.out, b.nacc, b.T if with_rows else None,
                   b.logits if with_rows else None)
    sd.spec_commit(ctx, b.out, b.nacc)
    sd.spec_sync(ctx)
    res = {"d": b.d.cpu().numpy().copy(), "out": b.out.cpu().numpy().copy(),
           "nacc": int(b.nacc.cpu().numpy()[0])}
    if with_rows:
        res["D"] = b.D.cpu().numpy().copy()
        res["T"] = b.T.cpu().numpy().copy()
        res["logits"] = b.logits.cpu().numpy().copy()
    return res


class Shadow:
    """Oracle copy of the pipeline state (committed history, cache lengths)."""

    def __init__(self, tcfg, tw_bits, dcfg, dw_bits, prompt, max_seq, K, seed, greedy, c=0):
        self.T = oracle.Model(tcfg, tw_bits)
        self.D = oracle.Model(dcfg, dw_bits)
        self.kvT = oracle.KV(self.T, max_seq)
        self.kvD = oracle.KV(self.D, max_seq)
        self.hist = [int(x) for x in prompt]
        self.LT = self.LD = len(prompt) - 1
        self.K, self.seed, self.greedy, self.c = K, seed, greedy, c
        self.V = tcfg.vocab
        if self.LT > 0:
            oracle.forward(self.T, self.kvT, self.hist[: self.LT], 0, want_logits=False)
            oracle.forward(self.D, self.kvD, self.hist[: self.LT], 0, want_logits=False)
        self.near_ties = 0
        self.max_logit_err = 0.0
        self.max_prob_err = 0.0
        self.max_draft_prob_err = 0.0

    def catch_up_draft(self):
        """The library's draft catch-up: when more committed rows lag than
        one draft step can carry (after plain steps or n-gram rounds), the
        draft cache is prefilled with them first."""
        if self.LT - self.LD > 7:
            oracle.forward(self.D, self.kvD, self.hist[self.LD: self.LT], self.LD, want_logits=False)
            self.LD = self.LT

    def check_plain(self, g):
        """One plain decode step (verify with K = 0): the row of the pending
        token, T_1 within tolerance, and the emitted token bit-exact on the
        GPU's own row (argmax, or inverse CDF with w2 at the new position)."""
        LT = self.LT
        lg = oracle.forward(self.T, self.kvT, [self.hist[LT]], LT)
        lerr = float(np.abs(lg - g["logits"]).max())
        self.max_logit_err = max(self.max_logit_err, lerr)
        assert lerr <= LOGIT_TOL, ("logits", lerr)
        Tor = oracle.softmax_f32(lg[0])
        perr = float(np.abs(Tor - g["T"][0]).max())
        self.max_prob_err = max(self.max_prob_err, perr)
        assert perr <= PROB_TOL, ("target row", perr)
        row = g["T"][0]
        if self.greedy:
            ref = oracle.argmax_low(row)
        else:
            u = oracle.u24(oracle.uniform_words(self.seed, LT + 1, 0, self.c)[2])
            ref = oracle.sample_icdf([oracle.fix(float(x)) for x in row], u)
            if ref < 0:
                ref = oracle.argmax_low(row)
        assert g["nacc"] == 0 and int(g["out"][0]) == ref, (g["nacc"], int(g["out"][0]), ref)
        self.hist.append(ref)
        self.LT = LT + 1
        return ref

    def check_round(self, g):
        self.catch_up_draft()
        K, LT, LD = self.K, self.LT, self.LD
        d = g["d"]
        # draft steps: rows, probabilities, samples
        for s in range(K):
            rows = self.hist[LD: LT + 1] if s == 0 else [int(d[s - 1])]
            pos0 = LD if s == 0 else LT + s
            lg = oracle.forward(self.D, self.kvD, rows, pos0)[-1]
            Dor = oracle.softmax_f32(lg)
            err = float(np.abs(Dor - g["D"][s]).max())
            self.max_draft_prob_err = max(self.max_draft_prob_err, err)
            assert err <= PROB_TOL, ("draft row", s, err)
            ref = oracle.draft_sample(g["D"][s], self.seed, LT + s + 1, 0, self.c, self.greedy)
            assert ref == int(d[s]), ("draft sample", s, ref, int(d[s]))
        # verify pass
        rows = [self.hist[LT]] + [int(x) for x in d]
        lgT = oracle.forward(self.T, self.kvT, rows, LT)
        lerr = float(np.abs(lgT - g["logits"]).max())
        self.max_logit_err = max(self.max_logit_err, lerr)
        assert lerr <= LOGIT_TOL, ("logits", lerr)
        Tor = np.stack([oracle.softmax_f32(r) for r in lgT])
        perr = float(np.abs(Tor - g["T"]).max())
        self.max_prob_err = max(self.max_prob_err, perr)
        assert perr <= PROB_TOL, ("target rows", perr)
        # accept/reject: bit-exact on the GPU's own rows
        if self.greedy:
            rc, n, out = oracle.verify_greedy(g["T"], d)
        else:
            rc, n, out = oracle.verify_sample(g["T"], g["D"], d, self.seed, 0, self.c, LT + 1)
        assert rc == 0 and n == g["nacc"] and list(out) == list(g["out"]), (n, out, g["nacc"], g["out"])
        assert 0 <= n <= K
        # greedy: every emitted token is the oracle's argmax or a near-tie
        if self.greedy:
            for j in range(n + 1):
                tok = int(g["out"][j])
                a = int(np.argmax(lgT[j]))
                if tok != a:
                    gap = float(lgT[j][a] - lgT[j][tok])
                    assert gap < NEAR_TIE, ("greedy mismatch beyond near-tie", j, gap)
                    self.near_ties += 1
        # commit
        self.hist += [int(x) for x in g["out"][: n + 1]]
        self.LD = LT + min(n + 1, K)
        self.LT = LT + n + 1
        return n
