"""Benchmark of the speculative-decoding hot path on one MI355X.

A step is one speculative round of the whole path: K draft-model steps
(hipGraph), the (K+1)-row target verify pass, the accept/reject rule and the
commit, at batch 1.  Workload: 8B-shaped Llama target (32 layers, d 4096,
32/8 heads x 128, FFN 14336, vocab 128256, RoPE theta 5e5) with a 1B-shaped
draft (16 layers, d 2048, 32/8 heads x 64, FFN 8192, tied head), bf16
random-init weights N(0, 0.02), 1024-token uniform prompt, K = 4,
temperature-1 sampling.  Inputs are resident in HBM before timing starts.

Prints one JSON line: accepted tokens/s (value), verify-pass HBM GB/s, the
roofline of the dominant kernel (the feed-forward gate/up GEMM) from hipEvents
around each of its launches, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak of the MI355X
# HBM traffic of the dominant kernel, from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE) of the native driver spec_run on the 8B-shaped pair
# at K = 4, with the hash of the kernel sources they were taken with; used only
# for that workload and while the sources still hash the same.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gateup_8b_k4_traffic.txt")
KERNEL_SOURCES = ("k_gemm.hip", "k_gemm.h", "common.h")  # the GEMM kernels and their launch plans
COPY_CALIB_BYTES = 1 << 30


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "speculative_decoding_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(target_only: bool = False):
    """(bytes per launch, note) from the committed counter summary -- the
    1:2 target/draft launch mix of the draft-model rounds, or the target
    launches alone -- or (None, reason) when there is none or the kernel
    sources changed since."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line:
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_digest():
            return None, "kernel sources changed since the counters were taken"
        key = "traffic_bytes_per_launch_target" if target_only else "traffic_bytes_per_launch"
        return int(kv[key]), os.path.relpath(TRAFFIC_FILE, ROOT) + " (" + key + ")"
    except (OSError, KeyError, ValueError):
        return None, "no counter summary"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Keys and values as the method needs them: one bf16 value per element.  The
# cache here keeps a second bf16 plane (the low part) for precision; those
# extra bytes are this design's overhead and are not counted as algorithmic.
KV_ELEM_BYTES = 2


def verify_pass_bytes(cfg, K: int, L: int, B: int = 1) -> int:
    """Algorithmic bytes of one verify pass over B sequences: every weight
    once, K+1 embedding rows per sequence, keys/values of L+K+1 positions read
    and K+1 written (bf16) per sequence, T rows written."""
    w = cfg.weight_bytes()
    emb = B * (K + 1) * cfg.d_model * 2
    kv_tok = cfg.n_layers * 2 * cfg.n_kv_heads * cfg.head_dim * KV_ELEM_BYTES
    kv = B * ((L + K + 1) * kv_tok + (K + 1) * kv_tok)
    t_rows = B * (K + 1) * cfg.vocab * 4
    return w + emb + kv + t_rows


def draft_step_bytes(cfg, L: int) -> int:
    kv_tok = cfg.n_layers * 2 * cfg.n_kv_heads * cfg.head_dim * KV_ELEM_BYTES
    return cfg.weight_bytes() + cfg.d_model * 2 + (L + 1) * kv_tok + kv_tok + cfg.vocab * 4


def gateup_bytes(cfg, rows: int) -> int:
    """Algorithmic bytes of one feed-forward gate/up GEMM launch: W_gate and
    W_up once, the norm gain, the input rows (fp32) and the SiLU*up output
    rows (fp32)."""
    d, F = cfg.d_model, cfg.d_ffn
    return 2 * F * d * 2 + d * 2 + rows * d * 4 + rows * F * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--k", type=int, default=4)
    ap.add_argument("--pair", default="8b", choices=["toy", "1.3b", "8b", "31b"])
    ap.add_argument("--prompt-len", type=int, default=None)
    ap.add_argument("--greedy", action="store_true")
    ap.add_argument("--drafter", default="model", choices=["model", "ngram", "heads"],
                    help="draft model (default), the prompt-lookup drafter (spec_draft_ngram) or "
                         "K multi-token-prediction heads on the target (spec_draft_heads)")
    ap.add_argument("--ngram-n", type=int, default=3, help="longest key of the n-gram drafter")
    ap.add_argument("--gemm-sweep", action="store_true",
                    help="batched verify: time the weight-streaming GEMM (spec_mat_mul) on the "
                         "8B-shaped matrices for M = B(K+1) = 1..128 rows")
    ap.add_argument("--batch-sweep", default=None, metavar="B1,B2,...",
                    help="batched verify (spec_batch_*): B sequences of the target verified in "
                         "one pass, n-gram drafts; prints one JSON line with a row per B")
    ap.add_argument("--ar-bench", action="store_true",
                    help="the accept/reject rule alone (spec_accept_reject and its allocation-free "
                         "variant) on 64 sequences x K = 8 x vocab 32000 at draft noise sigma = "
                         "0.1 / 0.5 / 2.0, five input sets rotated (696 MB, past the 256 MB MALL)")
    ap.add_argument("--adaptive-k", action="store_true",
                    help="choose K every few rounds from the measured acceptance rate "
                         "(spec_alpha_from_tokens + spec_choose_k) instead of a fixed K")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=16)
    ap.add_argument("--kernel-rounds", type=int, default=5)
    ap.add_argument("--plain-steps", type=int, default=40,
                    help="plain decode steps (verify with K = 0) timed after the rounds")
    ap.add_argument("--ceiling-gib", type=int, default=16,
                    help="buffer size of the streaming-read ceiling (0: skip)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="first run a plain copy of 1 GiB three times (calibrates HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the hot path is "
              "measured on a single MI355X; multi-GPU sharding is described in DESIGN.md, not run.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import speculative_decoding_02_amd as sd
    import synth

    if args.gemm_sweep:
        print(json.dumps(gemm_sweep(sd, torch, np)), flush=True)
        return
    if args.batch_sweep:
        print(json.dumps(batch_sweep(sd, torch, np, synth, args)), flush=True)
        return
    if args.ar_bench:
        print(json.dumps(ar_bench(sd, torch, np, synth, args)), flush=True)
        return

    tcfg, dcfg = synth.PAIRS[args.pair]
    K = args.k
    plen = args.prompt_len or {"toy": 32, "1.3b": 512, "8b": 1024, "31b": 2048}[args.pair]
    rounds_total = args.steps + args.warmup
    max_seq = plen + (K + 1) * (rounds_total + args.kernel_rounds) + args.plain_steps + 24
    torch.cuda.set_device(0)
    if args.copy_calib:
        # a plain elementwise copy (negation): COPY_CALIB_BYTES read and written per launch
        xs = torch.ones(COPY_CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        ys = torch.empty_like(xs)
        for _ in range(3):
            torch.neg(xs, out=ys)
        torch.cuda.synchronize()
        del xs, ys
        log("copy calibration: 3 launches of torch.neg over 1 GiB fp32")
    t0 = time.time()
    tw = synth.weights_torch(tcfg, device="cuda")
    share = ("embed", "lm_head") if args.pair in ("toy", "1.3b") else ()
    dw = synth.weights_torch(dcfg, seed=synth.SEED_WEIGHTS + 1, device="cuda", share_from=tw,
                             share=share)
    torch.cuda.synchronize()
    log(f"weights generated in {time.time() - t0:.1f}s")
    prompt = synth.prompt(tcfg.vocab, plen)
    t0 = time.time()
    if args.adaptive_k:
        K = sd.SPEC_K_MAX
        max_seq = plen + (K + 1) * (rounds_total + 3 * K + 8) + 16
    ctx = sd.spec_init(tcfg, tw, dcfg, dw, prompt, k_max=K, max_seq=max_seq, greedy=args.greedy,
                       use_graphs=True, profile_kernels=False)
    log(f"spec_init (pack + prefill {plen} tokens) in {time.time() - t0:.1f}s")
    if args.drafter == "heads":
        sd.spec_heads_init(ctx, synth.heads_torch(tcfg, K), K)

    V = tcfg.vocab
    d = torch.zeros(K, dtype=torch.int32, device="cuda")
    D = torch.zeros(K, V, dtype=torch.float32, device="cuda")
    out = torch.zeros(K + 1, dtype=torch.int32, device="cuda")
    nacc = torch.zeros(1, dtype=torch.int32, device="cuda")
    seed = synth.SEED_PHILOX
    stream = torch.cuda.ExternalStream(sd.spec_stream(ctx))

    def one_round(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if args.drafter == "ngram":
            sd.spec_draft_ngram(ctx, K, args.ngram_n, d, D)
        elif args.drafter == "heads":
            sd.spec_draft_heads(ctx, K, seed, d, D)
        else:
            sd.spec_draft(ctx, K, seed, d, D)
        if ev is not None:
            ev[1].record(stream)
        sd.spec_verify(ctx, K, seed, d, D, out, nacc)
        if ev is not None:
            ev[2].record(stream)
        sd.spec_commit(ctx, out, nacc)

    if args.adaptive_k:
        res = adaptive_k_run(sd, torch, ctx, stream, d, D, out, nacc, seed, args, tcfg, dcfg, plen)
        sd.spec_destroy(ctx)
        print(json.dumps(res), flush=True)
        return

    for _ in range(args.warmup):
        one_round()
    sd.spec_sync(ctx)
    st0 = sd.spec_get_state(ctx)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    w0 = time.perf_counter()
    for i in range(args.steps):
        one_round(evs[i])
    t_end.record(stream)
    sd.spec_sync(ctx)
    wall = time.perf_counter() - w0
    st1 = sd.spec_get_state(ctx)
    assert st1["device_error"] == 0, st1
    ms_total = t_start.elapsed_time(t_end)
    tokens = st1["target_len"] - st0["target_len"]
    draft_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    verify_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    tok_per_s = tokens / (ms_total / 1e3)
    tpr = tokens / args.steps
    L_mid = plen + tokens // 2 + st0["target_len"] - plen
    vbytes = verify_pass_bytes(tcfg, K, L_mid)
    vgbs = vbytes / (np.median(verify_ms) / 1e3) / 1e9
    # the prompt-lookup drafter reads the history and writes K one-hot rows;
    # the heads stream their K [d][d] matrices and the LM head once and
    # write K rows
    if args.drafter == "model":
        dbytes = K * draft_step_bytes(dcfg, L_mid)
    elif args.drafter == "heads":
        dbytes = K * tcfg.d_model ** 2 * 2 + V * tcfg.d_model * 2 + K * V * 4
    else:
        dbytes = K * V * 4 + (L_mid + 1) * 4
    dgbs = dbytes / (np.median(draft_ms) / 1e3) / 1e9

    # dominant kernel: the feed-forward gate/up GEMM.  A second timed region
    # replays the same rounds with plain launches and a hipEvent pair on the
    # context's stream around every gate/up launch (draft and target).
    # The gate/up GEMM and the O projection before it stamp their workgroups'
    # ends (device wall clock); a gate/up launch lasts from the O projection's
    # end to its own.  These rounds replay graphs captured with the stamps on,
    # back-to-back like the timed region.
    roof = None
    if not args.no_kernel_timing:
        sd.spec_set_profiling(ctx, True)
        kts, heads_ms = [], []
        for _ in range(args.kernel_rounds):
            one_round()
            kts.append(sd.spec_kernel_times(ctx))
            heads_ms.append(sd.spec_head_time(ctx))
        sd.spec_set_profiling(ctx, False)
        n_draft = K * dcfg.n_layers if args.drafter == "model" else 0
        kt_d = np.concatenate([k[:n_draft] for k in kts])
        kt_t = np.concatenate([k[n_draft:] for k in kts])
        b_d = gateup_bytes(dcfg, 1) * len(kt_d)
        b_t = gateup_bytes(tcfg, K + 1) * len(kt_t)
        n_l = len(kt_d) + len(kt_t)
        avg_bytes = (b_d + b_t) / n_l
        avg_ms = float((kt_d.sum() + kt_t.sum()) / n_l)
        ach = avg_bytes / (avg_ms / 1e3) / 1e9
        if args.pair == "8b" and (K == 4 or len(kt_d) == 0):
            traffic, traffic_note = measured_traffic(target_only=len(kt_d) == 0)
        else:  # the counters were taken on the 8B-shaped pair's K = 4 launch mix
            traffic, traffic_note = None, "counters cover the 8B-shaped pair at K = 4 only"
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                "traffic_note": traffic_note,
                "kernel": "gemm_skinny<..., EPI_SILU>: gate/up GEMM + RMSNorm scale + SiLU*up",
                "timing": f"device wall-clock end stamps (end of the preceding O projection "
                          f"to end of the gate/up launch) over {args.kernel_rounds} graph-replayed "
                          f"rounds",
                "launches": n_l, "avg_launch_us": round(avg_ms * 1e3, 2),
                "avg_algorithmic_bytes": int(avg_bytes),
                "target_launch_us": round(float(kt_t.mean()) * 1e3, 2),
                "target_GBs": round(gateup_bytes(tcfg, K + 1) / (float(kt_t.mean()) / 1e3) / 1e9, 1),
                "draft_launch_us": round(float(kt_d.mean()) * 1e3, 2) if len(kt_d) else None,
                "draft_GBs": (round(gateup_bytes(dcfg, 1) / (float(kt_d.mean()) / 1e3) / 1e9, 1)
                              if len(kt_d) else None)}

    # the verify pass's LM head: (K+1) rows x vocab x d, timed like the
    # gate/up GEMM in the stamped rounds; matrix-core use against the dense
    # bf16 peak, useful (K+1 rows) and issued (the 16-row MFMA tile)
    lm_head = None
    if roof is not None:
        hm = [x for x in heads_ms if x > 0]
        if hm:
            t = float(np.mean(hm)) / 1e3
            flop = 2 * (K + 1) * V * tcfg.d_model
            lm_bytes = V * tcfg.d_model * 2 + (K + 1) * V * 4
            lm_head = {"us": round(t * 1e6, 2), "launches": len(hm),
                       "GB_s": round(lm_bytes / t / 1e9, 1),
                       "useful_TFLOP_s": round(flop / t / 1e12, 2),
                       "mfma_util": round(flop / t / 1e12 / PEAK_BF16_TFLOPS, 5),
                       "mfma_util_issued": round(2 * 16 * V * tcfg.d_model / t / 1e12
                                                 / PEAK_BF16_TFLOPS, 5),
                       "peak_TFLOP_s": PEAK_BF16_TFLOPS}

    # acceptance record of the timed rounds: the context counts every commit
    # by (K, n_acc); alpha_i = P(d_i accepted | d_1..d_{i-1} accepted)
    acc = st1["accept_counts"][K] - st0["accept_counts"][K]
    reach = [int(acc[i:].sum()) for i in range(K + 1)]
    acceptance = {"rounds": reach[0],
                  "n_acc_histogram": [int(x) for x in acc[: K + 1]],
                  "alpha_per_position": [round(reach[i + 1] / reach[i], 4) if reach[i] else None
                                         for i in range(K)]}

    # plain decoding on the same kernels: verify with K = 0 (one row, the
    # next token from T_1) and commit, back to back
    plain = None
    if args.plain_steps > 0:
        pout = torch.zeros(1, dtype=torch.int32, device="cuda")
        pn = torch.zeros(1, dtype=torch.int32, device="cuda")

        def plain_step():
            sd.spec_verify(ctx, 0, seed, None, None, pout, pn)
            sd.spec_commit(ctx, pout, pn)

        for _ in range(3):
            plain_step()
        sd.spec_sync(ctx)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        for _ in range(args.plain_steps):
            plain_step()
        p1.record(stream)
        sd.spec_sync(ctx)
        assert sd.spec_get_state(ctx)["device_error"] == 0
        pms = p0.elapsed_time(p1) / args.plain_steps
        pbytes = verify_pass_bytes(tcfg, 0, L_mid)
        plain = {"steps": args.plain_steps, "ms_per_token": round(pms, 4),
                 "tokens_per_s": round(1e3 / pms, 2),
                 "one_row_pass_GB_s": round(pbytes / (pms / 1e3) / 1e9, 1)}

    # streaming-read ceiling over a buffer far larger than the 256 MB MALL
    ceiling = None
    if args.ceiling_gib > 0:
        buf = torch.zeros(args.ceiling_gib << 30, dtype=torch.uint8, device="cuda")
        c_gbs = sd.spec_read_ceiling(buf, reps=2)
        del buf
        torch.cuda.empty_cache()
        ceiling = {"GB_s": round(c_gbs, 1), "bytes": args.ceiling_gib << 30,
                   "frac_of_peak": round(c_gbs / PEAK_HBM_GBS, 4),
                   "verify_frac_of_ceiling": round(vgbs / c_gbs, 4),
                   "roofline_frac_of_ceiling": round(roof["achieved"] / c_gbs, 4) if roof else None}

    proj = {f"alpha_{a}": round(sd.spec_expected_tokens(a, K)
                                / ((np.median(draft_ms) + np.median(verify_ms)) / 1e3), 1)
            for a in (0.5, 0.7, 0.8)}
    res = {
        "metric": "accepted tokens/s at batch 1, K=4; verify-pass HBM GB/s as % of MI355X peak",
        "value": round(tok_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{tcfg.name} target + "
                        + {"model": f"{dcfg.name} draft",
                           "ngram": f"prompt-lookup drafter (keys up to {args.ngram_n} tokens)",
                           "heads": f"{K} multi-token-prediction heads (random-init, "
                                    f"z = h + silu(W h), target LM head)"}[args.drafter]
                        + f", batch 1, K={K}, prompt {plen}, "
                        f"{'greedy' if args.greedy else 'temperature-1 sampling'}, random-init bf16",
            "K": K, "batch": 1, "prompt_len": plen, "mode": "greedy" if args.greedy else "sampling",
        },
        "verify_pass": {"ms_median": round(float(np.median(verify_ms)), 4),
                        "algorithmic_GB": round(vbytes / 1e9, 4),
                        "GB_s": round(vgbs, 1), "frac_of_peak": round(vgbs / PEAK_HBM_GBS, 4)},
        "draft_loop": {"ms_median": round(float(np.median(draft_ms)), 4),
                       "algorithmic_GB": round(dbytes / 1e9, 4), "GB_s": round(dgbs, 1)},
        "tokens_per_round": round(tpr, 4),
        # what the measured round time would give at the acceptance rates of
        # the pages' examples ([en] Floor 6): a projection, not a measurement
        "projection_tokens_per_s": proj,
        "projection_speedup_vs_plain": ({k: round(v / plain["tokens_per_s"], 3) for k, v in proj.items()}
                                        if plain else None),
        "target_passes_per_token": round(args.steps / max(tokens, 1), 4),
        "acceptance": acceptance,
        "plain_decode": plain,
        "speedup_vs_plain": round(tok_per_s / plain["tokens_per_s"], 4) if plain else None,
        "read_ceiling": ceiling,
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
        "lm_head": lm_head,
        "cpu_baseline": None,
    }
    log(json.dumps({k: res[k] for k in ("value", "ms_per_step", "verify_pass", "draft_loop",
                                         "tokens_per_round")}))

    if not args.no_cpu_baseline and args.drafter == "model":
        res["cpu_baseline"] = cpu_baseline(tcfg, dcfg, tw, dw, K, args, tpr, plen)
    sd.spec_destroy(ctx)
    print(json.dumps(res), flush=True)


def ar_call_bytes(n_acc, K: int, V: int) -> int:
    """Algorithmic bytes of one call of the rule over a batch: per sequence
    the gathered T_i(d_i), D_i(d_i) of every accept test it decides (fp32
    pairs: n + 1 on a reject at n, K when all pass), then the row it samples
    from -- T_j and D_j of the residual after a reject, T_{K+1} for the
    bonus."""
    total = 0
    for n in n_acc:
        n = int(n)
        tests = n + 1 if n < K else K
        total += 2 * 4 * tests + (2 * V * 4 if n < K else V * 4)
    return total


def ar_bench(sd, torch, np, synth, args):
    """The isolated accept/reject rule: B = 64 sequences, K = 8, V = 32000;
    T and D are fp32 softmaxes of N(0, 2) logits, draft logits = target +
    N(0, sigma).  Five input sets per sigma (T + D = 139 MB each) are
    rotated so no call finds its rows in the 256 MB MALL.  200 back-to-back
    calls are captured in a graph whose replays on the same stream are timed
    with hipEvents (us_per_call); the same calls made eagerly from Python
    are reported beside it (us_per_call_eager)."""
    B, K, V, n_sets, reps = 64, 8, 32000, 5, 200
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    rows = []
    for sigma in (0.1, 0.5, 2.0):
        sets = []
        for i in range(n_sets):
            T, D = synth.logit_pair(B, K, V, sigma, seed=synth.SEED_LOGITS + 10 * i)
            d = synth.drafts_from_rows(D, seed=synth.SEED_LOGITS + 10 * i)
            pos = (np.arange(B, dtype=np.int64) * 37 + 100 + i)
            sets.append((torch.from_numpy(T).cuda(), torch.from_numpy(D).cuda(),
                         torch.from_numpy(d).cuda(), torch.from_numpy(pos).cuda()))
        out = torch.zeros(B, K + 1, dtype=torch.int32, device="cuda")
        nacc = torch.zeros(B, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        res = {"sigma": sigma}
        for name, fn in (("spec_accept_reject", sd.spec_accept_reject),
                         ("spec_accept_reject_noalloc", sd.spec_accept_reject_noalloc)):
            nbytes = []
            for T, D, d, pos in sets:  # warm-up, and the bytes each set's decisions move
                fn(T, D, d, synth.SEED_PHILOX, pos, 0, False, out, nacc, stream=stream.cuda_stream)
                stream.synchronize()
                nbytes.append(ar_call_bytes(nacc.cpu().numpy(), K, V))
            # the calls as a captured graph, replayed on the same stream (as
            # inside the decoding loop), so the host's per-call cost and eager
            # launches do not pace the device
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(reps):
                    T, D, d, pos = sets[r % n_sets]
                    fn(T, D, d, synth.SEED_PHILOX, pos, 0, False, out, nacc,
                       stream=stream.cuda_stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                g.replay()
                e0.record(stream)
                for _ in range(3):
                    g.replay()
                e1.record(stream)
            e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (3 * reps)
            # the same calls made eagerly from Python (ctypes, two plain launches each)
            e0.record(stream)
            for r in range(reps):
                T, D, d, pos = sets[r % n_sets]
                fn(T, D, d, synth.SEED_PHILOX, pos, 0, False, out, nacc, stream=stream.cuda_stream)
            e1.record(stream)
            e1.synchronize()
            us_eager = e0.elapsed_time(e1) * 1e3 / reps
            del g
            b = float(np.mean([nbytes[r % n_sets] for r in range(reps)]))
            res[name] = {"us_per_call": round(us, 2), "algorithmic_MB": round(b / 1e6, 3),
                         "GB_s": round(b / (us * 1e-6) / 1e9, 1),
                         "us_per_call_eager": round(us_eager, 2)}
        res["mean_accepted_per_sequence"] = round(float(nacc.float().mean().item()), 3)
        rows.append(res)
        log(f"accept/reject sigma={sigma}: " + json.dumps(res))
        del sets
        torch.cuda.empty_cache()
    return {"metric": "isolated accept/reject: time per call and algorithmic GB/s",
            "unit": "us per call", "n_gpus": 1, "dtype": "f32 rows, u64 fixed point",
            "data": "synthetic", "higher_is_better": False,
            "config": {"workload": f"rule alone, B={B} sequences, K={K}, vocab {V}, sampling, "
                                   f"{n_sets} rotated input sets per sigma"},
            "peak_hbm_GB_s": PEAK_HBM_GBS, "sweep": rows}


def gemm_sweep(sd, torch, np):
    """Batched verify: one weight-streaming GEMM (spec_mat_mul) per shape for
    M = B(K+1) activation rows.  Weights rotate over copies (>= 1 GB in
    total) so every launch streams them from HBM.  Reported per M: time,
    weight GB/s, useful TFLOP/s (2 M N K) and the matrix-core work issued
    (16 MFMA rows per 8 activation rows, high and low parts)."""
    shapes = {"8b gate/up": (28672, 4096), "8b down": (4096, 14336), "8b qkv": (6144, 4096)}
    Ms = (1, 5, 8, 16, 32, 64, 96, 128)
    res = {}
    g = torch.Generator(device="cuda").manual_seed(7)
    for name, (N, K) in shapes.items():
        copies = max(2, -(-(1 << 30) // (N * K * 2)))
        mats, keep = [], []
        for _ in range(copies):
            W = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
            mats.append(sd.Mat(W))
            keep.append(W)
        del keep
        rows = []
        for M in Ms:
            X = torch.randn(M, K, device="cuda", generator=g)
            Y = torch.empty(M, N, device="cuda")
            for m in mats:
                m.mul(X, Y)
            reps = 4 * copies
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                mats[i % copies].mul(X, Y)
            e1.record()
            e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            rt = 1
            while 8 * rt < M:
                rt *= 2
            rows.append({"M": M, "us": round(us, 2),
                         "weight_GB_s": round(N * K * 2 / (us * 1e-6) / 1e9, 1),
                         "useful_TFLOP_s": round(2 * M * N * K / (us * 1e-6) / 1e12, 2),
                         "mfma_TFLOP_s": round(2 * 16 * rt * N * K / (us * 1e-6) / 1e12, 1)})
        res[name] = rows
        log(f"gemm sweep {name}: " + ", ".join(f"M={r['M']}: {r['us']} us" for r in rows))
        del mats
        torch.cuda.empty_cache()
    return {"metric": "batched verify GEMM (spec_mat_mul) time vs activation rows M = B(K+1)",
            "unit": "us per launch", "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
            "peak_hbm_GB_s": PEAK_HBM_GBS, "peak_bf16_dense_TFLOP_s": 2500.0,
            "config": {"workload": "8B-shaped weight matrices, M activation rows, weights cold"},
            "sweep": res}


def batch_sweep(sd, torch, np, synth, args):
    """Batched verify: for each B, a context with B sequences (prompt plen
    each, different texts) drafts with the batched prompt-lookup drafter and
    verifies all B (K+1) rows in one pass per round.  Reported per B: the
    verify pass (median of the timed rounds, events on the context's stream),
    its algorithmic GB/s (weights once, every sequence's cache and rows) and
    useful TFLOP/s (2 per weight per row), the round time, and the accepted
    tokens/s of the whole batch."""
    tcfg = synth.PAIRS[args.pair][0]
    K = args.k
    plen = args.prompt_len or {"toy": 32, "1.3b": 512, "8b": 1024, "31b": 2048}[args.pair]
    Bs = [int(x) for x in args.batch_sweep.split(",")]
    torch.cuda.set_device(0)
    tw = synth.weights_torch(tcfg, device="cuda")
    torch.cuda.synchronize()
    V = tcfg.vocab
    stream = torch.cuda.Stream()
    rows = []
    for B in Bs:
        prompts = np.stack([synth.prompt(V, plen, seed=100 + b) for b in range(B)])
        max_seq = plen + (K + 1) * (args.steps + args.warmup) + 16
        t0 = time.time()
        bc = sd.spec_batch_init(tcfg, tw, prompts, k_max=K, max_seq=max_seq, greedy=args.greedy,
                                stream=stream.cuda_stream)
        log(f"batch B={B}: spec_batch_init (pack + prefill {B} x {plen}) in {time.time() - t0:.1f}s")
        d = torch.zeros(B, K, dtype=torch.int32, device="cuda")
        D = torch.zeros(B, K, V, dtype=torch.float32, device="cuda")
        out = torch.zeros(B, K + 1, dtype=torch.int32, device="cuda")
        nacc = torch.zeros(B, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

        def rnd(ev=None):
            sd.spec_batch_draft_ngram(bc, K, args.ngram_n, d, D)
            if ev is not None:
                ev[0].record(stream)
            sd.spec_batch_verify(bc, K, synth.SEED_PHILOX, d, D, out, nacc)
            if ev is not None:
                ev[1].record(stream)
            sd.spec_batch_commit(bc, out, nacc)

        for _ in range(args.warmup):
            rnd()
        len0 = sd.spec_batch_get_state(bc)["len"].astype(np.int64)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            rnd(evs[i])
        e1.record(stream)
        sd.spec_batch_sync(bc)
        st = sd.spec_batch_get_state(bc)
        assert np.all(st["device_error"] == 0), st
        tokens = int((st["len"].astype(np.int64) - len0).sum())
        ms = e0.elapsed_time(e1)
        vms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        L_mid = plen + int((st["len"].astype(np.int64) - len0).mean()) // 2
        M = B * (K + 1)
        vbytes = verify_pass_bytes(tcfg, K, L_mid, B)
        flops = 2 * M * tcfg.weight_bytes() // 2
        rows.append({"B": B, "M": M, "verify_ms": round(vms, 3),
                     "verify_GB_s": round(vbytes / (vms / 1e3) / 1e9, 1),
                     "useful_TFLOP_s": round(flops / (vms / 1e3) / 1e12, 2),
                     "round_ms": round(ms / args.steps, 3),
                     "tokens_per_round": round(tokens / args.steps, 3),
                     "tokens_per_s": round(tokens / (ms / 1e3), 1)})
        log(f"batch B={B} (M={M}): verify {vms:.3f} ms, {rows[-1]['verify_GB_s']} GB/s, "
            f"{rows[-1]['tokens_per_s']} tokens/s")
        sd.spec_batch_destroy(bc)
        del d, D, out, nacc
        torch.cuda.empty_cache()
    base = rows[0]["verify_ms"]
    for r in rows:
        r["verify_vs_first"] = round(r["verify_ms"] / base, 3)
    return {"metric": "batched verify: pass time and accepted tokens/s vs sequences B",
            "unit": "ms / tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "dtype": "bf16", "data": "synthetic",
            "peak_hbm_GB_s": PEAK_HBM_GBS, "peak_bf16_dense_TFLOP_s": PEAK_BF16_TFLOPS,
            "config": {"workload": f"{tcfg.name} target, K = {K}, prompt {plen} per sequence, "
                                   f"prompt-lookup drafts (n <= {args.ngram_n}), "
                                   f"{'greedy' if args.greedy else 'sampling at T = 1'}"},
            "sweep": rows}


def adaptive_k_run(sd, torch, ctx, stream, d, D, out, nacc, seed, args, tcfg, dcfg, plen):
    """Rounds with K chosen every 8 rounds: the acceptance rate is estimated
    from the tokens the last window committed (spec_alpha_from_tokens, the
    inverse of [en] Floor 6's mean), smoothed, and K is the value that
    maximises tokens per unit time under the measured draft-step and verify
    times (spec_choose_k)."""
    import numpy as np
    k_max = sd.SPEC_K_MAX

    def rnd(K, ev=None):
        if ev is not None:
            ev[0].record(stream)
        sd.spec_draft(ctx, K, seed, d, D)
        if ev is not None:
            ev[1].record(stream)
        sd.spec_verify(ctx, K, seed, d, D, out, nacc)
        if ev is not None:
            ev[2].record(stream)
        sd.spec_commit(ctx, out, nacc)

    for K in range(1, k_max + 1):  # capture every K's graphs before timing
        rnd(K)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(5)]
    for e in evs:
        rnd(4, e)
    sd.spec_sync(ctx)
    t_draft = float(np.median([e[0].elapsed_time(e[1]) for e in evs])) / 4
    t_verify = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    W, K, alpha = 8, 4, None
    traj = []
    st0 = sd.spec_get_state(ctx)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    last = st0["target_len"]
    for w in range(max(1, args.steps // W)):
        for _ in range(W):
            rnd(K)
        st = sd.spec_get_state(ctx)
        a = sd.spec_alpha_from_tokens((st["target_len"] - last) / W, K)
        last = st["target_len"]
        alpha = a if alpha is None else 0.5 * alpha + 0.5 * a
        traj.append(K)
        K = sd.spec_choose_k(alpha, t_draft, t_verify, k_max)
    t1.record(stream)
    sd.spec_sync(ctx)
    st1 = sd.spec_get_state(ctx)
    assert st1["device_error"] == 0, st1
    ms = t0.elapsed_time(t1)
    tokens = st1["target_len"] - st0["target_len"]
    rounds = W * len(traj)
    return {
        "metric": "accepted tokens/s at batch 1, K=4; verify-pass HBM GB/s as % of MI355X peak",
        "value": round(tokens / (ms / 1e3), 2), "unit": "tokens/s", "n_gpus": 1, "steps": rounds,
        "warmup": k_max + 5, "ms_per_step": round(ms / rounds, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{tcfg.name} target + {dcfg.name} draft, batch 1, K chosen every "
                               f"{W} rounds from the measured acceptance, prompt {plen}, "
                               f"{'greedy' if args.greedy else 'temperature-1 sampling'}, "
                               f"random-init bf16", "K": "adaptive", "batch": 1,
                   "prompt_len": plen},
        "adaptive_k": {"t_draft_step_ms": round(t_draft, 4), "t_verify_ms": round(t_verify, 4),
                       "alpha_estimate": round(alpha, 4), "k_per_window": traj,
                       "tokens_per_round": round(tokens / rounds, 4)},
        "roofline": None, "cpu_baseline": None,
    }


def cpu_baseline(tcfg, dcfg, tw, dw, K, args, gpu_tokens_per_round, plen):
    """The oracle (plain C, fp64 forward over the bf16 weights widened exactly,
    fp32 probability rows, OpenMP over output features) on the host cores,
    on bounded samples of the same workload:
      * speculative rounds of the same pair with an 8-token prompt (prefill
        untimed), scaled to tokens/s by the GPU run's tokens per round;
        attention over 8 instead of ~1000 keys is ~4% of the oracle's per-row
        work, so this bounds the sample without changing what a round
        computes;
      * one (K+1)-row verify pass of the target at the GPU run's context
        length (the prompt's length minus the pending token): the oracle's
        cache starts zero-filled, so the positions before the pass hold zero
        keys and values -- the same attention arithmetic as a prefilled
        cache, without an fp64 prefill of ~1000 tokens -- with GB/s on the
        same algorithmic-bytes model as the GPU's verify pass;
      * the rule alone on one 64 x 8 x 32000 batch (draft noise 0.5), GB/s on
        the same model as the GPU's --ar-bench."""
    import numpy as np
    import oracle
    import synth
    t0 = time.time()
    tb = synth.torch_to_bits(tw)
    db = synth.torch_to_bits(dw)
    log(f"host copies of the weights in {time.time() - t0:.1f}s")
    T = oracle.Model(tcfg, tb)
    Dm = oracle.Model(dcfg, db)
    prompt = synth.prompt(tcfg.vocab, 8, seed=7)
    # untimed prefill, then timed rounds: run spec_generate twice (n rounds
    # and 0 rounds) and subtract, so the prefill is excluded.
    t0 = time.perf_counter()
    oracle.spec_generate(T, Dm, prompt, 0, K, greedy=args.greedy, seed=synth.SEED_PHILOX)
    t_pre = time.perf_counter() - t0
    t0 = time.perf_counter()
    out, nacc, st = _rounds(oracle, T, Dm, prompt, K, args)
    t_all = time.perf_counter() - t0
    t_rounds = max(t_all - t_pre, 1e-9)
    rounds = st["rounds"]
    val = rounds * gpu_tokens_per_round / t_rounds
    # one verify pass: K+1 rows at the GPU run's context length, logits and rows
    n_ctx = max(plen - 1, 0)
    kv = oracle.KV(T, n_ctx + K + 2)
    rows = [int(x) for x in synth.prompt(tcfg.vocab, K + 1, seed=8)]
    t0 = time.perf_counter()
    lg = oracle.forward(T, kv, rows, n_ctx)
    _ = [oracle.softmax_f32(r) for r in lg]
    t_verify = time.perf_counter() - t0
    del kv
    vbytes = verify_pass_bytes(tcfg, K, n_ctx)
    # the rule alone on the isolated-rule workload
    Bq, Kq, Vq = 64, 8, 32000
    Tq, Dq = synth.logit_pair(Bq, Kq, Vq, 0.5)
    dq = synth.drafts_from_rows(Dq)
    pos = np.arange(Bq, dtype=np.uint64) * 37 + 100
    t0 = time.perf_counter()
    _, nq = oracle.accept_reject_batch(Tq, Dq, dq, synth.SEED_PHILOX, pos, 0, False)
    t_ar = time.perf_counter() - t0
    ar_bytes = ar_call_bytes(nq, Kq, Vq)
    return {"value": round(val, 4), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "precision": "fp64 forward (bf16 weights widened exactly), fp32 probability rows",
            "sample": f"{rounds} speculative rounds (K={K} draft steps + {K + 1}-row verify + "
                      f"accept/reject) of the same pair with an 8-token prompt, prefill excluded "
                      f"({t_pre:.1f}s); tokens/round taken from the GPU run "
                      f"({gpu_tokens_per_round:.3f}); oracle's own rounds emitted {st['emitted']}",
            "seconds": round(t_rounds, 3),
            "verify_pass": {"ms": round(t_verify * 1e3, 1), "context_tokens": n_ctx,
                            "algorithmic_GB": round(vbytes / 1e9, 4),
                            "GB_s": round(vbytes / t_verify / 1e9, 3)},
            "accept_reject": {"workload": f"B={Bq}, K={Kq}, V={Vq}, sigma=0.5, sampling",
                              "ms_per_call": round(t_ar * 1e3, 2),
                              "algorithmic_MB": round(ar_bytes / 1e6, 3),
                              "GB_s": round(ar_bytes / t_ar / 1e9, 3)}}


def _rounds(oracle, T, Dm, prompt, K, args):
    # at least one token per round: asking for cpu_tokens tokens bounds the
    # rounds by cpu_tokens; the stats report the rounds actually run.
    import synth
    return oracle.spec_generate(T, Dm, prompt, args.cpu_tokens, K, greedy=args.greedy,
                                seed=synth.SEED_PHILOX)


if __name__ == "__main__":
    main()
