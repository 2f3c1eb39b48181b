"""Summaries of rocprofv3 output for the speculative-decoding path.

Reads what `rocprofv3 --kernel-trace --stats` or `rocprofv3 --pmc ...` wrote
(CSV files, or the SQLite database of the default output format) and prints
short text summaries:

  trace DIR [--rounds R] [--skip-last S] [--kernel SUBSTR] [--kernel-window N]
      per-kernel totals over the whole run; then the steady state: the
      dispatches that follow the first commit kernel (i.e. the decoding rounds,
      without weight generation, packing or prefill), per kernel and per round
      (span, busy time, gaps between kernels over R rounds that end S rounds
      before the last one, e.g. to leave out steps that follow the timed
      rounds); with --kernel, the matching launches' average over the steady
      state and over the N rounds that end S rounds before the last, by kernel
      name and by grid size.
  pmc FETCH_DIR WRITE_DIR --kernel SUBSTR --copy-kernel SUBSTR --copy-bytes N
      HBM traffic per launch of one kernel in the steady state from the
      FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch), each scaled by the
      factor that makes the same counter read the known size of a plain copy
      kernel (N bytes read and N bytes written per launch).

  counters DIR [DIR ...] [--kernels "SUB1;SUB2;..."] [--cus N] [--ses N]
      L1 / address-unit / SQ counters of several `rocprofv3 --pmc` passes,
      averaged per launch for every kernel instance (or those matching the
      substrings) over the steady state, with the derived shares: kernel
      cycles (SQ_CYCLES over the shader engines), mean L2 read latency
      (TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ), and per-CU busy or stall
      cycles (TCP_*, TA_* over the CUs) as a share of the kernel's cycles.

Usage:  python -m speculative_decoding_02_amd.profsum trace prof/kt
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import sqlite3
import sys

ROUND_MARK = "commit_kernel"


def _find(d: str, pattern: str):
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    return hits[0] if hits else None


def _col(header, *names):
    low = [h.strip().lower() for h in header]
    for n in names:
        if n in low:
            return low.index(n)
    raise KeyError(f"none of {names} in {header}")


def load_dispatches(d: str):
    """[(dispatch_id, name, start_ns, end_ns, grid_x)] in dispatch order."""
    f = _find(d, "*kernel_trace.csv")
    if f:
        with open(f, newline="") as fh:
            rd = csv.reader(fh)
            hdr = next(rd)
            ci = _col(hdr, "dispatch_id")
            cn = _col(hdr, "kernel_name")
            cs = _col(hdr, "start_timestamp")
            ce = _col(hdr, "end_timestamp")
            try:
                cg = _col(hdr, "grid_size_x", "grid_x")
            except KeyError:
                cg = None
            rows = [(int(r[ci]), r[cn], int(r[cs]), int(r[ce]), int(r[cg]) if cg is not None else 0)
                    for r in rd]
    else:
        db = _find(d, "*.db")
        if not db:
            raise FileNotFoundError(f"no kernel_trace.csv or .db under {d}")
        con = sqlite3.connect(db)
        rows = con.execute("select dispatch_id, name, start, end, grid_x from kernels").fetchall()
    rows.sort(key=lambda r: r[2])
    return rows


def load_counters(d: str):
    """{dispatch_id: (name, {counter: value})} from counter_collection.csv."""
    f = _find(d, "*counter_collection.csv")
    if not f:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    out: dict = {}
    with open(f, newline="") as fh:
        rd = csv.reader(fh)
        hdr = next(rd)
        ci = _col(hdr, "dispatch_id")
        cn = _col(hdr, "kernel_name")
        cc = _col(hdr, "counter_name")
        cv = _col(hdr, "counter_value")
        for r in rd:
            k = int(r[ci])
            name, vals = out.setdefault(k, (r[cn], {}))
            vals[r[cc]] = vals.get(r[cc], 0.0) + float(r[cv])
    return out


def short(name: str, n: int = 70) -> str:
    name = name.replace("(anonymous namespace)", "")
    return name if len(name) <= n else name[: n - 3] + "..."


def _by_name_and_grid(sel, kernel: str, lines: list) -> None:
    by_name = collections.defaultdict(list)
    by_grid = collections.defaultdict(list)
    for _, n, s, e, g in sel:
        if kernel in n:
            by_name[n].append((e - s) / 1e3)
            by_grid[g].append((e - s) / 1e3)
    for n, v in sorted(by_name.items()):
        lines.append(f"  {short(n)}: {len(v)} launches, avg {sum(v) / len(v):.2f} us")
    for g, v in sorted(by_grid.items()):
        lines.append(f"  grid_x {g}: {len(v)} launches, avg {sum(v) / len(v):.2f} us")


def trace_summary(d: str, rounds: int, kernel: str | None, skip_last: int = 0,
                  kernel_window: int = 0, by_parity: bool = False) -> str:
    rows = load_dispatches(d)
    lines = []
    tot = collections.defaultdict(lambda: [0, 0.0])
    for _, n, s, e, _ in rows:
        tot[n][0] += 1
        tot[n][1] += (e - s) / 1e3
    lines.append(f"whole run: {len(rows)} dispatches")
    lines.append(f"  {'calls':>7} {'total us':>12} {'avg us':>9}  kernel")
    for n, (c, t) in sorted(tot.items(), key=lambda x: -x[1][1])[:16]:
        lines.append(f"  {c:7d} {t:12.1f} {t / c:9.2f}  {short(n)}")
    marks = [i for i, r in enumerate(rows) if ROUND_MARK in r[1]]
    if not marks:
        lines.append("no decoding rounds found (no commit kernel)")
        return "\n".join(lines)
    steady = rows[marks[0] + 1: marks[-1] + 1]
    agg = collections.defaultdict(lambda: [0, 0.0])
    for _, n, s, e, _ in steady:
        agg[n][0] += 1
        agg[n][1] += (e - s) / 1e3
    lines.append("")
    lines.append(f"steady state (dispatches after the first commit kernel): {len(steady)} dispatches, "
                 f"{len(marks) - 1} rounds")
    lines.append(f"  {'calls':>7} {'total us':>12} {'avg us':>9}  kernel")
    for n, (c, t) in sorted(agg.items(), key=lambda x: -x[1][1])[:16]:
        lines.append(f"  {c:7d} {t:12.1f} {t / c:9.2f}  {short(n)}")
    end = len(marks) - 1 - skip_last
    R = min(rounds, end)
    if R > 0:
        sel = rows[marks[end - R] + 1: marks[end] + 1]
        span = (sel[-1][3] - sel[0][2]) / 1e3
        busy = sum((e - s) / 1e3 for _, _, s, e, _ in sel)
        lines.append("")
        lines.append(f"{R} rounds ending {skip_last} before the last: span {span / R:.1f} us/round, "
                     f"kernel busy {busy / R:.1f} us/round, gaps {(span - busy) / R:.1f} us/round, "
                     f"{len(sel) / R:.0f} kernels/round")
    if kernel:
        ks = [(e - s) / 1e3 for _, n, s, e, _ in steady if kernel in n]
        if ks:
            lines.append("")
            lines.append(f"kernel '{kernel}' in the steady state: {len(ks)} launches, "
                         f"avg {sum(ks) / len(ks):.2f} us")
            _by_name_and_grid(steady, kernel, lines)
        W = min(kernel_window, end)
        if W > 0:
            win = rows[marks[end - W] + 1: marks[end] + 1]
            kw = [(e - s) / 1e3 for _, n, s, e, _ in win if kernel in n]
            if kw:
                lines.append("")
                lines.append(f"kernel '{kernel}' in the {W} rounds ending {skip_last} before the "
                             f"last: {len(kw)} launches, avg {sum(kw) / len(kw):.2f} us")
                _by_name_and_grid(win, kernel, lines)
                if by_parity:
                    # launches of one kernel that alternate within a round (e.g. the O and
                    # down projections of each layer): even and odd occurrences apart
                    par = ([], [])
                    for r in range(end - W, end):
                        k = 0
                        for _, n, s_, e, _ in rows[marks[r] + 1: marks[r + 1] + 1]:
                            if kernel in n:
                                par[k % 2].append((e - s_) / 1e3)
                                k += 1
                    for i, v in enumerate(par):
                        if v:
                            lines.append(f"  {'even' if i == 0 else 'odd'} occurrences in a round: "
                                         f"{len(v)} launches, avg {sum(v) / len(v):.2f} us")
    return "\n".join(lines)


def pmc_summary(dfetch: str, dwrite: str, kernel: str, copy_kernel: str, copy_bytes: int) -> str:
    lines = []
    res = {}
    for label, d, cname in (("read", dfetch, "FETCH_SIZE"), ("write", dwrite, "WRITE_SIZE")):
        cnt = load_counters(d)
        ids = sorted(cnt)
        marks = [k for k in ids if ROUND_MARK in cnt[k][0]]
        copies = [cnt[k][1].get(cname, 0.0) for k in ids if copy_kernel in cnt[k][0]]
        if not copies:
            raise RuntimeError(f"no '{copy_kernel}' dispatches in {d}")
        copy_kib = sum(copies) / len(copies)
        factor = (copy_bytes / 1024.0) / copy_kib
        first = marks[0] if marks else -1
        vals = [cnt[k][1].get(cname, 0.0) for k in ids if k > first and kernel in cnt[k][0]]
        if not vals:
            raise RuntimeError(f"no '{kernel}' dispatches after the first round mark in {d}")
        kib = sum(vals) / len(vals)
        res[label] = kib * 1024.0 * factor
        lines.append(f"{cname}: copy kernel reads {copy_kib:.1f} KiB per launch for "
                     f"{copy_bytes / 1024.0:.1f} KiB moved -> factor {factor:.4f}; "
                     f"'{kernel}' {len(vals)} steady-state launches, avg {kib:.1f} KiB raw, "
                     f"{res[label] / 1e6:.3f} MB scaled")
    lines.append(f"traffic_bytes_per_launch: {int(res['read'] + res['write'])}")
    return "\n".join(lines)


def counters_summary(dirs, kernels, cus: int, ses: int) -> str:
    """Per kernel instance: counter averages per launch over the steady state
    of each pass, merged across passes, and the derived shares."""
    per = collections.defaultdict(dict)   # kernel -> counter -> mean per launch
    launches = collections.defaultdict(dict)
    for d in dirs:
        cnt = load_counters(d)
        ids = sorted(cnt)
        marks = [k for k in ids if ROUND_MARK in cnt[k][0]]
        first = marks[0] if marks else -1
        acc = collections.defaultdict(lambda: collections.defaultdict(list))
        for k in ids:
            if k <= first:
                continue
            name, vals = cnt[k]
            if kernels and not any(sub in name for sub in kernels):
                continue
            for c, v in vals.items():
                acc[name][c].append(v)
        for name, cs in acc.items():
            for c, v in cs.items():
                per[name][c] = sum(v) / len(v)
                launches[name][c] = len(v)
    lines = []
    for name in sorted(per):
        c = per[name]
        lines.append(short(name, 90))
        cyc = c.get("SQ_CYCLES", 0.0) / ses if "SQ_CYCLES" in c else None
        if cyc:
            lines.append(f"  kernel cycles (SQ_CYCLES / {ses} SE): {cyc / 1e3:.1f} k")
        if "TCP_TCC_READ_REQ" in c and "TCP_TCC_READ_REQ_LATENCY" in c and c["TCP_TCC_READ_REQ"]:
            lines.append(f"  L1->L2 read requests: {c['TCP_TCC_READ_REQ'] / 1e6:.2f} M, mean L2 read "
                         f"latency {c['TCP_TCC_READ_REQ_LATENCY'] / c['TCP_TCC_READ_REQ']:.0f} cycles")
        for cname, label in (("TCP_PENDING_STALL_CYCLES", "L1 stalled on pending misses"),
                             ("TCP_UTCL1_STALL_INFLIGHT_MAX", "L1 TLB stalled at max in flight"),
                             ("TA_TA_BUSY", "address unit busy"),
                             ("TA_ADDR_STALLED_BY_TC_CYCLES", "address unit stalled by the cache"),
                             ("TA_DATA_STALLED_BY_TC_CYCLES", "address unit data stalled by the cache")):
            if cname in c and cyc:
                lines.append(f"  {label}: {100 * c[cname] / cus / cyc:.0f}% of the kernel's cycles")
        if "TCP_UTCL1_TRANSLATION_MISS" in c:
            lines.append(f"  TLB misses / hits: {c['TCP_UTCL1_TRANSLATION_MISS']:.0f} / "
                         f"{c.get('TCP_UTCL1_TRANSLATION_HIT', 0.0) / 1e6:.2f} M")
        if "SQ_WAIT_INST_ANY" in c and "SQ_WAVE_CYCLES" in c and c["SQ_WAVE_CYCLES"]:
            lines.append(f"  wave time in s_waitcnt: {100 * c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.0f}%")
        n = max(launches[name].values())
        lines.append(f"  ({n} launches; raw means: " +
                     ", ".join(f"{k} {v:.4g}" for k, v in sorted(c.items())) + ")")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--rounds", type=int, default=10)
    t.add_argument("--kernel", default=None)
    t.add_argument("--skip-last", type=int, default=0)
    t.add_argument("--kernel-window", type=int, default=0)
    t.add_argument("--by-parity", action="store_true",
                   help="split the kernel's launches in the window by occurrence parity in a round")
    p = sub.add_parser("pmc")
    p.add_argument("fetch_dir")
    p.add_argument("write_dir")
    p.add_argument("--kernel", required=True)
    p.add_argument("--copy-kernel", required=True)
    p.add_argument("--copy-bytes", type=int, required=True)
    q = sub.add_parser("counters")
    q.add_argument("dirs", nargs="+")
    q.add_argument("--kernels", default="")
    q.add_argument("--cus", type=int, default=256)
    q.add_argument("--ses", type=int, default=32)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace_summary(a.dir, a.rounds, a.kernel, a.skip_last, a.kernel_window, a.by_parity))
    elif a.cmd == "counters":
        ks = [k for k in a.kernels.split(";") if k]
        print(counters_summary(a.dirs, ks, a.cus, a.ses))
    else:
        print(pmc_summary(a.fetch_dir, a.write_dir, a.kernel, a.copy_kernel, a.copy_bytes))


if __name__ == "__main__":
    sys.exit(main())
