"""Summaries of rocprofv3 CSV output for the library's kernels.

    python -m rl_policy_gradient_amd.profsum copy --mib 1024 --reps 4
        a plain streaming kernel of known size (torch's elementwise negation:
        reads and writes each byte once), to run under
        ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE``: the counters'
        reading for it gives the factor from counter KiB to bytes moved.
    python -m rl_policy_gradient_amd.profsum stats TRACE_CSV --command "..."
        per-kernel count / average / min / max duration from a
        ``--kernel-trace`` CSV (text table).
    python -m rl_policy_gradient_amd.profsum traffic --fetch CSV --write CSV
            --copy-fetch CSV --copy-write CSV --copy-bytes B --kernel NAME
            --match SUBSTR --workload W --out JSON --command "..."
        HBM bytes per launch of one kernel: FETCH_SIZE and WRITE_SIZE (KiB per
        dispatch) averaged over its dispatches, each scaled by the factor the
        same counter shows on the plain copy.
    python -m rl_policy_gradient_amd.profsum hbm TRACE_CSV --rows N --active NA --H H --V V --splits S
            --chunks C [--entropy] --workload W [--fetch CSV --write CSV --copy-fetch CSV
            --copy-write CSV] --out TXT --command "..."
        the memory-bound kernels' algorithmic bytes per launch over their
        average duration (GB/s and fraction of 8 TB/s), with the counters'
        traffic beside them when the --pmc CSVs are given.
    python -m rl_policy_gradient_amd.profsum pmc PMC_CSV --match A,B --command "..."
        per-dispatch averages of every counter in a ``--pmc`` CSV for the
        kernels whose names contain A, B, ..., with the matrix-core and LDS
        utilisation derived from them (formulas in the output).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ("fwd_sweep.h", "lmhead_fwd.hip", "lmhead_fwd_o.hip", "lmhead_mfma.hip", "mfma_tile.h", "loss_stage.hip", "plp_api.cpp", "common.h")


def kernel_src_hash() -> str:
    """Hash of the sources and build options that define the sweeps' code and
    launch shapes; a traffic summary taken on other ones is stale."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rl_policy_gradient_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "rl_policy_gradient_amd", "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def _demangle(names):
    """Demangled kernel names (c++filt when present, else unchanged)."""
    import shutil
    import subprocess

    import re

    names = [n.strip('"') for n in names]
    if shutil.which("c++filt"):
        out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True).stdout.split("\n")
        if len(out) >= len(names):
            names = out[: len(names)]
    # names c++filt leaves mangled (bf16 parameters): namespace, name and the
    # integer / bool template arguments
    pretty = []
    for n in names:
        m = re.match(r"_ZN3plp12_GLOBAL__N_1(\d+)", n)
        if not m:
            pretty.append(n)
            continue
        k = int(m.group(1))
        base = n[m.end(): m.end() + k]
        rest = n[m.end() + k:]
        targs = []
        if rest.startswith("I"):
            for t, v in re.findall(r"L(i|b)(\d+)E", rest.split("EEv")[0]):
                targs.append(v if t == "i" else ("true" if v == "1" else "false"))
        pretty.append("plp::" + base + (f"<{', '.join(targs)}>" if targs else ""))
    return pretty


def _short(name: str, width: int = 90) -> str:
    name = name.strip('"')
    if name.startswith("void "):
        name = name[5:]
    return name if len(name) <= width else name[: width - 3] + "..."


def _rows(path):
    with open(path, newline="") as fh:
        yield from csv.DictReader(fh)


def kernel_durations(trace_csv: str, split_passes: bool = False) -> dict:
    """{kernel name: [duration ns, ...]} from a rocprofv3 kernel-trace CSV;
    with split_passes the two-role forward sweep's second pass over flagged
    rows and its pass over the compacted rows are keyed apart, as
    (name, label) (pass_label)."""
    seq = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), r["Kernel_Name"])
                  for r in _rows(trace_csv)), key=lambda x: x[0])
    out, prev = {}, ""
    for _, d, n in seq:
        key = n
        if "plp" in n:
            label = pass_label(n, prev) if split_passes else "main"
            key = n if label == "main" else (n, label)
            prev = n
        out.setdefault(key, []).append(d)
    return out


def pass_label(name: str, prev: str) -> str:
    """Which pass a launch of the two-role forward sweep is, from the library
    kernel launched before it: after the flag scan it is the second pass over
    the flagged rows, after the compaction the accumulator pass over the
    compacted rows with a gradient; any other launch is labelled "main"."""
    if "fwd_pp_kernel" in name:
        if "flag_scan_kernel" in prev:
            return "flagged"
        if "compact_scatter_kernel" in prev:
            return "compacted"
    return "main"


def _dispatch_labels(pmc_csv: str) -> dict:
    """{dispatch id: pass label} over the library's dispatches of a --pmc CSV."""
    names = {}
    for r in _rows(pmc_csv):
        names[int(r["Dispatch_Id"])] = r["Kernel_Name"]
    labels, prev = {}, ""
    for k in sorted(names):
        n = names[k]
        if "plp" not in n:
            continue
        labels[k] = pass_label(n, prev)
        prev = n
    return labels


def counter_per_dispatch(pmc_csv: str, counter: str, match: str, which: str = "main") -> list:
    """Values of `counter` for every dispatch whose kernel name contains
    `match` and whose pass label (pass_label) is `which` ("any": all)."""
    labels = _dispatch_labels(pmc_csv) if which != "any" else {}
    vals = {}
    for r in _rows(pmc_csv):
        if r["Counter_Name"] != counter or match not in r["Kernel_Name"]:
            continue
        key = int(r["Dispatch_Id"])
        if which != "any" and labels.get(key, "main") != which:
            continue
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals)]


def cmd_copy(args) -> int:
    import torch

    n = args.mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"streamed {n} bytes in and out x {args.reps}", flush=True)
    return 0


def cmd_pmc(args) -> int:
    per = {}  # match -> dispatch id -> counter -> value (summed over the CSV's rows)
    labels = _dispatch_labels(args.csv)
    for r in _rows(args.csv):
        for m in args.match.split(","):
            # a name:label entry takes that pass of the kernel only (pass_label)
            kname, _, want = m.partition(":")
            if kname in r["Kernel_Name"] and labels.get(int(r["Dispatch_Id"]), "main") == (want or "main"):
                d = per.setdefault(m, {}).setdefault(r["Dispatch_Id"], {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = ["# rocprofv3 counter summary (per-dispatch averages)", f"# command: {args.command}",
             f"# wall cycles = GRBM_GUI_ACTIVE / {args.xcds} (the counter is summed over the XCDs);",
             f"# MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (wall x {args.cus} CUs x {args.simds} SIMDs);",
             f"# LDS busy = SQ_LDS_IDX_ACTIVE / (wall x {args.cus} CUs); "
             "bank-conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE", ""]
    for m, disp in per.items():
        names = sorted({k for d in disp.values() for k in d})
        avg = {k: statistics.mean(d.get(k, 0.0) for d in disp.values()) for k in names}
        lines.append(f"{m}: {len(disp)} dispatches")
        for k in names:
            lines.append(f"   {k:<28} {avg[k]:>14.4g}")
        wall = avg.get("GRBM_GUI_ACTIVE", 0.0) / args.xcds
        if wall > 0 and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            lines.append(f"   MFMA busy                    {100.0 * avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (wall * args.cus * args.simds):>13.1f} %")
        if wall > 0 and "SQ_LDS_IDX_ACTIVE" in avg:
            lines.append(f"   LDS busy                     {100.0 * avg['SQ_LDS_IDX_ACTIVE'] / (wall * args.cus):>13.1f} %")
            if "SQ_LDS_BANK_CONFLICT" in avg and avg["SQ_LDS_IDX_ACTIVE"] > 0:
                lines.append(f"   LDS bank-conflict share      "
                             f"{100.0 * avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:>13.1f} %")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)
    return 0


_PASS_NAMES = {"flagged": "[second pass, flagged rows]", "compacted": "[compacted rows with a gradient]"}


def cmd_stats(args) -> int:
    d = kernel_durations(args.trace, split_passes=True)
    total = sum(sum(v) for v in d.values())
    lines = [f"# rocprofv3 kernel trace summary", f"# command: {args.command}",
             "# the two-role forward sweep's launches after the flag scan (second pass over flagged rows) and",
             "# after the compaction (rows with a gradient, entropy mask on) are listed on rows of their own", "",
             f"{'kernel':<92} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10} {'pct':>6}"]
    items = sorted(d.items(), key=lambda kv: -sum(kv[1]))
    raw = [k if isinstance(k, str) else k[0] for k, _ in items]
    for name, (key, v) in zip(_demangle(raw), items):
        if not isinstance(key, str):
            name = f"{_short(name, 60)} {_PASS_NAMES[key[1]]}"
        lines.append(f"{_short(name):<92} {len(v):>6} {statistics.mean(v) / 1e3:>10.2f} {min(v) / 1e3:>10.2f} "
                     f"{max(v) / 1e3:>10.2f} {sum(v) / 1e6:>10.3f} {100.0 * sum(v) / total:>6.2f}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)
    return 0


def cmd_traffic(args) -> int:
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE", args.match, args.which)
    write = counter_per_dispatch(args.write, "WRITE_SIZE", args.match, args.which)
    cf = counter_per_dispatch(args.copy_fetch, "FETCH_SIZE", args.copy_match, "any")
    cw = counter_per_dispatch(args.copy_write, "WRITE_SIZE", args.copy_match, "any")
    if not (fetch and write and cf and cw):
        print("missing dispatches: fetch %d write %d copy %d/%d" % (len(fetch), len(write), len(cf), len(cw)))
        return 1
    # the largest copy dispatches are the timed copies (fills and warm-up aside)
    f_factor = args.copy_bytes / (1024.0 * max(cf))
    w_factor = args.copy_bytes / (1024.0 * max(cw))
    fb = statistics.mean(fetch) * 1024.0 * f_factor
    wb = statistics.mean(write) * 1024.0 * w_factor
    d = {
        "kernel": args.kernel,
        "match": args.match,
        "pass": args.which,
        "workload": args.workload,
        "dispatches": [len(fetch), len(write)],
        "fetch_kib_per_dispatch": statistics.mean(fetch),
        "write_kib_per_dispatch": statistics.mean(write),
        "copy_bytes": args.copy_bytes,
        "copy_fetch_kib": max(cf),
        "copy_write_kib": max(cw),
        "fetch_factor": f_factor,
        "write_factor": w_factor,
        "fetch_bytes_per_launch": fb,
        "write_bytes_per_launch": wb,
        "bytes_per_launch": fb + wb,
        "kernel_src_hash": kernel_src_hash(),
        "command": args.command,
    }
    with open(args.out, "w") as fh:
        json.dump(d, fh, indent=1)
        fh.write("\n")
    print(json.dumps(d))
    return 0


def small_kernel_bytes(wl: dict) -> dict:
    """Algorithmic HBM bytes per launch of the memory-bound kernels of one
    fused call (bf16 hidden states and weights, fp32 per-token arrays), for
    a workload of `chunks` outer chunks of n rows, na of them with a
    gradient, H, V, Sv vocabulary splits of the forward sweep, an optional
    bias and q < 1 (statistics-only forward, then the grad_h accumulator
    over the na rows). Each value reads and writes every byte the kernel
    must move once; the bf16 element is 2 bytes, fp32 4."""
    n, na, H, V, Sv = wl["n"], wl["na"], wl["H"], wl["V"], wl["Sv"]
    q = wl["entropy"]
    nblk = -(-V // 64)
    rem = nblk % 256
    parts = min(4, 256 // rem) if rem else 1
    out = {
        # split statistics, the accumulator splits and v (with grad_h in the
        # forward), the row of h and the target row of W for the target logit;
        # lp, entropy and lse out
        "combine_kernel": Sv * n * 32 + Sv * n * H * 4 + n * H * 4 + 2 * n * H * 2 + 12 * n,
        "combine_kernel (statistics only)": Sv * n * 32 + 2 * n * H * 2 + 12 * n,
        # per-token inputs, g out; grad_h = g / tau v in bf16 (zeros when the
        # accumulator pass runs over the compacted rows)
        "token_kernel": 18 * n + (n * H * 2 if q else n * H * 4 + n * H * 2),
        "compact_scatter_kernel": 16 * n + 20 * na,
        # the fragment-major copy of W (once per call; rows padded to 64) and
        # of the gathered rows with a gradient (once per chunk)
        "frag_copy_kernel (W)": 2 * (-(-V // 64) * 64) * H * 2,
        "frag_copy_kernel (gathered rows)": 2 * na * H * 2,
        # parts fp32 partial sums of the shared tail blocks in, grad_W rows out
        "tail_reduce_kernel": rem * 64 * H * 4 * parts + rem * 64 * H * 2 if parts > 1 else 0,
        "select_hist_kernel": 5 * wl["N"],
        "mask_kernel": 6 * wl["N"],
        "grad_h_compact_kernel": na * (H * 4 + H * 2 + H * 2 + 32),
        "gather_rows_kernel": 2 * na * H * 2,
    }
    return out


def cmd_hbm(args) -> int:
    wl = {"n": args.rows, "na": args.active, "H": args.H, "V": args.V, "Sv": args.splits, "entropy": args.entropy,
          "chunks": args.chunks, "N": args.rows * args.chunks}
    alg = small_kernel_bytes(wl)
    d = kernel_durations(args.trace)
    names = dict(zip(d.keys(), _demangle(list(d.keys()))))
    traffic = {}
    if args.fetch and args.write and args.copy_fetch and args.copy_write:
        cf = counter_per_dispatch(args.copy_fetch, "FETCH_SIZE", "neg")
        cw = counter_per_dispatch(args.copy_write, "WRITE_SIZE", "neg")
        ff = args.copy_bytes / (1024.0 * max(cf))
        wf = args.copy_bytes / (1024.0 * max(cw))
        for k in {k.split(" ")[0] for k in alg}:
            f = counter_per_dispatch(args.fetch, "FETCH_SIZE", k)
            w = counter_per_dispatch(args.write, "WRITE_SIZE", k)
            if f and w:
                traffic[k] = statistics.mean(f) * 1024.0 * ff + statistics.mean(w) * 1024.0 * wf
    lines = ["# HBM-bound kernels: algorithmic bytes per launch / median duration (kernel trace), against 8 TB/s",
             f"# workload: {args.workload}; {args.chunks} chunk(s) of {args.rows} rows, {args.active} with a "
             f"gradient per chunk, H={args.H} V={args.V}, {args.splits} vocabulary split(s)"
             + ("; q < 1 (accumulator over the compacted rows)" if args.entropy else ""),
             f"# command: {args.command}",
             "# traffic: FETCH_SIZE + WRITE_SIZE per dispatch scaled by a plain copy's reading (when given)", "",
             f"{'kernel':<40} {'calls':>6} {'med_us':>10} {'alg_MB':>10} {'GB/s':>9} {'frac':>6} {'traffic_MB':>11}"]
    # Launches of one kernel name that move different amounts are told apart
    # by the library kernels around them in time: the copy of W precedes a
    # forward sweep and the gathered rows' copy the weight-gradient sweep;
    # the merge after the statistics-only sweep (and its second pass over
    # flagged rows) has no accumulator (with q = 1 that sweep is the setup's
    # log-prob pass, not part of a step).
    seq = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                   r["Kernel_Name"]) for r in _rows(args.trace)), key=lambda x: x[0])
    plp_seq = [x for x in seq if "plp" in x[2]]
    split = {}
    sweep = ""  # the last forward sweep over all rows (not a second pass over flagged rows)
    for i, (_, dur, name) in enumerate(plp_seq):
        nxt = plp_seq[i + 1][2] if i + 1 < len(plp_seq) else ""
        prv = plp_seq[i - 1][2] if i > 0 else ""
        if ("fwd_mfma_kernel" in name or "fwd_pp_kernel" in name) and pass_label(name, prv) == "main":
            sweep = name
        if "frag_copy_kernel" in name:
            label = "frag_copy_kernel (gathered rows)" if "bwd_pp_kernel" in nxt else "frag_copy_kernel (W)"
        elif "combine_kernel" in name:
            if "fwd_mfma_kernel" in sweep:
                if not args.entropy:
                    continue
                label = "combine_kernel (statistics only)"
            else:
                label = "combine_kernel"
        else:
            continue
        split.setdefault(label, []).append(dur)
    rows = [(k, k, v) for k, v in split.items()]
    for raw, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        if "frag_copy_kernel" in raw or "combine_kernel" in raw:
            continue
        key = next((k for k in alg if k in raw or k in names[raw]), None)
        if key is not None:
            rows.append((key, _short(names[raw], 40), v))
    for key, label, v in rows:
        if not v or alg.get(key, 0) == 0:
            continue
        us = statistics.median(v) / 1e3  # the median: setup calls of other sizes share some names
        gbs = alg[key] / (us * 1e-6) / 1e9
        tr = traffic.get(key) if " " not in key else None
        lines.append(f"{label:<40} {len(v):>6} {us:>10.2f} {alg[key] / 1e6:>10.2f} {gbs:>9.1f} {gbs / 8000.0:>6.3f} "
                     f"{(tr / 1e6) if tr else float('nan'):>11.2f}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=4)
    s = sub.add_parser("stats")
    s.add_argument("trace")
    s.add_argument("--out")
    s.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write", "kernel", "match", "workload", "out"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--copy-match", default="neg")
    t.add_argument("--which", default="main", choices=["main", "flagged", "compacted", "any"],
                   help="pass of the two-role forward sweep to take (pass_label)")
    t.add_argument("--command", default="")
    q = sub.add_parser("pmc")
    q.add_argument("csv")
    q.add_argument("--match", required=True)
    q.add_argument("--cus", type=int, default=256)
    q.add_argument("--xcds", type=int, default=8)
    q.add_argument("--simds", type=int, default=4)
    q.add_argument("--out")
    q.add_argument("--command", default="")
    b = sub.add_parser("hbm")
    b.add_argument("trace")
    for k in ("rows", "active", "H", "V", "splits", "chunks"):
        b.add_argument("--" + k, type=int, required=True)
    b.add_argument("--entropy", action="store_true")
    b.add_argument("--workload", required=True)
    for k in ("fetch", "write", "copy_fetch", "copy_write", "out"):
        b.add_argument("--" + k.replace("_", "-"))
    b.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    b.add_argument("--command", default="")
    args = ap.parse_args(argv)
    return {"copy": cmd_copy, "stats": cmd_stats, "traffic": cmd_traffic, "pmc": cmd_pmc, "hbm": cmd_hbm}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
