"""Short text summaries of rocprofv3 output for this library's kernels, and the per-launch HBM
traffic that bench.py reports beside its roofline.  Reads only what rocprofv3 wrote; needs no GPU.

  python3 -m chunked_scan_amd.profsum stats <dir> [--title T] [--command C]
      per-kernel calls and mean / min / max duration from a --kernel-trace --stats run
  python3 -m chunked_scan_amd.profsum pmc --fetch <dir> --write <dir> --calib-mib M [--title T]
          [--command C] [--traffic-json F --workload W --kernel K]
      per-kernel mean FETCH_SIZE / WRITE_SIZE per dispatch, scaled to bytes by the same counters on a
      plain device copy of M MiB made in the same run (bench.py --calib-copy-mib M); with
      --traffic-json, the scaled bytes per launch of trace name K are written for bench.py, keyed to
      the forward sources' hash (a file taken on other sources is ignored)

Kernels are named twice: by the name the library's event tracing gives each launch (what bench.py
reports) and by the template instance rocprofv3 saw.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FWD_SRCS = [os.path.join(ROOT, "chunked_scan_amd", "csrc", f) for f in ("chunk_fwd_split.hip", "chunk_fwd_pipe.hip")]
MODES = {"0": "NONE", "1": "HEAD", "2": "GATE"}

# kernel -> (index of its decay-mode argument, index of its state-only flag, trace name or prefix)
_KERNELS = {
    "pipe_fwd_kernel": (0, 1, "chunk_fwd_pipe"),
    "tiled_fwd_kernel": (3, 4, "chunk_fwd_tiled"),
    "small_fwd_kernel": (1, 2, "chunk_fwd_small"),
    "pipe_chain_kernel": (0, None, "chunk_fwd_chain_output_pass"),
    "chain_reset_kernel": (None, None, "chunk_fwd_chain_reset"),
    "state_correct_ws_kernel": (0, None, "state_correct_mfma"),
    "state_correct_small_kernel": (1, None, "state_correct_mfma"),
    "state_scan_vec_kernel": (None, None, "state_scan"),
    "state_scan_kernel": (None, None, "state_scan"),
    "state_scan4_kernel": (None, None, "state_scan"),
    "bwd_dq_kernel": (1, 2, "chunk_bwd_dq"),
    "bwd_dkdv_kernel": (1, 2, "chunk_bwd_dkdv"),
    "bwd_dkdv_head_kernel": (None, None, "chunk_bwd_dkdv"),
    "bwd_dq_gate_kernel": (None, 1, "chunk_bwd_dq"),
    "bwd_dkdv_gate_kernel": (None, 1, "chunk_bwd_dkdv"),
    "bwd_dlam_kernel": (None, 1, "chunk_bwd_dlam"),
    "dg_kernel": (None, None, "chunk_bwd_dg"),
}


def source_hash() -> str:
    """Hash of the forward-kernel sources: counter data taken on other sources is stale."""
    h = hashlib.sha256()
    for p in FWD_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _template_name(mangled):
    """`name<args>(` of a mangled kernel of this library whose template arguments are integers and
    booleans (c++filt leaves names with __bf16 parameters mangled)."""
    m = re.match(r"_ZN2la12_GLOBAL__N_1(\d+)", mangled)
    if not m:
        return mangled
    n = int(m.group(1))
    rest = mangled[m.end():]
    name, rest = rest[:n], rest[n:]
    args = []
    if rest.startswith("I"):
        rest = rest[1:]
        while True:
            a = re.match(r"L([ib])(\d+)E", rest)
            if not a:
                break
            args.append(a.group(2) if a.group(1) == "i" else ("true" if a.group(2) == "1" else "false"))
            rest = rest[a.end():]
    return name + ("<" + ", ".join(args) + ">" if args else "") + "("


def _demangle(names):
    todo = [n for n in names if n.startswith("_Z")]
    out = {n: n for n in names}
    if todo:
        try:
            r = subprocess.run(["c++filt"], input="\n".join(todo), capture_output=True, text=True, check=True)
            out.update(zip(todo, r.stdout.splitlines()))
        except (OSError, subprocess.CalledProcessError):
            pass
    for n in todo:
        if out[n].startswith("_Z"):
            out[n] = _template_name(n)
    return out


def _split_args(s):
    args, depth, cur = [], 0, ""
    for ch in s:
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        if ch == "," and depth == 0:
            args.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        args.append(cur.strip())
    return args


def label(demangled: str):
    """(trace name or None, short template instance) of one kernel name as rocprofv3 prints it."""
    s = demangled
    if s.startswith("void "):
        s = s[5:]
    s = s.replace("(anonymous namespace)::", "")
    m = re.match(r"([\w:]+)(<(.*)>)?\(", s)
    if not m:
        return None, s[:60]
    base = m.group(1).split("::")[-1]
    args = _split_args(m.group(3)) if m.group(3) else []
    if base not in _KERNELS:
        return None, base
    mi, si, name = _KERNELS[base]
    shown = list(args)
    if mi is not None and mi < len(shown):
        shown[mi] = MODES.get(shown[mi], shown[mi])
    so = si is not None and si < len(args) and args[si] in ("true", "1")
    if si is not None and si < len(shown):
        shown[si] = "state pass" if so else "outputs"
    if base == "pipe_fwd_kernel" and len(args) > 2:
        # the forward kernel on transposed states computes dq of the backward
        dq = args[2] in ("true", "1")
        inst = base + "<" + ", ".join(shown[:2] + (["dq"] if dq else [])) + ">"
        if dq:
            return "chunk_bwd_dq" + ("_state_pass" if so else ""), inst
        return name + ("_state_pass" if so else "_output_pass"), inst
    if base in ("bwd_dq_kernel", "bwd_dkdv_kernel") and len(args) > 3:
        # WIN: the gate's windowed redo; FACT (dk/dv, head decay): the factorised walk
        extra = ["windows"] if args[3] in ("true", "1") else []
        if len(args) > 4 and args[4] in ("true", "1"):
            extra.append("factorised")
        shown = shown[:3] + extra
    if si is not None:
        if name.startswith("chunk_bwd"):
            name += "_state_pass" if so else ""
            if base in ("bwd_dq_kernel", "bwd_dkdv_kernel") and len(args) > 3 and args[3] in ("true", "1"):
                name += "_windows"
        else:
            name += "_state_pass" if so else "_output_pass"
    return name, base + ("<" + ", ".join(shown) + ">" if shown else "")


def _one_csv(d, suffix):
    fs = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not fs:
        raise SystemExit(f"no *{suffix} under {d}")
    return fs[0]


def stats_rows(d):
    """Per kernel: calls, mean, min, max (us), from the --stats summary of a kernel-trace run."""
    rows = list(csv.DictReader(open(_one_csv(d, "kernel_stats.csv"))))
    names = _demangle([r["Name"] for r in rows])
    out = []
    for r in rows:
        name, inst = label(names[r["Name"]])
        if name is None:
            continue
        out.append((name, inst, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["MaxNs"]) / 1e3))
    return sorted(out, key=lambda x: -x[2] * x[3])


def pmc_means(d):
    """{rocprofv3 kernel name: [counter value per dispatch]} of a one-counter --pmc run."""
    acc = {}
    for r in csv.DictReader(open(_one_csv(d, "counter_collection.csv"))):
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def _calib(acc, calib_bytes):
    copies = [v for n, vs in acc.items() if "copy" in n.lower() for v in vs]
    if not copies:
        raise SystemExit("no copy dispatch found for the calibration")
    top = max(copies)
    return calib_bytes / (top * 1024.0), top


def _table(header, rows):
    out = ["| " + " | ".join(header) + " |", "|" + "---|" * len(header)]
    out += ["| " + " | ".join(str(c) for c in r) + " |" for r in rows]
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    a1 = sub.add_parser("stats")
    a1.add_argument("dir")
    a2 = sub.add_parser("pmc")
    a2.add_argument("--fetch", required=True)
    a2.add_argument("--write", required=True)
    a2.add_argument("--calib-mib", type=int, required=True)
    a2.add_argument("--traffic-json")
    a2.add_argument("--workload")
    a2.add_argument("--kernel")
    for a in (a1, a2):
        a.add_argument("--title", default="")
        a.add_argument("--command", action="append", default=[],
                       help="the rocprofv3 command that made the data (repeatable)")
        a.add_argument("--note", action="append", default=[], help="a paragraph printed before the table")
    args = ap.parse_args(argv)
    lines = []
    if args.what == "stats":
        lines.append(f"# Kernel durations, rocprofv3 --kernel-trace --stats{': ' + args.title if args.title else ''}")
        lines.append("")
        lines.append("Commands (the profiler from /tmp with TMPDIR=/tmp, $R the repository root; the summary from $R):")
        lines += [f"`{c}`" for c in args.command]
        lines.append("")
        lines.append("Only this library's kernels are listed; calls cover every launch of the run.")
        lines.append("")
        for n in args.note:
            lines += [n, ""]
        rows = [(n, i, c, f"{m:.1f}", f"{lo:.1f}", f"{hi:.1f}") for n, i, c, m, lo, hi in stats_rows(args.dir)]
        lines.append(_table(("trace name", "kernel", "calls", "mean us", "min us", "max us"), rows))
        print("\n".join(lines))
        return
    calib = args.calib_mib * (1 << 20)
    fetch, write = pmc_means(args.fetch), pmc_means(args.write)
    fs, ftop = _calib(fetch, calib)
    ws, wtop = _calib(write, calib)
    names = _demangle(sorted(set(fetch) | set(write)))
    per = {}
    for raw in sorted(set(fetch) | set(write)):
        name, inst = label(names[raw])
        if name is None:
            continue
        f, w = fetch.get(raw, []), write.get(raw, [])
        per[(name, inst)] = (len(f), statistics.mean(f) if f else 0.0, statistics.mean(w) if w else 0.0)
    lines.append(f"# HBM traffic per dispatch, rocprofv3 --pmc{': ' + args.title if args.title else ''}")
    lines.append("")
    lines.append("Commands (one counter per run, the profiler from /tmp with TMPDIR=/tmp, $R the repository root; "
                 "the summary from $R):")
    lines += [f"`{c}`" for c in args.command]
    lines.append("")
    lines.append(f"Calibration: a plain {args.calib_mib} MiB device copy in the same run read FETCH_SIZE = "
                 f"{ftop:.0f} KiB and WRITE_SIZE = {wtop:.0f} KiB, so bytes = FETCH_SIZE x 1024 x {fs:.4f} "
                 f"and WRITE_SIZE x 1024 x {ws:.4f}.  Means over every dispatch of the run.")
    lines.append("")
    for n in args.note:
        lines += [n, ""]
    rows = [(n, i, c, f"{f:.0f}", f"{w:.0f}", f"{f * 1024 * fs / 2**20:.1f}", f"{w * 1024 * ws / 2**20:.1f}")
            for (n, i), (c, f, w) in sorted(per.items(), key=lambda kv: -(kv[1][1] + kv[1][2]))]
    lines.append(_table(("trace name", "kernel", "dispatches", "FETCH_SIZE KiB", "WRITE_SIZE KiB",
                         "read MiB (scaled)", "written MiB (scaled)"), rows))
    print("\n".join(lines))
    if args.traffic_json:
        hits = [(n, i, v) for (n, i), v in per.items() if n == args.kernel]
        if len(hits) != 1:
            raise SystemExit(f"--kernel {args.kernel}: {len(hits)} kernel instances match")
        _, inst, (_, f, w) = hits[0]
        with open(args.traffic_json, "w") as fh:
            json.dump(dict(workload=args.workload, kernel=args.kernel, instance=inst,
                           source_sha256_16=source_hash(), fetch_kib=f, write_kib=w, fetch_scale=fs,
                           write_scale=ws, bytes_per_launch=int(round(f * 1024 * fs + w * 1024 * ws))), fh, indent=1)
        print(f"wrote {args.traffic_json}", file=sys.stderr)


if __name__ == "__main__":
    main()
