"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m sparse_communication_distributed_amd.prof_summary \
        --stats <dir>/run_kernel_stats.csv --fetch <dir>/run_counter_collection.csv \
        --write <dir>/run_counter_collection.csv --workload llama1.8b --out profiles/step_pass_llama1.8b

writes <out>.md (kernel table and HBM bytes) and <out>_counters.json (the
step pass's HBM bytes per launch, read by bench.py).  --stats may be given
several times, one file per process: the first gives the kernel table, and
every file's step-pass average is listed, since large allocations land
differently in each process and the step pass's duration follows them.
The HBM counters are scaled by what they read for the 1 GiB calibration
copy that bench.py --calib runs (reads 1 GiB, writes 1 GiB).  The JSON
records a hash of the step pass's sources and of the host code that picks
its variant; bench.py ignores it once they change.
"""

import argparse
import csv
import gzip
import hashlib
import json
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
STEP_KERNEL = "compress_kernel"
CALIB_KERNEL = "__amd_rocclr_copyBuffer"
GIB_KIB = float(1 << 20)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed (the files
    hashed here hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def step_pass_source_hash() -> str:
    """Hash of the step pass's code and of the host code that picks its
    variant (comments and layout ignored)."""
    h = hashlib.sha256()
    for name in ("compress.hip", "scape_internal.h", "api.hip"):
        with open(os.path.join(PKG, "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def short_name(full: str) -> str:
    """A kernel's name with its template arguments but without return type,
    namespaces and parameter list: 'void scape::(anonymous
    namespace)::compress_kernel<true, true, true, false>(scape::Geom, ...)'
    becomes 'compress_kernel<true, true, true, false>'; template argument
    lists longer than 48 characters become '<…>'.  Names that are already
    short pass through."""
    s = full.strip()
    if s.startswith("void "):
        s = s[5:]
    depth, cut = 0, len(s)
    for i, ch in enumerate(s):  # the parameter list opens at the first '(' outside <...>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not s.startswith("(anonymous", i):
            cut = i
            break
    s = s[:cut]
    head = s.split("<", 1)
    base = head[0].split("::")[-1]
    if len(head) == 1:
        return base
    targs = "<" + head[1]
    # long template arguments (library kernels' functors) are elided
    return base + (targs if len(targs) <= 48 else "<…>")


def step_pass_role(name: str):
    """Role of a launch in the step pass, from its template arguments
    compress_kernel<STEP, VEC, SEG, VOUT, MODE>: "worker" for a non-owner
    worker pass (STEP false, MODE 1), "owner" for the owner pass (MODE 2) or
    the single step pass (MODE 0, or its latency form for small layouts,
    MODE 3) that stores no v (STEP true, VOUT false), "owner_v" for those
    that store v; None for anything else (the component compression has
    STEP false, MODE 0)."""
    n = short_name(name)
    if not n.startswith(STEP_KERNEL + "<"):
        return None
    args = [x.strip() for x in n[len(STEP_KERNEL) + 1:-1].split(",")]
    if len(args) != 5:
        return None
    if args[0] == "false" and args[4] == "1":
        return "worker"
    if args[0] == "true" and args[4] in ("0", "2", "3"):  # the single pass, or the owner pass
        return "owner" if args[3] == "false" else "owner_v"
    return None


def step_pass_ms(run):
    """One process's step pass time from its kernel statistics: the owner
    pass's average plus (K - 1) worker-pass averages, K - 1 being the
    worker launches per owner launch (v-storing owner launches count too:
    their steps run the same worker passes)."""
    tot = defaultdict(float)  # role -> total ms over its kernel variants
    calls = defaultdict(int)
    for r in run:
        role = step_pass_role(r["Name"])
        if role:
            tot[role] += float(r["AverageNs"]) / 1e6 * int(r["Calls"])
            calls[role] += int(r["Calls"])
    if not calls["owner"]:
        return None
    owner = tot["owner"] / calls["owner"]
    wav = tot["worker"] / calls["worker"] if calls["worker"] else 0.0
    per = calls["worker"] / (calls["owner"] + calls["owner_v"])
    return owner, wav, per, owner + per * wav


def _open(path):
    """A CSV file, gzip-compressed or not."""
    return gzip.open(path, "rt") if path.endswith(".gz") else open(path)


def calibration_values(vals):
    """The counter values (KiB) of the 1 GiB calibration copies among all
    copy dispatches of a run.  The workload's own copies use the same copy
    kernel: small ones (uploads of host-drawn indices, a mask check's
    read-back) and whole-buffer ones (the error-feedback rows moved between
    allocations while their placement is chosen).  A calibration copy reads
    between an eighth and four times its 1 GiB on either counter; of the
    copies in that window, those within a factor of two of the largest are
    kept."""
    win = [v for v in vals if GIB_KIB / 8 <= v <= 4 * GIB_KIB]
    if not win:
        raise SystemExit("no 1 GiB calibration copy among the copy dispatches (run with --calib)")
    top = max(win)
    return [v for v in win if v >= 0.5 * top]


def read_counter(path, counter):
    per = defaultdict(list)
    for r in csv.DictReader(_open(path)):
        if r["Counter_Name"] == counter:
            per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return per


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True, action="append")
    ap.add_argument("--fetch", default=None, help="FETCH_SIZE run (omit with --write: kernel trace only)")
    ap.add_argument("--write", default=None)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", default="")
    ap.add_argument("--step-launches-skip", type=int, default=1,
                    help="step-pass launches to drop from the counter average (the first step)")
    a = ap.parse_args()

    runs = [list(csv.DictReader(_open(path))) for path in a.stats]
    rows = runs[0]
    lines = [f"# Kernel profile — {a.workload}", ""]
    if a.command:
        lines += ["Commands ($R: the repository root; $OUT: an output directory):", "", "```", a.command.strip(),
                  "```", ""]
    lines += ["## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | avg ms | min ms | max ms | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                     f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}% |")
    step_ms = [x for x in (step_pass_ms(run) for run in runs) if x is not None]
    multi = any(per > 0 for _, _, per, _ in step_ms)
    form = "worker passes, then the owner pass" if multi else "one pass"
    lines += ["", f"## Step pass ({STEP_KERNEL}, {form}; no v stored) in each profiled process", "",
              "| process | owner pass avg ms | worker pass avg ms | worker passes per step | step pass ms |",
              "|---|---|---|---|---|"]
    lines += [f"| {i + 1} | {ow:.3f} | {wk:.3f} | {per:.2f} | {tot:.3f} |"
              for i, (ow, wk, per, tot) in enumerate(step_ms)]
    if not (a.fetch and a.write):  # kernel trace only: no counters file
        with open(a.out + ".md", "w") as f:
            f.write("\n".join(lines) + "\n")
        return
    fetch = read_counter(a.fetch, "FETCH_SIZE")
    write = read_counter(a.write, "WRITE_SIZE")
    fcal, wcal = calibration_values(fetch[CALIB_KERNEL]), calibration_values(write[CALIB_KERNEL])
    f_scale = GIB_KIB / (sum(fcal) / len(fcal))
    w_scale = GIB_KIB / (sum(wcal) / len(wcal))
    lines += ["", "## HBM bytes (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              f"Calibration copy of 1 GiB ({len(fcal)} and {len(wcal)} dispatches): FETCH_SIZE scale {f_scale:.3f}, "
              f"WRITE_SIZE scale {w_scale:.3f}.", "",
              "| kernel | launches | read GB / launch (scaled) | write GB / launch (scaled) |", "|---|---|---|---|"]
    out, names = {}, {}
    roles = {k: step_pass_role(k) for k in set(fetch) | set(write)}
    owners = sum(len(fetch.get(k, [])) for k, r in roles.items() if r in ("owner", "owner_v"))
    workers = sum(len(fetch.get(k, [])) for k, r in roles.items() if r == "worker")
    per = workers / owners if owners else 0.0  # worker passes per step
    for k in sorted(set(fetch) | set(write)):
        fv, wv = fetch.get(k, []), write.get(k, [])
        role = roles[k]
        if role in ("owner", "worker"):  # the first step's launches dropped
            skip = a.step_launches_skip * (1 if role == "owner" else round(per))
            fv, wv = fv[skip:], wv[skip:]
            names[role] = k
        if not fv or not wv:
            continue
        rd = sum(fv) / len(fv) * 1024 * f_scale / 1e9
        wr = sum(wv) / len(wv) * 1024 * w_scale / 1e9
        out[k] = (rd, wr)
        if rd + wr > 0.05:
            lines.append(f"| {k} | {len(fv)} | {rd:.3f} | {wr:.3f} |")
    rd, wr = out[names["owner"]]
    if "worker" in names:
        rd += per * out[names["worker"]][0]
        wr += per * out[names["worker"]][1]
    what = f"owner pass + {per:.2f} worker passes" if per > 0 else "one pass"
    lines += ["", f"Step pass ({what}): {rd:.3f} GB read, {wr:.3f} GB written."]
    with open(a.out + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    doc = {"workload": a.workload, "kernels": names, "worker_passes_per_step": per,
           "source_hash": step_pass_source_hash(),
           "hbm_read_bytes_per_step_pass": rd * 1e9, "hbm_write_bytes_per_step_pass": wr * 1e9,
           "hbm_bytes_per_step_pass": (rd + wr) * 1e9, "fetch_scale": f_scale, "write_scale": w_scale,
           "step_pass_ms_per_process": [tot for _, _, _, tot in step_ms]}
    with open(a.out + "_counters.json", "w") as f:
        json.dump(doc, f, indent=1)
    print(json.dumps(doc, indent=1))


if __name__ == "__main__":
    main()
