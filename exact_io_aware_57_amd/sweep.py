"""Counters of every forward-kernel candidate on the two matrix-bound workloads.

    python -m exact_io_aware_57_amd.sweep build           # CPU: the candidate copies of the library
    python -m exact_io_aware_57_amd.sweep run OUT         # GPU: rocprofv3 passes, raw output under OUT
    python -m exact_io_aware_57_amd.sweep summarize OUT   # writes profiles/kernel_choice.txt

The library picks one kernel form per call (head size, key range, grid size).
This sweep measures the forms it could have picked instead, on the same
workload: each candidate is a copy of the library built with -DFA_FORCE_FWD=id
(exact_io_aware_57_amd.build --candidate id), which bench.py loads through
FA_MI355X_LIB.  Per (workload, candidate) four runs of bench.py (the timed
steps only, --no-others --no-cpu-baseline --no-extras):

  trace  rocprofv3 --kernel-trace --stats            kernel duration
  util   rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil LdsBankConflict
  fetch  rocprofv3 --pmc FETCH_SIZE  (+ a 256 MiB device copy: KiB -> bytes)
  write  rocprofv3 --pmc WRITE_SIZE  (+ the same copy)

The run step only starts rocprofv3 processes; it never touches the GPU itself.
"""
import csv
import glob
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from exact_io_aware_57_amd import build as B  # noqa: E402

# candidate id -> kernel form (the ids of launch_candidate in fa_fwd_bf16.hip)
FORMS = {1: "8-wave ping-pong, 64-key tiles", 2: "8-wave ping-pong, 128-key tiles", 3: "8-wave ping-pong, 32-key tiles",
         4: "4-wave, 32-key tiles", 5: "4-wave, 64-key tiles", 6: "4-wave, 128-key tiles",
         7: "4-wave, two key groups, 64-key tiles", 8: "4-wave, two key groups, 128-key tiles"}
# workload index -> candidate ids, the library's own choice first
CANDIDATES = {4: [2, 1, 6, 5, 4, 8, 7], 5: [1, 7, 4]}
UTIL = ["MfmaUtil", "VALUBusy", "LdsUtil", "LdsBankConflict"]
COPY_MB = 256
PASSES = ("trace", "util", "fetch", "write")


def bench_cmd(wl, pmc_pass):
    steps = "--steps 10 --warmup 5" if pmc_pass == "trace" else "--steps 3 --warmup 1"
    cmd = ["python3", os.path.join(ROOT, "bench.py"), "--workload", str(wl), *steps.split(), "--no-others",
           "--no-cpu-baseline", "--no-extras"]
    if pmc_pass in ("fetch", "write"):
        cmd += ["--calib-copy-mb", str(COPY_MB)]
    return cmd


def prof_cmd(pmc_pass, outdir):
    if pmc_pass == "trace":
        return ["rocprofv3", "--kernel-trace", "--stats", "-d", outdir, "-o", "p", "--output-format", "csv"]
    counters = {"util": UTIL, "fetch": ["FETCH_SIZE"], "write": ["WRITE_SIZE"]}[pmc_pass]
    return ["rocprofv3", "--pmc", *counters, "-d", outdir, "-o", "p", "--output-format", "csv"]


def command_line(pmc_pass):
    """The command of one pass, with W (workload), C (candidate) and OUT as placeholders."""
    lib = os.path.relpath(B.candidate_path(0), ROOT).replace("candidate0", "candidateC")
    bench = " ".join(bench_cmd(0, pmc_pass)).replace(os.path.join(ROOT, ""), "").replace("--workload 0", "--workload W")
    return f"FA_MI355X_LIB={lib} " + " ".join(prof_cmd(pmc_pass, os.path.join("OUT", "wW_cC", pmc_pass))) + " -- " + bench


def do_build():
    for cid in sorted({c for cs in CANDIDATES.values() for c in cs}):
        print(B.build_candidate(cid), flush=True)


def do_run(out):
    os.makedirs(out, exist_ok=True)
    for wl, cids in CANDIDATES.items():
        for cid in cids:
            for pmc_pass in PASSES:
                d = os.path.join(out, f"w{wl}_c{cid}", pmc_pass)
                env = dict(os.environ, FA_MI355X_LIB=B.candidate_path(cid))
                cmd = prof_cmd(pmc_pass, d) + ["--"] + bench_cmd(wl, pmc_pass)
                print(f"sweep: workload {wl} candidate {cid} ({FORMS[cid]}) pass {pmc_pass} {time.strftime('%T')}",
                      flush=True)
                os.makedirs(d, exist_ok=True)
                with open(os.path.join(d, "run.log"), "w") as log:
                    try:
                        r = subprocess.run(cmd, env=env, stdout=log, stderr=subprocess.STDOUT,
                                           timeout=150 if pmc_pass == "trace" else 90)
                    except subprocess.TimeoutExpired:
                        print("sweep: time limit reached; stopping", flush=True)
                        return 124
                if r.returncode != 0:
                    print(f"sweep: rocprofv3 exited with {r.returncode}; stopping (see {d}/run.log)", flush=True)
                    return r.returncode
    return 0


def _rows(pattern):
    files = glob.glob(pattern, recursive=True)
    return list(csv.DictReader(open(files[0]))) if files else []


def _is_fa(name):
    return "fwd_bf16" in name and "fa::" in name


def summarize(out):
    from bench import PEAK_BF16_TFLOPS, algorithmic_flops
    from exact_io_aware_57_amd.inputs import workload

    lines = []
    for wl, cids in CANDIDATES.items():
        w = workload(wl)
        flops = algorithmic_flops(w.B, w.H, w.N, w.d, w.causal)
        lines.append(f"## {w.describe()}  ({flops:.4g} FLOP per launch)")
        lines.append(f"{'cand':>4s}  {'kernel form':38s} {'kernel':34s} {'ms':>8s} {'TFLOP/s':>8s} {'frac':>6s} "
                     + " ".join(f"{u:>9s}" for u in UTIL) + f" {'fetch MB':>9s} {'write MB':>9s}")
        for cid in cids:
            base = os.path.join(out, f"w{wl}_c{cid}")
            stats = [r for r in _rows(os.path.join(base, "trace", "**", "*kernel_stats.csv")) if _is_fa(r["Name"])]
            if not stats:
                lines.append(f"{cid:4d}  {FORMS[cid]:38s} (no trace)")
                continue
            kname = stats[0]["Name"].replace("void fa::(anonymous namespace)::", "").split("(fa::")[0]
            ms = float(stats[0]["AverageNs"]) / 1e6
            util = {}
            for r in _rows(os.path.join(base, "util", "**", "*counter_collection.csv")):
                if _is_fa(r["Kernel_Name"]):
                    util.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            traffic = []
            for pmc_pass, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
                fa, copy = [], []
                for r in _rows(os.path.join(base, pmc_pass, "**", "*counter_collection.csv")):
                    if r["Counter_Name"] != counter:
                        continue
                    if _is_fa(r["Kernel_Name"]):
                        fa.append(float(r["Counter_Value"]))
                    elif "copyBuffer" in r["Kernel_Name"]:
                        copy.append(float(r["Counter_Value"]))
                traffic.append(sum(fa) / len(fa) * (COPY_MB << 20) / max(copy) / 1e6 if fa and copy else float("nan"))
            tf = flops / (ms * 1e-3) / 1e12
            u = [sum(util[c]) / len(util[c]) if util.get(c) else float("nan") for c in UTIL]
            lines.append(f"{cid:4d}  {FORMS[cid]:38s} {kname:34s} {ms:8.4f} {tf:8.1f} {tf / PEAK_BF16_TFLOPS:6.3f} "
                         + " ".join(f"{x:9.2f}" for x in u) + f" {traffic[0]:9.2f} {traffic[1]:9.2f}")
        lines.append("")
    path = os.path.join(ROOT, "profiles", "kernel_choice.txt")
    with open(path, "w") as f:
        f.write("# Kernel choice on the two matrix-bound workloads: every candidate form of the bf16 forward pass,\n")
        f.write("# measured on the same workload.  The first row of each table is the form the library picks.\n")
        f.write("# ms: average kernel duration (rocprofv3 --kernel-trace --stats); frac: of the bf16 dense peak\n")
        f.write("# 2516.6 TFLOP/s.  MfmaUtil, VALUBusy, LdsUtil, LdsBankConflict: rocprofv3's derived counters\n")
        f.write("# (percent of cycles; LdsBankConflict a ratio), averaged over the profiled dispatches.  fetch/write MB:\n")
        f.write(f"# FETCH_SIZE / WRITE_SIZE per dispatch scaled by the same counters on a {COPY_MB} MiB device copy.\n")
        f.write("# Commands (per workload W, candidate C and pass; the candidate library is built with\n")
        f.write("#   python -m exact_io_aware_57_amd.build --candidate C):\n")
        for pmc_pass in PASSES:
            f.write("#   " + command_line(pmc_pass) + "\n")
        f.write("# driven by: python -m exact_io_aware_57_amd.sweep run OUT; summarize OUT\n")
        f.write(f"# kernel sources sha {source_sha()}\n\n")
        f.write("\n".join(lines) + "\n")
    return path


def source_sha():
    from bench import TRAFFIC_ALL_SOURCES, source_hash

    return source_hash(TRAFFIC_ALL_SOURCES)


if __name__ == "__main__":
    if len(sys.argv) < 2 or sys.argv[1] not in ("build", "run", "summarize"):
        print(__doc__)
        sys.exit(2)
    if sys.argv[1] == "build":
        do_build()
    elif sys.argv[1] == "run":
        sys.exit(do_run(sys.argv[2]))
    else:
        print(summarize(sys.argv[2]))
