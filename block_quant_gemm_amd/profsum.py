"""Summaries of rocprofv3 output for the committed profiles.

  python -m block_quant_gemm_amd.profsum stats KERNEL_STATS_CSV
      Markdown table of a `rocprofv3 --kernel-trace --stats` summary
      (library kernels first; durations in microseconds).

  python -m block_quant_gemm_amd.profsum mfma DIR
      Matrix-unit utilisation of each library kernel from one `rocprofv3 --pmc
      SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE ...` run:
      busy cycles / (active cycles per XCC x SIMDs), from the run's agent info.

  python -m block_quant_gemm_amd.profsum traffic --fetch DIR --write DIR -o JSON
      HBM bytes per dispatch of each library kernel from two `rocprofv3 --pmc`
      runs of `bench.py --copy-calibration` (one with FETCH_SIZE, one with
      WRITE_SIZE; both counters are KiB per dispatch).  Each counter is scaled
      by the factor that makes the run's 1 GiB device-to-device copy read and
      write exactly 1 GiB.  The JSON records the kernel-source digest, so that
      bench.py reports the figures only while the kernels are unchanged.
"""

import argparse
import csv
import glob
import json
import os
import sys
from collections import defaultdict

LIB_PREFIX = ("void mxq::", "mxq::")
COPY_BYTES = 1 << 30


def short_name(name):
    """`void mxq::k_gemm<1, false, 0, true>(mxq::GemmArgs)` -> `k_gemm<1,false,0,true>`."""
    n = name
    for p in LIB_PREFIX:
        if n.startswith(p):
            n = n[len(p):]
    depth, out = 0, []
    for ch in n:
        if ch == "(" and depth == 0:
            break
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        out.append(ch)
    return "".join(out).replace(" ", "")


def is_lib(name):
    return name.startswith(LIB_PREFIX)


def stats(path):
    rows = list(csv.DictReader(open(path, newline="")))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = ["| kernel | calls | total us | average us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    other = [0, 0.0]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        if not is_lib(r["Name"]):
            other[0] += int(r["Calls"])
            other[1] += float(r["TotalDurationNs"])
            continue
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.1f | %.2f |" % (
            short_name(r["Name"]), r["Calls"], float(r["TotalDurationNs"]) / 1e3,
            float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            100.0 * float(r["TotalDurationNs"]) / total))
    lines.append("| (other: torch set-up and copies) | %d | %.1f | | | | %.2f |" % (
        other[0], other[1] / 1e3, 100.0 * other[1] / total))
    return "\n".join(lines)


def _counter_rows(d, counter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    out = []
    for f in files:
        for r in csv.DictReader(open(f, newline="")):
            if r["Counter_Name"] == counter:
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def _per_kernel(rows):
    acc = defaultdict(list)
    for _, name, v in rows:
        if is_lib(name):
            acc[short_name(name)].append(v)
    return acc


CALIBRATION_KERNEL = "__amd_rocclr_copyBuffer"     # the runtime's device-to-device copy


def _copy_kib(rows):
    """KiB the calibration copy reports: the largest dispatch of the runtime's
    copy kernel (the 1 GiB copy of `bench.py --copy-calibration`)."""
    vals = [v for _, name, v in rows if name.strip('"') == CALIBRATION_KERNEL]
    if not vals:
        raise SystemExit("no %s dispatch found (run bench.py --copy-calibration)"
                         % CALIBRATION_KERNEL)
    return max(vals)


def traffic(fetch_dir, write_dir):
    fr, wr = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / (_copy_kib(fr) * 1024.0)
    w_scale = COPY_BYTES / (_copy_kib(wr) * 1024.0)
    fk, wk = _per_kernel(fr), _per_kernel(wr)
    kernels = {}
    for k in sorted(set(fk) | set(wk)):
        f = sum(fk.get(k, [0])) / max(len(fk.get(k, [])), 1) * 1024.0 * f_scale
        w = sum(wk.get(k, [0])) / max(len(wk.get(k, [])), 1) * 1024.0 * w_scale
        kernels[k] = {"dispatches": max(len(fk.get(k, [])), len(wk.get(k, []))),
                      "fetch_bytes_per_launch": f, "write_bytes_per_launch": w,
                      "hbm_bytes_per_launch": f + w}
    from block_quant_gemm_amd.build import source_digest
    return {"what": "HBM bytes per dispatch (average over the run's dispatches of each "
                    "kernel) from rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by a 1 GiB "
                    "device-to-device copy",
            "fetch_scale": f_scale, "write_scale": w_scale,
            "source_digest": source_digest(), "kernels": kernels}


def mfma(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    agents = glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True)
    if not files or not agents:
        raise SystemExit("no counter_collection.csv / agent_info.csv under %s" % d)
    gpu = [r for r in csv.DictReader(open(agents[0], newline="")) if r.get("Agent_Type") == "GPU"][0]
    nxcc, nsimd = int(gpu["Num_Xcc"]), int(gpu["Simd_Count"])
    per = defaultdict(dict)
    for f in files:
        for r in csv.DictReader(open(f, newline="")):
            if is_lib(r["Kernel_Name"]):
                per[(int(r["Dispatch_Id"]), short_name(r["Kernel_Name"]))][r["Counter_Name"]] = \
                    float(r["Counter_Value"])
    acc = defaultdict(lambda: [0, 0.0, 0.0, 0.0])
    for (_, k), c in per.items():
        if c.get("SQ_INSTS_MFMA", 0) <= 0:
            continue
        a = acc[k]
        a[0] += 1
        a[1] += c["SQ_INSTS_MFMA"]
        a[2] += c["SQ_VALU_MFMA_BUSY_CYCLES"]
        a[3] += c["GRBM_GUI_ACTIVE"] / nxcc * nsimd
    lines = ["| kernel | dispatches | MFMA instructions per dispatch | MFMA busy / SIMD-cycles |",
             "|---|---:|---:|---:|"]
    for k in sorted(acc):
        n, ins, busy, avail = acc[k]
        lines.append("| %s | %d | %.0f | %.1f %% |" % (k, n, ins / n, 100.0 * busy / avail))
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("-o", "--out")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats(a.csv))
    elif a.cmd == "mfma":
        print(mfma(a.dir))
    else:
        rec = traffic(a.fetch, a.write)
        txt = json.dumps(rec, indent=1)
        if a.out:
            with open(a.out, "w") as f:
                f.write(txt + "\n")
        print(txt)


if __name__ == "__main__":
    ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    main()
