"""Short text summaries of rocprofv3 output.

    python bench_profsum.py <kernel_stats.csv> "<command>" [title]
        a ``--kernel-trace --stats`` kernel table.
    python bench_profsum.py traffic <workload> <fetch.csv> <write.csv> <copy_fetch.csv> \
            <copy_write.csv> <copy_MiB> "<commands>" <source files...>
        HBM bytes per launch of every kernel in a ``--pmc FETCH_SIZE`` and a
        ``--pmc WRITE_SIZE`` run, each counter scaled by what it reads for a
        plain copy of known size, plus a machine-readable line keyed by the
        SHA-256 of the kernel sources (a later source change voids it).
    python bench_profsum.py counters <counters.csv> "<command>" [title]
        per-kernel means of a ``--pmc`` run of SQ counters: matrix-core
        utilisation (MfmaUtil), matrix-core flops (MOPS x 512) over the
        dispatch time, and where the waves spend their cycles.
"""
from __future__ import annotations

import csv
import sys


def summarize(path: str, command: str, title: str = "") -> str:
    rows = list(csv.DictReader(open(path)))
    lines = [f"# {title}" if title else "# rocprofv3 kernel summary", "", f"command: {command}", "",
             f"{'kernel':<72} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'total%':>7}"]
    for r in rows:
        name = r["Name"]
        name = kernel_key(name) if ("::k_" in name or name.startswith("_ZN12_GLOBAL")) else name[:60]
        lines.append(f"{name[:72]:<72} {int(r['Calls']):>6} {float(r['AverageNs'])/1e3:>9.2f} "
                     f"{float(r['MinNs'])/1e3:>9.2f} {float(r['MaxNs'])/1e3:>9.2f} {float(r['Percentage']):>7.2f}")
    return "\n".join(lines) + "\n"


def kernel_key(name: str) -> str:
    """'k_causal_chunks<float,64,128,1,float,elu1>' from a demangled or an Itanium-mangled
    kernel name (template arguments in order; a row format Fmt<element, feature map>
    becomes its element and the map's short name)."""
    import re

    maps = {"PhiElu1": "elu1", "PhiRelu": "relu", "PhiSoftplus": "softplus"}
    if "::k_" in name:
        body = re.sub(r"\(anonymous namespace\)::", "", name.split("::", 1)[1])
        if "<" not in body.split("(")[0]:
            return body.split("(")[0]
        body = body.split(">(")[0] + ">"
        body = body.replace(" ", "").replace("__bf16", "bf16").replace("_Float16", "f16")
        body = re.sub(r"Fmt<([^,<>]+),(Phi\w+)>", lambda m: m.group(1) + "," + maps.get(m.group(2), m.group(2)), body)
        return body.replace(">>", ">")
    m = re.match(r"_ZN12_GLOBAL__N_1(\d+)", name)
    if not m:
        return name.split("(")[0][:72]
    n0 = m.end()
    kname = name[n0:n0 + int(m.group(1))]
    rest = name[n0 + int(m.group(1)):]
    if not rest.startswith("I"):
        return kname
    # the template arguments end where the (void) kernel's parameter list begins
    m = re.search(r"Ev[PKfi]", rest)
    region = rest[1:m.start()] if m else rest[1:]
    args = []
    toks = {"DF16b": "bf16", "DF16_": "f16", "f": "float", "d": "double", "i": "int"}
    for tok in re.findall(r"Li-?\d+E|Lb[01]E|Phi\w+?E|DF16b|DF16_|NS_\d+FmtI|[fdi]", region):
        if tok.startswith("NS_"):
            continue
        if tok.startswith("Li"):
            args.append(tok[2:-1])
        elif tok.startswith("Lb"):
            args.append("true" if tok[2] == "1" else "false")
        elif tok.startswith("Phi"):
            args.append(maps.get(tok[:-1], tok[:-1]))
        else:
            args.append(toks[tok])
    return f"{kname}<{','.join(args)}>"


def _per_dispatch(path: str, counter: str) -> dict:
    """Mean counter value (KiB) per dispatch, by kernel name."""
    tot, n = {}, {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = r["Kernel_Name"]
        tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
        n.setdefault(k, set()).add(r["Dispatch_Id"])
    return {k: tot[k] / len(n[k]) for k in tot}


def sources_sha256(files) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic(workload, fetch, write, cfetch, cwrite, copy_mib, commands, sources) -> str:
    import json

    f, w = _per_dispatch(fetch, "FETCH_SIZE"), _per_dispatch(write, "WRITE_SIZE")
    cf, cw = _per_dispatch(cfetch, "FETCH_SIZE"), _per_dispatch(cwrite, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    # the copy kernel is the one whose reading is largest in the calibration run
    ff = copy_kib / max(cf.values())
    fw = copy_kib / max(cw.values())
    lines = [f"# HBM traffic per launch, workload {workload} (rocprofv3 PMC, calibrated)", "",
             f"commands: {commands}", "",
             f"calibration: a plain copy of {copy_mib} MiB reads {max(cf.values()):.0f} KiB FETCH_SIZE and "
             f"{max(cw.values()):.0f} KiB WRITE_SIZE per launch: factors {ff:.3f} (fetch) and {fw:.3f} (write)", "",
             f"{'kernel':<72} {'fetch_MB':>10} {'write_MB':>10} {'total_MB':>10}"]
    table = {}
    for k in sorted(set(f) & set(w)):
        rb, wb = f[k] * ff * 1024.0, w[k] * fw * 1024.0
        short = kernel_key(k)
        lines.append(f"{short:<72} {rb / 1e6:>10.2f} {wb / 1e6:>10.2f} {(rb + wb) / 1e6:>10.2f}")
        table[short] = round(rb + wb)
    lines += ["", "json: " + json.dumps({"workload": workload, "sources_sha256": sources_sha256(sources),
                                         "bytes_per_launch": table})]
    return "\n".join(lines) + "\n"


# Dense matrix-core peaks of MI355X (TFLOP/s) by operand type.
PEAK_TFLOPS = {"F32": 157.3, "BF16": 2500.0, "F16": 2500.0}


def counters(path: str, command: str, title: str = "") -> str:
    """Per-kernel means over dispatches of a --pmc run.

    MfmaUtil: percent of SIMD cycles the matrix core is busy (rocprofv3's
    derived counter).  MOPS_<type> x 512 is the flop count of the matrix-core
    instructions; divided by the dispatch's own duration (counters serialise
    dispatches, so this is a per-launch figure) it gives TFLOP/s, priced
    against the type's dense peak.  SQ_WAIT_ANY, SQ_ACTIVE_INST_LDS and
    SQ_WAIT_INST_LDS are shares of SQ_WAVE_CYCLES (all in wave quad-cycles).
    """
    per = {}  # kernel -> dispatch -> {counter: value, "_ns": duration}
    for r in csv.DictReader(open(path)):
        k = kernel_key(r["Kernel_Name"])
        d = per.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])

    def mean(ds, c):
        v = [d[c] for d in ds if c in d]
        return sum(v) / len(v) if v else float("nan")

    lines = [f"# {title}" if title else "# rocprofv3 counters", "", f"command: {command}", "",
             f"{'kernel':<56} {'calls':>5} {'us':>8} {'MfmaUtil%':>9} {'mfma_TF/s':>9} {'of_peak':>7} "
             f"{'wait%':>6} {'lds%':>6} {'ldswait%':>8} {'bankconf':>9}"]
    for k in sorted(per):
        ds = list(per[k].values())
        us = mean(ds, "_ns") / 1e3
        flops, peak = 0.0, None
        for t in ("F32", "BF16", "F16"):
            m = mean(ds, "SQ_INSTS_VALU_MFMA_MOPS_" + t)
            if m == m and m > 0:
                flops += m * 512.0
                peak = PEAK_TFLOPS[t] if peak is None else min(peak, PEAK_TFLOPS[t])
        tf = flops / (us * 1e-6) / 1e12 if us > 0 else 0.0
        wc = mean(ds, "SQ_WAVE_CYCLES")
        share = lambda c: 100.0 * mean(ds, c) / wc if wc == wc and wc > 0 else float("nan")
        lines.append(f"{k[:56]:<56} {len(ds):>5} {us:>8.2f} {mean(ds, 'MfmaUtil'):>9.2f} {tf:>9.2f} "
                     f"{(tf / peak if peak else 0.0):>7.3f} {share('SQ_WAIT_ANY'):>6.1f} "
                     f"{share('SQ_ACTIVE_INST_LDS'):>6.1f} {share('SQ_WAIT_INST_LDS'):>8.1f} "
                     f"{mean(ds, 'SQ_LDS_BANK_CONFLICT'):>9.0f}")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    if sys.argv[1] == "counters":
        a = sys.argv[2:]
        print(counters(a[0], a[1], a[2] if len(a) > 2 else ""), end="")
    elif sys.argv[1] == "traffic":
        a = sys.argv[2:]
        print(traffic(a[0], a[1], a[2], a[3], a[4], float(a[5]), a[6], a[7:]), end="")
    else:
        print(summarize(sys.argv[1], sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""), end="")
