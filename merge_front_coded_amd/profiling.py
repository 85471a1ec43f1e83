"""Measurement helpers: source fingerprints of the kernels behind each C-ABI
call, and summaries of rocprofv3 output (kernel-trace statistics, HBM traffic
counters) written as short Markdown files.

A traffic summary records the fingerprint of the sources it was measured
with; ``bench.py`` reports a call's measured traffic only while the current
sources still hash to that fingerprint, so a figure is re-keyed only by
measuring it again.

Usage (from the repository root, after rocprofv3 runs that wrote CSV files):

  python -m merge_front_coded_amd.profiling traffic OUT.md WORKLOAD FETCH_DIRS WRITE_DIRS "COMMANDS"
  (FETCH_DIRS / WRITE_DIRS: comma-separated rocprofv3 output directories)
  python -m merge_front_coded_amd.profiling trace OUT.md "TITLE" STATS_CSV "COMMAND"
  python -m merge_front_coded_amd.profiling counters OUT.md "TITLE" DIRS "COMMANDS"
  (DIRS: comma-separated rocprofv3 output directories of --pmc runs)
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")

# The kernel sources each timed call depends on.
CALL_SOURCES = {
    "em_emit_merged": ("em_fc.hip", "em_tile.h", "em_internal.h"),
    "em_merge_lengths": ("em_merge_len.hip", "em_tile.h", "em_internal.h"),
    "em_merge_fc_onepass": ("em_onepass.hip", "em_tile.h", "em_internal.h"),
}

# The kernel (name prefix in the rocprofv3 output) behind each call's traffic.
CALL_KERNEL = {
    "em_emit_merged": "em::k_emit<true, true, true>",
    "em_merge_lengths": "em::k_merge_len<",
    "em_merge_fc_onepass": "em::k_onepass<",
}


def fingerprint(call: str) -> str | None:
    """First 16 hex digits of the SHA-256 of the call's kernel sources."""
    files = CALL_SOURCES.get(call)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        p = os.path.join(CSRC, f)
        if not os.path.exists(p):
            return None
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(workload_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload_name}.md")


_ROW = re.compile(r"^\|\s*`(?P<call>em_[a-z_0-9]+)`\s*\|.*\|\s*(?P<bytes>[0-9]+)\s*\|\s*`(?P<fp>[0-9a-f]{16})`\s*\|\s*$")


def measured_traffic(call: str, workload_name: str) -> int | None:
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch of the call's kernel on
    this workload, from its traffic summary, or None when there is none or
    the sources changed since it was measured."""
    path = traffic_path(workload_name)
    if not os.path.exists(path):
        return None
    want = fingerprint(call)
    with open(path) as f:
        for line in f:
            m = _ROW.match(line.strip())
            if m and m.group("call") == call:
                return int(m.group("bytes")) if m.group("fp") == want else None
    return None


def _counter_rows(dirs: str):
    """Rows of every rocprofv3 counter-collection CSV under the directories
    (comma-separated)."""
    rows = []
    for d in dirs.split(","):
        for p in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(p, newline="") as f:
                for r in csv.DictReader(f):
                    r["_file"] = p  # dispatch ids repeat across runs
                    rows.append(r)
    return rows


def kernel_short_name(name: str) -> str:
    """A rocprofv3 kernel name without its return type and argument list."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def _per_dispatch(rows, counter: str):
    """{kernel name: [value per dispatch]} for one counter (values summed over
    the rows of a dispatch)."""
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (kernel_short_name(r["Kernel_Name"]), r.get("_file"), r.get("Dispatch_Id") or r.get("Correlation_Id"))
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _, _), v in acc.items():
        out.setdefault(name, []).append(v)
    return out


def _median(v):
    s = sorted(v)
    return s[len(s) // 2]


def write_traffic(out_md: str, workload_name: str, fetch_dir: str, write_dir: str, command: str,
                  copy_bytes: int = 1 << 30) -> None:
    """Summarise FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every timed
    call's kernel, scaled by what each counter reads for the plain device copy
    of copy_bytes in the same run (``__amd_rocclr_copyBuffer``, the largest
    dispatch)."""
    fetch = _per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(write_dir), "WRITE_SIZE")
    copy_f = max(v for k, vs in fetch.items() if "copyBuffer" in k for v in vs)
    copy_w = max(v for k, vs in write.items() if "copyBuffer" in k for v in vs)
    kib = copy_bytes / 1024
    sf, sw = kib / copy_f, kib / copy_w
    lines = [f"# HBM traffic counters: {workload_name}", "",
             "Command (from the repository root, one MI355X; one counter per run, FETCH_SIZE then WRITE_SIZE):", "",
             "```", command, "```", "",
             f"Calibration: the plain device copy of {copy_bytes} bytes (`__amd_rocclr_copyBuffer`) reads and "
             f"writes {kib:.0f} KiB; its FETCH_SIZE reads {copy_f:.0f} KiB and its WRITE_SIZE {copy_w:.0f} KiB, so "
             f"FETCH_SIZE is scaled by {sf:.4f} and WRITE_SIZE by {sw:.4f}.", "",
             "| call | kernel | dispatches (median shown) | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes per "
             "launch | source fingerprint |",
             "|---|---|---|---|---|---|---|"]
    for call, kname in CALL_KERNEL.items():
        fk = [k for k in fetch if k.startswith(kname)]
        wk = [k for k in write if k.startswith(kname)]
        if not fk or not wk:
            continue
        fv = [v for k in fk for v in fetch[k]]
        wv = [v for k in wk for v in write[k]]
        f, w = _median(fv), _median(wv)
        nbytes = int(round((f * sf + w * sw) * 1024))
        lines.append(f"| `{call}` | `{fk[0]}` | {len(fv)} | {f:.0f} | {w:.0f} | {nbytes} | `{fingerprint(call)}` |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def write_trace(out_md: str, title: str, stats_csv: str, command: str, top: int = 40) -> None:
    """Summarise a rocprofv3 --kernel-trace --stats CSV (per-kernel calls and
    durations)."""
    with open(stats_csv, newline="") as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel-trace summary: {title}", "", "Command (from the repository root, one MI355X):", "",
             "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        lines.append(f"| `{kernel_short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _per_dispatch_all(rows):
    """{(kernel name, counter): [value per dispatch]} for every counter."""
    acc = {}
    for r in rows:
        key = (kernel_short_name(r["Kernel_Name"]), r["Counter_Name"], r.get("_file"),
               r.get("Dispatch_Id") or r.get("Correlation_Id"))
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, counter, _, _), v in acc.items():
        out.setdefault((name, counter), []).append(v)
    return out


def write_counters(out_md: str, title: str, dirs: str, command: str, cus: int = 256, simds: int = 1024,
                   clock_ghz: float = 2.4) -> None:
    """Summarise shader, LDS, address-unit and atomic counters per kernel
    (mean per dispatch), with the derived shares: cycles = GRBM_GUI_ACTIVE / 8
    (summed over the eight XCDs); VALU busy = 4 SQ_INSTS_VALU / (cycles x
    SIMDs) (a wave64 VALU instruction occupies a SIMD for four clocks); LDS
    conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; waiting share =
    SQ_WAIT_ANY / SQ_WAVE_CYCLES; resident waves per CU = 4 SQ_WAVE_CYCLES /
    (cycles x CUs) (SQ cycle counters tick once per four clocks); address unit
    busy = TA_TA_BUSY_sum / (cycles x CUs)."""
    vals = {k: sum(v) / len(v) for k, v in _per_dispatch_all(_counter_rows(dirs)).items()}
    names = sorted({k for k, _ in vals})
    g = lambda n, c: vals.get((n, c))
    lines = [f"# Shader, LDS, address-unit and atomic counters: {title}", "",
             "Commands (from the repository root, one MI355X; one counter group per run; values are means per "
             "dispatch):", "", "```", command, "```", "",
             "Derived: cycles = GRBM_GUI_ACTIVE / 8 (summed over the eight XCDs); VALU busy = 4 x SQ_INSTS_VALU / "
             f"(cycles x {simds} SIMDs); LDS conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; waiting share "
             "= SQ_WAIT_ANY / SQ_WAVE_CYCLES; resident waves per CU = 4 x SQ_WAVE_CYCLES / (cycles x "
             f"{cus}); address unit busy = TA_TA_BUSY_sum / (cycles x {cus}); cycles as ms at {clock_ghz} GHz.", "",
             "| kernel | waves | VALU instr | LDS instr | SALU instr | VALU busy | LDS conflict share | waiting share "
             "| resident waves/CU | address unit busy | cycles as ms |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    fmt = lambda x, f: "-" if x is None else f(x)
    atomic_rows = []
    for n in names:
        cyc = g(n, "GRBM_GUI_ACTIVE")
        cyc = cyc / 8 if cyc else None
        valu, lds, salu = g(n, "SQ_INSTS_VALU"), g(n, "SQ_INSTS_LDS"), g(n, "SQ_INSTS_SALU")
        if valu is not None:
            conf, idx = g(n, "SQ_LDS_BANK_CONFLICT"), g(n, "SQ_LDS_IDX_ACTIVE")
            wait, wc, ta = g(n, "SQ_WAIT_ANY"), g(n, "SQ_WAVE_CYCLES"), g(n, "TA_TA_BUSY_sum")
            pct = lambda a, b: None if a is None or not b else 100.0 * a / b
            lines.append(
                f"| `{n}` | {fmt(g(n, 'SQ_WAVES'), lambda x: f'{x:.0f}')} | {fmt(valu, lambda x: f'{x:.3g}')} | "
                f"{fmt(lds, lambda x: f'{x:.3g}')} | {fmt(salu, lambda x: f'{x:.3g}')} | "
                f"{fmt(pct(4 * valu, cyc * simds) if cyc else None, lambda x: f'{x:.0f}%')} | "
                f"{fmt(pct(conf, idx), lambda x: f'{x:.0f}%')} | {fmt(pct(wait, wc), lambda x: f'{x:.0f}%')} | "
                f"{fmt(4 * wc / (cyc * cus) if wc and cyc else None, lambda x: f'{x:.1f}')} | "
                f"{fmt(pct(ta, cyc * cus) if cyc else None, lambda x: f'{x:.0f}%')} | "
                f"{fmt(cyc / (clock_ghz * 1e6) if cyc else None, lambda x: f'{x:.3f}')} |")
        wr, wor = g(n, "TCP_TCC_ATOMIC_WITH_RET_REQ_sum"), g(n, "TCP_TCC_ATOMIC_WITHOUT_RET_REQ_sum")
        if wr is not None or wor is not None:
            atomic_rows.append(f"| `{n}` | {fmt(g(n, 'SQ_WAVES'), lambda x: f'{x:.0f}')} | "
                               f"{fmt(wor, lambda x: f'{x:.3g}')} | {fmt(wr, lambda x: f'{x:.3g}')} |")
    if atomic_rows:
        lines += ["", "| kernel | waves | atomics without return (TCP to TCC) | atomics with return |",
                  "|---|---|---|---|"] + atomic_rows
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    kind = sys.argv[1]
    if kind == "traffic":
        write_traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6])
    elif kind == "trace":
        write_trace(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif kind == "counters":
        write_counters(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    else:
        raise SystemExit(__doc__)
