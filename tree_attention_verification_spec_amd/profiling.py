"""rocprofv3 output -> short text summaries, and the HBM traffic figures those summaries record.

    python -m tree_attention_verification_spec_amd.profiling stats <kernel_stats.csv> <out.md> "<command>"
    python -m tree_attention_verification_spec_amd.profiling traffic <fetch.csv> <write.csv> <kernel> \
        <copy_bytes> <out.md> "<commands>"

``traffic`` reads two ``rocprofv3 --pmc`` runs (FETCH_SIZE, then WRITE_SIZE; both KiB per
dispatch), scales each by what the same counter read for a plain device copy of known size
(the copy kernel's dispatches are those whose name contains "copy" or "elementwise"), and
records the per-launch HBM bytes of ``kernel`` together with a hash of the kernel sources,
so a later benchmark can tell whether the figure still describes the current kernels.
"""

import csv
import hashlib
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def source_hash():
    """Hash of the HIP sources and the public header (the kernels the figures describe)."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    with open(os.path.join(os.path.dirname(PKG), "include", "spectree.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def _col(header, *names):
    low = [c.strip().lower() for c in header]
    for n in names:
        if n.lower() in low:
            return low.index(n.lower())
    raise KeyError(f"none of {names} in {header}")


def short_name(name):
    """void spectree::(anonymous namespace)::tree_attn_bf16_kernel<128, 4>(...) -> tree_attn_bf16_kernel<128, 4>"""
    name = name.replace("(anonymous namespace)::", "").strip()
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):          # end of the name: first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    name = name[:cut]
    head, sep, tmpl = name.partition("<")
    return (head.split("::")[-1] + sep + tmpl).strip()


def read_kernel_stats(path):
    """{kernel short name: (calls, avg_ns, total_ns)} from rocprofv3's kernel_stats.csv."""
    out = {}
    with open(path) as f:
        rows = list(csv.reader(f))
    hdr = rows[0]
    iname, icalls = _col(hdr, "Name", "KernelName"), _col(hdr, "Calls")
    iavg, itot = _col(hdr, "AverageNs", "Average_Ns"), _col(hdr, "TotalDurationNs", "Total_Duration_Ns")
    for r in rows[1:]:
        out[short_name(r[iname])] = (int(r[icalls]), float(r[iavg]), float(r[itot]))
    return out


def read_counter(path, counter):
    """{kernel short name: [value per dispatch]} for one counter of a rocprofv3 --pmc run."""
    vals = defaultdict(dict)
    with open(path) as f:
        rows = list(csv.reader(f))
    hdr = rows[0]
    ik = _col(hdr, "Kernel_Name", "KernelName", "Kernel-Name")
    ic = _col(hdr, "Counter_Name", "CounterName")
    iv = _col(hdr, "Counter_Value", "CounterValue")
    idd = _col(hdr, "Dispatch_Id", "DispatchId", "Correlation_Id")
    for r in rows[1:]:
        if r[ic] != counter:
            continue
        d = vals[short_name(r[ik])]
        d[r[idd]] = d.get(r[idd], 0.0) + float(r[iv])
    return {k: list(v.values()) for k, v in vals.items()}


def write_stats_summary(stats_csv, out_md, command):
    st = read_kernel_stats(stats_csv)
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | avg us | total us |", "|---|---|---|---|"]
    for name, (calls, avg, tot) in sorted(st.items(), key=lambda kv: -kv[1][2]):
        lines.append(f"| {name} | {calls} | {avg / 1e3:.2f} | {tot / 1e3:.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _is_copy(name):
    n = name.lower()
    return "copy" in n or "elementwise" in n


def write_traffic_summary(fetch_csv, write_csv, kernel, copy_bytes, out_md, commands):
    fetch = read_counter(fetch_csv, "FETCH_SIZE")
    wr = read_counter(write_csv, "WRITE_SIZE")
    kname = next(k for k in fetch if k.startswith(kernel))
    copy_f = max((v for k, vs in fetch.items() if _is_copy(k) for v in vs), default=None)
    copy_w = max((v for k, vs in wr.items() if _is_copy(k) for v in vs), default=None)
    f_kib = sum(fetch[kname]) / len(fetch[kname])
    w_kib = sum(wr[kname]) / len(wr[kname])
    f_scale = copy_bytes / (copy_f * 1024.0) if copy_f else 1.0
    w_scale = copy_bytes / (copy_w * 1024.0) if copy_w else 1.0
    fetch_b = f_kib * 1024.0 * f_scale
    write_b = w_kib * 1024.0 * w_scale
    lines = ["# HBM traffic per launch (rocprofv3 --pmc)", "",
             f"kernel: {kname}", f"source_hash: {source_hash()}",
             f"fetch_kib_per_dispatch: {f_kib:.1f}", f"write_kib_per_dispatch: {w_kib:.1f}",
             f"copy_bytes: {copy_bytes}", f"copy_fetch_kib: {copy_f}", f"copy_write_kib: {copy_w}",
             f"fetch_scale: {f_scale:.4f}", f"write_scale: {w_scale:.4f}",
             f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}", "", "Commands:", "", "```", commands, "```"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path):
    """(bytes per launch, kernel) from a traffic summary if its source hash is current, else None."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "`")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"]), kv.get("kernel")
    except (KeyError, ValueError):
        return None


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        write_stats_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        write_traffic_summary(sys.argv[2], sys.argv[3], sys.argv[4], float(sys.argv[5]), sys.argv[6], sys.argv[7])
    else:
        raise SystemExit(__doc__)
