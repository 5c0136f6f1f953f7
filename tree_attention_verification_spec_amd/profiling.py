"""rocprofv3 output -> short text summaries, and the HBM traffic figures those summaries record.

    python -m tree_attention_verification_spec_amd.profiling stats <kernel_stats.csv> <out.md> "<command>"
    python -m tree_attention_verification_spec_amd.profiling ea <reads.csv> <writes.csv> <kernel> \
        <copy_bytes> <algorithmic_bytes> <out.md> "<commands>"
    python -m tree_attention_verification_spec_amd.profiling mfma <mfma.csv> <kernel> \
        <algorithmic_flops> <out.md> "<command>"

``ea`` reads two ``rocprofv3 --pmc`` runs: the L2-to-memory read requests by size
(TCC_EA0_RDREQ_32B_sum, _64B_sum, _128B_sum) and the write requests (TCC_EA0_WRREQ_sum,
TCC_EA0_WRREQ_64B_sum; the rest are 32 bytes).  Bytes = 32 n32 + 64 n64 + 128 n128 read and
32 (n - n64) + 64 n64 written, per dispatch.  (FETCH_SIZE's expression takes 128-byte reads from
TCC_BUBBLE, which on this GPU does not count them, so it reads low.)  The same counters on a
plain device copy of known size are reported beside the figure as a check (no scaling is
applied).  The per-launch bytes of ``kernel`` are recorded with a hash of the file defining the
kernel and the shared header, so a later benchmark can tell whether the figure still describes
the current kernel.

``mfma`` reads SQ_VALU_MFMA_BUSY_CYCLES (summed over every SIMD) and
SQ_INSTS_VALU_MFMA_MOPS_BF16 (x 512 = bf16 FLOPs) per dispatch, and the dispatch's duration:
busy fraction = busy cycles / SIMDs / (duration x clock).
"""

import csv
import hashlib
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def kernel_sources(kname):
    """The HIP files a kernel's code comes from: the file defining it and the shared header."""
    base = kname.split("<")[0].strip()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith(".hip"):
            with open(os.path.join(csrc, f)) as fh:
                if re.search(r"__global__[^;{]*\b" + re.escape(base) + r"\s*\(", fh.read()):
                    return [f, "common.h"]
    raise KeyError(f"no source defines kernel {base}")


def _code(path):
    """A source file's code with comments removed and whitespace collapsed: an edited comment
    does not change the kernel a figure describes."""
    with open(path, encoding="utf-8") as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split()).encode()


def source_hash(files=None):
    """Hash of the code of the given csrc files (default: every HIP source and header, and the
    public header)."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    if files is None:
        files = [f for f in sorted(os.listdir(csrc)) if f.endswith((".hip", ".h"))]
        extra = [os.path.join(os.path.dirname(PKG), "include", "spectree.h")]
    else:
        extra = []
    for f in files:
        h.update(f.encode() + _code(os.path.join(csrc, f)))
    for f in extra:
        h.update(_code(f))
    return h.hexdigest()[:16]


def _hash_lines(kname):
    src = kernel_sources(kname)
    return [f"sources: {' '.join(src)}", f"source_hash: {source_hash(src)}"]


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


# How the commands in the summaries are run: from any directory, with REPO set to the
# repository root (the package built in place) and TMPDIR=/tmp.
RUN_NOTE = "`$REPO` is the repository root, with the library built in place; run with `TMPDIR=/tmp`."


def write_stats_summary(stats_csv, out_md, command):
    st = read_kernel_stats(stats_csv)
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "", RUN_NOTE, "",
             "| kernel | calls | avg us | total us |", "|---|---|---|---|"]
    for name, (calls, avg, tot) in sorted(st.items(), key=lambda kv: -kv[1][2]):
        lines.append(f"| {name} | {calls} | {avg / 1e3:.2f} | {tot / 1e3:.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _is_copy(name):
    n = name.lower()
    return "copy" in n or "elementwise" in n


def read_counters(path):
    """{dispatch id: (kernel short name, {counter: value}, duration ns)} of a --pmc run."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = out.setdefault(r["Dispatch_Id"], [short_name(r["Kernel_Name"]), defaultdict(float), 0])
            d[1][r["Counter_Name"]] += float(r["Counter_Value"])
            d[2] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return out


def _ea_reads(c):
    return 32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"] + 128 * c["TCC_EA0_RDREQ_128B_sum"]


def _ea_writes(c):
    return 32 * (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"]) + 64 * c["TCC_EA0_WRREQ_64B_sum"]


def write_ea_summary(reads_csv, writes_csv, kernel, copy_bytes, alg_bytes, out_md, commands):
    rd, wr = read_counters(reads_csv), read_counters(writes_csv)
    rk = [_ea_reads(c) for n, c, _ in rd.values() if n.startswith(kernel)]
    wk = [_ea_writes(c) for n, c, _ in wr.values() if n.startswith(kernel)]
    kname = next(n for n, _, _ in rd.values() if n.startswith(kernel))
    # the copy of known size: the copy dispatch whose byte count is nearest to it
    copy_r = min((_ea_reads(c) for n, c, _ in rd.values() if _is_copy(n)), key=lambda v: abs(v - copy_bytes),
                 default=0.0)
    copy_w = min((_ea_writes(c) for n, c, _ in wr.values() if _is_copy(n)), key=lambda v: abs(v - copy_bytes),
                 default=0.0)
    r_b, w_b = sum(rk) / len(rk), sum(wk) / len(wk)
    lines = ["# HBM traffic per launch (rocprofv3 --pmc, L2-to-memory requests by size)", "",
             f"kernel: {kname}", *_hash_lines(kname), f"launches: {len(rk)}",
             f"read_bytes_per_launch: {r_b:.0f}", f"write_bytes_per_launch: {w_b:.0f}",
             f"algorithmic_bytes_per_launch: {alg_bytes:.0f}",
             f"traffic_over_algorithmic: {(r_b + w_b) / alg_bytes:.3f}" if alg_bytes else "traffic_over_algorithmic: -",
             f"copy_check: a {copy_bytes:.0f}-byte device copy read {copy_r:.0f} and wrote {copy_w:.0f} bytes",
             f"traffic_bytes_per_launch: {r_b + w_b:.0f}", "", "Commands:", "", "```", commands, "```", "",
             RUN_NOTE]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_mfma_summary(mfma_csv, kernel, alg_flops, out_md, command, simds=1024, clock_ghz=2.4):
    mf = read_counters(mfma_csv)
    rows = [(c, d) for n, c, d in mf.values() if n.startswith(kernel)]
    kname = next(n for n, _, _ in mf.values() if n.startswith(kernel))
    busy = sum(c["SQ_VALU_MFMA_BUSY_CYCLES"] for c, _ in rows) / len(rows)
    flops = sum(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for c, _ in rows) / len(rows) * 512
    dur_ns = sum(d for _, d in rows) / len(rows)
    frac = busy / simds / (dur_ns * clock_ghz)
    lines = ["# MFMA use per launch (rocprofv3 --pmc)", "",
             f"kernel: {kname}", *_hash_lines(kname), f"launches: {len(rows)}",
             f"mfma_busy_cycles_per_simd: {busy / simds:.0f}",
             f"duration_us (serialised under the profiler): {dur_ns / 1e3:.2f}",
             f"mfma_busy_fraction: {frac:.3f}  (busy cycles per SIMD / (duration x {clock_ghz} GHz))",
             f"bf16_flops_executed: {flops:.4e}  (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)",
             f"algorithmic_flops: {alg_flops:.4e}",
             f"executed_tflops: {flops / dur_ns / 1e3:.1f}", "", "Command:", "", "```", command, "```", "",
             RUN_NOTE]
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
    files = kv["sources"].split() if "sources" in kv else None
    try:
        current = source_hash(files)
    except OSError:
        return None
    if kv.get("source_hash") != current:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"]), kv.get("kernel")
    except (KeyError, ValueError):
        return None


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        write_stats_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "ea":
        write_ea_summary(sys.argv[2], sys.argv[3], sys.argv[4], float(sys.argv[5]), float(sys.argv[6]), sys.argv[7],
                         sys.argv[8])
    elif sys.argv[1] == "mfma":
        write_mfma_summary(sys.argv[2], sys.argv[3], float(sys.argv[4]), sys.argv[5], sys.argv[6])
    else:
        raise SystemExit(__doc__)
