"""Summarise rocprofv3 counter passes over bench.py into per-kernel HBM traffic and MFMA use.

Each pass is its own `rocprofv3 --pmc ...` run of `bench.py --copy-calibration` (the counter
blocks cannot all be sampled in one run).  The plain 1 GiB device copy that --copy-calibration
adds reads and writes a known number of bytes; FETCH_SIZE / WRITE_SIZE of every kernel are scaled by
known / measured on that copy, so the figures are in true HBM bytes whatever unit the counters use.

    python profile_counters.py --trace TRACE_DIR --out-json profiles/gemm1_dsv3_share_traffic.json \
        PASS_DIR [PASS_DIR ...] > profiles/forward_dsv3_share_counters.md
    python profile_counters.py --variant mx --trace TRACE_DIR \
        --out-json profiles/mx_gemm1_wide_share_traffic.json PASS_DIR [...] > profiles/forward_mx_wide_share_counters.md
    python profile_counters.py latency PASS_DIR [...] > profiles/forward_dsv3_share_latency_counters.md
    python profile_counters.py --variant bwd --workload wide_share_fwd_bwd --trace TRACE_DIR \
        --out-json OUT.json PASS_DIR [...] > profiles/training_wide_share_counters.md

    python profile_counters.py stats TRACE_DIR --title TITLE --command CMD > profiles/<kernel>_<workload>_kernel_stats.md
    python profile_counters.py occupancy --pass DIR WORKLOAD [--pass DIR WORKLOAD] > profiles/forward_gemm_occupancy.md

Writes the L1 launch's HBM bytes (read + write) with the hash of the kernel source they were taken
on (bench.py reports them only while that source is unchanged) and prints a markdown table.  With
--variant mx the kernels are those of bench.py --mx (the FP8 x FP4 forward).
"""
import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "token_dispatch_grouped_route_amd", "csrc", "moe_grouped.hip")
MX_SRC = os.path.join(ROOT, "token_dispatch_grouped_route_amd", "csrc", "moe_mx.hip")
COPY_BYTES = 1 << 30   # bench.py --copy-calibration: one 1 GiB buffer copied to another
COMMON = (("combine_finish", "combine finish (multi-pair tokens)"),
          ("route_count", "prologue: count"), ("route_scan", "prologue: scan"),
          ("route_place", "prologue: place"))
BWD = (("dgrad_tile_kernel<moe::(anonymous namespace)::TrTile",
        "L2 dgrad NN, packed W2 read transposed + SwiGLU transpose + d(topk_w) partials + w*act"),
       ("dgrad_tile_kernel", "L2 dgrad NN on repacked W2 + SwiGLU transpose (many rows)"),
       ("l2_kernel<moe::(anonymous namespace)::TrTile", "L1 dgrad NN, packed W1 read transposed + combine rows"),
       ("wgrad_nt_kernel", "dW1 / dW2 TN on the forward pipeline (many rows)"),
       ("wgrad_tok_kernel<false>", "dW2 TN, variable K, dy fragments x hi/lo w*act in LDS"),
       ("wgrad_tok_kernel<true>", "dW1 TN, variable K, x fragments x hi/lo dhgu in LDS"),
       ("repack_t_kernel", "weight repack (many rows)"),
       ("rows_to_k_major_kernel", "row transforms of the weight-gradient operands"),
       ("dtopk_w_finish", "d(topk_w) finish"))
KERNEL_HEADERS = [os.path.join(ROOT, "token_dispatch_grouped_route_amd", "csrc", f) for f in ("moe_tiles.h", "moe_internal.h")]


def source_hash(src):
    """First 16 hex digits of the sha256 of the kernel source followed by the headers it includes
    (the same digest bench.py checks before it reports the traffic)."""
    h = hashlib.sha256()
    for f in [src] + KERNEL_HEADERS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


VARIANTS = {
    "bf16": {"title": "DeepSeek-V3 share forward", "src": GEMM_SRC, "l1": "l1_kernel", "workload": "dsv3_share_fwd",
             "kinds": (("l1_kernel", "L1: dispatch gather + grouped GEMM + SwiGLU"),
                       ("l2_kernel", "L2: grouped GEMM + weighted combine")) + COMMON},
    "mx": {"title": "MX (FP8 x FP4) forward, wide-expert share", "src": MX_SRC, "l1": "mx_l1",
           "workload": "wide_share_mx_fwd",
           "kinds": (("mx_l1", "MX L1: dispatch gather + FP8 x FP4 GEMM + clamped SwiGLU + FP8 cast"),
                     ("mx_l2", "MX L2: FP8 x FP4 GEMM + weighted combine")) + COMMON},
    "bwd": {"title": "training step", "src": os.path.join(ROOT, "token_dispatch_grouped_route_amd", "csrc",
                                                          "moe_gemm.hip"),
            "l1": None, "workload": "wide_share_fwd_bwd",
            "kinds": BWD + (("l1_kernel", "forward L1 (saves the fp32 pre-activation)"),
                            ("l2_kernel", "forward L2 + combine (also the L1 dgrad of many rows)")) + COMMON},
}
KINDS = VARIANTS["bf16"]["kinds"]


def kind_of(name):
    if "mx_gemm_kernel" in name:
        return "mx_l1" if ", true>" in name else "mx_l2"
    for key, _ in BWD + KINDS + VARIANTS["mx"]["kinds"]:
        if key in name:
            return key
    if "copyBuffer" in name:   # the runtime's plain device copy (--copy-calibration); conversion copies do not count
        return "copy"
    return None


def read_counters(dirs):
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    copies = collections.defaultdict(list)   # counter -> (grid size, value): other copies may run too
    for d in dirs:
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            k = kind_of(r["Kernel_Name"])
            if k == "copy":
                copies[r["Counter_Name"]].append((int(r["Grid_Size"]), float(r["Counter_Value"])))
            elif k:
                agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in agg.items()}
    if copies:   # the calibration copy is the largest one
        out["copy"] = {}
        for cname, vals in copies.items():
            g = max(v[0] for v in vals)
            sel = [v[1] for v in vals if v[0] == g]
            out["copy"][cname] = sum(sel) / len(sel)
    return out


def read_durations(trace_dir):
    dur = {}
    for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))):
        k = kind_of(r["Name"])
        if k and k not in dur:
            dur[k] = float(r["AverageNs"]) * 1e-9
    return dur


def stats_table(trace_dir, title, command, note, only=""):
    """Markdown table of a rocprofv3 --kernel-trace --stats run (every kernel whose name contains
    `only`, by total time; percentages of the listed kernels' total)."""
    rows = [r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))) if only in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print("# rocprofv3 kernel statistics: %s\n" % title)
    if command:
        print("Command (run from /tmp with TMPDIR=/tmp, repository at $R):\n\n```\n%s\n```\n" % command)
    if note:
        print(note + "\n")
    print("| kernel | calls | avg (us) | min (us) | max (us) | total (ms) | % |")
    print("|---|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        t = float(r["TotalDurationNs"])
        print("| `%s` | %s | %.1f | %.1f | %.1f | %.2f | %.1f |" % (
            r["Name"], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            t / 1e6, 100.0 * t / total))


def m_tiles_of(groups, max_groups):
    """M tiles of an expert of `groups` 32-row groups on the forward tile list: tiles of at most
    nine groups up to 18 groups and of eight beyond (bf16 GEMMs), of at most three (MX GEMMs)."""
    if max_groups == 9:
        return -(-groups // 9) if groups <= 18 else -(-groups // 8)
    return -(-groups // max_groups)


def occupancy_kind(name):
    """The forward GEMM launches of a run: bf16 L1 / L2 (the transposed-B l2_kernel is the L1 dgrad
    of a training step, not a forward launch) and the MX L1 / L2."""
    if "mx_gemm_kernel" in name:
        return "l1" if ", true>" in name else "l2"
    if "l1_kernel" in name:
        return "l1"
    if "l2_kernel" in name and "TrTile" not in name:
        return "l2"
    return None


def occupancy(dirs, workloads, command):
    """CU occupancy of the forward GEMM launches from SQ_WAVE_CYCLES (4-cycle units), SQ_BUSY_CYCLES
    (summed over the 32 shader engines) and GRBM_GUI_ACTIVE, one pass directory per workload, next
    to the L1 tile list those workloads produce: each expert's 32-row groups cut evenly into M tiles
    (m_tiles_of), 256-column N tiles.  A workload whose name contains "mx" is the MX forward (tiles
    of at most three groups)."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import moe_workloads as mw
    print("# CU occupancy of the forward GEMMs: tile lists and the tail of the persistent launches\n")
    if command:
        print("Commands (run from /tmp with TMPDIR=/tmp, repository at $R):\n\n```\n%s\n```\n" % command)
    print("Busy = 4 x SQ_WAVE_CYCLES / (4 waves x 256 CUs x kernel cycles), kernel cycles = SQ_BUSY_CYCLES / 32: "
          "the share of the launch during which a CU holds its persistent workgroup's waves.\n")
    print("| workload | local rows | largest expert | empty experts | L1 tiles by groups per M tile | L1 tiles per CU "
          "| L1 busy | L2 tiles per CU | L2 busy | L1 kernel cycles |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for d, name in zip(dirs, workloads):
        w = mw.get(name)
        max_groups = 3 if "mx" in name else 9
        idx, _ = mw.routing(w, 0)
        ids = idx.reshape(-1).astype(np.int64)
        ids = ids[(ids >= w.e_lo) & (ids < w.e_lo + w.EL)] - w.e_lo
        counts = np.bincount(ids, minlength=w.EL)
        tiles = collections.Counter()
        m_tiles = 0
        for g in (counts + 31) // 32:
            if g:
                mt = m_tiles_of(int(g), max_groups)
                base, rem = divmod(int(g), mt)
                tiles[base + 1] += rem * (2 * w.I // 256)
                tiles[base] += (mt - rem) * (2 * w.I // 256)
                m_tiles += mt
        tiles = collections.Counter({q: n for q, n in tiles.items() if n})
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            k = occupancy_kind(r["Kernel_Name"])
            if k:
                agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        busy, cyc = {}, {}
        for k, cs in agg.items():
            v = {c: sum(x) / len(x) for c, x in cs.items()}
            cyc[k] = v["SQ_BUSY_CYCLES"] / 32
            busy[k] = 4 * v["SQ_WAVE_CYCLES"] / (4 * 256 * cyc[k])
        print("| %s | %d | %d | %d | %s | %.2f | %.1f%% | %.2f | %.1f%% | %.0f |" % (
            name, counts.sum(), counts.max(), int((counts == 0).sum()),
            ", ".join("%d: %d" % (q, n) for q, n in sorted(tiles.items())), sum(tiles.values()) / 256,
            100 * busy.get("l1", float("nan")), m_tiles * (w.H // 256) / 256, 100 * busy.get("l2", float("nan")),
            cyc.get("l1", 0)))


LATENCY_ORDER = ("SQ_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_INSTS_VMEM", "SQ_INST_LEVEL_LDS", "SQ_INST_LEVEL_VMEM",
                 "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "TA_ADDR_STALLED_BY_TC_CYCLES_sum",
                 "TA_BUSY_avr", "TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum", "TCC_HIT_sum", "TCC_MISS_sum",
                 "TCP_PENDING_STALL_CYCLES_sum", "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum",
                 "TCP_TCR_TCP_STALL_CYCLES_sum")


def latency(dirs, command, title):
    """Memory-path table of the forward GEMMs (l1_kernel, l2_kernel, or the MX ones) from the pass directories of
    the counters in LATENCY_ORDER: per-dispatch averages and the ratios derived from them."""
    c = read_counters(dirs)
    ks = [k for k in ("l1_kernel", "l2_kernel", "mx_l1", "mx_l2") if k in c]
    v = {k: c[k] for k in ks}
    label = {"l1_kernel": "L1", "l2_kernel": "L2", "mx_l1": "MX L1", "mx_l2": "MX L2"}
    print("# rocprofv3 memory-path counters of the forward GEMMs (%s)\n" % title)
    if command:
        print("Commands (run from /tmp with TMPDIR=/tmp, repository at $R), one pass each:\n\n```\n%s\n```\n" % command)
    print("Averages per dispatch over every dispatch of each kernel in the passes.")
    print("Derived: kernel cycles = SQ_BUSY_CYCLES / 32 shader engines; TCP pending-stall share = "
          "TCP_PENDING_STALL_CYCLES / 256 CUs / kernel cycles;")
    print("L1-to-L2 read latency = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ; L2 hit rate = TCC_HIT / "
          "(TCC_HIT + TCC_MISS);")
    print("L2-to-memory read latency = TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ; wave time in s_waitcnt = "
          "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES.\n")
    print("| kernel | kernel cycles | TCP pending-stall share | L1→L2 read latency (cycles) | L2 hit rate "
          "| L2→memory read latency (cycles) | wave time waiting | LDS bank conflicts / LDS instruction |")
    print("|---|---|---|---|---|---|---|---|")
    for k in ks:
        x = v[k]
        cyc = x["SQ_BUSY_CYCLES"] / 32
        print("| %s | %.0f | %.0f%% | %.0f | %.0f%% | %.0f | %.0f%% | %.4f |" % (
            label[k], cyc, 100 * x["TCP_PENDING_STALL_CYCLES_sum"] / 256 / cyc,
            x["TCP_TCC_READ_REQ_LATENCY_sum"] / x["TCP_TCC_READ_REQ_sum"],
            100 * x["TCC_HIT_sum"] / (x["TCC_HIT_sum"] + x["TCC_MISS_sum"]),
            x["TCC_EA0_RDREQ_LEVEL_sum"] / x["TCC_EA0_RDREQ_sum"], 100 * x["SQ_WAIT_INST_ANY"] / x["SQ_WAVE_CYCLES"],
            x["SQ_LDS_BANK_CONFLICT"] / x["SQ_INSTS_LDS"]))
    print("\nRaw averages:\n")
    print("| counter | " + " | ".join(label[k] for k in ks) + " |")
    print("|---|" + "---|" * len(ks))
    for n in LATENCY_ORDER:
        print("| %s | %s |" % (n, " | ".join("%.0f" % v[k].get(n, float("nan")) for k in ks)))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "latency":
        ap = argparse.ArgumentParser(prog="profile_counters.py latency")
        ap.add_argument("passes", nargs="+")
        ap.add_argument("--command", default="")
        ap.add_argument("--title", default="DeepSeek-V3 share")
        a = ap.parse_args(sys.argv[2:])
        return latency(a.passes, a.command, a.title)
    if len(sys.argv) > 1 and sys.argv[1] == "occupancy":
        ap = argparse.ArgumentParser(prog="profile_counters.py occupancy")
        ap.add_argument("--pass", dest="passes", nargs=2, action="append", metavar=("DIR", "WORKLOAD"), required=True)
        ap.add_argument("--command", default="")
        a = ap.parse_args(sys.argv[2:])
        return occupancy([p[0] for p in a.passes], [p[1] for p in a.passes], a.command)
    if len(sys.argv) > 1 and sys.argv[1] == "stats":
        ap = argparse.ArgumentParser(prog="profile_counters.py stats")
        ap.add_argument("trace")
        ap.add_argument("--title", required=True)
        ap.add_argument("--command", default="")
        ap.add_argument("--note", default="")
        ap.add_argument("--only", default="", help="list only kernels whose name contains this")
        a = ap.parse_args(sys.argv[2:])
        return stats_table(a.trace, a.title, a.command, a.note, a.only)
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True, help="rocprofv3 --kernel-trace --stats output directory")
    ap.add_argument("--out-json", required=True)
    ap.add_argument("--command", default="", help="the command lines that made the passes, for the record")
    ap.add_argument("--variant", choices=sorted(VARIANTS), default="bf16")
    ap.add_argument("--workload", default="", help="workload name recorded in the json (bwd variant)")
    ap.add_argument("passes", nargs="+")
    a = ap.parse_args()
    var = VARIANTS[a.variant]
    c = read_counters(a.passes)
    dur = read_durations(a.trace)
    cp = c.get("copy", {})
    if "FETCH_SIZE" not in cp or "WRITE_SIZE" not in cp:
        sys.exit("no copy-calibration kernel with FETCH_SIZE and WRITE_SIZE in the passes")
    # counters are in KiB; scale each to the copy's known bytes
    fr = COPY_BYTES / (cp["FETCH_SIZE"] * 1024.0)
    fw = COPY_BYTES / (cp["WRITE_SIZE"] * 1024.0)
    print("# rocprofv3 counters per kernel (%s)\n" % (var["title"] + (", " + a.workload if a.workload else "")))
    if a.command:
        print("Commands (run from /tmp with TMPDIR=/tmp, repository at $R):\n\n```\n%s\n```\n" % a.command)
    print("FETCH_SIZE and WRITE_SIZE are scaled by what they read on a plain 1 GiB device copy: "
          "read x %.3f, write x %.3f.  Durations are the kernel-trace averages of the same workload; "
          "MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs.\n" % (fr, fw))
    print("| kernel | avg us | HBM read MB | HBM write MB | HBM GB/s | MFMA busy %% | %s |"
          % ("bf16 MFMA TFLOP/s" if a.variant in ("bf16", "bwd") else "MFMA TFLOP/s (not counted)"))
    print("|---|---|---|---|---|---|---|")
    rec = {}
    for key, label in var["kinds"]:
        if key not in c:
            continue
        v = c[key]
        rd = v.get("FETCH_SIZE", float("nan")) * 1024.0 * fr
        wr = v.get("WRITE_SIZE", float("nan")) * 1024.0 * fw
        t = dur.get(key)
        bw = (rd + wr) / t / 1e9 if t else float("nan")
        busy = v.get("MfmaUtil", float("nan"))
        mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        fl = mops * 512 if mops is not None else None   # None: the pass set holds no MFMA op counter
        tf = "%.0f" % (fl / t / 1e12) if (fl is not None and t) else "-"
        print("| %s | %.1f | %.1f | %.1f | %.0f | %.1f | %s |" % (label, (t or 0) * 1e6, rd / 1e6, wr / 1e6, bw, busy, tf))
        rec[key] = {"read_bytes": rd, "write_bytes": wr, "avg_s": t, "mfma_busy_pct": busy, "mfma_bf16_flops": fl}
    if var["l1"] is None:   # every kernel's figures, no single roofline kernel
        with open(a.out_json, "w") as f:
            json.dump({"workload": a.workload or var["workload"], "copy_scale_read": fr, "copy_scale_write": fw,
                       "kernels": rec, "command": a.command}, f, indent=1)
        return
    l1 = rec.get(var["l1"])
    if l1:
        out = {"kernel_source_sha256_16": source_hash(var["src"]),
               "workload": var["workload"],
               "hbm_bytes_per_launch": l1["read_bytes"] + l1["write_bytes"],
               "hbm_read_bytes_per_launch": l1["read_bytes"], "hbm_write_bytes_per_launch": l1["write_bytes"],
               "copy_scale_read": fr, "copy_scale_write": fw, "kernels": rec, "command": a.command}
        with open(a.out_json, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
