"""Summaries of rocprofv3 output for the library's kernels (host-side tooling, no GPU use).

rocprofv3 (ROCm 7.x) writes a SQLite database (``*_results.db``) per run. This module
reads it and prints

* ``stats DB``: per kernel, the dispatch count and total / average / min / max duration,
  the table that ``rocprofv3 --kernel-trace --stats`` summarises;
* ``counters``: per kernel, the average per dispatch of every counter in one or more ``--pmc`` runs, with
  the MFMA pipe's busy fraction and instructions per wave derived from them;
* ``traffic``: HBM bytes per launch of one kernel from two counter runs, ``--pmc
  FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (KiB per dispatch), each scaled by what the same
  counter reads for a plain copy kernel of known size in the same run (the int32
  elementwise bitwise-not that ``bench.py --copy-calib MiB`` launches before its timed steps).

Kernels are reported under the names the library's timers use (``reduce``, ``output``...).
"""
import argparse
import json
import os
import re
import sqlite3
import sys

# mangled kernel name fragment -> timer name used by the library and bench.py
_SHORT = [
    ("cbwd_fwd_kernel", "cbwd_fwd"),
    ("cbwd_q_kernel", "cbwd_q"),
    ("cbwd_v_kernel", "cbwd_v"),
    ("cbwd_t_kernel", "cbwd_t"),
    ("cbwd_k_kernel", "cbwd_k"),
    ("cbwd_rscan_kernel", "rscan"),
    ("omegaT_pair_kernel", "omega_frag"),
    ("bwd_q_kernel", "bwd_q"),
    ("bwd_k_kernel", "bwd_k"),
    ("combine_rows_kernel", "combine_rows"),
    ("omegaT_frag_kernel", "omega_frag"),
    ("kv_reduce_kernel", "reduce"),
    ("q_output_kernel", "output"),
    ("combine_kernel", "combine"),
    ("omega_frag_kernel", "omega_frag"),
    ("features_kernel", "features"),
    ("scan_kernel", "scan"),
    ("sweep_kernel", "sweep"),
    ("decode_kernel", "decode"),
    ("reduce_kernel", "reduce"),
]


def short_name(kernel: str) -> str:
    if "favor" in kernel:
        for frag, name in _SHORT:
            if frag in kernel:
                return name
    if "bitwise_not" in kernel:
        return "copy:bitwise_not"
    if "elementwise" in kernel or "copy" in kernel.lower():
        return "copy:" + re.sub(r"\W+", "_", kernel)[:48]
    return re.sub(r"\W+", "_", kernel)[:48]


def _con(db: str) -> sqlite3.Connection:
    if not os.path.exists(db):
        raise FileNotFoundError(db)
    return sqlite3.connect(db)


def kernel_stats(db: str):
    """[(name, calls, total_us, avg_us, min_us, max_us, pct)] sorted by total time."""
    con = _con(db)
    rows = con.execute("select name, start, end from kernels").fetchall()
    per = {}
    for name, s, e in rows:
        per.setdefault(short_name(name), []).append((e - s) * 1e-3)  # ns -> us
    total = sum(sum(v) for v in per.values()) or 1.0
    out = []
    for n, v in per.items():
        out.append((n, len(v), sum(v), sum(v) / len(v), min(v), max(v), 100.0 * sum(v) / total))
    return sorted(out, key=lambda r: -r[2])


def counter_per_dispatch(db: str, counter: str):
    """{name: [value per dispatch]} for one counter (summed over the counter's instances)."""
    con = _con(db)
    rows = con.execute(
        "select dispatch_id, kernel_name, counter_name, value from counters_collection").fetchall()
    per = {}
    for did, kn, cn, v in rows:
        if cn != counter:
            continue
        per.setdefault(short_name(kn), {}).setdefault(did, 0.0)
        per[short_name(kn)][did] += v
    return {n: list(d.values()) for n, d in per.items()}


def _copy_factor(vals: dict, copy_bytes: int) -> float:
    # the calibration copy is the int32 bitwise-not kernel that bench.py --copy-calib launches
    cands = [(n, v) for n, v in vals.items() if n.startswith("copy:") and "bitwise_not" in n]
    if len(cands) != 1 or len(cands[0][1]) != 1:
        raise SystemExit("expected exactly one calibration copy in the counter run (bench.py --copy-calib)")
    measured_kib = cands[0][1][0]
    return (copy_bytes / 1024.0) / measured_kib


def traffic(fetch_db: str, write_db: str, kernel: str, copy_bytes: int):
    f = counter_per_dispatch(fetch_db, "FETCH_SIZE")
    w = counter_per_dispatch(write_db, "WRITE_SIZE")
    if kernel not in f or kernel not in w:
        raise SystemExit(f"kernel {kernel} not in the counter runs")
    ff, wf = _copy_factor(f, copy_bytes), _copy_factor(w, copy_bytes)
    fk = sum(f[kernel]) / len(f[kernel])
    wk = sum(w[kernel]) / len(w[kernel])
    return {
        "kernel": kernel,
        "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
        "fetch_scale": ff, "write_scale": wf,
        "bytes_per_launch": int(round((fk * ff + wk * wf) * 1024)),
        "copy_bytes": copy_bytes,
    }


# SIMDs of the MI355X (256 CUs x 4), its XCDs (GRBM_GUI_ACTIVE as rocprofv3 reports it is the sum of the 8
# XCDs' active cycles) and the matrix-pipe cycles of one 16x16x32 16-bit MFMA on gfx950
N_SIMD = 1024
N_XCD = 8
MFMA_CYCLES = 16


def counters(dbs, kernels=None):
    """{kernel: {counter: average per dispatch}} over one or more counter runs (one pass per database), and derived
    figures over the kernel's active cycles (GRBM_GUI_ACTIVE / 8 XCDs): the MFMA pipe's busy fraction
    SQ_VALU_MFMA_BUSY_CYCLES / (cycles x SIMDs), the same from the instruction count (SQ_INSTS_MFMA x 16
    cycles), and instructions per wave."""
    out = {}
    for db in dbs:
        con = _con(db)
        rows = con.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection").fetchall()
        per = {}
        for did, kn, cn, v in rows:
            key = (short_name(kn), cn)
            per.setdefault(key, {}).setdefault(did, 0.0)
            per[key][did] += v
        grbm = {}
        for (k, cn), d in per.items():
            if kernels and k not in kernels:
                continue
            avg = sum(d.values()) / len(d)
            if cn == "GRBM_GUI_ACTIVE":
                grbm[k] = avg
            else:
                out.setdefault(k, {})[cn] = avg
        for k, g in grbm.items():
            out.setdefault(k, {}).setdefault("GRBM_GUI_ACTIVE", g)
    for k, c in out.items():
        g = c.get("GRBM_GUI_ACTIVE")
        if g:
            g /= N_XCD
            c["active_cycles"] = g
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                c["mfma_busy_frac"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * N_SIMD)
            if "SQ_INSTS_MFMA" in c:
                c["mfma_issue_frac"] = c["SQ_INSTS_MFMA"] * MFMA_CYCLES / (g * N_SIMD)
        if c.get("SQ_WAVES"):
            for n in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
                if n in c:
                    c[n + "_per_wave"] = c[n] / c["SQ_WAVES"]
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--src-hash", default=None)
    t.add_argument("--out", default=None)
    c = sub.add_parser("counters")
    c.add_argument("dbs", nargs="+")
    c.add_argument("--kernels", nargs="*", default=None)
    c.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        d = counters(a.dbs, a.kernels)
        js = json.dumps(d, indent=1, sort_keys=True)
        if a.out:
            with open(a.out, "w") as fh:
                fh.write(js + "\n")
        print(js)
        return 0
    if a.cmd == "stats":
        print(f"{'kernel':14s} {'calls':>6s} {'total_us':>12s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
        for n, k, tot, avg, mn, mx, pct in kernel_stats(a.db):
            print(f"{n:14s} {k:6d} {tot:12.2f} {avg:10.2f} {mn:10.2f} {mx:10.2f} {pct:6.2f}")
        return 0
    d = traffic(a.fetch, a.write, a.kernel, a.copy_bytes)
    if a.src_hash:
        d["src_hash"] = a.src_hash
    js = json.dumps(d, indent=1)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(js + "\n")
    print(js)
    return 0


if __name__ == "__main__":
    sys.exit(main())
