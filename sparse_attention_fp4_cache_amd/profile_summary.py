"""Short text summaries of rocprofv3 output for the library's kernels.

  python -m sparse_attention_fp4_cache_amd.profile_summary stats STATS_CSV --command "..."
      per-kernel calls and durations from a `--kernel-trace --stats` run.

  python -m sparse_attention_fp4_cache_amd.profile_summary traffic \
        --fetch FETCH_DIR --write WRITE_DIR --copy-mib N --workload NAME \
        --bytes-per-launch B --command-fetch "..." --command-write "..."
      Bytes per launch of the indexer scan that missed the L2 (to the fabric: the
      MALL or HBM; FETCH_SIZE cannot tell them apart), from two counter passes
      (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by what the
      same counter reads for a plain copy kernel of known size run in the same
      process (it reads N bytes and writes N bytes).

  python -m sparse_attention_fp4_cache_amd.profile_summary counters PMC_DIR \
        --counters A,B,... --kernels K1,K2,... --command "..."
      Mean per dispatch of each named counter for each named kernel (substring
      match), from one `--pmc` run; derived counters (MfmaUtil) are one value per
      dispatch, hardware counters are summed over their dimensions.

Only reads CSV files; touches no GPU.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import sys

SCAN_KERNEL = "index_score_kernel<4, 1, true, false, false>"  # the indexer stage's scan (64 heads, one query)
COPY_KERNEL = "MulFunctor"  # torch's elementwise multiply, used as a read-N/write-N copy


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(names)


def _short(name: str, width: int = 62) -> str:
    short = name.split("(")[0].replace("void ", "")
    return short if len(short) <= width else short[:width - 3] + "..."


def stats(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# rocprofv3 kernel statistics", f"# command: {command}", "#",
           f"{'kernel':64s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_%':>8s}"]
    for r in rows:
        name = _col(r, "Name", "KERNEL_NAME", "Kernel_Name")
        short = name.split("(")[0].replace("void ", "")
        if len(short) > 64:
            short = short[:61] + "..."
        calls = int(_col(r, "Calls"))
        avg = float(_col(r, "AverageNs")) / 1e3
        mn = float(_col(r, "MinNs")) / 1e3
        mx = float(_col(r, "MaxNs")) / 1e3
        pct = float(_col(r, "Percentage"))
        out.append(f"{short:64s} {calls:6d} {avg:9.2f} {mn:9.2f} {mx:9.2f} {pct:8.2f}")
    return "\n".join(out) + "\n"


def _per_dispatch(dirpath: str, counter: str):
    """{kernel name: [value per dispatch]} summed over counter dimensions."""
    files = glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {dirpath}")
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    for f in files:
        for r in csv.DictReader(open(f)):
            if _col(r, "Counter_Name", "Counter-Name") != counter:
                continue
            disp = _col(r, "Dispatch_Id", "Dispatch-Id", "Correlation_Id")
            acc[_col(r, "Kernel_Name", "Kernel-Name")][(f, disp)] += float(_col(r, "Counter_Value", "Counter-Value"))
    return {k: list(v.values()) for k, v in acc.items()}


def _pick(per, key):
    vals = [v for name, lst in per.items() if key in name for v in lst]
    if not vals:
        raise ValueError(f"no dispatch of a kernel named like {key!r}")
    return vals


def traffic(a) -> str:
    fetch = _per_dispatch(a.fetch, "FETCH_SIZE")
    write = _per_dispatch(a.write, "WRITE_SIZE")
    copy_kib = a.copy_mib * 1024.0
    cf = _pick(fetch, COPY_KERNEL)
    cw = _pick(write, COPY_KERNEL)
    f_fetch = copy_kib / max(cf)  # the largest multiply is the calibration copy
    f_write = copy_kib / max(cw)
    sf = _pick(fetch, a.kernel)
    sw = _pick(write, a.kernel)
    fetch_b = sum(sf) / len(sf) * 1024.0 * f_fetch
    write_b = sum(sw) / len(sw) * 1024.0 * f_write
    lines = [
        f"# L2-miss (fabric) traffic of the indexer scan ({a.kernel}) on workload {a.workload}",
        "# two rocprofv3 counter passes over the same benchmark command, FETCH_SIZE then WRITE_SIZE",
        "# (KiB per dispatch), each scaled by the same counter on a plain copy of known size;",
        "# bytes served by the MALL count here as well as bytes from HBM",
        f"command_fetch: {a.command_fetch}",
        f"command_write: {a.command_write}",
        f"kernel_source_sha256: {a.source_hash}",
        f"copy_probe_bytes_each_way: {int(copy_kib * 1024)}",
        f"copy_fetch_kib_measured: {max(cf):.1f}",
        f"copy_write_kib_measured: {max(cw):.1f}",
        f"fetch_scale: {f_fetch:.4f}",
        f"write_scale: {f_write:.4f}",
        f"scan_dispatches: {len(sf)} / {len(sw)}",
        f"scan_fetch_kib_per_dispatch: {sum(sf) / len(sf):.1f}",
        f"scan_write_kib_per_dispatch: {sum(sw) / len(sw):.1f}",
        f"scan_fetch_bytes_per_launch: {fetch_b:.0f}",
        f"scan_write_bytes_per_launch: {write_b:.0f}",
        f"algorithmic_bytes_per_launch: {a.bytes_per_launch}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"traffic_over_algorithmic: {(fetch_b + write_b) / a.bytes_per_launch:.3f}",
        "#",
        "# every kernel of the run: mean L2-miss bytes per dispatch (scaled as above)",
        f"# {'kernel':62s} {'calls':>6s} {'fetch_bytes':>13s} {'write_bytes':>13s}",
    ]
    for name in sorted(set(fetch) & set(write), key=lambda n: -sum(fetch[n]) / len(fetch[n])):
        f_, w_ = fetch[name], write[name]
        lines.append(f"# {_short(name):62s} {len(f_):6d} {sum(f_) / len(f_) * 1024 * f_fetch:13.0f} "
                     f"{sum(w_) / len(w_) * 1024 * f_write:13.0f}")
    return "\n".join(lines) + "\n"


def counters(a) -> str:
    names = [c for c in a.counters.split(",") if c]
    kernels = [k for k in a.kernels.split(",") if k]
    per = {c: _per_dispatch(a.dir, c) for c in names}
    lines = [f"# rocprofv3 counters, mean per dispatch", f"# command: {a.command}", "#",
             f"{'kernel':48s} {'calls':>6s} " + " ".join(f"{c:>30s}" for c in names)]
    for k in kernels:
        cols, calls = [], 0
        for c in names:
            vals = _pick(per[c], k)
            calls = len(vals)
            cols.append(f"{sum(vals) / len(vals):30.6g}")
        lines.append(f"{_short(k, 48):48s} {calls:6d} " + " ".join(cols))
    return "\n".join(lines) + "\n"


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--bytes-per-launch", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--source-hash", required=True)
    t.add_argument("--kernel", default=SCAN_KERNEL)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--counters", required=True)
    c.add_argument("--kernels", required=True)
    c.add_argument("--command", required=True)
    a = p.parse_args(argv)
    out = {"stats": lambda: stats(a.csv, a.command), "traffic": lambda: traffic(a),
           "counters": lambda: counters(a)}[a.cmd]()
    sys.stdout.write(out)


if __name__ == "__main__":
    main()
