"""Memory-side ceilings of the filter's two access patterns on this GPU, by
table size: random 32-byte shard reads (the query's and probe's access) and
random 32-byte shard OR-updates in three forms (the insert's flush is the
first): a device-scope atomic OR, a workgroup-scope atomic OR and a plain
load-OR-store, each over the whole table and confined per workgroup to one
eighth of it (the eighth its XCD would own under round-robin dispatch).
Measurement support for the speed-of-light analysis of "cuSBF: A
Minimizer-Aware Bloom Filter for Genomic Sequence Data on Modern GPUs"
§V-E; nothing here is part of the method.

    python -m minimizer_sharded_bloom_amd.ceilings [--ops N]

Prints one JSON line per table size (G operations/s, median of 3 runs after
one warm-up) and a markdown table.
"""
from __future__ import annotations

import argparse
import json
import sys

from . import check, lib

SIZES = (1 << 20, 4 << 20, 32 << 20, 256 << 20, 512 << 20, 4 << 30)
FORMS = (("atomic, device scope", 0), ("atomic, device scope, XCD eighth", 4), ("atomic, workgroup scope", 1),
         ("atomic, workgroup scope, XCD eighth", 5), ("plain load/OR/store", 2), ("plain, XCD eighth", 6))


def run(n_ops: int = 1 << 25, out=sys.stdout):
    import torch

    torch.cuda.set_device(0)
    L = lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    table = torch.zeros(max(SIZES) // 8, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int64, device="cuda")
    rows = []

    def rate(call):
        ts = []
        for rep in range(4):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            check(call(rep), "membench")
            b.record(stream)
            b.synchronize()
            if rep:
                ts.append(a.elapsed_time(b))
        ts.sort()
        return n_ops / (ts[1] * 1e-3) / 1e9

    for size in SIZES:
        nsh = size // 32
        row = {"table_bytes": size}
        row["reads"] = rate(lambda r: L.sbf_membench_shard_reads(table.data_ptr(), nsh, n_ops, 17 + r,
                                                                 sink.data_ptr(), sp))
        for name, mode in FORMS:
            row[name] = rate(lambda r, m=mode: L.sbf_membench_shard_rmw(table.data_ptr(), nsh, n_ops, 23 + r, m, sp))
        rows.append(row)
        print(json.dumps(row), file=out, flush=True)
    return rows


def table(rows) -> str:
    cols = ["reads"] + [f for f, _ in FORMS]
    lines = ["| table | random 32 B reads | " + " | ".join("OR-update: " + c for c in cols[1:]) + " |",
             "|---:|" + "---:|" * len(cols)]
    for r in rows:
        size = r["table_bytes"]
        label = "%d MiB" % (size >> 20) if size < (1 << 30) else "%d GiB" % (size >> 30)
        lines.append("| %s | " % label + " | ".join("%.1f" % r[c] for c in cols) + " |")
    return "\n".join(lines)


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--ops", type=int, default=1 << 25)
    a = ap.parse_args()
    print(table(run(a.ops)))
