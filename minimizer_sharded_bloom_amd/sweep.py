"""Parameter sweep of the Super Bloom filter against a per-k-mer blocked Bloom
filter at a fixed memory budget (the synthetic analogue of the (s, m, H)
exploration and the false-positive comparison in "cuSBF: A Minimizer-Aware
Bloom Filter for Genomic Sequence Data on Modern GPUs", §V-B and §V-D).

For every (s, m, H) in {24,26,28,30} x {12,16,20} x {2,3,4,6} at k = 31 and
2^30 bits: insert the 50 Mbp synthetic genome of workload 4, query its 1 M
reads, and count positives among 10^7 random 31-mers.  The blocked Bloom
comparator (one hash picks a 256-bit block, H bits from a second hash) runs
at the same budget for H in {2,3,4,6}, and the wide-block variant (512-bit
blocks, whole-block addressing; §V-D) at ten points around (28, 16, 4).  Prints one JSON line per point and a
summary table.  With --grid: the slices of the wider grid (Fig. 4) through
the operating point -- s = 16..31 at (m, H) = (16, 4), m = 8..31 at
(s, H) = (28, 4), H in {1,2,3,4,5,6,8,12,16} at (m, s) = (16, 28).  With
--grid2d: the whole two-dimensional grid of Fig. 4, s = 16..31 x m = 8..31,
at each H in --h-values (default 4, 8, 12, 16; H > 10 takes the salted bit
address).  Points outside the compiled parameter sets run on the run-time
kernels (sliding insert and query, run-time probe); each row says which.

    python -m minimizer_sharded_bloom_amd.sweep [--probe-n N] [--reps R] [--grid | --grid2d]
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np

from . import SuperBloomFilter, lib, check, packed_words
from . import synthetic as S

K = 31
BITS = 2**30
S_VALUES = (24, 26, 28, 30)
M_VALUES = (12, 16, 20)
H_VALUES = (2, 3, 4, 6)


def _time_ms(torch, stream, fn, reps, before=None):
    """Median kernel time of fn() over reps runs, events on `stream`;
    before(), if given, runs ahead of each timed run outside the events."""
    ts = []
    for _ in range(reps):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def run(probe_n: int = 10_000_000, reps: int = 3, seed: int = 0x5EED, grid: bool = False, out=sys.stdout,
        grid2d: bool = False, h_values=(4, 8, 12, 16)):
    import torch

    torch.cuda.set_device(0)
    w = S.workload(4)
    dev = torch.device("cuda:0")
    genome = torch.from_numpy(w["insert"]).to(dev)
    reads = torch.from_numpy(w["queries"][0]).to(dev)
    L = lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    packs = {}
    for name, t in (("genome", genome), ("reads", reads)):
        cw, vw = packed_words(t.numel())
        c = torch.empty(cw, dtype=torch.int32, device=dev)
        v = torch.empty(vw, dtype=torch.int32, device=dev)
        check(L.sbf_pack(t.data_ptr(), t.numel(), c.data_ptr(), v.data_ptr(), sp), "pack")
        packs[name] = (c, v, t.numel())
    gc, gv, LG = packs["genome"]
    rc, rv, LR = packs["reads"]
    hits_dev = torch.zeros(1, dtype=torch.int64, device=dev)
    rows = []

    def point(f, label):
        out_bits = torch.empty(max(1, f.num_answer_words(LR)), dtype=torch.int64, device=dev)

        def ins():
            check(L.sbf_insert_packed(f.handle, gc.data_ptr(), gv.data_ptr(), LG, sp), "insert")

        # each timed insert starts from a cleared filter; the clear is not timed
        t_ins = _time_ms(torch, stream, ins, reps, before=lambda: check(L.sbf_clear(f.handle, sp), "clear"))
        t_q = _time_ms(torch, stream, lambda: check(
            L.sbf_query_packed(f.handle, rc.data_ptr(), rv.data_ptr(), LR, out_bits.data_ptr(), sp), "query"), reps)
        t_p = _time_ms(torch, stream, lambda: check(
            L.sbf_fpr_probe_device(f.handle, probe_n, seed, hits_dev.data_ptr(), sp), "probe"), reps)
        hits = int(hits_dev.item())
        present = int(np.bitwise_count(out_bits.cpu().numpy().view(np.uint64)).sum())
        row = dict(label, insert_ms=t_ins, query_ms=t_q, probe_ms=t_p,
                   insert_gkmers_s=(LG - K + 1) / t_ins / 1e6, query_gkmers_s=(LR - K + 1) / t_q / 1e6,
                   probe_n=probe_n, hits=hits, fpr=hits / probe_n, specialized=f.specialized,
                   reads_positive_kmers=present)
        rows.append(row)
        print(json.dumps(row), file=out, flush=True)

    if grid2d:
        for H in h_values:
            for s in range(16, 32):
                for m in range(8, 32):
                    with SuperBloomFilter(K, m, s, H, BITS) as f:
                        point(f, {"kind": "grid2d", "s": s, "m": m, "H": H})
        return rows
    if grid:
        for kind, pts in (("slice_s", [(16, s, 4) for s in range(16, 32)]),
                          ("slice_m", [(m, 28, 4) for m in range(8, 32)]),
                          ("slice_h", [(16, 28, H) for H in (1, 2, 3, 4, 5, 6, 8, 12, 16)])):
            for m, s, H in pts:
                with SuperBloomFilter(K, m, s, H, BITS) as f:
                    point(f, {"kind": kind, "s": s, "m": m, "H": H})
        return rows
    for s in S_VALUES:
        for m in M_VALUES:
            for H in H_VALUES:
                with SuperBloomFilter(K, m, s, H, BITS) as f:
                    point(f, {"kind": "sbf", "s": s, "m": m, "H": H})
    for H in H_VALUES:
        with SuperBloomFilter.blocked(K, H, BITS) as f:
            point(f, {"kind": "bbf", "s": None, "m": None, "H": H})
    for m, s, H in [(16, 24, 4), (16, 26, 4), (16, 28, 4), (16, 30, 4), (16, 28, 2), (16, 28, 3), (16, 28, 6),
                    (16, 28, 8), (12, 28, 4), (20, 28, 4)]:
        with SuperBloomFilter.wide(K, m, s, H, BITS) as f:
            point(f, {"kind": "wide", "s": s, "m": m, "H": H})
    return rows


def grid_tables(rows) -> str:
    """Two-dimensional maps (rows s, columns m) per H of the FPR and of the
    insert and query rates, from --grid2d rows; '*' marks the points served
    by compiled (specialized) kernels."""
    out = []
    for H in sorted({r["H"] for r in rows}):
        rs = {(r["s"], r["m"]): r for r in rows if r["H"] == H}
        ms = sorted({m for _, m in rs})
        ss = sorted({s for s, _ in rs})
        for key, title, fmt in (("fpr", "FPR on 10^7 random 31-mers", "%.2g"),
                                ("insert_gkmers_s", "insert Gk-mers/s (k-mer starts)", "%.0f"),
                                ("query_gkmers_s", "query Gk-mers/s (k-mer starts)", "%.0f")):
            out.append("\nH = %d: %s ('*' = compiled kernel set)\n" % (H, title))
            out.append("| s \\ m | " + " | ".join(str(m) for m in ms) + " |")
            out.append("|---|" + "---:|" * len(ms))
            for s_ in ss:
                cells = []
                for m in ms:
                    r = rs.get((s_, m))
                    cells.append("" if r is None else (fmt % r[key]) + ("*" if r["specialized"] else ""))
                out.append("| %d | " % s_ + " | ".join(cells) + " |")
    return "\n".join(out)


def table(rows) -> str:
    lines = ["| kind | s | m | H | insert Gk-mers/s | query Gk-mers/s | FPR (random 31-mers) | specialized |",
             "|---|---|---|---|---:|---:|---:|---|"]
    for r in rows:
        lines.append("| %s | %s | %s | %d | %.1f | %.1f | %.3g | %s |" % (
            r["kind"], r["s"] if r["s"] else "-", r["m"] if r["m"] else "-", r["H"],
            r["insert_gkmers_s"], r["query_gkmers_s"], r["fpr"], "yes" if r["specialized"] else "no"))
    return "\n".join(lines)


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--probe-n", type=int, default=10_000_000)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--grid", action="store_true",
                    help="instead: the s-, m- and H-slices through (s, m, H) = (28, 16, 4)")
    ap.add_argument("--grid2d", action="store_true",
                    help="instead: the full s = 16..31 x m = 8..31 grid at each H of --h-values")
    ap.add_argument("--h-values", default="4,8,12,16", help="H values of --grid2d (comma-separated)")
    a = ap.parse_args()
    t0 = time.time()
    rows = run(a.probe_n, a.reps, grid=a.grid, grid2d=a.grid2d,
               h_values=tuple(int(x) for x in a.h_values.split(",")))
    print(grid_tables(rows) if a.grid2d else table(rows))
    print("sweep wall time %.1f s" % (time.time() - t0), file=sys.stderr)
