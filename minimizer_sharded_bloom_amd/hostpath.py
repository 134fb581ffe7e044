"""Host-resident input throughput on one MI355X, next to device-resident
input (the analogue of "cuSBF: A Minimizer-Aware Bloom Filter for Genomic
Sequence Data on Modern GPUs", §V-F, Fig. 8: throughput lost to host-device
transfer), plus FASTA/FASTQ files end to end (§IV-A, §IV-G).

On the configuration-3 workload (200 Mbp genome, 2^32-bit filter, 20 M reads
of 150 bp), at k=31, m=16, s=28, H=4:
  device   sequence already in HBM: insert / query, each kernel decoding
           the ASCII itself
  host     sequence in pageable host memory: the chunked pinned pipeline
  fasta    the genome as a FASTA file (plain, gzip, then BGZF, whose members the
           reader inflates on several threads) through sbf_insert_fastx
  fastq    2 M of the reads as a FASTQ file through sbf_query_fastx
and the raw host-to-device copy rate from pinned memory.  One JSON line per
measurement, then a table.

    python -m minimizer_sharded_bloom_amd.hostpath [--reps R] [--tmp DIR] [--chunk N] [--sweep N,N,...]
"""
from __future__ import annotations

import argparse
import gzip
import json
import os
import sys
import time

import numpy as np

from . import SuperBloomFilter
from . import synthetic as S

K, M_, S_, H_ = 31, 16, 28, 4


def _best(fn, reps):
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return min(ts)


def run(reps: int = 3, tmp: str = "/tmp", chunk: int | None = None, sweep=None, out=sys.stdout):
    import torch

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = S.workload(3)
    genome, reads = w["insert"], w["queries"][0]
    rows = []

    def emit(**kw):
        rows.append(kw)
        print(json.dumps(kw), file=out, flush=True)

    f = SuperBloomFilter(K, M_, S_, H_, w["bits"])
    if chunk:
        f.set_staging(chunk)
    nk_g, nk_r = genome.size - K + 1, reads.size - K + 1

    # raw host-to-device copy rate (pinned source)
    pinned = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dbuf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def h2d():
        dbuf.copy_(pinned, non_blocking=True)
        torch.cuda.synchronize()
    t = _best(h2d, reps)
    emit(what="h2d_pinned_copy", gbytes_s=(1 << 30) / t / 1e9)
    del pinned, dbuf

    # device-resident (sequence-native calls on device tensors: pack + kernel)
    g_dev = torch.from_numpy(genome).to(dev)
    r_dev = torch.from_numpy(reads).to(dev)
    out_dev = torch.empty(f.num_answer_words(reads.size), dtype=torch.int64, device=dev)

    def dev_insert():
        f.clear()
        f.insert_seq(g_dev)
        torch.cuda.synchronize()

    def dev_query():
        f.query_seq(r_dev, out=out_dev)
        torch.cuda.synchronize()
    t_clear = _best(lambda: (f.clear(), torch.cuda.synchronize()), reps)
    emit(what="device_insert", gkmers_s=nk_g / (_best(dev_insert, reps) - t_clear) / 1e9)
    emit(what="device_query", gkmers_s=nk_r / _best(dev_query, reps) / 1e9)
    del g_dev, r_dev, out_dev
    torch.cuda.empty_cache()

    # host-resident (pageable numpy arrays through the pipeline)
    def host_insert():
        f.clear()
        f.insert_seq(genome)
    for c in sweep or [None]:
        if c:
            f.set_staging(c)
        tag = {} if c is None else {"chunk": c}
        t = _best(host_insert, reps) - t_clear
        emit(what="host_insert", gkmers_s=nk_g / t / 1e9, gbytes_s_in=genome.size / t / 1e9, **tag)
        t = _best(lambda: f.query_seq(reads), reps)
        emit(what="host_query", gkmers_s=nk_r / t / 1e9, gbytes_s_in=reads.size / t / 1e9, **tag)
    if chunk:
        f.set_staging(chunk)

    # FASTA / FASTQ files
    fa = os.path.join(tmp, "sbf_hostpath_genome.fa")
    fagz = fa + ".gz"
    fabgz = fa + ".bgz"
    fq = os.path.join(tmp, "sbf_hostpath_reads.fq")
    t0 = time.perf_counter()
    fa_bytes = S.fasta_bytes(genome)
    fa_bytes.tofile(fa)
    with gzip.open(fagz, "wb", compresslevel=1) as g:
        g.write(fa_bytes.tobytes())
    with open(fabgz, "wb") as g:
        g.write(S.bgzf_bytes(fa_bytes.tobytes(), level=1))
    nreads = 2_000_000
    r2d = reads[: nreads * (S.READ_LEN + 1)].reshape(nreads, S.READ_LEN + 1)[:, : S.READ_LEN]
    S.fastq_bytes(np.ascontiguousarray(r2d)).tofile(fq)
    emit(what="files_written", seconds=time.perf_counter() - t0, fasta_bytes=os.path.getsize(fa),
         fasta_gz_bytes=os.path.getsize(fagz), fasta_bgzf_bytes=os.path.getsize(fabgz), fastq_bytes=os.path.getsize(fq))
    try:
        for path, label in ((fa, "fasta_insert"), (fagz, "fasta_gz_insert"), (fabgz, "fasta_bgzf_insert")):
            best = None
            for _ in range(reps):
                f.clear()
                st = f.insert_fastx(path)
                if best is None or st["total_seconds"] < best["total_seconds"]:
                    best = st
            emit(what=label, gkmers_s=nk_g / best["total_seconds"] / 1e9,
                 file_mbytes_s=os.path.getsize(path) / best["total_seconds"] / 1e6, **best)
        nk_q = nreads * (S.READ_LEN - K + 1)
        best = None
        for _ in range(reps):
            hits, kmers, st = f.query_fastx(fq, max_records=nreads)
            if best is None or st["total_seconds"] < best["total_seconds"]:
                best = st
        assert int(kmers.sum()) == nk_q
        emit(what="fastq_query", gkmers_s=nk_q / best["total_seconds"] / 1e9,
             file_mbytes_s=os.path.getsize(fq) / best["total_seconds"] / 1e6, **best)
    finally:
        for p in (fa, fagz, fabgz, fq):
            if os.path.exists(p):
                os.remove(p)
    f.close()
    return rows


def table(rows) -> str:
    lines = ["| measurement | rate |", "|---|---:|"]
    for r in rows:
        if "gkmers_s" in r:
            extra = "" if "parse_seconds" not in r else " (parse %.2f s of %.2f s)" % (r["parse_seconds"],
                                                                                    r["total_seconds"])
            if "chunk" in r:
                extra += " (chunk %d)" % r["chunk"]
            lines.append("| %s | %.1f Gk-mers/s%s |" % (r["what"], r["gkmers_s"], extra))
        elif "gbytes_s" in r:
            lines.append("| %s | %.1f GB/s |" % (r["what"], r["gbytes_s"]))
    return "\n".join(lines)


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--tmp", default="/tmp")
    ap.add_argument("--chunk", type=int, default=0, help="pipeline chunk (k-mer starts); 0 = library default")
    ap.add_argument("--sweep", default="", help="comma-separated chunk sizes for the host-memory measurements")
    a = ap.parse_args()
    rows = run(a.reps, a.tmp, a.chunk or None, [int(x) for x in a.sweep.split(",") if x])
    print(table(rows))
