#!/usr/bin/env python3
"""Benchmark of the Super Bloom filter hot path on one MI355X.

One step = one pass of the whole path over one batch of device-resident
synthetic input (the method of "cuSBF: A Minimizer-Aware Bloom Filter for
Genomic Sequence Data on Modern GPUs"):
    clear the filter
    insert every genome k-mer           (Algorithm 1), the insert kernel
                                        decoding the genome's ASCII itself
    query every read k-mer              (Algorithm 2), the query kernel
                                        decoding the reads' ASCII itself
    false-positive probe of n random k-mers (§V-D)
at k=31, m=16, s=28, H=4.  The reads of workloads 2-4 all have 150 bases:
they are queried read by read (sbf_query_reads), so no lane works on the
starts that straddle two reads.  (`--query-input text` queries them as one
'N'-joined sequence instead, `--query-input packed` packs that sequence in a
pass of its own and queries the packed codes; `--insert-input packed` packs
the genome in a pass of its own before the insert.)  Every launch goes to
torch's current stream, so the torch events recorded between launches time
each kernel on the stream it runs on.

The default workload is configuration 3: a 2^32-bit (512 MiB) filter, out of
every on-chip cache, a 200 Mbp genome inserted and 20 M reads of 150 bp
queried.  Before the warm-up steps the step is repeated, untimed, for
--prewarm-s seconds (default 1.5 s): the engine clock takes a fraction of a
second of load to settle, and a short run would otherwise time part of that
ramp.

Prints one JSON line.  `value` = valid k-mers processed per second over the
step: (valid genome k-mers + valid read k-mers + probe k-mers) / step time,
where a k-mer is valid when all of its bases are A, C, G or T; positions
whose k-mer spans a record separator are not counted ("kmer_starts" and the
*_starts_gkmers_s fields give the rates over all positions).

`--alphabet protein|triplet` times the same step over the protein (k=12,
m=6, s=10, H=4) or DNA-triplet (k=10, m=5, s=8, H=4) filter on its synthetic
workload (16 M symbols inserted into 2^28 bits, 2 M queries); those kernels
read the ASCII text directly, so the step has no pack launches.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

T0 = time.perf_counter()

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

K, M_, S_, H_ = 31, 16, 28, 4
METRIC = "insert & query Gk-mers/s (k=31,m=16,s=28,H=4) + fraction of HBM/L2 roofline"

# MI355X ALU peak from unit counts and clock: 256 CUs x 4 SIMDs.  A SIMD
# issues a wave64 instruction of the two-operand 32-bit kind (logic, add,
# shift on VGPRs, with at most a literal or inline constant; also bitop3 on
# three VGPRs) every 2 clocks, 32 lanes per clock, so the chip retires
# 256 * 4 * 32 lane-instructions per clock: 7.86e13 per second at 2.4 GHz,
# the fp32 vector rate (157.3 TFLOP/s counting an FMA as two).  64-bit
# shifts, compares and multiply-adds, 32-bit multiplies, three-input adds
# and shifts, alignbit, perm, bcnt, DPP moves and any form that reads an
# SGPR take 4 clocks: half that rate, the fp64 one.  matched_ceilings()
# measures both rates on the machine it runs on (sbf_membench_valu).
CUS, CLOCK_HZ = 256, 2.4e9
ALU_PEAK = CUS * 4 * 32 * CLOCK_HZ  # 7.86e13 lane-instructions/s
HBM_PEAK = 8.0e12               # bytes/s

# Algorithmic integer work per k-mer start at (k,m,s,H) = (31,16,28,4), in
# 32-bit VALU instructions, for the sliding formulation (each position hashes
# one m-mer and one s-mer; the minimizer is a sliding minimum; the Findere
# mask of a k-mer is one new doubling level per s-mer).
FRONT = {
    "m-mer window (funnel shift)": 1,
    "h_min: 32x64 multiply with folded offset (2 mad_u64), carry move, fold": 4,
    "sliding minimum: 3 x (64-bit compare + 2 selects)": 9,
    "shard mask": 1,
    "s-mer window (2 funnel shifts + shift)": 3,
    "h_s: 64-bit add, 3 x (64-bit shift + 2 xor), 2 x (2 mul_lo + mad_u64 + add3)": 18,
    "H=4 bit masks of the new s-mer (2 slice shifts + 4 64-bit shifts)": 6,
    "one new doubling level of the s-mer masks (4 words x 2 halves)": 8,
    "validity / run bookkeeping": 2,
}
TAIL = {
    "query": {"(T0|T1) & ~W per half (bitop3), one 64-bit compare per word, answer bit": 13},
    # a query that decodes its reads from ASCII (one base per k-mer start)
    "query_text": {"(T0|T1) & ~W per half (bitop3), one 64-bit compare per word, answer bit": 13,
                   "base from ASCII: 2 shifts + bitop3 code, multiply gather, letter lookup, "
                   "masked compare, add, flag (8 per 4 bases); 21 gathers per 32 bases": 2.66},
    "insert": {"T0|T1 and (Wr & keep) | t per half": 16, "record flush share (~0.12 runs/k-mer)": 1.5},
    # an insert that decodes its genome from ASCII, the same per base
    "insert_text": {"T0|T1 and (Wr & keep) | t per half": 16, "record flush share (~0.12 runs/k-mer)": 1.5,
                    "base from ASCII: 2 shifts + bitop3 code, multiply gather, letter lookup, "
                    "masked compare, add, flag (8 per 4 bases); 21 gathers per 32 bases": 2.66},
}


def alu_ops_per_kmer(kind: str) -> float:
    return float(sum(FRONT.values()) + sum(TAIL[kind].values()))


# How many of those instructions are of the forms that issue every 4 clocks,
# half the rate of the simple two-operand 32-bit forms (measured on the
# device: 64-bit shifts, compares and multiply-adds, 32-bit multiplies,
# alignbit, perm, v_cndmask, VOPC compares, DPP moves and anything reading an
# SGPR; xor/or/and/bitop3/shift-by-immediate on VGPRs issue every 2).  Per
# item of FRONT and TAIL, in the same order: the m-mer window is one
# alignbit; h_min two 64-bit multiply-adds (plus a move and a fold xor);
# the sliding minimum's 64-bit compares and selects all; the shard mask reads
# an SGPR; the s-mer window two alignbits; h_s its 64-bit add of G, three
# 64-bit shifts and both multiplies (2 mul_lo + mad_u64 + add3 each); the bit
# masks four 64-bit shifts; the doubling ORs none; the run bookkeeping a
# compare and a carry-in add.
FRONT_4CLK = (1, 2, 9, 1, 2, 12, 4, 0, 2)
TAIL_4CLK = {
    "query": (5,),                 # four 64-bit compares and the carry-in add; the bitop3s issue every 2
    "query_text": (5, 0.91),       # + per base: the multiply and perm of the code gather, perms of the flags
    "insert": (0, 1.5),            # ORs and bitop3s every 2; the record flush's atomics and address math
    "insert_text": (0, 1.5, 0.91),
}


def alu_issue_slots_per_kmer(kind: str) -> float:
    """The algorithmic instructions of alu_ops_per_kmer in 2-clock issue
    slots: a 4-clock form occupies two.  Against the same peak (one slot =
    one lane-instruction of the 2-clock forms) this is the share of the
    VALU's issue capacity the algorithm itself needs."""
    assert len(FRONT_4CLK) == len(FRONT) and len(TAIL_4CLK[kind]) == len(TAIL[kind])
    return alu_ops_per_kmer(kind) + float(sum(FRONT_4CLK) + sum(TAIL_4CLK[kind]))


# Other alphabets: the DNA kernels' work per k-mer start (windows cut from a
# packed stream, here 5- or 6-bit symbols packed in registers) plus decoding
# the symbol from ASCII in the kernel's text front end.
ALPHAS = {
    "protein": {"params": (12, 6, 10, 4), "bytes_per_symbol": 1,
                "decode": {"letter: SWAR codes, letter test and flag bits over 4 bytes (1/4 each), "
                           "5-bit field into the packed word": 5.5}},
    "triplet": {"params": (10, 5, 8, 4), "bytes_per_symbol": 3,
                "decode": {"codon: SWAR 2-bit codes and validity of its 3 bases (4.25 each), codon flag": 15.75}},
}


def alpha_alu_ops_per_kmer(alpha: str, kind: str) -> float:
    return float(sum(FRONT.values()) + sum(ALPHAS[alpha]["decode"].values()) + sum(TAIL[kind].values()))


def alpha_bytes_per_kmer(alpha: str, kind: str) -> float:
    """Text bytes of one symbol streamed once, one 32-byte shard read per run
    (a write-back too for an insert), a query's answer bit."""
    k, m = ALPHAS[alpha]["params"][:2]
    runs = 2.0 / (k - m + 2)
    b = ALPHAS[alpha]["bytes_per_symbol"]
    return b + 0.125 + 32 * runs if kind == "query" else b + 64 * runs


def _bytes_per_kmer(kind: str, w: int = K - M_ + 1) -> float:
    """Algorithmic HBM bytes per k-mer start: packed codes (2 bits) and
    validity (1 bit) streamed once, plus one 32-byte shard read per run of
    equal shards (and one 32-byte write-back per run for an insert); a query
    also writes its answer bit.  Random minimizers give 2/(w+1) runs per k-mer."""
    runs = 2.0 / (w + 1)
    seq = 0.25 + 0.125
    if kind == "query_text":  # one ASCII byte per base instead
        return 1.0 + 0.125 + 32 * runs
    if kind == "query":
        return seq + 0.125 + 32 * runs
    if kind == "insert_text":
        return 1.0 + 64 * runs
    return seq + 64 * runs


CSRC = os.path.join(ROOT, "minimizer_sharded_bloom_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# Sources each workload family's kernels are built from: the DNA step's
# pack/clear kernels and the specialized set at (31,16,28,4), or the alphabet
# kernels (their insert and query are sbf_spec.hpp's with a text front end).  A traffic summary is used only while these hash as when it was
# taken.
KERNEL_SOURCES = {
    "dna": ("minimizer_sharded_bloom_amd/csrc/inst_m16.hip", "minimizer_sharded_bloom_amd/csrc/sbf_spec.hpp",
            "minimizer_sharded_bloom_amd/csrc/sbf_spec_list.hpp", "minimizer_sharded_bloom_amd/csrc/sbf_device.hpp",
            "minimizer_sharded_bloom_amd/csrc/sbf_internal.hpp", "minimizer_sharded_bloom_amd/csrc/sbf_generic.hip"),
    "alpha": ("minimizer_sharded_bloom_amd/csrc/sbf_alpha.hip", "minimizer_sharded_bloom_amd/csrc/sbf_spec.hpp",
              "minimizer_sharded_bloom_amd/csrc/sbf_device.hpp", "minimizer_sharded_bloom_amd/csrc/sbf_internal.hpp",
              "minimizer_sharded_bloom_amd/csrc/sbf_generic.hip", "include/sbf.h"),
}


def kernel_sources_sha256(family: str = "dna") -> str:
    """Hash of the sources (names and bytes) that one family's kernels are
    built from (KERNEL_SOURCES)."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        h.update(rel.encode() + b"\0")
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str, sha: str):
    """HBM bytes per launch of `kernel` on `workload` from the rocprofv3
    FETCH_SIZE / WRITE_SIZE summaries under profiles/ (already scaled by the
    copy-kernel calibration), or None when no summary was taken at the
    current kernel sources."""
    if not os.path.isdir(PROFILES):
        return None
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith("_traffic.md"):
            continue
        kv = {}
        with open(os.path.join(PROFILES, name)) as f:
            for line in f:
                key, sep, val = line.strip().partition(":")
                if sep and line.startswith("    ") and key.replace("_", "").isalnum() and key.islower():
                    kv[key] = val.strip()
        if kv.get("workload") != workload or kv.get("kernel_sources_sha256") != sha:
            continue
        fetch, write = kv.get("%s_fetch_bytes" % kernel), kv.get("%s_write_bytes" % kernel)
        if fetch is not None and write is not None:
            return {"bytes": float(fetch) + float(write), "fetch": float(fetch), "write": float(write),
                    "source": "profiles/" + name}
    return None


def filter_level(nbytes: int) -> str:
    """Where a filter of nbytes lives once warm: within the 4 MB L2 of one
    XCD ("l2": every XCD sees the whole filter), within the 256 MB MALL
    ("mall"), else HBM ("hbm"); the memory fraction is against the 8 TB/s
    HBM peak in every case, and is only a bound for "hbm"."""
    if nbytes <= 4 << 20:
        return "l2"
    if nbytes <= 256 << 20:
        return "mall"
    return "hbm"


def valid_kmer_count(text, k: int, alpha: str = "dna", chunk: int = 3 << 26, segments: bool = False):
    """k-mer starts whose k symbols are all valid (positions with an invalid
    symbol, e.g. a record separator, are not): the throughput count of valid
    k-mers, next to the count of k-mer starts.  Counted chunk by chunk, with
    the valid run that crosses a chunk boundary carried over.  With
    segments=True also the number of maximal stretches of valid symbols that
    hold at least one k-mer, as (count, segments)."""
    import numpy as np

    ok = np.zeros(256, dtype=bool)
    if alpha == "protein":
        ok[[c for c in range(256) if ord("a") <= (c | 0x20) <= ord("z")]] = True
    else:
        ok[list(b"ACGTacgt")] = True
    sb = 3 if alpha == "triplet" else 1
    n_sym = text.size // sb
    total, cur, nseg = 0, 0, 0
    for lo in range(0, n_sym, chunk):
        hi = min(n_sym, lo + chunk)
        v = ok[text[lo * sb:hi * sb]]
        if sb > 1:
            v = v.reshape(hi - lo, sb).all(axis=1)
        bad = np.flatnonzero(~v)
        if bad.size == 0:
            cur += hi - lo
            continue
        total += max(0, cur + int(bad[0]) - k + 1)
        nseg += cur + int(bad[0]) >= k
        gaps = np.diff(bad) - 1  # stretches between invalid symbols
        total += int(np.maximum(gaps - k + 1, 0).sum())
        nseg += int((gaps >= k).sum())
        cur = hi - lo - 1 - int(bad[-1])
    total += max(0, cur - k + 1)
    nseg += cur >= k
    return (total, int(nseg)) if segments else total


def matched_ceilings(lib, torch, filt, stream, n_ops: int = 1 << 25) -> dict:
    """Random 32-byte shard reads over the filter itself and random 32-byte
    shard OR-updates (four lanes, one 64-bit atomic each) over a scratch table
    of the same size, in G operations/s (median of 3 after one warm-up):
    the memory ceilings the query / probe and the insert flush can reach.
    Also the VALU issue rate of a 2-clock and a 4-clock instruction form on
    this machine, the two ceilings of the ALU roofline."""
    n_sh = filt.num_shards
    table = lib.sbf_filter_device_ptr(filt.handle)
    scratch = torch.zeros(4 * n_sh, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int64, device="cuda")
    sp = stream.cuda_stream
    out = {"table_bytes": 32 * n_sh, "ops": n_ops}
    for name, call in (("shard_reads_g_per_s",
                        lambda seed: lib.sbf_membench_shard_reads(table, n_sh, n_ops, seed, sink.data_ptr(), sp)),
                       ("shard_ors_g_per_s",
                        lambda seed: lib.sbf_membench_shard_ors(scratch.data_ptr(), n_sh, n_ops, seed, sp))):
        ts = []
        for rep in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = call(0xC0FFEE + rep)
            e1.record(stream)
            if rc != 0:
                raise RuntimeError("%s failed (%d)" % (name, rc))
            torch.cuda.synchronize()
            if rep:
                ts.append(e0.elapsed_time(e1))
        ts.sort()
        out[name] = round(n_ops / (ts[1] * 1e-3) / 1e9, 3)
    del scratch
    # VALU issue rates of the 2-clock and 4-clock instruction forms, in
    # T lane-instructions/s (8192 workgroups x 256 lanes x 8 x iters)
    iters = 2048
    lane_instr = 8192 * 256 * 8 * iters
    for name, kind in (("valu_2clk_t_lane_instr_per_s", 0), ("valu_4clk_t_lane_instr_per_s", 1)):
        ts = []
        for rep in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.sbf_membench_valu(kind, iters, sink.data_ptr(), sp)
            e1.record(stream)
            if rc != 0:
                raise RuntimeError("%s failed (%d)" % (name, rc))
            torch.cuda.synchronize()
            if rep:
                ts.append(e0.elapsed_time(e1))
        ts.sort()
        out[name] = round(lane_instr / (ts[1] * 1e-3) / 1e12, 2)
    return out


def timed_steps(torch, step, n_phases: int, a):
    """a.warmup untimed steps, then exactly a.steps timed steps between two
    events on the current stream, bracketed by device synchronizations, with
    events recorded between the launches of every timed step on the stream
    the kernels run on.  Returns (ms per step, wall seconds of the timed
    region, per-step event lists)."""
    stream = torch.cuda.current_stream()
    t_pre = time.perf_counter()
    a.prewarm_steps = 0
    while time.perf_counter() - t_pre < a.prewarm_s:
        for _ in range(5):
            step(None, stream)
        a.prewarm_steps += 5
        torch.cuda.synchronize()
    for _ in range(a.warmup):
        step(None, stream)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_phases + 1)] for _ in range(a.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(a.steps):
        step(evs[i], stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return t_start.elapsed_time(t_end) / a.steps, wall, evs


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-s", type=float, default=1.5,
                    help="seconds of untimed steps before the warm-up steps, so the engine clock settles")
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5],
                    help="synthetic configuration (default 3: 512 MiB filter, 200 Mbp genome, 20 M reads; "
                         "2: 8 MiB filter, 5 Mbp genome, 2 M reads; 5: 4 GiB filter, 3 Gbp genome, "
                         "1 M long reads)")
    ap.add_argument("--alphabet", default="dna", choices=["dna", "protein", "triplet"],
                    help="dna (default, --workload applies) or the protein / DNA-triplet workload")
    ap.add_argument("--probe-n", type=int, default=10_000_000)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle baseline in seconds (0 disables it)")
    ap.add_argument("--no-membench", dest="membench", action="store_false",
                    help="skip the matched-ceiling microbenchmarks (random shard reads / OR-updates) run after timing")
    ap.add_argument("--data-cache", default="",
                    help="directory for the generated inputs: saved there (.npy) after generating, memory-mapped "
                         "from there when present (profiled runs then skip the forking long-read generator)")
    ap.add_argument("--query-input", default="auto", choices=["auto", "reads", "text", "packed"],
                    help="DNA reads as the query gets them: reads (sbf_query_reads, the per-read query of the "
                         "equal-length reads of workloads 2-4), text (sbf_query_seq of the reads joined by 'N', "
                         "whose kernel decodes the ASCII itself) or packed (sbf_pack, then sbf_query_packed); "
                         "auto (default) = reads where the workload's reads have one length, else text")
    ap.add_argument("--insert-input", default="text", choices=["text", "packed"],
                    help="DNA genome as the insert gets it: text (default; sbf_insert_seq, whose kernel decodes "
                         "the ASCII itself) or packed (sbf_pack, then sbf_insert_packed)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run one plain 256 MiB device copy (elementwise kernel) whose "
                         "FETCH_SIZE/WRITE_SIZE counters scale the filter kernels' counters")
    return ap.parse_args()


def cpu_baseline(w: dict, budget_s: float, params=(K, M_, S_, H_), alpha: str = "dna") -> dict:
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    the first genome bases and read bases (about budget_s seconds of work)
    through its threaded insert/query drivers on the host's cores, and the
    probe (single-threaded in the oracle) on a proportionate count."""
    from oracle import oracle as O

    g, reads = w["insert"], w["queries"][0]
    cores = O._threads(0)
    al = {"dna": O.ALPHA_DNA, "protein": O.ALPHA_PROTEIN, "triplet": O.ALPHA_TRIPLET}[alpha]
    sb = 3 if alpha == "triplet" else 1
    k = params[0]

    def nkm(nbytes):
        return max(0, nbytes // sb - k + 1)

    f = O.OracleFilter(*params, w["bits"], alpha=al)
    # calibrate insert and query on short pieces, then size the sample to the budget
    n0 = min(g.size, 2_000_000)
    t0 = time.perf_counter()
    f.insert_seq_mt(g[:n0], cores)
    t1 = time.perf_counter()
    f.query_seq_mt(reads[:n0], cores)
    per_i = (t1 - t0) / max(1, nkm(n0))
    per_q = (time.perf_counter() - t1) / max(1, nkm(n0))
    f = O.OracleFilter(*params, w["bits"], alpha=al)
    n_ins = int(min(g.size, max(1_000_000, budget_s * 0.3 / per_i)))
    n_q = int(min(reads.size, max(1_000_000, (budget_s * 0.9 - n_ins * per_i) / per_q)))
    n_p = int(max(100_000, budget_s * 0.1 / (per_q * cores)))
    t0 = time.perf_counter()
    f.insert_seq_mt(g[:n_ins], cores)
    t1 = time.perf_counter()
    f.query_seq_mt(reads[:n_q], cores)
    t2 = time.perf_counter()
    f.fpr_probe(n_p, 0x5EED)
    t3 = time.perf_counter()
    kmers = nkm(n_ins) + nkm(n_q) + n_p
    # the plain single-threaded oracle on a short sample of both inputs
    n1 = int(min(g.size, reads.size, 1_000_000))
    f1 = O.OracleFilter(*params, w["bits"], alpha=al)
    s0 = time.perf_counter()
    f1.insert_seq(g[:n1])
    f1.query_seq(reads[:n1])
    single = 2 * nkm(n1) / (time.perf_counter() - s0) / 1e9
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": kmers / (t3 - t0) / 1e9, "unit": "Gk-mers/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
            "sample": "C oracle, %d threads: insert of the first %d bytes of the inserted text, query of the first %d bytes of the "
                      "query text, %d probe k-mers on one thread (%.1f s)" % (cores, n_ins, n_q, n_p, t3 - t0),
            "insert_gkmers_s": nkm(n_ins) / (t1 - t0) / 1e9,
            "query_gkmers_s": nkm(n_q) / (t2 - t1) / 1e9,
            "single_thread_gkmers_s": single,
            "single_thread_sample": "insert then query of the first %d bytes of each text on one thread" % n1}


def progress(msg: str) -> None:
    """One progress line on stderr (the JSON result alone goes to stdout)."""
    print("[bench %.1fs] %s" % (time.perf_counter() - T0, msg), file=sys.stderr, flush=True)


def cached_workload(S, cfg: int, cache: str) -> dict:
    """S.workload(cfg), or its inserted and last query text memory-mapped
    from `cache` when saved there before (and saved there after generating)."""
    import numpy as np

    if not cache:
        return S.workload(cfg)
    names = [os.path.join(cache, "cfg%d_%s.npy" % (cfg, part)) for part in ("insert", "query")]
    if all(os.path.exists(n) for n in names):
        ins, qry = (np.load(n, mmap_mode="r") for n in names)
        return {"cfg": cfg, "bits": S.CONFIG_BITS[cfg], "insert": ins, "queries": [qry]}
    w = S.workload(cfg)
    progress("generated; saving to %s" % cache)
    os.makedirs(cache, exist_ok=True)
    for n, arr in zip(names, (w["insert"], w["queries"][-1])):
        np.save(n + ".tmp.npy", arr)
        os.replace(n + ".tmp.npy", n)
    return w


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (got --gpus %d)" % a.gpus,
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import minimizer_sharded_bloom_amd as M
    from minimizer_sharded_bloom_amd import synthetic as S

    if a.alphabet == "dna":
        # inputs first: the long-read generator forks workers, which must
        # happen before this process initializes the GPU
        t_gen = time.perf_counter()
        w = cached_workload(S, a.workload, a.data_cache)
        genome_h, reads_h = w["insert"], w["queries"][-1]
        gen_s = time.perf_counter() - t_gen
        progress("inputs ready (%.1f s): %d + %d bases" % (gen_s, genome_h.size, reads_h.size))
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    lib = M.lib()
    if a.alphabet != "dna":
        return main_alpha(a, torch, M, S, lib)

    dev = torch.device("cuda:0")
    genome = torch.from_numpy(genome_h).to(dev)
    reads = torch.from_numpy(reads_h).to(dev)
    LG, LR = genome.numel(), reads.numel()
    gcw, gvw = M.packed_words(LG)
    rcw, rvw = M.packed_words(LR)
    g_codes = torch.empty(gcw, dtype=torch.int32, device=dev)
    g_valid = torch.empty(gvw, dtype=torch.int32, device=dev)
    r_codes = torch.empty(rcw, dtype=torch.int32, device=dev)
    r_valid = torch.empty(rvw, dtype=torch.int32, device=dev)
    f = M.SuperBloomFilter(K, M_, S_, H_, w["bits"])
    assert f.specialized
    out = torch.empty(f.num_answer_words(LR), dtype=torch.int64, device=dev)
    hits = torch.zeros(1, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    # workloads 2-4 query reads of one length joined by one 'N'; workload 5's
    # long reads vary in length
    fixed_reads = a.workload in (2, 3, 4)
    qin = a.query_input if a.query_input != "auto" else ("reads" if fixed_reads else "text")
    if qin == "reads":
        assert fixed_reads, "--query-input reads needs equal-length reads (workloads 2-4)"
        RL, RS = S.READ_LEN, S.READ_LEN + 1
        n_reads = (LR + 1) // RS
        assert (n_reads - 1) * RS + RL == LR, "reads are not %d bases at a stride of %d" % (RL, RS)
        rout = torch.empty(n_reads * f.read_answer_words(RL), dtype=torch.int32, device=dev)
    text_query = qin in ("text", "reads")  # no packing pass for the reads
    assert qin != "text" or reads.data_ptr() % 16 == 0, "the ASCII query path needs 16-byte-aligned reads"
    text_insert = a.insert_input == "text"
    assert not text_insert or genome.data_ptr() % 16 == 0, "the ASCII insert path needs a 16-byte-aligned genome"
    names = (["clear"] + ([] if text_insert else ["pack_genome"]) + ["insert"]
             + ([] if text_query else ["pack_reads"]) + ["query", "probe"])

    def step(events, st):
        sp = st.cuda_stream
        marks = iter(range(len(names) + 1))

        def mark():
            i = next(marks)
            if events is not None:
                events[i].record(st)
        mark()
        M.check(lib.sbf_clear(f.handle, sp), "clear")
        mark()
        if text_insert:
            M.check(lib.sbf_insert_seq(f.handle, genome.data_ptr(), LG, M.SBF_DEVICE, sp), "insert")
        else:
            M.check(lib.sbf_pack(genome.data_ptr(), LG, g_codes.data_ptr(), g_valid.data_ptr(), sp), "pack")
            mark()
            M.check(lib.sbf_insert_packed(f.handle, g_codes.data_ptr(), g_valid.data_ptr(), LG, sp), "insert")
        mark()
        if qin == "reads":
            M.check(lib.sbf_query_reads(f.handle, reads.data_ptr(), n_reads, RL, RS, rout.data_ptr(), sp), "query")
        elif text_query:
            M.check(lib.sbf_query_seq(f.handle, reads.data_ptr(), LR, out.data_ptr(), M.SBF_DEVICE, sp), "query")
        else:
            M.check(lib.sbf_pack(reads.data_ptr(), LR, r_codes.data_ptr(), r_valid.data_ptr(), sp), "pack")
            mark()
            M.check(lib.sbf_query_packed(f.handle, r_codes.data_ptr(), r_valid.data_ptr(), LR, out.data_ptr(), sp),
                    "query")
        mark()
        M.check(lib.sbf_fpr_probe_device(f.handle, a.probe_n, 0x5EED, hits.data_ptr(), sp), "probe")
        mark()

    ms_step, wall, evs = timed_steps(torch, step, len(names), a)
    phase = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / a.steps for i, n in enumerate(names)}
    phase_med = {n: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    progress("timed steps done")
    ceilings = matched_ceilings(lib, torch, f, stream) if a.membench else None
    progress("matched ceilings done")

    if a.calibrate_copy:
        src = torch.ones(1 << 25, dtype=torch.int64, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.add(src, 0, out=dst)                                   # elementwise: reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del src, dst

    nk_g, nk_r = LG - K + 1, LR - K + 1
    (vk_g, seg_g), (vk_r, seg_r) = (valid_kmer_count(genome_h, K, segments=True),
                                    valid_kmer_count(reads_h, K, segments=True))
    total = vk_g + vk_r + a.probe_n
    value = total / (ms_step * 1e-3) / 1e9
    # rates over valid k-mers (the roofline's numerator counts only these)
    ins_rate = vk_g / (phase["insert"] * 1e-3)
    q_rate = vk_r / (phase["query"] * 1e-3)

    sha = kernel_sources_sha256()
    wl = "cfg%d" % a.workload

    def roof(kind, rate):
        model = kind + ("_text" if (text_query if kind == "query" else text_insert) else "")
        alu = rate * alu_ops_per_kmer(model)
        mem = rate * _bytes_per_kmer(model)
        tr = measured_traffic(wl, kind, sha)
        traffic = None if tr is None else tr["bytes"]
        extra = {} if tr is None else {"traffic_fetch": tr["fetch"], "traffic_write": tr["write"],
                                       "traffic_source": tr["source"],
                                       "traffic_per_valid_kmer": tr["bytes"] / (vk_r if kind == "query" else vk_g)}
        slots = rate * alu_issue_slots_per_kmer(model)
        return (dict({"bound": "alu", "achieved": alu / 1e12, "peak": ALU_PEAK / 1e12,
                      "unit": "T lane-instr/s", "frac": alu / ALU_PEAK, "traffic": traffic,
                      "kernel": kind, "per_valid_kmer_ops": alu_ops_per_kmer(model),
                      "per_valid_kmer_issue_slots": alu_issue_slots_per_kmer(model),
                      "issue_slot_frac": slots / ALU_PEAK, "ms_per_launch": phase[kind]}, **extra),
                dict({"bound": "hbm", "achieved": mem / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                      "frac": mem / HBM_PEAK, "traffic": traffic, "kernel": kind,
                      "per_valid_kmer_bytes": _bytes_per_kmer(model), "ms_per_launch": phase[kind],
                      "filter_resides": filter_level(w["bits"] // 8)}, **extra))

    def binding(kind, rate):
        """The two ceilings of one kernel, the binding one (higher fraction)
        first."""
        alu, mem = roof(kind, rate)
        return (alu, mem) if alu["frac"] >= mem["frac"] else (mem, alu)

    dom = "query" if phase["query"] >= phase["insert"] else "insert"
    primary, secondary = binding(dom, q_rate if dom == "query" else ins_rate)
    other = "insert" if dom == "query" else "query"
    other_primary, _ = binding(other, ins_rate if other == "insert" else q_rate)

    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "Gk-mers/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u64", "data": "synthetic",
        "config": {"workload": wl, "k": K, "m": M_, "s": S_, "H": H_, "filter_bits": w["bits"],
                   "genome_bases": LG, "read_bases": LR, "probe_kmers": a.probe_n,
                   "valid_kmers_per_step": total},
        "roofline": primary, "roofline_other": secondary, "roofline_" + other: other_primary,
        "insert_gkmers_s": round(ins_rate / 1e9, 3), "query_gkmers_s": round(q_rate / 1e9, 3),
        "insert_starts_gkmers_s": round(nk_g / (phase["insert"] * 1e-3) / 1e9, 3),
        "query_starts_gkmers_s": round(nk_r / (phase["query"] * 1e-3) / 1e9, 3),
        "value_starts_gkmers_s": round((nk_g + nk_r + a.probe_n) / (ms_step * 1e-3) / 1e9, 3),
        "prewarm": {"seconds": a.prewarm_s, "steps": a.prewarm_steps},
        "pack_gbases_s": (round(((0 if text_insert else LG) + (0 if text_query else LR))
                                / ((phase.get("pack_genome", 0.0) + phase.get("pack_reads", 0.0)) * 1e-3) / 1e9, 3)
                          if not (text_insert and text_query) else None),
        "insert_input": a.insert_input,
        "query_input": qin,
        "probe_gkmers_s": round(a.probe_n / (phase["probe"] * 1e-3) / 1e9, 3),
        "phase_ms": {k2: round(v, 4) for k2, v in phase.items()},
        "phase_ms_median": {k2: round(v, 4) for k2, v in phase_med.items()},
        "kmer_starts": {"insert": nk_g, "query": nk_r, "probe": a.probe_n},
        "valid_kmers": {"insert": vk_g, "query": vk_r},
        "wall_s_timed": round(wall, 3), "gen_s": round(gen_s, 2),
        "kernel_sources_sha256": sha,
    }
    if ceilings is not None:
        # runs of random minimizers: a stretch of n valid k-mers holds
        # 1 + (n-1) 2/(w+1) of them on average; one record flush per run for
        # the insert, one shard read per run for the query, set against the
        # matched ceilings
        runs = 2.0 / (K - M_ + 2)
        rec_g = vk_g * runs + seg_g * (1.0 - runs)
        rec_r = vk_r * runs + seg_r * (1.0 - runs)
        ceilings["insert_records_est_g_per_s"] = round(rec_g / (phase["insert"] * 1e-3) / 1e9, 3)
        ceilings["insert_frac_of_or_ceiling"] = round(ceilings["insert_records_est_g_per_s"]
                                                      / ceilings["shard_ors_g_per_s"], 3)
        ceilings["query_shard_reads_est_g_per_s"] = round(rec_r / (phase["query"] * 1e-3) / 1e9, 3)
        ceilings["query_frac_of_read_ceiling"] = round(ceilings["query_shard_reads_est_g_per_s"]
                                                       / ceilings["shard_reads_g_per_s"], 3)
        res["matched_ceilings"] = ceilings
    if a.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
        progress("cpu baseline done")
    print(json.dumps(res), flush=True)


def main_alpha(a, torch, M, S, lib):
    """The step over a protein or DNA-triplet filter: clear, insert the
    reference text, query the reads, probe (no pack launches: these kernels
    decode the ASCII themselves)."""
    alpha = a.alphabet
    k, m, s, H = ALPHAS[alpha]["params"]
    t_gen = time.perf_counter()
    w = S.alpha_workload(alpha)
    gen_s = time.perf_counter() - t_gen
    progress("inputs ready (%.1f s)" % gen_s)
    dev = torch.device("cuda:0")
    ref = torch.from_numpy(w["insert"]).to(dev)
    reads = torch.from_numpy(w["queries"][0]).to(dev)
    LG, LR = ref.numel(), reads.numel()
    f = (M.SuperBloomFilter.protein if alpha == "protein" else M.SuperBloomFilter.triplet)(k, m, s, H, w["bits"])
    out = torch.empty(f.num_answer_words(LR), dtype=torch.int64, device=dev)
    hits = torch.zeros(1, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    names = ["clear", "insert", "query", "probe"]

    def step(events, st):
        sp = st.cuda_stream

        def mark(i):
            if events is not None:
                events[i].record(st)
        mark(0)
        M.check(lib.sbf_clear(f.handle, sp), "clear")
        mark(1)
        M.check(lib.sbf_insert_seq(f.handle, ref.data_ptr(), LG, M.SBF_DEVICE, sp), "insert")
        mark(2)
        M.check(lib.sbf_query_seq(f.handle, reads.data_ptr(), LR, out.data_ptr(), M.SBF_DEVICE, sp), "query")
        mark(3)
        M.check(lib.sbf_fpr_probe_device(f.handle, a.probe_n, 0x5EED, hits.data_ptr(), sp), "probe")
        mark(4)

    ms_step, wall, evs = timed_steps(torch, step, len(names), a)
    phase = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / a.steps for i, n in enumerate(names)}
    import numpy as np
    phase_med = {n: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    progress("timed steps done")
    ceilings = matched_ceilings(lib, torch, f, stream) if a.membench else None
    progress("matched ceilings done")

    if a.calibrate_copy:
        src = torch.ones(1 << 25, dtype=torch.int64, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        torch.add(src, 0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    nk_g, nk_r = f.num_symbols(LG) - k + 1, f.num_symbols(LR) - k + 1
    (vk_g, seg_g), (vk_r, seg_r) = (valid_kmer_count(w["insert"], k, alpha, segments=True),
                                    valid_kmer_count(w["queries"][0], k, alpha, segments=True))
    total = vk_g + vk_r + a.probe_n
    value = total / (ms_step * 1e-3) / 1e9
    ins_rate = vk_g / (phase["insert"] * 1e-3)
    q_rate = vk_r / (phase["query"] * 1e-3)
    sha = kernel_sources_sha256("alpha")

    def roof(kind, rate):
        ops = alpha_alu_ops_per_kmer(alpha, kind)
        alu, mem = rate * ops, rate * alpha_bytes_per_kmer(alpha, kind)
        tr = measured_traffic(alpha, kind, sha)
        traffic = None if tr is None else tr["bytes"]
        extra = {} if tr is None else {"traffic_fetch": tr["fetch"], "traffic_write": tr["write"],
                                       "traffic_source": tr["source"],
                                       "traffic_per_valid_kmer": tr["bytes"] / (vk_r if kind == "query" else vk_g)}
        return (dict({"bound": "alu", "achieved": alu / 1e12, "peak": ALU_PEAK / 1e12, "unit": "T lane-instr/s",
                      "frac": alu / ALU_PEAK, "traffic": traffic, "kernel": kind, "per_valid_kmer_ops": ops,
                      "ms_per_launch": phase[kind]}, **extra),
                dict({"bound": "hbm", "achieved": mem / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                      "frac": mem / HBM_PEAK, "traffic": traffic, "kernel": kind,
                      "per_valid_kmer_bytes": alpha_bytes_per_kmer(alpha, kind), "ms_per_launch": phase[kind]},
                     **extra))

    dom = "query" if phase["query"] >= phase["insert"] else "insert"
    alu, mem = roof(dom, q_rate if dom == "query" else ins_rate)
    primary, secondary = (alu, mem) if alu["frac"] >= mem["frac"] else (mem, alu)
    res = {
        "metric": "insert & query Gk-mers/s, %s alphabet (k=%d,m=%d,s=%d,H=%d) + fraction of ALU/HBM roofline"
                  % (alpha, k, m, s, H),
        "value": round(value, 3), "unit": "Gk-mers/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u64", "data": "synthetic",
        "config": {"workload": alpha, "k": k, "m": m, "s": s, "H": H, "filter_bits": w["bits"],
                   "insert_bytes": LG, "query_bytes": LR, "probe_kmers": a.probe_n, "valid_kmers_per_step": total},
        "roofline": primary, "roofline_other": secondary,
        "insert_gkmers_s": round(ins_rate / 1e9, 3), "query_gkmers_s": round(q_rate / 1e9, 3),
        "insert_starts_gkmers_s": round(nk_g / (phase["insert"] * 1e-3) / 1e9, 3),
        "query_starts_gkmers_s": round(nk_r / (phase["query"] * 1e-3) / 1e9, 3),
        "value_starts_gkmers_s": round((nk_g + nk_r + a.probe_n) / (ms_step * 1e-3) / 1e9, 3),
        "prewarm": {"seconds": a.prewarm_s, "steps": a.prewarm_steps},
        "probe_gkmers_s": round(a.probe_n / (phase["probe"] * 1e-3) / 1e9, 3),
        "phase_ms": {k2: round(v, 4) for k2, v in phase.items()},
        "phase_ms_median": {k2: round(v, 4) for k2, v in phase_med.items()},
        "kmer_starts": {"insert": nk_g, "query": nk_r, "probe": a.probe_n},
        "valid_kmers": {"insert": vk_g, "query": vk_r},
        "wall_s_timed": round(wall, 3), "gen_s": round(gen_s, 2), "kernel_sources_sha256": sha,
    }
    if ceilings is not None:
        runs = 2.0 / (k - m + 2)  # as in main()
        rec_g = vk_g * runs + seg_g * (1.0 - runs)
        rec_r = vk_r * runs + seg_r * (1.0 - runs)
        ceilings["insert_records_est_g_per_s"] = round(rec_g / (phase["insert"] * 1e-3) / 1e9, 3)
        ceilings["insert_frac_of_or_ceiling"] = round(ceilings["insert_records_est_g_per_s"]
                                                      / ceilings["shard_ors_g_per_s"], 3)
        ceilings["query_shard_reads_est_g_per_s"] = round(rec_r / (phase["query"] * 1e-3) / 1e9, 3)
        ceilings["query_frac_of_read_ceiling"] = round(ceilings["query_shard_reads_est_g_per_s"]
                                                       / ceilings["shard_reads_g_per_s"], 3)
        res["matched_ceilings"] = ceilings
    if a.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds, (k, m, s, H), alpha)
        progress("cpu baseline done")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
