"""Seeded synthetic sequence workloads (numpy PCG64).  Random text only: this
module holds none of the filter's arithmetic, so both the GPU path and the CPU
oracle can take their inputs from it.

The workloads stand in for the genomes, reads and random k-mers of the
evaluation in "cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data
on Modern GPUs" (§V-A, §V-D), which are not available here:

  1  100 kbp uniform sequence (seed 0) inserted; queried: itself and an
     independent 100 kbp sequence (seed 1); filter 2^20 bits.
  2  5 Mbp genome: uniform bases, then copied 1-5 kbp segments (2%
     substitutions) until 5% of it is overwritten; 2 M reads of 150 bp, half
     sampled from the genome with 1% substitutions, half uniform, shuffled
     together and joined by 'N'; filter 2^26 bits.
  3  as 2 with a 200 Mbp genome and 20 M reads; filter 2^32 bits.
  4  as 2 with a 50 Mbp genome and 1 M reads; filter 2^30 bits.
  5  3 Gbp uniform genome with 'N' runs of 1-1000 bases at uniform positions
     until their lengths sum to 0.1% of it; 1 M long reads in 100 batches of
     10 k: length round(exp(N(ln 10000, 0.5^2))) clamped to 1-50 kbp, uniform
     forward-strand start, 5% errors split equally between substitution,
     insertion of a random base and deletion; reads joined by 'N'; filter
     2^35 bits.  The seeded 1% read subsample is one whole batch.

Other alphabets (§IV-A; the evaluation measures DNA only, so these follow
the DNA workloads' shapes):

  protein  a 16 M-residue proteome: residues i.i.d. uniform over the 20
           standard amino acids, copied 50-300-residue segments (5%
           substitutions) overwriting 5% of it, proteins of length
           round(exp(N(ln 350, 0.6^2))) clamped to 30-5000 joined by '*';
           queries: 2 M peptides of 50 residues, half sampled from the
           proteome at uniform starts with 1% substitutions, half uniform,
           shuffled and joined by '*'; filter 2^28 bits (16 per k-mer).
  triplet  a 48 Mbp genome as in 2 (16 M codons); queries: 2 M reads of 150
           bp, half sampled at codon-aligned starts with 1% substitutions,
           half uniform, joined by "NNN" so each read starts on a codon
           boundary; filter 2^28 bits.

Seeds: genome 0, foreign sequence 1, repeats 2, read starts 3, read errors 4,
random reads 5, shuffle 6, subsample 7, 'N' runs 8, long-read layout 9,
long-read errors 10, proteome 20, protein lengths 21, peptides 22.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

ACGT = np.frombuffer(b"ACGT", dtype=np.uint8)
N_BYTE = ord("N")

CONFIG_BITS = {1: 2**20, 2: 2**26, 3: 2**32, 4: 2**30, 5: 2**35}
CONFIG_GENOME = {1: 100_000, 2: 5_000_000, 3: 200_000_000, 4: 50_000_000, 5: 3_000_000_000}
CONFIG_READS = {2: 2_000_000, 3: 20_000_000, 4: 1_000_000, 5: 1_000_000}
READ_LEN = 150
LONG_BATCHES = 100          # configuration 5 reads come in 100 batches of 10 k
CHUNK = 1 << 27


def uniform_codes(n: int, seed: int) -> np.ndarray:
    """n i.i.d. uniform base codes 0..3 (uint8)."""
    return np.random.default_rng(seed).integers(0, 4, n, dtype=np.uint8)


def to_ascii(codes: np.ndarray) -> np.ndarray:
    return ACGT[codes]


def substitute(codes: np.ndarray, rate: float, rng: np.random.Generator, chunk: int = 1 << 24) -> None:
    """In place: each base becomes one of the other three with probability rate."""
    flat = codes.reshape(-1)
    for lo in range(0, flat.size, chunk):
        part = flat[lo:lo + chunk]
        hit = np.flatnonzero(rng.random(part.size, dtype=np.float32) < rate)
        if hit.size:
            part[hit] = (part[hit] + rng.integers(1, 4, hit.size, dtype=np.uint8)) & 3


def genome_with_repeats(G: int, frac: float = 0.05, seg=(1000, 5000), sub: float = 0.02,
                        seed_genome: int = 0, seed_repeats: int = 2) -> np.ndarray:
    """Codes of a uniform genome in which copied segments (with substitutions)
    overwrite at least `frac` of its length.  Source and destination of one
    copy do not overlap."""
    g = uniform_codes(G, seed_genome)
    rng = np.random.default_rng(seed_repeats)
    done, target = 0, int(frac * G)
    if G <= 2 * seg[1]:
        return g
    while done < target:
        L = int(rng.integers(seg[0], seg[1] + 1))
        src = int(rng.integers(0, G - L + 1))
        dst = int(rng.integers(0, G - L + 1))
        if abs(src - dst) < L:
            continue
        piece = g[src:src + L].copy()
        substitute(piece, sub, rng)
        g[dst:dst + L] = piece
        done += L
    return g


def sampled_reads(genome: np.ndarray, n: int, L: int, err: float, seed_start: int = 3, seed_err: int = 4,
                  chunk: int = 1 << 20) -> np.ndarray:
    """(n, L) codes of forward-strand reads at uniform starts, substituted
    with probability err per base."""
    out = np.empty((n, L), dtype=np.uint8)
    rs, re = np.random.default_rng(seed_start), np.random.default_rng(seed_err)
    off = np.arange(L, dtype=np.int64)
    for lo in range(0, n, chunk):
        m = min(chunk, n - lo)
        starts = rs.integers(0, genome.size - L + 1, m)
        out[lo:lo + m] = genome[starts[:, None] + off[None, :]]
    substitute(out, err, re)
    return out


def random_reads(n: int, L: int, seed: int = 5) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, 4, (n, L), dtype=np.uint8)


def join_records(reads: np.ndarray) -> np.ndarray:
    """ASCII of (n, L) read codes joined by a single 'N' (no trailing one)."""
    n, L = reads.shape
    out = np.empty((n, L + 1), dtype=np.uint8)
    out[:, :L] = ACGT[reads]
    out[:, L] = N_BYTE
    return out.reshape(-1)[:-1] if n else np.empty(0, dtype=np.uint8)


def short_read_set(genome: np.ndarray, R: int, L: int = READ_LEN, err: float = 0.01, seed_shuffle: int = 6) -> np.ndarray:
    """ASCII of R reads (R/2 sampled with errors, R/2 uniform), shuffled and
    joined by 'N'."""
    half = R // 2
    reads = np.concatenate([sampled_reads(genome, half, L, err), random_reads(R - half, L)])
    perm = np.random.default_rng(seed_shuffle).permutation(R)
    return join_records(reads[perm])


# every byte value -> its four 2-bit digits as bases, most significant first
_BYTE_TO_4BASES = ACGT[(np.arange(256)[:, None] >> np.array([6, 4, 2, 0])[None, :]) & 3].astype(np.uint8)
_BYTE_TO_4BASES_U32 = np.ascontiguousarray(_BYTE_TO_4BASES).view("<u4").reshape(-1)


def uniform_ascii_fast(n: int, seed: int) -> np.ndarray:
    """n i.i.d. uniform bases as ASCII: PCG64 random bytes, four bases per
    byte, in 2^27-byte chunks of one stream."""
    out = np.empty(((n + 3) // 4) * 4, dtype=np.uint8)
    view = out.view("<u4")
    rng = np.random.default_rng(seed)
    for lo in range(0, view.size, CHUNK):
        hi = min(view.size, lo + CHUNK)
        view[lo:hi] = _BYTE_TO_4BASES_U32[np.frombuffer(rng.bytes(hi - lo), dtype=np.uint8)]
    return out[:n]


def genome_with_n_runs(G: int, frac: float = 0.001, run=(1, 1000), seed_genome: int = 0,
                       seed_runs: int = 8) -> np.ndarray:
    """ASCII of a uniform genome (uniform_ascii_fast) with 'N' runs of length
    U{run} at uniform positions until the run lengths sum to `frac` of G."""
    out = uniform_ascii_fast(G, seed_genome)
    rr = np.random.default_rng(seed_runs)
    done, target = 0, int(frac * G)
    while done < target:
        L = int(rr.integers(run[0], run[1] + 1))
        p = int(rr.integers(0, G - L + 1))
        out[p:p + L] = N_BYTE
        done += L
    return out


_BASE_INDEX = np.full(256, 4, dtype=np.int64)  # ASCII -> 0..3 for A,C,G,T, 4 otherwise
_BASE_INDEX[ACGT] = np.arange(4)


def long_read_batch(genome: np.ndarray, b: int, n: int = 10_000, median: float = 10_000.0, sigma: float = 0.5,
                    lo: int = 1_000, hi: int = 50_000, err: float = 0.05, seed_layout: int = 9,
                    seed_err: int = 10) -> np.ndarray:
    """ASCII of batch b of long reads (n reads joined by 'N'): lengths
    round(exp(N(ln median, sigma^2))) clamped to [lo, hi], uniform
    forward-strand starts, per-base errors at rate err (positions from
    geometric gaps) split equally between substitution (another base),
    insertion of a random base before the base, and deletion."""
    G = genome.size
    rl = np.random.default_rng([seed_layout, b])
    lens = np.clip(np.rint(np.exp(rl.normal(np.log(median), sigma, n))), lo, min(hi, G)).astype(np.int64)
    starts = rl.integers(0, G - lens + 1)
    tmpl = np.concatenate([genome[s0:s0 + l0] for s0, l0 in zip(starts.tolist(), lens.tolist())])
    total = tmpl.size
    re_ = np.random.default_rng([seed_err, b])
    if err > 0:
        gaps = re_.geometric(err, int(total * err * 1.2) + 1000)
        pos = np.cumsum(gaps) - 1
        pos = pos[pos < total]
    else:
        pos = np.empty(0, dtype=np.int64)
    kind = re_.integers(0, 3, pos.size)  # 0 substitution, 1 insertion, 2 deletion
    sub, ins, dele = pos[kind == 0], pos[kind == 1], pos[kind == 2]
    cur = _BASE_INDEX[tmpl[sub]]
    tmpl[sub] = ACGT[(np.minimum(cur, 3) + re_.integers(1, 4, sub.size)) & 3]
    body = np.delete(tmpl, dele)
    ins_at = ins - np.searchsorted(dele, ins)  # insertion points after the deletions
    body = np.insert(body, ins_at, ACGT[re_.integers(0, 4, ins.size)])
    # read lengths after editing, then one 'N' between reads
    ends = np.cumsum(lens)
    read_of = lambda q: np.searchsorted(ends, q, side="right")
    out_lens = lens - np.bincount(read_of(dele), minlength=n) + np.bincount(read_of(ins), minlength=n)
    return np.insert(body, np.cumsum(out_lens)[:-1], N_BYTE)


def long_read_subsample_batch(seed: int = 7) -> int:
    """Index of the batch that is the seeded 1% read subsample."""
    return int(np.random.default_rng(seed).integers(0, LONG_BATCHES))


_FORK_GENOME = None  # the genome that forked batch workers read (set only while a pool runs)


def _long_read_batch_forked(bn) -> np.ndarray:
    return long_read_batch(_FORK_GENOME, bn[0], n=bn[1])


def long_read_set(genome: np.ndarray, batches=None, workers: int = 0, n: int = 10_000) -> np.ndarray:
    """ASCII of the given batches (default: all) joined by 'N'.  Batches are
    seeded by their index alone, so `workers` > 1 (forked processes that
    share the genome copy-on-write; 0 = min(16, CPUs)) gives the same bytes
    as one process.  `n` reads per batch.  Call it before the process
    initializes a GPU."""
    global _FORK_GENOME
    batches = list(range(LONG_BATCHES) if batches is None else batches)
    if workers <= 0:
        workers = min(16, os.cpu_count() or 1)
    workers = min(workers, len(batches))
    if workers > 1 and "fork" in mp.get_all_start_methods():
        _FORK_GENOME = genome
        try:
            with mp.get_context("fork").Pool(workers) as pool:
                parts = pool.map(_long_read_batch_forked, [(b, n) for b in batches], chunksize=1)
        finally:
            _FORK_GENOME = None
    else:
        parts = [long_read_batch(genome, b, n=n) for b in batches]
    if not parts:
        return np.empty(0, dtype=np.uint8)
    out = np.empty(sum(p.size for p in parts) + len(parts) - 1, dtype=np.uint8)
    at = 0
    for i in range(len(parts)):
        part = parts[i]
        parts[i] = None  # release each batch once copied
        if i:
            out[at] = N_BYTE
            at += 1
        out[at:at + part.size] = part
        at += part.size
    return out


def workload(cfg: int) -> dict:
    """Inputs of one configuration: ASCII uint8 arrays and the filter size."""
    if cfg == 1:
        ins = to_ascii(uniform_codes(CONFIG_GENOME[1], 0))
        foreign = to_ascii(uniform_codes(CONFIG_GENOME[1], 1))
        return {"cfg": 1, "bits": CONFIG_BITS[1], "insert": ins, "queries": [ins, foreign]}
    if cfg in (2, 3, 4):
        g = genome_with_repeats(CONFIG_GENOME[cfg])
        reads = short_read_set(g, CONFIG_READS[cfg])
        return {"cfg": cfg, "bits": CONFIG_BITS[cfg], "insert": to_ascii(g), "queries": [reads]}
    if cfg == 5:
        g = genome_with_n_runs(CONFIG_GENOME[5])
        return {"cfg": 5, "bits": CONFIG_BITS[5], "insert": g, "queries": [long_read_set(g)]}
    raise ValueError("workload %r is not generated by this module" % cfg)


AMINO = np.frombuffer(b"ACDEFGHIKLMNPQRSTVWY", dtype=np.uint8)
STOP_BYTE = ord("*")
PROTEIN_RESIDUES = 16_000_000
TRIPLET_GENOME = 48_000_000
ALPHA_READS = 2_000_000
ALPHA_BITS = 2**28


def proteome(n: int, frac: float = 0.05, seg=(50, 300), sub: float = 0.05, seed: int = 20,
             seed_len: int = 21) -> np.ndarray:
    """ASCII of about n residues of proteins joined by '*' (see the module
    docstring)."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, AMINO.size, n, dtype=np.uint8)
    done, target = 0, int(frac * n)
    while n > 2 * seg[1] and done < target:
        L = int(rng.integers(seg[0], seg[1] + 1))
        src, dst = (int(x) for x in rng.integers(0, n - L + 1, 2))
        if abs(src - dst) < L:
            continue
        piece = idx[src:src + L].copy()
        hit = rng.random(L) < sub
        piece[hit] = (piece[hit] + rng.integers(1, AMINO.size, int(hit.sum()), dtype=np.uint8)) % AMINO.size
        idx[dst:dst + L] = piece
        done += L
    out = AMINO[idx]
    # protein boundaries: overwrite one residue with '*' after each protein
    lr = np.random.default_rng(seed_len)
    lens = np.clip(np.round(np.exp(lr.normal(np.log(350.0), 0.6, n // 30 + 1))), 30, 5000).astype(np.int64)
    cuts = np.cumsum(lens + 1) - 1
    out[cuts[cuts < n]] = STOP_BYTE
    return out


def peptide_set(prot: np.ndarray, R: int, L: int = 50, err: float = 0.01, seed: int = 22) -> np.ndarray:
    """ASCII of R peptides of L residues (R/2 sampled from prot with
    substitutions, R/2 uniform), shuffled and joined by '*'."""
    rng = np.random.default_rng(seed)
    half = R // 2
    starts = rng.integers(0, prot.size - L + 1, half)
    samp = prot[starts[:, None] + np.arange(L)[None, :]]
    hit = rng.random(samp.shape) < err
    samp[hit] = AMINO[rng.integers(0, AMINO.size, int(hit.sum()))]
    rand = AMINO[rng.integers(0, AMINO.size, (R - half, L))]
    pep = np.concatenate([samp, rand])[rng.permutation(R)]
    out = np.empty((R, L + 1), dtype=np.uint8)
    out[:, :L] = pep
    out[:, L] = STOP_BYTE
    return out.reshape(-1)[:-1] if R else np.empty(0, dtype=np.uint8)


def codon_read_set(genome: np.ndarray, R: int, L: int = READ_LEN, err: float = 0.01, seed: int = 22) -> np.ndarray:
    """ASCII of R reads of L bases (L a multiple of 3; R/2 sampled at
    codon-aligned starts with substitutions, R/2 uniform), shuffled and
    joined by "NNN"."""
    assert L % 3 == 0
    rng = np.random.default_rng(seed)
    half = R // 2
    starts = 3 * rng.integers(0, (genome.size - L) // 3 + 1, half)
    samp = genome[starts[:, None] + np.arange(L)[None, :]]
    substitute(samp, err, rng)
    reads = np.concatenate([samp, rng.integers(0, 4, (R - half, L), dtype=np.uint8)])[rng.permutation(R)]
    out = np.empty((R, L + 3), dtype=np.uint8)
    out[:, :L] = ACGT[reads]
    out[:, L:] = N_BYTE
    return out.reshape(-1)[:-3] if R else np.empty(0, dtype=np.uint8)


def alpha_workload(name: str, scale: float = 1.0) -> dict:
    """Protein or triplet workload (module docstring); scale < 1 shrinks
    every size for tests."""
    R = max(2, int(ALPHA_READS * scale))
    if name == "protein":
        prot = proteome(max(1000, int(PROTEIN_RESIDUES * scale)))
        return {"name": name, "bits": max(256, int(ALPHA_BITS * scale)), "insert": prot,
                "queries": [peptide_set(prot, R)]}
    if name == "triplet":
        g = genome_with_repeats(max(3000, int(TRIPLET_GENOME * scale)) // 3 * 3)
        return {"name": name, "bits": max(256, int(ALPHA_BITS * scale)), "insert": to_ascii(g),
                "queries": [codon_read_set(g, R)]}
    raise ValueError("unknown alphabet workload %r" % name)


def split_records(stream: np.ndarray) -> list:
    """Records of an 'N'-joined stream as uint8 arrays (every 'N' is a record
    separator, so only streams whose records hold no 'N' round-trip)."""
    cuts = np.flatnonzero(stream == N_BYTE)
    return np.split(stream, cuts + 1) if cuts.size else [stream]


def bgzf_bytes(data: bytes, block: int = 0xFF00, level: int = 6, eof: bool = True) -> bytes:
    """`data` as a BGZF file (the blocked gzip of the SAM/BAM format
    specification, section 4.1): gzip members of at most `block` input bytes,
    each with the extra subfield 'BC' that holds the member's total size minus
    one, then (if eof) the empty end-of-file member."""
    import struct
    import zlib
    assert 0 < block <= 0xFF00
    pieces = [data[a:a + block] for a in range(0, len(data), block)] + ([b""] if eof else [])
    out = []
    for piece in pieces:
        z = zlib.compressobj(level, zlib.DEFLATED, -15)
        cdata = z.compress(piece) + z.flush()
        bsize = 12 + 6 + len(cdata) + 8 - 1
        assert bsize < 1 << 16
        out.append(b"\x1f\x8b\x08\x04" + struct.pack("<IBBH", 0, 0, 255, 6) + b"BC" + struct.pack("<HH", 2, bsize)
                   + cdata + struct.pack("<II", zlib.crc32(piece), len(piece)))
    return b"".join(out)


class _Sink:
    """A binary file that is written plain, gzip (gz=True) or BGZF
    (gz="bgzf"; assembled in memory and written on close)."""

    def __init__(self, path: str, gz):
        import gzip
        self.path, self.bgzf, self.parts = path, gz == "bgzf", []
        self.f = None if self.bgzf else (gzip.open(path, "wb") if gz else open(path, "wb"))

    def write(self, b: bytes) -> None:
        if self.bgzf:
            self.parts.append(b)
        else:
            self.f.write(b)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        if self.bgzf:
            with open(self.path, "wb") as f:
                f.write(bgzf_bytes(b"".join(self.parts)))
        else:
            self.f.close()


def write_fasta(path: str, records, width: int = 60, gz=False, crlf: bool = False,
                names: str = "read") -> None:
    """FASTA file of the given records (uint8 arrays or bytes, trailing 'N'
    separators stripped) with `width`-base lines; gzip if gz is True, BGZF if
    gz == "bgzf"."""
    eol = b"\r\n" if crlf else b"\n"
    with _Sink(path, gz) as f:
        for i, r in enumerate(records):
            s = bytes(r).rstrip(b"N")
            f.write(b">%s_%d length=%d" % (names.encode(), i, len(s)) + eol)
            for a in range(0, len(s), width):
                f.write(s[a:a + width] + eol)


def write_fastq(path: str, records, gz=False, seed_qual: int = 12) -> None:
    """FASTQ file (4-line records) of the given records with random quality
    strings (Phred+33 '!'..'J', seeded); gzip or BGZF as for write_fasta."""
    rng = np.random.default_rng(seed_qual)
    with _Sink(path, gz) as f:
        for i, r in enumerate(records):
            s = bytes(r).rstrip(b"N")
            q = (rng.integers(33, 75, len(s), dtype=np.uint8)).tobytes()
            f.write(b"@read_%d\n%s\n+\n%s\n" % (i, s, q))


def fasta_bytes(seq: np.ndarray, width: int = 80, name: bytes = b"chr1") -> np.ndarray:
    """One-record FASTA file contents (uint8) of a long sequence, `width`
    bases per line; vectorized for genome-sized inputs."""
    n = seq.size
    full = n // width
    body = np.empty((full, width + 1), dtype=np.uint8)
    body[:, :width] = seq[:full * width].reshape(full, width)
    body[:, width] = ord("\n")
    tail = seq[full * width:]
    parts = [np.frombuffer(b">" + name + b"\n", dtype=np.uint8), body.reshape(-1)]
    if tail.size:
        parts += [tail, np.frombuffer(b"\n", dtype=np.uint8)]
    return np.concatenate(parts)


def fastq_bytes(reads: np.ndarray, seed_qual: int = 12) -> np.ndarray:
    """FASTQ file contents (uint8) of equal-length reads given as an (n, L)
    ASCII array: '@r\\n', the read, '\\n+\\n', a seeded quality string, '\\n'."""
    n, L = reads.shape
    rec = np.empty((n, 3 + L + 3 + L + 1), dtype=np.uint8)
    rec[:, 0:3] = np.frombuffer(b"@r\n", dtype=np.uint8)
    rec[:, 3:3 + L] = reads
    rec[:, 3 + L:6 + L] = np.frombuffer(b"\n+\n", dtype=np.uint8)
    rec[:, 6 + L:6 + 2 * L] = np.random.default_rng(seed_qual).integers(33, 75, (n, L), dtype=np.uint8)
    rec[:, -1] = ord("\n")
    return rec.reshape(-1)
