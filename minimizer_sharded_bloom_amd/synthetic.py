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
  5  3 Gbp uniform genome with 'N' runs of 1-1000 bases covering 0.1% of it
     (not generated here yet).

Seeds: genome 0, foreign sequence 1, repeats 2, read starts 3, read errors 4,
random reads 5, shuffle 6.
"""
from __future__ import annotations

import numpy as np

ACGT = np.frombuffer(b"ACGT", dtype=np.uint8)
N_BYTE = ord("N")

CONFIG_BITS = {1: 2**20, 2: 2**26, 3: 2**32, 4: 2**30, 5: 2**35}
CONFIG_GENOME = {1: 100_000, 2: 5_000_000, 3: 200_000_000, 4: 50_000_000, 5: 3_000_000_000}
CONFIG_READS = {2: 2_000_000, 3: 20_000_000, 4: 1_000_000}
READ_LEN = 150


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
    raise ValueError("workload %r is not generated by this module" % cfg)
