"""Pure-Python helpers for the tests: independent routes to facts the oracle
must agree with, written from the definitions in "cuSBF: A Minimizer-Aware
Bloom Filter for Genomic Sequence Data on Modern GPUs" (§II-B, §IV-B..E).

They work on strings, not on packed k-mers: every sub-window is cut out of the
text and packed on its own, so a wrong shift, mask or index in the oracle's
integer arithmetic shows up as a mismatch.  They only call the oracle's hash
primitives, which are pinned separately (published SplitMix64 outputs and an
inverse of h_min).
"""
import math

import numpy as np

from oracle import oracle as O

CODE = {"A": 0, "C": 1, "G": 2, "T": 3, "a": 0, "c": 1, "g": 2, "t": 3}


def pack_str(s: str) -> int:
    """Base-4 number with the first base most significant."""
    v = 0
    for ch in s:
        v = v * 4 + CODE[ch]
    return v


def valid_str(s: str) -> bool:
    return all(ch in CODE for ch in s)


def minimizer_hash_str(kmer: str, m: int) -> int:
    return min(O.hmin(pack_str(kmer[i:i + m])) for i in range(len(kmer) - m + 1))


def kmer_bits_str(kmer: str, s: int, H: int):
    """{(sector, bit)} that the k-mer's s-mers set, from the text."""
    out = set()
    for j in range(len(kmer) - s + 1):
        h = O.hs(pack_str(kmer[j:j + s]))
        for t in range(H):
            out.add((t % 4, O.bitaddr(h, t, H)))
    return out


def num_shards(bits: int) -> int:
    need = -(-bits // 256)
    n = 1
    while n < need:
        n *= 2
    return n


def random_dna(rng: np.random.Generator, n: int, alphabet=b"ACGT") -> bytes:
    return np.frombuffer(alphabet, dtype=np.uint8)[rng.integers(0, len(alphabet), n)].tobytes()


def bits_of(words: np.ndarray, n: int) -> np.ndarray:
    """First n bits of LSB-first uint64 words as a 0/1 array."""
    b = np.unpackbits(np.ascontiguousarray(words, dtype="<u8").view(np.uint8), bitorder="little")
    return b[:n]


def binom_ok(hits: int, n: int, p: float, z: float = 3.5) -> bool:
    """hits within z standard deviations of Binomial(n, p) (normal approx.)."""
    mu = n * p
    sd = math.sqrt(max(n * p * (1 - p), 1e-12))
    return abs(hits - mu) <= z * sd + 1.0


def kmer_bits_wide_str(kmer: str, s: int, H: int):
    """{(word, bit)} that the k-mer's s-mers set in a 512-bit block of the
    wide variant, from the text: address a -> (a // 64, a % 64)."""
    out = set()
    for j in range(len(kmer) - s + 1):
        h = O.hs(pack_str(kmer[j:j + s]))
        for t in range(H):
            a = O.bitaddr_wide(h, t, H)
            out.add((a // 64, a % 64))
    return out


# ---- other alphabets (§IV-A: proteins 5 bits, DNA triplets 6 bits) ----------

BITS = {O.ALPHA_DNA: 2, O.ALPHA_PROTEIN: 5, O.ALPHA_TRIPLET: 6}


def symbols_of(alpha: int, text: bytes) -> list:
    """Symbol codes of a byte string, None for an invalid symbol.  Protein: a
    letter's place in A..Z (either case); triplet: the codons at bytes 3j..3j+2
    read as base-4 numbers of their bases; DNA: the base codes."""
    if alpha == O.ALPHA_PROTEIN:
        out = []
        for c in text:
            ch = chr(c)
            out.append(ord(ch.upper()) - ord("A") if ch.isascii() and ch.isalpha() else None)
        return out
    if alpha == O.ALPHA_TRIPLET:
        out = []
        for j in range(len(text) // 3):
            cod = text[3 * j:3 * j + 3].decode("latin-1")
            out.append(pack_str(cod) if valid_str(cod) else None)
        return out
    return [CODE.get(chr(c)) for c in text]


def pack_symbols(codes, b: int) -> int:
    v = 0
    for c in codes:
        v = (v << b) | c
    return v


def kmer_bits_alpha(codes, alpha: int, s: int, H: int):
    """{(sector, bit)} a k-mer of symbol codes sets, from its s-mers cut out
    of the code list and packed on their own."""
    b = BITS[alpha]
    out = set()
    for j in range(len(codes) - s + 1):
        h = O.hs(pack_symbols(codes[j:j + s], b))
        for t in range(H):
            out.add((t % 4, O.bitaddr(h, t, H)))
    return out


def minimizer_hash_alpha(codes, alpha: int, m: int) -> int:
    b = BITS[alpha]
    return min(O.hmin(pack_symbols(codes[i:i + m], b)) for i in range(len(codes) - m + 1))


def random_protein(rng: np.random.Generator, n: int, alphabet=b"ACDEFGHIKLMNPQRSTVWY") -> bytes:
    return np.frombuffer(alphabet, dtype=np.uint8)[rng.integers(0, len(alphabet), n)].tobytes()
