"""Host-side pieces of bench.py (no GPU): the count of valid k-mers that the
valid-k-mer throughput divides by, against a brute force over the text."""
import numpy as np

import bench
from tests import helpers as T


def brute(text: bytes, k: int, alpha: str) -> int:
    if alpha == "protein":
        sym = [chr(c).isascii() and chr(c).isalpha() for c in text]
    elif alpha == "triplet":
        sym = [T.valid_str(text[3 * j:3 * j + 3].decode("latin-1")) for j in range(len(text) // 3)]
    else:
        sym = [T.valid_str(chr(c)) for c in text]
    return sum(all(sym[p:p + k]) for p in range(len(sym) - k + 1))


def test_valid_kmer_count():
    rng = np.random.default_rng(3)
    for alpha, alphabet in [("dna", b"ACGTacgtN\n"), ("protein", b"ACDEFGHIKLMNPQRSTVWYxz*-1"),
                            ("triplet", b"ACGTacgtN")]:
        for k in (1, 2, 5, 12):
            for n in (0, 3, 50, 997):
                t = np.frombuffer(alphabet, dtype=np.uint8)[rng.integers(0, len(alphabet), n)]
                assert bench.valid_kmer_count(t, k, alpha) == brute(t.tobytes(), k, alpha), (alpha, k, n)
