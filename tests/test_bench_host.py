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


def test_valid_segments():
    """The maximal valid stretches holding a k-mer (the run-count estimate's
    per-stretch term), against a brute-force scan, also when the stretches
    cross the counting chunks."""
    rng = np.random.default_rng(4)

    def brute_seg(text, k):
        n = cur = 0
        for c in text + b"N":
            if T.valid_str(chr(c)):
                cur += 1
            else:
                n += cur >= k
                cur = 0
        return n

    for k in (1, 2, 5, 12):
        for n in (0, 3, 50, 997, 4000):
            t = np.frombuffer(b"ACGTacgtN\n", dtype=np.uint8)[rng.integers(0, 10, n)]
            for chunk in (7, 64, 3 << 26):
                got = bench.valid_kmer_count(t, k, chunk=chunk, segments=True)
                assert got == (bench.valid_kmer_count(t, k), brute_seg(t.tobytes(), k)), (k, n, chunk)


def test_roofline_models():
    """The ALU and byte models of the roofline: 52 front-end instructions per
    k-mer start, +13 for the query test, +2.66 for decoding ASCII, +17.5 for
    the insert (and 2.66 more from ASCII); 0.375 B of packed input (1 B of
    ASCII) plus a 32-byte shard
    per run at 2/(w+1) runs per k-mer; the peak of 256 CUs x 4 SIMDs x 32
    lanes per clock at 2.4 GHz."""
    import pytest
    assert bench.alu_ops_per_kmer("query") == pytest.approx(65.0)
    assert bench.alu_ops_per_kmer("query_text") == pytest.approx(67.66)
    assert bench.alu_ops_per_kmer("insert") == pytest.approx(69.5)
    assert bench.alu_ops_per_kmer("insert_text") == pytest.approx(69.5 + 2.66)
    runs = 2.0 / 17
    assert bench._bytes_per_kmer("query") == pytest.approx(0.375 + 0.125 + 32 * runs)
    assert bench._bytes_per_kmer("query_text") == pytest.approx(1.0 + 0.125 + 32 * runs)
    assert bench._bytes_per_kmer("insert") == pytest.approx(0.375 + 64 * runs)
    assert bench._bytes_per_kmer("insert_text") == pytest.approx(1.0 + 64 * runs)
    assert bench.ALU_PEAK == pytest.approx(256 * 4 * 32 * 2.4e9)
    # issue slots: every 4-clock form counts twice
    assert bench.alu_issue_slots_per_kmer("query") == pytest.approx(65.0 + 33 + 5)
    assert bench.alu_issue_slots_per_kmer("query_text") == pytest.approx(67.66 + 33 + 5.91)
    assert bench.alu_issue_slots_per_kmer("insert") == pytest.approx(69.5 + 33 + 1.5)
    assert bench.alu_issue_slots_per_kmer("insert_text") == pytest.approx(72.16 + 33 + 2.41)


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says why."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert p.returncode == 2 and "one GPU" in p.stderr, (p.returncode, p.stderr[-500:])


def test_filter_level():
    """The memory row names the level the filter lives in: 1 MiB in one
    XCD's L2, 8 MiB (configuration 2) and 128 MiB in the MALL, 512 MiB
    (configuration 3) and 4 GiB (configuration 5) in HBM."""
    assert bench.filter_level(1 << 20) == "l2"
    assert bench.filter_level(8 << 20) == "mall"
    assert bench.filter_level(128 << 20) == "mall"
    assert bench.filter_level(512 << 20) == "hbm"
    assert bench.filter_level(4 << 30) == "hbm"
