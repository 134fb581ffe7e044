"""The seeded workload generators produce the shapes and statistics their
recipes state (module docstring of minimizer_sharded_bloom_amd.synthetic)."""
import numpy as np

from minimizer_sharded_bloom_amd import synthetic as S


def test_uniform_is_seeded_and_uniform():
    a = S.uniform_codes(200000, 0)
    assert (a == S.uniform_codes(200000, 0)).all()
    assert not (a == S.uniform_codes(200000, 1)).all()
    counts = np.bincount(a, minlength=4)
    assert counts.size == 4 and abs(counts / a.size - 0.25).max() < 0.01


def test_genome_with_repeats():
    G = 400000
    base = S.uniform_codes(G, 0)
    g = S.genome_with_repeats(G)
    assert g.size == G and g.dtype == np.uint8 and g.max() <= 3
    changed = (g != base).mean()
    # about 5% of positions overwritten by copies, of which 3/4 differ from before
    assert 0.02 < changed < 0.08


def test_substitution_rate():
    rng = np.random.default_rng(3)
    a = np.zeros(10**6, dtype=np.uint8)
    S.substitute(a, 0.01, rng)
    assert abs((a != 0).mean() - 0.01) < 0.001
    assert set(np.unique(a)) <= {0, 1, 2, 3}


def test_short_read_set_layout():
    g = S.genome_with_repeats(50000)
    r = S.short_read_set(g, 1000)
    assert r.size == 1000 * 151 - 1
    seps = np.flatnonzero(r == ord("N"))
    assert (seps == np.arange(1, 1000) * 151 - 1).all()
    assert set(np.unique(r)) == set(b"ACGTN")


def test_workload1():
    w = S.workload(1)
    assert w["bits"] == 2**20 and w["insert"].size == 100000
    assert len(w["queries"]) == 2 and (w["queries"][0] == w["insert"]).all()


def test_uniform_ascii_fast():
    a = S.uniform_ascii_fast(1_000_003, 5)
    assert a.size == 1_000_003 and (a == S.uniform_ascii_fast(1_000_003, 5)).all()
    assert set(np.unique(a)) == set(b"ACGT")
    counts = np.array([(a == c).mean() for c in b"ACGT"])
    assert abs(counts - 0.25).max() < 0.003


def test_genome_with_n_runs():
    G = 10_000_000
    g = S.genome_with_n_runs(G)
    n = int((g == ord("N")).sum())
    # runs of 1..1000 until their lengths reach 0.1% of G; overlaps can only lower the count
    assert 0.8 * G * 0.001 < n <= G * 0.001 + 1000
    assert set(np.unique(g)) == set(b"ACGTN")
    assert ((g != ord("N")) == (S.uniform_ascii_fast(G, 0) == g)).all()


def _split_reads(batch):
    seps = np.flatnonzero(batch == ord("N"))
    return np.diff(np.concatenate([[-1], seps, [batch.size]])) - 1


def test_long_read_batch_layout_and_lengths():
    genome = S.uniform_ascii_fast(2_000_000, 0)
    b = S.long_read_batch(genome, 3, n=3000)
    assert (b == S.long_read_batch(genome, 3, n=3000)).all()
    assert not np.array_equal(b[:1000], S.long_read_batch(genome, 4, n=3000)[:1000])
    lens = _split_reads(b)
    assert lens.size == 3000 and set(np.unique(b)) == set(b"ACGTN")
    # log-normal around 10 kbp with sigma 0.5; indels change lengths by ~1%
    assert abs(np.median(lens) / 10_000 - 1) < 0.05
    assert abs(np.log(lens).std() - 0.5) < 0.03
    assert lens.min() >= 900 and lens.max() <= 51_000


def test_long_read_batch_error_free_reads_are_genome_substrings():
    genome = S.uniform_ascii_fast(500_000, 0)
    b = S.long_read_batch(genome, 0, n=200, err=0.0)
    lens = _split_reads(b)
    rl = np.random.default_rng([9, 0])
    want = np.clip(np.rint(np.exp(rl.normal(np.log(10_000.0), 0.5, 200))), 1000, 50_000).astype(np.int64)
    starts = rl.integers(0, genome.size - want + 1)
    assert (lens == want).all()
    pos = 0
    for s0, l0 in zip(starts, lens):
        assert (b[pos:pos + l0] == genome[s0:s0 + l0]).all()
        pos += l0 + 1


def test_long_read_batch_error_rate():
    """5% errors split equally over substitution, insertion and deletion:
    the length change of a read is its insertions minus its deletions (mean 0,
    variance 2 * 0.05/3 per template base), and the first base where a read
    leaves its error-free twin lies about 1/0.05 bases in."""
    genome = S.uniform_ascii_fast(1_000_000, 0)
    clean = S.long_read_batch(genome, 1, n=1000, err=0.0)
    noisy = S.long_read_batch(genome, 1, n=1000)
    lc, ln = _split_reads(clean), _split_reads(noisy)
    d = ln - lc
    assert abs(d.sum()) < 5 * np.sqrt(2 * 0.05 / 3 * lc.sum())
    assert abs(np.var(d / np.sqrt(lc)) - 2 * 0.05 / 3) < 0.004
    # an insertion or deletion that repeats the neighbouring base shows up a little later
    pc = np.concatenate([[0], np.cumsum(lc + 1)])
    pn = np.concatenate([[0], np.cumsum(ln + 1)])
    first = []
    for i in range(1000):
        a, c = clean[pc[i]:pc[i] + 200], noisy[pn[i]:pn[i] + 200]
        m = min(a.size, c.size)
        diff = np.flatnonzero(a[:m] != c[:m])
        first.append(diff[0] if diff.size else m)
    assert 15 < np.mean(first) < 30
