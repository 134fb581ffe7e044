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


def test_long_read_set_parallel_equals_sequential():
    """Forked batch workers give the bytes of one process: batches joined by
    one 'N' in the order asked for."""
    genome = S.uniform_ascii_fast(300_000, 0)
    order = [5, 2, 7]
    par = S.long_read_set(genome, order, workers=3, n=300)
    seq = S.long_read_set(genome, order, workers=1, n=300)
    parts = [S.long_read_batch(genome, b, n=300) for b in order]
    want = np.concatenate([parts[0], [ord("N")], parts[1], [ord("N")], parts[2]]).astype(np.uint8)
    assert np.array_equal(par, want) and np.array_equal(seq, want)
    assert S.long_read_set(genome, [], workers=3).size == 0


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


def test_proteome_layout():
    """Residues from the 20 standard amino acids, near-uniform; one '*' per
    protein with the stated mean length; copied segments make some 20-mers
    repeat; seeded."""
    p = S.proteome(400_000)
    assert p.size == 400_000 and (p == S.proteome(400_000)).all()
    stops = int((p == S.STOP_BYTE).sum())
    res = p[p != S.STOP_BYTE]
    assert set(np.unique(res).tolist()) <= set(S.AMINO.tolist())
    freq = np.bincount(res, minlength=256)[S.AMINO] / res.size
    assert abs(freq - 0.05).max() < 0.005
    mean_len = p.size / stops
    assert 380 < mean_len < 460  # exp(ln 350 + 0.6^2 / 2) ~ 419, plus the stop byte
    win = np.lib.stride_tricks.sliding_window_view(p[:200_000], 20)
    _, counts = np.unique(win, axis=0, return_counts=True)
    assert (counts > 1).sum() > 100  # copied segments


def test_peptide_set_layout():
    """50-residue peptides joined by '*'; with no substitutions the sampled
    half are proteome substrings and the uniform half (almost) never are."""
    p = S.proteome(50_000)
    q = S.peptide_set(p, 400, err=0.0)
    assert q.size == 400 * 51 - 1
    peps = np.append(q, np.uint8(S.STOP_BYTE)).reshape(400, 51)
    assert (peps[:, 50] == S.STOP_BYTE).all()
    text = p.tobytes()
    found = sum(peps[i, :50].tobytes() in text for i in range(400))
    assert 190 <= found <= 210


def test_codon_read_set_layout():
    """150-bp reads joined by "NNN" (every read starts on a codon of the
    stream); with no substitutions the sampled half are genome substrings at
    codon-aligned offsets."""
    g = S.genome_with_repeats(60_000)
    q = S.codon_read_set(g, 300, err=0.0)
    assert q.size == 300 * 153 - 3
    reads = np.append(q, np.full(3, S.N_BYTE, dtype=np.uint8)).reshape(300, 153)
    assert (reads[:, 150:] == S.N_BYTE).all()
    gt = S.to_ascii(g).tobytes()
    hits = 0
    for r in reads[:, :150]:
        at = gt.find(r.tobytes())
        if at >= 0:
            hits += 1
            assert at % 3 == 0
    assert 140 <= hits <= 160


def test_alpha_workload_sizes():
    w = S.alpha_workload("protein", scale=0.01)
    assert w["insert"].size == 160_000 and w["bits"] == int(S.ALPHA_BITS * 0.01)
    w = S.alpha_workload("triplet", scale=0.01)
    assert w["insert"].size % 3 == 0 and w["queries"][0].size == 20_000 * 153 - 3
