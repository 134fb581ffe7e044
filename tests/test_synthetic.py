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
