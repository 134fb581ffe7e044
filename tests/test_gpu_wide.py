"""GPU parity of the wide-block variant (512-bit blocks, each hash
addressing the whole block; the CPU reference's layout in "cuSBF: A
Minimizer-Aware Bloom Filter for Genomic Sequence Data on Modern GPUs",
§V-D) against the oracle: filter words, query bits, probe counts."""
import numpy as np
import pytest

from minimizer_sharded_bloom_amd import synthetic as S
from tests import gpu_common as G
from tests import helpers as T

pytestmark = pytest.mark.gpu

EDGE = [0, 1, 30, 31, 32, 63, 64, 65, 1007, 1008, 1009, 2016, 2047, 2048, 4033, 8192 + 31, 12345]


def _pair(params, bits, inserts, queries):
    g = G.gpu_filter(params, bits, "wide")
    o = G.oracle_filter(params, bits, "wide")
    assert g.words_per_shard == 8 and g.num_shards == o.num_shards
    for seq in inserts:
        o.insert_seq(seq)
        g.insert_seq(G.to_dev(seq))
    G.assert_words_equal(g.words(), o.words(), "wide filter %s" % (params,))
    for i, seq in enumerate(queries):
        G.assert_words_equal(G.dev_bits_to_np(g.query_seq(G.to_dev(seq))), o.query_seq(seq),
                             "wide query %d %s" % (i, params))
    return g, o


@pytest.mark.parametrize("params", [(31, 16, 28, 4), (31, 16, 24, 2), (31, 12, 30, 6), (31, 16, 28, 8),
                                    (21, 11, 19, 3), (32, 16, 28, 4), (9, 5, 6, 12)])
def test_wide_parity(params):
    genome = S.genome_with_repeats(40000, seed_genome=sum(params))
    reads = S.short_read_set(genome, 300)
    g, o = _pair(params, 2**17, [S.to_ascii(genome)], [reads])
    assert g.fpr_probe(50000, 9) == o.fpr_probe(50000, 9)


@pytest.mark.parametrize("params", [(31, 16, 28, 4), (31, 8, 28, 4)])
def test_wide_edge_lengths(params):
    rng = np.random.default_rng(61 + sum(params))
    ins = [T.random_dna(rng, L) for L in EDGE]
    qs = [T.random_dna(rng, L) for L in EDGE] + ins[-4:]
    _pair(params, 2**14, ins, qs)


def test_wide_config4_full():
    """2^30-bit wide filter over the 50 Mbp configuration-4 genome: whole
    filter, every read k-mer, probe counts; its FPR is below the sectorized
    filter's at the same budget."""
    w = S.workload(4)
    g = G.gpu_filter((31, 16, 28, 4), w["bits"], "wide")
    o = G.oracle_filter((31, 16, 28, 4), w["bits"], "wide")
    g.insert_seq(G.to_dev(w["insert"]))
    o.insert_seq_mt(w["insert"])
    G.assert_words_equal(g.words(), o.words(), "wide cfg4 filter")
    reads = w["queries"][0]
    G.assert_words_equal(G.dev_bits_to_np(g.query_seq(G.to_dev(reads))), o.query_seq_mt(reads), "wide cfg4 query")
    n = 2_000_000
    hw = g.fpr_probe(n, 0x5EED)
    assert hw == o.fpr_probe(n, 0x5EED)
    s = G.gpu_filter((31, 16, 28, 4), w["bits"])
    s.insert_seq(G.to_dev(w["insert"]))
    assert hw < s.fpr_probe(n, 0x5EED)


def test_wide_overflow_paths():
    """m = k: every k-mer is its own segment, so every wave has more segments
    than LDS records and takes the per-k-mer paths of insert and query."""
    rng = np.random.default_rng(71)
    ins = [T.random_dna(rng, L) for L in (5000, 20011)]
    qs = [T.random_dna(rng, 9000)] + ins
    g, _ = _pair((31, 31, 28, 4), 2**16, ins, qs)
    assert g.specialized
