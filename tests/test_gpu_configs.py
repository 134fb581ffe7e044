"""GPU parity at the full sizes of the synthetic configurations 3, 4 and 5
("cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data on Modern
GPUs", §V: out-of-cache filters, the (s, m, H) sweep and the blocked Bloom
comparison, a genome-scale filter).

The oracle side uses the threaded drivers of oracle/sbf_oracle.c (the same
per-k-mer definition, k-mer starts split over threads) and, for the 4 GiB
filter of configuration 5, the shard-sampled driver: the words of every shard
s with (s & 63) == 13 are compared exactly, and every read k-mer mapped to
one of them is answered by both sides.
"""
import os
import time

import numpy as np
import pytest

from minimizer_sharded_bloom_amd import synthetic as S
from tests import gpu_common as G
from tests import helpers as T

pytestmark = pytest.mark.gpu

MAIN = (31, 16, 28, 4)
K = 31


def progress(msg: str):
    """Progress line for long tests, appended to the file that the
    SBF_TEST_PROGRESS environment variable names (stdout is captured by
    pytest)."""
    path = os.environ.get("SBF_TEST_PROGRESS")
    if path:
        with open(path, "a") as f:
            f.write("%.1f %s\n" % (time.time(), msg))


def _full_filter_parity(params, bits, genome, kind="sbf", mt=True):
    g = G.gpu_filter(params, bits, kind)
    o = G.oracle_filter(params, bits, kind)
    g.insert_seq(G.to_dev(genome))
    progress("gpu insert done %s" % (params,))
    if mt:
        o.insert_seq_mt(genome)
    else:
        o.insert_seq(genome)
    progress("oracle insert done %s" % (params,))
    G.assert_words_equal(g.words(), o.words(), "filter %s %s" % (kind, params))
    return g, o


def test_config3_full():
    """512 MiB filter (out of every cache): the 200 Mbp genome's filter
    words all match; query bits match on every k-mer of the first 200 k reads
    and on 1 M sampled positions of all 20 M reads; probe counts match."""
    w = S.workload(3)
    progress("config 3 generated")
    g, o = _full_filter_parity(MAIN, w["bits"], w["insert"])
    reads = w["queries"][0]
    got = G.dev_bits_to_np(g.query_seq(G.to_dev(reads)))
    nk = reads.size - K + 1
    head = 200_000 * 151
    want_head = o.query_seq_mt(reads[:head])
    assert (T.bits_of(got, head - K + 1) == T.bits_of(want_head, head - K + 1)).all()
    pos = np.random.default_rng(93).integers(0, nk, 1_000_000).astype(np.uint64)
    assert (T.bits_of(got, nk)[pos.astype(np.int64)] == o.query_positions(reads, pos)).all()
    progress("config 3 query checked")
    assert g.fpr_probe(1_000_000, 0x5EED) == o.fpr_probe(1_000_000, 0x5EED)


@pytest.mark.parametrize("kind,params", [("sbf", MAIN), ("bbf", (31, 0, 0, 4))])
def test_config4_full(kind, params):
    """2^30-bit budget over the 50 Mbp genome: operating point and the
    blocked Bloom comparator, full filter, every read k-mer, probe counts."""
    w = S.workload(4)
    progress("config 4 generated")
    g, o = _full_filter_parity(params, w["bits"], w["insert"], kind)
    reads = w["queries"][0]
    got = G.dev_bits_to_np(g.query_seq(G.to_dev(reads)))
    G.assert_words_equal(got, o.query_seq_mt(reads), "config 4 query %s" % kind)
    assert g.fpr_probe(1_000_000, 0x5EED) == o.fpr_probe(1_000_000, 0x5EED)


def test_config4_sweep_points():
    """Six seeded points of the (s, m, H) grid on a 2 Mbp genome of the
    configuration-4 kind at 2^24 bits: full parity of filter, queries and probe."""
    rng = np.random.default_rng(95)
    genome = S.to_ascii(S.genome_with_repeats(2_000_000, seed_genome=11))
    reads = S.short_read_set(S.genome_with_repeats(2_000_000, seed_genome=11), 20_000)
    grid = [(s, m, H) for s in (24, 26, 28, 30) for m in (12, 16, 20) for H in (2, 3, 4, 6)]
    for idx in rng.choice(len(grid), 6, replace=False):
        s, m, H = grid[idx]
        g, o = _full_filter_parity((31, m, s, H), 2**24, genome)
        assert g.specialized
        got = G.dev_bits_to_np(g.query_seq(G.to_dev(reads)))
        G.assert_words_equal(got, o.query_seq_mt(reads), "sweep query %s" % ((s, m, H),))
        assert g.fpr_probe(300_000, s * m * H) == o.fpr_probe(300_000, s * m * H)


def test_config5_sampled():
    """2^35-bit (4 GiB) filter, 3 Gbp genome with 'N' runs: the words of every
    shard s with (s & 63) == 13 equal the oracle's (shard-sampled insert); on
    the seeded 1% long-read subsample every k-mer mapped to those shards has
    the oracle's answer; the genome's first 100 Mbp query exactly their valid
    k-mers (no false negatives, invalid k-mers false)."""
    bits = S.CONFIG_BITS[5]
    genome = S.genome_with_n_runs(S.CONFIG_GENOME[5])
    progress("config 5 genome generated")
    g = G.gpu_filter(MAIN, bits)
    g.insert_seq(G.to_dev(genome))
    progress("config 5 gpu insert done")
    words = g.words().reshape(-1, 4)
    o = G.oracle_filter(MAIN, bits)
    o.insert_seq_sampled_mt(genome, 63, 13)
    progress("config 5 oracle sampled insert done")
    want = o.words().reshape(-1, 4)
    sel = np.arange(13, want.shape[0], 64)
    G.assert_words_equal(words[sel].reshape(-1), want[sel].reshape(-1), "config 5 sampled shards")
    assert want[sel].any()
    del words, want
    # queries: the seeded 1% subsample (one batch of 10 k long reads)
    reads = S.long_read_batch(genome, S.long_read_subsample_batch())
    progress("config 5 subsample reads generated")
    got = G.dev_bits_to_np(g.query_seq(G.to_dev(reads)))
    ans, checked = o.query_seq_sampled_mt(reads, 63, 13)
    nk = reads.size - K + 1
    cb = T.bits_of(checked, nk).astype(bool)
    assert cb.sum() > 100_000
    assert (T.bits_of(got, nk)[cb] == T.bits_of(ans, nk)[cb]).all()
    # no false negatives on the genome itself, invalid k-mers answer false
    head = genome[:100_000_000]
    hb = T.bits_of(G.dev_bits_to_np(g.query_seq(G.to_dev(head))), head.size - K + 1)
    cum = np.concatenate([[0], np.cumsum(head == ord("N"), dtype=np.int64)])
    bad = (cum[K:] - cum[:-K]) > 0
    assert (hb == ~bad).all()
    progress("config 5 checked")
