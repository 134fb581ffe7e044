"""GPU parity at the full sizes of the synthetic configurations 3, 4 and 5
("cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data on Modern
GPUs", §V: out-of-cache filters, the (s, m, H) sweep and the blocked Bloom
comparison, a genome-scale filter).

The oracle side uses the threaded drivers of oracle/sbf_oracle.c (the same
per-k-mer definition, k-mer starts split over threads); every filter word is
compared, the 4 GiB filter of configuration 5 included.
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


@pytest.fixture(scope="module")
def cfg3():
    """Configuration 3 once per module: the 200 Mbp genome inserted into the
    512 MiB filter on both sides, and the GPU's answers for the 20 M reads."""
    w = S.workload(3)
    progress("config 3 generated")
    g, o = _full_filter_parity(MAIN, w["bits"], w["insert"])
    reads = w["queries"][0]
    progress("config 3 gpu query of %d bases" % reads.size)
    got = G.dev_bits_to_np(g.query_seq(G.to_dev(reads)))
    yield {"w": w, "g": g, "o": o, "reads": reads, "got": got}
    g.close()
    o.close()


def test_config3_full(cfg3):
    """512 MiB filter (out of every cache): the 200 Mbp genome's filter
    words all match, every answer bit of all 20 M reads (3.02 G k-mer
    starts) equals the threaded oracle's, and probe counts match."""
    g, o, reads, got = cfg3["g"], cfg3["o"], cfg3["reads"], cfg3["got"]
    progress("config 3 oracle query of %d bases" % reads.size)
    G.assert_words_equal(got, o.query_seq_mt(reads), "config 3 query, every k-mer")
    progress("config 3 query checked")
    assert g.fpr_probe(1_000_000, 0x5EED) == o.fpr_probe(1_000_000, 0x5EED)


def test_config3_reads(cfg3):
    """The per-read query of configuration 3's 20 M reads (150 bases at a
    stride of 151, one launch of the per-read kernel): every answer word
    equals the bits that the one-sequence query gave the same k-mers (checked
    against the oracle in test_config3_full), and 200 k seeded k-mers equal
    the oracle's own answers."""
    torch = G.torch_cuda()
    g, o, reads, got = cfg3["g"], cfg3["o"], cfg3["reads"], cfg3["got"]
    L, stride = S.READ_LEN, S.READ_LEN + 1
    n = (reads.size + 1) // stride
    assert (n - 1) * stride + L == reads.size
    progress("config 3 per-read query of %d reads" % n)
    res = g.query_reads(G.to_dev(reads), n, L, stride)
    torch.cuda.synchronize()
    res = res.cpu().numpy().view(np.uint32)
    nkr = L - K + 1
    R = (nkr + 31) // 32
    assert res.shape == (n, R)
    # the same bits cut out of the one-sequence answers, read by read
    b = (np.arange(n, dtype=np.uint64)[:, None] * np.uint64(stride) + np.uint64(32) * np.arange(R, dtype=np.uint64)[None, :])
    w = (b >> np.uint64(6)).astype(np.int64)
    sh = b & np.uint64(63)
    g2 = np.concatenate([got, np.zeros(1, dtype=np.uint64)])
    v = g2[w] >> sh
    hi = sh > np.uint64(32)
    v[hi] |= g2[w[hi] + 1] << (np.uint64(64) - sh[hi])
    left = nkr - 32 * np.arange(R)
    mask = np.where(left >= 32, 0xFFFFFFFF, (1 << np.minimum(left, 31)) - 1).astype(np.uint64)
    want = (v & mask[None, :]).astype(np.uint32)
    bad = np.argwhere(res != want)
    assert bad.size == 0, "per-read words differ: %d; first %s got %#x want %#x" % (
        bad.shape[0], bad[0], int(res[tuple(bad[0])]), int(want[tuple(bad[0])]))
    progress("config 3 per-read query equals the one-sequence query")
    rng = np.random.default_rng(98)
    r = rng.integers(0, n, 200_000)
    i = rng.integers(0, nkr, 200_000)
    bits = (res[r, i // 32] >> (i % 32).astype(np.uint32)) & 1
    want1 = o.query_positions(reads, (r * stride + i).astype(np.uint64))
    assert (bits.astype(np.uint8) == want1).all()
    assert want1.sum() > 1000


def _bit_slice(words: np.ndarray, start: int, n: int) -> np.ndarray:
    """Bits [start, start + n) of LSB-first uint64 words, as LSB-first words
    (bits past n zero)."""
    nw = (n + 63) // 64
    base, off = divmod(start, 64)
    w = np.zeros(nw + 1, dtype=np.uint64)
    avail = min(nw + 1, words.size - base)
    w[:avail] = words[base:base + avail]
    if off:
        out = (w[:nw] >> np.uint64(off)) | (w[1:nw + 1] << np.uint64(64 - off))
    else:
        out = w[:nw].copy()
    if n % 64:
        out[-1] &= np.uint64((1 << (n % 64)) - 1)
    return out


def test_query_beyond_2e32_starts(cfg3):
    """One query launch of more than 2^32 k-mer starts (the size of the
    genome-scale query, [cuSBF] §V-F): the configuration-3 reads twice,
    joined by one 'N' -- 6.04 G bases -- against the configuration-3 filter.
    The first copy's answers equal the single-copy answers (checked against
    the oracle in test_config3_full); the k k-mers that span the joining 'N'
    answer 0; the second copy's answers, which start at bit L + 1 (past 2^32
    for most of them), equal the first copy's word for word after the shift;
    and 200 k seeded positions past 2^32 equal the oracle's own answers for
    the same k-mers."""
    torch = G.torch_cuda()
    g, o, reads, got = cfg3["g"], cfg3["o"], cfg3["reads"], cfg3["got"]
    L = reads.size
    nk = L - K + 1
    one = G.to_dev(reads)
    sep = torch.tensor([ord("N")], dtype=torch.uint8, device=one.device)
    two = torch.cat([one, sep, one])
    del one
    assert two.numel() == 2 * L + 1 and two.numel() - K + 1 > 2**32
    assert two.data_ptr() % 16 == 0  # the kernel reads the ASCII itself
    progress("query of %d bases in one launch" % two.numel())
    res = G.dev_bits_to_np(g.query_seq(two))
    del two
    torch.cuda.synchronize()
    nk2 = 2 * L + 1 - K + 1
    assert res.size == (nk2 + 63) // 64
    progress("doubled query done")
    G.assert_words_equal(_bit_slice(res, 0, nk), _bit_slice(got, 0, nk), "first copy")
    assert not _bit_slice(res, nk, K).any(), "k-mers across the separator"
    G.assert_words_equal(_bit_slice(res, L + 1, nk), _bit_slice(got, 0, nk), "second copy (bit offset L + 1)")
    if nk2 % 64:
        assert int(res[-1]) >> (nk2 % 64) == 0, "bits past the last k-mer start"
    # the oracle on seeded positions past 2^32 (the same k-mers of the reads)
    rng = np.random.default_rng(97)
    pos = rng.integers(2**32, nk2, 200_000).astype(np.uint64)
    bits = (res[(pos >> np.uint64(6)).astype(np.int64)] >> (pos & np.uint64(63))) & np.uint64(1)
    want = o.query_positions(reads, pos - np.uint64(L + 1))
    assert (bits.astype(np.uint8) == want).all()
    assert want.sum() > 1000
    progress("doubled query checked")


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


def test_config5_full():
    """2^35-bit (4 GiB) filter, 3 Gbp genome with 'N' runs ([cuSBF] §V-F,
    genome-scale filters): every word of the filter equals the oracle's
    (threaded per-k-mer insert); every k-mer of the seeded 1% long-read
    subsample has the oracle's answer; the genome's first 100 Mbp query
    exactly their valid k-mers (no false negatives, invalid k-mers false)."""
    bits = S.CONFIG_BITS[5]
    genome = S.genome_with_n_runs(S.CONFIG_GENOME[5])
    progress("config 5 genome generated")
    g = G.gpu_filter(MAIN, bits)
    g.insert_seq(G.to_dev(genome))
    words = g.words()
    progress("config 5 gpu insert done")
    o = G.oracle_filter(MAIN, bits)
    o.insert_seq_mt(genome)
    progress("config 5 oracle insert done")
    ow = np.ctypeslib.as_array(O_words_ptr(o), shape=(words.size,))
    G.assert_words_equal(words, ow, "config 5 filter")
    assert (words != 0).mean() > 0.5
    del words, ow
    # queries: the seeded 1% subsample (one batch of 10 k long reads)
    reads = S.long_read_batch(genome, S.long_read_subsample_batch())
    progress("config 5 subsample reads generated (%d bases)" % reads.size)
    got = G.dev_bits_to_np(g.query_seq(G.to_dev(reads)))
    G.assert_words_equal(got, o.query_seq_mt(reads), "config 5 subsample query")
    # no false negatives on the genome itself, invalid k-mers answer false
    head = genome[:100_000_000]
    hb = T.bits_of(G.dev_bits_to_np(g.query_seq(G.to_dev(head))), head.size - K + 1)
    cum = np.concatenate([[0], np.cumsum(head == ord("N"), dtype=np.int64)])
    bad = (cum[K:] - cum[:-K]) > 0
    assert (hb == ~bad).all()
    progress("config 5 checked")
    g.close()
    o.close()


def O_words_ptr(o):
    """The oracle filter's own word array (no 4 GiB copy)."""
    from oracle import oracle as O
    return O.lib().osbf_words(o._h)
