"""Host-resident input on the GPU: the chunked pinned pipeline behind
SBF_HOST insert/query and the FASTA/FASTQ entry points ([cuSBF] §IV-A input
forms, §IV-F separators, §IV-G host staging), against the oracle.  Small
chunk sizes put many chunk boundaries (k-1 bases of overlap) inside the
inputs and inside records."""
import numpy as np
import pytest

from minimizer_sharded_bloom_amd import synthetic as S
from tests import fastx_ref as R
from tests import gpu_common as G
from tests import helpers as T

pytestmark = pytest.mark.gpu

MAIN = (31, 16, 28, 4)
K = 31


@pytest.mark.parametrize("chunk", [64, 4096, 1 << 16, 1 << 27])
def test_host_pipeline_chunks(chunk):
    g = S.to_ascii(S.genome_with_repeats(300_000, seed_genome=21))
    reads = S.short_read_set(S.genome_with_repeats(300_000, seed_genome=21), 3_000)
    f = G.gpu_filter(MAIN, 2**22)
    f.set_staging(chunk)
    o = G.oracle_filter(MAIN, 2**22)
    f.insert_seq(g.tobytes())
    o.insert_seq(g)
    G.assert_words_equal(f.words(), o.words(), "host insert, chunk %d" % chunk)
    got = f.query_seq(reads.tobytes())
    G.assert_words_equal(got, o.query_seq(reads), "host query, chunk %d" % chunk)


@pytest.mark.parametrize("params", [(31, 24, 27, 4), (25, 9, 20, 12)])
def test_host_pipeline_runtime_parameters(params):
    """Parameter sets without a compiled set (run-time sliding kernels)
    through the chunked host pipeline, with chunks that are not multiples of
    a wave step: filter words and every answer bit equal the oracle's."""
    g = S.to_ascii(S.genome_with_repeats(400_000, seed_genome=23))
    reads = S.short_read_set(S.genome_with_repeats(400_000, seed_genome=23), 4_000)
    for chunk in (64, 5000, 1 << 20):
        f = G.gpu_filter(params, 2**20)
        assert not f.specialized
        f.set_staging(chunk)
        o = G.oracle_filter(params, 2**20)
        f.insert_seq(g.tobytes())
        o.insert_seq(g)
        G.assert_words_equal(f.words(), o.words(), "host insert %s, chunk %d" % (params, chunk))
        G.assert_words_equal(f.query_seq(reads.tobytes()), o.query_seq(reads),
                             "host query %s, chunk %d" % (params, chunk))


@pytest.mark.parametrize("extra", [-1, 0, 1, 63, 64, 65])
def test_host_pipeline_boundary_lengths(extra):
    """Lengths around whole chunks: n chunks of 4096 k-mer starts + k - 1 + extra."""
    chunk = 4096
    for nchunks in (1, 3):
        n = nchunks * chunk + K - 1 + extra
        seq = S.to_ascii(S.uniform_codes(n, 40 + nchunks))
        f = G.gpu_filter(MAIN, 2**18)
        f.set_staging(chunk)
        o = G.oracle_filter(MAIN, 2**18)
        f.insert_seq(seq.tobytes())
        o.insert_seq(seq)
        G.assert_words_equal(f.words(), o.words(), "insert len %d" % n)
        G.assert_words_equal(f.query_seq(seq.tobytes()), o.query_seq(seq), "query len %d" % n)


def _record_counts(stream: bytes, ends, o):
    bits = T.bits_of(o.query_seq(stream), max(0, len(stream) - K + 1))
    hits, kmers, start = [], [], 0
    for e in ends:
        hits.append(int(bits[start:e].sum()))
        kmers.append(max(0, e - start - K + 1))
        start = e + 1
    return np.array(hits, dtype=np.uint64), np.array(kmers, dtype=np.uint64)


@pytest.mark.parametrize("fmt,gz,chunk", [("fasta", False, 1 << 27), ("fasta", True, 4096), ("fastq", False, 1000),
                                          ("fastq", True, 1 << 16), ("fasta", "bgzf", 1 << 16),
                                          ("fastq", "bgzf", 4096)])
def test_fastx_insert_and_query(tmp_path, fmt, gz, chunk):
    genome = S.genome_with_repeats(400_000, seed_genome=31)
    # the genome cut into contigs of mixed length, and reads from it
    cuts = np.sort(np.random.default_rng(3).integers(0, genome.size, 40))
    contigs = [c for c in np.split(S.to_ascii(genome), cuts) if c.size]
    reads = S.split_records(S.short_read_set(genome, 4_000))
    ins_path, q_path = str(tmp_path / ("g." + fmt)), str(tmp_path / ("r." + fmt))
    if fmt == "fasta":
        S.write_fasta(ins_path, contigs, width=61, gz=gz)
        S.write_fasta(q_path, reads, width=80, gz=gz)
    else:
        S.write_fastq(ins_path, contigs, gz=gz)
        S.write_fastq(q_path, reads, gz=gz)
    import gzip
    rd = (lambda p: gzip.open(p, "rb").read()) if gz else (lambda p: open(p, "rb").read())
    ins_stream, ins_ends = R.normalize(rd(ins_path))
    q_stream, q_ends = R.normalize(rd(q_path))
    assert len(ins_ends) == len(contigs) and len(q_ends) == len(reads)

    f = G.gpu_filter(MAIN, 2**22)
    f.set_staging(chunk)
    o = G.oracle_filter(MAIN, 2**22)
    st = f.insert_fastx(ins_path)
    assert st["records"] == len(contigs) and st["bases"] == len(ins_stream)
    o.insert_seq(ins_stream)
    G.assert_words_equal(f.words(), o.words(), "fastx insert")
    hits, kmers, st = f.query_fastx(q_path)
    want_hits, want_kmers = _record_counts(q_stream, q_ends, o)
    assert st["records"] == len(reads)
    assert (kmers == want_kmers).all()
    assert (hits == want_hits).all(), np.flatnonzero(hits != want_hits)[:10]
    # capped output: the first records only, the count of all
    h2, k2, st2 = f.query_fastx(q_path, max_records=10)
    assert h2.size == 10 and (h2 == want_hits[:10]).all() and st2["records"] == len(reads)


def test_host_pipeline_large_matches_device_path():
    """64 MB host inputs (copied into pinned memory by the copy threads) give
    the filter and answers of the device-resident path."""
    seq = S.to_ascii(S.uniform_codes(64_000_000, 77))
    dev = G.to_dev(seq)
    a = G.gpu_filter(MAIN, 2**26)
    b = G.gpu_filter(MAIN, 2**26)
    a.insert_seq(seq)  # host memory, default chunk
    b.insert_seq(dev)
    G.assert_words_equal(a.words(), b.words(), "host vs device insert")
    q = S.to_ascii(S.uniform_codes(48_000_000, 78))
    q[::997] = ord("N")
    G.assert_words_equal(a.query_seq(q), G.dev_bits_to_np(b.query_seq(G.to_dev(q))), "host vs device query")
