"""GPU parity of the protein (26 symbols, 5 bits) and DNA-triplet (64
codons, 6 bits, three bytes per symbol) Super Bloom filters of "cuSBF: A
Minimizer-Aware Bloom Filter for Genomic Sequence Data on Modern GPUs"
(§IV-A) against the oracle: filter words and query bits bit-exact, probe
counts equal, for device and host input, ragged lengths, invalid symbols,
the workload sizes the benchmark times, and the calls these filters refuse."""
import ctypes

import numpy as np
import pytest

import minimizer_sharded_bloom_amd as M
from minimizer_sharded_bloom_amd import _lib
from minimizer_sharded_bloom_amd import synthetic as S
from tests import gpu_common as G
from tests import helpers as T

pytestmark = pytest.mark.gpu

PARAMS = {
    "protein": [(12, 6, 10, 4), (9, 4, 7, 3), (5, 5, 5, 12), (12, 12, 12, 1), (1, 1, 1, 2), (8, 3, 8, 6),
                (12, 1, 1, 4)],
    "triplet": [(10, 5, 8, 4), (7, 3, 7, 2), (10, 10, 6, 11), (1, 1, 1, 4), (4, 2, 3, 4), (10, 2, 10, 8)],
}
CASES = [(a, p) for a in PARAMS for p in PARAMS[a]]
# parameter sets with compile-time kernels; every other set takes the
# run-time kernels of its alphabet
SPECIALIZED = {"protein": [(12, 6, 10, 4), (9, 4, 7, 3)], "triplet": [(10, 5, 8, 4), (7, 3, 7, 2)]}


def text(alpha, rng, nsym, bad=0.002):
    """nsym symbols of the alphabet (bytes: nsym or 3 nsym) with invalid
    symbols at rate `bad`."""
    if alpha == "protein":
        t = bytearray(T.random_protein(rng, nsym, b"ACDEFGHIKLMNPQRSTVWYacdefghXBZ"))
        for p in np.flatnonzero(rng.random(nsym) < bad):
            t[p] = b"*-.1 "[int(rng.integers(0, 5))]
    else:
        t = bytearray(T.random_dna(rng, 3 * nsym, b"ACGTacgt"))
        for p in np.flatnonzero(rng.random(3 * nsym) < bad / 3):
            t[p] = ord("N")
    return bytes(t)


def pair(alpha, params, bits, inserts, queries, host=False):
    g = G.gpu_filter(params, bits, alpha)
    o = G.oracle_filter(params, bits, alpha)
    assert g.num_shards == o.num_shards and g.alphabet == (1 if alpha == "protein" else 2)
    for seq in inserts:
        o.insert_seq(seq)
        g.insert_seq(seq if host else G.to_dev(seq))
    G.assert_words_equal(g.words(), o.words(), "%s filter %s" % (alpha, params))
    for i, seq in enumerate(queries):
        got = g.query_seq(seq) if host else G.dev_bits_to_np(g.query_seq(G.to_dev(seq)))
        G.assert_words_equal(got, o.query_seq(seq), "%s query %d %s" % (alpha, i, params))
    return g, o


@pytest.mark.parametrize("alpha,params", CASES)
def test_alpha_parity(alpha, params):
    """Several 2048-k-mer tasks, a ragged tail, a related and an unrelated
    query set, and the probe count."""
    rng = np.random.default_rng(sum(params) + len(alpha))
    ins = text(alpha, rng, 20011)
    qs = [ins[:9000], text(alpha, rng, 7777)]
    g, o = pair(alpha, params, 2**15, [ins], qs)
    assert g.specialized == (params in SPECIALIZED[alpha])
    assert g.fpr_probe(100_000, 0xA1) == o.fpr_probe(100_000, 0xA1)


@pytest.mark.parametrize("alpha", ["protein", "triplet"])
def test_alpha_edge_lengths(alpha):
    """Lengths around k, the 65-k k-mers of one wave step, the 2048-k-mer
    task and the 64-bit answer words; triplet texts with 1 or 2 bytes past
    the last codon."""
    params = PARAMS[alpha][0]
    k = params[0]
    rng = np.random.default_rng(7 + len(alpha))
    step = 65 - k
    lens = [0, 1, k - 1, k, k + 1, step + k - 1, step + k, 2 * step + k - 1, 63 + k, 64 + k, 2047 + k, 2048 + k - 1,
            2049 + k, 4096 + k - 1, 4097 + k, 6000]
    ins = [text(alpha, rng, L) for L in lens]
    if alpha == "triplet":
        ins += [text(alpha, rng, 3000) + b"AC", text(alpha, rng, 2500) + b"G", b"ACG" * k + b"TT"]
    qs = [text(alpha, rng, L) for L in lens] + ins[-5:]
    pair(alpha, params, 2**13, ins, qs)


@pytest.mark.parametrize("alpha,params", [(a, p) for a in SPECIALIZED for p in SPECIALIZED[a]])
def test_alpha_text_front_end_edges(alpha, params):
    """The compile-time sets read 16 symbols per lane, 1008 k-mer starts per
    wave, and take byte loads only in the wave that reaches the end of the
    text (one whose 1024 symbols are not all present): lengths around a lane,
    a wave and that limit, texts ending at every offset of a lane, invalid
    symbols at lane edges, triplet texts with stray bytes after the last
    codon."""
    k = params[0]
    rng = np.random.default_rng(11 + sum(params) + len(alpha))
    lens = [k, k + 1, 15 + k, 16 + k, 17 + k, 1007 + k, 1008 + k, 1009 + k, 1023, 1024, 1025, 1023 + k, 1024 + k,
            1040 + k, 2015 + k, 2016 + k, 2017 + k, 3024 + k] + [5000 + d for d in range(16)]
    ins = [text(alpha, rng, L) for L in lens]
    edge = bytearray(text(alpha, rng, 4000))
    sb = 3 if alpha == "triplet" else 1
    for lane_start in range(0, 4000, 16):
        for d in (-1, 0, 15):
            p = lane_start + d
            if 0 <= p < 4000 and rng.random() < 0.3:
                edge[sb * p] = ord("*" if alpha == "protein" else "N")
    ins.append(bytes(edge))
    if alpha == "triplet":
        ins += [text(alpha, rng, 1024) + b"A", text(alpha, rng, 1008 + k) + b"GT"]
    qs = [text(alpha, rng, L) for L in lens[::2]] + ins[-4:]
    g, _ = pair(alpha, params, 2**14, ins, qs)
    assert g.specialized


@pytest.mark.parametrize("alpha", ["protein", "triplet"])
def test_alpha_host_pipeline(alpha):
    """Host input through the chunked pipeline with tiny chunks (k-1 symbols
    of overlap, a triplet chunk is 3 bytes per symbol) equals the oracle."""
    params = PARAMS[alpha][0]
    rng = np.random.default_rng(17 + len(alpha))
    ins = text(alpha, rng, 50_000)
    qs = [text(alpha, rng, 33_333) + (b"AC" if alpha == "triplet" else b""), ins[:20000]]
    g = G.gpu_filter(params, 2**16, alpha)
    g.set_staging(64 * 37)
    o = G.oracle_filter(params, 2**16, alpha)
    o.insert_seq(ins)
    g.insert_seq(ins)
    G.assert_words_equal(g.words(), o.words(), "%s host insert" % alpha)
    for i, q in enumerate(qs):
        G.assert_words_equal(g.query_seq(q), o.query_seq(q), "%s host query %d" % (alpha, i))
    g.set_staging(1 << 20)
    for i, q in enumerate(qs):
        G.assert_words_equal(g.query_seq(q), o.query_seq(q), "%s host query %d, one chunk" % (alpha, i))


def test_alpha_refused_calls(tmp_path):
    """Packed input and FASTA/FASTQ files are DNA only; bad alphabets and k
    past the 64-bit packing are refused at creation."""
    g = G.gpu_filter(PARAMS["protein"][0], 2**12, "protein")
    L = M.lib()
    torch = G.torch_cuda()
    cw, vw = M.packed_words(100)
    codes = torch.zeros(cw, dtype=torch.int32, device="cuda")
    valid = torch.zeros(vw, dtype=torch.int32, device="cuda")
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    assert L.sbf_insert_packed(g.handle, codes.data_ptr(), valid.data_ptr(), 100, None) == _lib.SBF_EUNSUPPORTED
    assert L.sbf_query_packed(g.handle, codes.data_ptr(), valid.data_ptr(), 100, out.data_ptr(),
                              None) == _lib.SBF_EUNSUPPORTED
    p = tmp_path / "x.fa"
    p.write_bytes(b">a\nACDEFGHIKL\n")
    assert L.sbf_insert_fastx(g.handle, str(p).encode(), None) == _lib.SBF_EUNSUPPORTED
    assert L.sbf_query_fastx(g.handle, str(p).encode(), None, None, 0, None) == _lib.SBF_EUNSUPPORTED
    h = ctypes.c_void_p()
    for alpha, k in [(1, 13), (2, 11), (3, 5)]:
        assert L.sbf_create_alphabet(ctypes.byref(h), alpha, k, 2, 2, 4, 4096) == _lib.SBF_EINVAL
    assert not h.value
    torch.cuda.synchronize()


@pytest.mark.parametrize("alpha", ["protein", "triplet"])
def test_alpha_full_workload(alpha):
    """The timed workload at full size (16 M symbols inserted into 2^28 bits,
    2 M queries): whole filter and every query bit against the threaded
    oracle, probe counts equal."""
    w = S.alpha_workload(alpha)
    params = PARAMS[alpha][0]
    g = G.gpu_filter(params, w["bits"], alpha)
    o = G.oracle_filter(params, w["bits"], alpha)
    g.insert_seq(G.to_dev(w["insert"]))
    o.insert_seq_mt(w["insert"])
    G.assert_words_equal(g.words(), o.words(), "%s full filter" % alpha)
    q = w["queries"][0]
    got = G.dev_bits_to_np(g.query_seq(G.to_dev(q)))
    want = o.query_seq_mt(q)
    G.assert_words_equal(got, want, "%s full query" % alpha)
    frac = T.bits_of(want, g.num_symbols(q.size) - g.k + 1).mean()
    assert 0.05 < frac < 0.6  # sampled queries hit, uniform ones mostly do not
    n = 2_000_000
    assert g.fpr_probe(n, 0x5EED) == o.fpr_probe(n, 0x5EED)
