"""GPU parity: filter words after insert, query bit vectors and probe counts
of the HIP library must be bit-identical to the CPU oracle on the same seeded
inputs ("cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data on
Modern GPUs", Algorithms 1 and 2, §V-D)."""
import os

import numpy as np
import pytest

from minimizer_sharded_bloom_amd import synthetic as S
from oracle import oracle as O
from tests import gpu_common as G
from tests import helpers as T

pytestmark = pytest.mark.gpu

MAIN = (31, 16, 28, 4)


def _run_pair(params, bits, inserts, queries, kind="sbf", device=True):
    """Insert `inserts` then query `queries` on both sides; compare."""
    g = G.gpu_filter(params, bits, kind)
    o = G.oracle_filter(params, bits, kind)
    for seq in inserts:
        o.insert_seq(seq)
        g.insert_seq(G.to_dev(seq) if device else seq)
    G.assert_words_equal(g.words(), o.words(), "filter %s %s" % (kind, params))
    for qi, seq in enumerate(queries):
        want = o.query_seq(seq)
        if device:
            got = G.dev_bits_to_np(g.query_seq(G.to_dev(seq)))
        else:
            got = g.query_seq(seq)
        G.assert_words_equal(got, want, "query %d %s %s" % (qi, kind, params))
    return g, o


def test_pack_layout():
    """sbf_pack writes the layout of include/sbf.h: 16 bases per code word,
    first base in the top bits; validity bit j of word j/32."""
    import minimizer_sharded_bloom_amd as M
    rng = np.random.default_rng(31)
    alphabet = np.frombuffer(b"ACGTacgtNnRYX\n>", dtype=np.uint8)
    for n in [1, 15, 16, 17, 31, 32, 33, 1000, 4097, 65536 + 5]:
        a = alphabet[rng.integers(0, alphabet.size, n)]
        codes, valid = M.pack(G.to_dev(a))
        codes = codes.cpu().numpy().view(np.uint32)
        valid = valid.cpu().numpy().view(np.uint32)
        code = np.array([T.CODE.get(chr(c), 0) for c in a], dtype=np.uint64)
        ok = np.array([chr(c) in T.CODE for c in a], dtype=np.uint64)
        cw, vw = M.packed_words(n)
        want_c = np.zeros(cw, dtype=np.uint64)
        want_v = np.zeros(vw, dtype=np.uint64)
        j = np.arange(n, dtype=np.uint64)
        np.bitwise_or.at(want_c, j // 16, (code * ok) << (np.uint64(30) - np.uint64(2) * (j % 16)))
        np.bitwise_or.at(want_v, j // 32, ok << (j % 32))
        assert (codes[:cw] & _valid_code_mask(ok, n, cw)).tolist() == (want_c.astype(np.uint32)).tolist()
        assert valid[:vw].tolist() == want_v.astype(np.uint32).tolist()


def _valid_code_mask(ok, n, cw):
    """Codes of invalid bases are unspecified: mask them out."""
    m = np.zeros(cw, dtype=np.uint64)
    j = np.arange(n, dtype=np.uint64)
    np.bitwise_or.at(m, j // 16, (ok * np.uint64(3)) << (np.uint64(30) - np.uint64(2) * (j % 16)))
    return m.astype(np.uint32)


def test_config1_tiny():
    """Configuration 1: 100 kbp inserted, itself and a foreign 100 kbp queried."""
    w = S.workload(1)
    g, o = _run_pair(MAIN, w["bits"], [w["insert"]], w["queries"])
    assert g.specialized
    nk = w["insert"].size - 31 + 1
    own = T.bits_of(o.query_seq(w["insert"]), nk)
    assert own.all()  # no false negatives
    fp = int(T.bits_of(o.query_seq(w["queries"][1]), nk).sum())
    assert fp < 500  # FPR of random foreign 31-mers stays far below 1%


def test_host_entry_points():
    w = S.workload(1)
    _run_pair(MAIN, w["bits"], [w["insert"][:50000].tobytes()], [w["queries"][1][:30001].tobytes()], device=False)


EDGE_LENGTHS = [0, 1, 30, 31, 32, 33, 46, 47, 63, 64, 65, 95, 127, 1007, 1008, 1009, 1038, 1039, 1040,
                2016, 2047, 2048, 2049, 4031, 4032, 4033, 8192 + 31, 12345]


@pytest.mark.parametrize("params", [MAIN, (9, 5, 6, 3), (31, 31, 31, 4), (32, 16, 28, 4), (21, 1, 19, 5),
                                    (31, 16, 28, 12), (31, 12, 24, 6), (31, 20, 30, 2)])
def test_edge_lengths_specialized(params):
    rng = np.random.default_rng(41 + sum(params))
    ins = [T.random_dna(rng, L) for L in EDGE_LENGTHS]
    qs = [T.random_dna(rng, L) for L in EDGE_LENGTHS] + ins[-6:]
    _run_pair(params, 2**14, ins, qs)


@pytest.mark.parametrize("params", [(5, 3, 4, 2), (17, 9, 13, 7), (32, 32, 1, 1), (1, 1, 1, 3), (25, 14, 25, 11),
                                    (31, 15, 27, 4), (12, 12, 6, 64)])
def test_generic_kernels(params):
    """Parameter sets without a compiled specialization run the generic
    per-k-mer kernels and must agree as well."""
    rng = np.random.default_rng(43 + sum(params))
    ins = [T.random_dna(rng, L) for L in (0, 1, 31, 64, 200, 5000)]
    qs = [T.random_dna(rng, L) for L in (1, 33, 64, 65, 3000)] + ins[-2:]
    g, _ = _run_pair(params, 2**13, ins, qs)
    assert not g.specialized


def _noisy(rng, n, pN=0.02, plow=0.05):
    """Random DNA with 'N' bases, lower case and a few other bytes."""
    a = np.frombuffer(T.random_dna(rng, n), dtype=np.uint8).copy()
    r = rng.random(n)
    a[r < pN] = ord("N")
    low = (r >= pN) & (r < pN + plow)
    a[low] = a[low] | 0x20
    a[(r >= pN + plow) & (r < pN + plow + 0.002)] = ord("\n")
    return a.tobytes()


@pytest.mark.parametrize("seed", range(6))
def test_random_noisy(seed):
    rng = np.random.default_rng(100 + seed)
    params = [MAIN, (31, 12, 26, 3), (31, 20, 24, 6), (9, 5, 6, 3)][seed % 4]
    ins = [_noisy(rng, int(rng.integers(0, 20000))) for _ in range(3)]
    qs = [_noisy(rng, int(rng.integers(0, 20000))) for _ in range(2)] + ins
    _run_pair(params, int(2 ** rng.integers(8, 18)), ins, qs)


def test_degenerate_sequences():
    """All-N, poly-A (one shard, one long run across lanes and waves),
    tandem repeats, N at every position modulo a stride."""
    n = 20000
    polyA = b"A" * n
    allN = b"N" * n
    tandem = (b"ACGTTGCA" * (n // 8))
    rng = np.random.default_rng(51)
    base = bytearray(T.random_dna(rng, n))
    for i in range(0, n, 37):
        base[i] = ord("N")
    ins = [polyA, allN, tandem, bytes(base)]
    qs = ins + [b"C" * 5000, T.random_dna(rng, 9000)]
    for params in (MAIN, (31, 12, 24, 2)):
        _run_pair(params, 2**12, ins, qs)


@pytest.mark.parametrize("kind,params", [("bbf", (31, 0, 0, 4)), ("bbf", (31, 0, 0, 2)), ("bbf", (31, 0, 0, 6)),
                                         ("bbf", (20, 0, 0, 3)), ("bbf", (31, 0, 0, 16))])
def test_blocked_bloom(kind, params):
    rng = np.random.default_rng(61 + params[3])
    ins = [_noisy(rng, 30000), T.random_dna(rng, 1009)]
    qs = [_noisy(rng, 20000)] + ins
    _run_pair(params, 2**16, ins, qs, kind=kind)


@pytest.mark.parametrize("kind,params,n", [("sbf", MAIN, 300000), ("sbf", (9, 5, 6, 3), 100000),
                                           ("sbf", (17, 9, 13, 7), 50000), ("sbf", (31, 17, 26, 4), 100000),
                                           ("sbf", (25, 14, 25, 11), 50000), ("sbf", (12, 12, 6, 64), 50000),
                                           ("sbf", (32, 32, 1, 1), 50000), ("sbf", (1, 1, 1, 3), 20000),
                                           ("bbf", (31, 0, 0, 4), 200000)])
def test_fpr_probe(kind, params, n):
    """a7: probe hit counts equal the oracle's on the same SplitMix64 stream,
    for compiled sets and for run-time ones (compile-time H from 1 to 16, and
    H = 64 read at run time)."""
    rng = np.random.default_rng(71)
    g = G.gpu_filter(params, 2**15, kind)
    o = G.oracle_filter(params, 2**15, kind)
    seq = T.random_dna(rng, 40000)
    g.insert_seq(G.to_dev(seq))
    o.insert_seq(seq)
    for seed in (0, 0x5EED, 2**64 - 1):
        assert g.fpr_probe(n, seed) == o.fpr_probe(n, seed)
    assert g.fpr_probe(0, 1) == 0


@pytest.mark.parametrize("m", [12, 16, 20])
def test_sweep_instantiations(m):
    """Every (s, H) at this m of the k = 31 sweep grid is specialized and
    bit-exact on a short genome and a few reads."""
    rng = np.random.default_rng(80 + m)
    genome = S.genome_with_repeats(30000, seed_genome=m)
    reads = S.short_read_set(genome, 200)
    gs = S.to_ascii(genome)
    for s in (24, 26, 28, 30):
        for H in (2, 3, 4, 6):
            g, o = _run_pair((31, m, s, H), 2**16, [gs], [reads])
            assert g.specialized
            assert g.fpr_probe(20000, s * H) == o.fpr_probe(20000, s * H)


GRID_SLICES = ([(31, 16, s, 4) for s in (16, 17, 18, 19, 20, 21, 22, 23, 25, 27, 29, 31)]
               + [(31, m, 28, 4) for m in (8, 9, 10, 11, 13, 14, 15, 17, 18, 19, 21, 22, 23, 24, 25, 26, 27, 28,
                                          29, 30, 31)]
               + [(31, 16, 28, H) for H in (1, 5, 8, 16)]
               + [(31, m, s, 4) for s in (23, 24, 25, 26) for m in (21, 22, 23)])


def test_grid_slices():
    """Every set of the s-, m- and H-slices through the operating point, and
    of the lowest-FPR block of the (s, m) grid, is specialized and bit-exact
    on a short genome, reads and probes."""
    genome = S.genome_with_repeats(30000, seed_genome=90)
    reads = S.short_read_set(genome, 200)
    gs = S.to_ascii(genome)
    for params in GRID_SLICES:
        g, o = _run_pair(params, 2**16, [gs], [reads])
        assert g.specialized, params
        assert g.fpr_probe(20000, sum(params)) == o.fpr_probe(20000, sum(params))


@pytest.mark.parametrize("params", [(31, 16, 16, 4), (31, 8, 28, 4), (31, 14, 28, 4), (31, 16, 28, 16)])
def test_grid_slice_edges(params):
    """Edge lengths (lane, wave and word boundaries) on the widest Findere
    window (s = 16), the widest minimizer window (m = 8, 32 k-mers per lane),
    the first m with 32 k-mers per lane, and the most hashes (H = 16)."""
    rng = np.random.default_rng(43 + sum(params))
    ins = [T.random_dna(rng, L) for L in EDGE_LENGTHS]
    qs = [T.random_dna(rng, L) for L in EDGE_LENGTHS] + ins[-6:]
    _run_pair(params, 2**14, ins, qs)


def test_repeated_launches_same_result():
    """OR is idempotent: inserting the same data with the filter not cleared,
    and again after clear, gives the same words (no lost atomic updates)."""
    w = S.workload(1)
    g = G.gpu_filter(MAIN, 2**12)
    o = G.oracle_filter(MAIN, 2**12)
    o.insert_seq(w["insert"])
    d = G.to_dev(w["insert"])
    for _ in range(3):
        g.insert_seq(d)
    G.assert_words_equal(g.words(), o.words(), "3x insert")
    g.clear()
    g.insert_seq(d)
    G.assert_words_equal(g.words(), o.words(), "after clear")


def test_config2_full():
    """Configuration 2 at full size: the 5 Mbp genome's filter words all
    match, and every answer bit of all 2 M reads (302 M k-mer starts) equals
    the threaded oracle's."""
    torch = G.torch_cuda()
    w = S.workload(2)
    g = G.gpu_filter(MAIN, w["bits"])
    o = G.oracle_filter(MAIN, w["bits"])
    g.insert_seq(G.to_dev(w["insert"]))
    o.insert_seq(w["insert"])
    G.assert_words_equal(g.words(), o.words(), "config 2 filter")
    reads = w["queries"][0]
    got = G.dev_bits_to_np(g.query_seq(G.to_dev(reads)))
    G.assert_words_equal(got, o.query_seq_mt(reads), "config 2 query, every k-mer")
    torch.cuda.synchronize()


def test_library_first_then_torch():
    """Creating a filter before torch is imported still leaves one HIP runtime
    in the process (the binding loads torch's before libsbf.so): torch sees the
    device and a device-tensor insert/query works.  Runs in a fresh child
    process, since this one has torch loaded already."""
    import subprocess
    import sys
    code = (
        "import minimizer_sharded_bloom_amd as M\n"
        "f = M.SuperBloomFilter(31, 16, 28, 4, 2**20)\n"
        "import torch\n"
        "assert torch.cuda.is_available()\n"
        "s = torch.tensor(list(b'ACGT' * 100), dtype=torch.uint8, device='cuda')\n"
        "f.insert_seq(s)\n"
        "r = f.query_seq(s).cpu()\n"
        "n = 400 - 31 + 1\n"
        "assert int(sum(bin(int(w) & (2**64 - 1)).count('1') for w in r)) == n\n"
        "print('ok')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=100)
    assert p.returncode == 0 and p.stdout.strip().endswith("ok"), p.stdout + p.stderr


def _segments_per_wave(seq: bytes, k: int, m: int, wave: int, n_waves: int) -> list:
    """Runs of equal minimizer key (low 32 bits of the minimizer hash) that
    start in each of the first n_waves blocks of `wave` k-mer starts, counted
    with the oracle's per-k-mer definition (a run entering a block counts
    there too)."""
    counts = []
    prev = None
    for w in range(n_waves):
        c = 0
        for p in range(w * wave, (w + 1) * wave):
            x = O.pack_kmer(seq[p:p + k])
            key = None if x is None else O.minimizer_hash(x, k, m) & 0xFFFFFFFF
            if key is not None and (key != prev or p == w * wave):
                c += 1
            prev = key
        counts.append(c)
    return counts


@pytest.mark.parametrize("m", [17, 21, 27, 28, 31])
def test_query_waves_at_record_limits(m):
    """Genome-scale queries at minimizer densities 2/(w+1) near the query's
    LDS record slots.  m = 17: about 252 segments per 2016-k-mer wave (32
    k-mers per lane) against 280 slots.  From w <= 11 on the query takes 16
    k-mers per lane: m = 21, about 168 per 1008-k-mer wave against 256;
    m = 27, about 337 against 352, so one launch runs both the LDS path and
    the per-k-mer path; m = 28, about 404, the per-k-mer path.  The insert
    (1008-k-mer waves, 352 slots at w <= 8) goes through its slots in rounds:
    one or two at m = 27, two at m = 28, three at m = 31 (every k-mer its own
    run).  Filter words and every query bit match the oracle."""
    rng = np.random.default_rng(300 + m)
    params = (31, m, 28, 4)
    genome = T.random_dna(rng, 300_000)
    foreign = T.random_dna(rng, 1_000_000)
    if m == 27:
        # the input reaches both sides of the 352 slots, with a margin for
        # the record a wave's idle last lane may add
        seg = np.array(_segments_per_wave(foreign, 31, m, 1008, (len(foreign) - 30) // 1008))
        assert (seg < 348).sum() >= 5 and (seg > 356).sum() >= 5, (seg.min(), seg.max())
    mutated = bytearray(genome)
    for p in rng.integers(0, len(mutated), 3000):
        mutated[p] = ord("ACGT"[(("ACGT".index(chr(mutated[p]))) + 1) % 4])
    g, _ = _run_pair(params, 2**20, [genome], [genome, bytes(mutated), foreign])
    assert g.specialized


@pytest.mark.parametrize("params", [MAIN, (31, 21, 28, 4)])
def test_query_inputs_agree(params):
    """A DNA query reads its input three ways: the query kernel decoding the
    ASCII itself (a 16-byte-aligned device sequence, 32 k-mers per lane),
    the packing pass and then the packed kernel (an unaligned device
    sequence, or parameters with 16 k-mers per lane), and sbf_query_packed
    on codes from sbf_pack.  Every way gives the oracle's bits, on text with
    lower case, 'N' runs, other letters and bytes with bit 7 set, at lengths
    around a lane (32 bases) and a wave (2016 k-mers, 2048 bytes read)."""
    import minimizer_sharded_bloom_amd as M
    torch = G.torch_cuda()
    rng = np.random.default_rng(77 + params[1])
    genome = T.random_dna(rng, 60_000)
    g = G.gpu_filter(params, 2**18)
    o = G.oracle_filter(params, 2**18)
    g.insert_seq(G.to_dev(genome))
    o.insert_seq(genome)
    noise = np.frombuffer(b"acgtNNRYn\x00\xc1\xe1@*", dtype=np.uint8)
    for n in [31, 32, 33, 62, 63, 64, 2015, 2016, 2046, 2047, 2048, 2049, 4095, 4096 + 45, 40_000 + 3]:
        src = bytearray(genome[rng.integers(0, len(genome) - n):][:n])
        for p in rng.integers(0, n, max(1, n // 40)):
            src[p] = int(noise[rng.integers(0, noise.size)])
        if n > 100:
            p = int(rng.integers(0, n - 40))
            src[p:p + 33] = b"N" * 33
        seq = bytes(src)
        want = o.query_seq(seq)
        got = G.dev_bits_to_np(g.query_seq(G.to_dev(seq)))
        G.assert_words_equal(got, want, "aligned n=%d %s" % (n, params))
        for off in (1, 5, 15):
            buf = torch.zeros(n + 16, dtype=torch.uint8, device="cuda")
            buf[off:off + n] = torch.frombuffer(bytearray(seq), dtype=torch.uint8).cuda()
            view = buf[off:off + n]
            assert view.data_ptr() % 16 == off
            got = G.dev_bits_to_np(g.query_seq(view))
            G.assert_words_equal(got, want, "offset %d n=%d %s" % (off, n, params))
        codes, valid = M.pack(G.to_dev(seq))
        got = G.dev_bits_to_np(g.query_packed(codes, valid, n))
        G.assert_words_equal(got, want, "packed n=%d %s" % (n, params))


@pytest.mark.parametrize("params", [MAIN, (31, 12, 28, 4), (31, 20, 24, 2)])
def test_insert_inputs_agree(params):
    """A DNA insert reads its input three ways: the insert kernel decoding
    the ASCII itself (a 16-byte-aligned device sequence; 16 k-mers per lane
    load their 48 bases each, 32 per lane take lane l+1's by DPP), the
    packing pass and then the packed kernel (an unaligned device sequence),
    and sbf_insert_packed on codes from sbf_pack.  Every way gives the
    oracle's filter words, on text with lower case, 'N' runs, other letters
    and bytes with bit 7 set, at lengths around a lane and a wave (1008 and
    2016 k-mer starts) and over many waves."""
    import minimizer_sharded_bloom_amd as M
    torch = G.torch_cuda()
    rng = np.random.default_rng(78 + params[1])
    noise = np.frombuffer(b"acgtNNRYn\x00\xc1\xe1@*", dtype=np.uint8)
    for n in [31, 46, 47, 48, 62, 63, 1007 + 30, 1008 + 30, 1009 + 30, 1056, 2016 + 30, 2047, 2048, 2049,
              4096 + 45, 300_000 + 3]:
        src = bytearray(T.random_dna(rng, n))
        for p in rng.integers(0, n, max(1, n // 40)):
            src[p] = int(noise[rng.integers(0, noise.size)])
        if n > 100:
            p = int(rng.integers(0, n - 40))
            src[p:p + 33] = b"N" * 33
        seq = bytes(src)
        o = G.oracle_filter(params, 2**14)
        o.insert_seq(seq)
        want = o.words()
        o.close()
        g = G.gpu_filter(params, 2**14)
        g.insert_seq(G.to_dev(seq))
        G.assert_words_equal(g.words(), want, "aligned n=%d %s" % (n, params))
        for off in (1, 7):
            g.clear()
            buf = torch.zeros(n + 16, dtype=torch.uint8, device="cuda")
            buf[off:off + n] = torch.frombuffer(bytearray(seq), dtype=torch.uint8).cuda()
            view = buf[off:off + n]
            assert view.data_ptr() % 16 == off
            g.insert_seq(view)
            G.assert_words_equal(g.words(), want, "offset %d n=%d %s" % (off, n, params))
        g.clear()
        codes, valid = M.pack(G.to_dev(seq))
        g.insert_packed(codes, valid, n)
        G.assert_words_equal(g.words(), want, "packed n=%d %s" % (n, params))
        g.close()


def test_query_gaps_at_lane_and_wave_boundaries():
    """'N' runs of 1, 2, 31 and 40 bases placed at and around lane (32 k-mer
    starts) and wave (2016) boundaries, so runs of invalid k-mers start, end
    and continue across lanes and waves; both query widths (32 and 16 k-mers
    per lane) and an insert of the same text."""
    rng = np.random.default_rng(401)
    n = 60_000
    for params in (MAIN, (31, 16, 20, 4)):
        a = bytearray(T.random_dna(rng, n))
        for base in list(range(0, n, 2016)) + list(range(5000, 9000, 32)):
            off = int(rng.choice([-31, -30, -1, 0, 1, 30, 31]))
            L = int(rng.choice([1, 2, 31, 40]))
            p = max(0, base + off)
            a[p:p + L] = b"N" * min(L, n - p)
        seq = bytes(a)
        _run_pair(params, 2**15, [seq[: n // 2]], [seq, seq[1:], seq[31:], seq[2016 + 5:]])


SLIDE_PARAMS = [(32, 1, 32, 3), (32, 32, 1, 5), (31, 24, 27, 4), (20, 7, 11, 9), (31, 19, 22, 12), (2, 1, 2, 1),
                (31, 17, 24, 8)]


@pytest.mark.parametrize("params", SLIDE_PARAMS)
def test_sliding_kernels(params):
    """Parameter sets without a compiled set run the run-time sliding
    kernels: 65 - max(w, z) k-mers per wave step (33 at w = 32 or z = 32),
    tasks of 2048 k-mer starts.  Filter words and every answer bit equal the
    oracle's on noisy input whose lengths straddle the step and task
    boundaries, on a poly-A run across steps and tasks, all-'N' and 'N'
    every 37 bases, over several inserts into one filter."""
    k, m, s, H = params
    w, z = k - m + 1, k - s + 1
    E = 65 - max(w, z)
    rng = np.random.default_rng(61 + sum(params))
    lens = [0, 1, k - 1, k, k + 1, E + k - 1, E + k, 2048 + k - 2, 2048 + k - 1, 2048 + k, 4096 + E + k, 100_003]
    ins = [_noisy(rng, L) for L in lens[:6]] + [b"A" * 6000, _noisy(rng, 30_000)]
    every37 = bytearray(T.random_dna(rng, 9000))
    for i in range(0, len(every37), 37):
        every37[i] = ord("N")
    qs = [_noisy(rng, L) for L in lens] + [b"A" * 6000, b"N" * 500, bytes(every37)] + ins[-2:]
    g, _ = _run_pair(params, 2**16, ins, qs)
    assert not g.specialized


def test_sliding_kernels_many_tasks():
    """A 140 Mbp insert and a 20 Mbp query on a run-time parameter set: more
    tasks than the grid's waves (the grid-stride loop); full filter and every
    answer bit against the threaded oracle."""
    params = (31, 24, 27, 4)
    codes = S.genome_with_repeats(140_000_000, seed_genome=21)
    genome = S.to_ascii(codes)
    reads = S.short_read_set(codes, 130_000)  # half sampled from this genome
    del codes
    g = G.gpu_filter(params, 2**30)
    o = G.oracle_filter(params, 2**30)
    assert not g.specialized
    g.insert_seq(G.to_dev(genome))
    o.insert_seq_mt(genome)
    G.assert_words_equal(g.words(), o.words(), "sliding insert, 140 Mbp")
    got = G.dev_bits_to_np(g.query_seq(G.to_dev(reads)))
    G.assert_words_equal(got, o.query_seq_mt(reads), "sliding query, 20 Mbp")
