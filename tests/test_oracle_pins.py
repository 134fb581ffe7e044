"""Pins of the CPU oracle against facts that do not come from the oracle.

Source of the method: "cuSBF: A Minimizer-Aware Bloom Filter for Genomic
Sequence Data on Modern GPUs" (sections cited per test).  Each pin is chosen so
that a plausible slip in the oracle (dropped term, wrong shift or index, wrong
sector, a missing fold) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from tests import helpers as T

GOLD = os.path.join(os.path.dirname(__file__), "golden")
M64 = 2**64 - 1
GAMMA = 0x9E3779B97F4A7C15
C1 = 0xBF58476D1CE4E5B9


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---- hash primitives --------------------------------------------------------

def test_splitmix64_published_stream():
    """mix and the golden-ratio increment reproduce the published SplitMix64
    outputs; h_s(v) is the SplitMix64 output for state v and the probe stream
    is the SplitMix64 stream itself."""
    g = _gold("splitmix64_seed1234567.json")
    seed, outs = g["seed"], g["outputs"]
    for i, want in enumerate(outs):
        assert O.mix((seed + (i + 1) * GAMMA) & M64) == want
        assert O.hs((seed + i * GAMMA) & M64) == want
        assert O.probe_kmer(seed, i, 32) == want
        assert O.probe_kmer(seed, i, 31) == want >> 2
        assert O.probe_kmer(seed, i, 9) == want >> 46


def test_hmin_inverts():
    """h_min(v) = fold((v + G) * C1): undo it with the modular inverse of C1
    (the fold x ^ (x >> 32) is its own inverse)."""
    inv = pow(C1, -1, 2**64)
    rng = np.random.default_rng(11)
    vals = [0, 1, 2**32 - 1, 2**62, M64] + [int(x) for x in rng.integers(0, 2**63, 200, dtype=np.uint64)]
    for v in vals:
        h = O.hmin(v)
        u = h ^ (h >> 32)
        assert ((u * inv) - GAMMA) & M64 == v
    assert O.hmin(0) != 0  # the offset keeps poly-A off zero


def test_hmin_low_bits_depend_on_every_base():
    """§IV-B takes the shard from the low hash bits.  m-mers that share their
    last three bases must still spread over the low 6 bits (a chi-square
    test); without the fold they would all land on one value."""
    rng = np.random.default_rng(12)
    n = 64 * 200
    tail = 0b101101
    counts = np.zeros(64)
    for r in rng.integers(0, 2**26, n):
        counts[O.hmin((int(r) << 6) | tail) & 63] += 1
    chi2 = float(((counts - n / 64) ** 2 / (n / 64)).sum())
    assert chi2 < 120  # 63 dof, p ~ 1e-5


def test_bitaddr_slices():
    """§IV-G bit-slicing: for H <= 10 hash index t reads the low 6 bits of
    slice t of width floor(64/H); for H > 10 the salted multiply's top bits."""
    h = 0x0123456789ABCDEF
    for H in range(1, 11):
        w = 64 // H
        for t in range(H):
            assert O.bitaddr(h, t, H) == (h >> (t * w)) & 63
    # H = 4: the four 16-bit slices of 0x0123456789ABCDEF end in
    # 0xCDEF, 0x89AB, 0x4567, 0x0123 -> low 6 bits 0x2F, 0x2B, 0x27, 0x23
    assert [O.bitaddr(h, t, 4) for t in range(4)] == [0x2F, 0x2B, 0x27, 0x23]
    g = _gold("splitmix64_seed1234567.json")
    for t in range(12):
        salt = O.mix(((t + 1) * GAMMA) & M64)  # t-th SplitMix64 output of seed 0
        assert O.bitaddr(h, t, 12) == ((h * salt) & M64) >> 58
    # the salts are SplitMix64 outputs: for seed 1234567 the stream is published
    assert O.mix((g["seed"] + GAMMA) & M64) == g["outputs"][0]


# ---- encoding and packing ---------------------------------------------------

def test_code_table_exhaustive():
    """§IV-A: four DNA symbols; every other byte is invalid."""
    want = {ord(c): v for c, v in T.CODE.items()}
    for b in range(256):
        assert O.code(b) == want.get(b, -1)


def test_pack_known_answers():
    assert O.pack_kmer("ACGT") == 0x1B
    assert O.pack_kmer("A") == 0 and O.pack_kmer("T") == 3
    assert O.pack_kmer("T" * 32) == M64
    assert O.pack_kmer("acgt") == 0x1B
    assert O.pack_kmer("ACNT") is None
    rng = np.random.default_rng(13)
    for _ in range(50):
        k = int(rng.integers(1, 33))
        s = T.random_dna(rng, k).decode()
        assert O.pack_kmer(s) == T.pack_str(s)


def test_fig2b_smer_enumeration():
    """Fig. 2b: k = 9, s = 6 gives four s-mers, in order, cut from the k-mer."""
    g = _gold("cusbf_fig2.json")["fig2b"]
    x = O.pack_kmer(g["kmer"])
    k, s = len(g["kmer"]), g["s"]
    assert k - s + 1 == len(g["smers"]) == 4
    assert [O.subwindow(x, k, j, s) for j in range(4)] == [T.pack_str(t) for t in g["smers"]]


def test_fig2a_kmers_share_the_mmer():
    """Fig. 2a: the k-mers shown are consecutive 9-mers of the sequence and
    all contain the m-mer the figure marks as their shared minimizer."""
    g = _gold("cusbf_fig2.json")["fig2a"]
    seq, k, m = g["sequence"], g["k"], g["m"]
    kmers = [seq[p:p + k] for p in range(len(seq) - k + 1)]
    assert len(kmers) == 4 and kmers[1:] == g["kmers_shown"]
    mm = T.pack_str(g["shared_minimizer"])
    for km in g["kmers_shown"]:
        x = O.pack_kmer(km)
        assert mm in [O.subwindow(x, k, i, m) for i in range(k - m + 1)]


# ---- minimizer and shard ----------------------------------------------------

def test_minimizer_brute_force():
    """§II-B-1 / Algorithm 1: min over every m-mer cut from the text."""
    rng = np.random.default_rng(14)
    for _ in range(300):
        k = int(rng.integers(1, 33))
        m = int(rng.integers(1, k + 1))
        km = T.random_dna(rng, k).decode()
        assert O.minimizer_hash(O.pack_kmer(km), k, m) == T.minimizer_hash_str(km, m)


def test_minimizer_density():
    """§II-B-1: random minimizers on random text have density about 2/(w+1);
    for k = 31, m = 16 the mean super-k-mer is (w+1)/2 = 8.5 k-mers.  Over
    10^7 uniform bases the oracle's density must lie within 2 % of 2/(w+1)
    (its standard error there is about 0.1 %, so a hash whose minimizers are
    biased by a few percent fails); a brute-force recount on the first 2000
    k-mers checks that the batch call is the per-k-mer minimizer."""
    rng = np.random.default_rng(15)
    k, m = 31, 16
    w = k - m + 1
    seq = T.random_dna(rng, 10_000_000)
    mh = O.minimizer_hashes(seq, k, m)
    assert mh.size == len(seq) - k + 1
    for p in range(0, 2000):
        assert int(mh[p]) == T.minimizer_hash_str(seq[p:p + k].decode(), m)
    changes = int((mh[1:] != mh[:-1]).sum())
    density = changes / (mh.size - 1)
    assert abs(density - 2 / (w + 1)) < 0.02 * 2 / (w + 1)
    assert abs(1 / density - (w + 1) / 2) < 0.02 * (w + 1) / 2
    # other window lengths on a shorter piece (2 * 10^6 bases, +-2 %)
    for kk, mm in ((31, 12), (31, 20), (21, 11)):
        ww = kk - mm + 1
        d = float((np.diff(O.minimizer_hashes(seq[:2_000_000], kk, mm)) != 0).mean())
        assert abs(d - 2 / (ww + 1)) < 0.02 * 2 / (ww + 1), (kk, mm, d)


def test_shard_uniformity():
    f = O.OracleFilter(31, 16, 28, 4, 64 * 256)
    assert f.num_shards == 64
    rng = np.random.default_rng(16)
    counts = np.zeros(64)
    n = 64 * 150
    for x in rng.integers(0, 2**62, n, dtype=np.uint64):
        counts[f.shard_of(int(x))] += 1
    chi2 = float(((counts - n / 64) ** 2 / (n / 64)).sum())
    assert chi2 < 120


def test_shard_count_rounding():
    """§IV-B: shard count rounded up to a power of two, 256-bit shards."""
    for bits, n in [(1, 1), (256, 1), (257, 2), (2**20, 4096), (2**20 + 1, 8192), (3 * 256, 4)]:
        f = O.OracleFilter(31, 16, 28, 4, bits)
        assert f.num_shards == n == T.num_shards(bits)


# ---- single k-mer bit layout ------------------------------------------------

@pytest.mark.parametrize("k,m,s,H", [(31, 16, 28, 4), (9, 5, 6, 3), (31, 12, 24, 6), (20, 20, 20, 2), (16, 4, 10, 1), (31, 16, 28, 12)])
def test_single_kmer_bits(k, m, s, H):
    """§IV-B / Algorithm 1: one k-mer touches one shard; hash index t sets a
    bit in word t mod 4; the set bits are exactly those of its s-mers."""
    rng = np.random.default_rng(17 + k + m + s + H)
    for _ in range(20):
        f = O.OracleFilter(k, m, s, H, 2**14)
        km = T.random_dna(rng, k).decode()
        x = O.pack_kmer(km)
        f.insert_kmer(x)
        w = f.words().reshape(-1, 4)
        nz = np.nonzero(w.any(axis=1))[0]
        assert list(nz) == [f.shard_of(x)]
        assert f.shard_of(x) == T.minimizer_hash_str(km, m) % f.num_shards
        got = {(q, b) for q in range(4) for b in range(64) if (int(w[nz[0], q]) >> b) & 1}
        assert got == T.kmer_bits_str(km, s, H)
        assert 1 <= len(got) <= (k - s + 1) * H
        for q in range(H, 4):
            assert w[nz[0], q] == 0
        assert f.query_kmer(x)


def test_bbf_single_key():
    """Blocked Bloom comparator (§II-A, Fig. 1b): one hash of the key picks the
    block, H bits from a second hash of it."""
    f = O.OracleFilter(31, 0, 0, 4, 2**14, kind=O.KIND_BBF)
    x = O.pack_kmer("ACGTACGTACGTACGTACGTACGTACGTACG")
    f.insert_kmer(x)
    w = f.words().reshape(-1, 4)
    blk = O.hs(x) % f.num_shards
    assert list(np.nonzero(w.any(axis=1))[0]) == [blk]
    hb = O.hs(O.hs(x))
    want = np.zeros(4, dtype=np.uint64)
    for t in range(4):
        want[t % 4] |= np.uint64(1 << O.bitaddr(hb, t, 4))
    assert (w[blk] == want).all()


# ---- sequences ---------------------------------------------------------------

def test_no_false_negatives_and_invalid():
    """§II-A: a Bloom filter has no false negatives; §IV-F: a k-mer holding a
    separator is invalid and queries false."""
    rng = np.random.default_rng(18)
    k = 31
    seq = bytearray(T.random_dna(rng, 3000))
    for p in rng.integers(0, len(seq), 12):
        seq[p] = ord("N")
    seq = bytes(seq)
    f = O.OracleFilter(k, 16, 28, 4, 2**16)
    f.insert_seq(seq)
    nk = len(seq) - k + 1
    got = T.bits_of(f.query_seq(seq), nk)
    want = np.array([T.valid_str(seq[p:p + k].decode()) for p in range(nk)], dtype=np.uint8)
    assert (got == want).all()
    tail = f.query_seq(seq)
    assert tail[-1] >> np.uint64(nk % 64) == 0 if nk % 64 else True


def test_query_seq_matches_per_kmer():
    rng = np.random.default_rng(19)
    k = 21
    f = O.OracleFilter(k, 11, 19, 3, 2**12)
    f.insert_seq(T.random_dna(rng, 4000))
    q = T.random_dna(rng, 2000, alphabet=b"ACGTN" + b"ACGT" * 10)
    got = T.bits_of(f.query_seq(q), len(q) - k + 1)
    for p in range(len(q) - k + 1):
        km = q[p:p + k].decode()
        want = T.valid_str(km) and f.query_kmer(T.pack_str(km))
        assert got[p] == want
    pos = rng.integers(0, len(q), 300)
    qp = f.query_positions(q, pos)
    for i, p in enumerate(pos):
        assert qp[i] == (got[p] if p + k <= len(q) else 0)


def test_insert_is_a_union():
    """Insert is a set union: order-free, idempotent, and records joined by a
    separator insert exactly the k-mers of each record (§IV-F)."""
    rng = np.random.default_rng(20)
    a, b = T.random_dna(rng, 700), T.random_dna(rng, 500)
    args = (31, 16, 28, 4, 2**13)
    f1, f2, f3, f4 = (O.OracleFilter(*args) for _ in range(4))
    f1.insert_seq(a); f1.insert_seq(b)
    f2.insert_seq(b); f2.insert_seq(a)
    f3.insert_seq(a + b"N" + b)
    f4.insert_seq(a + b"N" + b); f4.insert_seq(a + b"N" + b)
    w = f1.words()
    for g in (f2, f3, f4):
        assert (g.words() == w).all()
    assert w.any()


def test_short_and_empty_sequences():
    f = O.OracleFilter(31, 16, 28, 4, 2**12)
    for L in (0, 1, 30):
        f.insert_seq(b"A" * L)
        assert f.query_seq(b"A" * L).size == 0
    assert not f.words().any()
    f.insert_seq(b"A" * 31)
    assert f.words().any()
    assert T.bits_of(f.query_seq(b"A" * 31), 1)[0] == 1


# ---- false-positive rate -----------------------------------------------------

def test_single_word_bloom_eq1():
    """Textbook reduction of Eq. (1): one 256-bit shard (bits = 256), s = m = k
    and H = 1 make word 0 a 64-bit Bloom filter with one hash.  After n
    distinct keys the chance that a random key hits is 1 - (1 - 1/64)^n,
    whose large-m form is Eq. (1)."""
    rng = np.random.default_rng(21)
    k, n, trials, probes = 31, 40, 60, 2000
    hits = 0
    for tr in range(trials):
        f = O.OracleFilter(k, k, k, 1, 256)
        for x in rng.choice(2**62, n, replace=False):
            f.insert_kmer(int(x))
        hits += f.fpr_probe(probes, 1000 + tr)
    p = 1 - (1 - 1 / 64) ** n
    assert T.binom_ok(hits, trials * probes, p, z=4.5)
    assert abs(p - (1 - math.exp(-n / 64))) < 0.01  # Eq. (1) with H = 1


def test_sector_independence():
    """With H = 4 and one shard, the four hash indices fill four separate
    words from separate hash slices: a random key hits with probability
    prod_q fill_q (fill measured on the filter itself)."""
    rng = np.random.default_rng(22)
    hits, expect, total = 0, 0.0, 0
    for tr in range(40):
        f = O.OracleFilter(31, 31, 31, 4, 256)
        for x in rng.choice(2**62, 30, replace=False):
            f.insert_kmer(int(x))
        w = f.words()
        p = float(np.prod([bin(int(v)).count("1") / 64 for v in w]))
        n = 3000
        hits += f.fpr_probe(n, 5000 + tr)
        expect += n * p
        total += n
    assert abs(hits - expect) <= 4.5 * math.sqrt(expect) + 2


@pytest.mark.parametrize("k,m,s,H", [(31, 16, 28, 4), (31, 16, 24, 2), (21, 11, 19, 3)])
def test_fpr_fill_based(k, m, s, H):
    """Eq. (2) refined by the actual shard loads: a random alien k-mer lands in
    a uniform shard and each of its k-s+1 s-mers must hit H bits, so
    P(hit) = mean over shards of prod_q (fill_q)^(c_q (k-s+1)), c_q the number
    of hash indices in word q."""
    rng = np.random.default_rng(23 + s)
    f = O.OracleFilter(k, m, s, H, 2**14)
    f.insert_seq(T.random_dna(rng, 6000))
    w = f.words().reshape(-1, 4)
    fill = np.array([[bin(int(v)).count("1") / 64 for v in row] for row in w])
    c = [sum(1 for t in range(H) if t % 4 == q) for q in range(4)]
    z1 = k - s + 1
    p = float(np.mean(np.prod([fill[:, q] ** (c[q] * z1) for q in range(4)], axis=0)))
    n = 200000
    hits = f.fpr_probe(n, 0x5EED)
    assert p > 1e-4
    assert T.binom_ok(hits, n, p, z=4.5)


def test_findere_suppresses_aliens():
    """§II-B-2: k-mers one substitution away from inserted ones share k-s of
    their s-mers and hit far more often than random aliens."""
    rng = np.random.default_rng(24)
    k = 31
    f = O.OracleFilter(k, 16, 28, 4, 2**16)
    seq = T.random_dna(rng, 3000)
    f.insert_seq(seq)
    near = 0
    trials = 1500
    for _ in range(trials):
        p = int(rng.integers(0, len(seq) - k))
        km = bytearray(seq[p:p + k])
        j = int(rng.integers(0, k))
        km[j] = ord("ACGT"[(T.CODE[chr(km[j])] + int(rng.integers(1, 4))) % 4])
        near += f.query_kmer(T.pack_str(km.decode()))
    alien = f.fpr_probe(trials * 20, 77)
    assert near / trials > 5 * (alien / (trials * 20) + 1e-4)


def test_salted_bit_addresses_independent():
    """§IV-G salted fallback (H > 10): with H = 12, one shard and s = m = k,
    word q receives the three hash indices t = q, q+4, q+8; if their salted
    addresses are independent a random key hits with prod_q fill_q^3."""
    rng = np.random.default_rng(25)
    hits, expect = 0, 0.0
    for tr in range(40):
        f = O.OracleFilter(31, 31, 31, 12, 256)
        for x in rng.choice(2**62, 30, replace=False):
            f.insert_kmer(int(x))
        fill = [bin(int(v)).count("1") / 64 for v in f.words()]
        n = 4000
        hits += f.fpr_probe(n, 9000 + tr)
        expect += n * float(np.prod([q ** 3 for q in fill]))
    assert expect > 200
    assert abs(hits - expect) <= 4.5 * math.sqrt(expect) + 2


def test_bbf_fill_based_fpr():
    """Blocked Bloom comparator (§II-A): a random key picks a uniform block and
    hits with prod_q fill_q^(c_q), c_q the hash indices in word q."""
    rng = np.random.default_rng(26)
    H = 6
    f = O.OracleFilter(31, 0, 0, H, 2**12, kind=O.KIND_BBF)
    for x in rng.choice(2**62, 700, replace=False):
        f.insert_kmer(int(x))
    w = f.words().reshape(-1, 4)
    fill = np.array([[bin(int(v)).count("1") / 64 for v in row] for row in w])
    c = [sum(1 for t in range(H) if t % 4 == q) for q in range(4)]
    p = float(np.mean(np.prod([fill[:, q] ** c[q] for q in range(4)], axis=0)))
    n = 200000
    hits = f.fpr_probe(n, 4242)
    assert p > 1e-3
    assert T.binom_ok(hits, n, p, z=4.5)


@pytest.mark.parametrize("kind,params", [(O.KIND_SBF, (31, 16, 28, 4)), (O.KIND_SBF, (21, 11, 19, 3)),
                                         (O.KIND_BBF, (31, 0, 0, 4)), (O.KIND_WIDE, (31, 16, 28, 4))])
def test_threaded_driver_equals_single_thread(kind, params):
    """The multi-threaded insert/query drivers split k-mer starts over
    threads; the union and the answers must equal the plain loop's."""
    rng = np.random.default_rng(27)
    k, m, s, H = params
    seq = bytearray(T.random_dna(rng, 50000))
    for p in rng.integers(0, len(seq), 40):
        seq[p] = ord("N")
    seq = bytes(seq)
    a = O.OracleFilter(k, m, s, H, 2**15, kind=kind)
    b = O.OracleFilter(k, m, s, H, 2**15, kind=kind)
    a.insert_seq(seq)
    b.insert_seq_mt(seq, 7)
    assert (a.words() == b.words()).all()
    q = T.random_dna(rng, 30001)
    assert (a.query_seq(q) == b.query_seq_mt(q, 5)).all()
    assert (a.query_seq(seq) == a.query_seq_mt(seq, 3)).all()


def test_shard_sampled_driver():
    """The shard-sampled insert reproduces the full insert on the sampled
    shards and nothing else; the sampled query marks exactly the valid k-mers
    of sampled shards and answers them as the full query does."""
    rng = np.random.default_rng(28)
    seq = bytearray(T.random_dna(rng, 40000))
    for p in rng.integers(0, len(seq), 30):
        seq[p] = ord("N")
    seq = bytes(seq)
    full = O.OracleFilter(31, 16, 28, 4, 2**14)
    full.insert_seq(seq)
    samp = O.OracleFilter(31, 16, 28, 4, 2**14)
    samp.insert_seq_sampled_mt(seq, 7, 3, 4)
    wf, ws = full.words().reshape(-1, 4), samp.words().reshape(-1, 4)
    sel = (np.arange(wf.shape[0]) & 7) == 3
    assert (ws[sel] == wf[sel]).all() and not ws[~sel].any() and wf[sel].any()
    q = T.random_dna(rng, 20000) + seq[:10000]
    ans, checked = full.query_seq_sampled_mt(q, 7, 3, 3)
    nk = len(q) - 31 + 1
    cb = T.bits_of(checked, nk)
    want = T.bits_of(full.query_seq(q), nk)
    assert (T.bits_of(ans, nk) == (want & cb)).all()
    for p in range(0, nk, 97):
        km = q[p:p + 31].decode()
        exp = T.valid_str(km) and (full.shard_of(T.pack_str(km)) & 7) == 3
        assert cb[p] == exp


# ---- wide variant: 512-bit blocks, whole-block addressing ([cuSBF] §V-D) ----

def test_wide_bitaddr_slices_and_salt():
    """Hand-sliced 9-bit addresses for H = 4 (slices of 16 bits, low 9 bits)
    and the salted form for H > 7 (top 9 bits of hs * mix((t+1) G))."""
    h = 0x0123456789ABCDEF
    assert [O.bitaddr_wide(h, t, 4) for t in range(4)] == [0x1EF, 0x1AB, 0x167, 0x123]
    assert [O.bitaddr_wide(h, t, 7) for t in range(7)] == [(h >> (9 * t)) & 511 for t in range(7)]
    G = 0x9E3779B97F4A7C15
    for H in (8, 12):
        for t in range(H):
            salt = O.mix(((t + 1) * G) & (2**64 - 1))
            assert O.bitaddr_wide(h, t, H) == ((h * salt) & (2**64 - 1)) >> 55


@pytest.mark.parametrize("k,m,s,H", [(31, 16, 28, 4), (21, 8, 15, 3), (31, 16, 28, 8)])
def test_wide_single_kmer_bits(k, m, s, H):
    """One k-mer touches one 512-bit block; the set bits are exactly the
    addresses of its s-mers cut from the text, anywhere in the block."""
    rng = np.random.default_rng(31 + k + m + s + H)
    for _ in range(20):
        f = O.OracleFilter(k, m, s, H, 2**15, kind=O.KIND_WIDE)
        assert f.words_per_shard == 8 and f.num_shards == 2**15 // 512
        km = T.random_dna(rng, k).decode()
        x = O.pack_kmer(km)
        f.insert_kmer(x)
        w = f.words().reshape(-1, 8)
        nz = np.nonzero(w.any(axis=1))[0]
        assert list(nz) == [f.shard_of(x)]
        assert f.shard_of(x) == T.minimizer_hash_str(km, m) % f.num_shards
        got = {(q, b) for q in range(8) for b in range(64) if (int(w[nz[0], q]) >> b) & 1}
        assert got == T.kmer_bits_wide_str(km, s, H)
        assert f.query_kmer(x)


def test_wide_classic_bloom_eq1():
    """Textbook reduction: one 512-bit block (bits = 512) and s = m = k make a
    classic Bloom filter of 512 bits with H = 4 hash functions.  Given the
    filter, a random key hits with probability fill^H (independent uniform
    addresses); the mean fill after n keys is 1 - (1 - 1/512)^(Hn), whose
    large-m form gives Eq. (1)."""
    rng = np.random.default_rng(32)
    k, H, n, trials, probes = 31, 4, 60, 50, 4000
    hits, expect, fills = 0, 0.0, []
    for tr in range(trials):
        f = O.OracleFilter(k, k, k, H, 512, kind=O.KIND_WIDE)
        for x in rng.choice(2**62, n, replace=False):
            f.insert_kmer(int(x))
        fill = sum(bin(int(v)).count("1") for v in f.words()) / 512
        fills.append(fill)
        hits += f.fpr_probe(probes, 7000 + tr)
        expect += probes * fill ** H
    assert abs(hits - expect) <= 4.5 * math.sqrt(expect) + 2
    mean_fill = 1 - (1 - 1 / 512) ** (H * n)
    assert abs(np.mean(fills) - mean_fill) < 4.5 * np.std(fills) / math.sqrt(trials) + 1e-3
    eq1 = (1 - math.exp(-H * n / 512)) ** H
    assert abs(mean_fill ** H - eq1) / eq1 < 0.05


@pytest.mark.parametrize("H,n_keys", [(8, 60), (12, 45)])
def test_wide_salted_addresses_independent(H, n_keys):
    """Salted addresses of the wide layout (H > 7: the top 9 bits of
    h_s * mix((t+1) G), the golden-ratio-derived salt of §IV-G over a 512-bit
    block).  With one block and s = m = k the filter is a classic 512-bit Bloom
    filter with H hash functions; if the H addresses of a key are independent
    and uniform over the block, a random key hits with probability fill^H,
    fill measured on the block itself.  Correlated salts (an arithmetic
    progression of addresses), a wrong shift (addresses confined to a few
    words) or a wrong word index fail this."""
    rng = np.random.default_rng(36 + H)
    k, trials, probes = 31, 40, 4000
    hits, expect = 0, 0.0
    for tr in range(trials):
        f = O.OracleFilter(k, k, k, H, 512, kind=O.KIND_WIDE)
        assert f.num_shards == 1 and f.words_per_shard == 8
        for x in rng.choice(2**62, n_keys, replace=False):
            f.insert_kmer(int(x))
        fill = sum(bin(int(v)).count("1") for v in f.words()) / 512
        hits += f.fpr_probe(probes, 11000 + 100 * H + tr)
        expect += probes * fill ** H
    assert expect > 500
    assert abs(hits - expect) <= 4.5 * math.sqrt(expect) + 2
    # every word of the block receives addresses (the 9-bit range is used)
    f = O.OracleFilter(k, k, k, H, 512, kind=O.KIND_WIDE)
    for x in rng.choice(2**62, 40, replace=False):
        f.insert_kmer(int(x))
    assert all(int(v) != 0 for v in f.words())


@pytest.mark.parametrize("k,m,s,H", [(31, 16, 28, 4), (31, 16, 24, 2)])
def test_wide_fpr_fill_based(k, m, s, H):
    """A random alien k-mer lands in a uniform block and each of its
    (k-s+1) H addresses is uniform over the block's 512 bits:
    P(hit) = mean over blocks of fill^((k-s+1) H)."""
    rng = np.random.default_rng(33 + s)
    f = O.OracleFilter(k, m, s, H, 2**14, kind=O.KIND_WIDE)
    f.insert_seq(T.random_dna(rng, 6000))
    w = f.words().reshape(-1, 8)
    fill = np.array([sum(bin(int(v)).count("1") for v in row) / 512 for row in w])
    p = float(np.mean(fill ** ((k - s + 1) * H)))
    n = 200000
    hits = f.fpr_probe(n, 0x5EED)
    assert p > 1e-4
    assert T.binom_ok(hits, n, p, z=4.5)


def test_wide_blocks_lower_fpr_than_sectors():
    """At one memory budget and input, whole-block addressing in 512-bit
    blocks gives a lower false-positive rate than 64-bit sectors in 256-bit
    shards ([cuSBF] §V-D: the CPU reference's layout; cuSBF trades dispersion
    for branch-free masks)."""
    rng = np.random.default_rng(34)
    seq = T.random_dna(rng, 60000)
    rates = {}
    for kind in (O.KIND_SBF, O.KIND_WIDE):
        f = O.OracleFilter(31, 16, 28, 4, 2**19, kind=kind)
        f.insert_seq(seq)
        rates[kind] = f.fpr_probe(400000, 77) / 400000
    assert rates[O.KIND_SBF] > 5e-4  # ~640 hits: the comparison is not noise
    assert rates[O.KIND_WIDE] < 0.5 * rates[O.KIND_SBF]


# ---- other alphabets (§IV-A, §IV-C) -------------------------------------------

def test_protein_code_table_exhaustive():
    """§IV-A: 26 protein symbols of 5 bits; letters of either case map to
    their place in the alphabet, every other byte is invalid."""
    for c in range(256):
        ch = chr(c)
        want = ord(ch.upper()) - 65 if ch.isascii() and ch.isalpha() else -1
        assert O.code_protein(c) == want, c
    assert O.symbol_bits(O.ALPHA_PROTEIN) == 5 and max(O.code_protein(c) for c in range(256)) == 25


def test_triplet_code_table_exhaustive():
    """§IV-A: 64 triplet symbols of 6 bits spanning three bytes.  Every codon
    over ACGTN (both cases) against 16 c0 + 4 c1 + c2; the valid ones form a
    bijection onto 0..63."""
    bases = "ACGTNacgtn"
    seen = set()
    for a in bases:
        for b in bases:
            for c in bases:
                cod = a + b + c
                got = O.code_triplet(cod)
                if "N" in cod.upper():
                    assert got == -1, cod
                else:
                    want = 16 * T.CODE[a] + 4 * T.CODE[b] + T.CODE[c]
                    assert got == want, cod
                    seen.add(got)
    assert seen == set(range(64)) and O.symbol_bits(O.ALPHA_TRIPLET) == 6


def test_alphabet_pack_known_answers():
    """§IV-C: shift-and-OR packing at the symbol width.  Hand-computed values:
    protein ACD = 0b00000_00010_00011 = 0x43; triplets AAA|CCC = 0*64 + 21.
    A triplet k-mer packs to the same integer as the 3k bases it spans packed
    as DNA (six bits = three 2-bit codes), at every codon start."""
    assert O.pack_kmer_alpha(O.ALPHA_PROTEIN, b"ACD", 0, 3) == 0x43
    assert O.pack_kmer_alpha(O.ALPHA_PROTEIN, b"acd", 0, 3) == 0x43
    assert O.pack_kmer_alpha(O.ALPHA_PROTEIN, b"ZZZZZZZZZZZZ", 0, 12) == int("11001" * 12, 2)
    assert O.pack_kmer_alpha(O.ALPHA_TRIPLET, b"AAACCC", 0, 2) == 21
    assert O.pack_kmer_alpha(O.ALPHA_TRIPLET, b"TTTTTTTTTTTTTTTTTTTTTTTTTTTTTT", 0, 10) == 2**60 - 1
    assert O.pack_kmer_alpha(O.ALPHA_PROTEIN, b"AC*D", 0, 4) is None
    assert O.pack_kmer_alpha(O.ALPHA_TRIPLET, b"AAACNC", 0, 2) is None
    rng = np.random.default_rng(40)
    seq = T.random_dna(rng, 300)
    for k in (1, 4, 10):
        for p in range(0, 100 - k):
            x = O.pack_kmer_alpha(O.ALPHA_TRIPLET, seq, p, k)
            assert x == O.pack_kmer(seq[3 * p:3 * p + 3 * k]), (k, p)
            assert x == O.pack_kmer_alpha(O.ALPHA_DNA, seq, 3 * p, 3 * k)


@pytest.mark.parametrize("alpha,k,m,s,H", [(O.ALPHA_PROTEIN, 12, 6, 10, 4), (O.ALPHA_PROTEIN, 9, 4, 7, 3),
                                           (O.ALPHA_PROTEIN, 5, 5, 5, 12), (O.ALPHA_TRIPLET, 10, 5, 8, 4),
                                           (O.ALPHA_TRIPLET, 7, 3, 7, 2)])
def test_alphabet_single_kmer_bits(alpha, k, m, s, H):
    """§II-B / §IV-B for other alphabets: the shard is the minimizer over the
    k-m+1 m-mers of symbols and the set bits are those of the k-s+1 s-mers,
    each cut out of the symbol list and packed on its own."""
    rng = np.random.default_rng(41 + alpha * 7 + k)
    b = T.BITS[alpha]
    for _ in range(20):
        f = O.OracleFilter(k, m, s, H, 2**14, alpha=alpha)
        text = T.random_protein(rng, k) if alpha == O.ALPHA_PROTEIN else T.random_dna(rng, 3 * k)
        codes = T.symbols_of(alpha, text)
        x = T.pack_symbols(codes, b)
        assert O.pack_kmer_alpha(alpha, text, 0, k) == x
        f.insert_seq(text)
        w = f.words().reshape(-1, 4)
        nz = np.nonzero(w.any(axis=1))[0]
        assert list(nz) == [T.minimizer_hash_alpha(codes, alpha, m) % f.num_shards]
        got = {(q, bit) for q in range(4) for bit in range(64) if (int(w[nz[0], q]) >> bit) & 1}
        assert got == T.kmer_bits_alpha(codes, alpha, s, H)
        assert f.query_kmer(x)


@pytest.mark.parametrize("alpha", [O.ALPHA_PROTEIN, O.ALPHA_TRIPLET])
def test_alphabet_query_seq_matches_per_kmer(alpha):
    """§II-A no false negatives, §IV-F invalid symbols: query_seq equals the
    per-k-mer answer from the text at every symbol start; a k-mer holding an
    invalid symbol answers 0; for triplets, trailing bytes short of a codon
    are ignored."""
    rng = np.random.default_rng(42 + alpha)
    k, m, s, H = (10, 5, 8, 4) if alpha == O.ALPHA_PROTEIN else (8, 4, 6, 3)
    f = O.OracleFilter(k, m, s, H, 2**12, alpha=alpha)
    if alpha == O.ALPHA_PROTEIN:
        ins = bytearray(T.random_protein(rng, 3000, b"ACDEFGHIKLMNPQRSTVWYacdefxbz"))
        bad = b"*-1 "
    else:
        ins = bytearray(T.random_dna(rng, 3 * 1000 + 2))
        bad = b"N"
    for p in rng.integers(0, len(ins), 10):
        ins[p] = bad[int(rng.integers(0, len(bad)))]
    ins = bytes(ins)
    f.insert_seq(ins)
    codes = T.symbols_of(alpha, ins)
    nk = len(codes) - k + 1
    got = T.bits_of(f.query_seq(ins), nk)
    want = np.array([all(c is not None for c in codes[p:p + k]) for p in range(nk)], dtype=np.uint8)
    assert (got == want).all()
    # a second, uninserted sequence: per-k-mer answers from the text
    q = bytes(T.random_protein(rng, 800) if alpha == O.ALPHA_PROTEIN else T.random_dna(rng, 3 * 300 + 1))
    qc = T.symbols_of(alpha, q)
    nq = len(qc) - k + 1
    got = T.bits_of(f.query_seq(q), nq)
    for p in range(nq):
        want = f.query_kmer(T.pack_symbols(qc[p:p + k], T.BITS[alpha]))
        assert got[p] == want
    pos = rng.integers(0, len(qc), 200)
    qp = f.query_positions(q, pos)
    for i, p in enumerate(pos):
        assert qp[i] == (got[p] if p + k <= len(qc) else 0)


@pytest.mark.parametrize("alpha", [O.ALPHA_PROTEIN, O.ALPHA_TRIPLET])
def test_alphabet_insert_union_and_edges(alpha):
    """Insert is a set union (order-free, idempotent) for any alphabet;
    sequences shorter than k symbols insert nothing; k = 12 proteins and
    k = 10 triplets (60 bits) are the largest k, one more is refused."""
    rng = np.random.default_rng(43 + alpha)
    gen = (lambda n: T.random_protein(rng, n)) if alpha == O.ALPHA_PROTEIN else (lambda n: T.random_dna(rng, 3 * n))
    a, b = gen(400), gen(300)
    kmax = 12 if alpha == O.ALPHA_PROTEIN else 10
    args = (kmax, kmax // 2, kmax - 2, 4, 2**13)
    f1, f2, f3 = (O.OracleFilter(*args, alpha=alpha) for _ in range(3))
    f1.insert_seq(a); f1.insert_seq(b)
    f2.insert_seq(b); f2.insert_seq(a); f2.insert_seq(a)
    f3.insert_seq(gen(kmax - 1))
    f3.insert_seq(b"")
    assert (f1.words() == f2.words()).all() and f1.words().any()
    assert not f3.words().any()
    with pytest.raises(ValueError):
        O.OracleFilter(kmax + 1, 4, 4, 4, 2**13, alpha=alpha)
    with pytest.raises(ValueError):
        O.OracleFilter(5, 4, 4, 4, 2**13, alpha=3)


def test_alphabet_probe_symbols_uniform():
    """§V-D random probes for other alphabets: protein probe symbols are
    uniform over the 26 letters at every position, triplet probe symbols
    uniform over the 64 codons (chi-square, 5 sigma)."""
    for alpha, k, q in [(O.ALPHA_PROTEIN, 12, 26), (O.ALPHA_TRIPLET, 10, 64)]:
        b = T.BITS[alpha]
        n = 20000
        counts = np.zeros((k, q), dtype=np.int64)
        for i in range(n):
            x = O.probe_kmer_alpha(alpha, 1234, i, k)
            assert x < 1 << (b * k)
            for j in range(k):
                counts[j, (x >> (b * (k - 1 - j))) & ((1 << b) - 1)] += 1
        assert counts.sum(axis=1).tolist() == [n] * k
        e = n / q
        chi = ((counts - e) ** 2 / e).sum(axis=1)
        dof = q - 1
        assert (chi < dof + 5 * math.sqrt(2 * dof)).all(), chi
    # DNA's alphabet-generic probe is the DNA probe
    assert all(O.probe_kmer_alpha(O.ALPHA_DNA, 9, i, 31) == O.probe_kmer(9, i, 31) for i in range(100))


@pytest.mark.parametrize("alpha,k,m,s,H", [(O.ALPHA_PROTEIN, 12, 6, 10, 4), (O.ALPHA_TRIPLET, 10, 5, 8, 4)])
def test_alphabet_fpr_fill_based(alpha, k, m, s, H):
    """Eq. (2) with the shard loads, as for DNA: a random alien k-mer of the
    alphabet lands in a uniform shard and each of its k-s+1 s-mers must hit."""
    rng = np.random.default_rng(44 + alpha)
    f = O.OracleFilter(k, m, s, H, 2**14, alpha=alpha)
    f.insert_seq(T.random_protein(rng, 5000) if alpha == O.ALPHA_PROTEIN else T.random_dna(rng, 3 * 5000))
    w = f.words().reshape(-1, 4)
    fill = np.array([[bin(int(v)).count("1") / 64 for v in row] for row in w])
    c = [sum(1 for t in range(H) if t % 4 == q) for q in range(4)]
    z1 = k - s + 1
    p = float(np.mean(np.prod([fill[:, q] ** (c[q] * z1) for q in range(4)], axis=0)))
    n = 200000
    hits = f.fpr_probe(n, 0xA1FA)
    assert p > 1e-4
    assert T.binom_ok(hits, n, p, z=4.5)
