"""GPU parity of the per-read query (sbf_query_reads): each read's answer
words must equal the oracle's query of that read as a sequence of its own,
bit for bit ("cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data
on Modern GPUs", §IV-E Algorithm 2), for the per-read kernel (parameter sets
with a compiled 32-k-mer query) and for the path that queries the batch as
one sequence (every other DNA filter), over read lengths around the 32-k-mer
chunks, reads longer than a wave, strides with and without separators,
unaligned batches and batches that end at the buffer's end."""
import numpy as np
import pytest

from minimizer_sharded_bloom_amd import _lib
from tests import gpu_common as G
from tests import helpers as T

pytestmark = pytest.mark.gpu

# (params, kind): the first five have a compiled 32-k-mer query (per-read
# kernel; m = 8 and 12 reach furthest past a lane's own bases, k = 32 spans
# 63 of its 64 bases), the rest go through the one-sequence path
FAST = [((31, 16, 28, 4), "sbf"), ((31, 20, 24, 2), "sbf"), ((31, 12, 28, 4), "sbf"), ((31, 8, 28, 4), "sbf"),
        ((32, 16, 28, 4), "sbf")]
SLOW = [((31, 24, 27, 4), "sbf"), ((31, 0, 0, 4), "bbf"), ((31, 16, 28, 4), "wide")]


def _noisy_reads(rng, n, L, stride, fill=b"N", rate=0.003):
    """n reads of L bases at `stride` (bytes between reads from `fill`), with
    a few non-ACGT and lower-case letters in the reads."""
    if n == 0:
        return np.zeros(0, dtype=np.uint8)
    size = (n - 1) * stride + L
    fillv = np.frombuffer(fill, dtype=np.uint8)
    buf = fillv[rng.integers(0, fillv.size, size)]
    acgt = np.frombuffer(b"ACGT", dtype=np.uint8)
    odd = np.frombuffer(b"NacgtRn", dtype=np.uint8)
    for r in range(n):
        read = acgt[rng.integers(0, 4, L)]
        hit = rng.random(L) < rate
        read[hit] = odd[rng.integers(0, odd.size, int(hit.sum()))]
        buf[r * stride:r * stride + L] = read
    return buf


def _oracle_reads(o, buf, n, L, stride, k):
    """(n, R) uint32 words: read r's k-mer 32j+i at bit i of word j."""
    nkr = L - k + 1
    R = (nkr + 31) // 32 if nkr > 0 else 0
    out = np.zeros((n, R), dtype=np.uint32)
    for r in range(n):
        bits = T.bits_of(o.query_seq(buf[r * stride:r * stride + L].tobytes()), nkr)
        padded = np.zeros(32 * R, dtype=np.uint8)
        padded[:nkr] = bits
        out[r] = np.packbits(padded, bitorder="little").view("<u4")
    return out


def _filters(params, kind, rng, reads_buf):
    """GPU and oracle filters of a small size (false positives occur) holding
    a random genome and every fourth kilobyte of the reads."""
    bits = 2**15
    g = G.gpu_filter(params, bits, kind)
    o = G.oracle_filter(params, bits, kind)
    genome = T.random_dna(rng, 30000)
    part = reads_buf[: (reads_buf.size // 4096) * 4096].reshape(-1, 4096)[::4].reshape(-1).tobytes()
    for seq in (genome, part):
        o.insert_seq(seq)
        g.insert_seq(G.to_dev(seq))
    return g, o


def _check(g, o, params, buf, n, L, stride, offset=0, what=""):
    torch = G.torch_cuda()
    k = params[0]
    dev = G.to_dev(np.concatenate([np.full(offset, ord("A"), dtype=np.uint8), buf]))[offset:]
    got = g.query_reads(dev, n, L, stride)
    torch.cuda.synchronize()
    want = _oracle_reads(o, buf, n, L, stride, k)
    got = got.cpu().numpy().view(np.uint32).reshape(want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        r, j = (int(x) for x in bad[0])
        raise AssertionError("%s: %d of %d words differ; first read %d word %d: got %#010x want %#010x"
                             % (what, bad.shape[0], want.size, r, j, int(got[r, j]), int(want[r, j])))
    return want


@pytest.mark.parametrize("params,kind", FAST + SLOW)
def test_reads_match_oracle(params, kind):
    rng = np.random.default_rng(71 + sum(params) + len(kind))
    cases = [  # (n, L, stride, fill)
        (700, 150, 151, b"N"),
        (300, 150, 150, b"N"),         # back to back: k-mers across reads are not the reads'
        (130, 63, 76, b"ACGT"),        # bases between reads, never part of an answer
        (257, 62, 62, b"N"),           # 32 k-mers per read: one full chunk
        (64, 31, 40, b"N"),            # one k-mer per read
        (40, 1000, 1001, b"N"),
        (3, 2200, 2213, b"N"),         # 68 chunks per read: a read spans two waves
        (1, 95, 0, b"N"),              # a single read; stride unused
    ]
    for idx, (n, L, stride, fill) in enumerate(cases):
        buf = _noisy_reads(rng, n, L, stride, fill)
        if idx == 0:
            g, o = _filters(params, kind, rng, buf)
        for offset in ((0, 1, 3) if idx in (0, 2) else (0,)):
            want = _check(g, o, params, buf, n, L, stride, offset, "%s %s case %d offset %d" % (kind, params, idx, offset))
        if idx == 0:
            ones = int(np.unpackbits(want.view(np.uint8)).sum())
            assert 0 < ones < n * (L - params[0] + 1), "answers should mix hits and misses"
    g.close()
    o.close()


def test_reads_with_gaps():
    """Reads with runs of 'N' (gaps that open, cut and end lanes, and reads
    that are all 'N'), where the per-read kernel's gap-free record numbering
    and last-k-mer-first writes decide which key each record holds."""
    params = (31, 16, 28, 4)
    rng = np.random.default_rng(9)
    n, L, stride = 500, 150, 151
    buf = _noisy_reads(rng, n, L, stride, rate=0.0)
    for r in range(n):
        kind = r % 5
        row = buf[r * stride:r * stride + L]
        if kind == 0:
            row[:] = ord("N")
        elif kind in (1, 2):
            p = int(rng.integers(0, L - 40))
            row[p:p + int(rng.integers(1, 40))] = ord("N")
        elif kind == 3:
            for p in rng.integers(0, L, 3):
                row[p] = ord("n")
    g, o = _filters(params, "sbf", rng, buf)
    want = _check(g, o, params, buf, n, L, stride, 0, "gaps")
    assert not want[::5].any(), "all-'N' reads have no hits"
    g.close()
    o.close()


def test_reads_fill_the_batch_end():
    """The last wave's reads end at the last byte of the device buffer (the
    kernel's byte-load path), for every residue of the batch size mod 4."""
    params = (31, 16, 28, 4)
    rng = np.random.default_rng(5)
    buf = _noisy_reads(rng, 200, 150, 151)
    g, o = _filters(params, "sbf", rng, buf)
    for n in (200, 199, 198, 197, 65, 64, 63):
        sub = buf[: (n - 1) * 151 + 150]
        _check(g, o, params, sub, n, 150, 151, 0, "end n=%d" % n)
    g.close()
    o.close()


def test_reads_errors_and_noops():
    torch = G.torch_cuda()
    from minimizer_sharded_bloom_amd import lib
    g = G.gpu_filter((31, 16, 28, 4), 2**14)
    buf = G.to_dev(_noisy_reads(np.random.default_rng(1), 4, 150, 151))
    out = torch.full((4, 4), -1, dtype=torch.int32, device="cuda")
    h = g._h
    C = lib()
    assert C.sbf_query_reads(h, buf.data_ptr(), 4, 150, 149, out.data_ptr(), None) == _lib.SBF_EINVAL
    assert C.sbf_query_reads(h, buf.data_ptr(), 4, 150, (1 << 25) + 1, out.data_ptr(), None) == _lib.SBF_EINVAL
    assert C.sbf_query_reads(h, None, 4, 150, 151, out.data_ptr(), None) == _lib.SBF_EINVAL
    assert C.sbf_query_reads(h, buf.data_ptr(), 4, 150, 151, None, None) == _lib.SBF_EINVAL
    assert C.sbf_query_reads(None, buf.data_ptr(), 4, 150, 151, out.data_ptr(), None) == _lib.SBF_EINVAL
    # 2^32 answer words or more: refused before any launch
    assert C.sbf_query_reads(h, buf.data_ptr(), 1 << 31, 150, 151, out.data_ptr(), None) == _lib.SBF_EINVAL
    # no reads, or reads shorter than k: nothing written
    assert C.sbf_query_reads(h, buf.data_ptr(), 0, 150, 151, out.data_ptr(), None) == _lib.SBF_OK
    assert C.sbf_query_reads(h, buf.data_ptr(), 4, 30, 151, out.data_ptr(), None) == _lib.SBF_OK
    torch.cuda.synchronize()
    assert int((out != -1).sum()) == 0
    # the binding checks a caller's output tensor before any call
    with pytest.raises(ValueError):
        g.query_reads(buf, 4, 150, 151, out=torch.empty(15, dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError):
        g.query_reads(buf, 4, 150, 151, out=torch.empty(16, dtype=torch.int64, device="cuda"))
    with pytest.raises(TypeError):
        g.query_reads(buf.cpu(), 4, 150, 151)
    with pytest.raises(ValueError):
        g.query_seq(buf, out=torch.empty(1, dtype=torch.int64, device="cuda"))
    g.close()
    p = G.gpu_filter((11, 5, 9, 3), 2**14, "protein")
    assert C.sbf_query_reads(p._h, buf.data_ptr(), 4, 150, 151, out.data_ptr(), None) == _lib.SBF_EUNSUPPORTED
    p.close()
