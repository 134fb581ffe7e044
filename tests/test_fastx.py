"""The library's FASTA/FASTQ reader (host code, no GPU) against the reference
normalization in tests/fastx_ref.py: records joined by one 'N', line breaks
and whitespace removed ([cuSBF] §IV-A input forms, §IV-F separators), for
plain, gzip and BGZF files, multi-line records, CRLF, comments, empty records
and FASTQ quality lines that start with '@'."""
import ctypes
import gzip
import os

import numpy as np
import pytest

import minimizer_sharded_bloom_amd as M
from minimizer_sharded_bloom_amd import _lib
from minimizer_sharded_bloom_amd import synthetic as S
from tests import fastx_ref as R


def read_all(path, piece=1 << 20, ends_cap=1 << 16):
    """Whole normalized stream and record ends through sbf_fastx_read with the
    given piece size and end-offset capacity."""
    L = M.lib()
    r = ctypes.c_void_p()
    assert L.sbf_fastx_open(ctypes.byref(r), os.fsencode(path)) == 0
    out, ends = bytearray(), []
    buf = np.empty(piece, dtype=np.uint8)
    eb = np.empty(ends_cap, dtype=np.uint64)
    n, ne = ctypes.c_uint64(), ctypes.c_uint64()
    try:
        while True:
            rc = L.sbf_fastx_read(r, buf.ctypes.data, piece, ctypes.byref(n), eb.ctypes.data, ends_cap,
                                  ctypes.byref(ne))
            if rc:
                raise M.SbfError(rc, "sbf_fastx_read")
            if n.value == 0 and ne.value == 0:
                break
            out += buf[:n.value].tobytes()
            ends += [int(x) for x in eb[:ne.value]]
        nrec = L.sbf_fastx_records(r)
    finally:
        L.sbf_fastx_close(r)
    return bytes(out), ends, nrec


def random_records(rng, n, max_len=400, alphabet=b"ACGTacgtN"):
    a = np.frombuffer(alphabet, dtype=np.uint8)
    lens = rng.integers(0, max_len, n)
    lens[rng.random(n) < 0.1] = 0  # some empty records
    return [a[rng.integers(0, a.size, l)].tobytes() for l in lens]


def fasta_text(rng, recs, crlf=False, comments=False):
    eol = b"\r\n" if crlf else b"\n"
    parts = []
    for i, s in enumerate(recs):
        parts.append(b">rec %d some description" % i + eol)
        if comments and rng.random() < 0.3:
            parts.append(b"; a comment line" + eol)
        w = int(rng.integers(1, 100))
        for a in range(0, len(s), w):
            parts.append(s[a:a + w] + eol)
        if rng.random() < 0.2:
            parts.append(eol)  # blank line
    return b"".join(parts)


def fastq_text(rng, recs, multiline=False):
    parts = []
    for i, s in enumerate(recs):
        q = bytes(rng.integers(33, 75, len(s), dtype=np.uint8))
        q = b"@" + q[1:] if len(q) > 1 and rng.random() < 0.3 else q  # quality starting with '@'
        parts.append(b"@read%d\n" % i)
        if multiline and len(s) > 10:
            w = int(rng.integers(5, 40))
            parts += [s[a:a + w] + b"\n" for a in range(0, len(s), w)]
            parts.append(b"+\n")
            parts += [q[a:a + w] + b"\n" for a in range(0, len(q), w)]
        else:
            parts.append(s + b"\n+read%d\n" % i + q + b"\n")
    return b"".join(parts)


def write(tmp_path, name, data, gz=False):
    p = tmp_path / name
    if gz:
        with gzip.open(p, "wb") as f:
            f.write(data)
    else:
        p.write_bytes(data)
    return str(p)


@pytest.mark.parametrize("gz", [False, True])
@pytest.mark.parametrize("kind", ["fasta", "fasta_crlf", "fastq", "fastq_multiline"])
def test_reader_matches_reference(tmp_path, kind, gz):
    rng = np.random.default_rng(["fasta", "fasta_crlf", "fastq", "fastq_multiline"].index(kind) * 2 + int(gz))
    recs = random_records(rng, 300)
    if kind.startswith("fasta"):
        text = fasta_text(rng, recs, crlf=kind.endswith("crlf"), comments=True)
    else:
        text = fastq_text(rng, recs, multiline=kind.endswith("multiline"))
    path = write(tmp_path, "in", text, gz)
    want, want_ends = R.normalize(text)
    assert want == b"N".join(recs)  # the reference agrees with how the file was built
    for piece, ecap in [(1 << 20, 1 << 16), (7, 1), (64, 3), (1000, 1)]:
        got, ends, nrec = read_all(path, piece, ecap)
        assert got == want, (piece, ecap)
        assert ends == want_ends, (piece, ecap)
        assert nrec == len(recs)


def test_reader_large_fasta(tmp_path):
    """A 3 MB FASTA file with random line widths, CRLF and LF lines, comments,
    blank lines, empty records, a '>' inside a sequence line and one 600 kB
    record on a single line matches the reference for piece sizes and end
    capacities that stop calls at every kind of place, and its gzip copy
    reads the same."""
    rng = np.random.default_rng(12)
    parts = []
    recs = random_records(rng, 2000, max_len=2500, alphabet=b"ACGTacgtNRY")
    for i, s in enumerate(recs):
        eol = b"\r\n" if rng.random() < 0.3 else b"\n"
        parts.append(b">r%d desc >not a header" % i + eol)
        if rng.random() < 0.1:
            parts.append(b";comment" + eol)
        if i == 700:
            s = bytes(rng.choice(np.frombuffer(b"ACGT", dtype=np.uint8), 600_000))
            recs[i] = s
            parts.append(s + eol)
            continue
        w = int(rng.integers(1, 200))
        for a in range(0, len(s), w):
            parts.append(s[a:a + w] + eol)
        if rng.random() < 0.1:
            parts.append(eol * int(rng.integers(1, 4)))
    parts.append(b"ACG>T\n")  # '>' inside a line is a base of the last record
    recs[-1] = recs[-1] + b"ACG>T"
    text = b"\n\n" + b"".join(parts)
    path = write(tmp_path, "big.fa", text)
    want, want_ends = R.normalize(text)
    assert want == b"N".join(recs)
    for piece, ecap in [(1 << 22, 1 << 16), (1 << 20, 5), (100_003, 1), (65_537, 64), (1 << 22, 1)]:
        got, ends, nrec = read_all(path, piece, ecap)
        assert got == want, (piece, ecap)
        assert ends == want_ends, (piece, ecap)
        assert nrec == len(recs)
    gz, gz_ends, _ = read_all(write(tmp_path, "big.fa.gz", text, gz=True), 1 << 22)
    assert gz == want and gz_ends == want_ends


def test_reader_multimember_gzip(tmp_path):
    rng = np.random.default_rng(5)
    a = fasta_text(rng, random_records(rng, 50))
    b = fasta_text(rng, random_records(rng, 50))
    p = tmp_path / "mm.fa.gz"
    p.write_bytes(gzip.compress(a) + gzip.compress(b))
    got, ends, _ = read_all(str(p))
    want, want_ends = R.normalize(a + b)
    assert got == want and ends == want_ends


def test_bgzf_writer_is_gzip():
    """The test writer's BGZF files are gzip files that Python's own decoder
    reads back, and the end-of-file member is the 28-byte empty block."""
    data = bytes(np.random.default_rng(1).integers(0, 256, 300_000, dtype=np.uint8))
    for block in (1, 999, 0xFF00):
        assert gzip.decompress(S.bgzf_bytes(data[:50_000] if block == 1 else data, block=block)) == \
            (data[:50_000] if block == 1 else data)
    assert len(S.bgzf_bytes(b"")) == 28


@pytest.mark.parametrize("block,level", [(0xFF00, 6), (4093, 1), (1, 0)])
def test_reader_bgzf(tmp_path, block, level):
    """BGZF input (members inflated in parallel, several batches of members)
    reads exactly as the plain file, for full 64 KiB blocks, odd block sizes
    that cut lines and records anywhere, and one-byte blocks."""
    rng = np.random.default_rng(block)
    recs = random_records(rng, 3000 if block > 1 else 300, max_len=3000)
    text = fasta_text(rng, recs, comments=True) + fastq_text(rng, [])
    want, want_ends = R.normalize(text)
    p = tmp_path / "x.fa.bgz"
    p.write_bytes(S.bgzf_bytes(text, block=block, level=level))
    for piece, ecap in [(1 << 20, 1 << 16), (4099, 7)]:
        got, ends, nrec = read_all(str(p), piece, ecap)
        assert got == want and ends == want_ends and nrec == len(recs), (piece, ecap)


def test_reader_bgzf_many_batches(tmp_path):
    """A 20 MB FASTQ file stored uncompressed in BGZF members spans three 8 MiB
    batches of compressed input, so members are cut by the batch ends; with
    empty members between the others and no end-of-file member it reads as
    the plain file."""
    recs = list(S.to_ascii(S.random_reads(120_000, 80, seed=3)))
    plain = tmp_path / "r.fq"
    S.write_fastq(str(plain), recs)
    text = plain.read_bytes()
    assert len(text) > 2 * (8 << 20)
    members = S.bgzf_bytes(text, block=30011, level=0, eof=False)
    empty = S.bgzf_bytes(b"", eof=True)
    # an empty member after every 100th one
    cut, parts, o = 0, [], 0
    import struct
    while o < len(members):
        size = struct.unpack_from("<H", members, o + 16)[0] + 1
        parts.append(members[o:o + size])
        cut += 1
        if cut % 100 == 0:
            parts.append(empty)
        o += size
    p = tmp_path / "r.fq.bgz"
    p.write_bytes(b"".join(parts))
    got, ends, nrec = read_all(str(p), 1 << 22)
    want, want_ends, _ = read_all(str(plain), 1 << 22)
    assert got == want == b"N".join(r.tobytes() for r in recs) and ends == want_ends and nrec == 120_000


def test_reader_bgzf_mixed_and_trailing(tmp_path):
    """A BGZF file followed by plain gzip members (another gzip file
    appended) reads as the whole text, the part after the BGZF members
    through gzread; bytes after the last member that are not gzip are
    ignored, as zlib ignores them."""
    rng = np.random.default_rng(4)
    a = fasta_text(rng, random_records(rng, 800))
    b = fasta_text(rng, random_records(rng, 300))
    c = fasta_text(rng, random_records(rng, 200))
    bg = S.bgzf_bytes(a, block=3000)
    for name, data, text in [("mixed", bg + gzip.compress(b), a + b),
                             ("mixed_then_bgzf", bg[:-28] + gzip.compress(b) + S.bgzf_bytes(c, block=777), a + b + c),
                             ("trailing", bg + b"garbage that is not gzip\n", a)]:
        got, ends, nrec = read_all(write(tmp_path, name, data), 4099, 7)
        want, want_ends = R.normalize(text)
        assert got == want and ends == want_ends, name
        assert read_all(write(tmp_path, name + ".gz_ref", gzip.compress(text)))[0] == want


def test_reader_bgzf_errors(tmp_path):
    """Damaged BGZF files end with SBF_EIO: a CRC-32 that does not match, a
    wrong ISIZE, a file cut inside a member."""
    rng = np.random.default_rng(8)
    text = fasta_text(rng, random_records(rng, 500))
    good = bytearray(S.bgzf_bytes(text, block=5000))
    bad_crc = bytearray(good)
    bad_crc[-28 - 8] ^= 1  # CRC of the last data member
    bad_isize = bytearray(good)
    bad_isize[-28 - 4] ^= 1
    cases = {"crc": bytes(bad_crc), "isize": bytes(bad_isize), "cut": bytes(good[:-28 - 100]),
             # a gzip member after the BGZF ones, cut before its end (read by gzread)
             "cut_tail": bytes(good[:-28]) + gzip.compress(b">x\nACGTACGT\n" * 50)[:-12]}
    assert read_all(write(tmp_path, "good", bytes(good)))[0] == R.normalize(text)[0]
    for name, data in cases.items():
        with pytest.raises(M.SbfError) as e:
            read_all(write(tmp_path, name, data))
        assert e.value.code == _lib.SBF_EIO, name


def test_reader_truncated_gzip(tmp_path):
    """A gzip file cut inside its member is an error, not a shorter input:
    gzread reports such an end as the end of the file, and the reader checks
    gzerror for it."""
    rng = np.random.default_rng(6)
    text = fasta_text(rng, random_records(rng, 200))
    full = gzip.compress(text)
    assert read_all(write(tmp_path, "full.gz", full))[0] == R.normalize(text)[0]
    for cut in (8, 100, len(full) // 2):
        with pytest.raises(M.SbfError) as e:
            read_all(write(tmp_path, "cut%d.gz" % cut, full[:-cut]))
        assert e.value.code == _lib.SBF_EIO, cut


def test_reader_mutated_texts(tmp_path):
    """Seeded random edits (deleted, inserted and replaced bytes among
    '@+>;', line breaks, CR, spaces and bases) of small FASTA and FASTQ
    files, read plain, as gzip and as BGZF with small blocks: the reader
    returns the reference normalization whenever the reference accepts the
    text, and SBF_EIO whenever it refuses it."""
    import random
    rng = np.random.default_rng(17)
    pr = random.Random(17)
    for it in range(300):
        recs = random_records(rng, int(rng.integers(1, 6)), max_len=50)
        if pr.random() < 0.5:
            text = fasta_text(rng, recs, crlf=pr.random() < 0.3, comments=True)
        else:
            text = fastq_text(rng, recs, multiline=pr.random() < 0.5)
        b = bytearray(text)
        for _ in range(pr.randint(1, 4)):
            op, pos = pr.random(), pr.randrange(len(b) + 1)
            if op < 0.33 and b:
                del b[min(pos, len(b) - 1)]
            elif op < 0.66:
                b.insert(pos, pr.choice(b"@+>;\n\r ACGTN!I\t"))
            elif b:
                b[min(pos, len(b) - 1)] = pr.choice(b"@+>;\n\r ACGTN!I")
        data = bytes(b)
        try:
            want = R.normalize(data)
        except (AssertionError, ValueError):
            want = None
        wrap = it % 3
        raw = data if wrap == 0 else gzip.compress(data) if wrap == 1 else S.bgzf_bytes(data, block=pr.choice([5, 64, 500]))
        path = write(tmp_path, "m%d" % it, raw)
        try:
            got = read_all(path, 1 << 12, 16)
            got = (got[0], got[1])
        except M.SbfError as e:
            assert e.code == _lib.SBF_EIO
            got = None
        assert got == want, (it, data)


def test_reader_synthetic_writers(tmp_path):
    """write_fasta / write_fastq of generated reads read back as the reads
    joined by 'N'."""
    g = S.genome_with_repeats(20_000)
    reads = S.short_read_set(g, 200)
    recs = S.split_records(reads)
    assert len(recs) == 200
    for name, fn in [("r.fa", lambda p: S.write_fasta(p, recs, width=70)),
                     ("r.fa.gz", lambda p: S.write_fasta(p, recs, gz=True, crlf=True)),
                     ("r.fa.bgz", lambda p: S.write_fasta(p, recs, gz="bgzf")),
                     ("r.fq", lambda p: S.write_fastq(p, recs))]:
        p = str(tmp_path / name)
        fn(p)
        got, ends, nrec = read_all(p)
        assert got == reads.tobytes() and nrec == 200
        assert ends == [int(x) for x in np.flatnonzero(np.append(reads, ord("N")) == ord("N"))]


def test_reader_empty_and_errors(tmp_path):
    L = M.lib()
    got, ends, nrec = read_all(write(tmp_path, "empty", b""))
    assert got == b"" and ends == [] and nrec == 0
    got, ends, _ = read_all(write(tmp_path, "hdr", b">only\n>two\n"))
    assert got == b"N" and ends == [0, 1]
    r = ctypes.c_void_p()
    assert L.sbf_fastx_open(ctypes.byref(r), b"/nonexistent/file.fa") == _lib.SBF_EIO
    for name, data in [("raw", b"ACGTACGT\n"), ("badfq", b"@r\nACGT\n+\nII\n"), ("badhdr", b"@r\nAC\n+\nII\nXX\n")]:
        with pytest.raises(M.SbfError) as e:
            read_all(write(tmp_path, name, data))
        assert e.value.code == _lib.SBF_EIO


def test_fastx_stream_helper(tmp_path):
    rng = np.random.default_rng(9)
    recs = random_records(rng, 100, alphabet=b"ACGT")
    path = write(tmp_path, "x.fa", fasta_text(rng, recs))
    pieces = list(M.fastx_stream(path, piece=1000))
    assert b"".join(p for p, _ in pieces) == b"N".join(recs)
    assert M.count_fastx_records(path) == 100
