"""CPU check of the integer arithmetic that the DNA query's text front end
runs per dword of four ASCII bases (the 2-bit code of a base and its
validity: "cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data on
Modern GPUs", §IV-A).  The kernel's instruction sequence (two shifts and a
3-input bit function for the codes, a multiply that gathers the codes, a byte
lookup of the expected letter, a masked compare, an add that turns nonzero
bytes into bit 7, and a multiply that gathers the invalid flags of two dwords)
is restated here with numpy and compared with the oracle's per-base code on
every byte value at every position of a lane's 32 bytes and on random text.
The GPU parity tests check the kernel itself."""
import numpy as np
import pytest

from oracle import oracle as O

M32 = np.uint64(0xFFFFFFFF)


def bitop3(a, b, c, table):
    """Bitwise 3-input function: result bit = bit (4a + 2b + c) of table."""
    a, b, c = (np.asarray(v, dtype=np.uint64) for v in (a, b, c))
    r = np.zeros(np.broadcast(a, b, c).shape, dtype=np.uint64)
    for idx in range(8):
        if (table >> idx) & 1:
            ta = a if idx & 4 else ~a
            tb = b if idx & 2 else ~b
            tc = c if idx & 1 else ~c
            r |= ta & tb & tc
    return r & M32


def perm(s0, s1, sel):
    """Byte permute of the 8 bytes (s0:s1), selector bytes 0-7, 12 -> 0x00."""
    s0, s1, sel = (np.asarray(v, dtype=np.uint64) for v in (s0, s1, sel))
    data = (s0 << np.uint64(32)) | s1
    r = np.zeros(np.broadcast(s0, s1, sel).shape, dtype=np.uint64)
    for j in range(4):
        sb = (sel >> np.uint64(8 * j)) & np.uint64(0xFF)
        byte = (data >> (np.uint64(8) * np.minimum(sb, np.uint64(7)))) & np.uint64(0xFF)
        byte = np.where(sb <= 7, byte, np.uint64(0))  # only 12 (zero) is used
        r |= byte << np.uint64(8 * j)
    return r


def decode_lane(q):
    """Code words S[0], S[1] and validity bits of 32 bases from 8 dwords."""
    q = np.asarray(q, dtype=np.uint64)
    cc = bitop3(q >> np.uint64(1), q >> np.uint64(2), 0x03030303, 0x28)
    P = (cc * np.uint64(0x40100401)) & M32
    e = perm(0x74676361, 0x74676361, cc)
    d7 = bitop3(q, 0xA0A0A0A0, e, 0x12)
    Zi = bitop3((d7 + np.uint64(0x7F7F7F7F)) & M32, q, 0x80808080, 0xA8)
    S = [perm(P[..., 4 * u], P[..., 4 * u + 1], 0x07030C0C) | perm(P[..., 4 * u + 2], P[..., 4 * u + 3], 0x0C0C0703)
         for u in range(2)]
    V = [(((Zi[..., 2 * g] >> np.uint64(4)) | Zi[..., 2 * g + 1]) * np.uint64(0x00204081)) & M32 for g in range(4)]
    inv = perm(V[1], V[0], 0x0C0C0703) | perm(V[3], V[2], 0x07030C0C)
    return S[0], S[1], (~inv) & M32


def expected(blocks):
    """Per-base definition through the oracle: code c (< 0: invalid)."""
    codes = np.array([O.code(int(b)) for b in range(256)])
    c = codes[blocks]
    ok = c >= 0
    cv = np.where(ok, c, 0).astype(np.uint64)
    pos = np.arange(32)
    shift = (np.uint64(30) - np.uint64(2) * (pos % 16).astype(np.uint64))
    s0 = np.bitwise_or.reduce(np.where(pos < 16, cv << shift, 0), axis=-1)
    s1 = np.bitwise_or.reduce(np.where(pos >= 16, cv << shift, 0), axis=-1)
    valid = np.bitwise_or.reduce(ok.astype(np.uint64) << pos.astype(np.uint64), axis=-1)
    return s0, s1, valid, ok


def check(blocks):
    q = blocks.astype(np.uint64).reshape(blocks.shape[0], 8, 4)
    q = q[..., 0] | (q[..., 1] << np.uint64(8)) | (q[..., 2] << np.uint64(16)) | (q[..., 3] << np.uint64(24))
    s0, s1, valid = decode_lane(q)
    w0, w1, wv, ok = expected(blocks)
    assert (valid == wv).all()
    # codes of invalid bases are unspecified: compare the valid ones
    pos = np.arange(32)
    shift = (np.uint64(30) - np.uint64(2) * (pos % 16).astype(np.uint64))
    m = (ok.astype(np.uint64) * np.uint64(3)) << shift
    m0 = np.bitwise_or.reduce(np.where(pos < 16, m, 0), axis=-1)
    m1 = np.bitwise_or.reduce(np.where(pos >= 16, m, 0), axis=-1)
    assert ((s0 & m0) == w0).all() and ((s1 & m1) == w1).all()


def test_oracle_codes():
    """The oracle's code: A/C/G/T in either case are 0..3, all else invalid."""
    for b in range(256):
        want = "ACGT".find(chr(b).upper()) if chr(b).upper() in "ACGT" else -1
        assert (O.code(b) if O.code(b) >= 0 else -1) == want, b


def test_every_byte_at_every_position():
    base = np.frombuffer(b"ACGT" * 8, dtype=np.uint8)
    blocks = np.tile(base, (256 * 32, 1))
    for pos in range(32):
        blocks[pos * 256:(pos + 1) * 256, pos] = np.arange(256, dtype=np.uint8)
    check(blocks)


@pytest.mark.parametrize("alphabet", [None, b"ACGTacgtNn\x00\xc1\xe1@*Z"])
def test_random_lanes(alphabet):
    rng = np.random.default_rng(11)
    if alphabet is None:
        blocks = rng.integers(0, 256, (20000, 32)).astype(np.uint8)
    else:
        a = np.frombuffer(alphabet, dtype=np.uint8)
        blocks = a[rng.integers(0, a.size, (20000, 32))]
    check(blocks)
