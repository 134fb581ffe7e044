"""ctypes binding of the CPU oracle (oracle/sbf_oracle.c).

TEST INFRASTRUCTURE ONLY.  The oracle is the plain per-k-mer definition of the
Super Bloom filter of "cuSBF: A Minimizer-Aware Bloom Filter for Genomic
Sequence Data on Modern GPUs"; the GPU library is checked against it.  Only
the tests, the smoke entry point and the benchmark's CPU-baseline leg may
import this module.  It imports nothing from the GPU package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sbf_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

KIND_SBF = 0
KIND_BBF = 1
KIND_WIDE = 2  # 512-bit blocks, each hash addressing the whole block

ALPHA_DNA = 0      # A C G T, 2 bits per symbol
ALPHA_PROTEIN = 1  # letters A-Z, 5 bits per symbol
ALPHA_TRIPLET = 2  # non-overlapping DNA codons, 6 bits per symbol


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no vectorisation flags)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=gnu99", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Werror", "-o", tmp, SRC])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        u64, u32, p = ctypes.c_uint64, ctypes.c_uint, ctypes.c_void_p
        L.osbf_code.argtypes = [ctypes.c_ubyte]
        L.osbf_code.restype = ctypes.c_int
        for name in ("osbf_hmin", "osbf_mix", "osbf_hs"):
            getattr(L, name).argtypes = [u64]
            getattr(L, name).restype = u64
        L.osbf_bitaddr.argtypes = [u64, u32, u32]
        L.osbf_bitaddr.restype = u32
        L.osbf_bitaddr_wide.argtypes = [u64, u32, u32]
        L.osbf_bitaddr_wide.restype = u32
        L.osbf_minimizer_hashes.argtypes = [p, u64, u32, u32, p]
        L.osbf_minimizer_hashes.restype = u64
        L.osbf_words_per_shard.argtypes = [p]
        L.osbf_words_per_shard.restype = u32
        L.osbf_probe_kmer.argtypes = [u64, u64, u32]
        L.osbf_probe_kmer.restype = u64
        L.osbf_pack_kmer.argtypes = [ctypes.c_char_p, u32, ctypes.POINTER(u64)]
        L.osbf_pack_kmer.restype = ctypes.c_int
        L.osbf_subwindow.argtypes = [u64, u32, u32, u32]
        L.osbf_subwindow.restype = u64
        L.osbf_minimizer_hash.argtypes = [u64, u32, u32]
        L.osbf_minimizer_hash.restype = u64
        L.osbf_create.argtypes = [ctypes.c_int, u32, u32, u32, u32, u64]
        L.osbf_create.restype = p
        L.osbf_create_alpha.argtypes = [ctypes.c_int, u32, u32, u32, u32, u32, u64]
        L.osbf_create_alpha.restype = p
        L.osbf_code_protein.argtypes = [ctypes.c_ubyte]
        L.osbf_code_protein.restype = ctypes.c_int
        L.osbf_code_triplet.argtypes = [ctypes.c_char_p]
        L.osbf_code_triplet.restype = ctypes.c_int
        L.osbf_symbol_bits.argtypes = [u32]
        L.osbf_symbol_bits.restype = u32
        L.osbf_pack_kmer_alpha.argtypes = [u32, p, u64, u32, ctypes.POINTER(u64)]
        L.osbf_pack_kmer_alpha.restype = ctypes.c_int
        L.osbf_probe_kmer_alpha.argtypes = [u32, u64, u64, u32]
        L.osbf_probe_kmer_alpha.restype = u64
        L.osbf_destroy.argtypes = [p]
        L.osbf_destroy.restype = None
        L.osbf_num_shards.argtypes = [p]
        L.osbf_num_shards.restype = u64
        L.osbf_words.argtypes = [p]
        L.osbf_words.restype = ctypes.POINTER(u64)
        L.osbf_shard_of.argtypes = [p, u64]
        L.osbf_shard_of.restype = u64
        L.osbf_insert_kmer.argtypes = [p, u64]
        L.osbf_insert_kmer.restype = None
        L.osbf_query_kmer.argtypes = [p, u64]
        L.osbf_query_kmer.restype = ctypes.c_int
        L.osbf_insert_seq.argtypes = [p, p, u64]
        L.osbf_insert_seq.restype = None
        L.osbf_query_seq.argtypes = [p, p, u64, p]
        L.osbf_query_seq.restype = None
        L.osbf_query_positions.argtypes = [p, p, u64, p, u64, p]
        L.osbf_query_positions.restype = None
        L.osbf_fpr_probe.argtypes = [p, u64, u64]
        L.osbf_fpr_probe.restype = u64
        L.osbf_insert_seq_mt.argtypes = [p, p, u64, u32]
        L.osbf_insert_seq_mt.restype = None
        L.osbf_query_seq_mt.argtypes = [p, p, u64, p, u32]
        L.osbf_query_seq_mt.restype = None
        L.osbf_insert_seq_sampled_mt.argtypes = [p, p, u64, u64, u64, u32]
        L.osbf_insert_seq_sampled_mt.restype = None
        L.osbf_query_seq_sampled_mt.argtypes = [p, p, u64, p, p, u64, u64, u32]
        L.osbf_query_seq_sampled_mt.restype = None
        _lib = L
    return _lib


def _buf(seq):
    """Return (numpy uint8 array, pointer) for bytes / str / uint8 arrays."""
    if isinstance(seq, str):
        seq = seq.encode("ascii")
    if isinstance(seq, (bytes, bytearray)):
        arr = np.frombuffer(bytes(seq), dtype=np.uint8)
    else:
        arr = np.ascontiguousarray(seq, dtype=np.uint8)
    return arr, arr.ctypes.data


# ---- primitives ------------------------------------------------------------

def code(c) -> int:
    if isinstance(c, str):
        c = ord(c)
    return lib().osbf_code(c)


def hmin(v: int) -> int:
    return lib().osbf_hmin(v & (2**64 - 1))


def mix(z: int) -> int:
    return lib().osbf_mix(z & (2**64 - 1))


def hs(v: int) -> int:
    return lib().osbf_hs(v & (2**64 - 1))


def bitaddr(h: int, t: int, H: int) -> int:
    return lib().osbf_bitaddr(h, t, H)


def bitaddr_wide(h: int, t: int, H: int) -> int:
    return lib().osbf_bitaddr_wide(h, t, H)


def probe_kmer(seed: int, i: int, k: int) -> int:
    return lib().osbf_probe_kmer(seed & (2**64 - 1), i, k)


def pack_kmer(s) -> int | None:
    if isinstance(s, str):
        s = s.encode("ascii")
    x = ctypes.c_uint64(0)
    rc = lib().osbf_pack_kmer(s, len(s), ctypes.byref(x))
    return None if rc != 0 else x.value


def code_protein(c) -> int:
    if isinstance(c, str):
        c = ord(c)
    return lib().osbf_code_protein(c)


def code_triplet(codon) -> int:
    if isinstance(codon, str):
        codon = codon.encode("ascii")
    assert len(codon) == 3
    return lib().osbf_code_triplet(codon)


def symbol_bits(alpha: int) -> int:
    return lib().osbf_symbol_bits(alpha)


def pack_kmer_alpha(alpha: int, seq, p: int, k: int) -> int | None:
    """k symbols from symbol p of seq, packed first-most-significant."""
    arr, ptr = _buf(seq)
    x = ctypes.c_uint64(0)
    rc = lib().osbf_pack_kmer_alpha(alpha, ptr, p, k, ctypes.byref(x))
    return None if rc != 0 else x.value


def probe_kmer_alpha(alpha: int, seed: int, i: int, k: int) -> int:
    return lib().osbf_probe_kmer_alpha(alpha, seed & (2**64 - 1), i, k)


def n_symbols(alpha: int, nbytes: int) -> int:
    return nbytes // 3 if alpha == ALPHA_TRIPLET else nbytes


def subwindow(x: int, k: int, i: int, w: int) -> int:
    return lib().osbf_subwindow(x, k, i, w)


def minimizer_hash(x: int, k: int, m: int) -> int:
    return lib().osbf_minimizer_hash(x, k, m)


def minimizer_hashes(seq, k: int, m: int) -> np.ndarray:
    """Minimizer hash of every k-mer start of a DNA text (oracle, one k-mer at
    a time); 2^64 - 1 where the k-mer is invalid."""
    arr, ptr = _buf(seq)
    n = max(0, arr.size - k + 1)
    out = np.empty(n, dtype=np.uint64)
    if n:
        lib().osbf_minimizer_hashes(ptr, arr.size, k, m, out.ctypes.data)
    return out


# ---- filter ----------------------------------------------------------------

def _threads(n: int) -> int:
    """Thread count for the threaded drivers: n, else the cores this process
    may use, at most 16."""
    if n:
        return n
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(16, avail))


class OracleFilter:
    """A Super Bloom filter (kind=KIND_SBF), its wide-block variant
    (KIND_WIDE) or a per-k-mer blocked Bloom filter (KIND_BBF) held in host
    memory by the C oracle."""

    def __init__(self, k, m, s, H, bits, kind=KIND_SBF, alpha=ALPHA_DNA):
        self.k, self.m, self.s, self.H, self.kind, self.alpha = k, m, s, H, kind, alpha
        self._h = lib().osbf_create_alpha(kind, alpha, k, m, s, H, bits)
        if not self._h:
            raise ValueError("oracle: invalid parameters (alphabet=%d k=%d m=%d s=%d H=%d bits=%d)"
                             % (alpha, k, m, s, H, bits))

    def _nk(self, nbytes: int) -> int:
        """k-mer starts in a sequence of nbytes bytes."""
        return max(0, n_symbols(self.alpha, nbytes) - self.k + 1)

    def close(self):
        if self._h:
            lib().osbf_destroy(self._h)
            self._h = None

    __del__ = close

    @property
    def num_shards(self) -> int:
        return lib().osbf_num_shards(self._h)

    @property
    def words_per_shard(self) -> int:
        return lib().osbf_words_per_shard(self._h)

    def words(self) -> np.ndarray:
        """Copy of the filter: uint64[words_per_shard * num_shards]."""
        n = self.words_per_shard * self.num_shards
        ptr = lib().osbf_words(self._h)
        return np.ctypeslib.as_array(ptr, shape=(n,)).copy()

    def shard_of(self, x: int) -> int:
        return lib().osbf_shard_of(self._h, x)

    def insert_kmer(self, x: int):
        lib().osbf_insert_kmer(self._h, x)

    def query_kmer(self, x: int) -> bool:
        return bool(lib().osbf_query_kmer(self._h, x))

    def insert_seq(self, seq):
        arr, ptr = _buf(seq)
        lib().osbf_insert_seq(self._h, ptr, arr.size)

    def query_seq(self, seq) -> np.ndarray:
        """uint64 bit words, bit p = answer for the k-mer starting at symbol p."""
        arr, ptr = _buf(seq)
        nk = self._nk(arr.size)
        out = np.zeros((nk + 63) // 64, dtype=np.uint64)
        if nk:
            lib().osbf_query_seq(self._h, ptr, arr.size, out.ctypes.data)
        return out

    def insert_seq_mt(self, seq, nthreads: int = 0):
        """insert_seq with the k-mer starts split over threads (0 = all cores)."""
        arr, ptr = _buf(seq)
        lib().osbf_insert_seq_mt(self._h, ptr, arr.size, _threads(nthreads))

    def query_seq_mt(self, seq, nthreads: int = 0) -> np.ndarray:
        arr, ptr = _buf(seq)
        nk = self._nk(arr.size)
        out = np.zeros((nk + 63) // 64, dtype=np.uint64)
        if nk:
            lib().osbf_query_seq_mt(self._h, ptr, arr.size, out.ctypes.data, _threads(nthreads))
        return out

    def insert_seq_sampled_mt(self, seq, sample_mask: int, sample_value: int, nthreads: int = 0):
        """Insert only k-mers whose shard s has (s & sample_mask) == sample_value."""
        arr, ptr = _buf(seq)
        lib().osbf_insert_seq_sampled_mt(self._h, ptr, arr.size, sample_mask, sample_value, _threads(nthreads))

    def query_seq_sampled_mt(self, seq, sample_mask: int, sample_value: int, nthreads: int = 0):
        """(answers, checked) bit words over the k-mers of sampled shards."""
        arr, ptr = _buf(seq)
        nk = self._nk(arr.size)
        out = np.zeros((nk + 63) // 64, dtype=np.uint64)
        checked = np.zeros_like(out)
        if nk:
            lib().osbf_query_seq_sampled_mt(self._h, ptr, arr.size, out.ctypes.data, checked.ctypes.data,
                                            sample_mask, sample_value, _threads(nthreads))
        return out, checked

    def query_positions(self, seq, positions) -> np.ndarray:
        arr, ptr = _buf(seq)
        pos = np.ascontiguousarray(positions, dtype=np.uint64)
        out = np.zeros(pos.size, dtype=np.uint8)
        lib().osbf_query_positions(self._h, ptr, arr.size, pos.ctypes.data, pos.size,
                                   out.ctypes.data)
        return out

    def fpr_probe(self, n: int, seed: int) -> int:
        return lib().osbf_fpr_probe(self._h, n, seed & (2**64 - 1))
