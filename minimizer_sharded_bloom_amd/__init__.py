"""MI355X (gfx950) Super Bloom filter: Python binding of libsbf.so.

The method is that of "cuSBF: A Minimizer-Aware Bloom Filter for Genomic
Sequence Data on Modern GPUs": a k-mer's minimizer hash picks a 256-bit shard,
its k-s+1 s-mers set or test H bits inside it, and a query answers present
only if every s-mer hits.  The functions and methods here marshal arguments
to the C ABI of include/sbf.h; PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import _lib
from ._lib import (SBF_ALPHABET_DNA, SBF_ALPHABET_PROTEIN, SBF_ALPHABET_TRIPLET, SBF_DEVICE, SBF_HOST, SbfError,
                   check)

__all__ = ["SuperBloomFilter", "pack", "packed_words", "SbfError", "lib", "fastx_stream", "count_fastx_records"]


def lib():
    return _lib.load()


def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> int | None:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _is_device_tensor(x) -> bool:
    try:
        torch = _torch()
    except ImportError:
        return False
    return isinstance(x, torch.Tensor) and x.is_cuda


def _device_bytes(seq, stream):
    """A contiguous 1-D view of a CUDA uint8 tensor.  A non-contiguous input
    is copied; the copy is recorded on `stream` so the caching allocator does
    not reuse it while the asynchronous call may still read it there."""
    torch = _torch()
    if seq.dtype != torch.uint8:
        raise TypeError("expected a CUDA uint8 tensor of ASCII bytes, got %s" % (seq.dtype,))
    a = seq.contiguous().view(-1)
    if not seq.is_contiguous() and stream is not None:
        st = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(_stream_ptr(stream))
        a.record_stream(st)
    return a


def _check_out(out, words: int, dtype, device):
    """A caller-supplied output tensor must be a contiguous device tensor of
    `dtype` with room for `words` elements on the input's device."""
    if not _is_device_tensor(out) or out.dtype != dtype or not out.is_contiguous():
        raise TypeError("out must be a contiguous CUDA %s tensor" % (dtype,))
    if out.device != device:
        raise ValueError("out is on %s, the input on %s" % (out.device, device))
    if out.numel() < words:
        raise ValueError("out holds %d elements; %d are needed" % (out.numel(), words))


def _host_bytes(seq) -> np.ndarray:
    if isinstance(seq, str):
        seq = seq.encode("ascii")
    if isinstance(seq, (bytes, bytearray, memoryview)):
        return np.frombuffer(bytes(seq), dtype=np.uint8)
    if _is_device_tensor(seq):
        raise TypeError("expected host data")
    if hasattr(seq, "numpy"):
        seq = seq.numpy()
    return np.ascontiguousarray(seq, dtype=np.uint8).reshape(-1)


def packed_words(length: int) -> tuple[int, int]:
    """(code words, validity words) of the packed layout of `length` bases."""
    cw, vw = ctypes.c_uint64(), ctypes.c_uint64()
    lib().sbf_packed_words(length, ctypes.byref(cw), ctypes.byref(vw))
    return cw.value, vw.value


def pack(ascii_dev, stream=None):
    """Pack a device uint8 tensor of ASCII bases into (codes, valid) int32
    device tensors in the layout of include/sbf.h.  Asynchronous."""
    torch = _torch()
    if not _is_device_tensor(ascii_dev) or ascii_dev.dtype != torch.uint8:
        raise TypeError("pack expects a CUDA uint8 tensor")
    a = _device_bytes(ascii_dev, stream)
    cw, vw = packed_words(a.numel())
    codes = torch.empty(max(cw, 1), dtype=torch.int32, device=a.device)
    valid = torch.empty(max(vw, 1), dtype=torch.int32, device=a.device)
    check(lib().sbf_pack(a.data_ptr(), a.numel(), codes.data_ptr(), valid.data_ptr(), _stream_ptr(stream)), "sbf_pack")
    return codes, valid


class SuperBloomFilter:
    """A Super Bloom filter (or, with `blocked()`, the per-k-mer blocked Bloom
    comparator; with `wide()`, the 512-bit whole-block variant) living in
    device memory."""

    def __init__(self, k: int, m: int, s: int, H: int, bits: int, *, _kind: int = _lib.SBF_KIND_SBF,
                 _alphabet: int = _lib.SBF_ALPHABET_DNA):
        h = ctypes.c_void_p()
        if _alphabet != _lib.SBF_ALPHABET_DNA:
            check(lib().sbf_create_alphabet(ctypes.byref(h), _alphabet, k, m, s, H, bits), "sbf_create_alphabet")
        elif _kind == _lib.SBF_KIND_BBF:
            check(lib().sbf_create_bbf(ctypes.byref(h), k, H, bits), "sbf_create_bbf")
        elif _kind == _lib.SBF_KIND_WIDE:
            check(lib().sbf_create_wide(ctypes.byref(h), k, m, s, H, bits), "sbf_create_wide")
        else:
            check(lib().sbf_create(ctypes.byref(h), k, m, s, H, bits), "sbf_create")
        self._h = h
        inf = _lib.SbfInfo()
        check(lib().sbf_info(self._h, ctypes.byref(inf)), "sbf_info")
        self.k, self.m, self.s, self.H = inf.k, inf.m, inf.s, inf.H
        self.kind = inf.kind
        self.specialized = bool(inf.specialized)
        self.num_shards = inf.num_shards
        self.filter_bytes = inf.filter_bytes
        self.words_per_shard = inf.words_per_shard
        self.alphabet = inf.alphabet

    @classmethod
    def blocked(cls, k: int, H: int, bits: int) -> "SuperBloomFilter":
        return cls(k, 0, 0, H, bits, _kind=_lib.SBF_KIND_BBF)

    @classmethod
    def wide(cls, k: int, m: int, s: int, H: int, bits: int) -> "SuperBloomFilter":
        """Wide-block variant: 512-bit blocks, each hash addressing the whole block."""
        return cls(k, m, s, H, bits, _kind=_lib.SBF_KIND_WIDE)

    @classmethod
    def protein(cls, k: int, m: int, s: int, H: int, bits: int) -> "SuperBloomFilter":
        """Protein alphabet: letters A-Z, 5 bits per symbol, k <= 12."""
        return cls(k, m, s, H, bits, _alphabet=_lib.SBF_ALPHABET_PROTEIN)

    @classmethod
    def triplet(cls, k: int, m: int, s: int, H: int, bits: int) -> "SuperBloomFilter":
        """DNA-triplet alphabet: codons of 3 bytes, 6 bits per symbol, k <= 10."""
        return cls(k, m, s, H, bits, _alphabet=_lib.SBF_ALPHABET_TRIPLET)

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            check(lib().sbf_destroy(self._h), "sbf_destroy")
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def handle(self) -> int:
        return self._h.value

    def num_symbols(self, length: int) -> int:
        """Symbols in `length` bytes (a triplet symbol is 3 bytes)."""
        return length // 3 if self.alphabet == _lib.SBF_ALPHABET_TRIPLET else length

    def num_answer_words(self, length: int) -> int:
        n = self.num_symbols(length)
        return 0 if n < self.k else (n - self.k + 1 + 63) // 64

    # ---- filter state ------------------------------------------------------
    def clear(self, stream=None):
        check(lib().sbf_clear(self._h, _stream_ptr(stream)), "sbf_clear")

    def words(self) -> np.ndarray:
        """Host copy of the filter words (uint64[W*N], W = words_per_shard); synchronizes."""
        out = np.empty(self.words_per_shard * self.num_shards, dtype=np.uint64)
        check(lib().sbf_copy_filter(self._h, out.ctypes.data, out.nbytes, SBF_HOST, None), "sbf_copy_filter")
        return out

    def words_device(self, stream=None):
        """Device copy of the filter words as an int64 tensor (asynchronous)."""
        torch = _torch()
        out = torch.empty(self.words_per_shard * self.num_shards, dtype=torch.int64, device="cuda")
        check(lib().sbf_copy_filter(self._h, out.data_ptr(), out.numel() * 8, SBF_DEVICE, _stream_ptr(stream)),
              "sbf_copy_filter")
        return out

    # ---- sequence-native calls ----------------------------------------------
    def insert_seq(self, seq, stream=None):
        """Insert every valid k-mer of an ASCII sequence: a CUDA uint8 tensor
        (asynchronous) or host bytes / str / numpy (synchronizes)."""
        if _is_device_tensor(seq):
            a = _device_bytes(seq, stream)
            check(lib().sbf_insert_seq(self._h, a.data_ptr(), a.numel(), SBF_DEVICE, _stream_ptr(stream)),
                  "sbf_insert_seq")
        else:
            a = _host_bytes(seq)
            check(lib().sbf_insert_seq(self._h, a.ctypes.data, a.size, SBF_HOST, _stream_ptr(stream)), "sbf_insert_seq")

    def query_seq(self, seq, out=None, stream=None):
        """One answer bit per k-mer start.  Device input gives an int64 CUDA
        tensor of bit words (asynchronous); host input a numpy uint64 array."""
        if _is_device_tensor(seq):
            torch = _torch()
            a = _device_bytes(seq, stream)
            nw = self.num_answer_words(a.numel())
            if out is None:
                out = torch.empty(max(nw, 1), dtype=torch.int64, device=a.device)
            else:
                _check_out(out, nw, torch.int64, a.device)
            if nw:
                check(lib().sbf_query_seq(self._h, a.data_ptr(), a.numel(), out.data_ptr(), SBF_DEVICE,
                                          _stream_ptr(stream)), "sbf_query_seq")
            return out[:nw]
        a = _host_bytes(seq)
        nw = self.num_answer_words(a.size)
        res = np.zeros(nw, dtype=np.uint64)
        if nw:
            check(lib().sbf_query_seq(self._h, a.ctypes.data, a.size, res.ctypes.data, SBF_HOST, _stream_ptr(stream)),
                  "sbf_query_seq")
        return res

    def read_answer_words(self, read_len: int) -> int:
        """uint32 answer words per read of sbf_query_reads: ceil((read_len - k + 1) / 32)."""
        nkr = read_len - self.k + 1
        return (nkr + 31) // 32 if nkr > 0 else 0

    def query_reads(self, reads, n_reads: int, read_len: int, stride: int = None, out=None, stream=None):
        """Per-read query of n_reads equal-length reads in a device uint8
        tensor (read r = bytes r*stride .. r*stride + read_len - 1; stride
        defaults to read_len + 1, reads joined by one separator).  Returns an
        int32 CUDA tensor (n_reads, ceil((read_len - k + 1) / 32)): k-mer
        32j + i of read r at bit i of [r, j] (asynchronous)."""
        torch = _torch()
        if stride is None:
            stride = read_len + 1
        if not _is_device_tensor(reads):
            raise TypeError("query_reads takes a CUDA uint8 tensor (device memory); "
                            "copy host reads to the device first")
        a = _device_bytes(reads, stream)
        need = (n_reads - 1) * stride + read_len if n_reads else 0
        if a.numel() < need:
            raise ValueError("reads holds %d bytes; %d reads of %d at stride %d need %d"
                             % (a.numel(), n_reads, read_len, stride, need))
        rch = self.read_answer_words(read_len)
        if out is None:
            out = torch.empty((n_reads, rch), dtype=torch.int32, device=a.device)
        else:
            _check_out(out, n_reads * rch, torch.int32, a.device)
        if n_reads and rch:
            check(lib().sbf_query_reads(self._h, a.data_ptr(), n_reads, read_len, stride, out.data_ptr(),
                                        _stream_ptr(stream)), "sbf_query_reads")
        return out

    # ---- packed (device-resident) calls ---------------------------------------
    def insert_packed(self, codes, valid, length: int, stream=None):
        check(lib().sbf_insert_packed(self._h, codes.data_ptr(), valid.data_ptr(), length, _stream_ptr(stream)),
              "sbf_insert_packed")

    def query_packed(self, codes, valid, length: int, out=None, stream=None):
        torch = _torch()
        nw = self.num_answer_words(length)
        if out is None:
            out = torch.empty(max(nw, 1), dtype=torch.int64, device=codes.device)
        else:
            _check_out(out, nw, torch.int64, codes.device)
        if nw:
            check(lib().sbf_query_packed(self._h, codes.data_ptr(), valid.data_ptr(), length, out.data_ptr(),
                                         _stream_ptr(stream)), "sbf_query_packed")
        return out[:nw]

    # ---- host pipeline and FASTA/FASTQ files -----------------------------------
    def set_staging(self, chunk_bases: int):
        """Chunk size (k-mer starts) of the host pipeline behind host-resident
        insert/query and the FASTX calls."""
        check(lib().sbf_set_staging(self._h, chunk_bases), "sbf_set_staging")

    def insert_fastx(self, path) -> dict:
        """Insert every valid k-mer of a FASTA/FASTQ file (plain or gzip);
        returns the reader/pipeline statistics."""
        st = _lib.SbfFastxStats()
        check(lib().sbf_insert_fastx(self._h, os.fsencode(path), ctypes.byref(st)), "sbf_insert_fastx")
        return _stats(st)

    def query_fastx(self, path, max_records: int | None = None):
        """Per-record (hits, kmers) uint64 arrays for a FASTA/FASTQ file, and
        the statistics.  Without max_records the file's records are counted
        first with the reader."""
        if max_records is None:
            max_records = count_fastx_records(path)
        hits = np.zeros(max(1, max_records), dtype=np.uint64)
        kmers = np.zeros_like(hits)
        st = _lib.SbfFastxStats()
        check(lib().sbf_query_fastx(self._h, os.fsencode(path), hits.ctypes.data, kmers.ctypes.data, max_records,
                                    ctypes.byref(st)), "sbf_query_fastx")
        n = min(max_records, st.records)
        return hits[:n], kmers[:n], _stats(st)

    # ---- false-positive probe ---------------------------------------------------
    def fpr_probe(self, n: int, seed: int) -> int:
        hits = ctypes.c_uint64()
        check(lib().sbf_fpr_probe(self._h, n, seed & (2**64 - 1), ctypes.byref(hits)), "sbf_fpr_probe")
        return hits.value

    def fpr_probe_device(self, n: int, seed: int, out, stream=None):
        check(lib().sbf_fpr_probe_device(self._h, n, seed & (2**64 - 1), out.data_ptr(), _stream_ptr(stream)),
              "sbf_fpr_probe_device")
        return out


def _stats(st) -> dict:
    return {"records": st.records, "bases": st.bases, "chunks": st.chunks,
            "parse_seconds": st.parse_seconds, "total_seconds": st.total_seconds}


def fastx_stream(path, piece: int = 1 << 24):
    """Iterate over (bytes of the normalized stream, record end offsets) pieces
    of a FASTA/FASTQ file as the library's reader produces them (host only):
    records joined by one 'N', line breaks and whitespace removed."""
    L = lib()
    r = ctypes.c_void_p()
    check(L.sbf_fastx_open(ctypes.byref(r), os.fsencode(path)), "sbf_fastx_open")
    try:
        buf = np.empty(piece, dtype=np.uint8)
        ends = np.empty(1 << 16, dtype=np.uint64)
        n, ne = ctypes.c_uint64(), ctypes.c_uint64()
        while True:
            check(L.sbf_fastx_read(r, buf.ctypes.data, buf.size, ctypes.byref(n), ends.ctypes.data, ends.size,
                                   ctypes.byref(ne)), "sbf_fastx_read")
            if n.value == 0 and ne.value == 0:
                return
            yield buf[:n.value].tobytes(), ends[:ne.value].copy()
    finally:
        L.sbf_fastx_close(r)


def count_fastx_records(path) -> int:
    """Number of records of a FASTA/FASTQ file (one pass of the reader)."""
    return int(sum(e.size for _, e in fastx_stream(path)))
