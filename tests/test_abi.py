"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/sbf.h declares, and rejects bad arguments before it
touches the device."""
import ctypes
import os
import subprocess

import pytest

from minimizer_sharded_bloom_amd import _lib

LIB = _lib.LIB_PATH


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libsbf.so is not built; run __graft_entry__.build()")
    return _lib.load()


def test_header_declares_the_boundary():
    names = _lib.header_symbols()
    for want in ("sbf_create", "sbf_insert_seq", "sbf_query_seq", "sbf_fpr_probe", "sbf_destroy",
                 "sbf_insert_packed", "sbf_query_packed", "sbf_pack", "sbf_create_bbf"):
        assert want in names
    assert set(names) == set(_lib.SIGNATURES)


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _lib.header_symbols():
        assert name in exported, name
        assert getattr(lib, name) is not None


@pytest.mark.parametrize("k,m,s,H,bits", [(0, 1, 1, 1, 256), (33, 16, 28, 4, 256), (31, 0, 28, 4, 256),
                                          (31, 32, 28, 4, 256), (31, 16, 0, 4, 256), (31, 16, 32, 4, 256),
                                          (31, 16, 28, 0, 256), (31, 16, 28, 65, 256), (31, 16, 28, 4, 0),
                                          (31, 16, 28, 4, 2**40 + 1)])
def test_create_rejects_bad_parameters(lib, k, m, s, H, bits):
    h = ctypes.c_void_p(0)
    rc = lib.sbf_create(ctypes.byref(h), k, m, s, H, bits)
    assert rc == _lib.SBF_EINVAL
    assert h.value is None
    assert lib.sbf_last_error()


def test_bbf_rejects_bad_parameters(lib):
    h = ctypes.c_void_p(0)
    assert lib.sbf_create_bbf(ctypes.byref(h), 33, 4, 256) == _lib.SBF_EINVAL
    assert lib.sbf_create_bbf(ctypes.byref(h), 31, 0, 256) == _lib.SBF_EINVAL
    assert lib.sbf_create_bbf(None, 31, 4, 256) == _lib.SBF_EINVAL


def test_null_handles(lib):
    assert lib.sbf_destroy(None) == _lib.SBF_OK
    assert lib.sbf_clear(None, None) == _lib.SBF_EINVAL
    assert lib.sbf_insert_seq(None, None, 10, _lib.SBF_HOST, None) == _lib.SBF_EINVAL
    assert lib.sbf_query_seq(None, None, 10, None, _lib.SBF_HOST, None) == _lib.SBF_EINVAL
    assert lib.sbf_insert_packed(None, None, None, 10, None) == _lib.SBF_EINVAL
    assert lib.sbf_query_packed(None, None, None, 10, None, None) == _lib.SBF_EINVAL
    assert lib.sbf_query_reads(None, None, 4, 150, 151, None, None) == _lib.SBF_EINVAL
    hits = ctypes.c_uint64()
    assert lib.sbf_fpr_probe(None, 1, 1, ctypes.byref(hits)) == _lib.SBF_EINVAL
    assert lib.sbf_info(None, None) == _lib.SBF_EINVAL
    assert lib.sbf_copy_filter(None, None, 0, _lib.SBF_HOST, None) == _lib.SBF_EINVAL
    assert lib.sbf_filter_device_ptr(None) is None
    assert lib.sbf_pack(None, 0, None, None, None) == _lib.SBF_OK  # empty input is a no-op
    assert lib.sbf_pack(None, 5, None, None, None) == _lib.SBF_EINVAL


def test_strerror(lib):
    for code in (_lib.SBF_OK, _lib.SBF_EINVAL, _lib.SBF_EUNSUPPORTED, _lib.SBF_ENOMEM, _lib.SBF_EDEVICE, 7):
        assert lib.sbf_strerror(code)


def test_packed_words(lib):
    cw, vw = ctypes.c_uint64(), ctypes.c_uint64()
    for n, c, v in [(0, 0, 0), (1, 1, 1), (16, 1, 1), (17, 2, 1), (32, 2, 1), (33, 3, 2), (10**10, 625000000, 312500000)]:
        lib.sbf_packed_words(n, ctypes.byref(cw), ctypes.byref(vw))
        assert (cw.value, vw.value) == (c, v)


def test_wide_rejects_bad_parameters(lib):
    h = ctypes.c_void_p(0)
    assert lib.sbf_create_wide(ctypes.byref(h), 31, 32, 28, 4, 512) == _lib.SBF_EINVAL
    assert lib.sbf_create_wide(ctypes.byref(h), 31, 16, 0, 4, 512) == _lib.SBF_EINVAL
    assert lib.sbf_create_wide(ctypes.byref(h), 31, 16, 28, 65, 512) == _lib.SBF_EINVAL
    assert lib.sbf_create_wide(ctypes.byref(h), 31, 16, 28, 4, 0) == _lib.SBF_EINVAL
    assert h.value is None


def test_alphabet_rejects_bad_parameters(lib):
    """Protein k <= 12 and triplet k <= 10 (k symbols of 5 or 6 bits in 64);
    unknown alphabets; the usual m, s, H, bits ranges.  Checked before any
    device use."""
    h = ctypes.c_void_p(0)
    P, TR = _lib.SBF_ALPHABET_PROTEIN, _lib.SBF_ALPHABET_TRIPLET
    for args in [(P, 13, 6, 10, 4, 4096), (P, 0, 1, 1, 4, 4096), (TR, 11, 5, 8, 4, 4096), (3, 5, 3, 4, 4, 4096),
                 (P, 12, 13, 10, 4, 4096), (P, 12, 6, 0, 4, 4096), (TR, 10, 5, 8, 65, 4096), (TR, 10, 5, 8, 4, 0)]:
        assert lib.sbf_create_alphabet(ctypes.byref(h), *args) == _lib.SBF_EINVAL, args
    assert h.value is None


def test_membench_rejects_bad_sizes(lib):
    """Refused before any device use: NULL tables, shard counts that are not
    powers of two."""
    assert lib.sbf_membench_shard_ors(None, 1024, 10, 1, None) == _lib.SBF_EINVAL
    assert lib.sbf_membench_shard_ors(8, 1000, 10, 1, None) == _lib.SBF_EINVAL
    assert lib.sbf_membench_shard_reads(8, 0, 10, 1, 8, None) == _lib.SBF_EINVAL
    assert lib.sbf_membench_shard_reads(8, 1024, 10, 1, None, None) == _lib.SBF_EINVAL
    assert lib.sbf_membench_valu(0, 10, None, None) == _lib.SBF_EINVAL
    assert lib.sbf_membench_valu(2, 10, 8, None) == _lib.SBF_EINVAL
    assert lib.sbf_membench_valu(1, 0, 8, None) == _lib.SBF_EINVAL
    assert lib.sbf_membench_valu(1, (1 << 32) + 1, 8, None) == _lib.SBF_EINVAL
