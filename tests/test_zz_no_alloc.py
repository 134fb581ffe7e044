"""The allocation-free insert, sbf_insert_seq_noalloc, through the C ABI: the
filter it builds equals the one sbf_insert_seq (SBF_DEVICE) builds from the
same inputs, word for word, over two calls in a row whose second input is
shorter than the first (its static staging keeps the first call's words past
the second's end); device free memory is unchanged by its calls; lengths over
its limit are refused before any device work."""
import ctypes

import numpy as np
import pytest

import minimizer_sharded_bloom_amd as M
from minimizer_sharded_bloom_amd import _lib
from minimizer_sharded_bloom_amd import synthetic as S
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

MAX_BASES = 1 << 26


def _create(lib, params, bits, alphabet=_lib.SBF_ALPHABET_DNA):
    h = ctypes.c_void_p()
    k, m, s, H = params
    if alphabet == _lib.SBF_ALPHABET_DNA:
        assert lib.sbf_create(ctypes.byref(h), k, m, s, H, bits) == _lib.SBF_OK
    else:
        assert lib.sbf_create_alphabet(ctypes.byref(h), alphabet, k, m, s, H, bits) == _lib.SBF_OK
    return h


def _words(lib, h):
    inf = _lib.SbfInfo()
    assert lib.sbf_info(h, ctypes.byref(inf)) == _lib.SBF_OK
    out = np.empty(inf.words_per_shard * inf.num_shards, dtype=np.uint64)
    assert lib.sbf_copy_filter(h, out.ctypes.data, out.nbytes, _lib.SBF_HOST, None) == _lib.SBF_OK
    return out


def _inputs():
    """A 3 Mbp genome-like text with 'N' runs, then a shorter, different one
    whose length is not a multiple of 16 or 32."""
    rng = np.random.default_rng(71)
    a = S.to_ascii(S.genome_with_repeats(3_000_000, seed_genome=12))
    a[rng.integers(0, a.size, 300)] = ord("N")
    b = S.to_ascii(S.genome_with_repeats(1_000_000, seed_genome=13))[:1_000_003].copy()
    b[rng.integers(0, b.size, 50)] = ord("n")
    return a, b


@pytest.mark.parametrize("params,alphabet", [((31, 16, 28, 4), _lib.SBF_ALPHABET_DNA),
                                              ((13, 7, 11, 5), _lib.SBF_ALPHABET_DNA),
                                              ((12, 6, 10, 4), _lib.SBF_ALPHABET_PROTEIN)])
def test_noalloc_insert_equals_insert_seq(params, alphabet):
    torch = G.torch_cuda()
    lib = M.lib()
    bits = 2**22
    a, b = _inputs()
    if alphabet == _lib.SBF_ALPHABET_PROTEIN:
        letters = np.frombuffer(b"ACDEFGHIKLMNPQRSTVWY", dtype=np.uint8)
        rng = np.random.default_rng(72)
        a = letters[rng.integers(0, 20, 2_000_000)].copy()
        b = letters[rng.integers(0, 20, 700_001)].copy()
        a[rng.integers(0, a.size, 100)] = ord("*")
    da, db = G.to_dev(a), G.to_dev(b)
    hn = _create(lib, params, bits, alphabet)
    hr = _create(lib, params, bits, alphabet)
    st = torch.cuda.current_stream()
    sp = st.cuda_stream
    try:
        for d in (da, db):
            # the reference first: its kernels' code is loaded and its staging
            # grown before free memory is read
            assert lib.sbf_insert_seq(hr, d.data_ptr(), d.numel(), _lib.SBF_DEVICE, sp) == _lib.SBF_OK
            torch.cuda.synchronize()
            free0 = torch.cuda.mem_get_info()[0]
            assert lib.sbf_insert_seq_noalloc(hn, d.data_ptr(), d.numel(), sp) == _lib.SBF_OK
            torch.cuda.synchronize()
            assert torch.cuda.mem_get_info()[0] == free0, "the allocation-free insert changed free device memory"
            G.assert_words_equal(_words(lib, hn), _words(lib, hr), "noalloc vs insert_seq %s" % (params,))
        # the second, shorter input alone into a fresh pair of filters
        assert lib.sbf_clear(hn, sp) == _lib.SBF_OK and lib.sbf_clear(hr, sp) == _lib.SBF_OK
        assert lib.sbf_insert_seq_noalloc(hn, db.data_ptr(), db.numel(), sp) == _lib.SBF_OK
        assert lib.sbf_insert_seq(hr, db.data_ptr(), db.numel(), _lib.SBF_DEVICE, sp) == _lib.SBF_OK
        torch.cuda.synchronize()
        w = _words(lib, hn)
        G.assert_words_equal(w, _words(lib, hr), "noalloc vs insert_seq, shorter input alone %s" % (params,))
        assert w.any()
    finally:
        lib.sbf_destroy(hn)
        lib.sbf_destroy(hr)


def test_noalloc_insert_matches_oracle_and_limits():
    """Against the oracle on its own, and the length limit: 2^26 bases are
    accepted, 2^26 + 1 refused with a message before any device work (the
    pointer is never read), a NULL sequence or handle refused, len < k a
    no-op."""
    torch = G.torch_cuda()
    lib = M.lib()
    params, bits = (31, 16, 28, 4), 2**24
    _, b = _inputs()
    h = _create(lib, params, bits)
    try:
        db = G.to_dev(b)
        sp = torch.cuda.current_stream().cuda_stream
        assert lib.sbf_insert_seq_noalloc(h, db.data_ptr(), db.numel(), sp) == _lib.SBF_OK
        torch.cuda.synchronize()
        o = G.oracle_filter(params, bits)
        o.insert_seq(b)
        G.assert_words_equal(_words(lib, h), o.words(), "noalloc vs oracle")
        assert lib.sbf_insert_seq_noalloc(h, db.data_ptr(), MAX_BASES + 1, sp) == _lib.SBF_EINVAL
        assert b"2^26" in lib.sbf_last_error()
        assert lib.sbf_insert_seq_noalloc(h, None, 100, sp) == _lib.SBF_EINVAL
        assert lib.sbf_insert_seq_noalloc(None, db.data_ptr(), 100, sp) == _lib.SBF_EINVAL
        assert lib.sbf_insert_seq_noalloc(h, None, 30, sp) == _lib.SBF_OK  # len < k
        big = torch.full((MAX_BASES,), ord("A"), dtype=torch.uint8, device="cuda")
        o2 = G.oracle_filter(params, bits)
        o2.insert_seq(b"A" * 64)  # poly-A: one k-mer, the same at every position
        assert lib.sbf_clear(h, sp) == _lib.SBF_OK
        assert lib.sbf_insert_seq_noalloc(h, big.data_ptr(), MAX_BASES, sp) == _lib.SBF_OK
        torch.cuda.synchronize()
        G.assert_words_equal(_words(lib, h), o2.words(), "noalloc at the length limit (poly-A)")
    finally:
        lib.sbf_destroy(h)
