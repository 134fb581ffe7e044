"""Error paths that need the device: a filter larger than the free device
memory (the allocation failure the C ABI reports as SBF_ENOMEM)."""
import ctypes

import numpy as np
import pytest

import minimizer_sharded_bloom_amd as M
from minimizer_sharded_bloom_amd import _lib
from tests import gpu_common as G
from tests import helpers as T

pytestmark = pytest.mark.gpu


def test_create_out_of_device_memory():
    """With less free device memory than a 2^40-bit (128 GiB) filter needs,
    sbf_create returns SBF_ENOMEM, leaves *out NULL and keeps no device memory;
    the device then serves a new filter as before."""
    torch = G.torch_cuda()
    lib = M.lib()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    bits = 1 << 40
    need = bits // 8
    free0, _ = torch.cuda.mem_get_info()
    hold = None
    if free0 >= need:
        # leave about half of what the filter needs free
        hold = torch.empty(free0 - need // 2, dtype=torch.uint8, device="cuda")
    free1, _ = torch.cuda.mem_get_info()
    assert free1 < need
    try:
        out = ctypes.c_void_p(None)
        rc = lib.sbf_create(ctypes.byref(out), 31, 16, 28, 4, bits)
        assert rc == _lib.SBF_ENOMEM, (rc, lib.sbf_last_error())
        assert out.value is None
        free2, _ = torch.cuda.mem_get_info()
        assert abs(free2 - free1) < (256 << 20), (free1, free2)
    finally:
        del hold
        torch.cuda.empty_cache()
    rng = np.random.default_rng(5)
    seq = T.random_dna(rng, 5000)
    g = G.gpu_filter((31, 16, 28, 4), 2**16)
    o = G.oracle_filter((31, 16, 28, 4), 2**16)
    g.insert_seq(G.to_dev(seq))
    o.insert_seq(seq)
    G.assert_words_equal(g.words(), o.words(), "filter after the failed create")
