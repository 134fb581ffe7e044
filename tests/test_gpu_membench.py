"""The matched-ceiling microbenchmarks stay inside the table they are given
and do what they say: every OR lands in the table (guard words around it stay
zero), the four words of an updated shard change together, and bad sizes are
refused before any launch.  The VALU issue-rate kernels run and leave their
sink word alone."""
import numpy as np
import pytest

import minimizer_sharded_bloom_amd as M
from minimizer_sharded_bloom_amd import _lib
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def test_membench_stays_in_bounds():
    torch = G.torch_cuda()
    L = M.lib()
    nsh, guard = 1 << 10, 4096
    buf = torch.zeros(4 * nsh + 2 * guard, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int64, device="cuda")
    table = buf.data_ptr() + 8 * guard
    assert L.sbf_membench_shard_ors(table, nsh, 5000, 7, None) == _lib.SBF_OK
    assert L.sbf_membench_shard_reads(table, nsh, 5000, 7, sink.data_ptr(), None) == _lib.SBF_OK
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint64)
    assert not h[:guard].any() and not h[guard + 4 * nsh:].any()
    sh = h[guard:guard + 4 * nsh].reshape(nsh, 4)
    touched = sh.any(axis=1)
    assert (sh[touched] != 0).all()          # all four words of an updated shard
    assert 0.9 < touched.mean() <= 1.0       # 5000 random shards cover ~99% of 1024
    assert L.sbf_membench_shard_ors(table, 1000, 10, 7, None) == _lib.SBF_EINVAL
    assert L.sbf_membench_shard_reads(table, 0, 10, 7, sink.data_ptr(), None) == _lib.SBF_EINVAL
    assert L.sbf_membench_shard_reads(table, nsh, 10, 7, None, None) == _lib.SBF_EINVAL


def test_valu_rate_kernels_run():
    torch = G.torch_cuda()
    L = M.lib()
    sink = torch.zeros(1, dtype=torch.int64, device="cuda")
    for kind in (0, 1):
        assert L.sbf_membench_valu(kind, 16, sink.data_ptr(), None) == _lib.SBF_OK
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_update_forms_stay_in_bounds():
    """sbf_membench_shard_rmw in every form stays inside its table; the
    device-scope atomic form sets the same words as sbf_membench_shard_ors
    for the same seed, the other whole-table forms a subset of them; the
    partitioned forms touch every eighth of the table; bad modes and sizes
    are refused."""
    torch = G.torch_cuda()
    L = M.lib()
    nsh, guard, n = 1 << 10, 4096, 3000
    ref = torch.zeros(4 * nsh, dtype=torch.int64, device="cuda")
    assert L.sbf_membench_shard_ors(ref.data_ptr(), nsh, n, 11, None) == _lib.SBF_OK
    torch.cuda.synchronize()
    want = ref.cpu().numpy().view(np.uint64)
    for mode in (0, 1, 2, 4, 5, 6):
        buf = torch.zeros(4 * nsh + 2 * guard, dtype=torch.int64, device="cuda")
        table = buf.data_ptr() + 8 * guard
        assert L.sbf_membench_shard_rmw(table, nsh, n, 11, mode, None) == _lib.SBF_OK
        torch.cuda.synchronize()
        h = buf.cpu().numpy().view(np.uint64)
        assert not h[:guard].any() and not h[guard + 4 * nsh:].any(), mode
        sh = h[guard:guard + 4 * nsh]
        if mode == 0:
            assert (sh == want).all(), mode
        elif mode in (1, 2):
            # workgroup scope is atomic only within a workgroup, and a plain
            # update not at all: bits may be lost, never invented
            assert not (sh & ~want).any(), mode
            assert sh.any(), mode
        else:
            eighths = sh.reshape(8, -1).any(axis=1)
            assert eighths.all(), mode
    table = ref.data_ptr()
    for bad in (3, 7, 8, 16):
        assert L.sbf_membench_shard_rmw(table, nsh, 10, 1, bad, None) == _lib.SBF_EINVAL
    assert L.sbf_membench_shard_rmw(table, 4, 10, 1, 4, None) == _lib.SBF_EINVAL
    assert L.sbf_membench_shard_rmw(table, 1000, 10, 1, 0, None) == _lib.SBF_EINVAL
