"""Helpers for the GPU parity tests: run the same seeded input through the
HIP library (through its C ABI) and through the CPU oracle."""
import numpy as np

from oracle import oracle as O


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def to_dev(arr):
    torch = torch_cuda()
    if isinstance(arr, (bytes, bytearray)):
        arr = np.frombuffer(bytes(arr), dtype=np.uint8)
    return torch.from_numpy(np.array(arr, dtype=np.uint8, copy=True)).cuda()


def gpu_filter(params, bits, kind="sbf"):
    import minimizer_sharded_bloom_amd as M
    k, m, s, H = params
    if kind == "protein":
        return M.SuperBloomFilter.protein(k, m, s, H, bits)
    if kind == "triplet":
        return M.SuperBloomFilter.triplet(k, m, s, H, bits)
    if kind == "bbf":
        return M.SuperBloomFilter.blocked(k, H, bits)
    if kind == "wide":
        return M.SuperBloomFilter.wide(k, m, s, H, bits)
    return M.SuperBloomFilter(k, m, s, H, bits)


def oracle_filter(params, bits, kind="sbf"):
    k, m, s, H = params
    if kind in ("protein", "triplet"):
        alpha = O.ALPHA_PROTEIN if kind == "protein" else O.ALPHA_TRIPLET
        return O.OracleFilter(k, m, s, H, bits, alpha=alpha)
    kinds = {"sbf": O.KIND_SBF, "bbf": O.KIND_BBF, "wide": O.KIND_WIDE}
    return O.OracleFilter(k, m, s, H, bits, kind=kinds[kind])


def dev_bits_to_np(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


def assert_words_equal(got: np.ndarray, want: np.ndarray, what: str):
    if got.shape != want.shape:
        raise AssertionError("%s: shape %s != %s" % (what, got.shape, want.shape))
    bad = np.flatnonzero(got != want)
    if bad.size:
        i = int(bad[0])
        raise AssertionError("%s: %d of %d words differ; first at %d: got %#018x want %#018x"
                             % (what, bad.size, got.size, i, int(got[i]), int(want[i])))
