"""The hot path captured in a HIP graph (bench.py replays its step this way):
the library's launches for clear, pack, insert, the query of a device
sequence and the FPR probe allocate nothing and record no memset, so a
captured step replays to the same filter words, answer bits and probe count
as the launched step.  Each replay follows other work launched eagerly and a
synchronization, and every replay is checked ("cuSBF: A Minimizer-Aware Bloom
Filter for Genomic Sequence Data on Modern GPUs", Algorithms 1 and 2, §V-D)."""
import numpy as np
import pytest

import minimizer_sharded_bloom_amd as M
from tests import gpu_common as G
from tests import helpers as T

pytestmark = pytest.mark.gpu


def _text(rng, n):
    b = bytearray(T.random_dna(rng, n))
    for p in rng.integers(0, n, n // 500):
        b[p] = ord("N")
    return bytes(b)


@pytest.mark.parametrize("alphabet", ["dna", "protein"])
def test_graph_replay_matches_launched_step(alphabet):
    torch = G.torch_cuda()
    L = M.lib()
    rng = np.random.default_rng(91)
    if alphabet == "dna":
        f = M.SuperBloomFilter(31, 16, 28, 4, 2**22)
        ref, qry = _text(rng, 300_000), _text(rng, 200_000)
    else:
        f = M.SuperBloomFilter.protein(12, 6, 10, 4, 2**22)
        letters = np.frombuffer(b"ACDEFGHIKLMNPQRSTVWY", dtype=np.uint8)
        ref = letters[rng.integers(0, letters.size, 100_000)].tobytes()
        qry = letters[rng.integers(0, letters.size, 80_000)].tobytes()
    g_ref, g_qry = G.to_dev(ref), G.to_dev(qry)
    assert g_qry.data_ptr() % 16 == 0
    LG, LR = g_ref.numel(), g_qry.numel()
    gcw, gvw = M.packed_words(LG)
    codes = torch.empty(max(gcw, 1), dtype=torch.int32, device="cuda")
    valid = torch.empty(max(gvw, 1), dtype=torch.int32, device="cuda")
    out = torch.empty(f.num_answer_words(LR), dtype=torch.int64, device="cuda")
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")

    def step(st):
        sp = st.cuda_stream
        M.check(L.sbf_clear(f.handle, sp), "clear")
        if alphabet == "dna":
            M.check(L.sbf_pack(g_ref.data_ptr(), LG, codes.data_ptr(), valid.data_ptr(), sp), "pack")
            M.check(L.sbf_insert_packed(f.handle, codes.data_ptr(), valid.data_ptr(), LG, sp), "insert")
        else:
            M.check(L.sbf_insert_seq(f.handle, g_ref.data_ptr(), LG, M.SBF_DEVICE, sp), "insert")
        M.check(L.sbf_query_seq(f.handle, g_qry.data_ptr(), LR, out.data_ptr(), M.SBF_DEVICE, sp), "query")
        M.check(L.sbf_fpr_probe_device(f.handle, 200_000, 0x5EED, hits.data_ptr(), sp), "probe")

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want_words, want_out, want_hits = f.words(), out.cpu().numpy().copy(), int(hits.item())
    assert want_out.any() and want_hits >= 0

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    other = M.SuperBloomFilter(31, 16, 28, 4, 2**16)
    for r in range(3):
        # eager work between replays: another filter's launches, scribbles
        # over the outputs, then a synchronization
        other.insert_seq(G.to_dev(_text(rng, 10_000)))
        out.fill_(-1)
        hits.fill_(12345)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        G.assert_words_equal(f.words(), want_words, "replay %d words" % r)
        G.assert_words_equal(out.cpu().numpy(), want_out, "replay %d answers" % r)
        assert int(hits.item()) == want_hits, r
