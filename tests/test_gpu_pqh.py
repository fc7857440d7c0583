"""Per-query-head selection on the GPU against the oracle.

With select_per_query_head = 1 each query head ranks the blocks by its own
bound and attends the dense set and its own blocks; the pages of the union of
a KV head's sets are read once ("An Efficient Hybrid Sparse Attention with
CPU-GPU Parallelism for Long-Context Inference", Figures 4 and 5: heads are
counted and budgeted one query head at a time).  The call chain is
select_topk -> sparse_attend -> fuse_lse.  Each query head's selection is
compared with oracle.select_heads (bit-exact except ties inside the band), its
output with oracle.attend_heads over the GPU's selection, and MAW (fed by the
dense set alone, as per KV head) with the oracle's MAW step; the bars are the
harness's.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_sparse_top_score_amd._abi import SDError
from tests import harness
from tests.harness import log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _w(base, **over):
    import dataclasses
    return dataclasses.replace(base, **over)


def _run(w, seed, N=None, units=None, q_override=None):
    N = w.N if N is None else N
    gen = "cpu" if w.B * N * w.Hkv * w.d < 2**24 else "cuda"
    x = synth.single_step(w, seed, device=gen, N=N)
    K, V, q = x["K"].cuda(), x["V"].cuda(), x["q"].cuda()
    if q_override is not None:
        q = q_override(q)
    eng = harness.make_engine(w, N + 64, per_query_head=True)
    try:
        harness.prefill(eng, 0, K, V)
        seqs = list(range(w.B))
        gpu = harness.run_gpu_step(eng, 0, seqs, q)
        assert gpu["blk_idx"].shape[1] == w.Hq
        qb, Kb, Vb = synth.bits(q), synth.bits(K), synth.bits(V)
        G = w.G
        units = units or [(b, h) for b in range(w.B) for h in range(w.Hkv)]
        st = dict(ties=0, max_abs=0.0, max_rel=0.0, max_dlse=0.0, distinct=0, union=0, per_head=0)
        for b, h in units:
            S, ppm = w.block_size[h], w.budget_ppm[h]
            mn, mx = harness.summaries_by_head(eng, 0, b, w, N)[h]
            qg = np.ascontiguousarray(qb[b, h * G:(h + 1) * G])
            Kh, Vh = np.ascontiguousarray(Kb[b, :, h]), np.ascontiguousarray(Vb[b, :, h])
            ref = oracle.select_heads(qg, mn, mx, N, S, w.n_sink, w.window, ppm)
            Uh, _, _ = oracle.score(qg, mn, mx)
            got = []
            for j in range(G):
                row = h * G + j
                cnt = int(gpu["blk_cnt"][b, row])
                g_sel = gpu["blk_idx"][b, row, :cnt]
                st["ties"] += harness.adjudicate(g_sel, dict(sel=ref[j], U=Uh[j]), len(ref[j]))
                got.append(g_sel.astype(np.int32))
            sets = [tuple(s) for s in got]
            st["distinct"] += len(set(sets))
            st["union"] += len(set().union(*[set(s) for s in sets]))
            st["per_head"] += sum(len(s) for s in sets)
            O, lse = oracle.attend_heads(qg, Kh, Vh, N, S, w.n_sink, w.window, got)
            ma, mr, ml = harness.compare_outputs(gpu["o"][b, h * G:(h + 1) * G],
                                                 gpu["lse"][b, h * G:(h + 1) * G], O, lse)
            st["max_abs"], st["max_rel"] = max(st["max_abs"], ma), max(st["max_rel"], mr)
            st["max_dlse"] = max(st["max_dlse"], ml)
            a = oracle.dense_mass(qg, Kh, N, S, w.n_sink, w.window)
            want = oracle.maw_step(np.zeros(len(a)), a, N, S, w.n_sink, w.window, w.maw_decay)
            maw = harness.maw_by_head(eng, 0, b, w, N)[h]
            assert (np.abs(maw - want) <= harness.MAW_ABS + harness.MAW_REL * np.abs(want)).all()
        st["gpu"] = gpu
        log("  units %d: ties %d, max_abs %.2e, max_rel %.2e, max_dlse %.2e; distinct sets "
            "per KV head %.2f, union %d of %d per-head blocks"
            % (len(units), st["ties"], st["max_abs"], st["max_rel"], st["max_dlse"],
               st["distinct"] / len(units), st["union"], st["per_head"]))
        assert st["max_abs"] <= harness.ABS_TOL and st["max_rel"] <= harness.REL_TOL
        assert st["max_dlse"] <= harness.LSE_TOL
        return st
    finally:
        eng.close()


@pytest.mark.parametrize("seed", range(4))
def test_tiny(seed):
    log("case: per-query-head tiny seed=%d" % seed)
    st = _run(synth.tiny(), seed)
    assert st["distinct"] > 1  # the heads do choose differently


@pytest.mark.parametrize("N", [17, 69, 1007, 2049])
def test_tiny_ragged(N):
    log("case: per-query-head tiny N=%d" % N)
    _run(synth.tiny(), 3, N=N)


def test_llama32k_shape():
    w = _w(synth.llama32k(), B=2, N=6000)
    log("case: per-query-head llama32k B=2 N=6000")
    _run(w, 1)


def test_llama32k_full_sampled():
    log("case: per-query-head llama32k full size, 6 sampled units")
    _run(synth.llama32k(), 2, units=[(0, 0), (1, 3), (3, 7), (4, 2), (6, 5), (7, 7)])


def test_qwen128k_shape():
    """G = 7, per-KV-head budgets up to 20% and block sizes 16 or 64."""
    w = _w(synth.qwen128k(), B=2, N=20000)
    log("case: per-query-head qwen128k B=2 N=20000 S=%s ppm=%s" % (w.block_size, w.budget_ppm))
    _run(w, 5)


def test_qwen128k_full_sampled():
    w = synth.qwen128k()
    log("case: per-query-head qwen128k full size, 4 sampled units")
    _run(w, 6, units=[(0, 0), (1, 1), (2, 2), (3, 3)])


def test_equal_heads_match_the_group_selection():
    """When the G query rows are equal every head selects the group's set
    and the union is that set with every head on: the selections equal the
    per-KV-head call's bit for bit, and the outputs agree to the fp32
    rounding of the softmax sums (the union's bound G k can give the call
    more attention parts, which split the same pages differently)."""
    w = _w(synth.llama32k(), B=2, N=6000)
    log("case: per-query-head equal rows")
    G = w.G

    def same_rows(q):
        return q.view(w.B, w.Hkv, G, w.d)[:, :, :1].expand(-1, -1, G, -1).reshape(w.B, w.Hq, w.d).contiguous()

    a = _run(w, 4, q_override=same_rows)
    x = synth.single_step(w, 4, device="cpu", N=6000)
    K, V, q = x["K"].cuda(), x["V"].cuda(), same_rows(x["q"].cuda())
    eng = harness.make_engine(w, 6064)
    try:
        harness.prefill(eng, 0, K, V)
        b = harness.run_gpu_step(eng, 0, list(range(w.B)), q)
    finally:
        eng.close()
    for bi in range(w.B):
        for h in range(w.Hkv):
            for j in range(G):
                cnt = a["gpu"]["blk_cnt"][bi, h * G + j]
                assert cnt == b["blk_cnt"][bi, h]
                np.testing.assert_array_equal(a["gpu"]["blk_idx"][bi, h * G + j, :cnt],
                                              b["blk_idx"][bi, h, :cnt])
    np.testing.assert_allclose(a["gpu"]["o"], b["o"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(a["gpu"]["lse"], b["lse"], rtol=0, atol=1e-5)


def test_one_launch_step_refused():
    w = synth.tiny()
    eng = harness.make_engine(w, 1100, per_query_head=True)
    try:
        x = synth.single_step(w, 0, device="cpu", N=1000)
        harness.prefill(eng, 0, x["K"].cuda(), x["V"].cuda())
        bufs = eng.alloc_step(1)
        with pytest.raises(SDError) as e:
            eng.decode_step(0, [0], x["q"].cuda(), bufs["blk_idx"], bufs["blk_cnt"],
                            bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"])
        assert e.value.status == -4
    finally:
        eng.close()
