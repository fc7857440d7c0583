"""The allocation-free one-launch step (sparse_decode_step_noalloc), whose
scratch lives in the library's static device array, against the existing
one-launch step (sparse_decode_step) on the same inputs: two contexts with the
same prefill, one driven by each entry point, on two calls in a row - all
sequences with their appends, then a smaller call (fewer sequences) - with
selection, O, lse and MAW compared after each call.  Both run the same
kernels in the same order, so the results must be bitwise equal (stricter
than the parity bars).  The second call's units are also checked against the
oracle.  Plus the refusal of a context whose scratch exceeds the array.
"""
import dataclasses

import numpy as np
import pytest
import torch

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


def _outputs(eng, bufs, seq_ids, w, N):
    out = {k: bufs[k][:len(seq_ids)].cpu().numpy() for k in ("blk_cnt", "o", "lse")}
    cnt = out["blk_cnt"]
    idx = bufs["blk_idx"][:len(seq_ids)].cpu().numpy()
    out["sel"] = [idx[i, g, :cnt[i, g]].copy() for i in range(len(seq_ids)) for g in range(w.Hkv)]
    out["maw"] = [harness.maw_by_head(eng, 0, s, w, N) for s in seq_ids]
    return out


def _assert_same(a, b):
    assert np.array_equal(a["blk_cnt"], b["blk_cnt"])
    for x, y in zip(a["sel"], b["sel"]):
        assert np.array_equal(x, y)
    assert np.array_equal(a["o"], b["o"])
    assert np.array_equal(a["lse"], b["lse"])
    for x, y in zip(a["maw"], b["maw"]):
        for p, q in zip(x, y):
            assert np.array_equal(p, q)


@pytest.mark.parametrize("shape", ["llama", "loop"])
def test_noalloc_step_equals_step_two_calls(shape):
    if shape == "llama":
        w = dataclasses.replace(synth.llama32k(), N=16384)
        x = synth.single_step(w, 21, device="cuda", N=w.N)
        K, V = x["K"], x["V"]
        q1, q2 = x["q"], synth.single_step(w, 22, device="cuda", N=64)["q"]
    else:  # MAW flags on (the full top-k)
        w = dataclasses.replace(synth.loop32(), B=4, N=8192, layers=1)
        dirs = synth.directions(w, 3, 0, 1, device="cuda")
        K, V, _ = synth.prefill_with_directions(w, 3, 0, w.N, dirs, device="cuda")
        q1 = synth.loop_query(w, 3, 0, 0, dirs, device="cuda")
        q2 = synth.loop_query(w, 3, 0, 1, dirs, device="cuda")
    log("case: no-alloc step vs step, %s shape B=%d N=%d" % (shape, w.B, w.N))
    engs = [harness.make_engine(w, w.N + 64), harness.make_engine(w, w.N + 64)]
    try:
        for e in engs:
            harness.prefill(e, 0, K, V)
        kn, vn = synth.step_kv(w, 5, 0, 0, device="cuda")
        kn = kn.view(w.B, w.Hkv, w.d).contiguous()
        vn = vn.view(w.B, w.Hkv, w.d).contiguous()
        # call 1: every sequence, one appended token each
        seqs = list(range(w.B))
        res = []
        for j, e in enumerate(engs):
            bufs = e.alloc_step(w.B)
            step = e.decode_step if j == 0 else e.decode_step_noalloc
            step(0, seqs, q1, bufs["blk_idx"], bufs["blk_cnt"], bufs["o_part"],
                 bufs["lse_part"], bufs["o"], bufs["lse"], k_new=kn, v_new=vn)
            e.sync()
            res.append(_outputs(e, bufs, seqs, w, w.N + 1))
        _assert_same(res[0], res[1])
        # call 2: a smaller input, fewer sequences (another token each)
        sub = [s for s in seqs if s % 3 != 0][:3]
        kn2, vn2 = synth.step_kv(w, 5, 0, 1, device="cuda")
        kn2 = kn2.view(w.B, w.Hkv, w.d)[sub].contiguous()
        vn2 = vn2.view(w.B, w.Hkv, w.d)[sub].contiguous()
        q2s = q2[sub].contiguous()
        res, gpus = [], []
        for j, e in enumerate(engs):
            bufs = e.alloc_step(len(sub))
            step = e.decode_step if j == 0 else e.decode_step_noalloc
            step(0, sub, q2s, bufs["blk_idx"], bufs["blk_cnt"], bufs["o_part"],
                 bufs["lse_part"], bufs["o"], bufs["lse"], k_new=kn2, v_new=vn2)
            e.sync()
            res.append(_outputs(e, bufs, sub, w, w.N + 2))
            gpus.append({k: v.cpu().numpy() for k, v in bufs.items()})
        _assert_same(res[0], res[1])
        # the smaller call against the oracle, every unit (MAW from zero,
        # through both steps, when the flag is on)
        Kb, Vb = synth.bits(K), synth.bits(V)
        k1, v1 = synth.bits(kn), synth.bits(vn)
        k2, v2 = synth.bits(kn2), synth.bits(vn2)
        K_bits, V_bits = {}, {}
        for i, s in enumerate(sub):
            K_bits[s] = np.concatenate([Kb[s], k1[s][None], k2[i][None]], 0)
            V_bits[s] = np.concatenate([Vb[s], v1[s][None], v2[i][None]], 0)
        st = harness.check_units(w, engs[1], 0, sub, synth.bits(q2s), K_bits, V_bits,
                                 {s: w.N + 2 for s in sub}, gpus[1], check_summ=True)
        harness.assert_parity(st)
    finally:
        for e in engs:
            e.close()


def test_noalloc_refuses_scratch_beyond_the_array():
    """A context whose step scratch exceeds the static array is refused with
    SD_EUNSUPPORTED before anything is enqueued; the other entry point still
    runs."""
    w = dataclasses.replace(synth.tiny(), B=64, Hq=8, Hkv=8, N=64, block_size=[16] * 8,
                            budget_ppm=[20000] * 8)
    log("case: no-alloc refusal")
    eng = harness.make_engine(w, 131072, max_seqs=64, extra_pages=-(64 * 8192) + 64 * 8)
    try:
        K = torch.zeros(64, 64, w.Hkv, w.d, dtype=torch.bfloat16, device="cuda")
        harness.prefill(eng, 0, K, K)
        q = torch.zeros(64, w.Hq, w.d, dtype=torch.bfloat16, device="cuda")
        bufs = eng.alloc_step(64)
        st = eng.decode_step_noalloc(0, list(range(64)), q, bufs["blk_idx"], bufs["blk_cnt"],
                                     bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"],
                                     check=False)
        assert st == -4, eng.error()
        assert "static array" in eng.error()
        eng.decode_step(0, list(range(64)), q, bufs["blk_idx"], bufs["blk_cnt"], bufs["o_part"],
                        bufs["lse_part"], bufs["o"], bufs["lse"])
        eng.sync()
    finally:
        eng.close()
