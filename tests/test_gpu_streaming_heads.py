"""Streaming heads: KV heads with budget 0 select nothing and attend to their
sinks and recent window only ([FLX] streaming heads).  Their units skip the
score tiles; in the one-launch step the fusion then decays their MAW.  Mixed
and all-streaming configurations are checked against the oracle, both call
forms, MAW included."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests import harness
from tests.harness import log

pytestmark = pytest.mark.gpu

MIXED = [0, 50000, 0, 50000, 0, 50000, 0, 50000]


def _w(base, **over):
    return dataclasses.replace(base, **over)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("fused", [False, True])
def test_mixed_streaming_heads(fused):
    w = _w(synth.llama32k(), B=2, N=6000, budget_ppm=MIXED)
    log("case: mixed streaming heads fused=%s" % fused)
    st = harness.run_single_step(w, 3, fused=fused)
    harness.assert_parity(st)
    cnt = st["gpu"]["blk_cnt"]
    assert np.all(cnt[:, 0::2] == 0) and np.all(cnt[:, 1::2] > 0)


def test_mixed_streaming_heads_fused_equals_separate():
    w = _w(synth.llama32k(), B=2, N=6000, budget_ppm=MIXED)
    log("case: mixed streaming heads, fused vs separate")
    a = harness.run_single_step(w, 5, fused=False)
    b = harness.run_single_step(w, 5, fused=True)
    for k in ("blk_idx", "blk_cnt"):
        assert np.array_equal(a["gpu"][k], b["gpu"][k]), k
    # the selecting heads' pages in key order against ascending order: fp32
    # rounding of the softmax sums; the streaming heads' outputs are bitwise equal
    np.testing.assert_allclose(b["gpu"]["o"], a["gpu"]["o"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(b["gpu"]["lse"], a["gpu"]["lse"], rtol=0, atol=1e-5)
    G = w.Hq // w.Hkv
    for g in range(0, w.Hkv, 2):
        sl = slice(g * G, (g + 1) * G)
        assert np.array_equal(a["gpu"]["o"][:, sl], b["gpu"]["o"][:, sl])
        assert np.array_equal(a["gpu"]["lse"][:, sl], b["gpu"]["lse"][:, sl])


@pytest.mark.parametrize("fused", [False, True])
def test_all_heads_streaming(fused):
    w = _w(synth.tiny(), N=3000, budget_ppm=[0])
    log("case: all heads streaming fused=%s" % fused)
    st = harness.run_single_step(w, 4, fused=fused)
    harness.assert_parity(st)
    assert st["gpu"]["blk_cnt"].max() == 0


def test_streaming_heads_maw_lockstep_fused():
    """Several one-launch steps (with their appends) and MAW flags on: the
    streaming heads' MAW decays in the fusion, the others' in the score
    tiles; MAW tables and outputs follow the oracle step by step."""
    w = _w(synth.loop32(), B=2, N=3000, layers=1, steps=6, budget_ppm=MIXED)
    log("case: streaming heads, MAW lockstep, one-launch step")
    eng = harness.make_engine(w, w.N + 64, layers=1)
    try:
        dirs = synth.directions(w, 0, 0, 1, device="cuda")
        K, V, _ = synth.prefill_with_directions(w, 0, 0, w.N - 1, dirs, device="cuda")
        harness.prefill(eng, 0, K, V)
        Kb, Vb = synth.bits(K), synth.bits(V)
        K_bits = {b: Kb[b] for b in range(w.B)}
        V_bits = {b: Vb[b] for b in range(w.B)}
        maw_state = {}
        N = w.N - 1
        for step in range(w.steps):
            N += 1
            kn, vn = synth.step_kv(w, 0, 0, step, device="cuda")
            q = synth.loop_query(w, 0, 0, step, dirs, device="cuda")
            bufs = eng.alloc_step(w.B)
            eng.decode_step(0, list(range(w.B)), q, bufs["blk_idx"], bufs["blk_cnt"],
                            bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"],
                            k_new=kn.view(w.B, w.Hkv, w.d).contiguous(),
                            v_new=vn.view(w.B, w.Hkv, w.d).contiguous())
            eng.sync()
            gpu = {k: v.cpu().numpy() for k, v in bufs.items()}
            knb, vnb = synth.bits(kn), synth.bits(vn)
            for b in range(w.B):
                K_bits[b] = np.concatenate([K_bits[b], knb[b]], 0)
                V_bits[b] = np.concatenate([V_bits[b], vnb[b]], 0)
            st = harness.check_units(w, eng, 0, list(range(w.B)), synth.bits(q), K_bits, V_bits,
                                     {b: N for b in range(w.B)}, gpu, maw_state=maw_state,
                                     check_summ=(step == 0))
            log("  step %d N=%d" % (step, N))
            harness.assert_parity(st)
            assert np.all(gpu["blk_cnt"][:, 0::2] == 0)
    finally:
        eng.close()
