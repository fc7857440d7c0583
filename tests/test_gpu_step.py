"""GPU parity of the one-launch decode step (the benchmarked path) against the
CPU oracle, including the full-size multi-step workloads on sampled units.

The one-launch step runs its own top-k (score tiles publish candidate lists
that the last tile ranks) where the separate calls run the full top-k, so it
is checked against the oracle directly, at the same bars as the separate calls
(tests/harness.py).
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests import harness
from tests.harness import log

pytestmark = pytest.mark.gpu


def _w(base, **over):
    return dataclasses.replace(base, **over)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _check(st):
    log("  ties=%d max|dO|=%.3g max rel=%.3g max|dlse|=%.3g" % (
        st["ties"], st["max_abs"], st["max_rel"], st["max_dlse"]))
    harness.assert_parity(st)


@pytest.mark.parametrize("seed", range(4))
def test_fused_tiny(seed):
    log("case: fused tiny seed %d" % seed)
    _check(harness.run_single_step(synth.tiny(), seed, fused=True))


@pytest.mark.parametrize("N", [1, 17, 100, 1007, 2049, 4111])
def test_fused_ragged(N):
    log("case: fused tiny N=%d" % N)
    _check(harness.run_single_step(_w(synth.tiny(), N=N), 3, fused=True))


@pytest.mark.parametrize("G,Hkv,d,S", [(7, 4, 128, 16), (8, 2, 64, 64), (1, 2, 128, 32)])
def test_fused_group_sizes(G, Hkv, d, S):
    w = _w(synth.tiny(), Hq=G * Hkv, Hkv=Hkv, d=d, N=9000, block_size=[S] * Hkv,
           budget_ppm=[40000] * Hkv)
    log("case: fused G=%d Hkv=%d d=%d S=%d" % (G, Hkv, d, S))
    _check(harness.run_single_step(w, 8, fused=True))


@pytest.mark.parametrize("B,S,pct", [(1, 16, 2), (8, 32, 5), (64, 16, 10), (32, 64, 10),
                                     (64, 32, 10)])
def test_fused_sweep_points(B, S, pct):
    log("case: fused sweep B=%d S=%d budget=%d%%" % (B, S, pct))
    _check(harness.run_single_step(synth.sweep(B, S, pct), 22, fused=True))


@pytest.mark.parametrize("B", [1, 8, 32, 64])
@pytest.mark.parametrize("S", [16, 32, 64])
@pytest.mark.parametrize("pct", [2, 5, 10])
def test_fused_sweep_grid_sampled(B, S, pct):
    """Every point of the batch x block size x budget sweep in the one-launch
    form, four sampled sequences (all when fewer) against the oracle."""
    log("case: fused sweep grid B=%d S=%d budget=%d%%" % (B, S, pct))
    units = sorted({(b, 0) for b in (0, B // 3, (2 * B) // 3, B - 1)})
    _check(harness.run_single_step(synth.sweep(B, S, pct), 23, fused=True, units=units))


def test_fused_llama32k_full():
    """The benchmarked workload at full size, every unit against the oracle."""
    log("case: fused llama32k full")
    st = harness.run_single_step(synth.llama32k(), 1, fused=True, shuffle_seed=12345)
    _check(st)
    assert len(st["units"]) == 64


def test_fused_qwen128k_full():
    w = synth.qwen128k(1)
    log("case: fused qwen128k S=%s ppm=%s" % (w.block_size, w.budget_ppm))
    _check(harness.run_single_step(w, 2, fused=True))


@pytest.mark.parametrize("n_eq,ppm", [(161, 50_000), (100, 175_000)],
                         ids=["k26_of_161_equal", "k90_of_100_equal"])
def test_fused_equal_scores_tie_order(n_eq, ppm):
    """Blocks with bitwise equal summaries have equal scores: the one-launch
    top-k must take them by index, as the oracle does.  With k = 26 the
    equal blocks fill the 64-key lists; with k = 90 the k-th place falls
    among 100 equal blocks, inside the 128-key lists of the fast top-k."""
    w = _w(synth.llama32k(), B=1, Hq=8, Hkv=2, N=16384, budget_ppm=[ppm, ppm])
    log("case: fused equal-score ties, %d equal blocks, ppm %d" % (n_eq, ppm))
    x = synth.single_step(w, 4, N=w.N)
    K, V, q = x["K"], x["V"], x["q"]
    # block 40's keys scaled x4 (a bound well above the rest), copied over
    # blocks 41..40 + n_eq - 1 of KV head 0: n_eq equal top scores
    S = w.block_size[0]
    src = (K[0, 40 * S:41 * S, 0].float() * 4.0).to(torch.bfloat16)
    for blk in range(40, 40 + n_eq):
        K[0, blk * S:(blk + 1) * S, 0] = src
    eng = harness.make_engine(w, w.N + 64)
    try:
        harness.prefill(eng, 0, K.cuda(), V.cuda())
        gpu = harness.run_gpu_step(eng, 0, [0], q.cuda(), fused=True)
        Kb, Vb = synth.bits(K), synth.bits(V)
        st = harness.check_units(w, eng, 0, [0], synth.bits(q), {0: Kb[0]}, {0: Vb[0]},
                                 {0: w.N}, gpu)
        _check(st)
        assert st["ties"] == 0
    finally:
        eng.close()


def test_qwen128k_drift_multistep_fused():
    """qwen128k at full size: four planted sets, one per 64-step epoch; one
    decode step (with its one-token append) in each epoch, every unit against
    the oracle."""
    w = synth.qwen128k(0)
    log("case: qwen128k drift S=%s ppm=%s" % (w.block_size, w.budget_ppm))
    seed, N0 = 5, w.N - 4
    qe, dirs = synth.drift_setup(w, seed, 4, device="cuda")
    K, V, _ = synth.prefill_with_directions(w, seed, 0, N0, dirs, device="cuda")
    eng = harness.make_engine(w, w.N + 64)
    try:
        harness.prefill(eng, 0, K, V)
        Kb, Vb = synth.bits(K), synth.bits(V)
        del K, V
        K_bits = {b: Kb[b] for b in range(w.B)}
        V_bits = {b: Vb[b] for b in range(w.B)}
        N = N0
        for e in range(4):
            step = 64 * e
            kn, vn = synth.step_kv(w, seed, 0, step, device="cuda")
            q = synth.drift_query(w, seed, step, qe, device="cuda")
            bufs = eng.alloc_step(w.B)
            eng.decode_step(0, list(range(w.B)), q, bufs["blk_idx"], bufs["blk_cnt"],
                            bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"],
                            k_new=kn.view(w.B, w.Hkv, w.d).contiguous(),
                            v_new=vn.view(w.B, w.Hkv, w.d).contiguous())
            eng.sync()
            gpu = {k: v.cpu().numpy() for k, v in bufs.items()}
            N += 1
            knb, vnb = synth.bits(kn), synth.bits(vn)
            for b in range(w.B):
                K_bits[b] = np.concatenate([K_bits[b], knb[b]], 0)
                V_bits[b] = np.concatenate([V_bits[b], vnb[b]], 0)
            log("  epoch %d N=%d" % (e, N))
            st = harness.check_units(w, eng, 0, list(range(w.B)), synth.bits(q), K_bits,
                                     V_bits, {b: N for b in range(w.B)}, gpu,
                                     check_summ=(e == 0))
            _check(st)
    finally:
        eng.close()


def test_qwen128k_drift_consecutive_steps_across_epoch():
    """qwen128k at full size: eight consecutive decode steps (60 .. 67, each
    with its one-token append) that cross the boundary between the first and
    the second planted set at step 64; four sampled units against the oracle
    at every step."""
    w = synth.qwen128k(0)
    log("case: qwen128k drift, consecutive steps 60..67")
    seed, N0 = 6, w.N - 8
    qe, dirs = synth.drift_setup(w, seed, 4, device="cuda")
    K, V, _ = synth.prefill_with_directions(w, seed, 0, N0, dirs, device="cuda")
    units = [(0, 0), (1, 1), (2, 2), (3, 3)]
    eng = harness.make_engine(w, w.N + 64)
    try:
        harness.prefill(eng, 0, K, V)
        Kb, Vb = synth.bits(K), synth.bits(V)
        del K, V
        K_bits = {b: Kb[b] for b in range(w.B)}
        V_bits = {b: Vb[b] for b in range(w.B)}
        N = N0
        bufs = eng.alloc_step(w.B)
        for step in range(60, 68):
            kn, vn = synth.step_kv(w, seed, 0, step, device="cuda")
            q = synth.drift_query(w, seed, step, qe, device="cuda")
            eng.decode_step(0, list(range(w.B)), q, bufs["blk_idx"], bufs["blk_cnt"],
                            bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"],
                            k_new=kn.view(w.B, w.Hkv, w.d).contiguous(),
                            v_new=vn.view(w.B, w.Hkv, w.d).contiguous())
            eng.sync()
            gpu = {k: v.cpu().numpy() for k, v in bufs.items()}
            N += 1
            knb, vnb = synth.bits(kn), synth.bits(vn)
            for b in range(w.B):
                K_bits[b] = np.concatenate([K_bits[b], knb[b]], 0)
                V_bits[b] = np.concatenate([V_bits[b], vnb[b]], 0)
            log("  step %d (epoch %d) N=%d" % (step, step // 64, N))
            st = harness.check_units(w, eng, 0, list(range(w.B)), synth.bits(q), K_bits,
                                     V_bits, {b: N for b in range(w.B)}, gpu, units=units,
                                     check_summ=(step == 60))
            _check(st)
    finally:
        eng.close()


def test_loop32_full_size_sampled():
    """The loop workload at its per-layer size (B=16, N=65536, MAW beta=1),
    two layer instances, three decode steps each with the one-launch step;
    sampled units are followed in lockstep by the oracle, MAW included."""
    w = _w(synth.loop32(), layers=2, steps=3)
    log("case: loop32 full size, sampled units")
    seed = 7
    N0 = w.N - 1
    sample = {(0, 0), (5, 3), (15, 7), (9, 1)}
    seqs = sorted({s for s, _ in sample})
    eng = harness.make_engine(w, w.N + 64, layers=w.layers)
    try:
        K_bits, V_bits, dirs_l, maw_state = {}, {}, {}, {}
        for layer in range(w.layers):
            dirs = synth.directions(w, seed, layer, 1, device="cuda")
            K, V, _ = synth.prefill_with_directions(w, seed, layer, N0, dirs, device="cuda")
            harness.prefill(eng, layer, K, V)
            K_bits[layer] = {s: synth.bits(K[s]) for s in seqs}
            V_bits[layer] = {s: synth.bits(V[s]) for s in seqs}
            del K, V
            dirs_l[layer] = dirs
            maw_state[layer] = {}
        torch.cuda.empty_cache()
        N = N0
        for step in range(w.steps):
            N += 1
            for layer in range(w.layers):
                kn, vn = synth.step_kv(w, seed, layer, step, device="cuda")
                q = synth.loop_query(w, seed, layer, step, dirs_l[layer], device="cuda")
                bufs = eng.alloc_step(w.B)
                eng.decode_step(layer, list(range(w.B)), q, bufs["blk_idx"], bufs["blk_cnt"],
                                bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"],
                                k_new=kn.view(w.B, w.Hkv, w.d).contiguous(),
                                v_new=vn.view(w.B, w.Hkv, w.d).contiguous())
                eng.sync()
                gpu = {k: v.cpu().numpy() for k, v in bufs.items()}
                knb, vnb = synth.bits(kn), synth.bits(vn)
                for s in seqs:
                    K_bits[layer][s] = np.concatenate([K_bits[layer][s], knb[s]], 0)
                    V_bits[layer][s] = np.concatenate([V_bits[layer][s], vnb[s]], 0)
                st = harness.check_units(w, eng, layer, list(range(w.B)), synth.bits(q),
                                         K_bits[layer], V_bits[layer],
                                         {s: N for s in range(w.B)}, gpu,
                                         maw_state=maw_state[layer], units=sample,
                                         check_summ=False)
                log("  step %d layer %d N=%d" % (step, layer, N))
                _check(st)
                assert len(st["units"]) == len(sample)
    finally:
        eng.close()


def test_loop32_256_steps_flags_fire():
    """The loop workload over its whole horizon on one layer at full per-layer
    size (B=16, N=65536 -> 65791, MAW beta=1): 256 one-launch steps with their
    appends, four sampled units in lockstep with the oracle at every step, MAW
    tables included.  The MAW flag fires on its own: blocks that leave the
    window with above-average mass keep a frozen MAW above beta*S/|D| and are
    ranked into the selection first; the run must see such selections."""
    w = _w(synth.loop32(), layers=1, steps=256)
    log("case: loop32 one layer, 256 steps, sampled units")
    seed = 7
    N0 = w.N - 1
    sample = {(0, 0), (5, 3), (9, 1), (15, 7)}
    seqs = sorted({s for s, _ in sample})
    eng = harness.make_engine(w, N0 + w.steps + 64)
    try:
        dirs = synth.directions(w, seed, 0, 1, device="cuda")
        K, V, _ = synth.prefill_with_directions(w, seed, 0, N0, dirs, device="cuda")
        harness.prefill(eng, 0, K, V)
        n_max = N0 + w.steps
        K_bits, V_bits = {}, {}
        for s in seqs:
            K_bits[s] = np.zeros((n_max, w.Hkv, w.d), np.uint16)
            V_bits[s] = np.zeros((n_max, w.Hkv, w.d), np.uint16)
            K_bits[s][:N0] = synth.bits(K[s])
            V_bits[s][:N0] = synth.bits(V[s])
        del K, V
        torch.cuda.empty_cache()
        maw_state = {}
        flagged = ties = 0
        max_dmaw = 0.0
        bufs = eng.alloc_step(w.B)
        N = N0
        for step in range(w.steps):
            kn, vn = synth.step_kv(w, seed, 0, step, device="cuda")
            q = synth.loop_query(w, seed, 0, step, dirs, device="cuda")
            eng.decode_step(0, list(range(w.B)), q, bufs["blk_idx"], bufs["blk_cnt"],
                            bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"],
                            k_new=kn.view(w.B, w.Hkv, w.d).contiguous(),
                            v_new=vn.view(w.B, w.Hkv, w.d).contiguous())
            eng.sync()
            gpu = {k: v.cpu().numpy() for k, v in bufs.items()}
            knb, vnb = synth.bits(kn), synth.bits(vn)
            for s in seqs:
                K_bits[s][N] = knb[s, 0]
                V_bits[s][N] = vnb[s, 0]
            N += 1
            st = harness.check_units(w, eng, 0, list(range(w.B)), synth.bits(q), K_bits,
                                     V_bits, {s: N for s in range(w.B)}, gpu,
                                     maw_state=maw_state, units=sample,
                                     check_summ=(step % 64 == 0), workers=4)
            harness.assert_parity(st)
            flagged += st["flagged"]
            ties += st["ties"]
            max_dmaw = max(max_dmaw, st["max_dmaw"])
            if step % 32 == 0 or step == w.steps - 1:
                log("  step %d N=%d flagged selections so far %d ties %d max|dMAW| %.2e "
                    "max|dO| %.2e" % (step, N, flagged, ties, max_dmaw, st["max_abs"]))
        assert flagged > 0, "no selection was decided by a MAW flag"
    finally:
        eng.close()


def test_loop32_all_layers_short_horizon():
    """All 32 layers of the loop workload at full per-layer size (B=16,
    N=65536: about 138 GB of KV resident), four decode steps through every
    layer with the one-launch step; one sampled unit per layer in lockstep
    with the oracle, MAW included."""
    w = _w(synth.loop32(), steps=4)
    log("case: loop32 all %d layers, %d steps" % (w.layers, w.steps))
    seed = 11
    N0 = w.N - 1
    eng = harness.make_engine(w, N0 + w.steps + 64, layers=w.layers)
    try:
        sample, K_bits, V_bits, dirs_l, maw_state = {}, {}, {}, {}, {}
        n_max = N0 + w.steps
        for layer in range(w.layers):
            dirs = synth.directions(w, seed, layer, 1, device="cuda")
            K, V, _ = synth.prefill_with_directions(w, seed, layer, N0, dirs, device="cuda")
            harness.prefill(eng, layer, K, V)
            s, g = (3 * layer + 1) % w.B, layer % w.Hkv
            sample[layer] = {(s, g)}
            kb = np.zeros((n_max, w.Hkv, w.d), np.uint16)
            vb = np.zeros((n_max, w.Hkv, w.d), np.uint16)
            kb[:N0] = synth.bits(K[s])
            vb[:N0] = synth.bits(V[s])
            K_bits[layer], V_bits[layer] = {s: kb}, {s: vb}
            dirs_l[layer] = dirs
            maw_state[layer] = {}
            del K, V
            torch.cuda.empty_cache()
        log("  prefilled %d layers" % w.layers)
        bufs = eng.alloc_step(w.B)
        N = N0
        for step in range(w.steps):
            for layer in range(w.layers):
                kn, vn = synth.step_kv(w, seed, layer, step, device="cuda")
                q = synth.loop_query(w, seed, layer, step, dirs_l[layer], device="cuda")
                eng.decode_step(layer, list(range(w.B)), q, bufs["blk_idx"], bufs["blk_cnt"],
                                bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"],
                                k_new=kn.view(w.B, w.Hkv, w.d).contiguous(),
                                v_new=vn.view(w.B, w.Hkv, w.d).contiguous())
                eng.sync()
                gpu = {k: v.cpu().numpy() for k, v in bufs.items()}
                (s, g), = sample[layer]
                K_bits[layer][s][N] = synth.bits(kn)[s, 0]
                V_bits[layer][s][N] = synth.bits(vn)[s, 0]
                st = harness.check_units(w, eng, layer, list(range(w.B)), synth.bits(q),
                                         K_bits[layer], V_bits[layer],
                                         {x: N + 1 for x in range(w.B)}, gpu,
                                         maw_state=maw_state[layer], units=sample[layer],
                                         check_summ=(step == 0))
                harness.assert_parity(st)
            N += 1
            log("  step %d done (N=%d)" % (step, N))
    finally:
        eng.close()


@pytest.mark.parametrize("window,S", [(0, 16), (8, 16), (16, 16), (32, 64), (64, 64)])
def test_fused_append_window_against_block_size(window, S):
    """The one-launch step with its one-token append, four steps in a row,
    every unit against the oracle (summaries included).  With W >= S the
    append runs inside the step (the new token's block lies wholly in the
    window); with W < S that block can be a candidate, so the append kernel
    runs first."""
    w = _w(synth.tiny(), B=3, N=3000, window=window, block_size=[S], budget_ppm=[100000])
    log("case: fused append, W=%d S=%d" % (window, S))
    x = synth.single_step(w, 4, device="cuda", N=w.N)
    N0 = w.N - 4
    eng = harness.make_engine(w, w.N + 64)
    try:
        harness.prefill(eng, 0, x["K"][:, :N0].contiguous(), x["V"][:, :N0].contiguous())
        Kb, Vb = synth.bits(x["K"]), synth.bits(x["V"])
        bufs = eng.alloc_step(w.B)
        for t in range(4):
            N = N0 + t + 1
            kn = x["K"][:, N - 1].contiguous()
            vn = x["V"][:, N - 1].contiguous()
            q = synth.single_step(w, 100 + t, device="cuda", N=16)["q"]
            eng.decode_step(0, list(range(w.B)), q, bufs["blk_idx"], bufs["blk_cnt"],
                            bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"],
                            k_new=kn, v_new=vn)
            eng.sync()
            gpu = {k: v.cpu().numpy() for k, v in bufs.items()}
            st = harness.check_units(w, eng, 0, list(range(w.B)), synth.bits(q),
                                     {b: Kb[b] for b in range(w.B)}, {b: Vb[b] for b in range(w.B)},
                                     {b: N for b in range(w.B)}, gpu, check_summ=True)
            _check(st)
    finally:
        eng.close()
