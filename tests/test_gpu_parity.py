"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (in tests/harness.py): selected indices bit-exact except counted ties
inside a 1e-6 relative score band; max |dO| <= 2e-3, max relative dO <= 1e-2
where |O| >= 0.1, |d lse| <= 1e-4; summaries equal; MAW within 1e-5 + 1e-3 rel.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import harness
from tests.harness import log
from block_sparse_top_score_amd._abi import SDError

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


@pytest.mark.parametrize("seed", range(10))
def test_tiny_workload(seed):
    log("case: tiny seed=%d" % seed)
    st = harness.run_single_step(synth.tiny(), seed)
    harness.assert_parity(st)
    assert st["ties"] == 0


@pytest.mark.parametrize("N", [1, 3, 17, 60, 68, 69, 100, 1000, 1007, 2049])
def test_tiny_ragged_lengths(N):
    """Ragged tails (partial pages and blocks), N inside the dense set, a
    single token."""
    log("case: tiny ragged N=%d" % N)
    st = harness.run_single_step(synth.tiny(), 3, N=N)
    harness.assert_parity(st)


@pytest.mark.parametrize("S", [16, 32, 48, 64])
def test_block_sizes(S):
    w = _w(synth.tiny(), block_size=[S], N=3000, n_plant=4)
    log("case: block size S=%d" % S)
    harness.assert_parity(harness.run_single_step(w, 5))


def test_full_budget_equals_dense():
    w = _w(synth.tiny(), budget_ppm=[1_000_000], N=1500)
    log("case: full budget")
    x = synth.single_step(w, 7)
    st = harness.run_single_step(w, 7)
    harness.assert_parity(st)
    q, K, V = synth.bits(x["q"]), synth.bits(x["K"]), synth.bits(x["V"])
    O, lse = oracle.dense(q[0], np.ascontiguousarray(K[0, :, 0]),
                          np.ascontiguousarray(V[0, :, 0]), 1500)
    ma, mr, ml = harness.compare_outputs(st["gpu"]["o"][0], st["gpu"]["lse"][0], O, lse)
    assert ma <= harness.ABS_TOL and ml <= harness.LSE_TOL


def test_no_sinks_no_window():
    w = _w(synth.tiny(), n_sink=0, window=0, N=2000)
    log("case: no dense set")
    harness.assert_parity(harness.run_single_step(w, 9))


def test_zero_budget_dense_only():
    w = _w(synth.tiny(), budget_ppm=[0], N=2000)
    log("case: zero budget")
    st = harness.run_single_step(w, 9)
    harness.assert_parity(st)
    assert st["gpu"]["blk_cnt"].max() == 0


def test_page_shuffle_invariance():
    """Scattered pages give bitwise the same results as sequential pages."""
    w = _w(synth.llama32k(), B=2, N=4099)
    log("case: page shuffle invariance")
    a = harness.run_single_step(w, 1, shuffle_seed=0)
    b = harness.run_single_step(w, 1, shuffle_seed=12345)
    harness.assert_parity(a)
    for k in ("blk_idx", "blk_cnt", "o", "lse"):
        assert np.array_equal(a["gpu"][k], b["gpu"][k]), k


def test_chunked_append_matches():
    """Prefill in uneven pieces: same summaries and outputs as one piece."""
    w = _w(synth.llama32k(), B=2, N=5000)
    log("case: chunked append")
    a = harness.run_single_step(w, 2, chunks=1)
    b = harness.run_single_step(w, 2, chunks=7)
    harness.assert_parity(b)
    for k in ("blk_idx", "blk_cnt", "o", "lse"):
        assert np.array_equal(a["gpu"][k], b["gpu"][k]), k


def test_fused_step_equals_separate_calls():
    """Same selection.  Without MAW flags the one-launch step hands the
    selection to its attention parts in key order, where the attend call
    takes the caller's ascending list, so the pages are visited in another
    order and O and lse agree to the fp32 rounding of the softmax sums."""
    w = _w(synth.llama32k(), B=2, N=6000)
    log("case: fused step")
    a = harness.run_single_step(w, 4, fused=False)
    b = harness.run_single_step(w, 4, fused=True)
    harness.assert_parity(b)
    for k in ("blk_idx", "blk_cnt"):
        assert np.array_equal(a["gpu"][k], b["gpu"][k]), k
    np.testing.assert_allclose(b["gpu"]["o"], a["gpu"]["o"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(b["gpu"]["lse"], a["gpu"]["lse"], rtol=0, atol=1e-5)


@pytest.mark.parametrize("shape", ["llama", "qwen"])
def test_fused_step_with_append_equals_separate_calls(shape):
    """sparse_decode_step with the one-token append equals append_kv +
    select_topk + sparse_attend + fuse_lse, over several steps (MAW on).
    qwen: per-head block sizes and budgets, so the units of one launch use
    different numbers of attention parts, and the 1500-block units take the
    four-wave top-k."""
    if shape == "llama":
        w = _w(synth.llama32k(), B=3, N=3000, maw_beta=1.0)
    else:
        w = _w(synth.qwen128k(0), B=3, N=24000, maw_beta=1.0)
    log("case: fused step with append (%s) S=%s ppm=%s" % (shape, w.block_size, w.budget_ppm))
    x = synth.single_step(w, 6, N=w.N)
    engs = [harness.make_engine(w, w.N + 64) for _ in range(2)]
    try:
        for e in engs:
            harness.prefill(e, 0, x["K"].cuda(), x["V"].cuda())
        seqs = [0, 1, 2]
        for step in range(5):
            kn, vn = synth.step_kv(w, 6, 0, step, device="cuda")
            kn = kn.view(w.B, w.Hkv, w.d).contiguous()
            vn = vn.view(w.B, w.Hkv, w.d).contiguous()
            q = synth.randn((w.B, w.Hq, w.d), 6, 700 + step, "cuda")
            a = engs[0].alloc_step(3)
            engs[0].append_kv(0, seqs, [1, 1, 1], kn, vn)
            engs[0].select_topk(0, seqs, q, a["blk_idx"], a["blk_cnt"])
            engs[0].sparse_attend(0, seqs, q, a["blk_idx"], a["blk_cnt"], a["o_part"], a["lse_part"])
            engs[0].fuse_lse(0, seqs, a["o_part"], a["lse_part"], a["o"], a["lse"])
            b = engs[1].alloc_step(3)
            engs[1].decode_step(0, seqs, q, b["blk_idx"], b["blk_cnt"], b["o_part"],
                                b["lse_part"], b["o"], b["lse"], k_new=kn, v_new=vn)
            torch.cuda.synchronize()
            for k in ("blk_cnt", "o", "lse"):
                assert torch.equal(a[k], b[k]), (step, k)
            for s_ in range(3):
                for g in range(w.Hkv):
                    n = int(a["blk_cnt"][s_, g])
                    assert torch.equal(a["blk_idx"][s_, g, :n], b["blk_idx"][s_, g, :n])
        for s_ in range(3):
            ma = engs[0].debug(harness.SD_DEBUG_MAW, 0, s_)
            mb = engs[1].debug(harness.SD_DEBUG_MAW, 0, s_)
            assert np.array_equal(ma, mb)
            assert ma.max() > 0
    finally:
        for e in engs:
            e.close()


def test_many_sequences_split_launches():
    w = _w(synth.tiny(), B=80, N=700)
    log("case: 80 sequences")
    harness.assert_parity(harness.run_single_step(w, 11))


@pytest.mark.parametrize("G,Hkv,d", [(1, 2, 128), (7, 4, 128), (8, 2, 64), (3, 3, 64)])
def test_group_sizes(G, Hkv, d):
    w = synth.Workload("g", B=2, Hq=G * Hkv, Hkv=Hkv, d=d, N=3333,
                       block_size=[16, 32, 64][:1] * Hkv, budget_ppm=[50000] * Hkv,
                       n_sink=4, window=128, plant_frac=0.02, sink_scale=4.0)
    log("case: G=%d Hkv=%d d=%d" % (G, Hkv, d))
    harness.assert_parity(harness.run_single_step(w, 13))


@pytest.mark.parametrize("N,fused", [(4096, False), (40000, False), (40000, True)])
def test_tied_scores_resolved_exactly(N, fused):
    """Coarse integer keys make many block scores exactly equal: every tie at
    the k-th key goes through the exact re-scoring and the index tie-break
    (N = 40000: 2500 blocks, the four-wave top-k of long units)."""
    w = _w(synth.tiny(), N=N, n_plant=0)
    log("case: tied scores N=%d fused=%s" % (N, fused))
    x = synth.single_step(w, 3, N=N)
    g = torch.Generator().manual_seed(3)
    K = torch.randint(-1, 2, x["K"].shape, generator=g).to(torch.bfloat16)
    eng = harness.make_engine(w, N + 64)
    try:
        harness.prefill(eng, 0, K.cuda(), x["V"].cuda())
        gpu = harness.run_gpu_step(eng, 0, [0], x["q"].cuda(), fused=fused)
        Kb, Vb = synth.bits(K), synth.bits(x["V"])
        st = harness.check_units(w, eng, 0, [0], synth.bits(x["q"]), {0: Kb[0]}, {0: Vb[0]},
                                 {0: N}, gpu)
        harness.assert_parity(st)
        assert st["ties"] == 0
    finally:
        eng.close()


def test_large_block_count_global_topk():
    """More blocks per unit than the top-k keeps in LDS (global-memory path)."""
    w = _w(synth.tiny(), N=70001, block_size=[16], budget_ppm=[30000])
    log("case: 4376 blocks per unit")
    harness.assert_parity(harness.run_single_step(w, 8))


def test_qwen128k_full_single_step():
    """Per-KV-head block sizes (16/64) and budgets (1-20%), G=7, N=131072."""
    w = synth.qwen128k(0)
    log("case: qwen128k S=%s ppm=%s" % (w.block_size, w.budget_ppm))
    st = harness.run_single_step(w, 0)
    log("  ties=%d max|dO|=%.3g max|dlse|=%.3g" % (st["ties"], st["max_abs"], st["max_dlse"]))
    harness.assert_parity(st)


def test_llama32k_full():
    """The metric workload at full size: every unit against the oracle."""
    log("case: llama32k full (B=8, 32/8 heads, d=128, N=32768)")
    st = harness.run_single_step(synth.llama32k(), 0)
    log("  ties=%d max|dO|=%.3g max rel=%.3g max|dlse|=%.3g" % (
        st["ties"], st["max_abs"], st["max_rel"], st["max_dlse"]))
    harness.assert_parity(st)
    assert len(st["units"]) == 64


@pytest.mark.parametrize("B,S,pct", [(1, 16, 2), (8, 32, 5), (32, 64, 10), (64, 16, 10),
                                     (64, 64, 2)])
def test_sweep_points(B, S, pct):
    w = synth.sweep(B, S, pct)
    log("case: sweep B=%d S=%d budget=%d%%" % (B, S, pct))
    harness.assert_parity(harness.run_single_step(w, 21))


def test_fuse_pure_identity():
    """fuse_lse(layer=-1) on random partials equals the oracle fusion; -inf
    partials drop out."""
    w = synth.llama32k()
    log("case: pure fusion")
    eng = harness.make_engine(_w(w, B=2), 256)
    try:
        n, P, d = 3, eng.p_cap, w.d
        g = torch.Generator().manual_seed(5)
        o_part = torch.randn(n, w.Hq, P, d, generator=g)
        lse_part = torch.randn(n, w.Hq, P, generator=g) * 5
        lse_part[:, :, P // 2:] = -float("inf")
        lse_part[0, 0, :] = -float("inf")     # an empty head
        o = torch.empty(n, w.Hq, d, device="cuda")
        lse = torch.empty(n, w.Hq, device="cuda")
        eng.fuse_lse(-1, None, o_part.cuda(), lse_part.cuda(), o, lse, n_seqs=n)
        eng.sync()
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        for i in range(n):
            for h in range(w.Hq):
                Oref, lref = oracle.fuse(o_part[i, h].double().numpy(),
                                         lse_part[i, h].double().numpy())
                if lref == -np.inf:
                    assert lse[i, h] == -np.inf and np.all(o[i, h] == 0)
                    continue
                assert abs(lse[i, h] - lref) <= 1e-5
                assert np.abs(o[i, h] - Oref).max() <= 1e-5
    finally:
        eng.close()


def test_error_paths():
    w = _w(synth.tiny(), N=2000, budget_ppm=[1000000])  # full budget: several partial slots
    log("case: error paths")
    eng = harness.make_engine(w, 2048)
    try:
        x = synth.single_step(w, 0, N=2000)
        K, V, q = x["K"].cuda(), x["V"].cuda(), x["q"].cuda()
        harness.prefill(eng, 0, K, V)
        bufs = eng.alloc_step(1)
        # fuse before attend
        st = eng.fuse_lse(0, [0], bufs["o_part"], bufs["lse_part"], bufs["o"],
                          bufs["lse"], check=False)
        assert st == -5
        # k_cap too small
        small = torch.zeros(1, 1, 1, dtype=torch.int32, device="cuda")
        assert eng.select_topk(0, [0], q, small, bufs["blk_cnt"], check=False) == -1
        # bad sequence / layer ids, repeated ids
        assert eng.select_topk(0, [5], q, bufs["blk_idx"], bufs["blk_cnt"], check=False) == -1
        assert eng.select_topk(3, [0], q, bufs["blk_idx"], bufs["blk_cnt"], check=False) == -1
        # page pool exhaustion leaves the sequence unchanged
        big = torch.zeros(4096, 1, w.d, dtype=torch.bfloat16, device="cuda")
        assert eng.append_kv(0, [0], [4096], big, big, check=False) == -1  # > max_seq_len
        assert eng.seq_len(0, 0) == 2000
        # p_cap too small (the engine needs more than one partial slot here)
        assert eng.p_cap > 1
        tiny_part = torch.zeros(1, w.Hq, 1, w.d, device="cuda")
        tiny_lse = torch.zeros(1, w.Hq, 1, device="cuda")
        eng.select_topk(0, [0], q, bufs["blk_idx"], bufs["blk_cnt"])
        assert eng.sparse_attend(0, [0], q, bufs["blk_idx"], bufs["blk_cnt"], tiny_part,
                                 tiny_lse, check=False) == -1
        # o_part not 16-byte aligned: both calls that read it refuse it
        flat = torch.zeros(bufs["o_part"].numel() + 4, device="cuda")
        skew = flat[1:1 + bufs["o_part"].numel()].view(bufs["o_part"].shape)
        assert eng.fuse_lse(-1, None, skew, bufs["lse_part"], bufs["o"], bufs["lse"],
                            check=False) == -1
        assert eng.decode_step(0, [0], q, bufs["blk_idx"], bufs["blk_cnt"], skew,
                               bufs["lse_part"], bufs["o"], bufs["lse"], check=False) == -1
        assert eng.seq_len(0, 0) == 2000
        # pure fusion over more slots than the fusion holds: refused, nothing runs
        wide_part = torch.zeros(1, w.Hq, 300, w.d, device="cuda")
        wide_lse = torch.full((1, w.Hq, 300), -float("inf"), device="cuda")
        assert eng.fuse_lse(-1, None, wide_part, wide_lse, bufs["o"], bufs["lse"], n_seqs=1,
                            check=False) == -4
        eng.sync()
    finally:
        eng.close()
    # sinks + window beyond the pages the fusion holds: refused at init
    with pytest.raises(SDError) as e:
        harness.make_engine(_w(synth.tiny(), window=40000), 41000)
    assert e.value.status == -4


def test_out_of_range_selection_entries_attend_nothing():
    """sparse_attend skips blk_idx entries outside [0, n_blk): O and lse equal
    the oracle's attention over the in-range entries, and MAW (fed by the
    dense pages only) equals the oracle's."""
    w = _w(synth.tiny(), N=1000)
    log("case: out-of-range selection entries")
    x = synth.single_step(w, 1, N=1000)
    K, V, q = x["K"].cuda(), x["V"].cuda(), x["q"].cuda()
    eng = harness.make_engine(w, 1064)
    try:
        harness.prefill(eng, 0, K, V)
        bufs = eng.alloc_step(1)
        eng.select_topk(0, [0], q, bufs["blk_idx"], bufs["blk_cnt"])
        eng.sync()
        cnt = int(bufs["blk_cnt"][0, 0])
        nb = -(-1000 // 16)
        assert cnt >= 3
        bufs["blk_idx"][0, 0, 0] = -3
        bufs["blk_idx"][0, 0, cnt - 1] = nb + 5
        eng.sparse_attend(0, [0], q, bufs["blk_idx"], bufs["blk_cnt"], bufs["o_part"],
                          bufs["lse_part"])
        eng.fuse_lse(0, [0], bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"])
        eng.sync()
        sel = bufs["blk_idx"][0, 0, :cnt].cpu().numpy()
        sel = sel[(sel >= 0) & (sel < nb)]
        assert len(sel) == cnt - 2
        Kb, Vb, qb = synth.bits(K[0, :, 0]), synth.bits(V[0, :, 0]), synth.bits(q[0])
        ref = oracle.attend(qb, Kb, Vb, 1000, 16, w.n_sink, w.window, sel)
        ma, mr, ml = harness.compare_outputs(bufs["o"][0].cpu().numpy(),
                                             bufs["lse"][0].cpu().numpy(), ref["O"], ref["lse"])
        harness.assert_parity(dict(max_abs=ma, max_rel=mr, max_dlse=ml))
        a = oracle.dense_mass(qb, Kb, 1000, 16, w.n_sink, w.window)
        want = oracle.maw_step(np.zeros(nb), a, 1000, 16, w.n_sink, w.window, w.maw_decay)
        got = harness.maw_by_head(eng, 0, 0, w, 1000)[0]
        assert np.all(np.abs(got - want) <= harness.MAW_ABS + harness.MAW_REL * np.abs(want))
    finally:
        eng.close()


def test_pool_exhaustion_enomem():
    w = _w(synth.tiny(), N=64)
    log("case: pool exhaustion")
    eng = harness.make_engine(w, 4096, extra_pages=-10)   # 246 pages
    try:
        K = torch.zeros(4096, 1, w.d, dtype=torch.bfloat16, device="cuda")
        eng.append_kv(0, [0], [3900], K, K)                 # 244 pages
        assert eng.seq_len(0, 0) == 3900
        assert eng.append_kv(0, [0], [100], K, K, check=False) == -2
        assert eng.seq_len(0, 0) == 3900
        eng.release_seq(0)
        assert eng.seq_len(0, 0) == 0
        eng.append_kv(0, [0], [246 * 16], K, K)
        assert eng.seq_len(0, 0) == 246 * 16
        eng.sync()
    finally:
        eng.close()


@pytest.mark.parametrize("N,fused", [(8000, False), (48000, False), (48000, True)])
def test_maw_flag_selection(N, fused):
    """MAW threshold flags rank blocks first (values set through the debug
    hook; the oracle reads the same fp32 values widened to double).  N =
    48000: 1500 blocks, the four-wave top-k of long units."""
    w = _w(synth.llama32k(), B=2, N=N, maw_beta=1.0)
    log("case: MAW flag selection N=%d fused=%s" % (N, fused))
    x = synth.single_step(w, 3, N=N)
    K, V, q = x["K"].cuda(), x["V"].cuda(), x["q"].cuda()
    eng = harness.make_engine(w, N + 64)
    try:
        harness.prefill(eng, 0, K, V)
        nb = N // 32
        rng = np.random.default_rng(0)
        maw_set, vals_by = {}, {}
        for s in range(2):
            vals = np.zeros(w.Hkv * nb, np.float32)
            # threshold beta*S/|D| = 32/516; put some blocks far above it
            for g in range(w.Hkv):
                hot = rng.choice(np.arange(1, nb - 20), size=12, replace=False)
                vals[g * nb + hot] = 0.5
                vals[g * nb + rng.choice(np.arange(1, nb - 20), size=5)] = 0.01
            eng.set_maw(0, s, vals)
            for g in range(w.Hkv):
                maw_set[(s, g)] = vals[g * nb:(g + 1) * nb].astype(np.float64)
                vals_by[(s, g)] = maw_set[(s, g)].copy()
        gpu = harness.run_gpu_step(eng, 0, [0, 1], q, fused=fused)
        Kb, Vb = synth.bits(K), synth.bits(V)
        st = harness.check_units(w, eng, 0, [0, 1], synth.bits(q), {0: Kb[0], 1: Kb[1]},
                                 {0: Vb[0], 1: Vb[1]}, {0: N, 1: N}, gpu,
                                 maw_state=maw_set)
        harness.assert_parity(st)
        for s in range(2):
            for g in range(w.Hkv):
                sel = set(gpu["blk_idx"][s, g, :gpu["blk_cnt"][s, g]].tolist())
                hot = set(np.nonzero(vals_by[(s, g)] >= 0.5)[0].tolist())
                assert hot <= sel, "flagged blocks must be selected first"
    finally:
        eng.close()


def test_multistep_maw_lockstep():
    """Several layers x decode steps with MAW on (a small loop workload):
    lockstep parity every step, MAW tables compared every step."""
    w = _w(synth.loop32(), B=2, N=3000, layers=2, steps=12)
    log("case: multistep MAW lockstep")
    eng = harness.make_engine(w, 3000 + 64, layers=w.layers)
    try:
        K_bits, V_bits, maw_state, dirs_l = {}, {}, {}, {}
        for layer in range(w.layers):
            dirs = synth.directions(w, 0, layer, 1, device="cuda")
            K, V, _ = synth.prefill_with_directions(w, 0, layer, w.N - 1, dirs, device="cuda")
            harness.prefill(eng, layer, K, V)
            Kb, Vb = synth.bits(K), synth.bits(V)
            K_bits[layer] = {b: Kb[b] for b in range(w.B)}
            V_bits[layer] = {b: Vb[b] for b in range(w.B)}
            maw_state[layer] = {}
            dirs_l[layer] = dirs
        N = w.N - 1
        for step in range(w.steps):
            N += 1
            for layer in range(w.layers):
                kn, vn = synth.step_kv(w, 0, layer, step, device="cuda")
                eng.append_kv(layer, list(range(w.B)), [1] * w.B,
                              kn.view(w.B, w.Hkv, w.d).contiguous(),
                              vn.view(w.B, w.Hkv, w.d).contiguous())
                knb, vnb = synth.bits(kn), synth.bits(vn)
                for b in range(w.B):
                    K_bits[layer][b] = np.concatenate([K_bits[layer][b], knb[b]], 0)
                    V_bits[layer][b] = np.concatenate([V_bits[layer][b], vnb[b]], 0)
                q = synth.loop_query(w, 0, layer, step, dirs_l[layer], device="cuda")
                gpu = harness.run_gpu_step(eng, layer, list(range(w.B)), q)
                st = harness.check_units(w, eng, layer, list(range(w.B)), synth.bits(q),
                                         K_bits[layer], V_bits[layer],
                                         {b: N for b in range(w.B)}, gpu,
                                         maw_state=maw_state[layer],
                                         check_summ=(step % 4 == 0))
                harness.assert_parity(st)
        log("  final N=%d" % N)
    finally:
        eng.close()
