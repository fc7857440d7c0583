"""Learn-from-the-past selection on the GPU against the oracle.

With lfps_select = 1 the selection ranks only the candidates of the vertical
and slash tables ("Learn from the Past: Fast Sparse Indexing for Large
Language Model Decoding", What carries the argument and Figure 4; block
granularity as the oracle reads it), fuse_lse updates the tables from the
step's block masses, and sd_lfps_init fills them from the last s prefill
positions (Assumptions & free parameters, s = 32).  Checked:
  * selection from given tables: bit-exact against oracle.lfps_select on the
    same fp32 table values (ties inside the score band counted), including
    candidate sets past the kernel's LDS list;
  * the init against oracle.lfps_init (fp32 softmax against fp64: |d| <=
    1e-6 + 1e-4 |ref|);
  * a run of steps in lockstep: each step's selection from the GPU's tables,
    its outputs (the harness's bars) and the tables after the update against
    oracle.lfps_update with the oracle's block masses over the GPU's
    selection (same tolerance).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from block_sparse_top_score_amd import _abi
from block_sparse_top_score_amd._abi import SDError
from tests import harness
from tests.harness import log

pytestmark = pytest.mark.gpu

A_LFPS = 0.2
TAB_ABS, TAB_REL = 1e-6, 1e-4


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _engine(w, N_max):
    pages = w.B * ((N_max + 15) // 16)
    return _abi.SparseDecode(max_seqs=w.B, num_layers=1, num_q_heads=w.Hq, num_kv_heads=w.Hkv,
                             head_dim=w.d, num_pages=pages, max_seq_len=N_max,
                             sink_tokens=w.n_sink, recent_window=w.window,
                             block_size=w.block_size, budget_ppm=w.budget_ppm,
                             maw_decay=0.95, maw_beta=0.0, lfps_select=1, lfps_a=A_LFPS)


def _tables(eng, b, w, N):
    raw = eng.debug(_abi.SD_DEBUG_LFPS, 0, b).astype(np.float64)
    out, off = [], 0
    for h in range(w.Hkv):
        nb = synth.n_blocks(N, w.block_size[h])
        out.append((raw[off:off + nb], raw[off + nb:off + 2 * nb]))
        off += 2 * nb
    return out


def _check_selection(w, eng, gpu, qb, N, tabs, summ):
    ties = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            S = w.block_size[h]
            mn, mx = summ[b][h]
            qg = np.ascontiguousarray(qb[b, h * w.G:(h + 1) * w.G])
            pv, ps = tabs[b][h]
            ref = oracle.lfps_select(qg, mn, mx, N, S, w.n_sink, w.window, w.budget_ppm[h],
                                     pv, ps, A_LFPS)
            cnt = int(gpu["blk_cnt"][b, h])
            ties += harness.adjudicate(gpu["blk_idx"][b, h, :cnt], ref, ref["k"])
            _, nC = oracle.lfps_candidates(pv, ps, N, S, w.n_sink, w.window, A_LFPS)
            assert int(eng.debug(_abi.SD_DEBUG_LFPS_CAND, 0, b)[h]) == nC, (b, h)
    return ties


@pytest.mark.parametrize("kind", ["random", "flat"])
def test_selection_from_given_tables(kind):
    """Random sparse tables; and nearly flat ones whose candidate set holds
    almost every block (past the 6144 entries the kernel keeps in LDS)."""
    w = synth.qwen128k()
    N = 120000 if kind == "flat" else 30000
    w = dataclasses.replace(w, B=2, N=N, block_size=[16, 64, 16, 32],
                                    budget_ppm=[20000, 50000, 150000, 100000])
    log("case: lfps tables %s N=%d" % (kind, N))
    x = synth.single_step(w, 3, device="cuda", N=N)
    eng = _engine(w, N + 64)
    try:
        harness.prefill(eng, 0, x["K"], x["V"])
        rng = np.random.default_rng(11)
        tabs = {}
        for b in range(w.B):
            tabs[b], flat = {}, []
            for h in range(w.Hkv):
                nb = synth.n_blocks(N, w.block_size[h])
                if kind == "random":
                    pv = (rng.random(nb) * (rng.random(nb) < 0.05)).astype(np.float32)
                    ps = (rng.random(nb) * (rng.random(nb) < 0.02)).astype(np.float32)
                else:
                    pv = np.ones(nb, np.float32)
                    pv[rng.integers(0, nb, 5)] = 0.0
                    ps = np.zeros(nb, np.float32)
                tabs[b][h] = (pv.astype(np.float64), ps.astype(np.float64))
                flat += [pv, ps]
            eng.set_lfps(0, b, np.concatenate(flat))
        bufs = eng.alloc_step(w.B)
        q = x["q"]
        eng.select_topk(0, list(range(w.B)), q, bufs["blk_idx"], bufs["blk_cnt"])
        eng.sync()
        gpu = {k: v.cpu().numpy() for k, v in bufs.items()}
        summ = {b: harness.summaries_by_head(eng, 0, b, w, N) for b in range(w.B)}
        ties = _check_selection(w, eng, gpu, synth.bits(q), N, tabs, summ)
        cands = [eng.debug(_abi.SD_DEBUG_LFPS_CAND, 0, b).tolist() for b in range(w.B)]
        log("  candidates per unit %s, ties %d" % (cands, ties))
        if kind == "flat":
            assert max(max(c) for c in cands) > 6144
    finally:
        eng.close()


def test_init_and_lockstep_steps():
    w = dataclasses.replace(synth.llama32k(), B=2, N=8000)
    N0, s_steps, steps = 8000, 32, 6
    G = w.G
    log("case: lfps init from %d prefill positions, then %d steps" % (s_steps, steps))
    x = synth.single_step(w, 5, device="cuda", N=N0)
    qp = synth.randn((w.B, s_steps, w.Hq, w.d), 5, 40, "cuda")
    eng = _engine(w, N0 + steps + 64)
    try:
        harness.prefill(eng, 0, x["K"], x["V"])
        eng.lfps_init(0, list(range(w.B)), qp)
        eng.sync()
        Kb, Vb, qpb = synth.bits(x["K"]), synth.bits(x["V"]), synth.bits(qp)
        worst = 0.0
        for b in range(w.B):
            got = _tables(eng, b, w, N0)
            for h in range(w.Hkv):
                pv, ps = oracle.lfps_init(np.ascontiguousarray(qpb[b, :, h * G:(h + 1) * G]),
                                          np.ascontiguousarray(Kb[b, :, h]), N0, w.block_size[h])
                for g_, r_ in ((got[h][0], pv), (got[h][1], ps)):
                    err = np.abs(g_ - r_)
                    assert (err <= TAB_ABS + TAB_REL * np.abs(r_)).all(), (b, h, float(err.max()))
                    worst = max(worst, float(err.max()))
        log("  init: max |d table| %.2e" % worst)
        K_bits = {b: list(Kb[b]) for b in range(w.B)}
        V_bits = {b: list(Vb[b]) for b in range(w.B)}
        bufs = eng.alloc_step(w.B)
        seqs = list(range(w.B))
        ties = 0
        ma = ml = 0.0
        for t in range(steps):
            kn = synth.randn((w.B, w.Hkv, w.d), 5, 100 + t, "cuda")
            vn = synth.randn((w.B, w.Hkv, w.d), 5, 200 + t, "cuda")
            q = synth.randn((w.B, w.Hq, w.d), 5, 300 + t, "cuda")
            eng.append_kv(0, seqs, [1] * w.B, kn, vn)
            for b in range(w.B):
                K_bits[b].append(synth.bits(kn)[b])
                V_bits[b].append(synth.bits(vn)[b])
            N = N0 + t + 1
            before = {b: _tables(eng, b, w, N) for b in seqs}
            eng.select_topk(0, seqs, q, bufs["blk_idx"], bufs["blk_cnt"])
            eng.sparse_attend(0, seqs, q, bufs["blk_idx"], bufs["blk_cnt"], bufs["o_part"],
                              bufs["lse_part"])
            eng.fuse_lse(0, seqs, bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"])
            eng.sync()
            gpu = {k: v.cpu().numpy() for k, v in bufs.items()}
            qb = synth.bits(q)
            summ = {b: harness.summaries_by_head(eng, 0, b, w, N) for b in seqs}
            ties += _check_selection(w, eng, gpu, qb, N, before, summ)
            for b in seqs:
                Kn, Vn = np.stack(K_bits[b]), np.stack(V_bits[b])
                after = _tables(eng, b, w, N)
                for h in range(w.Hkv):
                    S = w.block_size[h]
                    qg = np.ascontiguousarray(qb[b, h * G:(h + 1) * G])
                    Kh, Vh = np.ascontiguousarray(Kn[:, h]), np.ascontiguousarray(Vn[:, h])
                    sel = gpu["blk_idx"][b, h, :gpu["blk_cnt"][b, h]].astype(np.int32)
                    a = oracle.attend(qg, Kh, Vh, N, S, w.n_sink, w.window, sel)
                    d_abs, _, d_lse = harness.compare_outputs(gpu["o"][b, h * G:(h + 1) * G],
                                                              gpu["lse"][b, h * G:(h + 1) * G],
                                                              a["O"], a["lse"])
                    ma, ml = max(ma, d_abs), max(ml, d_lse)
                    mass = oracle.attend_mass(qg, Kh, N, S, w.n_sink, w.window, sel)
                    pv, ps = oracle.lfps_update(before[b][h][0], before[b][h][1], mass, 0.95)
                    for g_, r_ in ((after[h][0], pv), (after[h][1], ps)):
                        err = np.abs(g_ - r_)
                        assert (err <= TAB_ABS + TAB_REL * np.abs(r_)).all(), (t, b, h, float(err.max()))
        log("  %d steps: ties %d, max_abs %.2e, max_dlse %.2e" % (steps, ties, ma, ml))
        assert ma <= harness.ABS_TOL and ml <= harness.LSE_TOL
    finally:
        eng.close()


def test_refusals():
    w = synth.tiny()
    eng = _engine(w, 1100)
    try:
        x = synth.single_step(w, 0, device="cpu", N=1000)
        harness.prefill(eng, 0, x["K"].cuda(), x["V"].cuda())
        bufs = eng.alloc_step(1)
        with pytest.raises(SDError) as e:
            eng.decode_step(0, [0], x["q"].cuda(), bufs["blk_idx"], bufs["blk_cnt"],
                            bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"])
        assert e.value.status == -4
        with pytest.raises(SDError):
            eng.lfps_init(0, [0], torch.zeros(1, 2000, w.Hq, w.d, dtype=torch.bfloat16,
                                              device="cuda"))
    finally:
        eng.close()
    with pytest.raises(SDError):
        _abi.SparseDecode(max_seqs=1, num_layers=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                          num_pages=100, max_seq_len=1000, sink_tokens=4, recent_window=64,
                          block_size=[16], budget_ppm=[50000], maw_beta=1.0, lfps_select=1)
