"""GPU-vs-oracle parity harness (test infrastructure).

Runs workloads from `synth` through the HIP library (C ABI via the Python
binding) and through the CPU oracle on the same bf16 bits, and compares:

  * selected block indices: bit-exact, except ties inside the stated band
    (every block of the symmetric difference has an oracle score within
    1e-6 relative of the k-th selected score, or an oracle MAW within the
    MAW tolerance of the flag threshold beta*S/|D|: the GPU keeps MAW in
    fp32 from fp32 attention weights, so a flag decision closer to the
    threshold than that tolerance is not decided by the definition); ties
    are counted and the oracle then attends over the GPU's selection;
  * outputs: max |dO| <= 2e-3; max |dO|/|O| <= 1e-2 where |O| >= 0.1;
    |d lse| <= 1e-4 (bf16 inputs, fp32 accumulation);
  * block summaries: equal by value;
  * MAW: |d| <= 1e-5 + 1e-3 |ref|.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import synth
from block_sparse_top_score_amd import (SD_DEBUG_MAW, SD_DEBUG_SUMMARY,
                                        SparseDecode)

ABS_TOL = 2e-3
REL_TOL = 1e-2
REL_FLOOR = 0.1
LSE_TOL = 1e-4
TIE_BAND = 1e-6
MAW_ABS, MAW_REL = 1e-5, 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_engine(w: synth.Workload, N_max: int, *, layers=1, shuffle_seed=0,
                max_seqs=None, extra_pages=0, maw_beta=None, per_query_head=False):
    pages = w.B * ((N_max + 15) // 16) + extra_pages
    return SparseDecode(max_seqs=max_seqs or w.B, num_layers=layers,
                        num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.d,
                        num_pages=pages, max_seq_len=N_max,
                        sink_tokens=w.n_sink, recent_window=w.window,
                        block_size=w.block_size, budget_ppm=w.budget_ppm,
                        maw_decay=w.maw_decay,
                        maw_beta=w.maw_beta if maw_beta is None else maw_beta,
                        page_shuffle_seed=shuffle_seed,
                        select_per_query_head=1 if per_query_head else 0)


def prefill(eng, layer, K, V, seq_ids=None, chunks=1):
    """Append [B, N, Hkv, d] K/V (device) to sequences 0..B-1."""
    B, N = K.shape[0], K.shape[1]
    seq_ids = list(range(B)) if seq_ids is None else seq_ids
    bounds = np.linspace(0, N, chunks + 1).astype(int)
    for c in range(chunks):
        a, b = bounds[c], bounds[c + 1]
        if b <= a:
            continue
        kk = K[:, a:b].contiguous().view(B * (b - a), K.shape[2], K.shape[3])
        vv = V[:, a:b].contiguous().view(B * (b - a), V.shape[2], V.shape[3])
        eng.append_kv(layer, seq_ids, [b - a] * B, kk, vv)


def run_gpu_step(eng, layer, seq_ids, q, fused=False):
    bufs = eng.alloc_step(len(seq_ids), device=q.device)
    if fused:
        eng.decode_step(layer, seq_ids, q, bufs["blk_idx"], bufs["blk_cnt"],
                        bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"])
    else:
        eng.select_topk(layer, seq_ids, q, bufs["blk_idx"], bufs["blk_cnt"])
        eng.sparse_attend(layer, seq_ids, q, bufs["blk_idx"], bufs["blk_cnt"],
                          bufs["o_part"], bufs["lse_part"])
        eng.fuse_lse(layer, seq_ids, bufs["o_part"], bufs["lse_part"], bufs["o"],
                     bufs["lse"])
    eng.sync()
    return {k: v.cpu().numpy() for k, v in bufs.items()}


def summaries_by_head(eng, layer, seq, w, N):
    raw = eng.debug(SD_DEBUG_SUMMARY, layer, seq)
    out, off = [], 0
    for g in range(w.Hkv):
        nb = (N + w.block_size[g] - 1) // w.block_size[g]
        blk = raw[off:off + nb * w.d * 2].reshape(nb, w.d, 2)
        out.append((blk[:, :, 0], blk[:, :, 1]))
        off += nb * w.d * 2
    return out


def maw_by_head(eng, layer, seq, w, N):
    raw = eng.debug(SD_DEBUG_MAW, layer, seq)
    out, off = [], 0
    for g in range(w.Hkv):
        nb = (N + w.block_size[g] - 1) // w.block_size[g]
        out.append(raw[off:off + nb].astype(np.float64))
        off += nb
    return out


def adjudicate(gpu_sel, ores, k, maw_before=None, n_dense=None, beta=0.0, S=1):
    """Return number of tied blocks if the two selections differ only by
    ties inside the band; raise AssertionError otherwise."""
    a, b = set(gpu_sel.tolist()), set(ores["sel"].tolist())
    if a == b:
        return 0
    assert len(a) == len(b) == k, "selection sizes differ: gpu %d oracle %d k %d" % (
        len(a), len(b), k)
    U = ores["U"]
    kth = min(U[i] for i in b) if b else 0.0
    diff = a ^ b
    for i in diff:
        score_tie = abs(U[i] - kth) <= TIE_BAND * max(abs(U[i]), abs(kth), 1e-30)
        flag_tie = False
        if maw_before is not None and beta > 0 and n_dense > 0:
            thr = beta * S / n_dense   # flag iff MAW > thr (MAW*|D| > beta*S)
            flag_tie = abs(maw_before[i] - thr) <= MAW_ABS + MAW_REL * thr
        assert score_tie or flag_tie, (
            "block %d differs outside the tie band (U=%r, k-th=%r)" % (i, U[i], kth))
    return len(diff) // 2


def compare_outputs(O_gpu, lse_gpu, O_ref, lse_ref):
    dO = np.abs(O_gpu.astype(np.float64) - O_ref)
    max_abs = float(dO.max()) if dO.size else 0.0
    big = np.abs(O_ref) >= REL_FLOOR
    max_rel = float((dO[big] / np.abs(O_ref[big])).max()) if big.any() else 0.0
    dl = np.abs(lse_gpu.astype(np.float64) - lse_ref)
    finite = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), finite), "lse finiteness differs"
    max_dlse = float(dl[finite].max()) if finite.any() else 0.0
    return max_abs, max_rel, max_dlse


def _check_unit(w, seq, bi, g, N, q_bits, K_bits, V_bits, gpu, summ, maw_gpu, maw_state):
    """Oracle one (sequence, KV head) unit and compare it with the GPU's."""
    G = w.G
    S, ppm = w.block_size[g], w.budget_ppm[g]
    beta = w.maw_beta if maw_state is not None else 0.0
    qg = q_bits[bi, g * G:(g + 1) * G]
    Kg = np.ascontiguousarray(K_bits[seq][:N, g])
    Vg = np.ascontiguousarray(V_bits[seq][:N, g])
    mb = None if maw_state is None else maw_state.get((seq, g), np.zeros(0))
    ores = oracle.unit_step(qg, Kg, Vg, N, S, w.n_sink, w.window, ppm,
                            maw=mb, beta=beta, r=w.maw_decay)
    cnt = int(gpu["blk_cnt"][bi, g])
    assert cnt == ores["k"], "k differs: gpu %d oracle %d (seq %d head %d)" % (
        cnt, ores["k"], seq, g)
    gsel = gpu["blk_idx"][bi, g, :cnt]
    assert np.all(np.diff(gsel) > 0), "GPU selection not ascending"
    nd = oracle.dense_count(N, w.n_sink, w.window)
    ties = adjudicate(gsel, ores, cnt, ores.get("maw_before"), nd, beta, S)
    flagged = int(ores["flag"][ores["sel"]].sum()) if ores["k"] else 0
    if ties:
        ores = oracle.unit_step(qg, Kg, Vg, N, S, w.n_sink, w.window, ppm,
                                maw=mb, beta=beta, r=w.maw_decay, sel_override=gsel)
    r = dict(ties=ties, flagged=flagged)
    O_gpu = gpu["o"][bi, g * G:(g + 1) * G]
    lse_gpu = gpu["lse"][bi, g * G:(g + 1) * G]
    r["max_abs"], r["max_rel"], r["max_dlse"] = compare_outputs(O_gpu, lse_gpu, ores["O"],
                                                                ores["lse"])
    if summ is not None:
        mn, mx = summ[g]
        f = lambda a: synth.from_bits(a).float().numpy()
        assert np.array_equal(f(mn), f(ores["mn"])), "min summaries differ"
        assert np.array_equal(f(mx), f(ores["mx"])), "max summaries differ"
    r["max_dmaw"] = 0.0
    if maw_state is not None:
        ref = ores["maw"]
        got = maw_gpu[g]
        assert got.shape == ref.shape
        dm = np.abs(got - ref)
        assert np.all(dm <= MAW_ABS + MAW_REL * np.abs(ref)), (
            "MAW differs: max %g" % dm.max())
        r["max_dmaw"] = float(dm.max()) if dm.size else 0.0
        r["maw"] = ref
    return r


def check_units(w, eng, layer, seq_ids, q_bits, K_bits, V_bits, N_of, gpu,
                maw_state=None, units=None, check_summ=True, workers=1):
    """Oracle each (sequence, KV head) unit and compare with the GPU result.
    K_bits/V_bits: dict seq -> [>=N, Hkv, d] uint16.  maw_state: dict
    (seq, g) -> oracle MAW (updated in place) or None.  workers > 1 runs the
    units' oracles in threads (the C oracle releases the GIL).  Returns stats;
    "flagged" counts selected blocks that the oracle's MAW flag ranked first."""
    jobs = []
    for bi, seq in enumerate(seq_ids):
        if units is not None and not any((seq, g) in units for g in range(w.Hkv)):
            continue
        N = N_of[seq]
        summ = summaries_by_head(eng, layer, seq, w, N) if check_summ else None
        maw_gpu = maw_by_head(eng, layer, seq, w, N) if maw_state is not None else None
        for g in range(w.Hkv):
            if units is not None and (seq, g) not in units:
                continue
            jobs.append((seq, bi, g, N, summ, maw_gpu))

    def run(j):
        seq, bi, g, N, summ, maw_gpu = j
        return _check_unit(w, seq, bi, g, N, q_bits, K_bits, V_bits, gpu, summ, maw_gpu,
                           maw_state)

    if workers > 1 and len(jobs) > 1:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(min(workers, len(jobs))) as ex:
            res = list(ex.map(run, jobs))
    else:
        res = [run(j) for j in jobs]
    stats = dict(units=[], ties=0, flagged=0, max_abs=0.0, max_rel=0.0, max_dlse=0.0,
                 max_dmaw=0.0)
    for (seq, bi, g, N, _, _), r in zip(jobs, res):
        for k in ("ties", "flagged"):
            stats[k] += r[k]
        for k in ("max_abs", "max_rel", "max_dlse", "max_dmaw"):
            stats[k] = max(stats[k], r[k])
        if maw_state is not None:
            maw_state[(seq, g)] = r["maw"]
        stats["units"].append((seq, g))
    return stats


def assert_parity(st):
    assert st["max_abs"] <= ABS_TOL, "max |dO| %g > %g" % (st["max_abs"], ABS_TOL)
    assert st["max_rel"] <= REL_TOL, "max rel dO %g > %g" % (st["max_rel"], REL_TOL)
    assert st["max_dlse"] <= LSE_TOL, "max |dlse| %g > %g" % (st["max_dlse"], LSE_TOL)


def run_single_step(w: synth.Workload, seed: int, device="cuda", shuffle_seed=0,
                    chunks=1, N=None, fused=False, units=None, gen_device=None):
    """Prefill N tokens per sequence, one decode step, oracle every unit."""
    N = w.N if N is None else N
    gen_device = gen_device or ("cpu" if w.B * N * w.Hkv * w.d < 2**24 else device)
    x = synth.single_step(w, seed, device=gen_device, N=N)
    K, V, q = x["K"].to(device), x["V"].to(device), x["q"].to(device)
    eng = make_engine(w, N + 64, shuffle_seed=shuffle_seed)
    try:
        prefill(eng, 0, K, V, chunks=chunks)
        seq_ids = list(range(w.B))
        gpu = run_gpu_step(eng, 0, seq_ids, q, fused=fused)
        Kb, Vb = synth.bits(K), synth.bits(V)
        K_bits = {b: Kb[b] for b in range(w.B)}
        V_bits = {b: Vb[b] for b in range(w.B)}
        st = check_units(w, eng, 0, seq_ids, synth.bits(q), K_bits, V_bits,
                         {b: N for b in range(w.B)}, gpu, units=units)
        st["gpu"] = gpu
        return st
    finally:
        eng.close()
