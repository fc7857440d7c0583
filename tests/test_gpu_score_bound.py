"""The approximate block score's error bound, checked block by block on the GPU.

The score tiles compute each block's group score U(i) = max_h sum_c
max(q_hc m_ic, q_hc M_ic) with bf16 MFMAs accumulating in fp32, and a bound
eps from a second MFMA over absolute values; the top-k re-scores exactly every
block whose approximate score lies within the band of the k-th, so the
selection is the exact top-k only if |approx(i) - U(i)| <= eps for every
candidate block ("Learn from the Past: Fast Sparse Indexing for Large
Language Model Decoding", Core claim: the exact top-k is the reference).

Inputs (synth.adversarial) are built to stress that bound: key exponents
spread over 2^+-40 between blocks, blocks whose channel pairs cancel exactly
(exact score 0 with a large magnitude sum; 97% of the blocks, so the k-th
place falls among exact ties at 0, which the index breaks, and the band of
uncertain blocks outgrows the top-k's LDS list), and queries near and below
the smallest normal bf16.  For each
(sequence, KV head) the test reads back the approximate score of every block
and the unit's eps (SD_DEBUG_SCORES), computes U in fp64 from the summaries
the library holds, and checks:
  - the scored blocks are exactly the candidates;
  - |approx - U| <= eps for every one of them, and <= the per-block bound
    2 (gamma_64 + gamma_4) E_i + u |U_i| + 1e-30 that eps is the maximum of
    (E_i = max_h sum_c |q_hc u_hc|, u_hc the summary value the max takes);
  - the selection equals the oracle's (bit-exact, ties by index).
Both call forms run: select_topk, and the one-launch step.  The geometries
take the top-k paths: the fast one (no MAW flags, k <= 64, and with 128-key
lists for 64 < k <= 128), the one-wave full top-k (MAW flags on) and the
four-wave top-k (over 1280 scored blocks).  Attention outputs are not compared: with logits up to
2^49 the softmax is decided by fp32 rounding of the logits, outside the
input domain where the attention tolerances hold.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_sparse_top_score_amd import _abi
from tests.harness import log

pytestmark = pytest.mark.gpu

B, HKV, G, D = 2, 2, 4, 128
N_SINK, WINDOW = 4, 64
U32 = 2.0 ** -24
GAMMA = lambda n: n * U32 / (1 - n * U32)  # noqa: E731


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _bf16(a):
    """uint16 bf16 bit patterns -> float64."""
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _magnitude(q, mn, mx):
    """E_i = max_h sum_c |q_hc u_hc| with u_hc = M_ic for q_hc >= 0, else m_ic."""
    qf, lo, hi = _bf16(q), _bf16(mn), _bf16(mx)
    up = np.where(qf[:, None, :] >= 0, hi[None], lo[None])      # [G][nb][d]
    return np.abs(qf[:, None, :] * up).sum(-1).max(0)


@pytest.mark.parametrize("kind", synth.ADVERSARIAL_KINDS)
@pytest.mark.parametrize("form", ["select", "step"])
@pytest.mark.parametrize("N,S,beta,PPM", [(6000, 16, 0.0, 50_000), (6000, 16, 0.0, 250_000),
                                          (6000, 16, 1.0, 50_000), (30000, 16, 0.0, 50_000)],
                         ids=["fast", "fast128", "one-wave", "four-wave"])
def test_score_bound_and_selection(kind, form, N, S, beta, PPM):
    log("case: score bound kind=%s form=%s N=%d S=%d beta=%g ppm=%d" % (kind, form, N, S, beta, PPM))
    x = synth.adversarial(kind, B, HKV, G, D, N, S, seed=7)
    eng = _abi.SparseDecode(max_seqs=B, num_layers=1, num_q_heads=HKV * G, num_kv_heads=HKV,
                            head_dim=D, num_pages=B * (N // 16 + 2) + 8, max_seq_len=N + 16,
                            sink_tokens=N_SINK, recent_window=WINDOW, block_size=[S] * HKV,
                            budget_ppm=[PPM] * HKV, maw_beta=beta)
    try:
        seqs = list(range(B))
        eng.append_kv(0, seqs, [N] * B, x["K"].reshape(B * N, HKV, D).cuda(),
                      x["V"].reshape(B * N, HKV, D).cuda())
        q = x["q"].cuda()
        bufs = eng.alloc_step(B)
        if form == "select":
            eng.select_topk(0, seqs, q, bufs["blk_idx"], bufs["blk_cnt"])
        else:
            eng.decode_step(0, seqs, q, bufs["blk_idx"], bufs["blk_cnt"], bufs["o_part"],
                            bufs["lse_part"], bufs["o"], bufs["lse"])
        eng.sync()
        blk_idx, blk_cnt = bufs["blk_idx"].cpu().numpy(), bufs["blk_cnt"].cpu().numpy()
        if form == "step":
            assert torch.isfinite(bufs["lse"]).all()
        qb, Kb = synth.bits(x["q"]), synth.bits(x["K"])
        nb = synth.n_blocks(N, S)
        worst, worst_blk, n_checked, ties_at_kth = 0.0, 0.0, 0, 0
        for b in seqs:
            summ = eng.debug(_abi.SD_DEBUG_SUMMARY, 0, b).reshape(HKV, nb, D, 2)
            sc = eng.debug(_abi.SD_DEBUG_SCORES, 0, b).reshape(HKV, nb + 1)
            for h in range(HKV):
                mn, mx = summ[h, ..., 0], summ[h, ..., 1]
                omn, omx = oracle.summaries(np.ascontiguousarray(Kb[b, :, h]), S)
                assert np.array_equal(mn, omn) and np.array_equal(mx, omx), (b, h)
                qg = np.ascontiguousarray(qb[b, h * G:(h + 1) * G])
                _, U, _ = oracle.score(qg, mn, mx)
                eps = float(sc[h, 0])
                approx = sc[h, 1:].astype(np.float64)
                cmask, _ = oracle.candidates(N, S, N_SINK, WINDOW)
                scored = np.flatnonzero(~np.isnan(approx))
                assert np.array_equal(scored, np.flatnonzero(cmask)), (b, h)
                assert np.isfinite(eps) and eps > 0.0, eps
                err = np.abs(approx[scored] - U[scored])
                assert (err <= eps).all(), (b, h, int(scored[np.argmax(err - eps)]),
                                            float(err.max()), eps)
                E = _magnitude(qg, mn, mx)[scored]
                bound = 2 * (GAMMA(64) + GAMMA(4)) * E + U32 * np.abs(U[scored]) + 1e-30
                assert (err <= bound).all(), (b, h, float((err / bound).max()))
                worst = max(worst, float((err / eps).max()))
                worst_blk = max(worst_blk, float((err / bound).max()))
                n_checked += len(scored)
                ref = oracle.select(qg, mn, mx, N, S, N_SINK, WINDOW, PPM,
                                    maw=np.zeros(nb) if beta > 0 else None, beta=beta)
                got = blk_idx[b, h, :blk_cnt[b, h]]
                assert np.array_equal(got, ref["sel"]), (b, h, np.setxor1d(got, ref["sel"])[:8])
                kth = U[ref["sel"]].min() if len(ref["sel"]) else np.nan
                ties_at_kth += int((U[scored] == kth).sum()) - 1 if len(ref["sel"]) else 0
        log("  %d blocks: max |approx - U| / eps = %.3g, / per-block bound = %.3g; "
            "%d other blocks tie with the k-th" % (n_checked, worst, worst_blk, ties_at_kth))
        if kind == "cancel":
            assert ties_at_kth > 0
    finally:
        eng.close()
