"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these compares the oracle with itself: each check uses a hand-derived
value (tests/golden/hand_cases.json), a closed form, an identity between two
different code paths, a library routine (numpy), or brute force.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "hand_cases.json")))


def b16(x):
    """float array -> bf16 bit patterns (values here are bf16-exact or get
    rounded to nearest even)."""
    return synth.bits(torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16))


def f64(bits_):
    return synth.from_bits(bits_).double().numpy()


def rand_bits(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return synth.bits((torch.randn(*shape, generator=g) * scale).to(torch.bfloat16))


# ---------------------------------------------------------------- hand cases

def test_hand_quest_bound_group_max():
    c = GOLD["quest_bound_group_max"]
    K = b16(c["keys"])
    mn, mx = oracle.summaries(K, c["S"])
    assert np.array_equal(f64(mn), np.array(c["mn"]))
    assert np.array_equal(f64(mx), np.array(c["mx"]))
    Uh, U, u = oracle.score(b16(c["q"]), mn, mx)
    assert np.array_equal(Uh, np.array(c["Uh"]))
    assert np.array_equal(U, np.array(c["U"]))
    assert np.array_equal(u, np.array(c["U"], np.float32))


@pytest.mark.parametrize("case", GOLD["dense_candidates_k"]["cases"],
                         ids=lambda c: "N%d_S%d" % (c["N"], c["S"]))
def test_hand_dense_candidates_k(case):
    N, S, ns, W = case["N"], case["S"], case["n_s"], case["W"]
    assert oracle.dense_count(N, ns, W) == case["n_dense"]
    assert oracle.num_blocks(N, S) == case["n_blk"]
    cand, nc = oracle.candidates(N, S, ns, W)
    assert nc == case["n_cand"] and cand.sum() == nc
    assert oracle.num_selected(N, S, case["ppm"], nc) == case["k"]


def test_hand_softmax_two_tokens():
    c = GOLD["softmax_two_tokens"]
    O, lse = oracle.attend_tokens(b16(c["q"]), b16(c["K"]), b16(c["V"]),
                                  np.arange(2), scale=c["scale"])
    np.testing.assert_allclose(O, np.array(c["O"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-15)
    O2, lse2 = oracle.dense(b16(c["q"]), b16(c["K"]), b16(c["V"]), 2,
                            scale=c["scale"])
    np.testing.assert_allclose(O2, np.array(c["O"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse2, np.array(c["lse"]), rtol=0, atol=1e-15)


def test_hand_lse_fusion():
    c = GOLD["lse_fusion_two_parts"]
    O, lse = oracle.fuse(np.array(c["O_parts"]), np.array(c["lse_parts"]))
    np.testing.assert_allclose(O, c["O"], rtol=0, atol=1e-15)
    assert abs(lse - c["lse"]) < 1e-15
    g = c["large"]   # max subtraction keeps large lse finite
    O, lse = oracle.fuse(np.array(g["O_parts"]), np.array(g["lse_parts"]))
    np.testing.assert_allclose(O, g["O"], rtol=0, atol=1e-12)
    assert abs(lse - g["lse"]) < 1e-9


def test_hand_maw_decay():
    c = GOLD["maw_decay"]
    m = np.zeros(1)
    for want in c["constant_a1_from0"]:
        m = oracle.maw_update(m, np.ones(1), 0.95)
        assert abs(m[0] - want) < 1e-15
    m = np.zeros(1)
    for t, want in enumerate(c["impulse_a1_then0"]):
        m = oracle.maw_update(m, np.ones(1) if t == 0 else np.zeros(1), 0.95)
        assert abs(m[0] - want) < 1e-15


def test_hand_selection_order_flag_and_ties():
    c = GOLD["selection_order"]
    nb = c["N"]
    mn = b16(np.array(c["m"])[:, None])
    mx = b16(np.array(c["M"])[:, None])
    q = b16([[1.0]])
    r = oracle.select(q, mn, mx, c["N"], c["S"], c["n_s"], c["W"], c["ppm"],
                      maw=np.array(c["maw"]), beta=c["beta"])
    assert r["sel"].tolist() == c["sel"]
    r0 = oracle.select(q, mn, mx, c["N"], c["S"], c["n_s"], c["W"], c["ppm"])
    assert r0["sel"].tolist() == c["sel_without_flag"]
    assert nb == 8


# ----------------------------------------------------- P7: summaries (numpy)

@pytest.mark.parametrize("N,S", [(1, 16), (16, 16), (1000, 16), (1024, 32),
                                 (777, 64), (130, 1)])
def test_summaries_match_numpy_minmax(N, S):
    d = 24
    K = rand_bits((N, d), seed=N * 7 + S)
    mn, mx = oracle.summaries(K, S)
    Kf = f64(K)
    nb = -(-N // S)
    assert mn.shape == (nb, d)
    for i in range(nb):
        blk = Kf[i * S:min(N, (i + 1) * S)]
        assert np.array_equal(f64(mn[i]), blk.min(0))
        assert np.array_equal(f64(mx[i]), blk.max(0))


# -------------------------------------- P5/P6: score bound and its closed form

@pytest.mark.parametrize("G,d,S", [(1, 64, 16), (4, 64, 16), (7, 128, 64),
                                   (4, 128, 32)])
def test_score_upper_bound_and_second_form(G, d, S):
    N = 40 * S + 5
    K = rand_bits((N, d), seed=G * 100 + d + S)
    q = rand_bits((G, d), seed=G * 1000 + d + S)
    mn, mx = oracle.summaries(K, S)
    Uh, U, u = oracle.score(q, mn, mx)
    qf, Kf, mnf, mxf = f64(q), f64(K), f64(mn), f64(mx)
    dots = qf @ Kf.T                                   # [G, N]
    nb = mn.shape[0]
    for i in range(nb):
        blk = dots[:, i * S:min(N, (i + 1) * S)]
        # P5: U_h(i) >= max_j q_h . k_j (up to double rounding)
        assert np.all(Uh[:, i] >= blk.max(1) - 1e-9 * (1 + np.abs(blk).max()))
    # P6: sum_c [q_c (m_c+M_c)/2 + |q_c| (M_c-m_c)/2]
    alt = (qf @ ((mnf + mxf) / 2).T) + (np.abs(qf) @ ((mxf - mnf) / 2).T)
    np.testing.assert_allclose(Uh, alt, rtol=1e-12, atol=1e-12)
    # group max and fp32 rounding of the group score
    np.testing.assert_array_equal(U, Uh.max(0))
    np.testing.assert_array_equal(u, U.astype(np.float32))


def test_score_equals_dot_at_block_size_one():
    G, d, N = 3, 32, 50
    K = rand_bits((N, d), seed=5)
    q = rand_bits((G, d), seed=6)
    mn, mx = oracle.summaries(K, 1)
    Uh, _, _ = oracle.score(q, mn, mx)
    np.testing.assert_allclose(Uh, f64(q) @ f64(K).T, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------ P3: brute-force top-k

def _bruteforce_best(keys, cand_idx, k):
    """Lexicographically greatest k-subset by sorted (flag, u, -index) keys."""
    best, best_set = None, None
    for combo in itertools.combinations(cand_idx, k):
        sig = sorted((keys[i] for i in combo), reverse=True)
        if best is None or sig > best:
            best, best_set = sig, combo
    return sorted(best_set)


@pytest.mark.parametrize("seed", range(12))
def test_selection_bruteforce_tiny(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.choice([1, 2, 4]))
    n_s, W = int(rng.integers(0, 3)), int(rng.integers(0, 2 * S + 1))
    N = int(rng.integers(n_s + W + 1, n_s + W + 10 * S + 1))
    d, G = 4, int(rng.integers(1, 4))
    # coarse integer-valued keys force exact score ties
    K = b16(rng.integers(-2, 3, size=(N, d)).astype(np.float32))
    q = b16(rng.integers(-2, 3, size=(G, d)).astype(np.float32))
    mn, mx = oracle.summaries(K, S)
    cand, nc = oracle.candidates(N, S, n_s, W)
    if nc == 0 or nc > 10:
        pytest.skip("candidate count outside brute-force range")
    nb = oracle.num_blocks(N, S)
    maw = rng.choice([0.0, 0.5, 3.0], size=nb)
    beta = float(rng.choice([0.0, 1.0]))
    ppm = int(rng.integers(1, 1_000_001))
    r = oracle.select(q, mn, mx, N, S, n_s, W, ppm, maw=maw, beta=beta)
    k = oracle.num_selected(N, S, ppm, nc)
    assert r["k"] == k == len(r["sel"])
    nd = oracle.dense_count(N, n_s, W)
    keys = {i: (int(oracle.maw_flag(maw[i], nd, beta, S)), float(r["u"][i]), -i)
            for i in range(nb)}
    want = _bruteforce_best(keys, [i for i in range(nb) if cand[i]], k)
    assert r["sel"].tolist() == want


@pytest.mark.parametrize("seed", range(4))
def test_selection_order_statistic_invariant_large(seed):
    rng = np.random.default_rng(100 + seed)
    N, S, n_s, W, d, G = 8192, 16, 4, 64, 64, 4
    K = rand_bits((N, d), seed=200 + seed)
    q = rand_bits((G, d), seed=300 + seed)
    mn, mx = oracle.summaries(K, S)
    nb = oracle.num_blocks(N, S)
    maw = rng.random(nb) * 0.01
    r = oracle.select(q, mn, mx, N, S, n_s, W, 50000, maw=maw, beta=1.0)
    cand, nc = oracle.candidates(N, S, n_s, W)
    nd = oracle.dense_count(N, n_s, W)
    key = lambda i: (oracle.maw_flag(maw[i], nd, 1.0, S), r["u"][i], -i)
    sel = set(r["sel"].tolist())
    assert len(sel) == r["k"] == oracle.num_selected(N, S, 50000, nc)
    assert all(cand[i] for i in sel)
    worst_sel = min(key(i) for i in sel)
    best_uns = max(key(i) for i in range(nb) if cand[i] and i not in sel)
    assert worst_sel > best_uns
    assert np.all(np.diff(r["sel"]) > 0)


def test_selection_exact_token_topk_at_block_size_one():
    """P5: with S=1 the bound is the exact logit, so block top-k is exact
    token top-k over the non-dense tokens (the exact-top-k reference of
    'Learn from the Past', Core claim)."""
    N, d, n_s, W = 300, 32, 4, 16
    K = rand_bits((N, d), seed=11)
    q = rand_bits((1, d), seed=12)
    mn, mx = oracle.summaries(K, 1)
    r = oracle.select(q, mn, mx, N, 1, n_s, W, 100000)
    dots = (f64(q) @ f64(K).T)[0].astype(np.float32)
    idx = np.arange(n_s, N - W)
    order = sorted(idx, key=lambda j: (-dots[j], j))
    k = math.ceil(0.1 * N)
    assert r["sel"].tolist() == sorted(order[:k])


def test_selection_scale_invariant():
    """P9: doubling q (exact in bf16) doubles every bound exactly."""
    N, d, S = 2048, 64, 32
    K = rand_bits((N, d), seed=21)
    q = rand_bits((4, d), seed=22)
    q2 = b16(f64(q) * 2.0)
    mn, mx = oracle.summaries(K, S)
    a = oracle.select(q, mn, mx, N, S, 4, 64, 50000)
    b = oracle.select(q2, mn, mx, N, S, 4, 64, 50000)
    assert a["sel"].tolist() == b["sel"].tolist()


def test_maw_flag_monotone():
    for m in np.linspace(0, 0.2, 41):
        for m2 in np.linspace(m, 0.2, 5):
            assert oracle.maw_flag(m2, 516, 1.0, 32) >= oracle.maw_flag(m, 516, 1.0, 32)
    assert not oracle.maw_flag(1e9, 516, 0.0, 32)


# ------------------------------------------- P1: LSE identity over partitions

@pytest.mark.parametrize("seed", range(8))
def test_lse_fusion_partition_identity(seed):
    rng = np.random.default_rng(seed)
    G, d, N = 3, 32, 200
    K = rand_bits((N, d), seed=400 + seed, scale=2.0)
    V = rand_bits((N, d), seed=500 + seed)
    q = rand_bits((G, d), seed=600 + seed)
    T = np.sort(rng.choice(N, size=int(rng.integers(1, N)), replace=False))
    O, lse = oracle.attend_tokens(q, K, V, T)
    P = int(rng.integers(1, 17))
    lab = rng.integers(0, P, size=T.shape[0])
    if P > 2:
        lab[0] = P - 1          # a singleton part when possible
        lab[lab == P - 1] = np.where(np.arange((lab == P - 1).sum()) == 0, P - 1, 0)
    parts = [T[lab == p] for p in range(P)] + [np.zeros(0, np.int64)]  # + empty
    for h in range(G):
        Op, lp = [], []
        for part in parts:
            o, l = oracle.attend_tokens(q[h:h + 1], K, V, part)
            Op.append(o[0])
            lp.append(l[0])
        Of, lf = oracle.fuse(np.array(Op), np.array(lp))
        np.testing.assert_allclose(Of, O[h], rtol=0, atol=1e-12)
        assert abs(lf - lse[h]) < 1e-12


def test_fuse_all_empty():
    O, lse = oracle.fuse(np.zeros((3, 4)), np.full(3, -np.inf))
    assert lse == -np.inf and np.all(O == 0)


# ---------------------------------- P2/P10: reductions to dense attention

@pytest.mark.parametrize("N,S,n_s,W", [(1000, 16, 4, 64), (4096, 64, 4, 256),
                                       (333, 32, 0, 0), (50, 16, 4, 64)])
def test_full_budget_equals_dense(N, S, n_s, W):
    G, d = 4, 64
    K = rand_bits((N, d), seed=N + 1, scale=1.5)
    V = rand_bits((N, d), seed=N + 2)
    q = rand_bits((G, d), seed=N + 3)
    mn, mx = oracle.summaries(K, S)
    r = oracle.select(q, mn, mx, N, S, n_s, W, 1_000_000)
    a = oracle.attend(q, K, V, N, S, n_s, W, r["sel"])
    assert a["n_tok"] == N
    O, lse = oracle.dense(q, K, V, N)
    np.testing.assert_allclose(a["O"], O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(a["lse"], lse, rtol=0, atol=1e-12)


def test_everything_dense_when_short():
    G, d, N, S, n_s, W = 2, 16, 60, 16, 4, 64
    K, V, q = rand_bits((N, d), 1), rand_bits((N, d), 2), rand_bits((G, d), 3)
    mn, mx = oracle.summaries(K, S)
    r = oracle.select(q, mn, mx, N, S, n_s, W, 50000)
    assert r["k"] == 0
    a = oracle.attend(q, K, V, N, S, n_s, W, r["sel"])
    O, lse = oracle.dense(q, K, V, N)
    np.testing.assert_allclose(a["O"], O, atol=1e-12, rtol=0)
    np.testing.assert_allclose(a["lse"], lse, atol=1e-12, rtol=0)


@pytest.mark.parametrize("N,S,n_s,W", [(2000, 32, 4, 512), (777, 16, 0, 64), (5000, 64, 16, 0)])
def test_streaming_head_attends_dense_set_only(N, S, n_s, W):
    """A head with budget 0 (a streaming head) selects nothing and attends to
    its sinks and recent window only: the oracle's result equals a numpy
    softmax over those tokens."""
    G, d = 4, 64
    K = rand_bits((N, d), seed=N + 11, scale=1.5)
    V = rand_bits((N, d), seed=N + 12)
    q = rand_bits((G, d), seed=N + 13)
    mn, mx = oracle.summaries(K, S)
    r = oracle.select(q, mn, mx, N, S, n_s, W, 0)
    assert r["k"] == 0 and len(r["sel"]) == 0
    a = oracle.attend(q, K, V, N, S, n_s, W, r["sel"])
    tok = np.array(sorted(set(range(min(n_s, N))) | set(range(max(0, N - W), N))))
    assert a["n_tok"] == len(tok)
    s = f64(q) @ f64(K)[tok].T / math.sqrt(d)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    O = (p / p.sum(axis=1, keepdims=True)) @ f64(V)[tok]
    lse = m[:, 0] + np.log(p.sum(axis=1))
    np.testing.assert_allclose(a["O"], O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(a["lse"], lse, rtol=0, atol=1e-12)


def test_single_token():
    d = 16
    K, V, q = rand_bits((1, d), 7), rand_bits((1, d), 8), rand_bits((2, d), 9)
    O, lse = oracle.attend_tokens(q, K, V, np.array([0]))
    np.testing.assert_array_equal(O, np.repeat(f64(V), 2, 0))
    s = (f64(q) @ f64(K)[0]) / math.sqrt(d)
    np.testing.assert_allclose(lse, s, rtol=0, atol=1e-13)


def test_attended_set_is_a_union():
    """R4: a selected block overlapping the window counts its tokens once."""
    G, d, N, S, n_s, W = 1, 8, 100, 16, 4, 40
    K, V, q = rand_bits((N, d), 31), rand_bits((N, d), 32), rand_bits((G, d), 33)
    # block 3 = [48, 64) overlaps the window [60, 100)
    a = oracle.attend(q, K, V, N, S, n_s, W, np.array([3], np.int32))
    assert a["n_tok"] == 4 + 40 + 12
    toks = np.array(sorted(set(range(4)) | set(range(60, 100)) | set(range(48, 64))))
    O, lse = oracle.attend_tokens(q, K, V, toks)
    np.testing.assert_allclose(a["O"], O, atol=1e-15, rtol=0)
    np.testing.assert_allclose(a["lse"], lse, atol=1e-15, rtol=0)


# ------------------------------------------------ P4: MAW closed forms

def test_maw_closed_forms():
    r = 0.95
    m = np.zeros(4)
    a = np.array([0.3, 0.0, 1.0, 0.125])
    for t in range(1, 60):
        m = oracle.maw_update(m, a, r)
        np.testing.assert_allclose(m, a * (1 - r ** t), rtol=1e-12, atol=1e-15)
    m = oracle.maw_update(np.zeros(2), np.array([0.8, 0.0]), r)
    for t in range(2, 40):
        m = oracle.maw_update(m, np.zeros(2), r)
        np.testing.assert_allclose(m, [0.05 * 0.8 * r ** (t - 1), 0.0],
                                   rtol=1e-12, atol=1e-18)


def test_hand_maw_step_frozen_outside_dense():
    c = GOLD["maw_step_frozen_outside_dense"]
    got = oracle.maw_step(np.array(c["maw"]), np.array(c["a"]), c["N"], c["S"],
                          c["n_s"], c["W"], c["r"])
    np.testing.assert_allclose(got, c["want"], rtol=0, atol=1e-15)


def test_hand_dense_mass_two_heads():
    c = GOLD["dense_mass_two_heads"]
    a = oracle.dense_mass(b16(c["q"]), b16(c["K"]), c["N"], c["S"], c["n_s"],
                          c["W"], scale=c["scale"])
    np.testing.assert_allclose(a, c["a"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("N,S,n_s,W", [(2000, 16, 4, 64), (1000, 32, 4, 512),
                                       (777, 64, 0, 100), (300, 16, 40, 0)])
def test_dense_mass_matches_numpy_unequal_heads(N, S, n_s, W):
    """R8 input: per head, the softmax over D alone; summed per block and
    averaged over the heads (numpy, independent of the oracle's code).  The
    heads' queries differ, so their per-block masses differ."""
    G, d = 3, 32
    K = rand_bits((N, d), seed=N + 41, scale=1.5)
    q = rand_bits((G, d), seed=N + 43)
    a = oracle.dense_mass(q, K, N, S, n_s, W)
    tok = np.array(sorted(set(range(min(n_s, N))) | set(range(max(0, N - W), N))))
    s = f64(q) @ f64(K)[tok].T / math.sqrt(d)                # [G, |D|]
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    nb = -(-N // S)
    per_head = np.zeros((G, nb))
    for h in range(G):
        np.add.at(per_head[h], tok // S, p[h])
    want = per_head.mean(axis=0)
    np.testing.assert_allclose(a, want, rtol=0, atol=1e-13)
    assert abs(a.sum() - 1.0) < 1e-12              # conservation over D
    touch = np.zeros(nb, bool)
    touch[tok // S] = True
    assert np.all(a[~touch] == 0.0) and np.all(a[touch] > 0.0)
    # the heads really differ: a per-head mistake would change the result
    assert np.abs(per_head[0] - per_head[1]).max() > 1e-3


def test_maw_step_keeps_blocks_outside_dense():
    """R10: over several steps with the window moving, a block keeps its MAW
    from the step its oldest token leaves D, and blocks wholly inside D
    follow the update."""
    S, n_s, W, r = 16, 4, 64, 0.95
    N0 = 400
    m = np.zeros(oracle.num_blocks(N0, S))
    rng = np.random.default_rng(3)
    for t in range(40):
        N = N0 + t
        nb = oracle.num_blocks(N, S)
        m = np.concatenate([m, np.zeros(nb - m.shape[0])])
        a = rng.random(nb)
        new = oracle.maw_step(m, a, N, S, n_s, W, r)
        for i in range(nb):
            lo, hi = i * S, min(N, (i + 1) * S)
            inside = all(j < n_s or j >= N - W for j in range(lo, hi))
            want = r * m[i] + (1 - r) * a[i] if inside else m[i]
            assert new[i] == want
        m = new


def test_hand_maw_flag_block_size():
    c = GOLD["maw_flag_block_size"]
    for case in c["cases"]:
        assert oracle.maw_flag(case["maw"], c["n_dense"], c["beta"], case["S"]) == case["flag"]


def test_hand_maw_flag_selection_block_size():
    c = GOLD["maw_flag_selection_block_size"]
    S, N = c["S"], c["N"]
    K = b16(np.repeat(np.array(c["v"]), S)[:, None])      # both tokens of block i hold v_i
    mn, mx = oracle.summaries(K, S)
    q = b16([[1.0]])
    r = oracle.select(q, mn, mx, N, S, c["n_s"], c["W"], c["ppm"],
                      maw=np.array(c["maw"]), beta=c["beta"])
    assert r["sel"].tolist() == c["sel"]
    r0 = oracle.select(q, mn, mx, N, S, c["n_s"], c["W"], c["ppm"])
    assert r0["sel"].tolist() == c["sel_without_flag"]


# ---------------------------------------------- P11: generator sanity

def test_generator_logit_normality():
    """z = <q,k>/(|q| sqrt(D)) is N(0, 1/D) for N(0,1) keys (the statistic of
    Fluxion Figure 11)."""
    from scipy import stats
    D = 128
    K = synth.randn((100000, D), 7, 2).float().double().numpy()
    q = synth.randn((D,), 7, 1).float().double().numpy()
    z = K @ q / (np.linalg.norm(q) * math.sqrt(D))
    res = stats.kstest(z * math.sqrt(D), "norm")
    assert res.pvalue > 1e-3


def test_generator_planting_and_sinks():
    w = synth.llama32k()
    w = synth.Workload(**{**w.__dict__, "B": 1, "Hkv": 2, "Hq": 8, "N": 4096,
                          "block_size": [32, 32], "budget_ppm": [50000] * 2})
    x = synth.single_step(w, seed=0)
    assert x["K"].shape == (1, 4096, 2, 128)
    for (b, g), blocks in x["planted"].items():
        assert len(blocks) == round(0.02 * 128)
        assert np.all(blocks > 0) and np.all((blocks + 1) * 32 <= 4096 - 512)
    # sinks scaled x4: larger norm than ordinary rows
    n_sink = x["K"][0, :4].float().norm(dim=-1).mean()
    n_rest = x["K"][0, 600:700].float().norm(dim=-1).mean()
    assert n_sink > 3.0 * n_rest
    # determinism
    y = synth.single_step(w, seed=0)
    assert torch.equal(x["K"], y["K"]) and torch.equal(x["q"], y["q"])


# ------------------------------------ per-query-head selection and attention

@pytest.mark.parametrize("seed", range(10))
def test_select_heads_bruteforce_tiny(seed):
    """Each query head's set is the lexicographic optimum of its own bound:
    brute force over all k-subsets with that head's scores alone."""
    rng = np.random.default_rng(500 + seed)
    S = int(rng.choice([1, 2, 4]))
    n_s, W = int(rng.integers(0, 3)), int(rng.integers(0, 2 * S + 1))
    N = int(rng.integers(n_s + W + 1, n_s + W + 10 * S + 1))
    d, G = 4, 3
    K = b16(rng.integers(-2, 3, size=(N, d)).astype(np.float32))
    q = b16(rng.integers(-2, 3, size=(G, d)).astype(np.float32))
    mn, mx = oracle.summaries(K, S)
    cand, nc = oracle.candidates(N, S, n_s, W)
    if nc == 0 or nc > 10:
        pytest.skip("candidate count outside brute-force range")
    nb = oracle.num_blocks(N, S)
    maw = rng.choice([0.0, 0.5, 3.0], size=nb)
    beta = float(rng.choice([0.0, 1.0]))
    ppm = int(rng.integers(1, 1_000_001))
    sels = oracle.select_heads(q, mn, mx, N, S, n_s, W, ppm, maw=maw, beta=beta)
    k = oracle.num_selected(N, S, ppm, nc)
    Uh, _, _ = oracle.score(q, mn, mx)
    nd = oracle.dense_count(N, n_s, W)
    for h in range(G):
        u = Uh[h].astype(np.float32)
        keys = {i: (int(oracle.maw_flag(maw[i], nd, beta, S)), float(u[i]) + 0.0, -i)
                for i in range(nb)}
        want = _bruteforce_best(keys, [i for i in range(nb) if cand[i]], k)
        assert sels[h].tolist() == want, (h, sels[h].tolist(), want)


def test_select_heads_are_independent():
    """A head's set depends on its own query only; equal rows give the group
    selection (the max over equal bounds is that bound)."""
    N, S, n_s, W, d, G = 3000, 16, 4, 64, 32, 4
    K = rand_bits((N, d), seed=41)
    q = rand_bits((G, d), seed=42)
    mn, mx = oracle.summaries(K, S)
    a = oracle.select_heads(q, mn, mx, N, S, n_s, W, 50000)
    q2 = q.copy()
    q2[1] = rand_bits((1, d), seed=43)[0]
    b = oracle.select_heads(q2, mn, mx, N, S, n_s, W, 50000)
    for h in (0, 2, 3):
        np.testing.assert_array_equal(a[h], b[h])
    assert not np.array_equal(a[1], b[1])
    assert any(not np.array_equal(a[0], a[h]) for h in range(1, G))
    same = np.repeat(q[2:3], G, 0)
    c = oracle.select_heads(same, mn, mx, N, S, n_s, W, 50000)
    g = oracle.select(same, mn, mx, N, S, n_s, W, 50000)
    for h in range(G):
        np.testing.assert_array_equal(c[h], g["sel"])


def test_attend_heads_over_own_token_lists():
    """Head h attends D U tokens(its own blocks): the token list is built here
    from the ranges directly and attended by oracle_attend_tokens; full
    budget equals the independent dense softmax for every head."""
    G, d, N, S, n_s, W = 3, 16, 400, 16, 4, 40
    K, V, q = rand_bits((N, d), 51), rand_bits((N, d), 52), rand_bits((G, d), 53)
    sels = [np.array([2, 7], np.int32), np.array([5], np.int32), np.array([], np.int32)]
    O, lse = oracle.attend_heads(q, K, V, N, S, n_s, W, sels)
    for h in range(G):
        toks = set(range(n_s)) | set(range(N - W, N))
        for b in sels[h]:
            toks |= set(range(b * S, min(N, (b + 1) * S)))
        Oh, lh = oracle.attend_tokens(q[h:h + 1], K, V, np.array(sorted(toks)))
        np.testing.assert_allclose(O[h], Oh[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[h], lh[0], rtol=0, atol=1e-14)
    mn, mx = oracle.summaries(K, S)
    full = oracle.select_heads(q, mn, mx, N, S, n_s, W, 1_000_000)
    O, lse = oracle.attend_heads(q, K, V, N, S, n_s, W, full)
    Od, ld = oracle.dense(q, K, V, N)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ld, rtol=0, atol=1e-12)


# ------------------------------------------ learn-from-the-past tables (blocks)

@pytest.mark.parametrize("case", ["lfps_candidates", "lfps_candidates_slash"])
def test_lfps_candidates_hand_case(case):
    c = GOLD[case]
    inC, n = oracle.lfps_candidates(c["phi_v"], c["phi_s"], c["N"], c["S"], c["n_s"], c["W"],
                                    c["a"])
    assert np.flatnonzero(inC).tolist() == c["want_C"] and n == len(c["want_C"])


def _lfps_case(seed, N, S, n_s, W, G=2, d=8):
    rng = np.random.default_rng(seed)
    nb = oracle.num_blocks(N, S)
    K = rand_bits((N, d), seed=600 + seed)
    q = rand_bits((G, d), seed=700 + seed)
    phi_v = rng.random(nb) * (rng.random(nb) < 0.5)
    phi_s = rng.random(nb) * (rng.random(nb) < 0.3)
    return K, q, phi_v, phi_s


@pytest.mark.parametrize("seed", range(8))
def test_lfps_select_bruteforce_tiny(seed):
    """The selection is the lexicographic optimum of (u desc, index asc) over
    all k-subsets of the table candidates."""
    rng = np.random.default_rng(800 + seed)
    S = int(rng.choice([1, 2, 4]))
    n_s, W = int(rng.integers(0, 3)), int(rng.integers(0, 2 * S + 1))
    N = int(rng.integers(n_s + W + 1, n_s + W + 12 * S + 1))
    K, q, phi_v, phi_s = _lfps_case(seed, N, S, n_s, W, d=4)
    mn, mx = oracle.summaries(K, S)
    inC, nC = oracle.lfps_candidates(phi_v, phi_s, N, S, n_s, W)
    if nC == 0 or nC > 10:
        pytest.skip("candidate count outside brute-force range")
    ppm = int(rng.integers(1, 1_000_001))
    r = oracle.lfps_select(q, mn, mx, N, S, n_s, W, ppm, phi_v, phi_s)
    k = oracle.num_selected(N, S, ppm, nC)
    assert r["k"] == k == len(r["sel"])
    keys = {i: (0, float(r["u"][i]) + 0.0, -i) for i in range(len(inC))}
    assert r["sel"].tolist() == _bruteforce_best(keys, np.flatnonzero(inC).tolist(), k)


def test_lfps_select_equals_block_topk_when_candidates_cover_it():
    """When C holds the plain top-k of all candidates, restricting the ranking
    to C changes nothing."""
    N, S, n_s, W, d, G = 2000, 16, 4, 64, 16, 2
    K = rand_bits((N, d), seed=61)
    q = rand_bits((G, d), seed=62)
    mn, mx = oracle.summaries(K, S)
    nb = oracle.num_blocks(N, S)
    ref = oracle.select(q, mn, mx, N, S, n_s, W, 50000)
    phi_v = np.zeros(nb)
    phi_v[ref["sel"]] = 1.0             # every selected block far above the threshold
    phi_v[(ref["sel"][0] + 5) % nb] = 1.0  # and some other block
    r = oracle.lfps_select(q, mn, mx, N, S, n_s, W, 50000, phi_v, np.zeros(nb))
    np.testing.assert_array_equal(r["sel"], ref["sel"])
    inC, _ = oracle.lfps_candidates(phi_v, np.zeros(nb), N, S, n_s, W)
    assert inC.sum() < oracle.candidates(N, S, n_s, W)[1]


def test_attend_mass_is_the_block_sum_of_the_softmax():
    N, S, n_s, W, d, G = 300, 16, 4, 40, 8, 3
    K, q = rand_bits((N, d), 71), rand_bits((G, d), 72)
    sel = np.array([2, 9], np.int32)
    a = oracle.attend_mass(q, K, N, S, n_s, W, sel)
    toks = sorted(set(range(n_s)) | set(range(N - W, N)) | set(range(32, 48)) | set(range(144, 160)))
    s = f64(q) @ f64(K)[toks].T / math.sqrt(d)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    want = np.zeros(oracle.num_blocks(N, S))
    np.add.at(want, np.array(toks) // S, p.mean(0))
    np.testing.assert_allclose(a, want, rtol=0, atol=1e-14)
    assert abs(a.sum() - 1.0) < 1e-12


def test_lfps_update_closed_forms():
    r, nb = 0.95, 6
    a = np.array([0.1, 0.0, 0.5, 0.0, 0.0, 0.4])
    pv, ps = np.zeros(nb), np.zeros(nb)
    for t in range(1, 40):
        pv, ps = oracle.lfps_update(pv, ps, a, r)
        np.testing.assert_allclose(pv, a * (1 - r ** t), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(ps, a[::-1] * (1 - r ** t), rtol=1e-12, atol=1e-15)
    # an impulse on block 2 with newest block 5 lands on offset 3
    pv, ps = oracle.lfps_update(np.zeros(nb), np.zeros(nb), np.eye(nb)[2], r)
    assert ps.tolist() == [0.0, 0.0, 0.0, (1 - r), 0.0, 0.0]
    # a shorter step (3 blocks) leaves the later entries alone
    pv2, ps2 = oracle.lfps_update(np.ones(nb), np.ones(nb), np.array([0.2, 0.3, 0.5]), r)
    np.testing.assert_allclose(pv2, [r + (1 - r) * 0.2, r + (1 - r) * 0.3, r + (1 - r) * 0.5, 1, 1, 1])
    np.testing.assert_allclose(ps2, [r + (1 - r) * 0.5, r + (1 - r) * 0.3, r + (1 - r) * 0.2, 1, 1, 1])


def test_lfps_init_one_and_two_prefill_positions():
    """Init from the last s prefill positions: each attends causally to every
    earlier token; the masses enter with the decay in order."""
    N, S, d, G, r = 97, 16, 8, 2, 0.95  # the two positions 95, 96 lie in blocks 5 and 6
    K = rand_bits((N, d), 81)
    qp = rand_bits((2, G, d), 82).reshape(2, G, d)
    nb = oracle.num_blocks(N, S)

    def mass(qq, pos):
        s = f64(qq) @ f64(K)[:pos + 1].T / math.sqrt(d)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        out = np.zeros(nb)
        np.add.at(out, np.arange(pos + 1) // S, p.mean(0))
        return out

    pv, ps = oracle.lfps_init(qp[1:], K, N, S, r)
    a1 = mass(qp[1], N - 1)
    np.testing.assert_allclose(pv, (1 - r) * a1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ps[:nb], (1 - r) * a1[::-1], rtol=0, atol=1e-14)
    pv, ps = oracle.lfps_init(qp, K, N, S, r)
    a0 = mass(qp[0], N - 2)
    np.testing.assert_allclose(pv, r * (1 - r) * a0 + (1 - r) * a1, rtol=0, atol=1e-14)
    b0, b1 = (N - 2) // S, (N - 1) // S
    want_s = np.zeros(nb)
    want_s[:b0 + 1] += r * (1 - r) * a0[:b0 + 1][::-1]
    want_s[:b1 + 1] += (1 - r) * a1[:b1 + 1][::-1]
    np.testing.assert_allclose(ps, want_s, rtol=0, atol=1e-14)
