"""Plain double-precision CPU oracle (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and shares no code with it.

This module is a thin ctypes wrapper over ``liboracle.so`` (built from
``oracle.c`` with gcc) that takes numpy arrays.  bf16 tensors are passed as
their raw 16-bit patterns (``numpy.uint16``).  All arithmetic is in
``oracle.c``; the helpers here only marshal arguments.

Parity status: see the header comment of ``oracle.c``.  The group max (R1),
block-level MAW (R8), the beta/|D| flag scale (R9) and the flag-then-score
order (R11) are readings the pages do not fix; pins tie the oracle to them.

``ORACLE_LIB`` in the environment names another build of ``oracle.c`` to load
instead (used only by the mutation sweep in ``tests/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB") or _LIB_PATH
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(path)
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        P = ctypes.c_void_p
        L.oracle_num_blocks.restype = i64
        L.oracle_num_blocks.argtypes = [i64, i32]
        L.oracle_dense_count.restype = i64
        L.oracle_dense_count.argtypes = [i64, i32, i32]
        L.oracle_in_dense.restype = i32
        L.oracle_in_dense.argtypes = [i64, i64, i32, i32]
        L.oracle_candidates.restype = i64
        L.oracle_candidates.argtypes = [i64, i32, i32, i32, P]
        L.oracle_num_selected.restype = i64
        L.oracle_num_selected.argtypes = [i64, i32, i64, i64]
        L.oracle_summaries.restype = None
        L.oracle_summaries.argtypes = [P, i64, i64, i32, i32, P, P]
        L.oracle_score.restype = None
        L.oracle_score.argtypes = [P, i32, i32, P, P, i64, P, P, P]
        L.oracle_maw_flag.restype = i32
        L.oracle_maw_flag.argtypes = [dbl, i64, dbl, i32]
        L.oracle_select.restype = i64
        L.oracle_select.argtypes = [P, i32, i32, P, P, i64, i32, i32, i32, i64,
                                    P, dbl, P, P, P, P]
        L.oracle_select_heads.restype = i64
        L.oracle_select_heads.argtypes = [P, i32, i32, P, P, i64, i32, i32, i32, i64,
                                          P, dbl, P, i64]
        L.oracle_attend_heads.restype = None
        L.oracle_attend_heads.argtypes = [P, i32, i32, P, i64, P, i64, i64, i32, i32,
                                          i32, P, i64, P, dbl, P, P]
        L.oracle_lfps_candidates.restype = i64
        L.oracle_lfps_candidates.argtypes = [P, P, i64, i32, i32, i32, dbl, P]
        L.oracle_lfps_select.restype = i64
        L.oracle_lfps_select.argtypes = [P, i32, i32, P, P, i64, i32, i32, i32, i64,
                                         P, P, dbl, P, P, P]
        L.oracle_attend_mass.restype = None
        L.oracle_attend_mass.argtypes = [P, i32, i32, P, i64, i64, i32, i32, i32, P, i64,
                                         dbl, P]
        L.oracle_lfps_update.restype = None
        L.oracle_lfps_update.argtypes = [P, P, P, i64, dbl]
        L.oracle_lfps_init.restype = None
        L.oracle_lfps_init.argtypes = [P, i32, i32, i32, P, i64, i64, i32, dbl, dbl, P, P]
        L.oracle_attend_tokens.restype = None
        L.oracle_attend_tokens.argtypes = [P, i32, i32, P, i64, P, i64, P, i64,
                                           dbl, P, P, P]
        L.oracle_attend.restype = i64
        L.oracle_attend.argtypes = [P, i32, i32, P, i64, P, i64, i64, i32, i32,
                                    i32, P, i64, dbl, P, P]
        L.oracle_dense_mass.restype = None
        L.oracle_dense_mass.argtypes = [P, i32, i32, P, i64, i64, i32, i32, i32,
                                        dbl, P]
        L.oracle_dense.restype = None
        L.oracle_dense.argtypes = [P, i32, i32, P, i64, P, i64, i64, dbl, P, P]
        L.oracle_fuse.restype = None
        L.oracle_fuse.argtypes = [i64, i32, P, P, P, P]
        L.oracle_maw_update.restype = None
        L.oracle_maw_update.argtypes = [P, P, i64, dbl]
        L.oracle_maw_step.restype = None
        L.oracle_maw_step.argtypes = [P, P, i64, i32, i32, i32, dbl]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def num_blocks(N, S):
    return int(lib().oracle_num_blocks(N, S))


def dense_count(N, n_s, W):
    return int(lib().oracle_dense_count(N, n_s, W))


def in_dense(j, N, n_s, W):
    return bool(lib().oracle_in_dense(j, N, n_s, W))


def candidates(N, S, n_s, W):
    nb = num_blocks(N, S)
    cand = np.zeros(max(nb, 1), np.int8)
    n = lib().oracle_candidates(N, S, n_s, W, _p(cand))
    return cand[:nb].astype(bool), int(n)


def num_selected(N, S, budget_ppm, n_cand):
    return int(lib().oracle_num_selected(N, S, budget_ppm, n_cand))


def summaries(K, S):
    """K: [N, d] uint16 (bf16 bits) -> (mn, mx) [n_blk, d] uint16."""
    K = _u16(K)
    N, d = K.shape
    nb = num_blocks(N, S)
    mn = np.zeros((max(nb, 1), d), np.uint16)
    mx = np.zeros((max(nb, 1), d), np.uint16)
    lib().oracle_summaries(_p(K), d, N, d, S, _p(mn), _p(mx))
    return mn[:nb], mx[:nb]


def score(q, mn, mx):
    """q: [G, d]; mn, mx: [n_blk, d] -> (Uh [G, n_blk], U [n_blk], u fp32)."""
    q, mn, mx = _u16(q), _u16(mn), _u16(mx)
    G, d = q.shape
    nb = mn.shape[0]
    Uh = np.zeros((G, max(nb, 1)), np.float64)
    U = np.zeros(max(nb, 1), np.float64)
    u = np.zeros(max(nb, 1), np.float32)
    lib().oracle_score(_p(q), G, d, _p(mn), _p(mx), nb, _p(Uh), _p(U), _p(u))
    return Uh[:, :nb], U[:nb], u[:nb]


def maw_flag(maw, n_dense, beta, S):
    return bool(lib().oracle_maw_flag(maw, n_dense, beta, S))


def select(q, mn, mx, N, S, n_s, W, budget_ppm, maw=None, beta=0.0):
    """Returns dict(sel ascending int32, U, u, flag)."""
    q, mn, mx = _u16(q), _u16(mn), _u16(mx)
    G, d = q.shape
    nb = num_blocks(N, S)
    assert mn.shape == (nb, d) and mx.shape == (nb, d)
    sel = np.zeros(max(nb, 1), np.int32)
    U = np.zeros(max(nb, 1), np.float64)
    u = np.zeros(max(nb, 1), np.float32)
    flag = np.zeros(max(nb, 1), np.int8)
    mw = None
    if maw is not None:
        mw = np.ascontiguousarray(maw, dtype=np.float64)
        assert mw.shape[0] >= nb
    k = lib().oracle_select(_p(q), G, d, _p(mn), _p(mx), N, S, n_s, W,
                            int(budget_ppm), _p(mw), float(beta), _p(sel),
                            _p(U), _p(u), _p(flag))
    return dict(sel=sel[:k].copy(), U=U[:nb], u=u[:nb],
                flag=flag[:nb].astype(bool), k=int(k))


def select_heads(q, mn, mx, N, S, n_s, W, budget_ppm, maw=None, beta=0.0):
    """Per-query-head selection: list of G ascending int32 arrays."""
    q, mn, mx = _u16(q), _u16(mn), _u16(mx)
    G, d = q.shape
    nb = num_blocks(N, S)
    assert mn.shape == (nb, d) and mx.shape == (nb, d)
    ld = max(nb, 1)
    sel = np.zeros((G, ld), np.int32)
    mw = None
    if maw is not None:
        mw = np.ascontiguousarray(maw, dtype=np.float64)
        assert mw.shape[0] >= nb
    k = lib().oracle_select_heads(_p(q), G, d, _p(mn), _p(mx), N, S, n_s, W,
                                  int(budget_ppm), _p(mw), float(beta), _p(sel), ld)
    return [sel[h, :k].copy() for h in range(G)]


def attend_heads(q, K, V, N, S, n_s, W, sels, scale=None):
    """Per-query-head attention: head h over D U blocks(sels[h])."""
    q, K, V = _u16(q), _u16(K), _u16(V)
    G, d = q.shape
    assert len(sels) == G
    ld = max([1] + [len(s) for s in sels])
    sel = np.zeros((G, ld), np.int32)
    k = np.zeros(G, np.int64)
    for h, s in enumerate(sels):
        sel[h, :len(s)] = s
        k[h] = len(s)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.zeros((G, d), np.float64)
    lse = np.zeros(G, np.float64)
    lib().oracle_attend_heads(_p(q), G, d, _p(K), K.shape[1], _p(V), V.shape[1],
                              N, S, n_s, W, _p(sel), ld, _p(k), float(scale),
                              _p(O), _p(lse))
    return O, lse


def _f64(a, n):
    a = np.ascontiguousarray(a, dtype=np.float64)
    assert a.shape[0] >= n
    return a


def lfps_candidates(phi_v, phi_s, N, S, n_s, W, a=0.2):
    """Block mask of the table candidates C and |C|."""
    nb = num_blocks(N, S)
    pv, ps = _f64(phi_v, nb), _f64(phi_s, nb)
    inC = np.zeros(max(nb, 1), np.int8)
    n = lib().oracle_lfps_candidates(_p(pv), _p(ps), N, S, n_s, W, float(a), _p(inC))
    return inC[:nb].astype(bool), int(n)


def lfps_select(q, mn, mx, N, S, n_s, W, budget_ppm, phi_v, phi_s, a=0.2):
    """Selection among the table candidates: dict(sel, U, u, k)."""
    q, mn, mx = _u16(q), _u16(mn), _u16(mx)
    G, d = q.shape
    nb = num_blocks(N, S)
    assert mn.shape == (nb, d) and mx.shape == (nb, d)
    pv, ps = _f64(phi_v, nb), _f64(phi_s, nb)
    sel = np.zeros(max(nb, 1), np.int32)
    U = np.zeros(max(nb, 1), np.float64)
    u = np.zeros(max(nb, 1), np.float32)
    k = lib().oracle_lfps_select(_p(q), G, d, _p(mn), _p(mx), N, S, n_s, W, int(budget_ppm),
                                 _p(pv), _p(ps), float(a), _p(sel), _p(U), _p(u))
    return dict(sel=sel[:k].copy(), U=U[:nb], u=u[:nb], k=int(k))


def attend_mass(q, K, N, S, n_s, W, sel, scale=None):
    """Per-block mass under the softmax over D U blocks(sel), group mean."""
    q, K = _u16(q), _u16(K)
    G, d = q.shape
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nb = num_blocks(N, S)
    a = np.zeros(max(nb, 1), np.float64)
    lib().oracle_attend_mass(_p(q), G, d, _p(K), K.shape[1], N, S, n_s, W, _p(sel),
                             sel.shape[0], float(scale), _p(a))
    return a[:nb]


def lfps_update(phi_v, phi_s, a_blk, r=0.95):
    """Copies of the tables after one step's update (n_blk = len(a_blk))."""
    nb = len(a_blk)
    pv, ps = _f64(phi_v, nb).copy(), _f64(phi_s, nb).copy()
    a = np.ascontiguousarray(a_blk, dtype=np.float64)
    lib().oracle_lfps_update(_p(pv), _p(ps), _p(a), nb, float(r))
    return pv, ps


def lfps_init(q_prefill, K, N, S, r=0.95, scale=None):
    """Tables [n_blk] from the last s prefill positions (q_prefill: [s][G][d])."""
    q, K = _u16(q_prefill), _u16(K)
    s_, G, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nb = num_blocks(N, S)
    pv = np.zeros(max(nb, 1), np.float64)
    ps = np.zeros(max(nb, 1), np.float64)
    lib().oracle_lfps_init(_p(q), s_, G, d, _p(K), K.shape[1], N, S, float(scale), float(r),
                           _p(pv), _p(ps))
    return pv[:nb], ps[:nb]


def attend_tokens(q, K, V, tok, scale=None, want_p=False):
    q, K, V = _u16(q), _u16(K), _u16(V)
    G, d = q.shape
    tok = np.ascontiguousarray(tok, dtype=np.int64)
    n = tok.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.zeros((G, d), np.float64)
    lse = np.zeros(G, np.float64)
    p = np.zeros((G, max(n, 1)), np.float64) if want_p else None
    lib().oracle_attend_tokens(_p(q), G, d, _p(K), K.shape[1], _p(V),
                               V.shape[1], _p(tok), n, float(scale), _p(O),
                               _p(lse), _p(p))
    if want_p:
        return O, lse, p[:, :n]
    return O, lse


def attend(q, K, V, N, S, n_s, W, sel, scale=None):
    """Attention over D U blocks(sel).  K, V: [>=N, d] (row j = token j)."""
    q, K, V = _u16(q), _u16(K), _u16(V)
    G, d = q.shape
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.zeros((G, d), np.float64)
    lse = np.zeros(G, np.float64)
    nt = lib().oracle_attend(_p(q), G, d, _p(K), K.shape[1], _p(V), V.shape[1],
                             N, S, n_s, W, _p(sel), sel.shape[0], float(scale),
                             _p(O), _p(lse))
    return dict(O=O, lse=lse, n_tok=int(nt))


def dense_mass(q, K, N, S, n_s, W, scale=None):
    """MAW input per block: group-mean mass under the softmax over D alone."""
    q, K = _u16(q), _u16(K)
    G, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nb = num_blocks(N, S)
    a = np.zeros(max(nb, 1), np.float64)
    lib().oracle_dense_mass(_p(q), G, d, _p(K), K.shape[1], N, S, n_s, W,
                            float(scale), _p(a))
    return a[:nb]


def dense(q, K, V, N, scale=None):
    q, K, V = _u16(q), _u16(K), _u16(V)
    G, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.zeros((G, d), np.float64)
    lse = np.zeros(G, np.float64)
    lib().oracle_dense(_p(q), G, d, _p(K), K.shape[1], _p(V), V.shape[1], N,
                       float(scale), _p(O), _p(lse))
    return O, lse


def fuse(O_parts, lse_parts):
    O_parts = np.ascontiguousarray(O_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    P, d = O_parts.shape
    O = np.zeros(d, np.float64)
    lse = np.zeros(1, np.float64)
    lib().oracle_fuse(P, d, _p(O_parts), _p(lse_parts), _p(O), _p(lse))
    return O, float(lse[0])


def maw_update(maw, a, r=0.95):
    """Returns the updated copy."""
    m = np.array(maw, dtype=np.float64, copy=True)
    a = np.ascontiguousarray(a, dtype=np.float64)
    assert a.shape == m.shape
    lib().oracle_maw_update(_p(m), _p(a), m.shape[0], float(r))
    return m


def maw_step(maw, a, N, S, n_s, W, r=0.95):
    """One MAW step of a unit (blocks wholly inside D only); the updated copy."""
    m = np.array(maw, dtype=np.float64, copy=True)
    a = np.ascontiguousarray(a, dtype=np.float64)
    assert a.shape == m.shape == (num_blocks(N, S),)
    lib().oracle_maw_step(_p(m), _p(a), N, S, n_s, W, float(r))
    return m


def unit_step(q, K, V, N, S, n_s, W, budget_ppm, maw=None, beta=0.0,
              r=0.95, scale=None, sel_override=None):
    """One decode step of one (sequence, KV head) unit, in the pages' order:
    summaries -> scores and selection -> attention over D U Sel -> MAW (fed
    by the dense partial's per-block mass; blocks not wholly inside D keep
    theirs).

    sel_override lets a lockstep test continue from another legal selection
    (a tie inside the stated band).  Returns a dict with sel, O, lse, U, u,
    flag, k and (when maw is given) the updated maw.
    """
    nb = num_blocks(N, S)
    m = None
    if maw is not None:
        # blocks created since the last step start at 0 (R10)
        m = np.zeros(nb, np.float64)
        src = np.asarray(maw, np.float64)[:nb]
        m[:src.shape[0]] = src
    mn, mx = summaries(K[:N], S)
    sres = select(q, mn, mx, N, S, n_s, W, budget_ppm, maw=m, beta=beta)
    sel = sres["sel"] if sel_override is None else np.asarray(sel_override,
                                                               np.int32)
    ares = attend(q, K, V, N, S, n_s, W, sel, scale=scale)
    out = dict(sres)
    out.update(sel=sel, O=ares["O"], lse=ares["lse"], mn=mn, mx=mx,
               n_tok=ares["n_tok"], oracle_sel=sres["sel"])
    if m is not None:
        a = dense_mass(q, K, N, S, n_s, W, scale=scale)
        out["a"] = a
        out["maw_before"] = m
        out["maw"] = maw_step(m, a, N, S, n_s, W, r)
    return out
