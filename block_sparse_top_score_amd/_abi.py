"""ctypes binding of libsparse_decode.so (argument marshalling only).

Every step of the decode path runs in the library's HIP kernels; this module
only converts Python/torch arguments to the C ABI of include/sparse_decode.h.
torch is used for device memory and streams.  If the library has not been
built, loading fails loudly: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_decode.so")
# the measurement build with per-phase timestamps (build.py --timeline)
LIB_TIMELINE_PATH = os.path.join(_HERE, "libsparse_decode_timeline.so")

SD_OK, SD_EINVAL, SD_ENOMEM, SD_EHIP, SD_EUNSUPPORTED, SD_ESTATE = 0, -1, -2, -3, -4, -5
(SD_DEBUG_PAGE_TABLE, SD_DEBUG_SUMMARY, SD_DEBUG_MAW, SD_DEBUG_K, SD_DEBUG_V, SD_DEBUG_SCORES,
 SD_DEBUG_LFPS, SD_DEBUG_LFPS_CAND) = range(8)

# every symbol declared in include/sparse_decode.h
EXPORTS = [
    "sd_validate_config", "sparse_decode_init", "sparse_decode_destroy",
    "sd_caps", "append_kv", "select_topk", "sparse_attend", "fuse_lse",
    "sparse_decode_step", "sparse_decode_step_noalloc", "sd_release_seq", "sd_seq_len",
    "sd_sync",
    "sd_last_error", "sd_debug_bytes", "sd_debug_copy", "sd_debug_set_maw",
    "sd_debug_set_lfps", "sd_lfps_init", "sd_read_probe",
]


class SDError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("sparse_decode status %d: %s" % (status, msg))
        self.status = status


class SDConfig(ctypes.Structure):
    _fields_ = [
        ("max_seqs", ctypes.c_int32), ("num_layers", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("sink_tokens", ctypes.c_int32), ("recent_window", ctypes.c_int32),
        ("block_size", ctypes.POINTER(ctypes.c_int32)),
        ("budget_ppm", ctypes.POINTER(ctypes.c_int32)),
        ("softmax_scale", ctypes.c_float), ("maw_decay", ctypes.c_float),
        ("maw_beta", ctypes.c_float), ("page_shuffle_seed", ctypes.c_uint64),
        ("stream", ctypes.c_void_p), ("select_per_query_head", ctypes.c_int32),
        ("lfps_select", ctypes.c_int32), ("lfps_a", ctypes.c_float),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime; when torch is used for memory and
    # streams it must be loaded first so that the library binds to the same
    # runtime instance (one device context, valid stream handles).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(
            "libsparse_decode.so is not built (%s); run __graft_entry__.build() "
            "or python block_sparse_top_score_amd/build.py" % path)
    L = ctypes.CDLL(path)
    P, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    cfgp = ctypes.POINTER(SDConfig)
    sig = {
        "sd_validate_config": (i32, [cfgp, ctypes.c_char_p, sz]),
        "sparse_decode_init": (i32, [cfgp, ctypes.POINTER(P)]),
        "sparse_decode_destroy": (i32, [P]),
        "sd_caps": (i32, [P, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "append_kv": (i32, [P, i32, i32, P, P, P, P]),
        "select_topk": (i32, [P, i32, i32, P, P, P, P, i32]),
        "sparse_attend": (i32, [P, i32, i32, P, P, P, P, i32, P, P, i32]),
        "fuse_lse": (i32, [P, i32, i32, P, P, P, i32, P, P]),
        "sparse_decode_step": (i32, [P, i32, i32, P, P, P, P, P, P, i32, P, P, i32, P, P]),
        "sparse_decode_step_noalloc": (i32, [P, i32, i32, P, P, P, P, P, P, i32, P, P, i32, P, P]),
        "sd_release_seq": (i32, [P, i32]),
        "sd_seq_len": (i32, [P, i32, i32, ctypes.POINTER(i32)]),
        "sd_sync": (i32, [P]),
        "sd_last_error": (ctypes.c_char_p, [P]),
        "sd_debug_bytes": (i32, [P, i32, i32, i32, ctypes.POINTER(sz)]),
        "sd_debug_copy": (i32, [P, i32, i32, i32, P, sz]),
        "sd_debug_set_maw": (i32, [P, i32, i32, P, sz]),
        "sd_debug_set_lfps": (i32, [P, i32, i32, P, sz]),
        "sd_lfps_init": (i32, [P, i32, i32, P, P, i32]),
        "sd_read_probe": (i32, [P, sz, P, i32, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def make_config(*, max_seqs, num_layers, num_q_heads, num_kv_heads, head_dim,
                num_pages, max_seq_len, sink_tokens, recent_window,
                block_size: Sequence[int], budget_ppm: Sequence[int],
                softmax_scale=0.0, maw_decay=0.95, maw_beta=0.0,
                page_shuffle_seed=0, stream=None, page_size=16,
                select_per_query_head=0, lfps_select=0, lfps_a=0.2):
    bs = (ctypes.c_int32 * len(block_size))(*block_size)
    bp = (ctypes.c_int32 * len(budget_ppm))(*budget_ppm)
    cfg = SDConfig(max_seqs, num_layers, num_q_heads, num_kv_heads, head_dim,
                   page_size, num_pages, max_seq_len, sink_tokens,
                   recent_window, ctypes.cast(bs, ctypes.POINTER(ctypes.c_int32)),
                   ctypes.cast(bp, ctypes.POINTER(ctypes.c_int32)),
                   float(softmax_scale), float(maw_decay), float(maw_beta),
                   int(page_shuffle_seed), stream, int(select_per_query_head),
                   int(lfps_select), float(lfps_a))
    cfg._keep = (bs, bp)  # keep the arrays alive with the struct
    return cfg


def validate_config(cfg: SDConfig):
    """Host-only check; returns (status, message)."""
    L = load()
    buf = ctypes.create_string_buffer(256)
    st = L.sd_validate_config(ctypes.byref(cfg), buf, 256)
    return st, buf.value.decode()


def _i32arr(xs):
    a = np.ascontiguousarray(np.asarray(xs, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class SparseDecode:
    """One library context on the current torch device and stream."""

    def __init__(self, *, stream=None, **cfg_kwargs):
        import torch
        self.torch = torch
        self.L = load()
        if stream is None:
            stream = torch.cuda.current_stream()
        self.stream = stream
        cfg_kwargs["stream"] = ctypes.c_void_p(stream.cuda_stream)
        self.cfg = make_config(**cfg_kwargs)
        self.ctx = ctypes.c_void_p()
        st = self.L.sparse_decode_init(ctypes.byref(self.cfg), ctypes.byref(self.ctx))
        if st != SD_OK:
            msg = self.error()
            if self.ctx:
                self.L.sparse_decode_destroy(self.ctx)
                self.ctx = ctypes.c_void_p()
            raise SDError(st, msg)
        self.Hq = self.cfg.num_q_heads
        self.Hkv = self.cfg.num_kv_heads
        self.pqh = bool(self.cfg.select_per_query_head)
        self.sel_heads = self.Hq if self.pqh else self.Hkv  # rows of blk_idx per sequence
        self.d = self.cfg.head_dim
        k, p = ctypes.c_int32(), ctypes.c_int32()
        self.L.sd_caps(self.ctx, ctypes.byref(k), ctypes.byref(p))
        self.k_cap, self.p_cap = k.value, p.value

    # -- helpers ------------------------------------------------------------
    def error(self):
        return self.L.sd_last_error(self.ctx).decode() if self.ctx else "no context"

    def _check(self, st):
        if st != SD_OK:
            raise SDError(st, self.error())

    def close(self):
        if self.ctx:
            st = self.L.sparse_decode_destroy(self.ctx)
            self.ctx = ctypes.c_void_p()
            if st != SD_OK:
                raise SDError(st, "destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- ABI calls ----------------------------------------------------------
    def append_kv(self, layer, seq_ids, n_new, k, v, check=True):
        s, sp = _i32arr(seq_ids)
        n, np_ = _i32arr(n_new)
        st = self.L.append_kv(self.ctx, layer, len(s), sp, np_, _ptr(k), _ptr(v))
        if check:
            self._check(st)
        return st

    def select_topk(self, layer, seq_ids, q, blk_idx, blk_cnt, k_cap=None, check=True):
        s, sp = _i32arr(seq_ids)
        k_cap = blk_idx.shape[-1] if k_cap is None else k_cap
        st = self.L.select_topk(self.ctx, layer, len(s), sp, _ptr(q), _ptr(blk_idx),
                                _ptr(blk_cnt), k_cap)
        if check:
            self._check(st)
        return st

    def sparse_attend(self, layer, seq_ids, q, blk_idx, blk_cnt, o_part, lse_part,
                      k_cap=None, p_cap=None, check=True):
        s, sp = _i32arr(seq_ids)
        k_cap = blk_idx.shape[-1] if k_cap is None else k_cap
        p_cap = lse_part.shape[-1] if p_cap is None else p_cap
        st = self.L.sparse_attend(self.ctx, layer, len(s), sp, _ptr(q), _ptr(blk_idx),
                                  _ptr(blk_cnt), k_cap, _ptr(o_part), _ptr(lse_part),
                                  p_cap)
        if check:
            self._check(st)
        return st

    def fuse_lse(self, layer, seq_ids, o_part, lse_part, o, lse, n_seqs=None,
                 p_cap=None, check=True):
        if seq_ids is None:
            sp = None
            n = o.shape[0] if n_seqs is None else n_seqs
        else:
            s, sp = _i32arr(seq_ids)
            n = len(s)
        p_cap = lse_part.shape[-1] if p_cap is None else p_cap
        st = self.L.fuse_lse(self.ctx, layer, n, sp, _ptr(o_part), _ptr(lse_part),
                             p_cap, _ptr(o), _ptr(lse))
        if check:
            self._check(st)
        return st

    def decode_step(self, layer, seq_ids, q, blk_idx, blk_cnt, o_part, lse_part, o,
                    lse, k_new=None, v_new=None, check=True):
        """Fused step; k_new/v_new ([n][Hkv][d] bf16) append one token first."""
        s, sp = _i32arr(seq_ids)
        st = self.L.sparse_decode_step(self.ctx, layer, len(s), sp, _ptr(k_new),
                                       _ptr(v_new), _ptr(q),
                                       _ptr(blk_idx), _ptr(blk_cnt), blk_idx.shape[-1],
                                       _ptr(o_part), _ptr(lse_part), lse_part.shape[-1],
                                       _ptr(o), _ptr(lse))
        if check:
            self._check(st)
        return st

    def decode_step_noalloc(self, layer, seq_ids, q, blk_idx, blk_cnt, o_part, lse_part, o,
                            lse, k_new=None, v_new=None, check=True):
        """sparse_decode_step_noalloc: the fused step with its scratch in the
        library's static device array (allocates nothing)."""
        s, sp = _i32arr(seq_ids)
        st = self.L.sparse_decode_step_noalloc(self.ctx, layer, len(s), sp, _ptr(k_new),
                                               _ptr(v_new), _ptr(q),
                                               _ptr(blk_idx), _ptr(blk_cnt), blk_idx.shape[-1],
                                               _ptr(o_part), _ptr(lse_part), lse_part.shape[-1],
                                               _ptr(o), _ptr(lse))
        if check:
            self._check(st)
        return st

    def release_seq(self, seq):
        self._check(self.L.sd_release_seq(self.ctx, seq))

    def seq_len(self, layer, seq):
        x = ctypes.c_int32()
        self._check(self.L.sd_seq_len(self.ctx, layer, seq, ctypes.byref(x)))
        return x.value

    def sync(self):
        self._check(self.L.sd_sync(self.ctx))

    def debug(self, what, layer, seq):
        """Host numpy copy of a debug export (see sd_debug_copy)."""
        nb = ctypes.c_size_t()
        self._check(self.L.sd_debug_bytes(self.ctx, what, layer, seq, ctypes.byref(nb)))
        dt = {SD_DEBUG_PAGE_TABLE: np.int32, SD_DEBUG_MAW: np.float32,
              SD_DEBUG_SCORES: np.float32, SD_DEBUG_LFPS: np.float32,
              SD_DEBUG_LFPS_CAND: np.int32}.get(what, np.uint16)
        out = np.zeros(nb.value // np.dtype(dt).itemsize, dt)
        self._check(self.L.sd_debug_copy(self.ctx, what, layer, seq,
                                         out.ctypes.data_as(ctypes.c_void_p), nb.value))
        return out

    def set_lfps(self, layer, seq, values):
        """Overwrite the tables of one (layer, sequence), laid out as SD_DEBUG_LFPS."""
        a = np.ascontiguousarray(values, dtype=np.float32)
        self._check(self.L.sd_debug_set_lfps(self.ctx, layer, seq,
                                             a.ctypes.data_as(ctypes.c_void_p), a.nbytes))

    def lfps_init(self, layer, seq_ids, q_prefill, check=True):
        """sd_lfps_init: q_prefill [n][s][Hq][d] bf16 (device)."""
        s, sp = _i32arr(seq_ids)
        st = self.L.sd_lfps_init(self.ctx, layer, len(s), sp, _ptr(q_prefill), q_prefill.shape[1])
        if check:
            self._check(st)
        return st

    def set_maw(self, layer, seq, values):
        a = np.ascontiguousarray(values, dtype=np.float32)
        self._check(self.L.sd_debug_set_maw(self.ctx, layer, seq,
                                            a.ctypes.data_as(ctypes.c_void_p), a.nbytes))

    # -- allocation helpers (torch device memory) ---------------------------
    def alloc_step(self, n_seqs, device="cuda"):
        t = self.torch
        blk_idx = t.full((n_seqs, self.sel_heads, self.k_cap), -1, dtype=t.int32, device=device)
        blk_cnt = t.zeros((n_seqs, self.sel_heads), dtype=t.int32, device=device)
        o_part = t.empty((n_seqs, self.Hq, self.p_cap, self.d), dtype=t.float32, device=device)
        lse_part = t.empty((n_seqs, self.Hq, self.p_cap), dtype=t.float32, device=device)
        o = t.empty((n_seqs, self.Hq, self.d), dtype=t.float32, device=device)
        lse = t.empty((n_seqs, self.Hq), dtype=t.float32, device=device)
        return dict(blk_idx=blk_idx, blk_cnt=blk_cnt, o_part=o_part, lse_part=lse_part,
                    o=o, lse=lse)


def timeline_read(n_wg):
    """Timestamps of the last steps from the measurement build (loaded with
    load(LIB_TIMELINE_PATH)): uint64 [n_wg][slots]; the table is then zeroed."""
    L = load()
    if not hasattr(L, "sd_timeline_read"):
        raise RuntimeError("the loaded library is not the timeline build")
    L.sd_timeline_read.restype = ctypes.c_int32
    L.sd_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    slots, max_wg = ctypes.c_int32(), ctypes.c_int32()
    L.sd_timeline_read(None, 0, ctypes.byref(slots), ctypes.byref(max_wg))
    n_wg = min(n_wg, max_wg.value)
    out = np.zeros((n_wg, slots.value), np.uint64)
    st = L.sd_timeline_read(out.ctypes.data_as(ctypes.c_void_p), out.nbytes, None, None)
    if st != SD_OK:
        raise SDError(st, "sd_timeline_read")
    return out
