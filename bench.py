"""Throughput of the decode-step block-sparse top-score attention path on one
MI355X, on the Llama-3-8B-shaped 32K workload (B=8, 32 query / 8 KV heads,
d=128, N=32768, block 32, budget 5% of tokens, 4 sinks + 512 recent tokens).

One step = the whole hot path for one layer of one decode step: append the
step's token to every sequence (k_prep), then score + top-k select, split-K
attention over dense and selected chunks, LSE fusion and the MAW update
(k_step, one launch).  Steps rotate over --layers independent layer instances
(8 x 1.07 GB of KV) so that the ~105 MB per-step working set is not served
from the 256 MB last-level cache.  Inputs are resident in HBM when the timed
region starts.

Prints ONE JSON line (rank 0, N=1).  The `roofline` object covers the
dominant kernel, k_step: its algorithmic bytes per launch over its mean
duration, from HIP events on the library's stream around 64 back-to-back
step launches without append (k_step alone, same workload, rotating over the
layer instances); `traffic` is the HBM traffic per
launch from the committed FETCH_SIZE/WRITE_SIZE counter summary, null once the
kernel sources differ from those it was taken on.  `cpu_baseline` times the
CPU oracle (select + attend on precomputed summaries) on the last timed step's
inputs, on all host threads and on one; `parity` compares that step's GPU
outputs with those oracle results (every unit), and a failure exits non-zero.
`read_ceiling` is a plain streaming read of the same byte count on the same
GPU, for context.  --fused 0 runs the four separate ABI calls instead (same
selection and MAW, O and lse to fp32 rounding, for comparison).  Each timed
step draws a fresh query; a selection wait that runs out of time fails the run.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_step_llama32k_traffic.json")
KERNEL_SOURCES = ["block_sparse_top_score_amd/csrc/sd_kernels.hip",
                  "block_sparse_top_score_amd/csrc/sd_internal.h",
                  "block_sparse_top_score_amd/csrc/sd_runtime.hip"]


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--fused", type=int, default=1, help="use sparse_decode_step")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--parity", type=int, default=1,
                    help="check the last timed step against the CPU oracle (every unit)")
    ap.add_argument("--workload", choices=["llama32k", "qwen128k", "loop32", "sweep"],
                    default="llama32k",
                    help="llama32k: the headline step; qwen128k (per-head budgets and block "
                         "sizes, N=131072), loop32 (B=16, N=65536, MAW flags on) and sweep "
                         "(the 4-query-head, d=64 geometry at N=32768, see --sweep) are variants")
    ap.add_argument("--sweep", type=int, nargs=3, default=[64, 16, 10], metavar=("B", "S", "PCT"),
                    help="sweep point: batch, block size, budget in percent of tokens")
    ap.add_argument("--sweep-n", type=int, default=32768,
                    help="cached tokens of a sweep point (32768 in the sweep workload)")
    ap.add_argument("--streaming-heads", type=int, default=0,
                    help="give the first K KV heads budget 0 (streaming heads: sinks and "
                         "recent window only); a variant of the workload, not the headline")
    ap.add_argument("--per-query-head", action="store_true",
                    help="one block set per query head (select_per_query_head): the separate "
                         "calls select_topk, sparse_attend (with the union of each KV head's "
                         "sets) and fuse_lse; the kernel split is timed per call")
    ap.add_argument("--lfps", action="store_true",
                    help="selection among the learn-from-the-past table candidates "
                         "(lfps_select): tables filled from 32 prefill positions per layer, then "
                         "the separate calls; the kernel split is timed per call")
    ap.add_argument("--timeline", type=int, default=0, metavar="STEPS",
                    help="measurement build only (build.py --timeline): record the per-phase "
                         "timestamps of STEPS one-launch steps after the warm-up, print their "
                         "per-role medians and exit")
    ap.add_argument("--timeline-b2b", action="store_true",
                    help="with --timeline: launch each recorded step right behind another one "
                         "(no synchronisation between them) and record the second")
    ap.add_argument("--timeline-dump", default="", metavar="NPY",
                    help="with --timeline: also save the raw timestamp tables "
                         "([steps][workgroups][slots] ticks, 0 = not reached) to NPY")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="rocprofv3 --pmc csv dirs of k_step and of the copy; write the "
                         "per-launch traffic file and exit")
    return ap.parse_args()


def copy_calibration(nbytes=1 << 30, reps=4):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def _pmc_avg_kib(d, name_part):
    """Mean counter value (KiB) per dispatch of kernels whose name contains
    name_part, from a rocprofv3 --pmc csv output directory."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if name_part in row.get("Kernel_Name", ""):
                    key = (row.get("Dispatch_Id"), row.get("Counter_Name"))
                    vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit("no %s dispatches in %s" % (name_part, d))
    return sum(vals.values()) / len(vals), len(vals)


def traffic_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    f_kib, nf = _pmc_avg_kib(fetch_dir, "k_step")
    w_kib, nw = _pmc_avg_kib(write_dir, "k_step")
    cf_kib, ncf = _pmc_avg_kib(cal_fetch_dir, "copy")
    cw_kib, ncw = _pmc_avg_kib(cal_write_dir, "copy")
    copy_bytes = 1 << 30
    f_scale = copy_bytes / (cf_kib * 1024.0)
    w_scale = copy_bytes / (cw_kib * 1024.0)
    out = {"kernel": "k_step (llama32k)",
           "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
           "dispatches": [nf, nw],
           "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib, "copy_bytes": copy_bytes,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "traffic_bytes_per_launch": f_kib * 1024.0 * f_scale + w_kib * 1024.0 * w_scale,
           "source_sha256": sources_sha256()}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh)
        fh.write("\n")
    print(json.dumps(out), flush=True)
    return out


def measured_traffic():
    """Per-launch HBM bytes of k_step from the committed counter summary, or
    None when the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sources_sha256():
        return None
    return t.get("traffic_bytes_per_launch")


def algorithmic_bytes(w, N, blk_cnt, blk_idx, with_maw=True, lfps_cand=None):
    """Per-step algorithmic HBM bytes (each term counted once):
    summaries n_blk*2*d*2 per (seq, kv head) that selects; K+V of the distinct
    attended tokens |T|*2*d*2 (with one set per query head, T = D U the union
    of the group's sets: a KV page is read once for the whole group); MAW: the
    flag's read of every block, n_blk*4,
    when the flag is on (with_maw), plus the update of the blocks wholly inside
    the dense set, 4*2 each; q 2d, O 4d, lse 4 per query head.  Scratch and
    page tables are excluded."""
    summ = attend = maw = 0
    for b in range(w.B):
        for g in range(w.Hkv):
            S = w.block_size[g]
            nb = (N + S - 1) // S
            if blk_idx.shape[1] == w.Hq:  # one set per query head: their union
                G = w.G
                sel = np.unique(np.concatenate(
                    [blk_idx[b, g * G + j, :blk_cnt[b, g * G + j]] for j in range(G)]))
            else:
                sel = blk_idx[b, g, :blk_cnt[b, g]]
            inD = np.zeros(N, bool)
            inD[:min(w.n_sink, N)] = True
            inD[max(0, N - w.window):] = True
            inT = inD.copy()
            for i in sel:
                inT[i * S:min(N, (i + 1) * S)] = True
            if lfps_cand is not None:  # only the table candidates are scored; the two
                # tables are read by the selection and read and written by the update
                summ += int(lfps_cand[b][g]) * 2 * w.d * 2 + nb * 4 * 2 * 3
            else:
                summ += nb * 2 * w.d * 2 if w.budget_ppm[g] > 0 else 0  # streaming heads score nothing
            attend += int(inT.sum()) * 2 * w.d * 2
            inside = sum(1 for i in range(nb) if inD[i * S:min(N, (i + 1) * S)].all())
            maw += (nb * 4 if with_maw and w.budget_ppm[g] > 0 else 0) + inside * 4 * 2
    qol = w.B * w.Hq * (2 * w.d + 4 * w.d + 4)
    return dict(summaries=summ, attend=attend, maw=maw, q_o_lse=qol,
                total=summ + attend + maw + qol)


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only (this build has no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from block_sparse_top_score_amd import SparseDecode, _abi
    if args.timeline:
        _abi.load(_abi.LIB_TIMELINE_PATH)

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = {"llama32k": synth.llama32k, "qwen128k": lambda: synth.qwen128k(0),
         "loop32": synth.loop32, "sweep": lambda: dataclasses.replace(synth.sweep(*args.sweep), N=args.sweep_n)}[args.workload]()
    maw_beta = w.maw_beta  # MAW flags on for loop32 only
    if args.per_query_head or args.lfps:
        args.fused = 0  # the one-launch step ranks every block per KV head
    if args.lfps:
        args.cpu_baseline = 0  # (the lockstep tests check this mode against the oracle)
    if args.streaming_heads:
        K_s = min(args.streaming_heads, w.Hkv)
        w = dataclasses.replace(w, budget_ppm=[0] * K_s + list(w.budget_ppm[K_s:]))
    N0 = w.N - 1                      # the first timed visit appends token N
    L = args.layers
    max_len = w.N + (args.steps + args.warmup) * (args.trials + 2) // L + 64
    stream = torch.cuda.current_stream()
    eng = SparseDecode(max_seqs=w.B, num_layers=L, num_q_heads=w.Hq,
                       num_kv_heads=w.Hkv, head_dim=w.d,
                       num_pages=w.B * ((max_len + 15) // 16), max_seq_len=max_len,
                       sink_tokens=w.n_sink, recent_window=w.window,
                       block_size=w.block_size, budget_ppm=w.budget_ppm,
                       maw_decay=0.95, maw_beta=maw_beta,
                       page_shuffle_seed=12345, stream=stream,
                       select_per_query_head=1 if args.per_query_head else 0,
                       lfps_select=1 if args.lfps else 0, lfps_a=0.2)
    seqs = list(range(w.B))
    dirs_l = {}
    t0 = time.time()

    def layer_inputs(layer):
        """The prefill K, V [B, w.N, Hkv, d] of a layer instance, from its seed
        (the same call again gives the same bits)."""
        if args.workload == "loop32":  # a planted direction per (layer, seq, KV head)
            dirs = synth.directions(w, args.seed, layer, 1, device=dev)
            dirs_l[layer] = dirs
            K, V, _ = synth.prefill_with_directions(w, args.seed, layer, w.N, dirs, device=dev)
            return K, V
        x = synth.single_step(w, args.seed * 100 + layer, device=dev, N=w.N)
        return x["K"], x["V"]

    for layer in range(L):
        K, V = layer_inputs(layer)
        K, V = K[:, :N0].contiguous(), V[:, :N0].contiguous()
        eng.append_kv(layer, seqs, [N0] * w.B, K.view(-1, w.Hkv, w.d), V.view(-1, w.Hkv, w.d))
        del K, V
        torch.cuda.empty_cache()
    torch.cuda.synchronize()
    lfps_init_ms = None
    if args.lfps:  # the tables from the last 32 prefill positions of every layer
        g0 = torch.Generator(device=dev).manual_seed(args.seed + 7)
        ei, ej = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ei.record(stream)
        for layer in range(L):
            qp = torch.randn(w.B, 32, w.Hq, w.d, generator=g0, device=dev).to(torch.bfloat16)
            eng.lfps_init(layer, seqs, qp)
        ej.record(stream)
        torch.cuda.synchronize()
        lfps_init_ms = ei.elapsed_time(ej) / L
    setup_s = time.time() - t0
    g = torch.Generator(device=dev).manual_seed(args.seed)
    k_new = torch.randn(64, w.B, w.Hkv, w.d, generator=g, device=dev).to(torch.bfloat16)
    v_new = torch.randn(64, w.B, w.Hkv, w.d, generator=g, device=dev).to(torch.bfloat16)
    # a fresh query every step, drawn before timing from the workload's query
    # distribution (loop32: N(0,1) + 3u of the layer's directions; else N(0,1))
    n_total = args.warmup + args.trials * args.steps
    if args.workload == "loop32":
        q_pool = torch.stack([synth.loop_query(w, args.seed, s_ % L, s_, dirs_l[s_ % L], device=dev)
                              for s_ in range(n_total)])
    else:
        q_pool = torch.randn(n_total, w.B, w.Hq, w.d, generator=g, device=dev).to(torch.bfloat16)
    bufs = eng.alloc_step(w.B, device=dev)

    def step(s):
        layer = s % L
        kn, vn = k_new[s % 64], v_new[s % 64]
        q = q_pool[s]
        if args.fused:
            eng.decode_step(layer, seqs, q, bufs["blk_idx"], bufs["blk_cnt"],
                            bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"],
                            k_new=kn, v_new=vn)
            return
        eng.append_kv(layer, seqs, [1] * w.B, kn, vn)
        eng.select_topk(layer, seqs, q, bufs["blk_idx"], bufs["blk_cnt"])
        eng.sparse_attend(layer, seqs, q, bufs["blk_idx"], bufs["blk_cnt"],
                          bufs["o_part"], bufs["lse_part"])
        eng.fuse_lse(layer, seqs, bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"])

    s_global = 0
    for _ in range(args.warmup):
        step(s_global)
        s_global += 1
    eng.sync()
    if args.timeline:
        timeline(args, w, eng, step, s_global, L)
        eng.close()
        return

    # timed trials: exactly --steps steps each, median reported
    trial_ms = []
    for _ in range(args.trials):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step(s_global)
            s_global += 1
        e1.record(stream)
        torch.cuda.synchronize()
        trial_ms.append(e0.elapsed_time(e1) / args.steps)
    eng.sync()  # a selection wait that ran out of time fails the run here
    ms = float(np.median(trial_ms))

    # outputs of the last timed step, and what it ran on (rebuilt from the
    # seeds: the layer's prefill, then the token appended at each of its
    # visits), for the parity check of the CPU-baseline leg
    s_last = s_global - 1
    l_last = s_last % L
    last = {k: v.cpu().numpy() for k, v in bufs.items() if k in ("blk_idx", "blk_cnt", "o", "lse")}
    N_now = eng.seq_len(l_last, 0)
    cnt, idx = last["blk_cnt"], last["blk_idx"]

    # the dominant kernel timed alone: n_inst back-to-back launches between two
    # HIP events on the library's stream, rotating layers so that the working
    # set stays out of the last-level cache
    n_inst = 64

    def timed_loop(fn):
        ea = torch.cuda.Event(enable_timing=True)
        eb = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ea.record(stream)
        for i in range(n_inst):
            fn(i)
        eb.record(stream)
        torch.cuda.synchronize()
        eng.sync()
        return ea.elapsed_time(eb) / n_inst

    lfps_cand = None
    if args.lfps:
        lfps_cand = [eng.debug(_abi.SD_DEBUG_LFPS_CAND, l_last, b).tolist() for b in range(w.B)]
    ab = algorithmic_bytes(w, N_now, cnt, idx, with_maw=maw_beta > 0, lfps_cand=lfps_cand)
    if args.per_query_head or args.lfps:
        # select_topk alone, then sparse_attend (union + attention) alone on
        # each layer's own selection (no append in between)
        sel_bufs = [eng.alloc_step(w.B, device=dev) for _ in range(L)]
        t_sel = timed_loop(lambda i: eng.select_topk(i % L, seqs, q_pool[i % L],
                                                     sel_bufs[i % L]["blk_idx"],
                                                     sel_bufs[i % L]["blk_cnt"]))
        t_att = timed_loop(lambda i: eng.sparse_attend(i % L, seqs, q_pool[i % L],
                                                       sel_bufs[i % L]["blk_idx"],
                                                       sel_bufs[i % L]["blk_cnt"],
                                                       bufs["o_part"], bufs["lse_part"]))
        l_att = (n_inst - 1) % L
        eng.fuse_lse(l_att, seqs, bufs["o_part"], bufs["lse_part"], bufs["o"], bufs["lse"])
        eng.sync()
        kernel_ms = {"select_topk": t_sel,
                     ("sparse_attend (k_union + k_attend)" if args.per_query_head
                      else "sparse_attend"): t_att,
                     "timed_launches": n_inst}
        dom_name, t_dom = ("k_union + k_attend" if args.per_query_head else "k_attend"), t_att
        kstep_bytes = ab["attend"]  # the attention's K+V of the union's tokens
        sel_gbs = ab["summaries"] / (t_sel * 1e-3) / 1e9
    else:
        # k_step: steps without append, so that it is the only kernel
        t_step = timed_loop(lambda i: eng.decode_step(i % L, seqs, q_pool[i], bufs["blk_idx"],
                                                      bufs["blk_cnt"], bufs["o_part"],
                                                      bufs["lse_part"], bufs["o"], bufs["lse"]))
        kernel_ms = {"k_step": t_step, "timed_launches": n_inst}
        dom_name, t_dom = "k_step", t_step
        kstep_bytes = ab["total"]  # k_step moves every algorithmic byte of the step
    qheads = w.B * w.Hq
    value = qheads / (ms * 1e-3)
    step_gbs = ab["total"] / (ms * 1e-3) / 1e9
    kstep_gbs = kstep_bytes / (t_dom * 1e-3) / 1e9

    out = {
        "metric": "sparse-decode attn query-heads/s at Llama-3-8B 32K, 5% budget; % HBM peak",
        "value": value,
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d, Hq=%d, Hkv=%d, d=%d, N=%d (+1 per visit), S=%s, "
                               "budget ppm %s, %d sinks + %d recent, MAW flags %s, %d layer instances"
                               % (w.name, w.B, w.Hq, w.Hkv, w.d, w.N, w.block_size, w.budget_ppm,
                                  w.n_sink, w.window, "on" if maw_beta > 0 else "off", L)
                               + ("; KV heads 0-%d streaming (budget 0)" % (args.streaming_heads - 1)
                                  if args.streaming_heads else ""),
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)",
                   "fused_step": bool(args.fused),
                   "selection": "per query head" if args.per_query_head else
                   ("learn-from-the-past table candidates, a = 0.2" if args.lfps else "per KV head")},
        "step_hbm": {"algorithmic_bytes": ab["total"], "achieved_GBs": step_gbs,
                     "frac_of_8TBs": step_gbs / HBM_PEAK_GBS,
                     "breakdown_bytes": {k: ab[k] for k in ("summaries", "attend", "maw", "q_o_lse")}},
        "kernel_ms": kernel_ms,
        "roofline": {"kernel": dom_name, "bound": "hbm", "achieved": kstep_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kstep_gbs / HBM_PEAK_GBS,
                     # the committed counter summary is the headline workload's
                     "traffic": measured_traffic() if args.workload == "llama32k"
                     and not args.streaming_heads and not args.per_query_head
                     and not args.lfps else None,
                     "algorithmic_bytes_per_launch": kstep_bytes},
        "trials_ms": trial_ms,
        "setup_s": setup_s,
    }

    if args.lfps:
        out["select_topk_GBs"] = sel_gbs
        out["lfps"] = {"init_ms_per_layer": lfps_init_ms,
                       "candidates_per_unit": lfps_cand,
                       "note": "only the table candidates' summaries are read (the summaries "
                               "term), plus the two tables: read by the selection, read and "
                               "written by the update"}
    if args.per_query_head:
        out["select_topk_GBs"] = sel_gbs
        out["union_vs_group"] = {
            "attended_bytes_per_query_head_set": ab["attend"],
            "note": "K+V bytes of D U the union of each KV head's query-head sets; "
                    "the per-KV-head selection of the same step reads D U k blocks"}
    out["read_ceiling"] = read_ceiling(kstep_bytes, kstep_gbs)
    parity_ok = True
    if args.cpu_baseline:
        K, V = layer_inputs(l_last)
        visits = [s_ for s_ in range(s_global) if s_ % L == l_last]
        assert N_now == N0 + len(visits)
        Kb = np.concatenate([synth.bits(K[:, :N0])] +
                            [synth.bits(k_new[s_ % 64])[:, None] for s_ in visits], 1)
        Vb = np.concatenate([synth.bits(V[:, :N0])] +
                            [synth.bits(v_new[s_ % 64])[:, None] for s_ in visits], 1)
        del K, V
        torch.cuda.empty_cache()
        out["cpu_baseline"], out["parity"] = cpu_baseline_and_parity(
            w, Kb, Vb, synth.bits(q_pool[s_last]), N_now, last, args.cpu_seconds,
            check=bool(args.parity) and maw_beta <= 0.0, step_index=s_last,
            per_query_head=args.per_query_head)
        parity_ok = out["parity"].get("pass", True)
    print(json.dumps(out), flush=True)
    eng.close()
    if not parity_ok:
        print("parity of the last timed step FAILED: %s" % json.dumps(out["parity"]),
              file=sys.stderr)
        sys.exit(1)


def timeline(args, w, eng, step, s0, L):
    """Per-phase timestamps of --timeline one-launch steps (the measurement
    build): for each step, every workgroup's phase times in microseconds from
    the step's first workgroup start; printed as medians and 10th/90th
    percentiles per role and phase over all workgroups and steps, plus the
    per-step time of the last event (the end of the critical path)."""
    import torch
    from block_sparse_top_score_amd import _abi
    # score tiles per unit in the launch: blocks that can hold a candidate,
    # ceil((N - W) / S), in tiles of 256 (N about the current length)
    n_now = eng.seq_len(s0 % L, 0) + 1
    tiles = -(-max(-(-max(0, n_now - w.window) // S) for S in w.block_size) // 256)
    n_wg = w.Hkv * w.B * 64
    names = {"score": ["first instruction", "keys written", "tile list published", "arrived",
                       "top-k done", "(unused)",
                       "fast top-k gave up (full top-k runs)", "band re-score started"],
             "part": ["first instruction", "dense pages done (wave 0)", "selection count seen",
                      "selected pages done (wave 0)", "partial written, arrived",
                      "fusion done", "first dense page ids read (wave 0)", "(unused)"],
             "maw": ["first instruction", "(unused)", "(unused)", "(unused)", "(unused)",
                     "(unused)", "arrivals seen", "MAW updated"]}
    acc = {r: {k: [] for k in range(len(v))} for r, v in names.items()}
    # durations inside the last-arriver roles, per workgroup (us)
    spans = {"top-k (last tile: arrived -> done)": ("score", 3, 4),
             "fusion (last part: arrived -> done)": ("part", 4, 5),
             "MAW worker (arrivals seen -> MAW done)": ("maw", 6, 7),
             "top-k with the band re-score (arrived -> done)": ("score", 7, 4),
             "top-k after the fast one gave up (gave up -> done)": ("score", 6, 4),
             "tile: keys -> list published": ("score", 1, 2),
             "tile: list published -> arrived": ("score", 2, 3),
             "part: selected pages done -> partial written, arrived": ("part", 3, 4)}
    dur = {k: [] for k in spans}
    ends, raw = [], []
    _abi.timeline_read(n_wg)  # clear
    for t in range(args.timeline):
        if args.timeline_b2b:  # the recorded launch queued right behind another
            step(s0 + 2 * t)
            step(s0 + 2 * t + 1)
        else:
            step(s0 + t)
        torch.cuda.synchronize()
        tl = _abi.timeline_read(n_wg).astype(np.int64)
        used = tl[:, 0] > 0
        t0 = tl[used, 0].min()
        # (back to back: slots the recorded launch did not reach may still hold
        # the earlier launch's stamps, all before its first start)
        tl[tl < t0] = 0
        raw.append(tl)
        us = (tl - t0) / 100.0  # 100 MHz ticks -> us
        for wg in np.nonzero(used)[0]:
            z = wg // (w.Hkv * w.B)
            # (the MAW worker, last in z, is the role that stamps slot 6
            # without slot 1)
            role = ("score" if z < tiles else
                    "maw" if tl[wg, 6] > 0 and tl[wg, 1] == 0 else "part")
            for k in range(len(names[role])):
                if tl[wg, k] > 0:
                    acc[role][k].append(us[wg, k])
            for name, (r_, a_, b_) in spans.items():
                if r_ == role and tl[wg, a_] > 0 and tl[wg, b_] > 0:
                    dur[name].append(us[wg, b_] - us[wg, a_])
        ends.append(float(us[used].max()))
    if args.timeline_dump:
        np.save(args.timeline_dump, np.stack(raw))
    # dispatch: first instruction by XCD (workgroups go round-robin over the 8
    # XCDs in flat order) and by position in the flat order (octiles)
    first = np.stack([(r[:, 0] - r[r[:, 0] > 0, 0].min()) / 100.0 for r in raw])
    ok = np.stack([r[:, 0] > 0 for r in raw])
    wg_ids = np.arange(n_wg)
    by_xcd = [float(np.median(first[:, wg_ids % 8 == x][ok[:, wg_ids % 8 == x]])) for x in range(8)]
    n_used = int(ok.any(0).nonzero()[0].max()) + 1
    octile = wg_ids * 8 // n_used
    by_order = [float(np.median(first[:, octile == o][ok[:, octile == o]])) for o in range(8)]
    # (octiles of the flat order over the launch's workgroups)
    out = {"workload": w.name, "steps": args.timeline, "tiles_per_unit": tiles,
           "back_to_back": bool(args.timeline_b2b),
           "first_instruction_median_by_xcd_us": by_xcd,
           "first_instruction_median_by_order_octile_us": by_order,
           "last_event_us": {"median": float(np.median(ends)), "min": float(np.min(ends)),
                             "max": float(np.max(ends))}}
    for role, ph in names.items():
        rows = []
        for k, name in enumerate(ph):
            v = np.array(acc[role][k])
            if v.size and name != "(unused)":
                rows.append({"phase": name, "n": int(v.size), "p10": float(np.percentile(v, 10)),
                             "median": float(np.median(v)), "p90": float(np.percentile(v, 90)),
                             "max": float(v.max())})
        out[role] = rows
    out["durations"] = [{"span": k, "n": len(v), "median": float(np.median(v)),
                         "p90": float(np.percentile(v, 90))} for k, v in dur.items() if v]
    print(json.dumps(out), flush=True)
    for role in names:
        print("%s:" % role)
        for r in out[role]:
            print("  %-30s n=%6d  p10 %6.2f  median %6.2f  p90 %6.2f  max %6.2f us"
                  % (r["phase"], r["n"], r["p10"], r["median"], r["p90"], r["max"]))
    print("durations:")
    for r in out["durations"]:
        print("  %-62s n=%5d  median %5.2f  p90 %5.2f us" % (r["span"], r["n"], r["median"], r["p90"]))
    print("first instruction, median by XCD:", " ".join("%.2f" % v for v in by_xcd), "us")
    print("first instruction, median by flat-order octile:", " ".join("%.2f" % v for v in by_order), "us")
    print("last event per step: median %.2f us (min %.2f, max %.2f)"
          % (out["last_event_us"]["median"], out["last_event_us"]["min"],
             out["last_event_us"]["max"]), flush=True)


def read_ceiling(nbytes, kstep_gbs, n_buf=8, reps=64, wgs=4096):
    """A plain streaming read on the same GPU, for context: the library's read
    probe (each 16-byte word once, coalesced, eight in flight per thread, 4096
    workgroups) over n_buf
    rotating buffers of the step's algorithmic size (8 x ~106 MB, so the reads
    are not served from the 256 MB last-level cache), timed with events on
    torch's stream.  `k_step_frac` is k_step's rate over this one."""
    import ctypes
    import torch
    from block_sparse_top_score_amd import _abi
    L = _abi.load()
    n = nbytes // 16 * 16
    bufs = [torch.randint(0, 255, (n,), device="cuda", dtype=torch.uint8) for _ in range(n_buf)]
    sink = torch.zeros(wgs, device="cuda", dtype=torch.int32)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(b):
        st = L.sd_read_probe(ctypes.c_void_p(b.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                             wgs, stream)
        if st != 0:
            raise RuntimeError("sd_read_probe failed: %d" % st)

    for b in bufs:  # warm-up
        launch(b)
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ea.record()
    for r in range(reps):
        launch(bufs[r % n_buf])
    eb.record()
    torch.cuda.synchronize()
    t_ms = ea.elapsed_time(eb) / reps
    gbs = n / (t_ms * 1e-3) / 1e9
    del bufs
    return {"kind": "k_read_probe, %d rotating buffers, %d workgroups, 8 loads in flight per thread" % (n_buf, wgs), "bytes": n,
            "ms": t_ms, "achieved_GBs": gbs, "frac_of_8TBs": gbs / HBM_PEAK_GBS,
            "k_step_frac": kstep_gbs / gbs}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_and_parity(w, Kb, Vb, qb, N, gpu, budget_s, check=True, step_index=-1,
                            per_query_head=False):
    """The CPU-baseline leg: the CPU oracle (unchanged) on the inputs of the
    last timed step (every (sequence, KV head) unit; bf16 bits rebuilt from the
    seeds, none read back from the GPU).  Summaries are computed first, outside
    the timing, as the GPU path keeps them incrementally; oracle select +
    attend are then timed per unit, one unit per task, on all the host threads
    the box gives one GPU (16) and on one thread, each for about budget_s / 2
    seconds.  The oracle's results of the first pass over the units also serve
    the parity check of the GPU's outputs of that step (check=True): selection
    bit-exact except ties inside the 1e-6 relative score band, max |dO| <=
    2e-3, max relative dO <= 1e-2 where |O| >= 0.1, |dlse| <= 1e-4.
    per_query_head: the oracle's per-query-head selection and attention, and
    the same check per query head."""
    import concurrent.futures as cf
    import oracle
    G = w.G
    units = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    Kg = {u: np.ascontiguousarray(Kb[u[0], :N, u[1]]) for u in units}
    Vg = {u: np.ascontiguousarray(Vb[u[0], :N, u[1]]) for u in units}
    summ = {u: oracle.summaries(Kg[u], w.block_size[u[1]]) for u in units}

    def run(u):
        b, g = u
        S, qg = w.block_size[g], qb[b, g * G:(g + 1) * G]
        if per_query_head:
            sels = oracle.select_heads(qg, summ[u][0], summ[u][1], N, S, w.n_sink, w.window,
                                       w.budget_ppm[g])
            O, lse = oracle.attend_heads(qg, Kg[u], Vg[u], N, S, w.n_sink, w.window, sels)
            return u, dict(sels=sels), dict(O=O, lse=lse)
        r = oracle.select(qg, summ[u][0], summ[u][1], N, S, w.n_sink, w.window, w.budget_ppm[g])
        a = oracle.attend(qg, Kg[u], Vg[u], N, S, w.n_sink, w.window, r["sel"])
        return u, r, a

    def timed(threads):
        done, t0, results = 0, time.time(), None
        with cf.ThreadPoolExecutor(threads) as ex:
            while True:
                res = list(ex.map(run, units))
                done += len(units)
                results = results or res
                if time.time() - t0 >= budget_s / 2:
                    break
        return done, time.time() - t0, results

    threads = max(1, min(16, os.cpu_count() or 1))
    done, dt, results = timed(threads)
    done1, dt1, _ = timed(1)
    base = {"value": done * G / dt, "unit": "query-heads/s", "cores": threads, "kind": "oracle",
            "sample": "%d (sequence, KV head) units (%d full steps) of the %s step at N=%d, "
                      "oracle select + attend%s on precomputed summaries, %d threads, %.1f s"
                      % (done, done // len(units), w.name, N,
                         " per query head" if per_query_head else "", threads, dt),
            "ms_per_step": dt / (done / len(units)) * 1e3,
            "t1": {"value": done1 * G / dt1, "cores": 1,
                   "ms_per_step": dt1 / (done1 / len(units)) * 1e3,
                   "sample": "%d units, one thread, %.1f s" % (done1, dt1)},
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}
    if not check:
        return base, {"checked": False,
                      "reason": "MAW flags depend on the layer's whole history (the lockstep "
                                "tests cover them)" if w.maw_beta > 0 else "disabled"}
    ties = 0
    ma = mr = ml = 0.0
    fails = []
    if per_query_head:
        # one row per query head: (selection, oracle result) pairs
        flat = []
        for (b, g), r, a in results:
            S, qg = w.block_size[g], qb[b, g * G:(g + 1) * G]
            Uh, _, _ = oracle.score(qg, summ[(b, g)][0], summ[(b, g)][1])
            gs = []
            for j in range(G):
                cnt = int(gpu["blk_cnt"][b, g * G + j])
                gsel, osel = set(gpu["blk_idx"][b, g * G + j, :cnt].tolist()), set(r["sels"][j].tolist())
                if cnt != len(osel):
                    fails.append("head (%d,%d): k %d vs %d" % (b, g * G + j, cnt, len(osel)))
                elif gsel != osel:
                    kth = min(Uh[j][i] for i in osel)
                    if not all(abs(Uh[j][i] - kth) <= 1e-6 * max(abs(Uh[j][i]), abs(kth), 1e-30)
                               for i in gsel ^ osel):
                        fails.append("head (%d,%d): selection differs outside the tie band"
                                     % (b, g * G + j))
                    ties += len(gsel ^ osel) // 2
                gs.append(np.array(sorted(gsel), np.int32))
            O, lse = oracle.attend_heads(qg, Kg[(b, g)], Vg[(b, g)], N, S, w.n_sink, w.window, gs)
            flat.append(((b, g), dict(O=O, lse=lse)))
        results = [(u, None, a) for u, a in flat]
    for (b, g), r, a in results:
        if not per_query_head:
            cnt = int(gpu["blk_cnt"][b, g])
            gsel = set(gpu["blk_idx"][b, g, :cnt].tolist())
            osel = set(r["sel"].tolist())
            if cnt != r["k"]:
                fails.append("unit (%d,%d): k %d vs %d" % (b, g, cnt, r["k"]))
                continue
            if gsel != osel:
                kth = min(r["U"][i] for i in osel)
                band = all(abs(r["U"][i] - kth) <= 1e-6 * max(abs(r["U"][i]), abs(kth), 1e-30)
                           for i in gsel ^ osel)
                if not band:
                    fails.append("unit (%d,%d): selection differs outside the tie band" % (b, g))
                    continue
                ties += len(gsel ^ osel) // 2
                a = oracle.attend(qb[b, g * G:(g + 1) * G], Kg[(b, g)], Vg[(b, g)], N,
                                  w.block_size[g], w.n_sink, w.window,
                                  np.array(sorted(gsel), np.int32))
        Og = gpu["o"][b, g * G:(g + 1) * G].astype(np.float64)
        dO = np.abs(Og - a["O"])
        ma = max(ma, float(dO.max()))
        big = np.abs(a["O"]) >= 0.1
        if big.any():
            mr = max(mr, float((dO[big] / np.abs(a["O"][big])).max()))
        ml = max(ml, float(np.abs(gpu["lse"][b, g * G:(g + 1) * G] - a["lse"]).max()))
    ok = not fails and ma <= 2e-3 and mr <= 1e-2 and ml <= 1e-4
    par = {"checked": True, "step": step_index, "units": len(results), "ties": ties,
           "max_abs": ma, "max_rel": mr, "max_dlse": ml,
           "gates": {"max_abs": 2e-3, "max_rel": 1e-2, "rel_floor": 0.1, "max_dlse": 1e-4,
                     "tie_band": 1e-6},
           "pass": ok}
    if fails:
        par["failures"] = fails[:8]
    return base, par


if __name__ == "__main__":
    main()
