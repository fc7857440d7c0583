"""The oracle may be called from several threads at once (one unit each), as
the parity harness and the CPU baseline do: threaded selections must equal
serial ones.  CPU only."""
import concurrent.futures as cf

import numpy as np
import torch

import oracle
import synth


def test_threaded_selection_equals_serial():
    g = torch.Generator().manual_seed(1)
    jobs = []
    for _ in range(16):
        K = synth.bits(torch.randn(8192, 64, generator=g).to(torch.bfloat16))
        q = synth.bits(torch.randn(4, 64, generator=g).to(torch.bfloat16))
        mn, mx = oracle.summaries(K, 16)
        jobs.append((q, mn, mx))
    run = lambda j: oracle.select(j[0], j[1], j[2], 8192, 16, 4, 64, 50000)["sel"]
    serial = [run(j) for j in jobs]
    for _ in range(3):
        with cf.ThreadPoolExecutor(8) as ex:
            par = list(ex.map(run, jobs))
        assert all(np.array_equal(a, b) for a, b in zip(serial, par))
