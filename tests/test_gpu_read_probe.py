"""The streaming-read probe (a measurement aid beside the decode path): the
XOR of its sink words must equal the XOR of every 32-bit word of the buffer,
so each word is read exactly once, including a ragged tail shorter than one
grid stride."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from block_sparse_top_score_amd import _abi
from tests.harness import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16,wgs", [(1, 1), (255, 3), (4 * 2048 * 256 + 77, 2048),
                                     (6_603_136, 2048)])
def test_read_probe_reads_every_word_once(n16, wgs):
    log("read probe: %d words of 16 B, %d workgroups" % (n16, wgs))
    L = _abi.load()
    rng = np.random.default_rng(n16)
    host = rng.integers(0, 2**32, size=4 * n16, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(wgs, device="cuda", dtype=torch.int32)
    st = L.sd_read_probe(ctypes.c_void_p(buf.data_ptr()), 16 * n16,
                         ctypes.c_void_p(sink.data_ptr()), wgs,
                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
