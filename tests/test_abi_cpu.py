"""Host-side tests of the C-ABI library (no GPU is touched).

The library must load, export every function include/sparse_decode.h declares,
and reject bad configurations in sd_validate_config without a device.
"""
import ctypes
import os
import re

import pytest

import block_sparse_top_score_amd as bsts
from block_sparse_top_score_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        txt = open(os.path.join(ROOT, "include", fn)).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names += re.findall(r"^\s*(?:sd_status|const char \*)\s*(\w+)\s*\(", txt, re.M)
    return sorted(set(names))


def test_library_loads_and_exports_every_declared_symbol():
    L = bsts.load()
    declared = header_functions()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(L, name), "symbol %s missing from the library" % name
    assert sorted(_abi.EXPORTS) == declared


def base_cfg(**over):
    kw = dict(max_seqs=8, num_layers=1, num_q_heads=32, num_kv_heads=8,
              head_dim=128, num_pages=1024, max_seq_len=4096, sink_tokens=4,
              recent_window=512, block_size=[32] * 8, budget_ppm=[50000] * 8)
    kw.update(over)
    return bsts.make_config(**kw)


def test_valid_config_accepted():
    st, msg = bsts.validate_config(base_cfg())
    assert st == bsts.SD_OK, msg
    st, msg = bsts.validate_config(base_cfg(num_q_heads=28, num_kv_heads=4,
                                            block_size=[16, 64, 16, 64],
                                            budget_ppm=[10000, 200000, 5, 999999]))
    assert st == bsts.SD_OK, msg


@pytest.mark.parametrize("over,needle", [
    (dict(head_dim=96), "head_dim"),
    (dict(num_q_heads=30), "multiple"),
    (dict(num_q_heads=80, num_kv_heads=8), "group size"),
    (dict(block_size=[24] * 8), "block_size"),
    (dict(block_size=[128] * 8), "block_size"),
    (dict(budget_ppm=[1000001] * 8), "budget_ppm"),
    (dict(budget_ppm=[-1] * 8), "budget_ppm"),
    (dict(page_size=32), "page_size"),
    (dict(max_seqs=0), "max_seqs"),
    (dict(num_pages=0), "num_pages"),
    (dict(max_seq_len=0), "max_seq_len"),
    (dict(sink_tokens=-1), "sink_tokens"),
    (dict(recent_window=-5), "recent_window"),
    (dict(maw_decay=1.0), "maw_decay"),
    (dict(softmax_scale=-1.0), "softmax_scale"),
    (dict(num_layers=0), "num_layers"),
])
def test_invalid_configs_rejected(over, needle):
    st, msg = bsts.validate_config(base_cfg(**over))
    assert st == bsts.SD_EINVAL
    assert needle in msg


def test_null_config_rejected():
    L = bsts.load()
    buf = ctypes.create_string_buffer(128)
    assert L.sd_validate_config(None, buf, 128) == bsts.SD_EINVAL


def test_product_path_does_not_import_oracle():
    """The HIP binding must not reach the CPU oracle."""
    pkg = os.path.join(ROOT, "block_sparse_top_score_amd")
    for dp, _, fns in os.walk(pkg):
        for fn in fns:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dp, fn)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, fn
                assert "oracle.h" not in txt, fn


def test_read_probe_rejects_bad_arguments_before_any_launch():
    """Argument checks of the streaming-read probe run on the host, so they
    return SD_EINVAL here without a device."""
    import ctypes
    L = bsts.load()
    dummy = ctypes.c_void_p(16)  # never dereferenced: every call below is rejected
    assert L.sd_read_probe(None, 16, dummy, 1, None) == -1
    assert L.sd_read_probe(dummy, 16, None, 1, None) == -1
    assert L.sd_read_probe(dummy, 0, dummy, 1, None) == -1
    assert L.sd_read_probe(dummy, 24, dummy, 1, None) == -1
    assert L.sd_read_probe(ctypes.c_void_p(8), 16, dummy, 1, None) == -1
    assert L.sd_read_probe(dummy, 16, dummy, 0, None) == -1


def test_timeline_export_only_in_the_measurement_build():
    """sd_timeline_read (include/sparse_decode_timeline.h) belongs to the
    SD_TIMELINE measurement build only; the product library does not export
    it."""
    L = bsts.load()
    assert not hasattr(L, "sd_timeline_read")
    if not os.path.exists(_abi.LIB_TIMELINE_PATH):
        pytest.skip("measurement build not present")
    T = ctypes.CDLL(_abi.LIB_TIMELINE_PATH)
    assert hasattr(T, "sd_timeline_read")
