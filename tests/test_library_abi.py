"""CPU checks of the C-ABI library: it loads without a GPU and exports every
entry point include/tkv.h declares; host-side argument checks."""
import ctypes as C
import os
import re

import pytest

from thought_adaptive_mixed_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol():
    lib = binding.load()
    names = declared_functions()
    assert set(names) == set(binding.SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n


def test_layout_validation_and_sizes():
    good = binding.make_layout(8, 32, 128, 64, (10, 20, 30), 4, 16, 32, 256)
    sizes = binding.buffer_sizes(good)
    assert sizes[0] == 10 * 8 * (4 * 128 * 8 + 128 * 2)
    assert sizes[1] == 20 * 8 * (4 * 128 * 4 + 128 * 2)
    assert sizes[2] == 30 * 8 * (4 * 128 * 2 + 128 * 2)
    for bad in [binding.make_layout(8, 30, 128, 64, (1, 1, 1), 4, 16, 32),      # Hq % Hkv
                binding.make_layout(1, 32, 128, 64, (1, 1, 1), 4, 16, 32),      # G > 16
                binding.make_layout(8, 32, 96, 32, (1, 1, 1), 4, 16, 32),       # D
                binding.make_layout(8, 32, 64, 128, (1, 1, 1), 4, 16, 32),      # g > D
                binding.make_layout(8, 32, 128, 64, (1, 1, 1), 4, 300, 32),     # blocks per seq
                binding.make_layout(8, 32, 128, 64, (1, 1, 1), 2000, 16, 32),   # seqs
                binding.make_layout(8, 32, 128, 64, (1, 0, 1), 4, 16, 32),      # empty pool
                binding.make_layout(8, 32, 128, 64, (1, 1, 1), 4, 16, 32, 9000),
                binding.make_layout(8, 32, 128, 64, (1, 1, 1), 4, 16, 32, 100, (8, 3, 2))]:
        with pytest.raises(binding.TkvError) as e:
            binding.buffer_sizes(bad)
        assert e.value.code == binding.TKV_EINVAL


def test_null_handle_and_strerror():
    lib = binding.load()
    assert lib.tkv_destroy(None) == binding.TKV_EINVAL
    assert lib.kv_append_quant(None, 1, None, None, None, None, None, None, None) == binding.TKV_EINVAL
    assert lib.kv_classify_append(None, 1, None, None, None, 4, C.c_float(0.3), C.c_float(0.8), 0, None, None,
                                  None, None, None) == binding.TKV_EINVAL
    assert lib.kv_plan_budget_evict(None, 1, None, 1, 10, 4, None, None, None, None, None, None) == binding.TKV_EINVAL
    assert lib.kv_plan_anneal_evict(None, 1, None, 64, 4, None, None, None, None, None, None) == binding.TKV_EINVAL
    assert lib.thought_classify(-1, 4, None, C.c_float(0.3), C.c_float(0.8), 0, None, None) == binding.TKV_EINVAL
    assert lib.thought_classify(1, 4, None, C.c_float(0.3), C.c_float(0.8), 2, None, None) == binding.TKV_EINVAL
    assert binding.strerror(binding.TKV_ENOSEG) == "unknown or evicted segment"
    assert lib.tkv_stream_read(None, 16, None, None) == binding.TKV_EINVAL
    assert lib.tkv_kernel_timing(None, 1) == binding.TKV_EINVAL
    assert lib.tkv_kernel_times(None, 0, None, None, None, None) == binding.TKV_EINVAL
    assert lib.tkv_stream_read(C.c_void_p(16), 15, C.c_void_p(16), None) == binding.TKV_EINVAL
