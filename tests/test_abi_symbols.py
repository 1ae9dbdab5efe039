"""The C-ABI library loads and exports every entry point the header declares
(no GPU work: only host-side functions are called)."""
import ctypes
import pathlib
import re

import pytest

from sparse_attention_kv_request_amd import binding

HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "hisparse.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(hisparse_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("hisparse_state_create", "hisparse_swap_in_selected",
                 "hisparse_swap_in_spec_multistep", "hisparse_state_destroy"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = binding.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) == set(binding.EXPORTED)


def test_default_build_carries_no_instrumentation():
    """The phase-clock hooks exist only in the opt-in instrumented build."""
    lib = binding.lib()
    for name in ("hisparse_phase_clocks", "hisparse_attention_wait_clocks",
                 "hisparse_attention_phase_clocks", "hisparse_topk_phase_clocks",
                 "hisparse_topk_merge_phase_clocks"):
        assert not hasattr(lib, name), name


def test_strerror_and_rows_are_host_only():
    assert binding.strerror(0) == "success"
    assert binding.strerror(binding.HISPARSE_E_INVAL) == "invalid argument"
    cfg = binding.HisparseConfig(max_requests=4, num_layers=1, hot_buffer_size=100, top_k=60,
                                 max_steps=3, page_size=1, item_size_bytes=32, max_seq_len=500,
                                 policy=1, max_batch=4)
    assert binding.hisparse_device_rows_per_request(cfg) == 100 + 3 * 60 - 100
    cfg.policy = 0
    cfg.max_steps = 1
    assert binding.hisparse_device_rows_per_request(cfg) == 100


@pytest.mark.parametrize("field,value,code", [
    ("hot_buffer_size", 0, -1), ("hot_buffer_size", 32769, -1), ("top_k", 101, -1),
    ("item_size_bytes", 24, -1), ("max_steps", 2, -1), ("max_batch", 5, -1),
    ("policy", 7, -1), ("top_k", 8193, -4), ("max_seq_len", 1 << 28, -4),
    ("admission", 3, -1), ("admission", -1, -1), ("extra_rows", -1, -1),
    ("extra_rows", 501, -1),
])
def test_config_validation(field, value, code):
    cfg = binding.HisparseConfig(max_requests=4, num_layers=1, hot_buffer_size=100, top_k=60,
                                 max_steps=1, page_size=1, item_size_bytes=32, max_seq_len=500,
                                 policy=0, max_batch=4)
    if field == "top_k" and value > 8192:
        cfg.hot_buffer_size = 32768
    setattr(cfg, field, value)
    assert binding.hisparse_device_rows_per_request(cfg) == code


def test_page_mode_and_clock_limits():
    cfg = binding.HisparseConfig(max_requests=2, num_layers=1, hot_buffer_size=64, top_k=512,
                                 max_steps=1, page_size=256, item_size_bytes=656,
                                 max_seq_len=65536, policy=0, max_batch=2)
    assert binding.hisparse_device_rows_per_request(cfg) == 64
    cfg.max_seq_len = 65536 + 1
    assert binding.hisparse_device_rows_per_request(cfg) == -1
    cfg = binding.HisparseConfig(max_requests=2, num_layers=1, hot_buffer_size=4096, top_k=2048,
                                 max_steps=5, page_size=1, item_size_bytes=656,
                                 max_seq_len=32768, policy=1, max_batch=2)
    assert binding.hisparse_device_rows_per_request(cfg) == -1
    cfg.max_steps = 4
    assert binding.hisparse_device_rows_per_request(cfg) == 4096 + 4 * 2048 - 4096
    cfg.max_steps = 1
    assert binding.hisparse_device_rows_per_request(cfg) == -1


def test_topk_sizes_and_host_validation():
    """Host-side sizes and argument checks of the top-k entry points (no
    kernel is launched: every call below is rejected before any HIP call)."""
    import math
    for B, N, k in [(1, 1, 1), (64, 32768, 2048), (128, 131072, 2048), (3, 32769, 2048),
                    (7, 64 * 32768, 512), (5, 30000, 30000)]:
        chunks = max(1, math.ceil(N / 32768))
        assert binding.hisparse_topk_plan_ints(B, N) == 2 + 2 * B + 4 * B * chunks
        ws = binding.hisparse_topk_workspace_bytes(B, N, k)
        assert ws == (0 if chunks == 1 else 8 * B * chunks * k + 4 * B * chunks)
    assert binding.hisparse_topk_plan_ints(0, 10) == 0
    assert binding.hisparse_topk_workspace_bytes(4, 17 * 32768, 2048) == 0   # 17 x 2048 > 32768
    assert binding.hisparse_topk_workspace_bytes(4, 65 * 32768, 16) == 0     # 65 chunks
    assert binding.hisparse_topk_plan(4, 100, None, None, 100, None) == binding.HISPARSE_E_INVAL
    c = binding.HisparseTopkCall(batch=2, max_len=100, k=0)
    assert binding.hisparse_topk_index_build(c, None) == binding.HISPARSE_E_INVAL
    c.k = 40000
    assert binding.hisparse_topk_index_build(c, None) == binding.HISPARSE_E_UNSUPPORTED
    c.k, c.max_len = 8192, 5 * 32768               # 5 chunks x 8192 candidates > 32768
    assert binding.hisparse_topk_index_build(c, None) == binding.HISPARSE_E_UNSUPPORTED
    c.k, c.max_len = 16, 100
    assert binding.hisparse_topk_index_build(c, None) == binding.HISPARSE_E_INVAL  # NULL pointers


def test_extra_rows_extend_the_token_rows():
    """The extra-row ring adds E rows after the hot (and scratch) rows of a
    token-mode request; page mode has no ring."""
    cfg = binding.HisparseConfig(max_requests=4, num_layers=1, hot_buffer_size=100, top_k=60,
                                 max_steps=3, page_size=1, item_size_bytes=32, max_seq_len=500,
                                 policy=1, max_batch=4, admission=2, extra_rows=500)
    assert binding.hisparse_device_rows_per_request(cfg) == 100 + 3 * 60 - 100 + 500
    cfg.policy, cfg.max_steps, cfg.extra_rows = 0, 1, 7
    assert binding.hisparse_device_rows_per_request(cfg) == 107
    cfg = binding.HisparseConfig(max_requests=2, num_layers=1, hot_buffer_size=64, top_k=512,
                                 max_steps=1, page_size=256, item_size_bytes=656,
                                 max_seq_len=65536, policy=0, max_batch=2, extra_rows=1)
    assert binding.hisparse_device_rows_per_request(cfg) == binding.HISPARSE_E_UNSUPPORTED


def test_batch_limit_of_the_copy():
    """The miss copy holds a call's per-row prefix of miss counts in LDS, so a
    state may not accept batches beyond HISPARSE_MAX_BATCH: a larger batch
    would commit cache state whose copies could not launch."""
    cfg = binding.HisparseConfig(max_requests=20000, num_layers=1, hot_buffer_size=100,
                                 top_k=60, max_steps=1, page_size=1, item_size_bytes=32,
                                 max_seq_len=500, policy=0, max_batch=16000)
    assert binding.hisparse_device_rows_per_request(cfg) == 100
    cfg.max_batch = 16001
    assert binding.hisparse_device_rows_per_request(cfg) == binding.HISPARSE_E_UNSUPPORTED
    cfg.max_batch = 20000
    assert binding.hisparse_device_rows_per_request(cfg) == binding.HISPARSE_E_UNSUPPORTED
