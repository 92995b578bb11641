"""CPU tests of the C ABI (no GPU needed): libmd.so loads, exports every
function include/md.h declares, and rejects bad arguments on the host before
any device work."""
import ctypes
import os
import re

import pytest

from decode_megakernel_md_amd import _lib
from synth import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p


def declared_functions():
    text = open(os.path.join(ROOT, "include", "md.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(md_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 15
    so = ctypes.CDLL(_lib.SO)
    for n in names:
        assert hasattr(so, n), f"{n} declared in md.h but not exported"
    assert sorted(_lib.EXPORTS) == names


def _cfg(name="mini_dense", **kw):
    c = _lib.config_from(WL.get(name))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _err():
    return _lib.lib().md_last_error().decode()


def test_inventory_matches_the_workload_tensor_list():
    for name in ("tiny_dense", "mini_moe", "mini_hybrid", "hybrid_moe"):
        w = WL.get(name)
        inv = _lib.weight_inventory(_lib.config_from(w))
        assert inv == [(t.name, t.rows, t.cols) for t in WL.tensor_inventory(w)]


def test_weight_layouts():
    L = _lib.lib()
    w = WL.mini_hybrid()
    c = _lib.config_from(w)
    for i, t in enumerate(WL.tensor_inventory(w)):
        want = 0 if (i == 0 or t.rows == 1 or t.name.endswith("mla_wkvb")) else 1
        assert L.md_weight_layout(ctypes.byref(c), i) == want, t.name
    assert L.md_weight_layout(ctypes.byref(c), 10 ** 6) == -1


def test_packed_bytes():
    L = _lib.lib()
    assert L.md_packed_bytes(16, 32) == 1024
    assert L.md_packed_bytes(17, 64) == 2 * 2 * 1024
    assert L.md_packed_bytes(5, 31) == 0
    assert L.md_packed_bytes(0, 32) == 0


def test_kv_bytes_match_the_documented_layout():
    L = _lib.lib()
    for name in ("mini_dense", "mini_moe", "mini_hybrid", "dense_27b", "hybrid_moe"):
        w = WL.get(name)
        _, total = WL.kv_layout(w)
        c = _lib.config_from(w)
        assert L.md_kv_bytes(ctypes.byref(c), w.max_batch, w.max_ctx) == total, name
        # other slot counts and capacities: the same layout with those sizes
        for B, C in ((1, w.max_ctx), (3, w.max_ctx + 32), (8, 64), (64, 64)):
            _, t2 = WL.kv_layout(w.replace(max_batch=B, max_ctx=C))
            assert L.md_kv_bytes(ctypes.byref(c), B, C) == t2, (name, B, C)
    c = _lib.config_from(WL.mini_dense())
    assert L.md_kv_bytes(ctypes.byref(c), 0, 64) == 0 and "batch" in _err()
    assert L.md_kv_bytes(ctypes.byref(c), 65, 64) == 0
    assert L.md_kv_bytes(ctypes.byref(c), 2, 80) == 0     # not a multiple of the 32-position V tiles


def test_paged_kv_bytes_match_the_pool_layout():
    """Paged configurations: md_kv_bytes is the page pool (pages in place of
    slots for GQA and MLA layers, one state per slot for delta-rule layers)."""
    L = _lib.lib()
    for name, page, pages in (("mini_dense", 32, 7), ("mini_hybrid", 32, 5), ("dense_27b", 128, 300),
                              ("hybrid_moe", 256, 40), ("mini_moe", 64, 3)):
        w = WL.get(name)
        w = w.replace(max_ctx=(w.max_ctx + page - 1) // page * page, kv_page=page, kv_pages=pages)
        _, total = WL.kv_pool_layout(w)
        c = _lib.config_from(w)
        assert L.md_kv_bytes(ctypes.byref(c), w.max_batch, w.max_ctx) == total, name
        assert L.md_workspace_bytes(ctypes.byref(c)) > 0, name


@pytest.mark.parametrize("page,pages,max_ctx,msg", [
    (48, 4, 96, "power of two"),
    (16, 4, 64, "power of two"),
    (64, 4, 96, "multiple of kv_page"),
    (32, 0, 64, "kv_pages"),
    (0, 4, 64, "kv_pages must be 0"),
])
def test_invalid_paged_configs_are_rejected(page, pages, max_ctx, msg):
    L = _lib.lib()
    c = _cfg(kv_page=page, kv_pages=pages, max_ctx=max_ctx)
    assert L.md_workspace_bytes(ctypes.byref(c)) == 0
    h = P()
    assert L.md_init_model(ctypes.byref(c), None, 0, None, 0, None, ctypes.byref(h)) == _lib.MD_EINVAL
    assert msg in _err()


def test_paged_entry_point_argument_checks():
    L = _lib.lib()
    assert L.md_decode_step_paged(None, None, None, None, None, None, 1, None, None, None) == _lib.MD_EINVAL
    assert "block_table" in _err()
    assert L.md_verify_step_paged(None, None, None, None, None, None, None, None, None, 1, 4, None) == _lib.MD_EINVAL
    assert L.md_kv_copy_pages(None, None, None, None, 0, None) == _lib.MD_EINVAL
    assert L.md_kv_copy_slot(None, None, 0, 1, None) == _lib.MD_EINVAL
    assert "model is NULL" in _err()


@pytest.mark.parametrize("field,value,status", [
    ("max_batch", 65, _lib.MD_EINVAL),
    ("max_batch", 0, _lib.MD_EINVAL),
    ("hidden", 330, _lib.MD_EUNSUPPORTED),
    ("head_dim", 96, _lib.MD_EUNSUPPORTED),
    ("n_kv_heads", 4, _lib.MD_EINVAL),       # 6 q heads are not a multiple of 4
    ("ffn_dim", 100, _lib.MD_EUNSUPPORTED),
    ("max_ctx", 80, _lib.MD_EUNSUPPORTED),    # the V cache is stored in 32-position tiles
    ("attn_kind", 2, _lib.MD_EINVAL),
    ("flags", 1, _lib.MD_EINVAL),
])
def test_invalid_configs_are_rejected(field, value, status):
    L = _lib.lib()
    c = _cfg(**{field: value})
    assert L.md_workspace_bytes(ctypes.byref(c)) == 0
    h = P()
    assert L.md_init_model(ctypes.byref(c), None, 0, None, 0, None, ctypes.byref(h)) == status
    assert _err()
    assert not h.value


def test_moe_and_hybrid_limits():
    L = _lib.lib()
    h = P()
    c = _cfg("mini_moe", n_experts=65)
    assert L.md_init_model(ctypes.byref(c), None, 0, None, 0, None, ctypes.byref(h)) == _lib.MD_EUNSUPPORTED
    c = _cfg("mini_moe", top_k=9)
    assert L.md_init_model(ctypes.byref(c), None, 0, None, 0, None, ctypes.byref(h)) == _lib.MD_EINVAL
    c = _cfg("mini_hybrid", kv_lora=256)
    assert L.md_init_model(ctypes.byref(c), None, 0, None, 0, None, ctypes.byref(h)) == _lib.MD_EUNSUPPORTED
    c = _cfg("mini_hybrid", kda_dv=48)
    assert L.md_init_model(ctypes.byref(c), None, 0, None, 0, None, ctypes.byref(h)) == _lib.MD_EUNSUPPORTED


def test_kv_head_count_fits_the_attention_counters():
    """The GQA attention phase counts each (row, kv head)'s finished chunks in
    one word of a sync point: 288 words for up to 8 rows (8 x 36 kv heads
    fit, 37 do not: they would spill into the next layer's counters), 544
    for up to 64 rows (max_batch > 8: 8 kv heads fit, 9 do not)."""
    L = _lib.lib()
    h = P()
    ok = _cfg("mini_dense", n_q_heads=36, n_kv_heads=36, head_dim=64)
    assert L.md_workspace_bytes(ctypes.byref(ok)) > 0
    bad = _cfg("mini_dense", n_q_heads=37, n_kv_heads=37, head_dim=64)
    assert L.md_workspace_bytes(ctypes.byref(bad)) == 0
    assert L.md_init_model(ctypes.byref(bad), None, 0, None, 0, None, ctypes.byref(h)) == _lib.MD_EUNSUPPORTED
    assert "kv heads" in _err()
    ok = _cfg("mini_dense", max_batch=64, n_q_heads=8, n_kv_heads=8, head_dim=64)
    assert L.md_workspace_bytes(ctypes.byref(ok)) > 0
    bad = _cfg("mini_dense", max_batch=9, n_q_heads=9, n_kv_heads=9, head_dim=64)
    assert L.md_workspace_bytes(ctypes.byref(bad)) == 0
    assert "kv heads" in _err()


def test_wide_batch_workspace_and_expert_limit():
    """max_batch > 8 runs on the 64-row kernel build: the activation buffers
    hold 64 token rows whatever the model's max_batch, and the routed-expert
    union of a step may reach min(n_experts, 64 * top_k) experts, two matrices
    each, of the 72 a phase's tables hold."""
    L = _lib.lib()
    h = P()
    w8 = L.md_workspace_bytes(ctypes.byref(_cfg("mini_dense", max_batch=8)))
    w9 = L.md_workspace_bytes(ctypes.byref(_cfg("mini_dense", max_batch=9)))
    w64 = L.md_workspace_bytes(ctypes.byref(_cfg("mini_dense", max_batch=64)))
    assert 0 < w8 < w9 == w64
    assert L.md_workspace_bytes(ctypes.byref(_cfg("mini_moe", max_batch=64))) > 0   # 12 experts
    c = _cfg("mini_moe", n_experts=37, max_batch=8)       # union <= 8 * 3 = 24 experts
    assert L.md_workspace_bytes(ctypes.byref(c)) > 0
    c = _cfg("mini_moe", n_experts=37, max_batch=16)      # union up to all 37
    assert L.md_workspace_bytes(ctypes.byref(c)) == 0
    assert L.md_init_model(ctypes.byref(c), None, 0, None, 0, None, ctypes.byref(h)) == _lib.MD_EUNSUPPORTED
    assert "distinct experts" in _err()


def test_init_argument_checks_before_any_device_call():
    L = _lib.lib()
    c = _cfg()
    h = P()
    assert L.md_init_model(ctypes.byref(c), None, 0, None, 0, None, None) == _lib.MD_EINVAL
    assert L.md_init_model(ctypes.byref(c), None, 0, None, 0, None, ctypes.byref(h)) == _lib.MD_EINVAL
    assert "weight pointers" in _err()
    n = L.md_weight_count(ctypes.byref(c))
    ptrs = (P * n)(*([0] * n))
    assert L.md_init_model(ctypes.byref(c), ptrs, n, None, 0, None, ctypes.byref(h)) == _lib.MD_EINVAL
    assert "NULL" in _err()


def test_null_model_and_bad_step_arguments():
    L = _lib.lib()
    assert L.md_decode_step(None, None, None, None, None, 1, None, None, None) == _lib.MD_EINVAL
    assert L.md_decode_step_multilaunch(None, None, None, None, None, 1, None, None, None) == _lib.MD_EINVAL
    assert L.md_decode_step_noalloc(None, None, None, None, None, 1, None, None, None) == _lib.MD_EINVAL
    assert L.md_verify_step(None, None, None, None, None, None, None, None, 2, 8, None) == _lib.MD_EUNSUPPORTED
    assert L.md_verify_step(None, None, None, None, None, None, None, None, 1, 9, None) == _lib.MD_EINVAL
    assert L.md_verify_step(None, None, None, None, None, None, None, None, 1, 1, None) == _lib.MD_EINVAL
    assert L.md_get_device_status(None) == _lib.MD_EINVAL
    assert L.md_set_trace(None, None, 0) == _lib.MD_EINVAL
    assert L.md_grid_size(None) == 0
    L.md_free_model(None)


def test_pack_argument_checks():
    L = _lib.lib()
    assert L.md_pack_weight(None, None, 16, 32, None) == _lib.MD_EINVAL
    assert L.md_pack_weight(P(16), P(32), 16, 33, None) == _lib.MD_EINVAL
    assert L.md_pack_weight(P(8), P(32), 16, 32, None) == _lib.MD_EINVAL


def test_workspace_sizes():
    """The workspace holds one activation buffer per use within a step (two
    norm inputs per layer plus the final one, and per layer the attention
    output and FFN hidden): it grows with the layer count by at least those
    buffers, and the benchmark models stay within the 32-bit offsets the
    kernels use."""
    L = _lib.lib()
    for name in ("dense_27b", "hybrid_moe", "verify_hybrid", "small_moe"):
        c = _cfg(name)
        assert L.md_workspace_bytes(ctypes.byref(c)) < 0xFFFFFF00, name
    w = WL.get("mini_dense")
    c1, c2 = _cfg("mini_dense", n_layers=3), _cfg("mini_dense", n_layers=6)
    grow = L.md_workspace_bytes(ctypes.byref(c2)) - L.md_workspace_bytes(ctypes.byref(c1))
    per_layer = 2 * (2 * 2 * 8 * w.hidden) + 2 * 2 * 8 * w.n_q_heads * w.head_dim + 2 * 2 * 8 * w.ffn_dim
    assert grow >= 3 * per_layer
