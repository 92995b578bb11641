"""GPU: decode steps of more than 8 sequences (models with max_batch up to
64, which run on the library's 64-row kernel build) against the oracle.

Kimi K3 post, section "Future work" (higher concurrency, where the vector
work grows with the batch): every weight is still read once per step, its
rows multiplied by 16-token B tiles.  The cases span one tile plus a ragged
one (B = 23), ragged counts across several tiles (37), and the full 64
rows; the models have dense, MoE (union of chosen experts) and hybrid
(delta-rule + MLA) layers."""
import numpy as np
import pytest

import synth
from synth import workloads as WL
from tests import gpu_util as GU

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def wide(w, max_batch=64):
    return w.replace(name=w.name + f"_b{max_batch}", max_batch=max_batch)


def ragged_positions(w, B):
    """Positions spread over the cache: some near the end, some at 0."""
    rng = np.random.default_rng(100 + B)
    pos = rng.integers(0, w.max_ctx, size=B)
    pos[0] = w.context
    pos[-1] = 0
    if B > 2:
        pos[1] = w.max_ctx - 1
    return [int(x) for x in pos]


def _model(w, bt=None):
    from decode_megakernel_md_amd.model import DeviceModel
    return DeviceModel(w, block_table=bt)


@pytest.mark.parametrize("name,B", [("mini_dense", 9), ("mini_dense", 23), ("mini_dense", 37), ("mini_dense", 64),
                                    ("mini_moe", 40), ("mini_moe", 64), ("mini_hybrid", 23), ("mini_hybrid", 64)])
def test_wide_decode_matches_oracle(torch_cuda, name, B):
    w = wide(WL.get(name))
    toks = synth.tokens(w, B)
    pos = ragged_positions(w, B)
    print(f"case {w.name} B={B}", flush=True)
    m = _model(w)
    g = GU.run_gpu_step(m, toks, pos)
    o, kv_ref = GU.run_oracle_step(w, toks, pos)
    err = GU.compare_step(w, g, o, f"{w.name} B={B}")
    GU.compare_kv_rows(w, m.kv_host(), kv_ref, pos, B)
    print(f"  max|dlogit|/rms = {err:.2e}")
    m.close()


def test_wide_multilaunch_matches_the_megakernel(torch_cuda):
    """The one-launch-per-phase step of the 64-row build gives the same
    logits as its megakernel, bit for bit (same phases, same grid)."""
    w = wide(WL.mini_hybrid())
    B = 41
    toks = synth.tokens(w, B)
    pos = ragged_positions(w, B)
    print(f"case {w.name} B={B} multilaunch", flush=True)
    m = _model(w)
    g1 = GU.run_gpu_step(m, toks, pos, multilaunch=True)
    m.reset_kv()
    g0 = GU.run_gpu_step(m, toks, pos)
    assert np.array_equal(g0["logits"], g1["logits"])
    assert np.array_equal(g0["next"], g1["next"])
    m.close()


def test_wide_paged_decode_matches_oracle(torch_cuda):
    """A paged cache on the 64-row build (pages of 32 positions, shuffled)."""
    from tests.test_gpu_paged import paged, shuffled_table
    w = paged(wide(WL.mini_hybrid(), 48), 32)
    B = 48
    toks = synth.tokens(w, B)
    pos = ragged_positions(w, B)
    print(f"case {w.name} B={B}", flush=True)
    m = _model(w, shuffled_table(w, 5))
    g = GU.run_gpu_step(m, toks, pos)
    o, kv_ref = GU.run_oracle_step(w, toks, pos)
    GU.compare_step(w, g, o, f"{w.name} B={B}")
    GU.compare_kv_rows(w, m.kv_host(), kv_ref, pos, B)
    m.close()


@pytest.mark.parametrize("name,B", [("dense_27b", 64), ("hybrid_moe", 32)])
def test_wide_full_shape_layers_match_oracle(torch_cuda, name, B):
    """The two large models at full width and context (4 layers; the hybrid
    model's 4th is MLA over 8192 positions), max_batch 64, in bench.py's
    launch configuration."""
    w = wide(WL.get(name).replace(n_layers=4))
    toks = synth.tokens(w, B)
    pos = [w.context - 37 * b for b in range(B)]
    print(f"case {w.name} 4 layers B={B}", flush=True)
    m = _model(w)
    g = GU.run_gpu_step(m, toks, pos)
    o, kv_ref = GU.run_oracle_step(w, toks, pos)
    err = GU.compare_step(w, g, o, f"{w.name} B={B}")
    GU.compare_kv_rows(w, m.kv_host(), kv_ref, pos, B)
    print(f"  max|dlogit|/rms = {err:.2e}")
    m.close()


def test_wide_model_refuses_verify(torch_cuda):
    """The verify step runs on the 8-row build only: a model with
    max_batch > 8 reports MD_EUNSUPPORTED and launches nothing."""
    import ctypes
    torch = torch_cuda
    from decode_megakernel_md_amd import _lib
    w = wide(WL.mini_dense(), 16)
    m = _model(w)
    dev = m.device
    t = torch.zeros(8, dtype=torch.int32, device=dev)
    p = torch.tensor([w.context], dtype=torch.int32, device=dev)
    logits = torch.empty((8, w.vocab), dtype=torch.float32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    L = _lib.lib()
    st = L.md_verify_step(m.handle, ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(p.data_ptr()),
                          ctypes.c_void_p(m.kv.data_ptr()), ctypes.c_void_p(logits.data_ptr()),
                          ctypes.c_void_p(acc.data_ptr()), ctypes.c_void_p(nxt.data_ptr()), None, 1, 8,
                          ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == _lib.MD_EUNSUPPORTED and "max_batch" in L.md_last_error().decode()
    m.close()
