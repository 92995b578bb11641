"""GPU: the allocation-free decode step (md_decode_step_noalloc, scratch from
the library's static device array) against md_decode_step (scratch from the
model's workspace), through the C ABI.  Both run the same kernels, so their
logits, greedy tokens, expert ids and cache / state updates must be bitwise
equal.  Two calls in a row on each model, the second with a smaller batch,
with another model's call in between (the array keeps the last call's
contents), and a model whose step needs more scratch than the array holds is
refused with MD_ENOMEM before anything is enqueued."""
import numpy as np
import pytest

import synth
from synth import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _step(m, toks, pos, noalloc):
    import torch
    w, dev = m.w, m.device
    B = len(toks)
    t = torch.tensor(np.asarray(toks, dtype=np.int32), device=dev)
    p = torch.tensor(np.asarray(pos, dtype=np.int32), device=dev)
    logits = torch.full((B, w.vocab), float("nan"), dtype=torch.float32, device=dev)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=dev)
    ids = torch.full((w.n_layers, B, w.top_k), -7, dtype=torch.int32, device=dev) if w.is_moe else None
    m.decode(t, p, logits, nxt, ids, noalloc=noalloc)
    torch.cuda.synchronize(dev)
    m.device_status()
    return logits.cpu().numpy(), nxt.cpu().numpy(), (ids.cpu().numpy() if ids is not None else None)


def _check_pair(m, toks, pos, label):
    """The workspace step and the allocation-free step from the same cache
    state: equal outputs and equal caches afterwards.  Leaves the cache as the
    allocation-free step wrote it."""
    kv0 = m.kv.clone()
    a = _step(m, toks, pos, noalloc=False)
    kv_a = m.kv.clone()
    m.kv.copy_(kv0)
    print(f"case {label}: noalloc B={len(toks)} pos={pos}", flush=True)
    b = _step(m, toks, pos, noalloc=True)
    assert np.array_equal(a[0], b[0]), f"{label}: logits differ"
    assert np.array_equal(a[1], b[1]), f"{label}: greedy tokens differ"
    if a[2] is not None:
        assert np.array_equal(a[2], b[2]), f"{label}: expert ids differ"
    assert bool((m.kv == kv_a).all()), f"{label}: cache / state updates differ"


def test_noalloc_step_equals_workspace_step(torch_cuda):
    from decode_megakernel_md_amd.model import DeviceModel
    wa, wb = WL.mini_moe(), WL.mini_hybrid()
    ma, mb = DeviceModel(wa), DeviceModel(wb)
    _check_pair(ma, synth.tokens(wa, 6), [wa.context - 3 * b for b in range(6)], "mini_moe 1")
    _check_pair(mb, synth.tokens(wb, 5), [wb.context - 2 * b for b in range(5)], "mini_hybrid 1")
    # the second call of each model: a smaller batch, later positions, after the
    # other model's call has left its own contents in the array
    _check_pair(ma, synth.tokens(wa.replace(seed_base=77), 2), [wa.context + 1, wa.context - 2], "mini_moe 2")
    _check_pair(mb, synth.tokens(wb.replace(seed_base=78), 1), [wb.context + 1], "mini_hybrid 2")
    ma.close()
    mb.close()


def test_noalloc_refuses_a_step_larger_than_the_array(torch_cuda):
    """A hybrid model with 12 small-hidden layers of 32 delta-rule heads: its
    workspace (dominated by the verify snapshots of 9 such layers) exceeds
    the 128 MiB array, so the allocation-free step is refused up front and
    the output buffers are left untouched."""
    import ctypes
    torch = torch_cuda
    from decode_megakernel_md_amd import _lib
    from decode_megakernel_md_amd.model import DeviceModel
    w = WL.mini_hybrid().replace(name="wide_state_hybrid", n_layers=12, kda_heads=32, kda_dk=128, kda_dv=128)
    L = _lib.lib()
    need = L.md_workspace_bytes(ctypes.byref(_lib.config_from(w)))
    assert need > (128 << 20), need
    m = DeviceModel(w)
    dev = m.device
    t = torch.tensor(synth.tokens(w, 1), dtype=torch.int32, device=dev)
    p = torch.tensor([w.context], dtype=torch.int32, device=dev)
    logits = torch.full((1, w.vocab), -3.0, dtype=torch.float32, device=dev)
    st = L.md_decode_step_noalloc(m.handle, ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(p.data_ptr()),
                                  ctypes.c_void_p(m.kv.data_ptr()), ctypes.c_void_p(logits.data_ptr()), 1, None, None,
                                  ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == _lib.MD_ENOMEM
    assert "static scratch" in L.md_last_error().decode()
    torch.cuda.synchronize(dev)
    assert bool((logits == -3.0).all())
    # the workspace step of the same model still runs
    m.decode(t, p, logits, None, None)
    torch.cuda.synchronize(dev)
    m.device_status()
    assert bool(torch.isfinite(logits).all())
    m.close()
