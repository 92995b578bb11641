"""GPU: the in-kernel phase trace (md_set_trace).  A traced step computes the
same logits as an untraced one, bit for bit, and every workgroup's stamps
are complete and in order: the step's start, then for every phase the end of
its wait before the end of its work, and no wait on a sync point ending
before the last workgroup has arrived there."""
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


@pytest.mark.parametrize("name,B,max_batch", [("mini_hybrid", 3, 8), ("mini_dense", 5, 8), ("mini_moe", 11, 16)])
def test_traced_step_matches_and_stamps_are_ordered(torch_cuda, name, B, max_batch):
    from decode_megakernel_md_amd.model import DeviceModel
    from decode_megakernel_md_amd.trace import Tracer, phase_names
    w = WL.get(name)
    if max_batch != w.max_batch:
        w = w.replace(name=w.name + f"_b{max_batch}", max_batch=max_batch)
    toks = synth.tokens(w, B)
    pos = [w.context - b for b in range(B)]
    print(f"case {w.name} B={B} traced", flush=True)
    m = DeviceModel(w)
    g0 = GU.run_gpu_step(m, toks, pos)
    m.reset_kv()
    tr = Tracer(m)
    g1 = GU.run_gpu_step(m, toks, pos)
    tr.stop()
    assert np.array_equal(g0["logits"], g1["logits"])
    assert np.array_equal(g0["next"], g1["next"])
    raw = tr.buf.cpu().numpy()
    names = phase_names(w)
    ns = len(names)
    start = raw[:, -1]
    ends, wends = raw[:, 0: 2 * ns: 2], raw[:, 1: 2 * ns - 1: 2]
    assert np.all(start > 0) and np.all(ends > 0) and np.all(wends > 0)
    # phase 0 (embedding) has no wait; phase s >= 1 waits on sync point s-1
    assert np.all(ends[:, 0] >= start)
    assert np.all(wends >= ends[:, :-1]), "a wait ended before this workgroup's own arrival"
    assert np.all(ends[:, 1:] >= wends), "a phase ended before its wait"
    # the last arrival of sync point s precedes every wait end on it (but
    # MoE phase A has no arrival: the next phase validates the router
    # logits' tags instead of waiting)
    full = np.array([n != "moe_a" for n in names[:-1]])
    assert np.all(wends.min(axis=0)[full] >= ends[:, :-1].max(axis=0)[full])
    out, total = tr.summary(names)
    assert total > 0 and set(out) == set(names)
    m.close()
