"""GPU parity: the megakernel step against the oracle on identical seeded
inputs (the oracle never sees anything the GPU produced)."""
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


def _model(w, overrides=None):
    from decode_megakernel_md_amd.model import DeviceModel
    return DeviceModel(w, overrides=overrides)


def test_device_draws_match_host_draws(torch_cuda):
    torch = torch_cuda
    w = WL.mini_dense()
    m = _model(w)
    for s, o in zip(m.specs[:6], m.offsets[:6]):
        got = m.wbuf[o:o + s.numel * 2].cpu().numpy().view(np.uint16).reshape(s.rows, s.cols)
        assert np.array_equal(got, synth.weight_host(w, s)), s.name
    kv = m.kv_host()
    for l in range(w.n_layers):
        assert np.array_equal(kv[l], synth.kv_layer_host(w, l))


@pytest.mark.parametrize("name,B", [("tiny_dense", 1), ("mini_dense", 1), ("mini_dense", 3), ("mini_dense", 8)])
def test_decode_step_matches_oracle(torch_cuda, name, B):
    w = WL.get(name)
    m = _model(w)
    toks = synth.tokens(w, B)
    # ragged positions: every sequence has its own history length
    pos = [min(w.context + 5 * b, w.max_ctx - 1) if b % 2 == 0 else max(w.context - 7 * b, 0) for b in range(B)]
    print(f"case {name} B={B} pos={pos}", flush=True)
    g = GU.run_gpu_step(m, toks, pos)
    o, kv_ref = GU.run_oracle_step(w, toks, pos)
    err = GU.compare_step(w, g, o, f"{name} B={B}")
    n_ulp = GU.compare_kv_rows(w, m.kv_host(), kv_ref, pos, B)
    print(f"  max|dlogit|/rms = {err:.2e}; cache entries 1 ulp apart: {n_ulp}")


def test_zero_layer_weights_identity(torch_cuda):
    """Zeroed layer matrices: the residual stays the embedding row, so the
    logits equal the LM head applied to the normalised embedding."""
    w = WL.mini_dense()
    over = {t.name: np.zeros((t.rows, t.cols), np.uint16) for t in synth.tensor_inventory(w)
            if t.kind != "gain" and t.name not in ("embed", "lm_head")}
    m = _model(w, overrides=over)
    toks = synth.tokens(w, 2)
    pos = [3, 40]
    g = GU.run_gpu_step(m, toks, pos)
    o, _ = GU.run_oracle_step(w, toks, pos, overrides=over)
    GU.compare_step(w, g, o, "zero-weights")


def test_repeated_steps_are_bitwise_deterministic(torch_cuda):
    torch = torch_cuda
    w = WL.mini_dense()
    m = _model(w)
    toks = synth.tokens(w, 4)
    pos = [10, 20, 30, 40]
    a = GU.run_gpu_step(m, toks, pos)
    m.reset_kv()
    b = GU.run_gpu_step(m, toks, pos)
    assert np.array_equal(a["logits"], b["logits"])
