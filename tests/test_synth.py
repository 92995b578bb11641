"""The seeded input generator: determinism, independence of tensors, moments."""
import numpy as np

import synth
from synth import workloads as WL


def test_same_seed_same_bytes_and_offsets():
    a = synth.normal_bf16(1000, "L0.wq", 5000, 0.02)
    b = synth.normal_bf16(1000, "L0.wq", 5000, 0.02)
    assert np.array_equal(a, b)
    # any slice can be drawn on its own
    c = synth.normal_bf16(1000, "L0.wq", 1000, 0.02, offset=2500)
    assert np.array_equal(c, a[2500:3500])
    # other names / seeds give other streams
    assert not np.array_equal(a, synth.normal_bf16(1000, "L0.wk", 5000, 0.02))
    assert not np.array_equal(a, synth.normal_bf16(1001, "L0.wq", 5000, 0.02))


def test_moments():
    n = 1 << 20
    for sigma in (0.02, 0.1, 1.0):
        z = synth.bf16_bits_to_f32(synth.normal_bf16(7, "m", n, sigma)).astype(np.float64)
        assert abs(z.mean()) < 4 * sigma / np.sqrt(n)
        assert abs(z.std() / sigma - 1) < 0.01
        f = synth.normal_f32(7, "m", n, sigma).astype(np.float64)
        assert abs(f.std() / sigma - 1) < 0.005
        # bf16 draw is the nearest-even rounding of the fp32 draw
        assert np.array_equal(synth.normal_bf16(7, "m", 4096, sigma), synth.f32_to_bf16_bits(f[:4096].astype(np.float32)))


def test_tokens_in_range_and_spread():
    t = synth.uniform_i32(4000, "tokens.step0", 100000, 1000)
    assert t.min() >= 0 and t.max() < 1000
    counts = np.bincount(t, minlength=1000)
    assert counts.min() > 50 and counts.max() < 160


def test_inventory_shapes_dense_27b():
    w = WL.dense_27b()
    total = synth.workloads.weight_bytes(w)
    # 22.70 B parameters, untied embedding and LM head
    assert abs(total / 2 / 1e9 - 22.70) < 0.01
    lay, kvb = synth.workloads.kv_layout(w)
    assert len(lay) == 64 and lay[0][3] == (8, 8, 4352, 128)


def test_inventory_shapes_hybrid():
    w = WL.hybrid_moe()
    kinds = [w.layer_kind(l) for l in range(w.n_layers)]
    assert kinds.count("mla") == 23 and kinds.count("kda") == 69 and kinds[3] == "mla"
    assert abs(synth.workloads.weight_bytes(w) / 2 / 1e9 - 80.71) < 0.02
