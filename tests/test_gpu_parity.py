"""GPU parity: the megakernel step against the oracle on identical seeded
inputs (the oracle never sees anything the GPU produced)."""
import os

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


def unpack_tiled(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Inverse of the tiled layout md.h documents, written from that text:
    block (t, s) at (t*S + s)*1024 bytes, chunk c -> row 16t + 4*(c//16) + c%4,
    columns 32s + 8*((c%16)//4) .. +7."""
    S, T = cols // 32, (rows + 15) // 16
    blocks = raw.view(np.uint16).reshape(T, S, 64, 8)
    out = np.zeros((T * 16, cols), dtype=np.uint16)
    for c in range(64):
        rr = 4 * (c // 16) + c % 4
        j = (c % 16) // 4
        for t in range(T):
            out[t * 16 + rr].reshape(S, 32)[:, 8 * j:8 * j + 8] = blocks[t, :, c, :]
    assert not out[rows:].any(), "padding rows must be zero"
    return out[:rows]


def test_device_draws_match_host_draws(torch_cuda):
    torch = torch_cuda
    w = WL.mini_dense()
    m = _model(w)
    for s, o, n, pk in list(zip(m.specs, m.offsets, m.sizes, m.packed))[:8]:
        raw = m.wbuf[o:o + n].cpu().numpy()
        got = unpack_tiled(raw, s.rows, s.cols) if pk else raw.view(np.uint16).reshape(s.rows, s.cols)
        assert np.array_equal(got, synth.weight_host(w, s)), s.name
    kv = m.kv_host()
    for l in range(w.n_layers):
        assert np.array_equal(kv[l], synth.kv_layer_host(w, l))


@pytest.mark.parametrize("name,B", [("tiny_dense", 1), ("mini_dense", 1), ("mini_dense", 3), ("mini_dense", 8),
                                    ("mini_moe", 1), ("mini_moe", 3), ("mini_moe", 8),
                                    ("small_moe", 1), ("small_moe", 8),
                                    ("mini_hybrid", 1), ("mini_hybrid", 3), ("mini_hybrid", 8)])
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


@pytest.mark.parametrize("B", [1, 5])
def test_moe_without_shared_expert_matches_oracle(torch_cuda, B):
    """A MoE model with no shared expert: every workgroup streams router rows
    and every workgroup publishes them (the other layout of the router's
    sync point), then the routed experts as usual."""
    w = WL.mini_moe().replace(name="mini_moe_noshared", n_shared=0)
    m = _model(w)
    toks = synth.tokens(w, B)
    pos = [max(w.context - 9 * b, 0) for b in range(B)]
    print(f"case {w.name} B={B} pos={pos}", flush=True)
    g = GU.run_gpu_step(m, toks, pos)
    o, kv_ref = GU.run_oracle_step(w, toks, pos)
    err = GU.compare_step(w, g, o, f"{w.name} B={B}")
    GU.compare_kv_rows(w, m.kv_host(), kv_ref, pos, B)
    print(f"  max|dlogit|/rms = {err:.2e}")
    m.close()


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


def test_zero_router_picks_lowest_ids(torch_cuda):
    """Zeroed layer matrices in a MoE model: every router logit is 0, all
    experts tie, and the tie rule picks experts 0..k-1 for every token."""
    w = WL.mini_moe()
    over = {t.name: np.zeros((t.rows, t.cols), np.uint16) for t in synth.tensor_inventory(w)
            if t.kind != "gain" and t.name not in ("embed", "lm_head")}
    m = _model(w, overrides=over)
    toks = synth.tokens(w, 3)
    pos = [3, 40, 7]
    g = GU.run_gpu_step(m, toks, pos)
    want = np.broadcast_to(np.arange(w.top_k, dtype=np.int32), g["expert_ids"].shape)
    assert np.array_equal(g["expert_ids"], want)
    o, _ = GU.run_oracle_step(w, toks, pos, overrides=over)
    GU.compare_step(w, g, o, "zero-weights moe")


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


@pytest.mark.parametrize("name,B", [("mini_dense", 3), ("mini_moe", 3), ("mini_hybrid", 3)])
def test_chained_steps_match_oracle(torch_cuda, name, B):
    """Several greedy decode steps in a row, each a launch of its own: the
    GPU's cache rows and delta-rule states advance in place and its sync
    counters alternate between their two banks, while the oracle advances its
    own copy of the cache; every step's logits, tokens and expert ids must
    match, and so must the caches and states at the end."""
    from tests.harness import HostWeights, host_kv
    from oracle import step as ostep
    w = WL.get(name)
    m = _model(w)
    W = HostWeights(w)
    kv_ref = host_kv(w)
    toks = list(synth.tokens(w, B))
    pos0 = [w.context - 4 * b for b in range(B)]
    steps = 5
    for s in range(steps):
        pos = [p + s for p in pos0]
        print(f"case {name} B={B} step {s} pos={pos} toks={toks}", flush=True)
        g = GU.run_gpu_step(m, toks, pos)
        o = ostep.decode_step(w, W, np.asarray(toks), np.asarray(pos), kv_ref)
        GU.compare_step(w, g, o, f"{name} step {s}")
        toks = [int(t) for t in o["next"]]
    kvg = m.kv_host()
    for s in range(steps):
        GU.compare_kv_rows(w, kvg, kv_ref, [p + s for p in pos0], B)


def _greedy_drafts(w, W, kv, p0, accept, n=8):
    """Tokens t_0..t_{n-1}: the anchor, then the oracle's greedy continuation
    for accept-1 tokens, then (when accept < n) a token that differs from the
    greedy one at that point, then arbitrary tokens.  Verifying them must
    accept exactly `accept` tokens."""
    from oracle import step as ostep
    from tests.harness import kv_copy
    anchor = int(synth.tokens(w, 1)[0])
    seq = [anchor]
    kv_g = kv_copy(kv)
    for j in range(min(accept, n - 1)):
        o = ostep.decode_step(w, W, [seq[-1]], [p0 + j], kv_g)
        seq.append(int(o["next"][0]))
    if accept < n:
        seq[accept] = (seq[accept] + 1) % w.vocab
    rng = np.random.default_rng(5000 + accept)
    while len(seq) < n:
        seq.append(int(rng.integers(0, w.vocab)))
    return seq[:n]


def _gpu_verify(m, toks, p0):
    """One verify launch through the C ABI: logits [n][V], expert ids
    [L][n][k] (MoE models; else None), accepted length, next token."""
    import torch
    w, dev, n = m.w, m.device, len(toks)
    t = torch.tensor([toks], dtype=torch.int32, device=dev)
    pp = torch.tensor([p0], dtype=torch.int32, device=dev)
    logits = torch.full((1, n, w.vocab), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((1,), -7, dtype=torch.int32, device=dev)
    nxt = torch.full((1,), -7, dtype=torch.int32, device=dev)
    ids = torch.full((w.n_layers, n, w.top_k), -7, dtype=torch.int32, device=dev) if w.is_moe else None
    m.verify(t, pp, logits, acc, nxt, ids)
    torch.cuda.synchronize(dev)
    m.device_status()
    return (logits.cpu().numpy()[0], ids.cpu().numpy() if ids is not None else None, int(acc.cpu()[0]),
            int(nxt.cpu()[0]))


@pytest.mark.parametrize("name", ["mini_dense", "mini_moe", "mini_hybrid"])
@pytest.mark.parametrize("accept", [1, 3, 8])
def test_verify_matches_oracle(torch_cuda, name, accept):
    torch = torch_cuda
    from oracle import step as ostep
    from tests.harness import HostWeights, host_kv, kv_copy
    w = WL.get(name)
    n = 8
    p0 = w.max_ctx - n - 3
    W = HostWeights(w)
    kv = host_kv(w)
    toks = _greedy_drafts(w, W, kv, p0, accept, n)
    print(f"case {name} accept={accept} p0={p0} toks={toks}", flush=True)
    kv_ref = kv_copy(kv)
    v = ostep.verify_step(w, W, np.array([toks]), np.array([p0]), kv_ref)
    assert int(v["accept_len"][0]) == accept
    m = _model(w)
    logits, ids, acc, nxt = _gpu_verify(m, toks, p0)
    assert acc == accept
    err = GU.compare_verify(w, logits, ids, acc, nxt, v, f"verify {name} a={accept}")
    kvg = m.kv_host()
    for j in range(n):
        GU.compare_kv_rows(w, kvg, kv_ref, [p0 + j], 1)
    print(f"  max|dlogit|/rms = {err:.2e}")


@pytest.mark.parametrize("name,B", [("mini_dense", 3), ("mini_moe", 8), ("mini_hybrid", 3)])
def test_multilaunch_equals_megakernel(torch_cuda, name, B):
    """The one-launch-per-phase baseline runs the same device code: its
    logits, tokens and expert ids are bitwise those of the megakernel, and
    both match the oracle."""
    w = WL.get(name)
    m = _model(w)
    toks = synth.tokens(w, B)
    pos = [w.context - 3 * b for b in range(B)]
    a = GU.run_gpu_step(m, toks, pos)
    m.reset_kv()
    b = GU.run_gpu_step(m, toks, pos, multilaunch=True)
    assert np.array_equal(a["logits"], b["logits"])
    assert np.array_equal(a["next"], b["next"])
    if "expert_ids" in a:
        assert np.array_equal(a["expert_ids"], b["expert_ids"])
    o, _ = GU.run_oracle_step(w, toks, pos)
    GU.compare_step(w, b, o, f"multilaunch {name}")


@pytest.mark.slow
@pytest.mark.parametrize("name,B", [("dense_27b", 1), ("dense_27b", 2), ("dense_27b", 4), ("dense_27b", 8),
                                    ("hybrid_moe", 1), ("hybrid_moe", 8)])
def test_full_shape_layers_match_oracle(torch_cuda, name, B):
    """The two large models at their full layer shapes, vocabulary and
    context, in the launch configuration bench.py times (grid = CU count,
    same batch), reduced to 4 layers so that the fp64 oracle finishes in
    seconds (the hybrid model's 4 layers are 3 delta-rule layers and 1 MLA
    layer, each with the 16-expert MoE)."""
    w = WL.get(name).replace(n_layers=4)
    toks = synth.tokens(w, B)
    pos = [w.context - 97 * b for b in range(B)]
    print(f"case {name} 4 layers B={B} pos={pos}", flush=True)
    m = _model(w)
    g = GU.run_gpu_step(m, toks, pos)
    o, kv_ref = GU.run_oracle_step(w, toks, pos)
    err = GU.compare_step(w, g, o, f"{name} B={B}")
    GU.compare_kv_rows(w, m.kv_host(), kv_ref, pos, B)
    print(f"  max|dlogit|/rms = {err:.2e}")


@pytest.mark.slow
@pytest.mark.parametrize("name,B", [("dense_27b", 1), ("dense_27b", 8), ("hybrid_moe", 1)])
def test_full_depth_step_matches_oracle(torch_cuda, name, B):
    """A whole decode step of the 64-layer dense model (batches 1 and 8) and
    of the 92-layer hybrid MoE (batch 1) at full context, in bench.py's
    launch configuration, against the oracle's unfused layer-by-layer step:
    greedy tokens and every layer's expert ids bit-exact, logits within
    2e-2 x row RMS, every new cache row and delta-rule state within its
    tolerance.  The GPU model is freed before the oracle runs (its weights are
    drawn again on the host, layer by layer, from the same seeded generator)."""
    torch = torch_cuda
    w = WL.get(name)
    toks = synth.tokens(w, B)
    pos = [w.context - 97 * b for b in range(B)]
    print(f"case {name} full depth ({w.n_layers} layers) B={B} pos={pos}", flush=True)
    m = _model(w)
    g = GU.run_gpu_step(m, toks, pos)
    rows = GU.kv_rows_dev(m, pos, B)
    m.close()
    del m
    torch.cuda.empty_cache()
    o, kv_ref = GU.run_oracle_step(w, toks, pos)
    err = GU.compare_step(w, g, o, f"{name} full depth B={B}")
    GU.compare_kv_rows(w, rows, kv_ref, pos, B)
    print(f"  max|dlogit|/rms = {err:.2e}", flush=True)


@pytest.mark.slow
@pytest.mark.skipif(not os.environ.get("MD_FULL_DEPTH_B8"), reason="hybrid 92 layers at batch 8: about 6 minutes of "
                    "fp64 oracle (8 x 23 MLA layers over 8192 positions); run with MD_FULL_DEPTH_B8=1")
def test_full_depth_hybrid_batch8_matches_oracle(torch_cuda):
    test_full_depth_step_matches_oracle(torch_cuda, "hybrid_moe", 8)


@pytest.mark.slow
@pytest.mark.parametrize("accept", [3, 6])
def test_full_shape_verify_matches_oracle(torch_cuda, accept):
    """Verify of 1 anchor + 7 drafts on the hybrid model at its full layer
    shapes, vocabulary and context (8192), in bench.py's launch configuration
    (4 layers: 3 delta-rule and 1 MLA, each with the 16-expert MoE, so that
    the a-1 greedy steps and the 8 sequential verify rows of the fp64 oracle
    finish in under a minute), at the acceptance lengths bench.py times:
    drafts are the oracle's greedy continuation for a-1 tokens, then a token
    that differs from the greedy one.  The acceptance length, the next token,
    every row's greedy token and expert ids, all 8 logit rows, the new cache
    rows and the committed delta-rule states must match the oracle."""
    torch = torch_cuda
    from oracle import step as ostep
    from tests.harness import HostWeights, host_kv, kv_copy
    w = WL.get("verify_hybrid").replace(n_layers=4)
    n = 8
    p0 = w.context
    W = HostWeights(w)
    kv = host_kv(w)
    toks = _greedy_drafts(w, W, kv, p0, accept, n)
    print(f"case verify_hybrid 4 layers accept={accept} p0={p0} toks={toks}", flush=True)
    kv_ref = kv_copy(kv)
    v = ostep.verify_step(w, W, np.array([toks]), np.array([p0]), kv_ref)
    assert int(v["accept_len"][0]) == accept
    m = _model(w)
    logits, ids, acc, nxt = _gpu_verify(m, toks, p0)
    assert acc == accept
    err = GU.compare_verify(w, logits, ids, acc, nxt, v, f"verify_hybrid 4 layers a={accept}")
    kvg = m.kv_host()
    for j in range(n):
        GU.compare_kv_rows(w, kvg, kv_ref, [p0 + j], 1)
    print(f"  max|dlogit|/rms = {err:.2e}")


@pytest.mark.slow
@pytest.mark.skipif(not os.environ.get("MD_LONG_CHAIN"), reason="256 chained full-width steps: about 2-3 minutes of "
                    "fp64 oracle; run with MD_LONG_CHAIN=1")
@pytest.mark.parametrize("B,steps,sampled", [(1, 256, (0, 1, 127, 255)), (8, 64, (0, 1, 31, 63))])
def test_long_chain_full_width(torch_cuda, B, steps, sampled):
    """Chained greedy decode steps of the 27B-shaped dense model at its full
    width, vocabulary and context 4096 (2 layers, so that the fp64 oracle can
    run every step): 256 steps at batch 1, 64 at batch 8, each step one
    launch in bench.py's launch configuration.  The GPU and the oracle each
    advance their own caches (the oracle never sees a value the GPU
    produced); every step's greedy tokens must agree (the next step's input),
    and at the sampled steps the logits and that step's new cache rows are
    compared."""
    from tests.harness import HostWeights, host_kv
    from oracle import step as ostep
    torch = torch_cuda
    w = WL.get("dense_27b").replace(n_layers=2)
    m = _model(w)
    W = HostWeights(w)
    kv_ref = host_kv(w)
    toks = [int(t) for t in synth.tokens(w, B)]
    pos0 = [w.context - 13 * b for b in range(B)]
    for s in range(steps):
        pos = [p + s for p in pos0]
        if s in sampled:
            print(f"case long chain B={B} step {s} pos={pos} toks={toks}", flush=True)
        g = GU.run_gpu_step(m, toks, pos)
        o = ostep.decode_step(w, W, np.asarray(toks), np.asarray(pos), kv_ref)
        assert np.array_equal(g["next"], o["next"]), f"step {s}: greedy tokens {g['next']} != oracle {o['next']}"
        if s in sampled:
            GU.compare_step(w, g, o, f"long chain B={B} step {s}")
            GU.compare_kv_rows(w, GU.kv_rows_dev(m, pos, B), kv_ref, pos, B)
        toks = [int(t) for t in o["next"]]


@pytest.mark.parametrize("name,B", [("mini_moe", 3), ("mini_hybrid", 2)])
def test_multilaunch_graph_replays_match_eager(torch_cuda, name, B):
    """The multi-launch baseline captured in a HIP graph (two steps per
    graph, one per counter bank): three replays, each with eager steps
    between them, and the timed replays after them must all give the eager
    multi-launch step's logits bitwise."""
    import bench
    w = WL.get(name)
    m = _model(w)
    print(f"case graph {name} B={B}", flush=True)
    ms, ok = bench.time_multilaunch_graph(m, B, reps=4)
    assert ok, f"{name}: a graph replay differs from the eager multi-launch step"
    m.close()
