"""Helpers for GPU parity tests: run the HIP path and the oracle on the same
seeded inputs and compare."""
from __future__ import annotations

import numpy as np

import synth
from oracle import step as ostep
from tests.harness import HostWeights, host_kv

LOGIT_TOL = 2e-2   # max |logit diff| per row, relative to the oracle row's RMS


def run_gpu_step(m, toks, pos, multilaunch=False):
    import torch
    B = len(toks)
    dev = m.device
    t = torch.tensor(np.asarray(toks, dtype=np.int32), device=dev)
    p = torch.tensor(np.asarray(pos, dtype=np.int32), device=dev)
    logits = torch.full((B, m.w.vocab), float("nan"), dtype=torch.float32, device=dev)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=dev)
    ids = None
    if m.w.is_moe:
        ids = torch.full((m.w.n_layers, B, m.w.top_k), -7, dtype=torch.int32, device=dev)
    m.decode(t, p, logits, nxt, ids, multilaunch=multilaunch)
    torch.cuda.synchronize(dev)
    m.device_status()
    out = {"logits": logits.cpu().numpy(), "next": nxt.cpu().numpy()}
    if ids is not None:
        out["expert_ids"] = ids.cpu().numpy()
    return out


def run_oracle_step(w, toks, pos, overrides=None, kv=None):
    W = HostWeights(w, cache=False)
    if overrides:
        W.overrides.update(overrides)
    kv = host_kv(w) if kv is None else kv
    o = ostep.decode_step(w, W, np.asarray(toks), np.asarray(pos), kv)
    return o, kv


def compare_step(w, g, o, label=""):
    """Assert GPU outputs g match oracle outputs o; returns the worst rel err."""
    B = o["logits"].shape[0]
    worst = 0.0
    for b in range(B):
        ref = o["logits"][b].astype(np.float64)
        got = g["logits"][b].astype(np.float64)
        assert np.all(np.isfinite(got)), f"{label} b={b}: non-finite logits"
        rms = float(np.sqrt(np.mean(ref ** 2)))
        err = float(np.max(np.abs(got - ref))) / rms
        worst = max(worst, err)
        top2 = np.sort(ref)[-2:]
        assert err <= LOGIT_TOL, f"{label} b={b}: max|dlogit|/rms = {err:.3e} > {LOGIT_TOL}"
        assert int(g["next"][b]) == int(o["next"][b]), \
            f"{label} b={b}: argmax {g['next'][b]} != oracle {o['next'][b]} (oracle top-2 margin {top2[1]-top2[0]:.3e})"
    if "expert_ids" in o:
        assert np.array_equal(g["expert_ids"], o["expert_ids"]), f"{label}: expert selection differs"
    return worst


def compare_kv_rows(w, kv_gpu, kv_ref, positions, B):
    """New cache rows.  Layer 0's row depends only on the embedding and the
    layer's weights, so GPU (fp32) and oracle (fp64) values round to the same
    bf16 or to neighbours: at most 1 ulp apart.  Deeper rows inherit the
    residual's fp32-vs-fp64 difference: 1 ulp plus 1e-3 of the row's RMS."""
    from tests.ref_numpy import widen
    n_off = 0
    for l in range(w.n_layers):
        kind = w.layer_kind(l)
        if kind == "kda":
            # delta-rule state, rewritten in place: max |diff| <= 1e-3 of the state's RMS
            for b in range(B):
                a = kv_gpu[l][b].astype(np.float64)
                r = kv_ref[l][b].astype(np.float64)
                rms = float(np.sqrt(np.mean(r ** 2)))
                err = float(np.max(np.abs(a - r)))
                assert err <= 1e-3 * rms, f"layer {l} b={b}: delta-rule state max|diff| {err:.3e} > 1e-3 * rms {rms:.3e}"
            continue
        if kind == "mla":
            for b in range(B):
                p = int(positions[b])
                a, r = kv_gpu[l][b, p], kv_ref[l][b, p]
                af, rf = widen(a), widen(r)
                rms = np.sqrt(np.mean(rf ** 2))
                bad = np.abs(af - rf) > np.abs(rf) * 2.0 ** -7 + 1e-3 * rms
                assert not bad.any(), f"MLA layer {l} b={b}: {int(bad.sum())} cache entries beyond tolerance"
                n_off += int((a != r).sum())
            continue
        for b in range(B):
            p = int(positions[b])
            a = kv_gpu[l][:, b, :, p, :]
            r = kv_ref[l][:, b, :, p, :]
            d_ulp = np.abs(a.astype(np.int32) - r.astype(np.int32))
            if l == 0:
                assert d_ulp.max() <= 1, f"layer 0 b={b}: cache row differs by {d_ulp.max()} ulp"
            else:
                af, rf = widen(a), widen(r)
                rms = np.sqrt(np.mean(rf ** 2, axis=-1, keepdims=True))
                ulp = np.abs(rf) * 2.0 ** -7
                bad = np.abs(af - rf) > ulp + 1e-3 * rms
                assert not bad.any(), f"layer {l} b={b}: {int(bad.sum())} cache entries beyond tolerance"
            n_off += int((d_ulp > 0).sum())
    return n_off
