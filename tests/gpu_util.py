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


def lm_margin(ref_row: np.ndarray) -> float:
    """Oracle's top-1 minus top-2 logit, relative to the row's RMS."""
    r = ref_row.astype(np.float64)
    top2 = np.sort(r)[-2:]
    return float(top2[1] - top2[0]) / float(np.sqrt(np.mean(r ** 2)))


def router_margins(router_logits: np.ndarray, k: int) -> np.ndarray:
    """Per (layer, token): the oracle's k-th largest router logit minus the
    (k+1)-th (the gap that decides the selection), relative to the logits'
    spread; +inf when every expert is chosen."""
    lg = np.sort(router_logits.astype(np.float64), axis=-1)[..., ::-1]
    if lg.shape[-1] <= k:
        return np.full(lg.shape[:-1], np.inf)
    sd = np.std(lg, axis=-1)
    sd = np.where(sd > 0, sd, 1.0)
    return (lg[..., k - 1] - lg[..., k]) / sd


def log_margins(w, o, label=""):
    """Print the oracle's decision margins of a step: the smallest LM-head
    top-2 gap and, for MoE models, the smallest router k-th vs (k+1)-th gap,
    so that a mismatch can be told from a near-tie.  Returns them."""
    lm = min(lm_margin(o["logits"].reshape(-1, o["logits"].shape[-1])[i])
             for i in range(o["logits"].reshape(-1, o["logits"].shape[-1]).shape[0]))
    msg = f"  margins {label}: LM-head top-2 >= {lm:.3e} x rms"
    rm = None
    if "router_logits" in o:
        rm = float(np.min(router_margins(o["router_logits"], w.top_k)))
        msg += f"; router k-th vs (k+1)-th >= {rm:.3e} x sd"
    print(msg, flush=True)
    return lm, rm


def compare_step(w, g, o, label=""):
    """Assert GPU outputs g match oracle outputs o; returns the worst rel err.
    Prints the oracle's decision margins first (every case, pass or fail)."""
    B = o["logits"].shape[0]
    worst = 0.0
    log_margins(w, o, label)
    for b in range(B):
        ref = o["logits"][b].astype(np.float64)
        got = g["logits"][b].astype(np.float64)
        assert np.all(np.isfinite(got)), f"{label} b={b}: non-finite logits"
        rms = float(np.sqrt(np.mean(ref ** 2)))
        err = float(np.max(np.abs(got - ref))) / rms
        worst = max(worst, err)
        assert err <= LOGIT_TOL, f"{label} b={b}: max|dlogit|/rms = {err:.3e} > {LOGIT_TOL}"
        assert int(g["next"][b]) == int(o["next"][b]), \
            f"{label} b={b}: argmax {g['next'][b]} != oracle {o['next'][b]} (oracle top-2 margin {lm_margin(ref):.3e} x rms)"
    if "expert_ids" in o:
        same = g["expert_ids"] == o["expert_ids"]
        if not same.all():
            l, b = [int(i) for i in np.argwhere(~same.all(axis=-1))[0]]
            m = router_margins(o["router_logits"][l, b], w.top_k)
            raise AssertionError(f"{label}: expert selection differs at layer {l} token {b}: gpu "
                                 f"{g['expert_ids'][l, b].tolist()} oracle {o['expert_ids'][l, b].tolist()} "
                                 f"(oracle router margin {float(m):.3e} x sd)")
    return worst


def gpu_argmax_rows(logits: np.ndarray) -> np.ndarray:
    """Greedy token of every row of the GPU's logits (lowest index on ties)."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def compare_verify(w, logits, ids, acc, nxt, v, label=""):
    """Verify outputs of the GPU (logits [n][V], expert ids [L][n][k] or None,
    accepted length, next token) against the oracle's verify_step of one
    sequence: every row's argmax and, for MoE models, every row's experts
    bit-exact; logits within the tolerance; acceptance and next token equal."""
    o = {"logits": v["logits"][0], "next": v["argmax"][0]}
    g = {"logits": logits, "next": gpu_argmax_rows(logits)}
    if ids is not None:
        o["expert_ids"] = v["expert_ids"][0]          # [L][n][k]: row j plays the part of token j
        o["router_logits"] = v["router_logits"][0]
        g["expert_ids"] = ids
    err = compare_step(w, g, o, label)
    assert int(acc) == int(v["accept_len"][0]), f"{label}: accepted {acc} != oracle {v['accept_len'][0]}"
    assert int(nxt) == int(v["next"][0]), f"{label}: next token {nxt} != oracle {v['next'][0]}"
    return err


def kv_rows(w, kv, positions, B):
    """From full host caches (the oracle's layout), the entries a step wrote:
    per layer, GQA [2][B][n_kv][head_dim] at each sequence's position, MLA
    [B][row] likewise, delta-rule states [B][heads][dk][dv] whole."""
    out = []
    for l in range(w.n_layers):
        kind = w.layer_kind(l)
        if kind == "kda":
            out.append(np.ascontiguousarray(kv[l][:B]))
        elif kind == "mla":
            out.append(np.stack([kv[l][b, int(positions[b])] for b in range(B)]))
        else:
            out.append(np.stack([kv[l][:, b, :, int(positions[b]), :] for b in range(B)], axis=1))
    return out


def kv_rows_dev(m, positions, B):
    """The same entries read from the GPU's cache (only those rows are copied
    to the host; GQA V rows are taken from their 32-position tiles)."""
    from synth.workloads import V_TILE
    out = []
    for l in range(m.w.n_layers):
        kind = m.w.layer_kind(l)
        t = m.kv_layer(l)
        if kind == "kda":
            out.append(t[:B].cpu().numpy())
        elif kind == "mla":
            out.append(np.stack([t[b, int(positions[b])].cpu().numpy().view(np.uint16) for b in range(B)]))
        else:
            rows = []
            for b in range(B):
                p = int(positions[b])
                k = t[0, b, :, p, :]
                vt = t[1, b].reshape(t.shape[2], t.shape[3] // V_TILE, t.shape[4], V_TILE)  # [nkv][tile][hd][32]
                v = vt[:, p // V_TILE, :, p % V_TILE]
                rows.append(np.stack([k.cpu().numpy(), v.cpu().numpy()]).view(np.uint16))
            out.append(np.stack(rows, axis=1))
    return out


def compare_kv_rows(w, kv_gpu, kv_ref, positions, B):
    """New cache rows.  Layer 0's row depends only on the embedding and the
    layer's weights, so GPU (fp32) and oracle (fp64) values round to the same
    bf16 or to neighbours: at most 1 ulp apart (entries far below the row's
    RMS: within 2^-12 of it).  Deeper rows inherit the
    residual's fp32-vs-fp64 difference: 1 ulp plus 1e-3 of the row's RMS.
    kv_gpu: full host caches (DeviceModel.kv_host) or kv_rows_dev's rows."""
    from tests.ref_numpy import widen
    if len(kv_gpu) and kv_gpu[0].ndim == kv_ref[0].ndim and kv_gpu[0].shape == kv_ref[0].shape:
        kv_gpu = kv_rows(w, kv_gpu, positions, B)
    ref = kv_rows(w, kv_ref, positions, B)
    n_off = 0
    for l in range(w.n_layers):
        kind = w.layer_kind(l)
        if kind == "kda":
            # delta-rule state, rewritten in place: max |diff| <= 1e-3 of the state's RMS
            for b in range(B):
                a = kv_gpu[l][b].astype(np.float64)
                r = ref[l][b].astype(np.float64)
                rms = float(np.sqrt(np.mean(r ** 2)))
                err = float(np.max(np.abs(a - r)))
                assert err <= 1e-3 * rms, f"layer {l} b={b}: delta-rule state max|diff| {err:.3e} > 1e-3 * rms {rms:.3e}"
            continue
        if kind == "mla":
            for b in range(B):
                a, r = kv_gpu[l][b], ref[l][b]
                af, rf = widen(a), widen(r)
                rms = np.sqrt(np.mean(rf ** 2))
                bad = np.abs(af - rf) > np.abs(rf) * 2.0 ** -7 + 1e-3 * rms
                assert not bad.any(), f"MLA layer {l} b={b}: {int(bad.sum())} cache entries beyond tolerance"
                n_off += int((a != r).sum())
            continue
        for b in range(B):
            a = kv_gpu[l][:, b]
            r = ref[l][:, b]
            d_ulp = np.abs(a.astype(np.int32) - r.astype(np.int32))
            if l == 0:
                # within 1 ulp, or (an entry much smaller than its row, from a
                # cancelling dot product over inputs split into two bf16
                # halves, about 16 significant bits) within 2^-12 of the row's RMS
                af, rf = widen(a), widen(r)
                rms = np.sqrt(np.mean(rf ** 2, axis=-1, keepdims=True))
                bad = (d_ulp > 1) & (np.abs(af - rf) > 2.0 ** -12 * rms)
                assert not bad.any(), f"layer 0 b={b}: {int(bad.sum())} cache entries beyond 1 ulp (max {d_ulp.max()})"
            else:
                af, rf = widen(a), widen(r)
                rms = np.sqrt(np.mean(rf ** 2, axis=-1, keepdims=True))
                ulp = np.abs(rf) * 2.0 ** -7
                bad = np.abs(af - rf) > ulp + 1e-3 * rms
                assert not bad.any(), f"layer {l} b={b}: {int(bad.sum())} cache entries beyond tolerance"
            n_off += int((d_ulp > 0).sum())
    return n_off
