"""ORACLE -- test infrastructure only.

Composition of one decode step from the fp64 blocks in oracle.c, in the order
of the pages' layer schedule (Inferact, "700 TPS on Kimi K3: A Case for TPU
Megakernels", section "Our Kimi K3 megakernel": attention chosen by layer
index, then router, shared expert and routed experts), with pre-norm residual
blocks, a final RMSNorm, the LM head and greedy decoding (section "Results").

Weights reach the oracle through `get_weight(name) -> uint16[rows, cols]`
(bf16 bits, logical row-major [out, in]); the caller may draw them lazily so
that full-size models never need to sit in host memory at once.  The cache /
state of each layer is a host array in the layout `synth.kv_layout` documents
and is updated in place.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional

import numpy as np

from . import lib, ptr

GetW = Callable[[str], np.ndarray]


def _w(get_weight: GetW, name: str) -> np.ndarray:
    a = get_weight(name)
    return np.ascontiguousarray(a, dtype=np.uint16)


def _layer(w, get_weight: GetW, l: int, xs: np.ndarray, positions, kv_l, B: int,
           ids_out: Optional[np.ndarray], wts_out: Optional[np.ndarray],
           rlog_out: Optional[np.ndarray] = None) -> None:
    """Apply layer l to the residuals xs[B, H] (fp64, in place)."""
    L = lib()
    H = w.hidden
    p = f"L{l}."
    kind = w.layer_kind(l)
    g_attn = _w(get_weight, p + "attn_norm")
    # ---- attention block (pre-norm inside each block function)
    if kind == "gqa":
        wq, wk, wv, wo = (_w(get_weight, p + n) for n in ("wq", "wk", "wv", "wo"))
        for b in range(B):
            kc = kv_l[0, b]
            vc = kv_l[1, b]
            assert kc.flags["C_CONTIGUOUS"] and vc.flags["C_CONTIGUOUS"]
            x = xs[b]
            rc = L.orc_gqa_block(H, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rms_eps, w.rope_theta,
                                 ptr(g_attn), ptr(wq), ptr(wk), ptr(wv), ptr(wo),
                                 ptr(x), int(positions[b]), ptr(kc), ptr(vc), w.max_ctx)
            assert rc == 0
        del wq, wk, wv, wo
    elif kind == "mla":
        names = ("mla_wqa", "mla_q_norm", "mla_wqb", "mla_wkva", "mla_kv_norm", "mla_wkvb", "mla_wo")
        wqa, gq, wqb, wkva, gkv, wkvb, wo = (_w(get_weight, p + n) for n in names)
        for b in range(B):
            cache = kv_l[b]
            rc = L.orc_mla_block(H, w.mla_heads, w.q_lora, w.kv_lora, w.rope_dim, w.nope_dim, w.v_dim,
                                 w.rms_eps, w.rope_theta, ptr(g_attn), ptr(wqa), ptr(gq), ptr(wqb),
                                 ptr(wkva), ptr(gkv), ptr(wkvb), ptr(wo),
                                 ptr(xs[b]), int(positions[b]), ptr(cache), w.max_ctx)
            assert rc == 0
    else:
        names = ("kda_wq", "kda_wk", "kda_wv", "kda_walpha", "kda_wbeta", "kda_wo")
        wq, wk, wv, wa, wb, wo = (_w(get_weight, p + n) for n in names)
        for b in range(B):
            st = kv_l[b]
            rc = L.orc_kda_block(H, w.kda_heads, w.kda_dk, w.kda_dv, w.kda_qk_l2norm, w.rms_eps,
                                 ptr(g_attn), ptr(wq), ptr(wk), ptr(wv), ptr(wa), ptr(wb), ptr(wo),
                                 ptr(xs[b]), ptr(st))
            assert rc == 0
    # ---- FFN / MoE block
    g_ffn = _w(get_weight, p + "ffn_norm")
    xn = np.empty(H, dtype=np.float64)
    acc = np.empty(H, dtype=np.float64)
    if not w.is_moe:
        wg, wu, wd = (_w(get_weight, p + n) for n in ("w_gate", "w_up", "w_down"))
        for b in range(B):
            L.orc_rmsnorm(H, ptr(xs[b]), ptr(g_ffn), w.rms_eps, ptr(xn))
            acc[:] = 0.0
            L.orc_swiglu_add(H, w.ffn_dim, ptr(wg), ptr(wu), ptr(wd), ptr(xn), 1.0, ptr(acc))
            xs[b] += acc
        return
    wr = _w(get_weight, p + "router")
    k = w.top_k
    xns = np.empty((B, H), dtype=np.float64)
    ids = np.empty((B, k), dtype=np.int32)
    wts = np.empty((B, k), dtype=np.float64)
    rlog = np.empty((B, w.n_experts), dtype=np.float32)
    for b in range(B):
        L.orc_rmsnorm(H, ptr(xs[b]), ptr(g_ffn), w.rms_eps, ptr(xns[b]))
        L.orc_router(H, w.n_experts, k, w.norm_topk, ptr(wr), ptr(xns[b]), ptr(ids[b]), ptr(wts[b]), ptr(rlog[b]))
    if rlog_out is not None:
        rlog_out[:] = rlog
    if ids_out is not None:
        ids_out[:] = ids
    if wts_out is not None:
        wts_out[:] = wts
    accs = np.zeros((B, H), dtype=np.float64)
    # shared expert(s): weight 1
    for s in range(w.n_shared):
        wg, wu, wd = (_w(get_weight, p + f"sh{s}_{n}") for n in ("gate", "up", "down"))
        for b in range(B):
            L.orc_swiglu_add(H, w.shared_ffn, ptr(wg), ptr(wu), ptr(wd), ptr(xns[b]), 1.0, ptr(accs[b]))
    # routed experts: each selected expert, in ascending id order, for the
    # tokens that selected it (only those experts' weights are fetched)
    for e in sorted(set(int(i) for i in ids.reshape(-1))):
        wg, wu, wd = (_w(get_weight, p + f"e{e}_{n}") for n in ("gate", "up", "down"))
        for b in range(B):
            sel = np.nonzero(ids[b] == e)[0]
            if sel.size:
                j = int(sel[0])
                L.orc_swiglu_add(H, w.expert_ffn, ptr(wg), ptr(wu), ptr(wd), ptr(xns[b]),
                                 float(wts[b, j]), ptr(accs[b]))
    xs += accs


def decode_step(w, get_weight: GetW, tokens, positions, kv: List[np.ndarray],
                layer_dump: Optional[List[np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """One decode step for a batch.  kv[l] is updated in place.

    Returns logits fp32[B, V], next int32[B] (greedy argmax, lowest index on
    ties), expert_ids int32[n_layers, B, top_k], expert_w fp64[...] and the
    fp32 router logits router_logits[n_layers, B, n_experts] on which the
    choice was made (MoE only), and the final residual fp64[B, H]."""
    L = lib()
    tokens = np.asarray(tokens, dtype=np.int32)
    positions = np.asarray(positions, dtype=np.int64)
    B = tokens.shape[0]
    H, V = w.hidden, w.vocab
    emb = _w(get_weight, "embed")
    xs = np.empty((B, H), dtype=np.float64)
    for b in range(B):
        L.orc_embed(H, ptr(emb), int(tokens[b]), ptr(xs[b]))
    del emb
    k = max(w.top_k, 1)
    ids = np.full((w.n_layers, B, k), -1, dtype=np.int32)
    wts = np.zeros((w.n_layers, B, k), dtype=np.float64)
    rlog = np.zeros((w.n_layers, B, max(w.n_experts, 1)), dtype=np.float32)
    for l in range(w.n_layers):
        _layer(w, get_weight, l, xs, positions, kv[l], B,
               ids[l] if w.is_moe else None, wts[l] if w.is_moe else None, rlog[l] if w.is_moe else None)
        if layer_dump is not None:
            layer_dump.append(xs.copy())
    g_final = _w(get_weight, "final_norm")
    wlm = _w(get_weight, "lm_head")
    logits = np.empty((B, V), dtype=np.float32)
    nxt = np.empty(B, dtype=np.int32)
    for b in range(B):
        nxt[b] = L.orc_head(H, V, w.rms_eps, ptr(g_final), ptr(wlm), ptr(xs[b]), ptr(logits[b]))
    out = {"logits": logits, "next": nxt, "x_final": xs}
    if w.is_moe:
        out["expert_ids"] = ids
        out["expert_w"] = wts
        out["router_logits"] = rlog
    return out


def acceptance(tokens_row: np.ndarray, argmax_rows: np.ndarray) -> int:
    """Accepted length a = 1 + m, m the largest j with t_i == argmax(row i-1)
    for every 1 <= i <= j (the anchor always counts, plus the bonus token)."""
    n = tokens_row.shape[0]
    m = 0
    for j in range(1, n):
        if int(tokens_row[j]) == int(argmax_rows[j - 1]):
            m = j
        else:
            break
    return 1 + m


def verify_step(w, get_weight: GetW, tokens, positions, kv: List[np.ndarray]) -> Dict[str, np.ndarray]:
    """Speculative verify of n = tokens.shape[1] tokens per sequence (anchor
    + drafts) at positions p..p+n-1, defined as n sequential decode steps.

    Row j of the logits is the decode-step output after t_0..t_j.  The
    delta-rule states are committed as they stand after token m (accepted
    length a = m + 1); cache rows p..p+n-1 are all written.  kv is updated
    in place accordingly.  MoE models also return, per sequence, the experts
    every row chose, expert_ids int32[B, n_layers, n, top_k], and the router
    logits behind them, router_logits fp32[B, n_layers, n, n_experts]."""
    tokens = np.asarray(tokens, dtype=np.int32)
    positions = np.asarray(positions, dtype=np.int64)
    B, n = tokens.shape
    V = w.vocab
    logits = np.empty((B, n, V), dtype=np.float32)
    arg = np.empty((B, n), dtype=np.int32)
    kda_layers = [l for l in range(w.n_layers) if w.layer_kind(l) == "kda"]
    snaps = []  # per token j: copies of the KDA states after token j
    k = max(w.top_k, 1)
    ids = np.full((B, w.n_layers, n, k), -1, dtype=np.int32)
    rlog = np.zeros((B, w.n_layers, n, max(w.n_experts, 1)), dtype=np.float32)
    for j in range(n):
        o = decode_step(w, get_weight, tokens[:, j], positions + j, kv)
        logits[:, j] = o["logits"]
        arg[:, j] = o["next"]
        if w.is_moe:
            ids[:, :, j] = np.swapaxes(o["expert_ids"], 0, 1)
            rlog[:, :, j] = np.swapaxes(o["router_logits"], 0, 1)
        snaps.append({l: kv[l].copy() for l in kda_layers})
    acc = np.array([acceptance(tokens[b], arg[b]) for b in range(B)], dtype=np.int32)
    for b in range(B):
        m = int(acc[b]) - 1
        for l in kda_layers:
            kv[l][b] = snaps[m][l][b]
    nxt = np.array([arg[b, int(acc[b]) - 1] for b in range(B)], dtype=np.int32)
    out = {"logits": logits, "argmax": arg, "accept_len": acc, "next": nxt}
    if w.is_moe:
        out["expert_ids"] = ids
        out["router_logits"] = rlog
    return out
