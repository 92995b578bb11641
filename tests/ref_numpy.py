"""A second, separately written fp64 reference in vectorised NumPy, used only
to cross-check the oracle (it is not the oracle).  It covers the dense GQA
decoder and the textbook pieces the pin tests need: rotate-half RoPE,
softmax attention with grouped KV heads, SwiGLU and RMSNorm, written as
whole-array expressions rather than the oracle's element loops."""
from __future__ import annotations

import numpy as np


def widen(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_round_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) and return them as
    fp64; via np.round on the significand scaled to 8 bits."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.round(m * 256.0)  # numpy rounds halves to even
    return np.ldexp(r, e - 8)


def rms_norm(x, g_bits, eps):
    x = np.asarray(x, dtype=np.float64)
    return widen(g_bits) * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_half(v, pos, theta):
    """v[..., d]; rotate-half pairs (i, i + d/2) by pos * theta^(-2i/d)."""
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    ang = pos * theta ** (-2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., : d // 2], v[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def attention(q, K, V, scale):
    """q[nq, d], K/V[nkv, T, d]; q head h reads kv head h // (nq/nkv)."""
    nq, nkv = q.shape[0], K.shape[0]
    Kr = np.repeat(K, nq // nkv, axis=0)
    Vr = np.repeat(V, nq // nkv, axis=0)
    s = np.einsum("hd,htd->ht", q, Kr) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return np.einsum("ht,htd->hd", p, Vr)


def silu(z):
    return z / (1.0 + np.exp(-z))


def dense_step(w, W, tokens, positions, kv):
    """Dense GQA decoder step.  W: name -> bf16 bits; kv[l]: uint16[2, Bm, nkv, cap, hd]
    (updated in place).  Returns fp64 logits[B, V] and the final residual."""
    H, nq, nkv, hd = w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim
    X = widen(W["embed"])[np.asarray(tokens)]
    for l in range(w.n_layers):
        p = f"L{l}."
        for b in range(X.shape[0]):
            pos = int(positions[b])
            xn = rms_norm(X[b], W[p + "attn_norm"].reshape(-1), w.rms_eps)
            q = (widen(W[p + "wq"]) @ xn).reshape(nq, hd)
            k = (widen(W[p + "wk"]) @ xn).reshape(nkv, hd)
            v = (widen(W[p + "wv"]) @ xn).reshape(nkv, hd)
            q = rope_half(q, pos, w.rope_theta)
            k = rope_half(k, pos, w.rope_theta)
            kr = bf16_round_f64(k)
            vr = bf16_round_f64(v)
            kv[l][0, b, :, pos, :] = _f64_bf16_bits(kr)
            kv[l][1, b, :, pos, :] = _f64_bf16_bits(vr)
            K = widen(kv[l][0, b, :, : pos + 1, :])
            V = widen(kv[l][1, b, :, : pos + 1, :])
            o = attention(q, K, V, 1.0 / np.sqrt(hd)).reshape(-1)
            X[b] = X[b] + widen(W[p + "wo"]) @ o
        for b in range(X.shape[0]):
            xn = rms_norm(X[b], W[p + "ffn_norm"].reshape(-1), w.rms_eps)
            h = silu(widen(W[p + "w_gate"]) @ xn) * (widen(W[p + "w_up"]) @ xn)
            X[b] = X[b] + widen(W[p + "w_down"]) @ h
    xn = rms_norm(X, W["final_norm"].reshape(-1), w.rms_eps)
    return xn @ widen(W["lm_head"]).T, X


def _f64_bf16_bits(x):
    """bits of fp64 values that are already exactly bf16-representable."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)
