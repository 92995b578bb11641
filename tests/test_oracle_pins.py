"""Pins of the oracle against facts that do not come from the oracle itself:
closed forms, invariants, special cases with hand-derived values, brute
force on tiny inputs, and a separately written NumPy reference.  Each test
names the mistake it is there to catch."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synth
from oracle import step as ostep
from synth import workloads as WL
from tests import ref_numpy as R
from tests.harness import HostWeights, host_kv, kv_copy, zeros_like_weights

BF1 = 0x3F80


def bits(x):
    """bf16 bits of values that are exactly bf16 (fp32 truncation is exact)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rand_bits(rng, shape, sigma):
    return synth.f32_to_bf16_bits(rng.normal(0, sigma, size=shape).astype(np.float32))


# ------------------------------------------------------------------ bf16
def test_to_bf16_ties_and_double_rounding():
    # exact values stay exact
    assert oracle.to_bf16(1.0) == 0x3F80
    assert oracle.to_bf16(-2.0) == 0xC000
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    assert oracle.to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert oracle.to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above the tie must round up; going through fp32 first would land on
    # the tie and round down (double rounding) -- the oracle must not.
    assert oracle.to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert oracle.to_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == 0xBF81


def test_to_bf16_matches_integer_rne_on_fp32_values():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 3, size=4000).astype(np.float32)
    want = synth.f32_to_bf16_bits(x)
    got = np.array([oracle.to_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.normal(size=333)
    g = np.full(333, BF1, dtype=np.uint16)
    eps = 1e-6
    y = oracle.rmsnorm(x, g, eps)
    m = np.mean(x * x)
    # with unit gains the output RMS is sqrt(m / (m + eps))
    assert abs(np.sqrt(np.mean(y * y)) - math.sqrt(m / (m + eps))) < 1e-14
    # a constant vector c maps to g * c / sqrt(c^2 + eps)
    c = np.full(64, -0.37)
    g2 = bits(np.full(64, 2.0))
    y2 = oracle.rmsnorm(c, g2, eps)
    assert np.allclose(y2, 2.0 * -0.37 / math.sqrt(0.37 ** 2 + eps), rtol=0, atol=1e-15)
    # gains scale elementwise (a dropped gain fails this)
    g3 = bits(np.where(np.arange(333) % 2 == 0, 1.0, 0.5))
    y3 = oracle.rmsnorm(x, g3, eps)
    assert np.allclose(y3[1::2], 0.5 * y[1::2], rtol=0, atol=1e-15)


# ------------------------------------------------------------------ matvec
def test_matvec_against_blas_and_selector():
    rng = np.random.default_rng(2)
    W = rand_bits(rng, (37, 129), 0.5)
    x = rng.normal(size=129)
    assert np.allclose(oracle.matvec(W, x), R.widen(W) @ x, rtol=1e-13, atol=1e-13)
    # a one-hot row picks one element: catches a transposed operand
    S = np.zeros((3, 129), dtype=np.uint16)
    S[0, 5] = BF1
    S[1, 128] = BF1
    S[2, 0] = bits(-2.0)
    assert np.array_equal(oracle.matvec(S, x), np.array([x[5], x[128], -2 * x[0]]))


# ------------------------------------------------------------------ RoPE
def test_rope_identity_at_zero_and_unit_vector_closed_form():
    d, theta = 16, 1e4
    v = np.arange(1, d + 1, dtype=np.float64)
    assert np.array_equal(oracle.rope(v, 0, theta), v)
    # unit vector at index i < d/2 turns into the (i, i + d/2) plane
    for i in (0, 3, 7):
        e = np.zeros(d)
        e[i] = 1.0
        pos = 11
        ang = pos * theta ** (-2.0 * i / d)
        want = np.zeros(d)
        want[i] = math.cos(ang)
        want[i + d // 2] = math.sin(ang)
        assert np.allclose(oracle.rope(e, pos, theta), want, atol=1e-15)


def test_rope_invariants():
    rng = np.random.default_rng(3)
    d, theta = 64, 1e4
    q, k = rng.normal(size=d), rng.normal(size=d)
    for pos in (1, 17, 4096, 8199):
        r = oracle.rope(q, pos, theta)
        # pairwise norms preserved
        h = d // 2
        assert np.allclose(r[:h] ** 2 + r[h:] ** 2, q[:h] ** 2 + q[h:] ** 2, rtol=1e-12)
    # q(m) . k(n) depends only on m - n
    a = oracle.rope(q, 100, theta) @ oracle.rope(k, 93, theta)
    b = oracle.rope(q, 7, theta) @ oracle.rope(k, 0, theta)
    assert abs(a - b) < 1e-10


def test_rope_matches_vectorised_reference():
    rng = np.random.default_rng(4)
    v = rng.normal(size=128)
    assert np.allclose(oracle.rope(v, 4097, 1e4), R.rope_half(v, 4097, 1e4), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ softmax
def test_softmax_values():
    p = oracle.softmax([0.0, math.log(3.0)])
    assert np.allclose(p, [0.25, 0.75], rtol=1e-15)
    rng = np.random.default_rng(5)
    s = rng.normal(size=1000) * 30
    p = oracle.softmax(s)
    assert abs(p.sum() - 1.0) < 1e-12
    assert np.allclose(oracle.softmax(s + 123.0), p, rtol=1e-12)


# ------------------------------------------------------------------ router
def test_router_topk_brute_force_and_weights():
    rng = np.random.default_rng(6)
    for trial in range(20):
        E, k, H = int(rng.integers(4, 70)), None, 48
        k = int(rng.integers(1, min(E, 9)))
        wr = rand_bits(rng, (E, H), 0.3)
        xn = rng.normal(size=H)
        ids, w, lg = oracle.router(wr, xn, k, 1)
        r32 = (R.widen(wr) @ xn).astype(np.float32)
        order = sorted(range(E), key=lambda e: (-float(r32[e]), e))[:k]
        assert list(ids) == order
        assert np.array_equal(lg, r32)
        # renormalised weights = softmax over the selected logits
        sel = r32[order].astype(np.float64)
        ws = np.exp(sel - sel.max())
        assert np.allclose(w, ws / ws.sum(), rtol=1e-12)
        assert abs(w.sum() - 1.0) < 1e-12
        ids0, w0, _ = oracle.router(wr, xn, k, 0)
        full = np.exp(r32.astype(np.float64) - r32.max())
        full /= full.sum()
        assert np.allclose(w0, full[order], rtol=1e-12)


def test_router_ties_pick_lowest_ids():
    wr = np.zeros((16, 32), dtype=np.uint16)
    ids, w, _ = oracle.router(wr, np.ones(32), 8, 1)
    assert list(ids) == list(range(8))
    assert np.allclose(w, 1.0 / 8)


# ------------------------------------------------------------------ SwiGLU
def test_swiglu_closed_form():
    acc = np.zeros(1)
    oracle.swiglu_add(bits([[1.0]]), bits([[2.0]]), bits([[0.5]]), np.array([1.0]), 1.0, acc)
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(acc[0] - 0.5 * silu1 * 2.0) < 1e-15
    # zero gate weights give silu(0) = 0
    rng = np.random.default_rng(7)
    acc = np.zeros(8)
    oracle.swiglu_add(np.zeros((5, 8), np.uint16), rand_bits(rng, (5, 8), 1), rand_bits(rng, (8, 5), 1),
                      rng.normal(size=8), 1.0, acc)
    assert np.all(acc == 0.0)
    # scale multiplies, and gate/up are not swapped: silu(a) * b != silu(b) * a
    acc = np.zeros(1)
    oracle.swiglu_add(bits([[1.0]]), bits([[3.0]]), bits([[1.0]]), np.array([1.0]), 0.25, acc)
    assert abs(acc[0] - 0.25 * silu1 * 3.0) < 1e-15


# ------------------------------------------------------------------ GQA block
def _gqa_setup(nq, nkv, hd, pos, cap, rng, H=None):
    H = H or nq * hd
    g = np.full(H, BF1, np.uint16)
    wq = rand_bits(rng, (nq * hd, H), 0.2)
    wk = rand_bits(rng, (nkv * hd, H), 0.2)
    wv = rand_bits(rng, (nkv * hd, H), 0.2)
    wo = np.zeros((H, nq * hd), np.uint16)
    np.fill_diagonal(wo, BF1)  # x += o: lets the test read o directly
    kc = rand_bits(rng, (nkv, cap, hd), 1.0)
    vc = rand_bits(rng, (nkv, cap, hd), 1.0)
    x = rng.normal(size=H)
    return H, g, wq, wk, wv, wo, kc, vc, x


def _run_gqa(H, nq, nkv, hd, g, wq, wk, wv, wo, x, pos, kc, vc, cap, theta=1e4):
    x2 = x.copy()
    rc = oracle.lib().orc_gqa_block(H, nq, nkv, hd, 1e-6, theta, oracle.ptr(g), oracle.ptr(wq), oracle.ptr(wk),
                                    oracle.ptr(wv), oracle.ptr(wo), oracle.ptr(x2), pos, oracle.ptr(kc),
                                    oracle.ptr(vc), cap)
    assert rc == 0
    return x2


def test_gqa_single_token_returns_its_value_row():
    rng = np.random.default_rng(8)
    nq = nkv = 2
    hd, cap = 32, 8
    H, g, wq, wk, wv, wo, kc, vc, x = _gqa_setup(nq, nkv, hd, 0, cap, rng)
    x2 = _run_gqa(H, nq, nkv, hd, g, wq, wk, wv, wo, x, 0, kc, vc, cap)
    # softmax over one row is 1: o_h is exactly the stored bf16 value row
    want = np.concatenate([R.widen(vc[0, 0]), R.widen(vc[1, 0])])
    assert np.array_equal(x2, x + want)
    # and the stored row is v = W_v xn rounded to bf16
    xn = R.rms_norm(x, g, 1e-6)
    v = R.widen(wv) @ xn
    assert np.array_equal(R.widen(vc[:, 0].reshape(-1)), R.bf16_round_f64(v))


def test_gqa_equal_scores_average_values():
    rng = np.random.default_rng(9)
    nq, nkv, hd, cap, pos = 2, 1, 16, 12, 9
    H, g, wq, wk, wv, wo, kc, vc, x = _gqa_setup(nq, nkv, hd, pos, cap, rng)
    wk[:] = 0
    kc[:] = 0  # every key zero: uniform softmax over rows 0..pos
    x2 = _run_gqa(H, nq, nkv, hd, g, wq, wk, wv, wo, x, pos, kc, vc, cap)
    mean_v = R.widen(vc[0, : pos + 1]).mean(axis=0)
    assert np.allclose((x2 - x)[:hd], mean_v, atol=1e-12)
    assert np.allclose((x2 - x)[hd:], mean_v, atol=1e-12)


@pytest.mark.parametrize("nq,nkv", [(4, 4), (6, 2), (8, 1)])
def test_gqa_matches_textbook_attention(nq, nkv):
    rng = np.random.default_rng(10 + nq)
    hd, cap, pos = 32, 40, 33
    H = 96
    _, g, wq, wk, wv, _, kc, vc, x = _gqa_setup(nq, nkv, hd, pos, cap, rng, H=H)
    g = synth.f32_to_bf16_bits(1.0 + rng.normal(0, 0.2, size=H).astype(np.float32))
    wo = rand_bits(rng, (H, nq * hd), 0.2)
    kc0, vc0 = kc.copy(), vc.copy()
    x2 = _run_gqa(H, nq, nkv, hd, g, wq, wk, wv, wo, x, pos, kc, vc, cap)
    # textbook: pre-norm, rotate-half RoPE, bf16 cache rows, softmax(qK^T/sqrt(d))V, W_o
    xn = R.rms_norm(x, g, 1e-6)
    q = R.rope_half((R.widen(wq) @ xn).reshape(nq, hd), pos, 1e4)
    k = R.bf16_round_f64(R.rope_half((R.widen(wk) @ xn).reshape(nkv, hd), pos, 1e4))
    v = R.bf16_round_f64((R.widen(wv) @ xn).reshape(nkv, hd))
    K = R.widen(kc0[:, : pos + 1]).copy()
    V = R.widen(vc0[:, : pos + 1]).copy()
    K[:, pos] = k
    V[:, pos] = v
    o = R.attention(q, K, V, 1.0 / math.sqrt(hd)).reshape(-1)
    want = x + R.widen(wo) @ o
    assert np.allclose(x2, want, rtol=1e-11, atol=1e-11)
    # untouched rows of the cache stay untouched
    assert np.array_equal(kc[:, :pos], kc0[:, :pos]) and np.array_equal(kc[:, pos + 1:], kc0[:, pos + 1:])


# ------------------------------------------------------------------ KDA block
def _kda(H, nh, dk, dv, g, wq, wk, wv, wa, wb, wo, x, S):
    x2 = x.copy()
    rc = oracle.lib().orc_kda_block(H, nh, dk, dv, 1, 1e-6, *(oracle.ptr(a) for a in (g, wq, wk, wv, wa, wb, wo)),
                                    oracle.ptr(x2), oracle.ptr(S))
    assert rc == 0
    return x2


def _kda_setup(rng, nh=2, dk=8, dv=8):
    H = nh * dv
    g = np.full(H, BF1, np.uint16)
    wq = rand_bits(rng, (nh * dk, H), 0.3)
    wk = rand_bits(rng, (nh * dk, H), 0.3)
    wv = rand_bits(rng, (nh * dv, H), 0.3)
    wa = rand_bits(rng, (nh, H), 0.3)
    wb = rand_bits(rng, (nh, H), 0.3)
    wo = np.zeros((H, nh * dv), np.uint16)
    np.fill_diagonal(wo, BF1)
    x = rng.normal(size=H)
    return H, g, wq, wk, wv, wa, wb, wo, x


def test_kda_from_zero_state_closed_form():
    rng = np.random.default_rng(20)
    nh, dk, dv = 2, 8, 8
    H, g, wq, wk, wv, wa, wb, wo, x = _kda_setup(rng, nh, dk, dv)
    S = np.zeros((nh, dk, dv), np.float32)
    x2 = _kda(H, nh, dk, dv, g, wq, wk, wv, wa, wb, wo, x, S)
    xn = R.rms_norm(x, g, 1e-6)
    q = (R.widen(wq) @ xn).reshape(nh, dk)
    k = (R.widen(wk) @ xn).reshape(nh, dk)
    v = (R.widen(wv) @ xn).reshape(nh, dv)
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    beta = 1.0 / (1.0 + np.exp(-(R.widen(wb) @ xn)))
    # S1 = beta k v^T and o = beta v (k . q)
    for h in range(nh):
        assert np.allclose(S[h], (beta[h] * np.outer(k[h], v[h])).astype(np.float32), rtol=1e-6, atol=1e-7)
        assert np.allclose((x2 - x)[h * dv:(h + 1) * dv], beta[h] * v[h] * (k[h] @ q[h]), rtol=1e-6, atol=1e-7)


def test_kda_unit_gates_store_value_along_key():
    rng = np.random.default_rng(21)
    nh, dk, dv = 1, 16, 8
    H, g, wq, wk, wv, wa, wb, wo, x = _kda_setup(rng, nh, dk, dv)
    # drive alpha and beta to 1 (sigmoid(z) = 1 - 1e-14 at z ~ 32)
    xn = R.rms_norm(x, g, 1e-6)
    j = int(np.argmax(np.abs(xn)))
    wa[:] = 0
    wb[:] = 0
    wa[0, j] = synth.f32_to_bf16_bits(np.float32(np.sign(xn[j]) * 64.0 / max(abs(xn[j]), 1e-3)).reshape(1))[0]
    wb[0, j] = wa[0, j]
    S = rng.normal(size=(nh, dk, dv)).astype(np.float32)
    _kda(H, nh, dk, dv, g, wq, wk, wv, wa, wb, wo, x, S)
    k = R.widen(wk) @ xn
    k /= np.linalg.norm(k)
    v = R.widen(wv) @ xn
    # with alpha = beta = 1 and |k| = 1 the new state maps k onto v
    assert np.allclose(S[0].T.astype(np.float64) @ k, v, atol=2e-5)


def test_kda_zero_weights_halve_state():
    rng = np.random.default_rng(22)
    nh, dk, dv = 2, 8, 8
    H, g, wq, wk, wv, wa, wb, wo, x = _kda_setup(rng, nh, dk, dv)
    for a in (wq, wk, wv, wa, wb, wo):
        a[:] = 0
    S = rng.normal(size=(nh, dk, dv)).astype(np.float32)
    S0 = S.copy()
    x2 = _kda(H, nh, dk, dv, g, wq, wk, wv, wa, wb, wo, x, S)
    assert np.array_equal(S, S0 * np.float32(0.5))   # sigmoid(0) = 1/2, q = k = 0
    assert np.array_equal(x2, x)


# ------------------------------------------------------------------ MLA block
def _mla_setup(rng, nh=3, q_lora=24, kv_lora=16, rope=8, nope=8, vdim=8, H=40, cap=12):
    g = synth.f32_to_bf16_bits(1.0 + rng.normal(0, 0.2, size=H).astype(np.float32))
    gq = synth.f32_to_bf16_bits(1.0 + rng.normal(0, 0.2, size=q_lora).astype(np.float32))
    gkv = synth.f32_to_bf16_bits(1.0 + rng.normal(0, 0.2, size=kv_lora).astype(np.float32))
    wqa = rand_bits(rng, (q_lora, H), 0.3)
    wqb = rand_bits(rng, (nh * (nope + rope), q_lora), 0.3)
    wkva = rand_bits(rng, (kv_lora + rope, H), 0.3)
    wkvb = rand_bits(rng, (nh * (nope + vdim), kv_lora), 0.3)
    wo = rand_bits(rng, (H, nh * vdim), 0.3)
    cache = rand_bits(rng, (cap, kv_lora + rope), 1.0)
    x = rng.normal(size=H)
    return dict(nh=nh, q_lora=q_lora, kv_lora=kv_lora, rope=rope, nope=nope, vdim=vdim, H=H, cap=cap,
                g=g, gq=gq, gkv=gkv, wqa=wqa, wqb=wqb, wkva=wkva, wkvb=wkvb, wo=wo, cache=cache, x=x)


def _mla(d, pos):
    x2 = d["x"].copy()
    c = d["cache"]
    rc = oracle.lib().orc_mla_block(d["H"], d["nh"], d["q_lora"], d["kv_lora"], d["rope"], d["nope"], d["vdim"],
                                    1e-6, 1e4, *(oracle.ptr(d[n]) for n in ("g", "wqa", "gq", "wqb", "wkva", "gkv",
                                                                             "wkvb", "wo")),
                                    oracle.ptr(x2), pos, oracle.ptr(c), d["cap"])
    assert rc == 0
    return x2


def test_mla_matches_absorbed_form():
    """The plain form equals the weight-absorbed form (scores from
    (W_uk^T q_nope) . c_t, output W_uv (sum_t p_t c_t)), written here in NumPy."""
    rng = np.random.default_rng(30)
    d = _mla_setup(rng)
    pos = 9
    c0 = d["cache"].copy()
    x2 = _mla(d, pos)
    nh, nope, rope, vdim, kvl = d["nh"], d["nope"], d["rope"], d["vdim"], d["kv_lora"]
    xn = R.rms_norm(d["x"], d["g"], 1e-6)
    cq = R.rms_norm(R.widen(d["wqa"]) @ xn, d["gq"], 1e-6)
    q = (R.widen(d["wqb"]) @ cq).reshape(nh, nope + rope)
    qn, qp = q[:, :nope], R.rope_half(q[:, nope:], pos, 1e4)
    ckv = R.widen(d["wkva"]) @ xn
    c_new = R.bf16_round_f64(R.rms_norm(ckv[:kvl], d["gkv"], 1e-6))
    kpe_new = R.bf16_round_f64(R.rope_half(ckv[kvl:], pos, 1e4))
    C = R.widen(c0[: pos + 1]).copy()
    C[pos, :kvl] = c_new
    C[pos, kvl:] = kpe_new
    # the block must have written exactly this row
    assert np.array_equal(R.widen(d["cache"][pos]), C[pos])
    Wkvb = R.widen(d["wkvb"]).reshape(nh, nope + vdim, kvl)
    Wuk, Wuv = Wkvb[:, :nope], Wkvb[:, nope:]
    o = []
    for h in range(nh):
        qt = Wuk[h].T @ qn[h]                       # absorbed query in latent space
        s = (C[:, :kvl] @ qt + C[:, kvl:] @ qp[h]) / math.sqrt(nope + rope)
        p = np.exp(s - s.max())
        p /= p.sum()
        o.append(Wuv[h] @ (p @ C[:, :kvl]))
    want = d["x"] + R.widen(d["wo"]) @ np.concatenate(o)
    assert np.allclose(x2, want, rtol=1e-10, atol=1e-10)


def test_mla_single_row_returns_projected_latent():
    rng = np.random.default_rng(31)
    d = _mla_setup(rng, H=24, nh=3, vdim=8)
    d["wo"] = np.zeros((24, 24), np.uint16)
    np.fill_diagonal(d["wo"], BF1)
    x2 = _mla(d, 0)
    kvl, nope, vdim, nh = d["kv_lora"], d["nope"], d["vdim"], d["nh"]
    c = R.widen(d["cache"][0, :kvl])
    Wkvb = R.widen(d["wkvb"]).reshape(nh, nope + vdim, kvl)
    want = np.concatenate([Wkvb[h, nope:] @ c for h in range(nh)])
    assert np.allclose(x2 - d["x"], want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ whole step
def test_zero_layer_weights_identity_residual_dense():
    w = WL.mini_dense()
    W = HostWeights(w)
    zeros_like_weights(w, W)
    kv = host_kv(w)
    toks = synth.tokens(w, 3)
    pos = np.array([5, 37, 0])
    out = ostep.decode_step(w, W, toks, pos, kv)
    # every block adds exactly zero: the residual is the embedding row, bit for bit
    assert np.array_equal(out["x_final"], R.widen(W("embed"))[toks])
    want = R.rms_norm(R.widen(W("embed"))[toks], W("final_norm").reshape(-1), w.rms_eps) @ R.widen(W("lm_head")).T
    assert np.allclose(out["logits"], want.astype(np.float32), rtol=1e-6, atol=1e-6)


def test_zero_layer_weights_hybrid_moe():
    w = WL.mini_hybrid()
    W = HostWeights(w)
    zeros_like_weights(w, W)
    kv = host_kv(w)
    kv0 = kv_copy(kv)
    toks = synth.tokens(w, 2)
    pos = np.array([3, 28])
    out = ostep.decode_step(w, W, toks, pos, kv)
    assert np.array_equal(out["x_final"], R.widen(W("embed"))[toks])
    # router of zeros: probabilities 1/E, experts 0..k-1, weights 1/k
    assert np.array_equal(out["expert_ids"], np.broadcast_to(np.arange(w.top_k), out["expert_ids"].shape))
    assert np.allclose(out["expert_w"], 1.0 / w.top_k)
    # delta-rule state halves exactly (sigmoid(0) = 1/2, q = k = 0)
    for l in range(w.n_layers):
        if w.layer_kind(l) == "kda":
            assert np.array_equal(kv[l][:2], kv0[l][:2] * np.float32(0.5))
            assert np.array_equal(kv[l][2:], kv0[l][2:])


def test_moe_identical_experts_sum_to_two_shared():
    """With every routed expert equal to the shared one, renormalised routing
    weights sum to 1, so the block adds exactly 2x the shared SwiGLU."""
    w = WL.mini_moe().replace(n_layers=1)
    W = HostWeights(w)
    for e in range(w.n_experts):
        W.overrides[f"L0.e{e}_gate"] = np.ascontiguousarray(W("L0.sh0_gate")[: w.expert_ffn])
        W.overrides[f"L0.e{e}_up"] = np.ascontiguousarray(W("L0.sh0_up")[: w.expert_ffn])
        W.overrides[f"L0.e{e}_down"] = np.ascontiguousarray(W("L0.sh0_down")[:, : w.expert_ffn])
    # make the shared expert as narrow as a routed one by zeroing the rest
    sg, su, sd = W("L0.sh0_gate").copy(), W("L0.sh0_up").copy(), W("L0.sh0_down").copy()
    sg[w.expert_ffn:] = 0
    su[w.expert_ffn:] = 0
    sd[:, w.expert_ffn:] = 0
    W.overrides["L0.sh0_gate"], W.overrides["L0.sh0_up"], W.overrides["L0.sh0_down"] = sg, su, sd
    for n in ("wq", "wk", "wv", "wo"):
        W.overrides["L0." + n] = np.zeros_like(W("L0." + n))
    kv = host_kv(w)
    toks = synth.tokens(w, 2)
    out = ostep.decode_step(w, W, toks, np.array([4, 9]), kv)
    x0 = R.widen(W("embed"))[toks]
    xn = R.rms_norm(x0, W("L0.ffn_norm").reshape(-1), w.rms_eps)
    f = (R.silu(xn @ R.widen(sg).T) * (xn @ R.widen(su).T)) @ R.widen(sd).T
    assert np.allclose(out["x_final"], x0 + 2.0 * f, rtol=1e-10, atol=1e-12)


def test_dense_step_matches_numpy_reference():
    w = WL.tiny_dense()
    W = HostWeights(w)
    kv_a = host_kv(w)
    kv_b = kv_copy(kv_a)
    toks = synth.tokens(w, 1)
    pos = np.array([w.context])
    out = ostep.decode_step(w, W, toks, pos, kv_a)
    ref_logits, ref_x = R.dense_step(w, W.all(), toks, pos, kv_b)
    assert np.allclose(out["x_final"], ref_x, rtol=1e-10, atol=1e-10)
    rms = np.sqrt(np.mean(ref_logits ** 2))
    assert np.max(np.abs(out["logits"] - ref_logits)) < 1e-6 * rms
    assert out["next"][0] == int(np.argmax(ref_logits[0].astype(np.float32)))
    for l in range(w.n_layers):
        assert np.array_equal(kv_a[l], kv_b[l])


def test_batch_rows_are_independent():
    w = WL.mini_moe()
    W = HostWeights(w)
    kv = host_kv(w)
    toks = synth.tokens(w, 3)
    pos = np.array([44, 10, 30])
    full = ostep.decode_step(w, W, toks, pos, kv_copy(kv))
    for b in range(3):
        kvb = kv_copy(kv)
        # move sequence b into slot 0 of a batch of one
        for l in range(w.n_layers):
            if kvb[l].ndim == 5:
                kvb[l][:, 0] = kv[l][:, b]
            else:
                kvb[l][0] = kv[l][b]
        one = ostep.decode_step(w, W, toks[b:b + 1], pos[b:b + 1], kvb)
        assert np.array_equal(one["logits"][0], full["logits"][b])
        assert np.array_equal(one["expert_ids"][:, 0], full["expert_ids"][:, b])


# ------------------------------------------------------------------ verify
def test_acceptance_brute_force():
    rng = np.random.default_rng(40)
    for _ in range(500):
        n = 8
        arg = rng.integers(0, 4, size=n)
        toks = rng.integers(0, 4, size=n)
        # brute force: the longest prefix of drafts that each equal the argmax before them
        best = 0
        for j in range(1, n):
            if all(toks[i] == arg[i - 1] for i in range(1, j + 1)):
                best = j
        assert ostep.acceptance(toks, arg) == best + 1


def test_verify_rows_equal_sequential_decode_and_commit():
    w = WL.mini_hybrid()
    W = HostWeights(w)
    kv = host_kv(w)
    p = 20
    # drafts: greedy continuation for 3 tokens, then a wrong one -> accept 4... unless a chance match
    anchor = int(synth.tokens(w, 1)[0])
    seq = [anchor]
    kv_g = kv_copy(kv)
    for j in range(4):
        o = ostep.decode_step(w, W, [seq[-1]], [p + j], kv_g)
        seq.append(int(o["next"][0]))
    toks = seq[:4] + [(seq[4] + 1) % w.vocab] + [0, 1, 2]
    kv_v = kv_copy(kv)
    v = ostep.verify_step(w, W, np.array([toks]), np.array([p]), kv_v)
    assert int(v["accept_len"][0]) == 4
    assert int(v["next"][0]) == seq[4]
    kv_s = kv_copy(kv)
    for j in range(8):
        o = ostep.decode_step(w, W, [toks[j]], [p + j], kv_s)
        assert np.array_equal(o["logits"][0], v["logits"][0, j])
        if j == 3:
            committed = {l: kv_s[l].copy() for l in range(w.n_layers) if w.layer_kind(l) == "kda"}
    for l, st in committed.items():
        assert np.array_equal(kv_v[l][0], st[0])


def test_kda_general_gates_projection_identities():
    """For unit k: S'^T k = (alpha - beta) S^T k + beta v, and for z orthogonal
    to k: S'^T z = alpha S^T z (alpha scales the old state outside the delta)."""
    rng = np.random.default_rng(23)
    nh, dk, dv = 2, 16, 8
    H, g, wq, wk, wv, wa, wb, wo, x = _kda_setup(rng, nh, dk, dv)
    S = rng.normal(size=(nh, dk, dv)).astype(np.float32)
    S0 = S.astype(np.float64)
    _kda(H, nh, dk, dv, g, wq, wk, wv, wa, wb, wo, x, S)
    xn = R.rms_norm(x, g, 1e-6)
    k = (R.widen(wk) @ xn).reshape(nh, dk)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = (R.widen(wv) @ xn).reshape(nh, dv)
    al = 1.0 / (1.0 + np.exp(-(R.widen(wa) @ xn)))
    be = 1.0 / (1.0 + np.exp(-(R.widen(wb) @ xn)))
    for h in range(nh):
        assert 0.05 < al[h] < 0.95 and abs(al[h] - be[h]) > 1e-3
        want = (al[h] - be[h]) * (S0[h].T @ k[h]) + be[h] * v[h]
        assert np.allclose(S[h].T.astype(np.float64) @ k[h], want, atol=1e-5)
        z = rng.normal(size=dk)
        z -= (z @ k[h]) * k[h]
        assert np.allclose(S[h].T.astype(np.float64) @ z, al[h] * (S0[h].T @ z), atol=1e-5)


def test_head_argmax_ties_pick_lowest_index():
    w = WL.tiny_dense()
    W = HostWeights(w)
    zeros_like_weights(w, W)
    lm = W("lm_head").copy()
    lm[:] = 0
    lm[5] = W("embed")[0]
    lm[900] = W("embed")[0]        # rows 5 and 900 tie for the maximum
    W.overrides["lm_head"] = lm
    out = ostep.decode_step(w, W, np.array([0]), np.array([3]), host_kv(w))
    assert out["logits"][0, 5] == out["logits"][0, 900] > 0
    assert int(out["next"][0]) == 5
    lm[:] = 0
    out = ostep.decode_step(w, W, np.array([0]), np.array([3]), host_kv(w))
    assert int(out["next"][0]) == 0


def test_moe_routed_weights_reach_their_own_experts():
    """Each routed expert writes a one-hot pattern of its own: its gate and up
    matrices have one nonzero row (the same vector a for every expert), so its
    hidden state is s = silu(a.xn) * (a.xn) in unit 0 only, and its down
    projection maps unit 0 to residual row e.  With attention and the shared
    expert zeroed, the block adds w_e * s to row e for every chosen expert e
    and nothing elsewhere, so each expert's weight is read off the residual.
    The expected ids and weights come from a brute-force sort of a NumPy
    softmax of the router logits.  Catches a weight given to the wrong expert
    (a permutation of the chosen ones), a missing or wrong renormalisation, a
    weight applied to the wrong token, and an expert added twice or never."""
    w = WL.mini_moe().replace(n_layers=1)
    assert w.hidden >= w.n_experts
    W = HostWeights(w)
    rng = np.random.default_rng(7)
    for n in ("wq", "wk", "wv", "wo"):
        W.overrides["L0." + n] = np.zeros_like(W("L0." + n))
    for n in ("gate", "up", "down"):
        W.overrides[f"L0.sh0_{n}"] = np.zeros_like(W(f"L0.sh0_{n}"))
    a_bits = rand_bits(rng, (w.hidden,), 0.05)
    for e in range(w.n_experts):
        g = np.zeros((w.expert_ffn, w.hidden), np.uint16)
        g[0] = a_bits
        d = np.zeros((w.hidden, w.expert_ffn), np.uint16)
        d[e, 0] = BF1
        W.overrides[f"L0.e{e}_gate"] = g
        W.overrides[f"L0.e{e}_up"] = g.copy()
        W.overrides[f"L0.e{e}_down"] = d
    kv = host_kv(w)
    B = 4
    toks = synth.tokens(w, B)
    out = ostep.decode_step(w, W, toks, np.array([3, 9, 17, 30]), kv)
    x0 = R.widen(W("embed"))[toks]
    xn = R.rms_norm(x0, W("L0.ffn_norm").reshape(-1), w.rms_eps)
    lg = (xn @ R.widen(W("L0.router")).T).astype(np.float32).astype(np.float64)
    for b in range(B):
        order = sorted(range(w.n_experts), key=lambda e: (-lg[b, e], e))[: w.top_k]
        p = np.exp(lg[b] - lg[b].max())
        p /= p.sum()
        wts = p[order] / p[order].sum()
        assert list(out["expert_ids"][0, b]) == order
        av = float(xn[b] @ R.widen(a_bits))
        s = R.silu(av) * av
        want = np.zeros(w.hidden)
        want[order] = wts * s
        got = out["x_final"][b] - x0[b]
        assert np.allclose(got, want, rtol=1e-9, atol=1e-12 * abs(s)), f"token {b}"
        # the weights differ from expert to expert, so a permutation would show
        assert len(set(np.round(wts, 12))) == w.top_k
