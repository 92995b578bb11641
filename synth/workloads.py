"""Workload shapes and the inventory of synthetic tensors each one draws.

This file describes inputs only: model shapes, the names and shapes of the
bf16 weight tensors, their draw parameters and the seeds.  It holds none of
the decode step's arithmetic.  The oracle and the GPU path both receive their
inputs through it; the GPU library independently enumerates the tensors it
expects and a test checks that the two lists agree.

The decode step these shapes feed is the whole-model decode pass of the TPU
megakernel write-up (Inferact, "700 TPS on Kimi K3: A Case for TPU
Megakernels", sections "Why megakernels?" and "Our Kimi K3 megakernel"):
attention (GQA, or MLA / gated delta rule by layer index), router, shared
expert, routed experts, residual adds and RMSNorm, then the LM head.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

# Draw standard deviations.
W_SIGMA = 0.02          # every weight matrix
KV_SIGMA = 1.0          # cached K/V rows, MLA latent rows, KDA state
V_TILE = 32             # positions per tile of the GQA V cache


@dataclass
class Workload:
    name: str
    n_layers: int
    hidden: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e4
    attn_kind: int = 0              # 0: GQA in every layer; 1: hybrid MLA / KDA
    # GQA
    n_q_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 0
    # MLA (layer l is MLA iff l % mla_every == mla_every - 1)
    mla_every: int = 0
    mla_heads: int = 0
    q_lora: int = 0
    kv_lora: int = 0
    rope_dim: int = 0
    nope_dim: int = 0
    v_dim: int = 0
    # KDA (gated delta rule)
    kda_heads: int = 0
    kda_dk: int = 0
    kda_dv: int = 0
    kda_qk_l2norm: int = 1
    # FFN: dense if n_experts == 0
    ffn_dim: int = 0
    n_experts: int = 0
    top_k: int = 0
    expert_ffn: int = 0
    n_shared: int = 0
    shared_ffn: int = 0
    norm_topk: int = 1
    router_sigma: float = W_SIGMA
    # norm gains: 0 -> all ones (the stated workloads); > 0 -> 1 + N(0, gain_sigma)
    gain_sigma: float = 0.0
    # batch / context used by tests and the benchmark
    batches: Tuple[int, ...] = (1,)
    context: int = 16               # prior cached positions per sequence
    max_ctx: int = 32               # cache capacity in positions
    max_batch: int = 8
    # paged attention caches: positions per page (0: contiguous) and pool pages per layer
    kv_page: int = 0
    kv_pages: int = 0
    steps: int = 1
    seed_base: int = 0              # seeds: weights 1000+s, kv 2000+s, state 3000+s, tokens 4000+s, drafts 5000+s

    # ---- derived -------------------------------------------------------
    def layer_kind(self, l: int) -> str:
        if self.attn_kind == 0:
            return "gqa"
        return "mla" if (l % self.mla_every) == self.mla_every - 1 else "kda"

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0

    @property
    def mla_qk_dim(self) -> int:
        return self.nope_dim + self.rope_dim

    @property
    def mla_row(self) -> int:
        return self.kv_lora + self.rope_dim

    def seed(self, what: str) -> int:
        base = {"weights": 1000, "kv": 2000, "state": 3000, "tokens": 4000, "drafts": 5000}[what]
        return base + self.seed_base

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class TensorSpec:
    name: str
    rows: int
    cols: int
    kind: str          # "normal" (bf16 N(0, sigma)), "gain" (norm gain)
    sigma: float

    @property
    def numel(self) -> int:
        return self.rows * self.cols


def tensor_inventory(w: Workload) -> List[TensorSpec]:
    """Every bf16 weight tensor of the model, logical row-major [out, in].

    Order: embedding, then per layer (attention block, FFN block), then the
    final norm gain and the LM head.
    """
    T: List[TensorSpec] = []
    H = w.hidden

    def mat(name, rows, cols, sigma=W_SIGMA):
        T.append(TensorSpec(name, rows, cols, "normal", sigma))

    def gain(name, n):
        T.append(TensorSpec(name, 1, n, "gain", w.gain_sigma))

    mat("embed", w.vocab, H)
    for l in range(w.n_layers):
        p = f"L{l}."
        kind = w.layer_kind(l)
        gain(p + "attn_norm", H)
        if kind == "gqa":
            mat(p + "wq", w.n_q_heads * w.head_dim, H)
            mat(p + "wk", w.n_kv_heads * w.head_dim, H)
            mat(p + "wv", w.n_kv_heads * w.head_dim, H)
            mat(p + "wo", H, w.n_q_heads * w.head_dim)
        elif kind == "mla":
            mat(p + "mla_wqa", w.q_lora, H)
            gain(p + "mla_q_norm", w.q_lora)
            mat(p + "mla_wqb", w.mla_heads * w.mla_qk_dim, w.q_lora)
            mat(p + "mla_wkva", w.mla_row, H)
            gain(p + "mla_kv_norm", w.kv_lora)
            mat(p + "mla_wkvb", w.mla_heads * (w.nope_dim + w.v_dim), w.kv_lora)
            mat(p + "mla_wo", H, w.mla_heads * w.v_dim)
        else:
            hd = w.kda_heads
            mat(p + "kda_wq", hd * w.kda_dk, H)
            mat(p + "kda_wk", hd * w.kda_dk, H)
            mat(p + "kda_wv", hd * w.kda_dv, H)
            mat(p + "kda_walpha", hd, H)
            mat(p + "kda_wbeta", hd, H)
            mat(p + "kda_wo", H, hd * w.kda_dv)
        gain(p + "ffn_norm", H)
        if not w.is_moe:
            mat(p + "w_gate", w.ffn_dim, H)
            mat(p + "w_up", w.ffn_dim, H)
            mat(p + "w_down", H, w.ffn_dim)
        else:
            mat(p + "router", w.n_experts, H, w.router_sigma)
            for s in range(w.n_shared):
                mat(p + f"sh{s}_gate", w.shared_ffn, H)
                mat(p + f"sh{s}_up", w.shared_ffn, H)
                mat(p + f"sh{s}_down", H, w.shared_ffn)
            for e in range(w.n_experts):
                mat(p + f"e{e}_gate", w.expert_ffn, H)
                mat(p + f"e{e}_up", w.expert_ffn, H)
                mat(p + f"e{e}_down", H, w.expert_ffn)
    gain("final_norm", H)
    mat("lm_head", w.vocab, H)
    return T


def weight_bytes(w: Workload) -> int:
    return sum(t.numel for t in tensor_inventory(w)) * 2


# --------------------------------------------------------------------------
# Cache / state layout of the single caller-owned KV buffer.  Per layer, in
# layer order:
#   GQA: K bf16[max_batch][n_kv][max_ctx][head_dim], then V with the same
#        logical shape stored in V_TILE-position tiles, dim-major within a
#        tile: bf16[max_batch][n_kv][max_ctx / V_TILE][head_dim][V_TILE]
#        (max_ctx a multiple of V_TILE).  kv_layout gives the logical shape.
#   MLA: latent rows bf16[max_batch][max_ctx][kv_lora + rope_dim]
#   KDA: state fp32[max_batch][kda_heads][kda_dk][kda_dv]
# Each layer's region starts on a 256-byte boundary.
# --------------------------------------------------------------------------
def _align(x: int, a: int = 256) -> int:
    return (x + a - 1) // a * a


def kv_layout(w: Workload):
    """List of (kind, offset_bytes, nbytes, shape, dtype) per layer, and the total."""
    out = []
    off = 0
    Bm, C = w.max_batch, w.max_ctx
    for l in range(w.n_layers):
        kind = w.layer_kind(l)
        if kind == "gqa":
            shape = (Bm, w.n_kv_heads, C, w.head_dim)
            n = 2 * Bm * w.n_kv_heads * C * w.head_dim * 2
            out.append(("gqa", off, n, shape, "bf16"))
        elif kind == "mla":
            shape = (Bm, C, w.mla_row)
            n = Bm * C * w.mla_row * 2
            out.append(("mla", off, n, shape, "bf16"))
        else:
            shape = (Bm, w.kda_heads, w.kda_dk, w.kda_dv)
            n = Bm * w.kda_heads * w.kda_dk * w.kda_dv * 4
            out.append(("kda", off, n, shape, "f32"))
        off = _align(off + n)
    return out, off


def kv_pool_layout(w: Workload):
    """Paged form of kv_layout (w.kv_page > 0): per layer (kind, offset_bytes,
    nbytes, shape, dtype) with N = w.kv_pages pages of P = w.kv_page positions
    in place of the slots of a GQA or MLA layer; delta-rule states stay one
    per slot.  Returns the list and the total."""
    out = []
    off = 0
    N, P = w.kv_pages, w.kv_page
    for l in range(w.n_layers):
        kind = w.layer_kind(l)
        if kind == "gqa":
            shape = (N, w.n_kv_heads, P, w.head_dim)
            n = 2 * N * w.n_kv_heads * P * w.head_dim * 2
        elif kind == "mla":
            shape = (N, P, w.mla_row)
            n = N * P * w.mla_row * 2
        else:
            shape = (w.max_batch, w.kda_heads, w.kda_dk, w.kda_dv)
            n = w.max_batch * w.kda_heads * w.kda_dk * w.kda_dv * 4
        out.append((kind, off, n, shape, "f32" if kind == "kda" else "bf16"))
        off = _align(off + n)
    return out, off


# --------------------------------------------------------------------------
# The workloads.
# --------------------------------------------------------------------------
def tiny_dense() -> Workload:
    """2-layer dense decoder, hidden 256, 4/4 heads of 64, FFN 1024, vocab 1024."""
    return Workload(name="tiny_dense_2L_h256", n_layers=2, hidden=256, vocab=1024,
                    n_q_heads=4, n_kv_heads=4, head_dim=64, ffn_dim=1024,
                    batches=(1,), context=16, max_ctx=32, max_batch=8, steps=1, seed_base=0)


def small_moe() -> Workload:
    """8-layer MoE decoder, hidden 2048, GQA 16/4 x 128, 64 experts top-4 + 1 shared."""
    return Workload(name="small_moe_8L_h2048_e64", n_layers=8, hidden=2048, vocab=32000,
                    n_q_heads=16, n_kv_heads=4, head_dim=128,
                    n_experts=64, top_k=4, expert_ffn=1024, n_shared=1, shared_ffn=2048,
                    router_sigma=0.1, batches=(1, 8), context=1024, max_ctx=1024 + 64,
                    max_batch=8, steps=32, seed_base=1)


def dense_27b() -> Workload:
    """64-layer dense decoder shaped like a 27B model: hidden 5120, GQA 40/8 x 128, FFN 17408."""
    return Workload(name="dense_27b_64L_h5120", n_layers=64, hidden=5120, vocab=152064,
                    n_q_heads=40, n_kv_heads=8, head_dim=128, ffn_dim=17408,
                    batches=(1, 2, 4, 8), context=4096, max_ctx=4096 + 256,
                    max_batch=8, steps=256, seed_base=2)


def hybrid_moe() -> Workload:
    """One GPU's share of a 92-layer hybrid MoE: MLA every 4th layer, gated delta rule otherwise."""
    return Workload(name="hybrid_moe_92L_h7168", n_layers=92, hidden=7168, vocab=163840,
                    attn_kind=1, mla_every=4, mla_heads=32, q_lora=1536, kv_lora=512,
                    rope_dim=64, nope_dim=128, v_dim=128,
                    kda_heads=32, kda_dk=128, kda_dv=128, kda_qk_l2norm=1,
                    n_experts=16, top_k=8, expert_ffn=2048, n_shared=1, shared_ffn=2048,
                    batches=(1, 8), context=8192, max_ctx=8192 + 32, max_batch=8, steps=32,
                    seed_base=3)


def verify_hybrid() -> Workload:
    """Speculative verify on the hybrid model: 1 anchor + 7 drafts, context 8192."""
    return hybrid_moe().replace(name="verify_hybrid_92L_h7168", batches=(1,), seed_base=4)


# Reduced-size variants with the same structure, for tests the oracle finishes
# in seconds.  Sizes are chosen to span several GPU tiles with ragged tails.
def mini_dense() -> Workload:
    return Workload(name="mini_dense", n_layers=3, hidden=320, vocab=1000,
                    n_q_heads=6, n_kv_heads=2, head_dim=64, ffn_dim=864, gain_sigma=0.1,
                    batches=(1, 3, 8), context=37, max_ctx=64, max_batch=8, steps=2, seed_base=10)


def mini_moe() -> Workload:
    return Workload(name="mini_moe", n_layers=3, hidden=384, vocab=1500,
                    n_q_heads=4, n_kv_heads=2, head_dim=64,
                    n_experts=12, top_k=3, expert_ffn=192, n_shared=1, shared_ffn=256,
                    router_sigma=0.1, gain_sigma=0.1,
                    batches=(1, 5, 8), context=45, max_ctx=96, max_batch=8, steps=2, seed_base=11)


def mini_hybrid() -> Workload:
    return Workload(name="mini_hybrid", n_layers=4, hidden=384, vocab=1200,
                    attn_kind=1, mla_every=4, mla_heads=4, q_lora=128, kv_lora=512,
                    rope_dim=64, nope_dim=64, v_dim=64,
                    kda_heads=3, kda_dk=64, kda_dv=64, kda_qk_l2norm=1,
                    n_experts=8, top_k=4, expert_ffn=160, n_shared=1, shared_ffn=192,
                    gain_sigma=0.1, batches=(1, 8), context=29, max_ctx=48, max_batch=8,
                    steps=2, seed_base=12)


ALL = {
    "tiny_dense": tiny_dense,
    "small_moe": small_moe,
    "dense_27b": dense_27b,
    "hybrid_moe": hybrid_moe,
    "verify_hybrid": verify_hybrid,
    "mini_dense": mini_dense,
    "mini_moe": mini_moe,
    "mini_hybrid": mini_hybrid,
}


def get(name: str) -> Workload:
    return ALL[name]()
