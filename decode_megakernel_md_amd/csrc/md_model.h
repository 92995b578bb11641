// Kernel parameter block and per-layer table of the decode megakernel.
#pragma once
#include <stdint.h>

namespace md {

// device error bits (md_get_device_status)
enum : int { MDE_WATCHDOG = 1, MDE_TOKEN = 2, MDE_POSITION = 4, MDE_CAPACITY = 8, MDE_PAGE = 16 };

enum LayerKind : int { LK_GQA = 0, LK_MLA = 1, LK_KDA = 2 };

// One entry per layer, in device memory (the workspace).  Pointers are the
// caller's bf16 weight tensors; unused ones are null.
struct LayerDesc {
  int kind;
  int kda_idx;      // index among the delta-rule layers (verify snapshots), else -1
  uint64_t kv_off;  // byte offset of this layer's region in the KV / state buffer
  const uint16_t* attn_norm;
  // GQA
  const uint16_t *wq, *wk, *wv, *wo;
  // MLA
  const uint16_t *mla_wqa, *mla_qnorm, *mla_wqb, *mla_wkva, *mla_kvnorm, *mla_wkvb, *mla_wo;
  // KDA
  const uint16_t *kda_wq, *kda_wk, *kda_wv, *kda_wa, *kda_wb, *kda_wo;
  // FFN
  const uint16_t* ffn_norm;
  const uint16_t *w_gate, *w_up, *w_down;   // dense
  const uint16_t* router;                   // MoE
  const uint16_t *sh_gate, *sh_up, *sh_down;
  const uint16_t* const* experts;           // [n_experts][3] gate, up, down (device array)
};

struct Params {
  // model
  const LayerDesc* layers;
  const uint16_t* embed;
  const uint16_t* final_norm;
  const uint16_t* lm_head;
  int n_layers, H, V, max_batch, max_ctx;
  float eps, theta;
  int nq, nkv, hd;
  int ffn;
  int n_experts, top_k, expert_ffn, n_shared, shared_ffn, norm_topk;
  int mla_h, q_lora, nope, vdim, mla_chunks;   // MLA (kv_lora 512, rope 64)
  int kda_h, kda_dk, kda_dv, kda_l2;           // gated delta rule
  int n_kda;                                   // number of delta-rule layers
  // step
  int B;              // token rows: sequences (decode) or the verified tokens of one sequence
  int verify;         // 1: rows are tokens p..p+B-1 of sequence 0
  int ml_phase;       // >= 0: run only this phase (multi-launch step), of layer ml_layer
  int ml_layer;
  uint8_t* kda_ring;  // verify: per delta-rule layer, the state after each row fp32[L_kda][MAXB][nh][dk][dv]
  int32_t* out_accept;
  int32_t* out_next;
  int attn_chunks;
  const int32_t* tokens;
  const int32_t* positions;
  uint8_t* kv;
  // Attention-cache addressing.  A GQA or MLA layer's cache is n_pages pages
  // of pg_cap positions.  Contiguous caches have one page per sequence slot
  // (n_pages = max_batch, pg_cap = max_ctx, bt = null); paged caches
  // (pg_cap = 1 << pg_shift) find position pos of sequence s in page
  // bt[s * bt_stride + (pos >> pg_shift)], row pos & (pg_cap - 1).
  const int32_t* bt;
  int bt_stride, pg_cap, pg_shift, n_pages;
  float* logits;
  int32_t* out_tokens;
  int32_t* out_ids;
  // workspace
  uint8_t* ws;
  uint32_t ws_bytes;
  float* x;           // residual fp32[MAXB][H] (rows owned by their workgroup)
  // The GEMV inputs (hi/lo activations) have one buffer per use within a
  // step, so that no address is read before it is written in the same launch
  // (their loads may then hit a copy in the local L2, see md_device.h):
  // index 2l = attention input of layer l, 2l+1 = its FFN input, 2L = the
  // final norm's input; the others one per layer.
  uint32_t off_u;     // hi/lo bf16[2][MAXB][H] x (2L+1), u_stride apart: norm input (gain folded, not yet scaled)
  uint32_t u_stride, ou_stride, h_stride, hs_stride, hr_lstride, uq_stride;  // bytes per use
  uint32_t ssq_stride, ssq2_stride;  // the partial sums of squares that scale them, one buffer per use too
  uint32_t off_ssq;   // fp32[G][MAXB] x (2L+1), ssq_stride apart: partial sums of squares of x (indexed as u)
  uint32_t off_qkv;   // fp32[MAXB][nq+2nkv][hd]
  uint32_t off_attn;  // attention partial outputs fp32[MAXB][nq][C][hd]
  uint32_t off_attn_ml; // attention partial (max, sum) fp32[MAXB][nq][C][2]
  uint32_t off_ou;    // hi/lo bf16[2][MAXB][nq*hd] per layer
  uint32_t off_h;     // hi/lo bf16[2][MAXB][F]           dense FFN hidden, per layer
  uint32_t off_rl;    // {f32, u32}[MAXB][n_experts]       router logits, each with its layer's tag
  uint32_t off_hs;    // hi/lo bf16[2][MAXB][shared_ffn]   shared expert hidden, per layer
  uint32_t off_hr;    // hi/lo bf16[nu][2][MAXB][expert_ffn] routed hidden (x routing weight), U order, per layer
  uint32_t hr_stride; // bytes per routed expert slot
  uint32_t off_uq;    // hi/lo bf16[2][MAXB][q_lora]        g_q * c_q0 (MLA), per layer
  uint32_t off_ssq2;  // fp32[G][MAXB]                      partial sums of squares of c_q0, per layer
  uint32_t off_ckv;   // fp32[MAXB][576]                    raw latent + key rope part
  uint32_t off_qm;    // fp32[MAXB][nh][nope + 64]          q (MLA)
  uint32_t off_qabs;  // fp32[MAXB][nh][576]                absorbed, rotated, scaled q
  uint32_t off_mz;    // fp32[MAXB][C][nh][512]             attention partial z
  uint32_t off_mml;   // fp32[MAXB][C][nh][2]               attention partial (max, sum)
  uint32_t off_mzc;   // fp32[MAXB][nh][512]                z combined over the chunks
  uint32_t off_kda;   // fp32[MAXB][2 nh dk + nh dv + 2 nh] delta-rule projections
  uint32_t off_cand;  // argmax candidates {f32, i32}[G][MAXB]
  uint32_t off_zero;  // 1 KB that stays zero (target of masked loads)
  const float* rope;  // (cos, sin) fp32[max_ctx][rope_d/2][2]
  int rope_d;
  unsigned* sync;     // counters, 2 banks
  int* err;
  int n_sync;
  int sync_attn_base;
  int bank;
  unsigned spin_limit;
  uint64_t* trace;    // optional: per WG trace_n wall-clock stamps (phase end, then start after the wait)
  int trace_n;
  int moe_all;        // 1: the routed gate/up phase streams every expert (the step's tokens are expected to
                      // choose them all), so its stream starts before the routing is known
  uint32_t step_seq;  // steps of this model enqueued before this one (router-logit tags)
};

}  // namespace md
