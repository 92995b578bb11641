/*
 * md.h -- C ABI of the MI355X decode megakernel library (libmd.so).
 *
 * One decode step of a whole transformer / MoE decoder for a batch of 1..64
 * sequences runs as ONE persistent HIP launch on gfx950: embedding, and per
 * layer RMSNorm, attention (GQA, or multi-head latent attention / gated delta
 * rule chosen by layer index), router, shared and routed SwiGLU experts and
 * residual adds, then the final norm, LM head and greedy argmax.  This is the
 * decode megakernel of Inferact, "700 TPS on Kimi K3: A Case for TPU
 * Megakernels": section "Why megakernels?" (the whole decoder step inside one
 * program so that weight loads are not tied to kernel boundaries and the HBM
 * interface stays busy) and section "Our Kimi K3 megakernel" (one call over
 * all layers; attention kind chosen by layer index; per layer attention,
 * router, shared expert, routed experts).  Section "DSpark" defines the
 * verify step: one launch scores an anchor and 7 proposed continuations.
 *
 * Conventions.
 *  - All functions have C linkage; no C++ exception crosses this boundary.
 *  - Every pointer marked "dev" is a device pointer owned by the caller; the
 *    library never allocates or frees bulk device memory and keeps raw
 *    pointers only until md_free_model.  "host" pointers are read during the
 *    call only.
 *  - Calls that take a stream enqueue work and return; results are valid once
 *    the stream has synchronised.  A model handle is used by one stream at a
 *    time; calls on one handle must not overlap.
 *  - Return values are md_status codes.  On failure nothing is enqueued and
 *    md_last_error() describes the cause.
 *  - Weights are bf16, one device buffer per tensor, in the order
 *    md_weight_info enumerates (16-byte aligned).  The embedding table and
 *    the norm gains are plain row-major; every other matrix (logical
 *    row-major [out][in]) is passed in the tiled layout md_pack_weight
 *    writes (md_weight_layout tells which).
 *  - Activations and accumulations are fp32; projections run on bf16 matrix
 *    cores with each fp32 activation split into two bf16 halves (hi + lo),
 *    which keeps about 16 significant bits of the activation.
 */
#ifndef MD_H
#define MD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct md_model md_model; /* opaque; owned by the library */

typedef enum {
  MD_OK = 0,
  MD_EINVAL = -1,       /* bad argument: size, pointer, alignment, range */
  MD_EUNSUPPORTED = -2, /* device or configuration outside what the kernels support */
  MD_ENOMEM = -3,       /* a caller-provided buffer is too small */
  MD_EHIP = -4,         /* a HIP runtime call failed */
  MD_EDEVICE = -5       /* the device reported an error (watchdog, bad token) */
} md_status;

/* Model shape.  attn_kind 0: GQA in every layer.  attn_kind 1: hybrid, layer
 * l is multi-head latent attention when l % mla_every == mla_every - 1 and a
 * gated delta-rule layer otherwise.  n_experts == 0 selects a dense SwiGLU FFN
 * of width ffn_dim; otherwise each layer routes every token to top_k of
 * n_experts SwiGLU experts of width expert_ffn (softmax over all experts,
 * renormalised over the chosen ones when norm_topk) plus n_shared always-on
 * experts of width shared_ffn.
 *
 * max_batch (1..64) is the number of sequence slots.  Models with max_batch
 * <= 8 run on the library's 8-row kernel build, which also runs the verify
 * step; larger ones on its 64-row build (decode only: section "Future work"
 * of the post, higher concurrency), whose step reads every weight once for
 * all the sequences and whose workspace holds 64 token rows.  On the 64-row
 * build a GQA model has at most 8 kv heads and a MoE model's experts that a
 * step's tokens may choose, min(n_experts, 64 * top_k), are at most 36. */
typedef struct md_config {
  int32_t n_layers, hidden, vocab, max_batch, max_ctx;
  float rms_eps, rope_theta;
  int32_t attn_kind;
  int32_t n_q_heads, n_kv_heads, head_dim;
  int32_t mla_every, mla_heads, q_lora, kv_lora, rope_dim, nope_dim, v_dim;
  int32_t kda_heads, kda_dk, kda_dv, kda_qk_l2norm;
  int32_t ffn_dim;
  int32_t n_experts, top_k, expert_ffn, n_shared, shared_ffn, norm_topk;
  int32_t flags; /* reserved, must be 0 */
  /* Paged attention caches (GQA and MLA layers).  kv_page = 0: contiguous,
   * one region of max_ctx positions per sequence slot (md_kv_bytes).
   * kv_page > 0 (a power of two, >= 32, dividing max_ctx): every GQA / MLA
   * layer's cache is a pool of kv_pages pages of kv_page positions, and the
   * _paged steps map each sequence's positions to pages through a block
   * table (see md_decode_step_paged).  Delta-rule states stay one per slot. */
  int32_t kv_page, kv_pages;
} md_config;

/* Number of weight tensors the model expects. */
size_t md_weight_count(const md_config* cfg);

/* Name and logical shape [rows][cols] of weight tensor i (bf16).  name
 * receives a NUL-terminated string truncated to name_cap.  Returns MD_EINVAL
 * for i out of range. */
md_status md_weight_info(const md_config* cfg, size_t i, char* name, size_t name_cap, int64_t* rows,
                         int64_t* cols);

/* Layout tensor i must be passed in: 0 = plain row-major, 1 = tiled
 * (md_pack_weight); -1 for an index out of range. */
int32_t md_weight_layout(const md_config* cfg, size_t i);

/* Tiled weight layout.  A matrix W[rows][cols] (cols a multiple of 32) is
 * cut into tiles of 16 rows (the last one zero-padded) and each tile into
 * k-steps of 32 columns.  Block (t, s) is 1024 contiguous bytes at offset
 * (t * cols/32 + s) * 1024, made of 64 chunks of 16 bytes; chunk c holds the
 * 8 bf16 values W[16t + 4*(c/16) + c%4][32s + 8*((c%16)/4) .. +7].  So a
 * block is exactly the operand one wave's 16x16x32 matrix instruction needs,
 * split into four 256-byte quarters of 4 rows, and a tile's blocks follow
 * each other: streaming a tile is one sequential read.
 * md_packed_bytes returns 0 for shapes the layout does not support. */
size_t md_packed_bytes(int64_t rows, int64_t cols);

/* Convert one row-major bf16 matrix (dev src) into the tiled layout (dev dst,
 * md_packed_bytes(rows, cols) bytes, must not overlap src).  Enqueued on
 * hip_stream. */
md_status md_pack_weight(const void* src, void* dst, int64_t rows, int64_t cols, void* hip_stream);

/* Bytes of device workspace the library needs (layer table, activation
 * buffers, partial results, sync counters).  The workspace is owned by the
 * caller, must stay allocated while the model lives, and must not be touched
 * by the caller. */
size_t md_workspace_bytes(const md_config* cfg);

/* Bytes of a KV / state buffer for `batch` sequence slots of `ctx_cap`
 * positions each, for a model of shape cfg (cfg's own max_batch and max_ctx
 * are replaced by batch and ctx_cap).  The buffer a model's steps take must
 * be sized and laid out for that model's own slots and capacity:
 * md_kv_bytes(cfg, cfg->max_batch, cfg->max_ctx).  Per layer, in layer
 * order, each region starting on a 256-byte boundary (Bm = slots, C =
 * capacity):
 *   GQA layer: K bf16[Bm][n_kv_heads][C][head_dim], then
 *              V bf16[Bm][n_kv_heads][C / 32][head_dim][32]:
 *              32-position tiles, dimension-major within a tile, so that
 *              V[b][h][t][d] sits at ((b*n_kv_heads + h)*C + t/32*32)*head_dim
 *              + d*32 + t%32 (C must be a multiple of 32)
 *   MLA layer: latent rows bf16[Bm][C][kv_lora + rope_dim]
 *              (RMS-normalised latent, then the rotated key part)
 *   KDA layer: state fp32[Bm][kda_heads][kda_dk][kda_dv]
 * Sequence b of a batch uses slot b.  Returns 0 (md_last_error says why) for
 * an invalid cfg, batch outside [1, 64] or a capacity the cfg does not allow.
 *
 * Paged configurations (cfg->kv_page = P > 0, cfg->kv_pages = N) give the
 * size of a page pool instead: the GQA and MLA regions hold N pages of P
 * positions each (ctx_cap must still be a multiple of P; it only bounds
 * positions), laid out as above with one page in place of one slot:
 *   GQA layer: K bf16[N][n_kv_heads][P][head_dim], then
 *              V bf16[N][n_kv_heads][P / 32][head_dim][32]
 *   MLA layer: latent rows bf16[N][P][kv_lora + rope_dim]
 *   KDA layer: state fp32[batch][kda_heads][kda_dk][kda_dv] (one per slot)
 * Page q of every layer belongs to the same owner: one block table serves
 * all layers. */
size_t md_kv_bytes(const md_config* cfg, int32_t batch, int32_t ctx_cap);

/* Validate cfg, check the device (gfx950, cooperative launch, LDS), record
 * the weight pointers (dev, n_weights of them) and build the layer table in
 * the workspace (dev, workspace_bytes >= md_workspace_bytes).  Copies are
 * issued on hip_stream and complete before return. */
md_status md_init_model(const md_config* cfg, const void* const* weights, size_t n_weights, void* workspace,
                        size_t workspace_bytes, void* hip_stream, md_model** out);

/* One decode step for `batch` sequences (1 <= batch <= max_batch).
 *   tokens       dev int32[batch]     current token of each sequence (0 <= t < vocab)
 *   positions    dev int32[batch]     number of cached positions before it; the new
 *                                     key/value (or latent row) is written at this row,
 *                                     so positions[b] < max_ctx is required
 *   kv_cache     dev, md_kv_bytes     read and updated in place
 *   out_logits   dev fp32[batch][vocab]
 *   out_tokens   dev int32[batch] or NULL: greedy argmax (lowest index on ties)
 *   out_expert_ids dev int32[n_layers][batch][top_k] or NULL (MoE only): experts
 *                chosen per layer and token, in descending router order
 * Token and position values live on the device and are checked there: an
 * out-of-range value sets the device error word (md_get_device_status) and
 * the step's outputs are undefined.  Each call alternates the model's bank
 * of sync counters and advances its step counter (the tag of the router
 * logits), both passed by value to the kernel: a HIP graph that captured
 * this call would replay stale ones, so capture md_decode_step_noalloc,
 * which clears what it relies on with kernels of its own. */
md_status md_decode_step(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                         float* out_logits, int32_t batch, int32_t* out_tokens, int32_t* out_expert_ids,
                         void* hip_stream);

/* md_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, kernels and results, but the step's scratch buffers
 * (activations, partial results, sync counters, error word) come from a
 * static device array of the library, 128 MiB per device, held from the
 * library's load until the process ends, instead of the model's workspace
 * (which still holds the layer table, expert pointers and rotary table
 * written by md_init_model).  The call allocates nothing and frees nothing;
 * it enqueues small fill kernels (clearing the counters, error word and zero
 * line the step relies on, and for MoE models the tagged router logits: the
 * array keeps whatever the last call on this device left) and the megakernel.  Returns MD_ENOMEM, enqueuing
 * nothing, when the model's step needs more scratch than the array holds
 * (md_workspace_bytes(cfg) > 128 MiB).  Every call on a device shares that
 * device's array: calls that overlap on one device (other streams, other
 * models, other threads) race and their results are undefined.
 * md_get_device_status reports this call's device errors like any step's. */
md_status md_decode_step_noalloc(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                                 float* out_logits, int32_t batch, int32_t* out_tokens, int32_t* out_expert_ids,
                                 void* hip_stream);

/* Paged attention caches (the agentic / serving workloads of the Kimi K3
 * post's section "Future work": KV cache movement and management).  The
 * model must be configured with kv_page = P > 0 and kv_pages = N, and kv_pool
 * is the pool md_kv_bytes(cfg, cfg->max_batch, cfg->max_ctx) describes.
 *   block_table  dev int32[batch][max_ctx / P]  row b maps sequence b's
 *                positions: positions j*P .. j*P + P-1 live in page
 *                block_table[b][j] (in [0, N)) of every GQA / MLA layer.
 *                Only the entries covering positions 0 .. positions[b] (for
 *                verify: positions[0] + n_tok - 1) are read.
 * Everything else is md_decode_step's (md_verify_step's): same arguments,
 * same results; the delta-rule states of sequence b stay in slot b.  Pages
 * may be shared between sequences for positions that are only read (a
 * common prefix); the page that receives a sequence's new row must be its
 * own for the step (two rows of one step writing one page position race).
 * A page id outside [0, N) sets the device error (md_get_device_status:
 * MD_EDEVICE) and page 0 is read in its place.  A contiguous model
 * (kv_page = 0) rejects these calls with MD_EINVAL, and a paged model
 * rejects md_decode_step / md_verify_step / md_decode_step_noalloc /
 * md_decode_step_multilaunch. */
md_status md_decode_step_paged(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_pool,
                               const int32_t* block_table, float* out_logits, int32_t batch, int32_t* out_tokens,
                               int32_t* out_expert_ids, void* hip_stream);
md_status md_verify_step_paged(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_pool,
                               const int32_t* block_table, float* out_logits, int32_t* out_accept_len,
                               int32_t* out_next_token, int32_t* out_expert_ids, int32_t batch, int32_t n_tok,
                               void* hip_stream);

/* KV movement on the device, enqueued on hip_stream (ordered with the steps
 * of that stream).
 * md_kv_copy_pages: page src_pages[i] -> dst_pages[i] (dev int32[n] each,
 *   n >= 0) of every GQA layer (K and V) and every MLA layer of a paged
 *   model: the copy-on-write of a shared page before a sequence writes into
 *   it, or a move.  A destination must not also be a source of the same
 *   call.  Ids outside [0, kv_pages) set the device error and are skipped.
 * md_kv_copy_slot: sequence slot src_slot -> dst_slot (both in
 *   [0, max_batch)): every delta-rule state and, for a contiguous model, the
 *   slot's GQA / MLA cache rows too (a paged model's rows are shared or
 *   copied through the block table and md_kv_copy_pages).  Forking a
 *   sequence = copy its slot (and, paged, point the new row of the block
 *   table at the same pages, copying the last partly-filled one). */
md_status md_kv_copy_pages(md_model* m, void* kv_pool, const int32_t* src_pages, const int32_t* dst_pages,
                           int32_t n, void* hip_stream);
md_status md_kv_copy_slot(md_model* m, void* kv, int32_t src_slot, int32_t dst_slot, void* hip_stream);

/* The same step as md_decode_step executed as one kernel launch per
 * operation (no megakernel): the baseline that exposes the inter-kernel
 * bubbles.  Same arguments and results. */
md_status md_decode_step_multilaunch(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                                     float* out_logits, int32_t batch, int32_t* out_tokens,
                                     int32_t* out_expert_ids, void* hip_stream);

/* Speculative verify of n_tok (2..8) tokens of one sequence in one launch
 * (section "DSpark": an anchor plus proposed continuations per launch).  The
 * sequence uses cache / state slot 0.
 *   tokens     dev int32[batch][n_tok]  t_0 (anchor) .. t_{n-1} (drafts), each in [0, vocab)
 *   positions  dev int32[batch]         position p of the anchor; cache rows p..p+n-1 are
 *                                       written, so p + n_tok <= max_ctx is required
 *   out_logits dev fp32[batch][n_tok][vocab]: row j is the next-token distribution after t_j,
 *              i.e. what n_tok successive decode steps would produce
 *   out_accept_len dev int32[batch]: a = 1 + m, m the largest j with t_i == argmax(row i-1)
 *              for all 1 <= i <= j (lowest index on argmax ties)
 *   out_next_token dev int32[batch]: argmax of row a-1
 *   out_expert_ids dev int32[n_layers][n_tok][top_k] or NULL (MoE only): experts chosen
 *              per layer and row, in descending router order
 * Delta-rule states are committed as they stand after token a-1 (the
 * per-token states pass through the workspace).  batch must be 1.  Out-of-
 * range tokens or positions are reported by md_get_device_status.  Models
 * with max_batch > 8 return MD_EUNSUPPORTED. */
md_status md_verify_step(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                         float* out_logits, int32_t* out_accept_len, int32_t* out_next_token,
                         int32_t* out_expert_ids, int32_t batch, int32_t n_tok, void* hip_stream);

/* Synchronises the model's last stream and reports the device error word:
 * MD_OK, or MD_EDEVICE with md_last_error() naming the cause (a sync wait
 * that exceeded its bound, an out-of-range token, position or page id).
 * Clears it. */
md_status md_get_device_status(md_model* m);

/* Profiling aid.  When dev_buf is non-NULL, every later step records
 * wall-clock stamps (hipDeviceAttributeWallClockRate ticks) into
 * dev_buf[wg * n_per_wg + i]: slot 2s is when workgroup wg finished the work
 * before sync point s, slot 2s+1 when its wait there ended, and the last
 * slot when the workgroup started; slots n_per_wg/2 + 8p + k hold phase p's
 * own stamps (k < 4, after its wait; k = 4 its work tables built, k = 5 its
 * wait started).  Stamps that do not fit are dropped.  dev_buf holds
 * md_grid_size(m) * n_per_wg uint64 values; NULL turns recording off. */
md_status md_set_trace(md_model* m, uint64_t* dev_buf, int32_t n_per_wg);

/* Number of workgroups (one per CU) a step launches. */
int32_t md_grid_size(const md_model* m);

/* Text of the calling thread's last error; valid until its next md_* call. */
const char* md_last_error(void);

/* Release a model handle (NULL: nothing).  Waits for the last stream a call
 * of this handle enqueued work on, so that every step, verify or copy of the
 * handle has finished when it returns and the caller may free the weights,
 * workspace and caches.  The caller's buffers are not freed. */
void md_free_model(md_model* m);

#ifdef __cplusplus
}
#endif
#endif /* MD_H */
