// Host side of libmd.so: the C ABI declared in md.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "md.h"
#include "md_model.h"

namespace md {
// the two builds of the kernel: up to 8 token rows (decode and verify) and
// up to 64 (decode)
hipError_t launch_megakernel(const Params& p, int grid, hipStream_t stream);
hipError_t megakernel_occupancy(int* blocks_per_cu);
hipError_t launch_multilaunch(const Params& p, const int* kinds, int grid, hipStream_t stream);
hipError_t launch_megakernel_w64(const Params& p, int grid, hipStream_t stream);
hipError_t megakernel_occupancy_w64(int* blocks_per_cu);
hipError_t launch_multilaunch_w64(const Params& p, const int* kinds, int grid, hipStream_t stream);
hipError_t launch_pack(const void* src, void* dst, int64_t rows, int64_t cols, hipStream_t stream);
size_t scratch_bytes();
hipError_t scratch_address(int dev, void** out);
hipError_t launch_fill_u32(void* dst, uint32_t v, uint32_t n_words, hipStream_t stream);
hipError_t launch_kv_copy(const Params& p, const int32_t* src, const int32_t* dst, int n, int src_slot, int dst_slot,
                          hipStream_t stream);
}  // namespace md

using namespace md;

namespace {

thread_local std::string g_err;

md_status fail(md_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

constexpr int MAXB_ = 8;          // token rows of the 8-row build (verify: n_tok)
constexpr int MAXB_W = 64;        // sequences of the 64-row build
constexpr int GMAX = 1024;        // largest grid the workspace is sized for
constexpr int CMAX = 256;         // largest number of KV chunks per (sequence, kv head)
constexpr int PHASES_PER_LAYER = 10;  // upper bound on sync points per layer

// The kernel build a model runs on, by its max_batch, and what follows from
// it: the token-row stride of the workspace's activation buffers and the
// words per sync point (the 64-row build's attention phase counts up to
// 64 x 8 (row, kv head) pairs in one).
bool wide_model(const md_config* c) { return c->max_batch > MAXB_; }
int row_stride(const md_config* c) { return wide_model(c) ? MAXB_W : MAXB_; }
int sp_words(const md_config* c) { return wide_model(c) ? 17 * 32 : 9 * 32; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Tensor {
  std::string name;
  int64_t rows, cols;
};

bool is_mla(const md_config* c, int l) { return c->attn_kind == 1 && (l % c->mla_every) == c->mla_every - 1; }

// The weight inventory, in the order the caller passes pointers.
std::vector<Tensor> inventory(const md_config* c) {
  std::vector<Tensor> T;
  auto mat = [&](std::string n, int64_t r, int64_t k) { T.push_back({n, r, k}); };
  int64_t H = c->hidden;
  mat("embed", c->vocab, H);
  for (int l = 0; l < c->n_layers; ++l) {
    std::string p = "L" + std::to_string(l) + ".";
    mat(p + "attn_norm", 1, H);
    if (c->attn_kind == 0) {
      mat(p + "wq", (int64_t)c->n_q_heads * c->head_dim, H);
      mat(p + "wk", (int64_t)c->n_kv_heads * c->head_dim, H);
      mat(p + "wv", (int64_t)c->n_kv_heads * c->head_dim, H);
      mat(p + "wo", H, (int64_t)c->n_q_heads * c->head_dim);
    } else if (is_mla(c, l)) {
      mat(p + "mla_wqa", c->q_lora, H);
      mat(p + "mla_q_norm", 1, c->q_lora);
      mat(p + "mla_wqb", (int64_t)c->mla_heads * (c->nope_dim + c->rope_dim), c->q_lora);
      mat(p + "mla_wkva", c->kv_lora + c->rope_dim, H);
      mat(p + "mla_kv_norm", 1, c->kv_lora);
      mat(p + "mla_wkvb", (int64_t)c->mla_heads * (c->nope_dim + c->v_dim), c->kv_lora);
      mat(p + "mla_wo", H, (int64_t)c->mla_heads * c->v_dim);
    } else {
      mat(p + "kda_wq", (int64_t)c->kda_heads * c->kda_dk, H);
      mat(p + "kda_wk", (int64_t)c->kda_heads * c->kda_dk, H);
      mat(p + "kda_wv", (int64_t)c->kda_heads * c->kda_dv, H);
      mat(p + "kda_walpha", c->kda_heads, H);
      mat(p + "kda_wbeta", c->kda_heads, H);
      mat(p + "kda_wo", H, (int64_t)c->kda_heads * c->kda_dv);
    }
    mat(p + "ffn_norm", 1, H);
    if (c->n_experts == 0) {
      mat(p + "w_gate", c->ffn_dim, H);
      mat(p + "w_up", c->ffn_dim, H);
      mat(p + "w_down", H, c->ffn_dim);
    } else {
      mat(p + "router", c->n_experts, H);
      for (int s = 0; s < c->n_shared; ++s) {
        std::string q = p + "sh" + std::to_string(s) + "_";
        mat(q + "gate", c->shared_ffn, H);
        mat(q + "up", c->shared_ffn, H);
        mat(q + "down", H, c->shared_ffn);
      }
      for (int e = 0; e < c->n_experts; ++e) {
        std::string q = p + "e" + std::to_string(e) + "_";
        mat(q + "gate", c->expert_ffn, H);
        mat(q + "up", c->expert_ffn, H);
        mat(q + "down", H, c->expert_ffn);
      }
    }
  }
  mat("final_norm", 1, H);
  mat("lm_head", c->vocab, H);
  return T;
}

md_status validate(const md_config* c) {
  if (!c) return fail(MD_EINVAL, "config is NULL");
  if (c->flags != 0) return fail(MD_EINVAL, "flags must be 0");
  if (c->n_layers < 1 || c->hidden < 32 || c->vocab < 1 || c->max_ctx < 1)
    return fail(MD_EINVAL, "n_layers, hidden, vocab and max_ctx must be positive");
  if (c->max_batch < 1 || c->max_batch > MAXB_W) return fail(MD_EINVAL, "max_batch must be in [1, %d]", MAXB_W);
  if (c->hidden % 32) return fail(MD_EUNSUPPORTED, "hidden must be a multiple of 32");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return fail(MD_EINVAL, "rms_eps and rope_theta must be > 0");
  if (c->attn_kind == 0) {
    if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads)
      return fail(MD_EINVAL, "n_q_heads must be a positive multiple of n_kv_heads");
    if (c->n_q_heads / c->n_kv_heads > 8) return fail(MD_EUNSUPPORTED, "at most 8 query heads per kv head");
    if (c->head_dim != 64 && c->head_dim != 128) return fail(MD_EUNSUPPORTED, "head_dim must be 64 or 128");
    if (c->max_ctx % 32) return fail(MD_EUNSUPPORTED, "max_ctx must be a multiple of 32 (V cache tiles)");
    // the attention phase counts the finished chunks of every (row, kv head)
    // in one word of a layer's sync point
    const int rs = row_stride(c), spw = sp_words(c);
    if (rs * c->n_kv_heads > spw)
      return fail(MD_EUNSUPPORTED, "at most %d kv heads (%d rows x kv heads must fit a sync point's %d words)",
                  spw / rs, rs, spw);
  } else if (c->attn_kind == 1) {
    if (c->mla_every < 1) return fail(MD_EINVAL, "mla_every must be >= 1");
    bool has_mla = c->n_layers >= c->mla_every, has_kda = c->mla_every > 1;
    if (has_mla) {
      if (c->mla_heads < 1 || c->mla_heads > 32) return fail(MD_EUNSUPPORTED, "mla_heads must be in [1, 32]");
      if (c->kv_lora != 512 || c->rope_dim != 64) return fail(MD_EUNSUPPORTED, "MLA needs kv_lora 512 and rope_dim 64");
      if (c->nope_dim < 16 || c->nope_dim > 128 || c->nope_dim % 16)
        return fail(MD_EUNSUPPORTED, "nope_dim must be a multiple of 16 in [16, 128]");
      if (c->v_dim < 32 || c->v_dim % 32) return fail(MD_EUNSUPPORTED, "v_dim must be a positive multiple of 32");
      if (c->q_lora < 128 || c->q_lora % 32) return fail(MD_EUNSUPPORTED, "q_lora must be a multiple of 32, at least 128");
      if (c->mla_heads * c->v_dim < 128) return fail(MD_EUNSUPPORTED, "mla_heads * v_dim must be at least 128");
    }
    if (has_kda) {
      if (c->kda_heads < 1) return fail(MD_EINVAL, "kda_heads must be positive");
      if (c->kda_dk < 1 || c->kda_dk > 128) return fail(MD_EUNSUPPORTED, "kda_dk must be in [1, 128]");
      if (c->kda_dv < 32 || c->kda_dv % 32) return fail(MD_EUNSUPPORTED, "kda_dv must be a positive multiple of 32");
      if (c->kda_heads * c->kda_dv < 128) return fail(MD_EUNSUPPORTED, "kda_heads * kda_dv must be at least 128");
      if (c->kda_qk_l2norm != 0 && c->kda_qk_l2norm != 1) return fail(MD_EINVAL, "kda_qk_l2norm must be 0 or 1");
    }
  } else {
    return fail(MD_EINVAL, "attn_kind must be 0 or 1");
  }
  if (c->kv_page != 0) {
    if (c->kv_page < 32 || (c->kv_page & (c->kv_page - 1)))
      return fail(MD_EINVAL, "kv_page must be 0 (contiguous caches) or a power of two >= 32");
    if (c->max_ctx % c->kv_page) return fail(MD_EINVAL, "max_ctx must be a multiple of kv_page");
    if (c->kv_pages < 1) return fail(MD_EINVAL, "a paged cache needs kv_pages >= 1");
  } else if (c->kv_pages != 0) {
    return fail(MD_EINVAL, "kv_pages must be 0 when kv_page is 0");
  }
  {
    // an MLA layer's cache is read through one buffer resource (32-bit range)
    const int64_t rows = c->kv_page ? (int64_t)c->kv_pages * c->kv_page : (int64_t)c->max_batch * c->max_ctx;
    if (c->attn_kind == 1 && rows * (c->kv_lora + c->rope_dim) * 2 >= ((int64_t)1 << 32))
      return fail(MD_EUNSUPPORTED, "an MLA layer's cache must stay below 4 GiB");
  }
  if (c->hidden < 128) return fail(MD_EUNSUPPORTED, "hidden must be at least 128");
  if (c->attn_kind == 0 && c->n_q_heads * c->head_dim < 128)
    return fail(MD_EUNSUPPORTED, "n_q_heads * head_dim must be at least 128");
  auto width_ok = [](int f) { return f >= 128 && f % 32 == 0; };
  if (c->n_experts == 0) {
    if (!width_ok(c->ffn_dim)) return fail(MD_EUNSUPPORTED, "ffn_dim must be a multiple of 32, at least 128");
  } else {
    if (c->n_experts < 1 || c->n_experts > 64) return fail(MD_EUNSUPPORTED, "n_experts must be in [1, 64]");
    if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts)
      return fail(MD_EINVAL, "top_k must be in [1, min(8, n_experts)]");
    if (!width_ok(c->expert_ffn)) return fail(MD_EUNSUPPORTED, "expert_ffn must be a multiple of 32, at least 128");
    if (c->n_shared < 0 || c->n_shared > 1) return fail(MD_EUNSUPPORTED, "n_shared must be 0 or 1");
    if (c->n_shared == 1 && !width_ok(c->shared_ffn))
      return fail(MD_EUNSUPPORTED, "shared_ffn must be a multiple of 32, at least 128");
    if (c->norm_topk != 0 && c->norm_topk != 1) return fail(MD_EINVAL, "norm_topk must be 0 or 1");
    const int rs = row_stride(c);
    int nu = c->n_experts < rs * c->top_k ? c->n_experts : rs * c->top_k;
    if (2 * nu > 72)
      return fail(MD_EUNSUPPORTED, "too many distinct experts per step (2 * min(n_experts, %d * top_k) > 72)", rs);
  }
  return MD_OK;
}

struct WsLayout {
  size_t layers, experts, x, u, ssq, qkv, attn, attn_ml, ou, h, rl, hs, hr, hr_stride, uq, ssq2, ckv, qm, qabs, mz, mml, mzc,
      kda, ring, cand, zero, rope, sync, err, total;
  size_t u_stride, ou_stride, h_stride, hs_stride, hr_lstride, uq_stride;  // one GEMV input buffer per use
  size_t ssq_stride, ssq2_stride;
  int rope_d;
  int n_sync, sync_attn_base;
};

// GQA key/value chunks per (row, kv head): enough tasks to cover the grid,
// at most one per 32-position tile of the cache.
int attn_chunks(const md_config* c, int grid, int rows) {
  const int pairs = rows * (c->n_kv_heads > 0 ? c->n_kv_heads : 1);
  int C = grid / pairs;
  const int tiles = (c->max_ctx + 31) / 32;
  if (C > tiles) C = tiles;
  if (C > CMAX) C = CMAX;
  return C < 1 ? 1 : C;
}

WsLayout ws_layout(const md_config* c) {
  WsLayout w{};
  size_t o = 0;
  const int64_t RS = row_stride(c);  // token rows of the activation buffers
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  int64_t H = c->hidden;
  int64_t nqkv = c->attn_kind == 0 ? (int64_t)(c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim : 0;
  int64_t attn_out = c->attn_kind == 0 ? (int64_t)c->n_q_heads * c->head_dim : 0;
  if (c->attn_kind == 1) {
    int64_t a = (int64_t)c->mla_heads * c->v_dim, b = (int64_t)c->kda_heads * c->kda_dv;
    attn_out = a > b ? a : b;
  }
  const bool hyb = c->attn_kind == 1;
  const int64_t mh = hyb ? (c->mla_heads > 0 ? c->mla_heads : 1) : 1;
  int64_t F = c->ffn_dim;
  if (c->expert_ffn > F) F = c->expert_ffn;
  if (c->shared_ffn > F) F = c->shared_ffn;
  w.layers = take(sizeof(LayerDesc) * (size_t)c->n_layers);
  w.experts = take(sizeof(void*) * 3 * (size_t)c->n_layers * (size_t)(c->n_experts > 0 ? c->n_experts : 1));
  w.x = take(4 * RS * H);
  const size_t L = (size_t)c->n_layers;
  w.u_stride = align256(2 * 2 * RS * H);
  w.u = take(w.u_stride * (2 * L + 1));
  w.ssq_stride = align256(4 * (size_t)GMAX * RS);
  w.ssq = take(w.ssq_stride * (2 * L + 1));
  w.qkv = take(4 * RS * (size_t)nqkv);
  w.attn = take(4 * (size_t)RS * (c->n_q_heads > 0 ? c->n_q_heads : 1) * CMAX * (size_t)c->head_dim);
  w.attn_ml = take(8 * (size_t)RS * (c->n_q_heads > 0 ? c->n_q_heads : 1) * CMAX);
  w.ou_stride = align256(2 * 2 * RS * (size_t)attn_out);
  w.ou = take(w.ou_stride * L);
  w.h_stride = align256(2 * 2 * RS * (size_t)F);
  w.h = take(w.h_stride * L);
  w.rl = take(8 * (size_t)RS * (c->n_experts > 0 ? c->n_experts : 1));
  w.hs_stride = align256(2 * 2 * RS * (size_t)(c->n_shared > 0 ? c->shared_ffn : 1));
  w.hs = take(w.hs_stride * L);
  int nu = c->n_experts < RS * c->top_k ? c->n_experts : RS * c->top_k;
  w.hr_stride = align256(2 * 2 * RS * (size_t)(c->expert_ffn > 0 ? c->expert_ffn : 1));
  w.hr_lstride = w.hr_stride * (size_t)(nu > 0 ? nu : 1);
  w.hr = take(w.hr_lstride * L);
  w.uq_stride = align256(2 * 2 * RS * (size_t)(hyb ? c->q_lora : 1));
  w.uq = take(w.uq_stride * L);
  w.ssq2_stride = align256(4 * (size_t)GMAX * RS);
  w.ssq2 = take(w.ssq2_stride * L);
  w.ckv = take(4 * RS * 576);
  w.qm = take(4 * RS * (size_t)mh * (hyb ? c->nope_dim + 64 : 1));
  w.qabs = take(4 * RS * (size_t)mh * 576);
  w.mz = take(hyb ? 4 * (size_t)GMAX * mh * 512 : 256);
  w.mml = take(8 * (size_t)GMAX * mh);
  w.kda = take(hyb ? 4 * RS * (size_t)(2 * c->kda_heads * c->kda_dk + c->kda_heads * c->kda_dv + 2 * c->kda_heads) : 256);
  int n_kda = 0;
  for (int l = 0; l < c->n_layers; ++l) n_kda += (hyb && !is_mla(c, l)) ? 1 : 0;
  // delta-rule snapshots of the verify step (8-row build only)
  w.ring = take((size_t)n_kda * (RS > 8 ? 0 : RS) * (hyb ? (size_t)c->kda_heads * c->kda_dk * c->kda_dv * 4 : 0));
  w.cand = take(8 * (size_t)GMAX * RS);
  w.zero = take(1024);
  w.rope_d = c->attn_kind == 0 ? c->head_dim : c->rope_dim;
  w.rope = take(sizeof(float) * 2 * (size_t)c->max_ctx * (size_t)(w.rope_d / 2));
  w.sync_attn_base = 1 + PHASES_PER_LAYER * c->n_layers + 2;
  w.n_sync = w.sync_attn_base + c->n_layers + 2;
  w.sync = take(4 * 2 * (size_t)w.n_sync * sp_words(c));
  w.err = take(256);
  w.mzc = take(hyb ? 4 * RS * (size_t)mh * 512 : 256);
  w.total = o;
  return w;
}

// Attention caches are n_pages pages of cap positions: one page per sequence
// slot (contiguous) or the configured pool (paged).
size_t kv_n_pages(const md_config* c) { return c->kv_page ? (size_t)c->kv_pages : (size_t)c->max_batch; }
size_t kv_page_cap(const md_config* c) { return c->kv_page ? (size_t)c->kv_page : (size_t)c->max_ctx; }

std::vector<size_t> kv_offsets(const md_config* c, size_t* total) {
  std::vector<size_t> off;
  size_t o = 0;
  const size_t np = kv_n_pages(c), cap = kv_page_cap(c);
  for (int l = 0; l < c->n_layers; ++l) {
    off.push_back(o);
    size_t n;
    if (c->attn_kind == 0)
      n = 2 * 2 * np * c->n_kv_heads * cap * c->head_dim;
    else if (is_mla(c, l))
      n = 2 * np * cap * (c->kv_lora + c->rope_dim);
    else
      n = 4 * (size_t)c->max_batch * c->kda_heads * c->kda_dk * c->kda_dv;
    o = align256(o + n);
  }
  if (total) *total = o;
  return off;
}

}  // namespace

struct md_model {
  md_config cfg;
  WsLayout lay;
  std::vector<const void*> weights;
  std::vector<size_t> kv_off;
  uint8_t* ws = nullptr;
  size_t ws_bytes = 0;
  int grid = 0;
  int bank = 0;
  uint32_t step_seq = 0;  // steps enqueued so far (tags the router logits of each step)
  hipStream_t last_stream = nullptr;
  std::vector<int> kinds;  // layer kinds (host copy of the layer table's)
  uint64_t* trace = nullptr;
  int trace_n = 0;
  int dev = 0;                  // the device the model lives on
  uint8_t* scratch = nullptr;   // that device's static scratch (md_decode_step_noalloc)
  hipError_t scratch_err = hipSuccess;
  int* last_err_word = nullptr; // error word of the last step (workspace or static scratch)
  bool wide = false;            // runs on the 64-row build (max_batch > 8)
};

// Whether the routed gate/up phase of a step of `rows` token rows streams
// every expert: when the tokens are expected to leave fewer than half an
// expert unchosen (uniform routing: E (1 - k/E)^rows < 0.5), streaming them
// all costs almost no bytes and lets the stream start before the routing is
// known.  Needs room for every expert in the routed hidden buffers and the
// phase's matrix table.
static int moe_all_experts(const md_config* c, int rows) {
  if (c->n_experts <= 0) return 0;
  const int E = c->n_experts, k = c->top_k;
  const int nu_max = E < row_stride(c) * k ? E : row_stride(c) * k;
  if (nu_max < E || 2 * E > 72) return 0;
  return (double)E * pow(1.0 - (double)k / (double)E, (double)rows) < 0.5 ? 1 : 0;
}

// One decode or verify step on the model's kernel build.
static hipError_t launch_step(const md_model* m, const Params& p, hipStream_t stream) {
  return m->wide ? launch_megakernel_w64(p, m->grid, stream) : launch_megakernel(p, m->grid, stream);
}

extern "C" {

const char* md_last_error(void) { return g_err.c_str(); }

size_t md_weight_count(const md_config* cfg) {
  if (!cfg || cfg->n_layers < 1) return 0;
  return inventory(cfg).size();
}

md_status md_weight_info(const md_config* cfg, size_t i, char* name, size_t name_cap, int64_t* rows, int64_t* cols) {
  if (!cfg) return fail(MD_EINVAL, "config is NULL");
  auto T = inventory(cfg);
  if (i >= T.size()) return fail(MD_EINVAL, "tensor index %zu out of range (%zu tensors)", i, T.size());
  if (name && name_cap) {
    strncpy(name, T[i].name.c_str(), name_cap - 1);
    name[name_cap - 1] = 0;
  }
  if (rows) *rows = T[i].rows;
  if (cols) *cols = T[i].cols;
  return MD_OK;
}

int32_t md_weight_layout(const md_config* cfg, size_t i) {
  if (!cfg) return -1;
  auto T = inventory(cfg);
  if (i >= T.size()) return -1;
  // the embedding table, the norm gains and the MLA up-projection (read by
  // the vector units along both of its axes) stay row-major
  const std::string& n = T[i].name;
  bool wkvb = n.size() >= 8 && n.compare(n.size() - 8, 8, "mla_wkvb") == 0;
  return (i == 0 || T[i].rows == 1 || wkvb) ? 0 : 1;
}

size_t md_workspace_bytes(const md_config* cfg) {
  if (validate(cfg) != MD_OK) return 0;
  return ws_layout(cfg).total;
}

size_t md_kv_bytes(const md_config* cfg, int32_t batch, int32_t ctx_cap) {
  if (validate(cfg) != MD_OK) return 0;
  if (batch < 1 || batch > MAXB_W || ctx_cap < 1) {
    fail(MD_EINVAL, "batch must be in [1, %d] and ctx_cap positive", MAXB_W);
    return 0;
  }
  md_config c = *cfg;
  c.max_batch = batch;
  c.max_ctx = ctx_cap;
  if (validate(&c) != MD_OK) return 0;
  size_t t = 0;
  kv_offsets(&c, &t);
  return t;
}

md_status md_init_model(const md_config* cfg, const void* const* weights, size_t n_weights, void* workspace,
                        size_t workspace_bytes, void* hip_stream, md_model** out) {
  if (!out) return fail(MD_EINVAL, "out is NULL");
  *out = nullptr;
  md_status st = validate(cfg);
  if (st != MD_OK) return st;
  auto T = inventory(cfg);
  if (!weights || n_weights != T.size())
    return fail(MD_EINVAL, "expected %zu weight pointers, got %zu", T.size(), n_weights);
  for (size_t i = 0; i < T.size(); ++i) {
    if (!weights[i]) return fail(MD_EINVAL, "weight %zu (%s) is NULL", i, T[i].name.c_str());
    if ((uintptr_t)weights[i] & 15) return fail(MD_EINVAL, "weight %zu (%s) is not 16-byte aligned", i, T[i].name.c_str());
    if (md_weight_layout(cfg, i) == 1 && (T[i].cols % 32 || md_packed_bytes(T[i].rows, T[i].cols) > 0xFFFFFFF0ull))
      return fail(MD_EUNSUPPORTED, "weight %s: columns must be a multiple of 32 and the packed size under 4 GiB",
                  T[i].name.c_str());
  }
  WsLayout lay = ws_layout(cfg);
  if (!workspace || ((uintptr_t)workspace & 255)) return fail(MD_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < lay.total) return fail(MD_ENOMEM, "workspace needs %zu bytes, got %zu", lay.total, workspace_bytes);
  if (lay.total > 0xFFFFFF00ull) return fail(MD_EUNSUPPORTED, "workspace exceeds 4 GiB");
  // device checks
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MD_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(MD_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MD_EUNSUPPORTED, "device is %s; the kernels are built for gfx950", prop.gcnArchName);
  if (!prop.cooperativeLaunch) return fail(MD_EUNSUPPORTED, "device lacks cooperative launch");
  int per_cu = 0;
  e = wide_model(cfg) ? megakernel_occupancy_w64(&per_cu) : megakernel_occupancy(&per_cu);
  if (e != hipSuccess) return fail(MD_EHIP, "occupancy query: %s", hipGetErrorString(e));
  if (per_cu < 1) return fail(MD_EUNSUPPORTED, "megakernel does not fit on a CU");
  int grid = prop.multiProcessorCount;
  if (grid > GMAX) grid = GMAX;

  md_model* m = new md_model();
  m->cfg = *cfg;
  m->lay = lay;
  m->weights.assign(weights, weights + n_weights);
  m->kv_off = kv_offsets(cfg, nullptr);
  m->ws = (uint8_t*)workspace;
  m->ws_bytes = workspace_bytes;
  m->grid = grid;
  m->wide = wide_model(cfg);

  // layer table
  std::vector<LayerDesc> L(cfg->n_layers);
  std::vector<const void*> ex;
  size_t wi = 1;  // after embed
  auto W = [&]() { return (const uint16_t*)weights[wi++]; };
  int kda_count = 0;
  for (int l = 0; l < cfg->n_layers; ++l) {
    LayerDesc& d = L[l];
    memset(&d, 0, sizeof d);
    d.kda_idx = -1;
    d.kv_off = m->kv_off[l];
    d.attn_norm = W();
    if (cfg->attn_kind == 0) {
      d.kind = LK_GQA;
      d.wq = W(); d.wk = W(); d.wv = W(); d.wo = W();
    } else if (is_mla(cfg, l)) {
      d.kind = LK_MLA;
      d.mla_wqa = W(); d.mla_qnorm = W(); d.mla_wqb = W(); d.mla_wkva = W(); d.mla_kvnorm = W();
      d.mla_wkvb = W(); d.mla_wo = W();
    } else {
      d.kind = LK_KDA;
      d.kda_idx = kda_count++;
      d.kda_wq = W(); d.kda_wk = W(); d.kda_wv = W(); d.kda_wa = W(); d.kda_wb = W(); d.kda_wo = W();
    }
    d.ffn_norm = W();
    if (cfg->n_experts == 0) {
      d.w_gate = W(); d.w_up = W(); d.w_down = W();
    } else {
      d.router = W();
      if (cfg->n_shared > 0) { d.sh_gate = W(); d.sh_up = W(); d.sh_down = W(); }
      for (int s = 1; s < cfg->n_shared; ++s) { W(); W(); W(); }
      d.experts = (const uint16_t* const*)(m->ws + lay.experts) + (size_t)l * cfg->n_experts * 3;
      for (int x = 0; x < cfg->n_experts * 3; ++x) ex.push_back(weights[wi++]);
    }
  }
  // rotary table: angle pos * theta^(-2i/d) in fp64, cos and sin rounded to fp32
  std::vector<float> rope((size_t)cfg->max_ctx * (lay.rope_d / 2) * 2);
  for (int pos = 0; pos < cfg->max_ctx; ++pos)
    for (int i = 0; i < lay.rope_d / 2; ++i) {
      double a = (double)pos * pow((double)cfg->rope_theta, -2.0 * i / (double)lay.rope_d);
      rope[((size_t)pos * (lay.rope_d / 2) + i) * 2] = (float)cos(a);
      rope[((size_t)pos * (lay.rope_d / 2) + i) * 2 + 1] = (float)sin(a);
    }
  hipStream_t s = (hipStream_t)hip_stream;
  e = hipMemcpyAsync(m->ws + lay.layers, L.data(), sizeof(LayerDesc) * L.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(m->ws + lay.rope, rope.data(), sizeof(float) * rope.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !ex.empty())
    e = hipMemcpyAsync(m->ws + lay.experts, ex.data(), sizeof(void*) * ex.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemsetAsync(m->ws + lay.sync, 0, lay.err + 256 - lay.sync, s);
  if (e == hipSuccess) e = hipMemsetAsync(m->ws + lay.zero, 0, 1024, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete m;
    return fail(MD_EHIP, "uploading the layer table: %s", hipGetErrorString(e));
  }
  m->kinds.resize(cfg->n_layers);
  for (int l = 0; l < cfg->n_layers; ++l) m->kinds[l] = L[l].kind;
  // the static scratch of the allocation-free step: its address on this
  // device, taken here at set-up with the device current
  m->dev = dev;
  void* sp = nullptr;
  m->scratch_err = scratch_address(dev, &sp);
  m->scratch = (uint8_t*)sp;
  m->last_err_word = (int*)(m->ws + lay.err);
  *out = m;
  return MD_OK;
}

// The kernel parameters of one step.  block_table: the step's page map (paged
// caches only: a paged model needs one, a contiguous model takes none).
static md_status fill_params(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv,
                             float* out_logits, int32_t batch, int32_t* out_tokens, int32_t* out_ids, Params& p,
                             const int32_t* block_table = nullptr) {
  if (!m) return fail(MD_EINVAL, "model is NULL");
  const md_config* c = &m->cfg;
  if (batch < 1 || batch > c->max_batch) return fail(MD_EINVAL, "batch %d outside [1, %d]", batch, c->max_batch);
  if (!tokens || !positions || !kv || !out_logits) return fail(MD_EINVAL, "tokens, positions, kv_cache and out_logits must be non-NULL");
  if (((uintptr_t)kv & 255) || ((uintptr_t)out_logits & 3) || ((uintptr_t)tokens & 3) || ((uintptr_t)positions & 3))
    return fail(MD_EINVAL, "misaligned pointer (kv_cache needs 256-byte alignment)");
  if (c->kv_page && !block_table)
    return fail(MD_EINVAL, "the model's caches are paged (kv_page %d): use the _paged step with a block table", c->kv_page);
  if (!c->kv_page && block_table) return fail(MD_EINVAL, "a block table needs a paged model (kv_page > 0)");
  if ((uintptr_t)block_table & 3) return fail(MD_EINVAL, "misaligned block table");
  memset(&p, 0, sizeof p);
  p.bt = block_table;
  p.n_pages = (int)kv_n_pages(c);
  p.pg_cap = (int)kv_page_cap(c);
  p.bt_stride = c->kv_page ? c->max_ctx / c->kv_page : 0;
  p.pg_shift = 0;
  while (c->kv_page && (1 << p.pg_shift) < c->kv_page) ++p.pg_shift;
  p.ml_phase = -1;
  const WsLayout& w = m->lay;
  p.layers = (const LayerDesc*)(m->ws + w.layers);
  p.embed = (const uint16_t*)m->weights.front();
  p.final_norm = (const uint16_t*)m->weights[m->weights.size() - 2];
  p.lm_head = (const uint16_t*)m->weights.back();
  p.n_layers = c->n_layers; p.H = c->hidden; p.V = c->vocab; p.max_batch = c->max_batch; p.max_ctx = c->max_ctx;
  p.eps = c->rms_eps; p.theta = c->rope_theta;
  p.nq = c->n_q_heads; p.nkv = c->n_kv_heads; p.hd = c->head_dim;
  p.ffn = c->ffn_dim;
  p.n_experts = c->n_experts; p.top_k = c->top_k; p.expert_ffn = c->expert_ffn; p.n_shared = c->n_shared;
  p.shared_ffn = c->shared_ffn; p.norm_topk = c->norm_topk;
  p.B = batch;
  p.moe_all = moe_all_experts(c, batch);
  p.attn_chunks = attn_chunks(c, m->grid, batch);
  p.tokens = tokens; p.positions = positions; p.kv = (uint8_t*)kv; p.logits = out_logits;
  p.out_tokens = out_tokens; p.out_ids = out_ids;
  p.ws = m->ws; p.ws_bytes = (uint32_t)w.total;
  p.x = (float*)(m->ws + w.x);
  p.u_stride = (uint32_t)w.u_stride; p.ou_stride = (uint32_t)w.ou_stride; p.h_stride = (uint32_t)w.h_stride;
  p.hs_stride = (uint32_t)w.hs_stride; p.hr_lstride = (uint32_t)w.hr_lstride; p.uq_stride = (uint32_t)w.uq_stride;
  p.ssq_stride = (uint32_t)w.ssq_stride; p.ssq2_stride = (uint32_t)w.ssq2_stride;
  p.off_u = (uint32_t)w.u; p.off_ssq = (uint32_t)w.ssq; p.off_qkv = (uint32_t)w.qkv; p.off_attn = (uint32_t)w.attn; p.off_attn_ml = (uint32_t)w.attn_ml;
  p.off_ou = (uint32_t)w.ou; p.off_h = (uint32_t)w.h;
  p.mla_h = c->mla_heads; p.q_lora = c->q_lora; p.nope = c->nope_dim; p.vdim = c->v_dim;
  p.kda_h = c->kda_heads; p.kda_dk = c->kda_dk; p.kda_dv = c->kda_dv; p.kda_l2 = c->kda_qk_l2norm;
  {
    int cm = m->grid / batch;
    int by_ctx = (c->max_ctx + 31) / 32;
    if (cm > by_ctx) cm = by_ctx;
    if (cm > CMAX) cm = CMAX;
    if (cm < 1) cm = 1;
    p.mla_chunks = cm;
  }
  p.off_uq = (uint32_t)w.uq; p.off_ssq2 = (uint32_t)w.ssq2; p.off_ckv = (uint32_t)w.ckv; p.off_qm = (uint32_t)w.qm;
  p.off_qabs = (uint32_t)w.qabs; p.off_mz = (uint32_t)w.mz; p.off_mml = (uint32_t)w.mml; p.off_mzc = (uint32_t)w.mzc; p.off_kda = (uint32_t)w.kda;
  p.n_kda = 0;
  for (int l = 0; l < c->n_layers; ++l) p.n_kda += (c->attn_kind == 1 && !is_mla(c, l)) ? 1 : 0;
  p.kda_ring = m->ws + w.ring;
  p.off_rl = (uint32_t)w.rl; p.off_hs = (uint32_t)w.hs; p.off_hr = (uint32_t)w.hr; p.hr_stride = (uint32_t)w.hr_stride; p.off_cand = (uint32_t)w.cand; p.off_zero = (uint32_t)w.zero;
  p.rope = (const float*)(m->ws + w.rope); p.rope_d = w.rope_d;
  p.sync = (unsigned*)(m->ws + w.sync);
  p.err = (int*)(m->ws + w.err);
  p.n_sync = w.n_sync;
  p.sync_attn_base = w.sync_attn_base;
  p.spin_limit = 1u << 22;
  p.trace = m->trace;
  p.trace_n = m->trace_n;
  p.step_seq = m->step_seq++;
  return MD_OK;
}

md_status md_decode_step(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                         float* out_logits, int32_t batch, int32_t* out_tokens, int32_t* out_expert_ids,
                         void* hip_stream) {
  Params p;
  md_status st = fill_params(m, tokens, positions, kv_cache, out_logits, batch, out_tokens, out_expert_ids, p);
  if (st != MD_OK) return st;
  p.bank = m->bank;
  hipError_t e = launch_step(m, p, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(MD_EHIP, "megakernel launch: %s", hipGetErrorString(e));
  m->bank ^= 1;
  m->last_stream = (hipStream_t)hip_stream;
  m->last_err_word = p.err;
  return MD_OK;
}

md_status md_decode_step_noalloc(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                                 float* out_logits, int32_t batch, int32_t* out_tokens, int32_t* out_expert_ids,
                                 void* hip_stream) {
  Params p;
  md_status st = fill_params(m, tokens, positions, kv_cache, out_logits, batch, out_tokens, out_expert_ids, p);
  if (st != MD_OK) return st;
  if (m->scratch_err != hipSuccess || !m->scratch)
    return fail(MD_EHIP, "the static scratch's device address is unavailable: %s", hipGetErrorString(m->scratch_err));
  const WsLayout& w = m->lay;
  if (w.total > scratch_bytes())
    return fail(MD_ENOMEM, "this model's step needs %zu bytes of scratch; the static scratch holds %zu "
                "(use md_decode_step with the model's workspace)", w.total, scratch_bytes());
  // Per-step buffers from the static scratch, at the workspace layout's own
  // offsets; the layer table, expert pointers and rotary table stay in the
  // model's workspace (written once at md_init_model).
  uint8_t* s = m->scratch;
  p.ws = s;
  p.x = (float*)(s + w.x);
  p.sync = (unsigned*)(s + w.sync);
  p.err = (int*)(s + w.err);
  p.kda_ring = s + w.ring;
  p.bank = 0;
  // The scratch keeps whatever the last call on this device left: clear the
  // counters this step uses, its error word and the zero line.
  hipStream_t stream = (hipStream_t)hip_stream;
  hipError_t e = launch_fill_u32(s + w.sync, 0u, (uint32_t)((size_t)w.n_sync * sp_words(&m->cfg)), stream);
  if (e == hipSuccess) e = launch_fill_u32(s + w.err, 0u, 1u, stream);
  if (e == hipSuccess) e = launch_fill_u32(s + w.zero, 0u, 1024u / 4u, stream);
  // router logits carry the step's tag; another model's entries could match it
  if (e == hipSuccess && m->cfg.n_experts > 0)
    e = launch_fill_u32(s + w.rl, 0u, (uint32_t)(2 * (size_t)row_stride(&m->cfg) * m->cfg.n_experts), stream);
  if (e != hipSuccess) return fail(MD_EHIP, "clearing the static scratch: %s", hipGetErrorString(e));
  e = launch_step(m, p, stream);
  if (e != hipSuccess) return fail(MD_EHIP, "megakernel launch: %s", hipGetErrorString(e));
  m->last_stream = stream;
  m->last_err_word = p.err;
  return MD_OK;
}

md_status md_decode_step_multilaunch(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                                     float* out_logits, int32_t batch, int32_t* out_tokens, int32_t* out_expert_ids,
                                     void* hip_stream) {
  Params p;
  md_status st = fill_params(m, tokens, positions, kv_cache, out_logits, batch, out_tokens, out_expert_ids, p);
  if (st != MD_OK) return st;
  p.bank = m->bank;
  hipError_t e = m->wide ? launch_multilaunch_w64(p, m->kinds.data(), m->grid, (hipStream_t)hip_stream)
                          : launch_multilaunch(p, m->kinds.data(), m->grid, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(MD_EHIP, "phase launch: %s", hipGetErrorString(e));
  m->bank ^= 1;
  m->last_stream = (hipStream_t)hip_stream;
  m->last_err_word = p.err;
  return MD_OK;
}

static md_status verify_step(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                             const int32_t* block_table, float* out_logits, int32_t* out_accept_len,
                             int32_t* out_next_token, int32_t* out_expert_ids, int32_t batch, int32_t n_tok,
                             void* hip_stream) {
  if (m && m->wide)
    return fail(MD_EUNSUPPORTED, "verify runs on models with max_batch <= %d (this one has %d)", MAXB_, m->cfg.max_batch);
  if (batch != 1) return fail(MD_EUNSUPPORTED, "verify runs one sequence per launch (batch must be 1)");
  if (n_tok < 2 || n_tok > MAXB_) return fail(MD_EINVAL, "n_tok %d outside [2, %d]", n_tok, MAXB_);
  if (!out_accept_len || !out_next_token) return fail(MD_EINVAL, "out_accept_len and out_next_token must be non-NULL");
  if (((uintptr_t)out_accept_len & 3) || ((uintptr_t)out_next_token & 3)) return fail(MD_EINVAL, "misaligned pointer");
  Params p;
  // the n_tok rows of the one sequence travel as the step's token rows
  md_status st = fill_params(m, tokens, positions, kv_cache, out_logits, 1, nullptr, out_expert_ids, p, block_table);
  if (st != MD_OK) return st;
  const md_config* c = &m->cfg;
  p.B = n_tok;
  p.moe_all = moe_all_experts(c, n_tok);
  p.verify = 1;
  p.out_accept = out_accept_len;
  p.out_next = out_next_token;
  {
    p.attn_chunks = attn_chunks(c, m->grid, n_tok);
    int cm = m->grid / n_tok;
    int by_ctx = (c->max_ctx + 31) / 32;
    if (cm > by_ctx) cm = by_ctx;
    p.mla_chunks = cm < 1 ? 1 : (cm > CMAX ? CMAX : cm);
  }
  p.bank = m->bank;
  hipError_t e = launch_step(m, p, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(MD_EHIP, "megakernel launch: %s", hipGetErrorString(e));
  m->bank ^= 1;
  m->last_stream = (hipStream_t)hip_stream;
  m->last_err_word = p.err;
  return MD_OK;
}

md_status md_verify_step(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                         float* out_logits, int32_t* out_accept_len, int32_t* out_next_token,
                         int32_t* out_expert_ids, int32_t batch, int32_t n_tok, void* hip_stream) {
  return verify_step(m, tokens, positions, kv_cache, nullptr, out_logits, out_accept_len, out_next_token,
                     out_expert_ids, batch, n_tok, hip_stream);
}

md_status md_decode_step_paged(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_pool,
                               const int32_t* block_table, float* out_logits, int32_t batch, int32_t* out_tokens,
                               int32_t* out_expert_ids, void* hip_stream) {
  if (!block_table) return fail(MD_EINVAL, "block_table must be non-NULL");
  Params p;
  md_status st = fill_params(m, tokens, positions, kv_pool, out_logits, batch, out_tokens, out_expert_ids, p,
                             block_table);
  if (st != MD_OK) return st;
  p.bank = m->bank;
  hipError_t e = launch_step(m, p, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(MD_EHIP, "megakernel launch: %s", hipGetErrorString(e));
  m->bank ^= 1;
  m->last_stream = (hipStream_t)hip_stream;
  m->last_err_word = p.err;
  return MD_OK;
}

md_status md_verify_step_paged(md_model* m, const int32_t* tokens, const int32_t* positions, void* kv_pool,
                               const int32_t* block_table, float* out_logits, int32_t* out_accept_len,
                               int32_t* out_next_token, int32_t* out_expert_ids, int32_t batch, int32_t n_tok,
                               void* hip_stream) {
  if (!block_table) return fail(MD_EINVAL, "block_table must be non-NULL");
  return verify_step(m, tokens, positions, kv_pool, block_table, out_logits, out_accept_len, out_next_token,
                     out_expert_ids, batch, n_tok, hip_stream);
}

// Parameters of a copy: the model's layer table and cache geometry only.
static md_status copy_params(md_model* m, void* kv, Params& p) {
  if (!m) return fail(MD_EINVAL, "model is NULL");
  if (!kv || ((uintptr_t)kv & 255)) return fail(MD_EINVAL, "kv must be non-NULL and 256-byte aligned");
  const md_config* c = &m->cfg;
  memset(&p, 0, sizeof p);
  p.layers = (const LayerDesc*)(m->ws + m->lay.layers);
  p.n_layers = c->n_layers;
  p.kv = (uint8_t*)kv;
  p.nkv = c->n_kv_heads;
  p.hd = c->head_dim;
  p.kda_h = c->kda_heads;
  p.kda_dk = c->kda_dk;
  p.kda_dv = c->kda_dv;
  p.n_pages = (int)kv_n_pages(c);
  p.pg_cap = (int)kv_page_cap(c);
  p.bt_stride = c->kv_page ? c->max_ctx / c->kv_page : 0;  // > 0: the caches are paged
  p.err = (int*)(m->ws + m->lay.err);
  return MD_OK;
}

md_status md_kv_copy_pages(md_model* m, void* kv_pool, const int32_t* src_pages, const int32_t* dst_pages,
                           int32_t n, void* hip_stream) {
  Params p;
  md_status st = copy_params(m, kv_pool, p);
  if (st != MD_OK) return st;
  if (!m->cfg.kv_page) return fail(MD_EINVAL, "page copies need a paged model (kv_page > 0)");
  if (n < 0) return fail(MD_EINVAL, "n must be >= 0");
  if (n > 0 && (!src_pages || !dst_pages)) return fail(MD_EINVAL, "src_pages and dst_pages must be non-NULL");
  if (((uintptr_t)src_pages & 3) || ((uintptr_t)dst_pages & 3)) return fail(MD_EINVAL, "misaligned page list");
  hipError_t e = launch_kv_copy(p, src_pages, dst_pages, n, 0, 0, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(MD_EHIP, "page copy launch: %s", hipGetErrorString(e));
  m->last_stream = (hipStream_t)hip_stream;
  m->last_err_word = p.err;
  return MD_OK;
}

md_status md_kv_copy_slot(md_model* m, void* kv, int32_t src_slot, int32_t dst_slot, void* hip_stream) {
  Params p;
  md_status st = copy_params(m, kv, p);
  if (st != MD_OK) return st;
  const int bm = m->cfg.max_batch;
  if (src_slot < 0 || src_slot >= bm || dst_slot < 0 || dst_slot >= bm)
    return fail(MD_EINVAL, "slots must be in [0, %d)", bm);
  if (src_slot == dst_slot) return MD_OK;
  hipError_t e = launch_kv_copy(p, nullptr, nullptr, 1, src_slot, dst_slot, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(MD_EHIP, "slot copy launch: %s", hipGetErrorString(e));
  m->last_stream = (hipStream_t)hip_stream;
  m->last_err_word = p.err;
  return MD_OK;
}

md_status md_get_device_status(md_model* m) {
  if (!m) return fail(MD_EINVAL, "model is NULL");
  hipError_t e = m->last_stream ? hipStreamSynchronize(m->last_stream) : hipDeviceSynchronize();
  if (e != hipSuccess) return fail(MD_EHIP, "synchronise: %s", hipGetErrorString(e));
  int err = 0;
  int* word = m->last_err_word ? m->last_err_word : (int*)(m->ws + m->lay.err);
  e = hipMemcpy(&err, word, sizeof err, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(MD_EHIP, "reading the device error word: %s", hipGetErrorString(e));
  if (err) {
    int zero = 0;
    // a failed step leaves its counter bank in an unknown state: clear both
    // (and the error word), so that the handle can run again (the static
    // scratch's counters are cleared by every allocation-free step itself)
    hipError_t c = hipMemcpy(word, &zero, sizeof zero, hipMemcpyHostToDevice);
    if (c == hipSuccess) c = hipMemset(m->ws + m->lay.sync, 0, (size_t)4 * 2 * m->lay.n_sync * sp_words(&m->cfg));
    if (c == hipSuccess) c = hipDeviceSynchronize();
    if (c != hipSuccess)
      return fail(MD_EHIP, "device error 0x%x, and resetting the error word and counters failed: %s", err,
                  hipGetErrorString(c));
    return fail(MD_EDEVICE, "device error 0x%x:%s%s%s%s%s", err, (err & MDE_WATCHDOG) ? " sync wait exceeded its bound" : "",
                (err & MDE_TOKEN) ? " token out of range" : "", (err & MDE_POSITION) ? " position out of range" : "",
                (err & MDE_CAPACITY) ? " a phase's work exceeds the per-workgroup tables (shape too large for this grid)" : "",
                (err & MDE_PAGE) ? " page id out of range" : "");
  }
  return MD_OK;
}

md_status md_set_trace(md_model* m, uint64_t* dev_buf, int32_t n_per_wg) {
  if (!m) return fail(MD_EINVAL, "model is NULL");
  if (dev_buf && n_per_wg < 2) return fail(MD_EINVAL, "n_per_wg must be >= 2");
  m->trace = dev_buf;
  m->trace_n = dev_buf ? n_per_wg : 0;
  return MD_OK;
}

int32_t md_grid_size(const md_model* m) { return m ? m->grid : 0; }

size_t md_packed_bytes(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 32 || cols % 32) return 0;
  return (size_t)((rows + 15) / 16) * (size_t)(cols / 32) * 1024;
}

md_status md_pack_weight(const void* src, void* dst, int64_t rows, int64_t cols, void* hip_stream) {
  if (!src || !dst) return fail(MD_EINVAL, "src and dst must be non-NULL");
  if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return fail(MD_EINVAL, "src and dst must be 16-byte aligned");
  if (rows < 1 || cols < 32 || cols % 32) return fail(MD_EINVAL, "cols must be a positive multiple of 32");
  if (md_packed_bytes(rows, cols) > 0xFFFFFFF0ull) return fail(MD_EUNSUPPORTED, "packed matrix exceeds 4 GiB");
  hipError_t e = launch_pack(src, dst, rows, cols, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(MD_EHIP, "pack kernel: %s", hipGetErrorString(e));
  return MD_OK;
}

void md_free_model(md_model* m) {
  if (!m) return;
  // nothing of this handle may still run on the device once it is gone
  if (m->last_stream) (void)hipStreamSynchronize(m->last_stream);
  delete m;
}

}  // extern "C"
