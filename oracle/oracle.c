/*
 * ORACLE -- test infrastructure only.
 *
 * A plain, slow, unfused CPU implementation of one decode step of the
 * megakernel's model, used to check the GPU path.  Only tests/, the smoke
 * entry and the benchmark's CPU-baseline leg may call it; the product path
 * never does.  It shares no code, header or table with the GPU library.
 *
 * Arithmetic: every activation, score and accumulator is a C double; bf16
 * weights and cache rows are widened exactly; the recurrent delta-rule state
 * is stored as fp32 between steps and widened on use; new cache rows are
 * rounded to bf16 (nearest-even) when written; logits are rounded to fp32
 * before the greedy argmax, and router logits are rounded to fp32 before the
 * top-k decision, so that integer decisions are taken on fp32 values exactly
 * as on the GPU.  Sums run in ascending index order.  OpenMP splits only
 * independent output elements; it never reorders a sum.
 *
 * What each function follows.  The pages (Inferact, "700 TPS on Kimi K3: A
 * Case for TPU Megakernels") name the blocks of a decode step -- attention
 * (KDA or MLA chosen by layer index), router, shared expert, routed experts,
 * attention residuals and RMSNorm, greedy decoding -- in sections "Our Kimi K3
 * megakernel" and "Results", but give no formulas.  The formulas below are the
 * standard definitions of those blocks, with the readings recorded in the
 * design notes (pre-norm residual blocks, rotate-half RoPE, softmax top-k with
 * renormalised weights, lowest-index tie-breaks, the gated delta rule
 * S <- a*S + b*k*(v - S^T k)^T with o = S^T q on L2-normalised q and k).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 */
double orc_bf16(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)b << 16;
  return (double)v.f;
}

/* Round a double to the nearest bf16 value (ties to even), directly from the
 * double so that no intermediate rounding to fp32 can double-round. */
uint16_t orc_to_bf16(double d) {
  if (d != d) return 0x7FC0;
  /* bf16 keeps 8 significant bits.  Scale to [2^7, 2^8), round the integer
   * part to nearest even, scale back. */
  if (d == 0.0) return signbit(d) ? 0x8000 : 0x0000;
  int e;
  double m = frexp(fabs(d), &e);     /* |d| = m * 2^e, m in [0.5, 1) */
  double q = ldexp(m, 8);            /* [128, 256) */
  double r = nearbyint(q);           /* default rounding mode: ties to even */
  double y = ldexp(r, e - 8);
  if (e - 1 < -126) {                /* below the fp32/bf16 normal range */
    /* subnormal bf16: quantum is 2^-133 */
    double qq = nearbyint(fabs(d) * ldexp(1.0, 133));
    y = ldexp(qq, -133);
  }
  float f = (float)y;                /* exact: y has <= 8 significant bits */
  if (d < 0) f = -f;
  union { float f; uint32_t u; } v = {f};
  return (uint16_t)(v.u >> 16);
}

/* -------------------------------------------------------------- building blocks */

/* RMSNorm: y_i = g_i * x_i / sqrt(mean(x^2) + eps). */
void orc_rmsnorm(int n, const double* x, const uint16_t* g, double eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) y[i] = orc_bf16(g[i]) * (x[i] * inv);
}

/* y = W x for a bf16 matrix W[rows][cols] (row-major, logical [out, in]). */
void orc_matvec(int64_t rows, int64_t cols, const uint16_t* W, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* w = W + r * cols;
    double acc = 0.0;
    for (int64_t c = 0; c < cols; ++c) acc += orc_bf16(w[c]) * x[c];
    y[r] = acc;
  }
}

/* Rotary embedding, rotate-half convention: element i < d/2 pairs with
 * i + d/2 and both turn by angle pos * theta^(-2i/d). */
void orc_rope(int d, double* v, int64_t pos, double theta) {
  int h = d / 2;
  for (int i = 0; i < h; ++i) {
    double ang = (double)pos * pow(theta, -2.0 * i / d);
    double c = cos(ang), s = sin(ang);
    double a = v[i], b = v[i + h];
    v[i] = a * c - b * s;
    v[i + h] = a * s + b * c;
  }
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }
double orc_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* In-place softmax with the maximum subtracted. */
void orc_softmax(int n, double* s) {
  double m = s[0];
  for (int i = 1; i < n; ++i) if (s[i] > m) m = s[i];
  double sum = 0.0;
  for (int i = 0; i < n; ++i) { s[i] = exp(s[i] - m); sum += s[i]; }
  for (int i = 0; i < n; ++i) s[i] /= sum;
}

/* ------------------------------------------------------------------ GQA block
 * One token of one sequence.  x[H] is the residual (updated in place).
 * kc, vc: this sequence's K and V cache of this layer, [nkv][cap][hd] bf16.
 * The new key and value are rounded to bf16 and stored at row `pos`; the
 * attention then reads rows 0..pos (including the new one) from the cache. */
int orc_gqa_block(int H, int nq, int nkv, int hd, double eps, double theta,
                  const uint16_t* g_norm, const uint16_t* wq, const uint16_t* wk,
                  const uint16_t* wv, const uint16_t* wo,
                  double* x, int64_t pos, uint16_t* kc, uint16_t* vc, int64_t cap) {
  if (pos < 0 || pos >= cap || nq % nkv) return -1;
  double* xn = malloc(sizeof(double) * H);
  double* q = malloc(sizeof(double) * nq * hd);
  double* k = malloc(sizeof(double) * nkv * hd);
  double* v = malloc(sizeof(double) * nkv * hd);
  double* o = malloc(sizeof(double) * nq * hd);
  double* a = malloc(sizeof(double) * H);
  double* s = malloc(sizeof(double) * (pos + 1));
  orc_rmsnorm(H, x, g_norm, eps, xn);
  orc_matvec(nq * hd, H, wq, xn, q);
  orc_matvec(nkv * hd, H, wk, xn, k);
  orc_matvec(nkv * hd, H, wv, xn, v);
  for (int h = 0; h < nq; ++h) orc_rope(hd, q + h * hd, pos, theta);
  for (int g = 0; g < nkv; ++g) orc_rope(hd, k + g * hd, pos, theta);
  for (int g = 0; g < nkv; ++g)
    for (int i = 0; i < hd; ++i) {
      kc[((int64_t)g * cap + pos) * hd + i] = orc_to_bf16(k[g * hd + i]);
      vc[((int64_t)g * cap + pos) * hd + i] = orc_to_bf16(v[g * hd + i]);
    }
  int group = nq / nkv;
  double scale = 1.0 / sqrt((double)hd);
  for (int h = 0; h < nq; ++h) {
    int g = h / group;
    for (int64_t t = 0; t <= pos; ++t) {
      const uint16_t* kr = kc + ((int64_t)g * cap + t) * hd;
      double d = 0.0;
      for (int i = 0; i < hd; ++i) d += q[h * hd + i] * orc_bf16(kr[i]);
      s[t] = d * scale;
    }
    orc_softmax((int)(pos + 1), s);
    for (int i = 0; i < hd; ++i) o[h * hd + i] = 0.0;
    for (int64_t t = 0; t <= pos; ++t) {
      const uint16_t* vr = vc + ((int64_t)g * cap + t) * hd;
      for (int i = 0; i < hd; ++i) o[h * hd + i] += s[t] * orc_bf16(vr[i]);
    }
  }
  orc_matvec(H, nq * hd, wo, o, a);
  for (int i = 0; i < H; ++i) x[i] += a[i];
  free(xn); free(q); free(k); free(v); free(o); free(a); free(s);
  return 0;
}

/* ------------------------------------------------------------------ MLA block
 * Multi-head latent attention in its plain (non-absorbed) form.
 *   c_q   = RMSNorm(W_qa xn; g_q)                       [q_lora]
 *   q_h   = (W_qb c_q)_h = [q_nope (nope) | q_pe (rope)], RoPE on q_pe
 *   [c | kpe] = W_kva xn;  c = RMSNorm(c; g_kv);  RoPE on kpe; cache row = bf16([c | kpe])
 *   for every cached row t:  k_{h,t} = [W_uk,h c_t | kpe_t],  v_{h,t} = W_uv,h c_t
 *   where W_kvb rows for head h are [uk: nope rows | uv: vdim rows]
 *   s_t = q_h . k_{h,t} / sqrt(nope + rope);  o_h = sum_t softmax(s)_t v_{h,t}
 *   x += W_o concat_h(o_h)
 * cache: this sequence's rows of this layer, [cap][kv_lora + rope] bf16. */
int orc_mla_block(int H, int nh, int q_lora, int kv_lora, int rope, int nope, int vdim,
                  double eps, double theta,
                  const uint16_t* g_norm, const uint16_t* wqa, const uint16_t* g_q,
                  const uint16_t* wqb, const uint16_t* wkva, const uint16_t* g_kv,
                  const uint16_t* wkvb, const uint16_t* wo,
                  double* x, int64_t pos, uint16_t* cache, int64_t cap) {
  if (pos < 0 || pos >= cap) return -1;
  int row = kv_lora + rope, qk = nope + rope;
  double* xn = malloc(sizeof(double) * H);
  double* cq0 = malloc(sizeof(double) * q_lora);
  double* cq = malloc(sizeof(double) * q_lora);
  double* q = malloc(sizeof(double) * nh * qk);
  double* ckv = malloc(sizeof(double) * row);
  double* cn = malloc(sizeof(double) * kv_lora);
  double* o = malloc(sizeof(double) * nh * vdim);
  double* a = malloc(sizeof(double) * H);
  orc_rmsnorm(H, x, g_norm, eps, xn);
  orc_matvec(q_lora, H, wqa, xn, cq0);
  orc_rmsnorm(q_lora, cq0, g_q, eps, cq);
  orc_matvec((int64_t)nh * qk, q_lora, wqb, cq, q);
  for (int h = 0; h < nh; ++h) orc_rope(rope, q + h * qk + nope, pos, theta);
  orc_matvec(row, H, wkva, xn, ckv);
  orc_rmsnorm(kv_lora, ckv, g_kv, eps, cn);
  orc_rope(rope, ckv + kv_lora, pos, theta);
  for (int i = 0; i < kv_lora; ++i) cache[pos * row + i] = orc_to_bf16(cn[i]);
  for (int i = 0; i < rope; ++i) cache[pos * row + kv_lora + i] = orc_to_bf16(ckv[kv_lora + i]);
  double scale = 1.0 / sqrt((double)qk);
  /* heads are independent: one head per OpenMP iteration, each with its own
   * scratch.  Per head, W_uk,h and W_uv,h are widened once and stored
   * column-major (wt[c][r]) so that all rows of k_t and v_t accumulate side
   * by side; every element is still the plain sum over c in ascending order. */
#pragma omp parallel for schedule(dynamic)
  for (int h = 0; h < nh; ++h) {
    double* ct = malloc(sizeof(double) * kv_lora);
    double* kt = malloc(sizeof(double) * nope);
    double* s = malloc(sizeof(double) * (pos + 1));
    double* vall = malloc(sizeof(double) * (pos + 1) * vdim);
    double* wukt = malloc(sizeof(double) * kv_lora * nope);
    double* wuvt = malloc(sizeof(double) * kv_lora * vdim);
    const uint16_t* wuk = wkvb + (int64_t)h * (nope + vdim) * kv_lora;
    const uint16_t* wuv = wuk + (int64_t)nope * kv_lora;
    for (int r = 0; r < nope; ++r)
      for (int c = 0; c < kv_lora; ++c) wukt[(int64_t)c * nope + r] = orc_bf16(wuk[(int64_t)r * kv_lora + c]);
    for (int r = 0; r < vdim; ++r)
      for (int c = 0; c < kv_lora; ++c) wuvt[(int64_t)c * vdim + r] = orc_bf16(wuv[(int64_t)r * kv_lora + c]);
    const double* qh = q + h * qk;
    for (int64_t t = 0; t <= pos; ++t) {
      for (int i = 0; i < kv_lora; ++i) ct[i] = orc_bf16(cache[t * row + i]);
      double* vt = vall + t * vdim;
      for (int r = 0; r < nope; ++r) kt[r] = 0.0;      /* k_nope = W_uk,h c_t */
      for (int r = 0; r < vdim; ++r) vt[r] = 0.0;      /* v = W_uv,h c_t */
      for (int c = 0; c < kv_lora; ++c) {
        const double cc = ct[c];
        const double* wk = wukt + (int64_t)c * nope;
        const double* wv = wuvt + (int64_t)c * vdim;
        for (int r = 0; r < nope; ++r) kt[r] += wk[r] * cc;
        for (int r = 0; r < vdim; ++r) vt[r] += wv[r] * cc;
      }
      double d = 0.0;
      for (int i = 0; i < nope; ++i) d += qh[i] * kt[i];
      for (int i = 0; i < rope; ++i) d += qh[nope + i] * orc_bf16(cache[t * row + kv_lora + i]);
      s[t] = d * scale;
    }
    orc_softmax((int)(pos + 1), s);
    for (int i = 0; i < vdim; ++i) {
      double acc = 0.0;
      for (int64_t t = 0; t <= pos; ++t) acc += s[t] * vall[t * vdim + i];
      o[h * vdim + i] = acc;
    }
    free(ct); free(kt); free(s); free(vall); free(wukt); free(wuvt);
  }
  orc_matvec(H, (int64_t)nh * vdim, wo, o, a);
  for (int i = 0; i < H; ++i) x[i] += a[i];
  free(xn); free(cq0); free(cq); free(q); free(ckv); free(cn); free(o); free(a);
  return 0;
}

/* ------------------------------------------------------------------ KDA block
 * Gated delta rule, per head h (state S_h is dk x dv, row-major, dv fastest):
 *   q, k, v = W_q xn, W_k xn, W_v xn;  alpha_h = sigmoid(w_alpha,h . xn);
 *   beta_h = sigmoid(w_beta,h . xn);  q, k L2-normalised per head when l2norm
 *   (divided by max(||.||, 1e-6));
 *   u = S^T k;  S <- alpha * S + beta * k (v - u)^T;  o = S^T q (new S)
 *   x += W_o concat_h(o_h)
 * state: this sequence's state of this layer, fp32 [nh][dk][dv], updated in place. */
int orc_kda_block(int H, int nh, int dk, int dv, int l2norm, double eps,
                  const uint16_t* g_norm, const uint16_t* wq, const uint16_t* wk,
                  const uint16_t* wv, const uint16_t* walpha, const uint16_t* wbeta,
                  const uint16_t* wo, double* x, float* state) {
  double* xn = malloc(sizeof(double) * H);
  double* q = malloc(sizeof(double) * nh * dk);
  double* k = malloc(sizeof(double) * nh * dk);
  double* v = malloc(sizeof(double) * nh * dv);
  double* al = malloc(sizeof(double) * nh);
  double* be = malloc(sizeof(double) * nh);
  double* S = malloc(sizeof(double) * dk * dv);
  double* u = malloc(sizeof(double) * dv);
  double* o = malloc(sizeof(double) * nh * dv);
  double* a = malloc(sizeof(double) * H);
  orc_rmsnorm(H, x, g_norm, eps, xn);
  orc_matvec((int64_t)nh * dk, H, wq, xn, q);
  orc_matvec((int64_t)nh * dk, H, wk, xn, k);
  orc_matvec((int64_t)nh * dv, H, wv, xn, v);
  orc_matvec(nh, H, walpha, xn, al);
  orc_matvec(nh, H, wbeta, xn, be);
  for (int h = 0; h < nh; ++h) {
    al[h] = orc_sigmoid(al[h]);
    be[h] = orc_sigmoid(be[h]);
    if (l2norm) {
      double nq2 = 0.0, nk2 = 0.0;
      for (int i = 0; i < dk; ++i) { nq2 += q[h * dk + i] * q[h * dk + i]; nk2 += k[h * dk + i] * k[h * dk + i]; }
      double dq = fmax(sqrt(nq2), 1e-6), dkk = fmax(sqrt(nk2), 1e-6);
      for (int i = 0; i < dk; ++i) { q[h * dk + i] /= dq; k[h * dk + i] /= dkk; }
    }
  }
  for (int h = 0; h < nh; ++h) {
    float* Sh = state + (int64_t)h * dk * dv;
    const double* kh = k + h * dk;
    const double* qh = q + h * dk;
    const double* vh = v + h * dv;
    for (int i = 0; i < dk * dv; ++i) S[i] = (double)Sh[i];
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * kh[i];
      u[j] = acc;
    }
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j)
        S[i * dv + j] = al[h] * S[i * dv + j] + be[h] * kh[i] * (vh[j] - u[j]);
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * qh[i];
      o[h * dv + j] = acc;
    }
    for (int i = 0; i < dk * dv; ++i) Sh[i] = (float)S[i];
  }
  orc_matvec(H, (int64_t)nh * dv, wo, o, a);
  for (int i = 0; i < H; ++i) x[i] += a[i];
  free(xn); free(q); free(k); free(v); free(al); free(be); free(S); free(u); free(o); free(a);
  return 0;
}

/* ------------------------------------------------------------------ FFN pieces */

/* acc += scale * W_d (silu(W_g xn) * (W_u xn))   (SwiGLU) */
void orc_swiglu_add(int H, int F, const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                    const double* xn, double scale, double* acc) {
  double* g = malloc(sizeof(double) * F);
  double* u = malloc(sizeof(double) * F);
  double* y = malloc(sizeof(double) * H);
  orc_matvec(F, H, wg, xn, g);
  orc_matvec(F, H, wu, xn, u);
  for (int i = 0; i < F; ++i) g[i] = orc_silu(g[i]) * u[i];
  orc_matvec(H, F, wd, g, y);
  for (int i = 0; i < H; ++i) acc[i] += scale * y[i];
  free(g); free(u); free(y);
}

/* Router: r = W_r xn, rounded to fp32; p = softmax(r);  the k experts with
 * the largest r (equal r: lower id first) are selected in that order; their
 * weights are p_e / sum_S p (norm_topk) or p_e.  ids[k] int32, w[k] double.
 * logits_out (nullable) receives the fp32 router logits. */
void orc_router(int H, int E, int k, int norm_topk, const uint16_t* wr, const double* xn,
                int32_t* ids, double* w, float* logits_out) {
  double* r = malloc(sizeof(double) * E);
  double* p = malloc(sizeof(double) * E);
  float* rf = malloc(sizeof(float) * E);
  char* taken = calloc(E, 1);
  orc_matvec(E, H, wr, xn, r);
  for (int e = 0; e < E; ++e) { rf[e] = (float)r[e]; p[e] = (double)rf[e]; }
  if (logits_out) memcpy(logits_out, rf, sizeof(float) * E);
  orc_softmax(E, p);
  double sel = 0.0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || rf[e] > rf[best]) best = e;   /* strict: equal keeps the lower id */
    }
    taken[best] = 1;
    ids[j] = best;
    w[j] = p[best];
    sel += p[best];
  }
  if (norm_topk)
    for (int j = 0; j < k; ++j) w[j] /= sel;
  free(r); free(p); free(rf); free(taken);
}

/* Final RMSNorm + LM head; logits rounded to fp32; greedy argmax over the
 * fp32 logits with the lowest index winning ties.  Returns the argmax. */
int32_t orc_head(int H, int64_t V, double eps, const uint16_t* g_final, const uint16_t* wlm,
                 const double* x, float* logits) {
  double* xn = malloc(sizeof(double) * H);
  double* l = malloc(sizeof(double) * V);
  orc_rmsnorm(H, x, g_final, eps, xn);
  orc_matvec(V, H, wlm, xn, l);
  int32_t best = 0;
  for (int64_t i = 0; i < V; ++i) {
    logits[i] = (float)l[i];
    if (logits[i] > logits[best]) best = (int32_t)i;
  }
  free(xn); free(l);
  return best;
}

/* Embedding: x = widen(E[tok]). */
void orc_embed(int H, const uint16_t* emb, int32_t tok, double* x) {
  for (int i = 0; i < H; ++i) x[i] = orc_bf16(emb[(int64_t)tok * H + i]);
}
