// The decode megakernel for gfx950 (MI355X) and the C ABI of libmd.so.
//
// One persistent cooperative launch runs a whole decode step: one workgroup
// per CU, each walking the same phase list; phases are separated by
// device-wide sync points (hierarchical counters, see md_sync.h).  This is the
// megakernel of Inferact, "700 TPS on Kimi K3: A Case for TPU Megakernels",
// section "Why megakernels?" (the decoder step inside one program, so no
// kernel boundary leaves the HBM interface idle) and section "Our Kimi K3
// megakernel" (the layer loop inside the kernel; attention kind by layer
// index; per layer attention, router, shared expert, routed experts).
//
// What differs from the pages' TPU design: the pages run one sequential
// program per TensorCore that stages weights into 64 MiB of VMEM with
// asynchronous DMAs.  Here 256 workgroups each stream a balanced share of
// every weight matrix straight from HBM into matrix-core operand registers
// with 16-byte buffer loads, several k-steps ahead of use.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "md.h"
#include "md_device.h"
#include "md_model.h"

namespace md {

// ===================================================================== sync
// One sync point = 8 sub-counters (one per workgroup class blockIdx % 8,
// which on this part is the XCD the workgroup runs on) and one top counter,
// each on its own 128-byte line.  A workgroup increments its sub-counter;
// the last arrival of a class increments the top counter; waiters poll the
// top counter.  Counters live in two banks used by alternate steps; every
// step clears the bank of the next step (nobody touches it during this step).
constexpr int SP_WORDS = 9 * 32;          // 9 lines of 128 B
constexpr int NGRP = 8;

__device__ __forceinline__ unsigned* sync_pt(const Params& p, int idx) {
  return p.sync + (size_t)p.bank * p.n_sync * SP_WORDS + (size_t)idx * SP_WORDS;
}

__device__ __forceinline__ bool dev_failed(const Params& p) {
  return __hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__device__ __forceinline__ void set_err(const Params& p, int code) {
  __hip_atomic_fetch_or(p.err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// every wave: make this wave's stores complete, then the workgroup arrives
// once.  Returns (in thread 0) whether this workgroup was the last to arrive.
__device__ bool arrive(const Params& p, int idx) {
  wait_stores();
  __builtin_amdgcn_s_barrier();
  bool last = false;
  if (threadIdx.x == 0) {
    unsigned* sp = sync_pt(p, idx);
    int grp = blockIdx.x & (NGRP - 1);
    int members = (gridDim.x - grp + NGRP - 1) / NGRP;
    unsigned ngrp = gridDim.x < NGRP ? gridDim.x : NGRP;
    unsigned old = __hip_atomic_fetch_add(sp + 32 * grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == (unsigned)members)
      last = __hip_atomic_fetch_add(sp + 32 * NGRP, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == ngrp;
  }
  return last;
}

// wait until every group has fully arrived at sync point idx
__device__ void wait_all(const Params& p, int idx) {
  if (threadIdx.x == 0) {
    unsigned* top = sync_pt(p, idx) + 32 * NGRP;
    unsigned ngrp = gridDim.x < NGRP ? gridDim.x : NGRP;
    unsigned spins = 0;
    while (__hip_atomic_load(top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < ngrp) {
      __builtin_amdgcn_s_sleep(1);
      if (((++spins) & 1023u) == 0 && (spins > p.spin_limit || dev_failed(p))) {
        set_err(p, MDE_WATCHDOG);
        break;
      }
    }
  }
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ void stamp(const Params& p, int slot) {
  if (p.trace && threadIdx.x == 0 && slot < p.trace_n) p.trace[(size_t)blockIdx.x * p.trace_n + slot] = wall_clock64();
}

// Sync point sidx: stamps 2*sidx (work done) and 2*sidx+1 (wait over).
__device__ __forceinline__ void grid_sync(const Params& p, int& sidx) {
  stamp(p, 2 * sidx);
  arrive(p, sidx);
  wait_all(p, sidx);
  stamp(p, 2 * sidx + 1);
  ++sidx;
}

// clear this WG's share of the other bank (used by the next step)
__device__ void clear_next_bank(const Params& p) {
  unsigned* nb = p.sync + (size_t)(p.bank ^ 1) * p.n_sync * SP_WORDS;
  size_t n = (size_t)p.n_sync * SP_WORDS;
  size_t per = (n + gridDim.x - 1) / gridDim.x;
  size_t a = per * blockIdx.x, e = a + per < n ? a + per : n;
  for (size_t i = a + threadIdx.x; i < e; i += NT) nb[i] = 0u;
}

// ===================================================================== GEMV
// Y[r][t] = sum_k W[r][k] * U[t][k] for this workgroup's rows of up to
// MAXM matrices that share K.  W is bf16 [N][K] row-major; U is the
// activation in "hi/lo" form: bf16[2][MAXB][K] (part, token, k) so that the
// matrix-core B operand (32 k x 16 columns: token t hi at column 2t, lo at
// 2t+1) is a single 16-byte load per lane.  Each workgroup owns rows
// [N*w/G, N*(w+1)/G) of every matrix; rows are cut into 16-row tiles whose
// tail rows fall outside the buffer resource and load as zero (no branch,
// no bandwidth).  The four waves split the k-steps; each keeps DS k-steps
// of weight and activation loads in flight.
constexpr int MAXM = 3;
constexpr int CMAX_DEV = 256;  // largest chunk count per (sequence, kv head)
constexpr int MAXT = 8;

struct GemvJob {
  const uint16_t* W[MAXM];
  int N[MAXM];
  int nm;
  int K;
  uint32_t u_off;  // byte offset of U in the workspace
  int B;
};

__device__ __forceinline__ const void* urs_base_dummy() { return nullptr; }

struct RowSplit {
  int r0, r1;
};
__device__ __forceinline__ RowSplit rows_of(int N, int w, int G) {
  RowSplit s;
  s.r0 = (int)((int64_t)N * w / G);
  s.r1 = (int)((int64_t)N * (w + 1) / G);
  return s;
}

// LDS layout used by the GEMV: per-wave partial tiles, then reduced Y.
struct GemvSmem {
  float red[NW][MAXT][16][16];
  float y[MAXT][16][MAXB];
};

// A planned GEMV: this workgroup's share of each matrix, cut into chunks of
// up to MAXT tiles (local tile indices [i0, i1) of every matrix).
struct GemvPlan {
  const void* wbase[MAXM];
  uint32_t wbytes[MAXM];
  int r0[MAXM], nrows[MAXM];
  int nm, K, B, per, maxtiles;
  uint32_t u_off;
};

__device__ __forceinline__ GemvPlan plan_gemv(const Params& p, const GemvJob& job) {
  GemvPlan g;
  const int G = gridDim.x, w = blockIdx.x;
  g.nm = job.nm;
  g.K = job.K;
  g.B = job.B;
  g.u_off = job.u_off;
  g.maxtiles = 0;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    if (m < job.nm) {
      RowSplit s = rows_of(job.N[m], w, G);
      g.r0[m] = s.r0;
      g.nrows[m] = s.r1 - s.r0;
      int nt = (g.nrows[m] + 15) >> 4;
      g.maxtiles = nt > g.maxtiles ? nt : g.maxtiles;
      g.wbase[m] = job.W[m] + (size_t)s.r0 * job.K;
      g.wbytes[m] = (uint32_t)((size_t)g.nrows[m] * job.K * 2);
    } else {
      g.r0[m] = 0;
      g.nrows[m] = 0;
      g.wbase[m] = p.ws;
      g.wbytes[m] = 0;
    }
  }
  g.per = MAXT / job.nm;
  return g;
}

// Sweep K for T tile slots; slot t is local tile i0 + t % per of matrix
// t / per (slots past the last matrix read nothing).
template <int T, int DS>
__device__ __forceinline__ void gemv_sweep(const GemvPlan& g, int i0, rsrc_t urs, GemvSmem& sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int K = g.K;
  const int ksteps = K >> 5;
  const int nks = (ksteps - wv + NW - 1) / NW;
  rsrc_t ars[T];
  uint32_t aoff[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int m = t / g.per, i = i0 + t % g.per;
    const void* wb = m == 0 ? g.wbase[0] : (m == 1 ? g.wbase[1] : g.wbase[2]);
    uint32_t nb = m == 0 ? g.wbytes[0] : (m == 1 ? g.wbytes[1] : g.wbytes[2]);
    if (m >= g.nm) nb = 0;
    ars[t] = make_rsrc_u(wb, nb);
    aoff[t] = ((uint32_t)(i * 16) + (lane & 15)) * (uint32_t)K * 2u + (lane >> 4) * 16u + wv * 64u;
  }
  const int n = lane & 15, tok = n >> 1, part = n & 1;
  const uint32_t boff = tok < g.B ? g.u_off + (uint32_t)((part * MAXB + tok) * K) * 2u + (lane >> 4) * 16u + wv * 64u : OOB;
  const uint32_t kstride = NW * 64u;
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  i32x4 ra[DS][T];
  i32x4 rb[DS];
#pragma unroll
  for (int d = 0; d < DS; ++d) {
    bool ok = d < nks;
    uint32_t ko = (uint32_t)d * kstride;
    rb[d] = ld_x4<CP_SC1>(urs, ok && boff != OOB ? boff + ko : OOB);
#pragma unroll
    for (int t = 0; t < T; ++t) ra[d][t] = ld_x4<CP_NT>(ars[t], ok ? aoff[t] + ko : OOB);
  }
  for (int base = 0; base < nks; base += DS) {
#pragma unroll
    for (int d = 0; d < DS; ++d) {
      bf16x8 bop = __builtin_bit_cast(bf16x8, rb[d]);
#pragma unroll
      for (int t = 0; t < T; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ra[d][t]), bop, acc[t], 0, 0, 0);
      int nx = base + d + DS;
      bool ok = nx < nks;
      uint32_t ko = (uint32_t)nx * kstride;
      rb[d] = ld_x4<CP_SC1>(urs, ok && boff != OOB ? boff + ko : OOB);
#pragma unroll
      for (int t = 0; t < T; ++t) ra[d][t] = ld_x4<CP_NT>(ars[t], ok ? aoff[t] + ko : OOB);
    }
  }
  // per-wave partial tiles -> LDS; lane holds rows 4*(lane/16)+i, column lane%16
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.red[wv][t][4 * (lane >> 4) + i][n] = acc[t][i];
  __syncthreads();
  // reduce the waves and merge hi/lo columns: y[t][row][tok]
  for (int e = threadIdx.x; e < T * 16 * MAXB; e += NT) {
    int t = e / (16 * MAXB), r = (e / MAXB) % 16, k = e % MAXB;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += sm.red[w][t][r][2 * k] + sm.red[w][t][r][2 * k + 1];
    sm.y[t][r][k] = s;
  }
  __syncthreads();
}

// One chunk of a planned GEMV; leaves Y in sm.y (slot m*per + local tile).
__device__ __noinline__ void gemv_chunk(const Params& p, const GemvPlan& g, int i0, GemvSmem& sm) {
  rsrc_t urs = make_rsrc_u(p.ws, p.ws_bytes);
  int i1 = i0 + g.per < g.maxtiles ? i0 + g.per : g.maxtiles;
  int cnt = (i1 - i0) * g.nm;
  GemvPlan gg = g;
  gg.per = i1 - i0;   // slots are packed: matrix m's tiles at m*(i1-i0)
  if (cnt <= 1) gemv_sweep<1, 16>(gg, i0, urs, sm);
  else if (cnt <= 2) gemv_sweep<2, 10>(gg, i0, urs, sm);
  else if (cnt <= 4) gemv_sweep<4, 6>(gg, i0, urs, sm);
  else gemv_sweep<8, 4>(gg, i0, urs, sm);
}

struct Chunk {
  int i0, i1, nm;
  int r0[MAXM], nrows[MAXM];
};

// Runs a GEMV over all of this WG's tiles; after each chunk `epi(sm, chunk)`
// consumes sm.y, where slot m*(i1-i0) + (i - i0) holds local tile i of matrix m.
template <class Epi>
__device__ __forceinline__ void run_gemv(const Params& p, const GemvJob& job, GemvSmem& sm, Epi&& epi) {
  GemvPlan g = plan_gemv(p, job);
  Chunk ch;
  ch.nm = g.nm;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) { ch.r0[m] = g.r0[m]; ch.nrows[m] = g.nrows[m]; }
  for (int i0 = 0; i0 < g.maxtiles; i0 += g.per) {
    ch.i0 = i0;
    ch.i1 = i0 + g.per < g.maxtiles ? i0 + g.per : g.maxtiles;
    gemv_chunk(p, g, i0, sm);
    epi(sm, ch);
    __syncthreads();
  }
}

// ===================================================================== phases

// inv_rms[t] from the per-WG partial sums of squares (fixed order: identical
// in every workgroup).  ssq: fp32[G][MAXB] at ws offset p.off_ssq.
__device__ __noinline__ void load_inv_rms(const Params& p, float* inv_rms, int n_feat) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
    for (int t = 0; t < p.B; ++t) {
      float s = 0.f;
      for (int g = lane; g < (int)gridDim.x; g += 64) s += ld_f32(r, p.off_ssq + (uint32_t)(g * MAXB + t) * 4u);
      s = wave_sum(s);
      if (lane == 0) inv_rms[t] = 1.0f / sqrtf(s / (float)n_feat + p.eps);
    }
  }
  __syncthreads();
}

// Write U[part][t][k] = hilo(v) for one element.
__device__ __forceinline__ void put_hilo(rsrc_t r, uint32_t u_off, int K, int t, int k, float v) {
  uint16_t hi, lo;
  split_hilo(v, hi, lo);
  st_u16(r, u_off + (uint32_t)((0 * MAXB + t) * K + k) * 2u, hi);
  st_u16(r, u_off + (uint32_t)((1 * MAXB + t) * K + k) * 2u, lo);
}

// Residual owner epilogue (shared by the O-projection, the dense down
// projection and the embedding): x[t][r] += y (or = y), then the next
// norm's input U = hilo(g[r] * x) and this WG's sum of squares of x.
struct SsqAcc {
  float v[MAXB];
};

// --- embedding: x[t] = E[tok_t] on this WG's hidden rows
__device__ __noinline__ void phase_embed(const Params& p, float* sm_f) {
  RowSplit s = rows_of(p.H, blockIdx.x, gridDim.x);
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  const uint16_t* g = p.layers[0].attn_norm;
  float* part = sm_f;  // [NT][MAXB]
  for (int t = 0; t < MAXB; ++t) part[threadIdx.x * MAXB + t] = 0.f;
  for (int e = threadIdx.x; e < (s.r1 - s.r0) * p.B; e += NT) {
    int t = e / (s.r1 - s.r0), i = s.r0 + e % (s.r1 - s.r0);
    int tok = p.tokens[t];
    if (tok < 0 || tok >= p.V) {
      set_err(p, MDE_TOKEN);
      tok = tok < 0 ? 0 : p.V - 1;
    }
    float x = bf16_f32(p.embed[(size_t)tok * p.H + i]);
    p.x[t * p.H + i] = x;
    put_hilo(r, p.off_u, p.H, t, i, bf16_f32(g[i]) * x);
    part[threadIdx.x * MAXB + t] += x * x;
  }
  __syncthreads();
  if (threadIdx.x < MAXB) {
    float a = 0.f;
    for (int i = 0; i < NT; ++i) a += part[i * MAXB + threadIdx.x];
    st_f32(r, p.off_ssq + (uint32_t)(blockIdx.x * MAXB + threadIdx.x) * 4u, a);
  }
}

// --- QKV projection (GQA): raw q, k, v (RMS-normalised input) -> qkv[t][row]
__device__ __noinline__ void phase_qkv(const Params& p, const LayerDesc& L, char* smem) {
  GemvSmem& sm = *(GemvSmem*)smem;
  float* inv = (float*)(smem + sizeof(GemvSmem));
  load_inv_rms(p, inv, p.H);
  GemvJob j;
  j.nm = 3;
  j.W[0] = L.wq; j.N[0] = p.nq * p.hd;
  j.W[1] = L.wk; j.N[1] = p.nkv * p.hd;
  j.W[2] = L.wv; j.N[2] = p.nkv * p.hd;
  j.K = p.H;
  j.u_off = p.off_u;
  j.B = p.B;
  const int nqkv = (p.nq + 2 * p.nkv) * p.hd;
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  run_gemv(p, j, sm, [&](GemvSmem& s, const Chunk& c) {
    int per = c.i1 - c.i0;
    int col0[3] = {0, p.nq * p.hd, (p.nq + p.nkv) * p.hd};
    for (int e = threadIdx.x; e < c.nm * per * 16 * p.B; e += NT) {
      int t = e % p.B, rr = (e / p.B) % 16, slot = e / (p.B * 16);
      int m = slot / per, i = c.i0 + slot % per;
      int lr = i * 16 + rr;
      if (lr >= c.nrows[m]) continue;
      float v = s.y[slot][rr][t] * inv[t];
      st_f32(r, p.off_qkv + (uint32_t)(t * nqkv + col0[m] + c.r0[m] + lr) * 4u, v);
    }
  });
}

// RoPE angle for pair index i of a head of dim d at position pos, from fp64.
__device__ __forceinline__ void rope_cs(int64_t pos, int i, int d, float theta, float& c, float& s) {
  double inv = pow((double)theta, -2.0 * (double)i / (double)d);
  double a = (double)pos * inv;
  double sd, cd;
  sincos(a, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// --- GQA decode attention.  Task (b, kv head g, chunk c) covers cached
// positions [c*P, (c+1)*P) of sequence b (positions 0..pos inclusive, the new
// row included).  Each wave takes a quarter of the chunk in 32-position
// blocks, with the next block's K and V rows in flight while the current one
// is used: scores on the matrix cores (K rows as the A operand, the group's
// rotated q heads as hi/lo B columns), an online softmax per head, and P.V on
// the vector ALUs.  The chunk's partial (max, sum, o) per head goes to the
// workspace; the last workgroup to finish a (b, g) combines the chunks.
struct AttnSmem {
  float q[MAXB][128];           // rotated, scaled q of the group's heads
  float s[NW][32][MAXB];        // per-wave scores / probabilities of a block
  float wm[NW][MAXB], wl[NW][MAXB];
  float wo[NW][MAXB][128];
  float cw[MAXB][CMAX_DEV];     // combine weights
  float cl[MAXB];
  int last;
};

template <int HD>
struct KVBlock {
  i32x4 k[2][HD / 32];          // 2 tiles of 16 positions x HD/32 k-steps
  i32x4 v[HD / 16];             // 32 positions x HD bf16 = HD/16 loads of 1 KB per wave
};

template <int HD>
__device__ __forceinline__ void load_block(KVBlock<HD>& r, rsrc_t krs, rsrc_t vrs, int blk, int w1, int lane) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    int prow = blk + tt * 16 + (lane & 15);
#pragma unroll
    for (int s = 0; s < HD / 32; ++s) {
      uint32_t off = (prow < w1 && blk < w1) ? (uint32_t)(prow * HD + s * 32 + (lane >> 4) * 8) * 2u : OOB;
      r.k[tt][s] = ld_x4<0>(krs, off);
    }
  }
  // V: lanes split a row into HD/8 chunks of 8 dims; one instruction covers 64/(HD/8) rows
  constexpr int LPR = HD / 8;
  constexpr int RPI = 64 / LPR;
#pragma unroll
  for (int q = 0; q < HD / 16; ++q) {
    int t = blk + q * RPI + lane / LPR;
    uint32_t off = (t < w1 && blk < w1) ? (uint32_t)(t * HD + (lane % LPR) * 8) * 2u : OOB;
    r.v[q] = ld_x4<0>(vrs, off);
  }
}

template <int HD>
__device__ __noinline__ void attn_task_wave(const Params& p, AttnSmem& sm, int gs, const uint16_t* kc,
                                            const uint16_t* vc, uint32_t nbytes, int w0, int w1) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const rsrc_t krs = make_rsrc_u(kc, nbytes), vrs = make_rsrc_u(vc, nbytes);
  gs = __builtin_amdgcn_readfirstlane(gs);
  w0 = __builtin_amdgcn_readfirstlane(w0);
  w1 = __builtin_amdgcn_readfirstlane(w1);
  const int nn = lane & 15, hh = nn >> 1, pp = nn & 1;
  constexpr int LPR = HD / 8, RPI = 64 / LPR;
  bf16x8 qb[HD / 32];
#pragma unroll
  for (int s = 0; s < HD / 32; ++s) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int d = s * 32 + (lane >> 4) * 8 + k;
      float v = hh < gs ? sm.q[hh][d] : 0.f;
      uint16_t hi, lo;
      split_hilo(v, hi, lo);
      qb[s][k] = __builtin_bit_cast(__bf16, pp ? lo : hi);
    }
  }
  float m_run[MAXB], l_run[MAXB], acc[MAXB][8];
#pragma unroll
  for (int h = 0; h < MAXB; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
  }
  auto block = [&](const KVBlock<HD>& cur, int blk) __attribute__((always_inline)) {
    // scores of the 32 positions
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < HD / 32; ++s)
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[tt][s]), qb[s], a, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = a[i] + __shfl_xor(a[i], 1, 64);
        int pr = tt * 16 + 4 * (lane >> 4) + i;
        if (!pp && hh < gs) sm.s[wv][pr][hh] = (blk + pr < w1) ? v : -INFINITY;
      }
    }
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_wave_barrier();
    // online softmax per head over this block; probabilities replace scores
#pragma unroll
    for (int h = 0; h < MAXB; ++h) {
      if (h < gs) {
        float sv = lane < 32 ? sm.s[wv][lane][h] : -INFINITY;
        float mb = wave_max(sv);
        float mn = fmaxf(m_run[h], mb);
        float corr = __expf(m_run[h] - mn);
        float pv = lane < 32 ? __expf(sv - mn) : 0.f;
        l_run[h] = l_run[h] * corr + wave_sum(pv);
        m_run[h] = mn;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] *= corr;
        if (lane < 32) sm.s[wv][lane][h] = pv;
      }
    }
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_wave_barrier();
    // P.V: this lane holds 8 dims of the rows q*RPI + lane/LPR
#pragma unroll
    for (int q = 0; q < HD / 16; ++q) {
      int t = q * RPI + lane / LPR;
      uint32_t u[4] = {(uint32_t)cur.v[q][0], (uint32_t)cur.v[q][1], (uint32_t)cur.v[q][2], (uint32_t)cur.v[q][3]};
      float vv[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vv[2 * j] = __uint_as_float(u[j] << 16);
        vv[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
      }
#pragma unroll
      for (int h = 0; h < MAXB; ++h) {
        if (h < gs) {
          float pw = sm.s[wv][t][h];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[h][j] += pw * vv[j];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  KVBlock<HD> ba, bb;
  load_block<HD>(ba, krs, vrs, w0, w1, lane);
  for (int blk = w0; blk < w1; blk += 64) {
    load_block<HD>(bb, krs, vrs, blk + 32, w1, lane);
    block(ba, blk);
    if (blk + 32 >= w1) break;
    load_block<HD>(ba, krs, vrs, blk + 64, w1, lane);
    block(bb, blk + 32);
  }
  // sum the lane groups that hold the same dims (different rows)
#pragma unroll
  for (int h = 0; h < MAXB; ++h) {
    if (h < gs) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[h][j];
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
        acc[h][j] = v;
      }
      if (lane == 0) { sm.wm[wv][h] = m_run[h]; sm.wl[wv][h] = l_run[h]; }
      if (lane < LPR) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.wo[wv][h][lane * 8 + j] = acc[h][j];
      }
    }
  }
}

__device__ __noinline__ void phase_attn_gqa(const Params& p, const LayerDesc& L, int layer, char* smem) {
  AttnSmem& sm = *(AttnSmem*)smem;
  const int wv = threadIdx.x >> 6;
  const int hd = p.hd, gs = p.nq / p.nkv, B = p.B;
  const int C = p.attn_chunks;
  const int ntask = B * p.nkv * C;
  const int nqkv = (p.nq + 2 * p.nkv) * hd;
  rsrc_t wr = make_rsrc_u(p.ws, p.ws_bytes);
  const float scale = 1.0f / sqrtf((float)hd);
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int c = task % C, g = (task / C) % p.nkv, b = task / (C * p.nkv);
    int pos = p.positions[b];
    if (pos < 0 || pos >= p.max_ctx) {
      set_err(p, MDE_POSITION);
      pos = pos < 0 ? 0 : p.max_ctx - 1;
    }
    const int n = pos + 1;
    const int P = (n + C - 1) / C;
    const int a0 = c * P < n ? c * P : n, a1 = (c + 1) * P < n ? (c + 1) * P : n;
    uint16_t* kc = (uint16_t*)(p.kv + L.kv_off) + (size_t)(b * p.nkv + g) * p.max_ctx * hd;
    uint16_t* vc = kc + (size_t)p.max_batch * p.nkv * p.max_ctx * hd;
    for (int e = threadIdx.x; e < gs * (hd / 2); e += NT) {
      int h = e / (hd / 2), i = e % (hd / 2);
      int col = (g * gs + h) * hd;
      float a = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + col + i) * 4u);
      float bb = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + col + i + hd / 2) * 4u);
      float cs, sn;
      rope_cs(pos, i, hd, p.theta, cs, sn);
      sm.q[h][i] = (a * cs - bb * sn) * scale;
      sm.q[h][i + hd / 2] = (a * sn + bb * cs) * scale;
    }
    if (a0 <= pos && pos < a1) {
      for (int i = threadIdx.x; i < hd / 2; i += NT) {
        int colk = p.nq * hd + g * hd;
        float a = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colk + i) * 4u);
        float bb = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colk + i + hd / 2) * 4u);
        float cs, sn;
        rope_cs(pos, i, hd, p.theta, cs, sn);
        kc[(size_t)pos * hd + i] = bf16_rne(a * cs - bb * sn);
        kc[(size_t)pos * hd + i + hd / 2] = bf16_rne(a * sn + bb * cs);
      }
      for (int i = threadIdx.x; i < hd; i += NT) {
        int colv = (p.nq + p.nkv) * hd + g * hd;
        vc[(size_t)pos * hd + i] = bf16_rne(ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colv + i) * 4u));
      }
      wait_stores();
    }
    __syncthreads();
    const int len = a1 - a0;
    const int wq = ((len + NW - 1) / NW + 31) / 32 * 32;
    const int w0 = a0 + wv * wq < a1 ? a0 + wv * wq : a1;
    const int w1 = w0 + wq < a1 ? w0 + wq : a1;
    const uint32_t nb = (uint32_t)((size_t)n * hd * 2);
    if (hd == 128) attn_task_wave<128>(p, sm, gs, kc, vc, nb, w0, w1);
    else attn_task_wave<64>(p, sm, gs, kc, vc, nb, w0, w1);
    __syncthreads();
    // this task's partial: m, l in part_ml[b][head][c]; o in part_o[b][head][c][hd]
    for (int e = threadIdx.x; e < gs * hd; e += NT) {
      int h = e / hd, d = e % hd;
      float M = -INFINITY;
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.wm[w][h]);
      float o = 0.f, l = 0.f;
      for (int w = 0; w < NW; ++w) {
        float f = sm.wm[w][h] == -INFINITY ? 0.f : __expf(sm.wm[w][h] - M);
        o += f * sm.wo[w][h][d];
        l += f * sm.wl[w][h];
      }
      uint32_t head = (uint32_t)((b * p.nq + g * gs + h) * C + c);
      if (d == 0) {
        st_f32(wr, p.off_attn_ml + head * 8u, M);
        st_f32(wr, p.off_attn_ml + head * 8u + 4u, l);
      }
      st_f32(wr, p.off_attn + (head * (uint32_t)hd + d) * 4u, o);
    }
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned* ctr = sync_pt(p, p.sync_attn_base + layer) + (b * p.nkv + g);
      unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.last = (old + 1 == (unsigned)C);
    }
    __syncthreads();
    if (sm.last) {
      // combine weights per head: w_c = exp(m_c - M), 1 / sum_c w_c l_c
      for (int e = threadIdx.x; e < gs * C; e += NT) {
        int h = e / C, cc = e % C;
        uint32_t hb = (uint32_t)((b * p.nq + g * gs + h) * C);
        sm.cw[h][cc] = ld_f32(wr, p.off_attn_ml + (hb + cc) * 8u);
      }
      __syncthreads();
      if (threadIdx.x < gs) {
        int h = threadIdx.x;
        uint32_t hb = (uint32_t)((b * p.nq + g * gs + h) * C);
        float M = -INFINITY;
        for (int cc = 0; cc < C; ++cc) M = fmaxf(M, sm.cw[h][cc]);
        float den = 0.f;
        for (int cc = 0; cc < C; ++cc) {
          float f = sm.cw[h][cc] == -INFINITY ? 0.f : __expf(sm.cw[h][cc] - M);
          sm.cw[h][cc] = f;
          den += f * ld_f32(wr, p.off_attn_ml + (hb + cc) * 8u + 4u);
        }
        sm.cl[h] = 1.0f / den;
      }
      __syncthreads();
      // o = sum_c w_c o_c: thread per (head, 4 dims), 16 chunk loads in flight
      for (int e = threadIdx.x; e < gs * (hd / 4); e += NT) {
        int h = e / (hd / 4), d4 = (e % (hd / 4)) * 4;
        uint32_t hb = (uint32_t)((b * p.nq + g * gs + h) * C);
        float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
        for (int c0 = 0; c0 < C; c0 += 16) {
          i32x4 v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            v[u] = ld_x4<CP_SC1>(wr, c0 + u < C ? p.off_attn + ((hb + c0 + u) * (uint32_t)hd + d4) * 4u : OOB);
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            float f = c0 + u < C ? sm.cw[h][c0 + u] : 0.f;
            o0 += f * __int_as_float(v[u][0]);
            o1 += f * __int_as_float(v[u][1]);
            o2 += f * __int_as_float(v[u][2]);
            o3 += f * __int_as_float(v[u][3]);
          }
        }
        float il = sm.cl[h];
        int col = (g * gs + h) * hd + d4;
        put_hilo(wr, p.off_ou, p.nq * hd, b, col + 0, o0 * il);
        put_hilo(wr, p.off_ou, p.nq * hd, b, col + 1, o1 * il);
        put_hilo(wr, p.off_ou, p.nq * hd, b, col + 2, o2 * il);
        put_hilo(wr, p.off_ou, p.nq * hd, b, col + 3, o3 * il);
      }
    }
    __syncthreads();
  }
}

// --- residual-owning projection: x[t][r] += W . U; next norm input + ssq
__device__ __noinline__ void phase_residual_gemv(const Params& p, const uint16_t* W, int K, uint32_t u_off,
                                    const uint16_t* g_next, char* smem) {
  GemvSmem& sm = *(GemvSmem*)smem;
  float* part = (float*)(smem + sizeof(GemvSmem));  // [NT][MAXB]
  GemvJob j;
  j.nm = 1;
  j.W[0] = W;
  j.N[0] = p.H;
  j.K = K;
  j.u_off = u_off;
  j.B = p.B;
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  for (int t = 0; t < MAXB; ++t) part[threadIdx.x * MAXB + t] = 0.f;
  run_gemv(p, j, sm, [&](GemvSmem& s, const Chunk& c) {
    int per = c.i1 - c.i0;
    for (int e = threadIdx.x; e < per * 16 * p.B; e += NT) {
      int t = e % p.B, rr = (e / p.B) % 16, slot = e / (p.B * 16);
      int lr = (c.i0 + slot) * 16 + rr;
      if (lr >= c.nrows[0]) continue;
      int row = c.r0[0] + lr;
      float x = p.x[t * p.H + row] + s.y[slot][rr][t];
      p.x[t * p.H + row] = x;
      put_hilo(r, p.off_u, p.H, t, row, bf16_f32(g_next[row]) * x);
      part[threadIdx.x * MAXB + t] += x * x;
    }
  });
  __syncthreads();
  if (threadIdx.x < MAXB) {
    float a = 0.f;
    for (int i = 0; i < NT; ++i) a += part[i * MAXB + threadIdx.x];
    st_f32(r, p.off_ssq + (uint32_t)(blockIdx.x * MAXB + threadIdx.x) * 4u, a);
  }
}

// --- dense SwiGLU gate/up: h = silu(inv*Wg U) * (inv*Wu U) -> hi/lo
__device__ __noinline__ void phase_gateup(const Params& p, const uint16_t* Wg, const uint16_t* Wu, int F, char* smem) {
  GemvSmem& sm = *(GemvSmem*)smem;
  float* inv = (float*)(smem + sizeof(GemvSmem));
  load_inv_rms(p, inv, p.H);
  GemvJob j;
  j.nm = 2;
  j.W[0] = Wg; j.N[0] = F;
  j.W[1] = Wu; j.N[1] = F;
  j.K = p.H;
  j.u_off = p.off_u;
  j.B = p.B;
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  run_gemv(p, j, sm, [&](GemvSmem& s, const Chunk& c) {
    int per = c.i1 - c.i0;
    for (int e = threadIdx.x; e < per * 16 * p.B; e += NT) {
      int t = e % p.B, rr = (e / p.B) % 16, li = e / (p.B * 16);
      int lr = (c.i0 + li) * 16 + rr;
      if (lr >= c.nrows[0]) continue;
      float a = s.y[li][rr][t] * inv[t];
      float u = s.y[per + li][rr][t] * inv[t];
      put_hilo(r, p.off_h, F, t, c.r0[0] + lr, silu(a) * u);
    }
  });
}

// --- final norm + LM head: logits, per-WG argmax candidates
__device__ __noinline__ void phase_lmhead(const Params& p, char* smem) {
  GemvSmem& sm = *(GemvSmem*)smem;
  float* inv = (float*)(smem + sizeof(GemvSmem));
  float* bv = inv + MAXB;                 // [NT][MAXB] best value
  int* bi = (int*)(bv + NT * MAXB);       // [NT][MAXB] best index
  load_inv_rms(p, inv, p.H);
  for (int t = 0; t < MAXB; ++t) { bv[threadIdx.x * MAXB + t] = -INFINITY; bi[threadIdx.x * MAXB + t] = 0x7FFFFFFF; }
  GemvJob j;
  j.nm = 1;
  j.W[0] = p.lm_head;
  j.N[0] = p.V;
  j.K = p.H;
  j.u_off = p.off_u;
  j.B = p.B;
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  run_gemv(p, j, sm, [&](GemvSmem& s, const Chunk& c) {
    int per = c.i1 - c.i0;
    for (int e = threadIdx.x; e < per * 16 * p.B; e += NT) {
      int t = e % p.B, rr = (e / p.B) % 16, slot = e / (p.B * 16);
      int lr = (c.i0 + slot) * 16 + rr;
      if (lr >= c.nrows[0]) continue;
      int v = c.r0[0] + lr;
      float lg = s.y[slot][rr][t] * inv[t];
      p.logits[(size_t)t * p.V + v] = lg;
      float& cb = bv[threadIdx.x * MAXB + t];
      int& ci = bi[threadIdx.x * MAXB + t];
      if (lg > cb || (lg == cb && v < ci)) { cb = lg; ci = v; }
    }
  });
  __syncthreads();
  if (threadIdx.x < p.B) {
    int t = threadIdx.x;
    float best = -INFINITY;
    int idx = 0x7FFFFFFF;
    for (int i = 0; i < NT; ++i) {
      float v = bv[i * MAXB + t];
      int k = bi[i * MAXB + t];
      if (v > best || (v == best && k < idx)) { best = v; idx = k; }
    }
    st_f32(r, p.off_cand + (uint32_t)(blockIdx.x * MAXB + t) * 8u, best);
    st_u32(r, p.off_cand + (uint32_t)(blockIdx.x * MAXB + t) * 8u + 4u, (uint32_t)idx);
  }
}

// final argmax over the WG candidates (one workgroup)
__device__ __noinline__ void final_argmax(const Params& p) {
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    for (int t = 0; t < p.B; ++t) {
      float best = -INFINITY;
      int idx = 0x7FFFFFFF;
      for (int g = lane; g < (int)gridDim.x; g += 64) {
        float v = ld_f32(r, p.off_cand + (uint32_t)(g * MAXB + t) * 8u);
        int k = (int)ld_u32(r, p.off_cand + (uint32_t)(g * MAXB + t) * 8u + 4u);
        if (v > best || (v == best && k < idx)) { best = v; idx = k; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        float ov = __shfl_xor(best, o, 64);
        int oi = __shfl_xor(idx, o, 64);
        if (ov > best || (ov == best && oi < idx)) { best = ov; idx = oi; }
      }
      if (lane == 0 && p.out_tokens) p.out_tokens[t] = idx;
    }
  }
}

// ===================================================================== kernel
extern "C" __global__ __launch_bounds__(NT) void md_megakernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  if (p.B < 1 || p.B > MAXB) return;
  if (p.trace && threadIdx.x == 0 && p.trace_n > 0) p.trace[(size_t)blockIdx.x * p.trace_n + p.trace_n - 1] = wall_clock64();
  clear_next_bank(p);
  int sidx = 0;
  phase_embed(p, (float*)smem);
  grid_sync(p, sidx);
  for (int l = 0; l < p.n_layers; ++l) {
    const LayerDesc& L = p.layers[l];
    const uint16_t* g_next = (l + 1 < p.n_layers) ? p.layers[l + 1].attn_norm : p.final_norm;
    phase_qkv(p, L, smem);
    grid_sync(p, sidx);
    phase_attn_gqa(p, L, l, smem);
    grid_sync(p, sidx);
    phase_residual_gemv(p, L.wo, p.nq * p.hd, p.off_ou, L.ffn_norm, smem);
    grid_sync(p, sidx);
    phase_gateup(p, L.w_gate, L.w_up, p.ffn, smem);
    grid_sync(p, sidx);
    phase_residual_gemv(p, L.w_down, p.ffn, p.off_h, g_next, smem);
    grid_sync(p, sidx);
    if (dev_failed(p)) return;
  }
  phase_lmhead(p, smem);
  // the last workgroup to arrive reduces the argmax candidates
  bool last = arrive(p, sidx);
  if (threadIdx.x == 0) ((int*)smem)[0] = last;
  __syncthreads();
  if (((int*)smem)[0]) final_argmax(p);
}

}  // namespace md

// ===================================================================== launch helpers
namespace md {

size_t megakernel_smem_bytes() {
  size_t gemv = sizeof(GemvSmem) + MAXB * 4 + (size_t)NT * MAXB * 8 + 64;
  size_t attn = sizeof(AttnSmem) + 64;
  return gemv > attn ? gemv : attn;
}

hipError_t launch_megakernel(const Params& p, int grid, hipStream_t stream) {
  void* args[] = {(void*)&p};
  return hipLaunchCooperativeKernel((const void*)md_megakernel, dim3(grid), dim3(NT), args,
                                    (unsigned)megakernel_smem_bytes(), stream);
}

hipError_t megakernel_occupancy(int* blocks_per_cu) {
  hipError_t e = hipFuncSetAttribute((const void*)md_megakernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)megakernel_smem_bytes());
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)md_megakernel, NT,
                                                      megakernel_smem_bytes());
}

}  // namespace md
