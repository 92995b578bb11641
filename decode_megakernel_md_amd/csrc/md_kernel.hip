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

// Sub-phase stamps: slot trace_n/2 + 4*(phase index) + k, k < 4.
__shared__ int md_cur_phase;
__device__ __forceinline__ void sub_stamp(const Params& p, int k) {
  if (p.trace && threadIdx.x == 0) {
    int slot = p.trace_n / 2 + 4 * md_cur_phase + k;
    if (slot < p.trace_n - 1) p.trace[(size_t)blockIdx.x * p.trace_n + slot] = wall_clock64();
  }
}

// Sync point sidx: stamps 2*sidx (work done) and 2*sidx+1 (wait over).
__device__ __forceinline__ void grid_sync(const Params& p, int& sidx) {
  stamp(p, 2 * sidx);
  arrive(p, sidx);
  wait_all(p, sidx);
  stamp(p, 2 * sidx + 1);
  ++sidx;
  if (threadIdx.x == 0) md_cur_phase = sidx;
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
// Y[r][t] = sum_k W[r][k] * U[t][k] for this workgroup's rows of up to MAXM
// matrices that share K.
//
// Weights are in the tiled layout md_pack_weight writes: 16-row tiles, and
// within a tile one contiguous 1 KB block per 32-column k-step holding the
// matrix-core A operand (lane l: row l%16, columns 8*(l/16)..+7), the block
// ordered as four 256-byte quarters of 4 rows.  A tile's blocks are
// consecutive, so every wave instruction reads 1 KB contiguous and each tile
// is one sequential stream.
//
// U is the activation in hi/lo form, bf16[2][MAXB][K] (part, token, k): the
// B operand (32 k x 16 columns: token t hi at column 2t, lo at 2t+1) is one
// 16-byte load per lane.
//
// Work split: each matrix's rows are cut into 4-row quarters and workgroup w
// owns quarters [Q*w/G, Q*(w+1)/G), so every workgroup streams the same
// number of bytes.  Its rows form "slots" (tiles, possibly partial: lanes of
// other quarters load nothing).  Slots are consumed in pairs; the four waves
// split the k-steps of a pair and keep DS k-steps of loads in flight in one
// continuous stream across pairs (no pipeline drain between tiles).
// The workgroup's dynamic LDS.  Phases address it through this symbol (not
// through a pointer argument) so that accesses compile to LDS instructions.
extern __shared__ __attribute__((aligned(16))) char md_smem[];

constexpr int MAXM = 3;
constexpr int CMAX_DEV = 256;  // largest chunk count per (sequence, kv head)
constexpr int TG = 2;          // tiles consumed together (share one B operand load)
constexpr int GDS = 12;        // k-steps in flight per wave
constexpr int MAXSLOT = 48;    // slots per workgroup and phase (LM head: <= 41)

struct GemvJob {
  const uint16_t* W[MAXM];
  int N[MAXM];
  int nm;
  int K;
  uint32_t u_off;  // byte offset of U in the workspace
  int B;
  bool pair;       // slot list interleaves matrices 0 and 1 tile by tile (SwiGLU)
};

struct RowSplit {
  int r0, r1;
};
__device__ __forceinline__ RowSplit rows_of(int N, int w, int G) {
  RowSplit s;
  s.r0 = (int)((int64_t)N * w / G);
  s.r1 = (int)((int64_t)N * (w + 1) / G);
  return s;
}

// One slot = one matrix-core tile of 16 output rows assembled from four
// 4-row quarters, each from any matrix of the phase (a "virtual tile"): the
// lanes of quarter position e read matrix m[e], global quarter gq[e]
// (rows 4*gq .. 4*gq+3), through their own 64-bit addresses.  gq < 0: empty.
struct Slot {
  int8_t m[4];
  int gq[4];
};

struct GemvSmem {
  float red[NW][TG][16][16];   // also reused as [NT][MAXB] scratch after the stream
  float y[TG][16][MAXB];
  Slot slots[MAXSLOT];
  int nslots;
  // epilogue staging, indexed [slot*16 + row-in-slot][token]: inputs read
  // before the weight stream starts, outputs written after it ends, so the
  // stream itself issues no other memory operation
  float in[MAXSLOT * 16][MAXB];
  float out[MAXSLOT * 16][MAXB];
  float gain[MAXSLOT * 16];
  float inv[MAXB];
};

// Build this workgroup's slot list (thread 0) into LDS.  Normal mode packs
// the workgroup's quarters of matrix 0, then 1, then 2, four per slot.  Pair
// mode (SwiGLU) emits a slot of 4 gate quarters followed by the slot of the
// same 4 up quarters.
__device__ void build_slots(const GemvJob& job, GemvSmem& sm) {
  if (threadIdx.x == 0) {
    const int G = gridDim.x, w = blockIdx.x;
    int n = 0, fill = 0;
    Slot cur;
    auto reset = [&]() {
      for (int e = 0; e < 4; ++e) { cur.m[e] = 0; cur.gq[e] = -1; }
      fill = 0;
    };
    reset();
    if (job.pair) {
      RowSplit q = rows_of((job.N[0] + 3) >> 2, w, G);
      for (int g0 = q.r0; g0 < q.r1 && n + 2 <= MAXSLOT; g0 += 4) {
        Slot a, b;
        for (int e = 0; e < 4; ++e) {
          int gq = g0 + e < q.r1 ? g0 + e : -1;
          a.m[e] = 0; a.gq[e] = gq;
          b.m[e] = 1; b.gq[e] = gq;
        }
        sm.slots[n++] = a;
        sm.slots[n++] = b;
      }
    } else {
      for (int m = 0; m < job.nm; ++m) {
        RowSplit q = rows_of((job.N[m] + 3) >> 2, w, G);
        for (int gq = q.r0; gq < q.r1; ++gq) {
          cur.m[fill] = (int8_t)m;
          cur.gq[fill] = gq;
          if (++fill == 4) {
            if (n < MAXSLOT) sm.slots[n++] = cur;
            reset();
          }
        }
      }
      if (fill > 0 && n < MAXSLOT) sm.slots[n++] = cur;
    }
    sm.nslots = n;
  }
  __syncthreads();
}

// Run the GEMV; after each pair of slots epi(sm, slot_index0, count) reads
// sm.y[i][row-in-slot][token] for slots slot_index0 + i (slot_row maps a row
// of a slot back to its matrix and row).
// The GEMV's LDS block, addressed through the LDS symbol itself (never
// through a pointer held in a closure or passed by value), so that every
// access compiles to an LDS instruction: a flat or scratch access inside the
// stream would make the next wait drain the whole prefetch ring.
#define GSM (*reinterpret_cast<GemvSmem*>(md_smem))

// Per-lane source of one slot of the current group.
__device__ __forceinline__ void slot_src(int si, int nslots, int lq, uint64_t w0, uint64_t w1, uint64_t w2,
                                         uint64_t tstride, uint32_t lchunk, int wv, uint64_t zero_addr, uint64_t& pa,
                                         uint32_t& pstep) {
  bool v = si < nslots;
  int gq = v ? GSM.slots[si].gq[lq] : -1;
  int m = v ? GSM.slots[si].m[lq] : 0;
  uint64_t W = m == 0 ? w0 : (m == 1 ? w1 : w2);
  bool lv = gq >= 0;
  pa = lv ? W + (uint64_t)(gq >> 2) * tstride + (uint64_t)((gq & 3) * 256) + lchunk + (uint64_t)wv * 1024u : zero_addr;
  pstep = lv ? (uint32_t)(NW * 1024) : 0u;
}

// Reduce the four waves' partial tiles of a finished group into GSM.y.
__device__ __forceinline__ void gemv_reduce(const f32x4 (&acc)[TG], int wv, int lane) {
#pragma unroll
  for (int i = 0; i < TG; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) GSM.red[wv][i][4 * (lane >> 4) + r][lane & 15] = acc[i][r];
  __syncthreads();
  for (int e = threadIdx.x; e < TG * 16 * MAXB; e += NT) {
    int i = e / (16 * MAXB), r = (e / MAXB) % 16, k = e % MAXB;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += GSM.red[w][i][r][2 * k] + GSM.red[w][i][r][2 * k + 1];
    GSM.y[i][r][k] = s;
  }
  __syncthreads();
}

// Run the GEMV over GSM's slot list.  After each finished pair of slots,
// epi(slot_index0, count) reads GSM.y[i][row-in-slot][token] (LDS only).
template <class Epi>
__device__ __forceinline__ void run_gemv(const GemvJob& job, const uint8_t* ws, uint32_t ws_bytes, uint32_t off_zero,
                                         Epi epi) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = job.K, KS = K >> 5;
  const int nslots = __builtin_amdgcn_readfirstlane(GSM.nslots);
  const int ngroups = (nslots + TG - 1) / TG;
  const int nks = (KS - wv + NW - 1) / NW;
  const int total = ngroups * nks;
  const rsrc_t urs = make_rsrc_u(ws, ws_bytes);
  const int lq = (lane & 15) >> 2;
  const uint32_t lchunk = (uint32_t)(((lane >> 4) * 4 + (lane & 3)) * 16);
  const int n16 = lane & 15, tok = n16 >> 1, part = n16 & 1;
  const uint32_t boff = tok < job.B ? job.u_off + (uint32_t)((part * MAXB + tok) * K) * 2u + (lane >> 4) * 16u : OOB;
  const uint64_t tstride = (uint64_t)KS * 1024u;
  const uint64_t zero_addr = (uint64_t)(ws + off_zero);
  const uint64_t w0 = (uint64_t)job.W[0], w1 = job.nm > 1 ? (uint64_t)job.W[1] : w0,
                 w2 = job.nm > 2 ? (uint64_t)job.W[2] : w0;
  int ig = 0, is = 0;
  uint64_t pa0, pa1;
  uint32_t ps0, ps1;
  slot_src(0, nslots, lq, w0, w1, w2, tstride, lchunk, wv, zero_addr, pa0, ps0);
  slot_src(1, nslots, lq, w0, w1, w2, tstride, lchunk, wv, zero_addr, pa1, ps1);
  static_assert(TG == 2, "the stream handles slot pairs");
#define GEMV_ISSUE(RA, RB)                                                                                      \
  {                                                                                                             \
    bool ok_ = ig < ngroups;                                                                                    \
    RA[0] = __builtin_nontemporal_load((const __attribute__((address_space(1))) i32x4*)(ok_ ? pa0 : zero_addr)); \
    RA[1] = __builtin_nontemporal_load((const __attribute__((address_space(1))) i32x4*)(ok_ ? pa1 : zero_addr)); \
    pa0 += ps0;                                                                                                 \
    pa1 += ps1;                                                                                                 \
    RB = ld_x4<CP_SC1>(urs, ok_ && boff != OOB ? boff + (uint32_t)(is * NW + wv) * 64u : OOB);                  \
    if (++is == nks) {                                                                                          \
      is = 0;                                                                                                   \
      ++ig;                                                                                                     \
      if (ig < ngroups) {                                                                                       \
        slot_src(ig * TG, nslots, lq, w0, w1, w2, tstride, lchunk, wv, zero_addr, pa0, ps0);                   \
        slot_src(ig * TG + 1, nslots, lq, w0, w1, w2, tstride, lchunk, wv, zero_addr, pa1, ps1);               \
      }                                                                                                         \
    }                                                                                                           \
  }
  f32x4 acc[TG];
#pragma unroll
  for (int i = 0; i < TG; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  i32x4 ra[GDS][TG], rb[GDS];
#pragma unroll
  for (int d = 0; d < GDS; ++d) GEMV_ISSUE(ra[d], rb[d]);
  int cg = 0, cs = 0;
  if (nks == 0) {
    for (; cg < ngroups; ++cg) {
      gemv_reduce(acc, wv, lane);
      int n = nslots - cg * TG;
      epi(cg * TG, n < TG ? n : TG);
      __syncthreads();
    }
    return;
  }
  // The body is unconditional: steps past the end read the zero block and
  // add nothing.  (A guarded body would make the compiler assume the later
  // loads of the previous round may be missing and wait for all of them.)
  for (int j0 = 0; j0 < total; j0 += GDS) {
#pragma unroll
    for (int d = 0; d < GDS; ++d) {
      bf16x8 bop = __builtin_bit_cast(bf16x8, rb[d]);
#pragma unroll
      for (int i = 0; i < TG; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ra[d][i]), bop, acc[i], 0, 0, 0);
      GEMV_ISSUE(ra[d], rb[d]);
      if (j0 + d < total) {
        if (++cs == nks) {
          cs = 0;
          gemv_reduce(acc, wv, lane);
#pragma unroll
          for (int i = 0; i < TG; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
          int n = nslots - cg * TG;
          epi(cg * TG, n < TG ? n : TG);
          __syncthreads();
          ++cg;
        }
      }
    }
  }
#undef GEMV_ISSUE
}

// Row rr (0..15) of a slot: matrix and global row; false for an empty
// quarter or a row past the matrix end.
__device__ __forceinline__ bool slot_row(const Slot& sl, int rr, const int* N, int& m, int& row) {
  int gq = sl.gq[rr >> 2];
  if (gq < 0) return false;
  m = sl.m[rr >> 2];
  row = gq * 4 + (rr & 3);
  return row < N[m];
}

// Rows of an N-row output this workgroup owns: 4-row quarters
// [Q*w/G, Q*(w+1)/G), the split every projection uses.  The residual x is
// private to the owner of its rows, so every phase that touches x must use
// this same split.
__device__ __forceinline__ RowSplit owned_rows(int N, int w, int G) {
  RowSplit q = rows_of((N + 3) >> 2, w, G);
  RowSplit r;
  r.r0 = q.r0 * 4 < N ? q.r0 * 4 : N;
  r.r1 = q.r1 * 4 < N ? q.r1 * 4 : N;
  return r;
}


// ===================================================================== phases

// inv_rms[t] from the per-WG partial sums of squares (fixed order: identical
// in every workgroup).  ssq: fp32[G][MAXB] at ws offset p.off_ssq.
__device__ __noinline__ void load_inv_rms(const Params& p, float* inv_rms, int n_feat) {
  // every thread fetches one workgroup's partials for all tokens (one round
  // trip), then wave w reduces tokens 2w, 2w+1 in a fixed order
  float* stage = (float*)(md_smem + sizeof(GemvSmem));  // [G][MAXB]
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  for (int g = threadIdx.x; g < (int)gridDim.x; g += NT) {
    i32x4 a = ld_x4<CP_SC1>(r, p.off_ssq + (uint32_t)(g * MAXB) * 4u);
    i32x4 b = ld_x4<CP_SC1>(r, p.off_ssq + (uint32_t)(g * MAXB + 4) * 4u);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      stage[g * MAXB + k] = __int_as_float(a[k]);
      stage[g * MAXB + 4 + k] = __int_as_float(b[k]);
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    int t = 2 * wv + k;
    float s = 0.f;
    for (int g = lane; g < (int)gridDim.x; g += 64) s += stage[g * MAXB + t];
    s = wave_sum(s);
    if (lane == 0) inv_rms[t] = 1.0f / sqrtf(s / (float)n_feat + p.eps);
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
__device__ __noinline__ void phase_embed(const Params& p) {
  RowSplit s = owned_rows(p.H, blockIdx.x, gridDim.x);
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  const uint16_t* g = p.layers[0].attn_norm;
  float* part = (float*)md_smem;  // [NT][MAXB]
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
__device__ __noinline__ void phase_qkv(const Params& p, const LayerDesc& L) {
  GemvSmem& sm = *(GemvSmem*)md_smem;
  GemvJob j;
  j.nm = 3;
  j.W[0] = L.wq; j.N[0] = p.nq * p.hd;
  j.W[1] = L.wk; j.N[1] = p.nkv * p.hd;
  j.W[2] = L.wv; j.N[2] = p.nkv * p.hd;
  j.K = p.H;
  j.u_off = p.off_u;
  j.B = p.B;
  j.pair = false;
  const int B = p.B;
  build_slots(j, sm);
  load_inv_rms(p, sm.inv, p.H);
  sub_stamp(p, 0);
  run_gemv(j, p.ws, p.ws_bytes, p.off_zero, [=](int slot0, int n) {
    for (int e = threadIdx.x; e < n * 16 * B; e += NT) {
      int t = e % B, rr = (e / B) % 16, i = e / (B * 16);
      GSM.out[(slot0 + i) * 16 + rr][t] = GSM.y[i][rr][t] * GSM.inv[t];
    }
  });
  sub_stamp(p, 2);
  const int nqkv = (p.nq + 2 * p.nkv) * p.hd;
  const int col0[3] = {0, p.nq * p.hd, (p.nq + p.nkv) * p.hd};
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  for (int e = threadIdx.x; e < sm.nslots * 16 * B; e += NT) {
    int t = e % B, sr = e / B;
    int m, row;
    if (!slot_row(sm.slots[sr >> 4], sr & 15, j.N, m, row)) continue;
    st_f32(r, p.off_qkv + (uint32_t)(t * nqkv + col0[m] + row) * 4u, sm.out[sr][t]);
  }
}

// RoPE rotation of pair i at position pos: (cos, sin) from the table the
// host fills at init (angles pos * theta^(-2i/d) evaluated in fp64, rounded
// to fp32), fp32[max_ctx][d/2][2].
__device__ __forceinline__ void rope_cs(const Params& p, int pos, int i, float& c, float& s) {
  const float* t = p.rope + ((size_t)pos * (p.rope_d / 2) + i) * 2;
  c = t[0];
  s = t[1];
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

#define ASM (*reinterpret_cast<AttnSmem*>(md_smem))

template <int HD, int GS>
__device__ __noinline__ void attn_task_wave(const uint16_t* kc, const uint16_t* vc, uint32_t nbytes, int w0, int w1) {
  constexpr int gs = GS;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const rsrc_t krs = make_rsrc_u(kc, nbytes), vrs = make_rsrc_u(vc, nbytes);
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
      float v = hh < gs ? ASM.q[hh][d] : 0.f;
      uint16_t hi, lo;
      split_hilo(v, hi, lo);
      qb[s][k] = __builtin_bit_cast(__bf16, pp ? lo : hi);
    }
  }
  float m_run[GS], l_run[GS], acc[GS][8];
#pragma unroll
  for (int h = 0; h < GS; ++h) {
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
        float v = a[i] + dpp_f<DPP_QXOR1>(a[i]);
        int pr = tt * 16 + 4 * (lane >> 4) + i;
        if (!pp && hh < gs) ASM.s[wv][pr][hh] = (blk + pr < w1) ? v : -INFINITY;
      }
    }
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_wave_barrier();
    // online softmax per head over this block; probabilities replace scores
#pragma unroll
    for (int h = 0; h < GS; ++h) {
      {
        float sv = lane < 32 ? ASM.s[wv][lane][h] : -INFINITY;
        float mb = wave_max(sv);
        float mn = fmaxf(m_run[h], mb);
        float corr = __expf(m_run[h] - mn);
        float pv = lane < 32 ? __expf(sv - mn) : 0.f;
        l_run[h] = l_run[h] * corr + wave_sum(pv);
        m_run[h] = mn;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] *= corr;
        if (lane < 32) ASM.s[wv][lane][h] = pv;
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
      for (int h = 0; h < GS; ++h) {
        {
          float pw = ASM.s[wv][t][h];
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
  for (int h = 0; h < GS; ++h) {
    {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[h][j];
        if (LPR == 8) v += dpp_f<DPP_ROR8>(v);  // lanes i and i^8 hold the same dims
        acc[h][j] = rows_sum(v);
      }
      if (lane == 0) { ASM.wm[wv][h] = m_run[h]; ASM.wl[wv][h] = l_run[h]; }
      if (lane < LPR) {
#pragma unroll
        for (int j = 0; j < 8; ++j) ASM.wo[wv][h][lane * 8 + j] = acc[h][j];
      }
    }
  }
}

template <int HD>
__device__ __forceinline__ void attn_dispatch(int gs, const uint16_t* kc, const uint16_t* vc, uint32_t nb, int w0, int w1) {
  switch (gs) {
    case 1: attn_task_wave<HD, 1>(kc, vc, nb, w0, w1); break;
    case 2: attn_task_wave<HD, 2>(kc, vc, nb, w0, w1); break;
    case 3: attn_task_wave<HD, 3>(kc, vc, nb, w0, w1); break;
    case 4: attn_task_wave<HD, 4>(kc, vc, nb, w0, w1); break;
    case 5: attn_task_wave<HD, 5>(kc, vc, nb, w0, w1); break;
    case 6: attn_task_wave<HD, 6>(kc, vc, nb, w0, w1); break;
    case 7: attn_task_wave<HD, 7>(kc, vc, nb, w0, w1); break;
    default: attn_task_wave<HD, 8>(kc, vc, nb, w0, w1); break;
  }
}

__device__ __noinline__ void phase_attn_gqa(const Params& p, const LayerDesc& L, int layer) {
  AttnSmem& sm = *(AttnSmem*)md_smem;
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
      rope_cs(p, pos, i, cs, sn);
      sm.q[h][i] = (a * cs - bb * sn) * scale;
      sm.q[h][i + hd / 2] = (a * sn + bb * cs) * scale;
    }
    if (a0 <= pos && pos < a1) {
      for (int i = threadIdx.x; i < hd / 2; i += NT) {
        int colk = p.nq * hd + g * hd;
        float a = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colk + i) * 4u);
        float bb = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colk + i + hd / 2) * 4u);
        float cs, sn;
        rope_cs(p, pos, i, cs, sn);
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
    sub_stamp(p, 0);
    const int len = a1 - a0;
    const int wq = ((len + NW - 1) / NW + 31) / 32 * 32;
    const int w0 = a0 + wv * wq < a1 ? a0 + wv * wq : a1;
    const int w1 = w0 + wq < a1 ? w0 + wq : a1;
    const uint32_t nb = (uint32_t)((size_t)n * hd * 2);
    if (hd == 128) attn_dispatch<128>(gs, kc, vc, nb, w0, w1);
    else attn_dispatch<64>(gs, kc, vc, nb, w0, w1);
    __syncthreads();
    sub_stamp(p, 3);
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
    sub_stamp(p, 1);
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
    sub_stamp(p, 2);
  }
}

// --- residual-owning projection: x[t][r] += W . U; next norm input + ssq
__device__ __noinline__ void phase_residual_gemv(const Params& p, const uint16_t* W, int K, uint32_t u_off,
                                                 const uint16_t* g_next) {
  GemvSmem& sm = *(GemvSmem*)md_smem;
  GemvJob j;
  j.nm = 1;
  j.W[0] = W;
  j.N[0] = p.H;
  j.K = K;
  j.u_off = u_off;
  j.B = p.B;
  j.pair = false;
  const int B = p.B, H = p.H;
  build_slots(j, sm);
  // stage the residual rows and next-norm gains this workgroup owns
  for (int e = threadIdx.x; e < sm.nslots * 16 * B; e += NT) {
    int t = e % B, sr = e / B;
    int m, row;
    if (!slot_row(sm.slots[sr >> 4], sr & 15, j.N, m, row)) continue;
    sm.in[sr][t] = p.x[t * H + row];
    if (t == 0) sm.gain[sr] = bf16_f32(g_next[row]);
  }
  __syncthreads();
  sub_stamp(p, 0);
  run_gemv(j, p.ws, p.ws_bytes, p.off_zero, [=](int slot0, int n) {
    for (int e = threadIdx.x; e < n * 16 * B; e += NT) {
      int t = e % B, rr = (e / B) % 16, i = e / (B * 16);
      int sr = (slot0 + i) * 16 + rr;
      GSM.out[sr][t] = GSM.in[sr][t] + GSM.y[i][rr][t];
    }
  });
  sub_stamp(p, 2);
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  static_assert(sizeof(GemvSmem::red) >= sizeof(float) * NT * MAXB, "partial sums reuse the reduction scratch");
  float* part = (float*)sm.red;  // [NT][MAXB], reuses the reduction scratch
  for (int t = 0; t < MAXB; ++t) part[threadIdx.x * MAXB + t] = 0.f;
  for (int e = threadIdx.x; e < sm.nslots * 16 * B; e += NT) {
    int t = e % B, sr = e / B;
    int m, row;
    if (!slot_row(sm.slots[sr >> 4], sr & 15, j.N, m, row)) continue;
    float x = sm.out[sr][t];
    p.x[t * H + row] = x;
    put_hilo(r, p.off_u, H, t, row, sm.gain[sr] * x);
    part[threadIdx.x * MAXB + t] += x * x;
  }
  __syncthreads();
  if (threadIdx.x < MAXB) {
    float a = 0.f;
    for (int i = 0; i < NT; ++i) a += part[i * MAXB + threadIdx.x];
    st_f32(r, p.off_ssq + (uint32_t)(blockIdx.x * MAXB + threadIdx.x) * 4u, a);
  }
}

// --- dense SwiGLU gate/up: h = silu(inv*Wg U) * (inv*Wu U) -> hi/lo
__device__ __noinline__ void phase_gateup(const Params& p, const uint16_t* Wg, const uint16_t* Wu, int F) {
  GemvSmem& sm = *(GemvSmem*)md_smem;
  GemvJob j;
  j.nm = 2;
  j.W[0] = Wg; j.N[0] = F;
  j.W[1] = Wu; j.N[1] = F;
  j.K = p.H;
  j.u_off = p.off_u;
  j.B = p.B;
  j.pair = true;
  const int B = p.B;
  build_slots(j, sm);
  load_inv_rms(p, sm.inv, p.H);
  sub_stamp(p, 0);
  // slots come as (gate quarters, the same up quarters); h goes to the gate slot's rows
  run_gemv(j, p.ws, p.ws_bytes, p.off_zero, [=](int slot0, int n) {
    for (int e = threadIdx.x; e < 16 * B; e += NT) {
      int t = e % B, rr = e / B;
      float a = GSM.y[0][rr][t] * GSM.inv[t];
      float u = GSM.y[1][rr][t] * GSM.inv[t];
      GSM.out[slot0 * 16 + rr][t] = silu(a) * u;
    }
  });
  sub_stamp(p, 2);
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  for (int e = threadIdx.x; e < sm.nslots * 16 * B; e += NT) {
    int t = e % B, sr = e / B;
    int slot = sr >> 4;
    if (slot & 1) continue;  // up slots carry no output
    int m, row;
    if (!slot_row(sm.slots[slot], sr & 15, j.N, m, row)) continue;
    put_hilo(r, p.off_h, F, t, row, sm.out[sr][t]);
  }
}

// --- final norm + LM head: logits, per-WG argmax candidates
__device__ __noinline__ void phase_lmhead(const Params& p) {
  GemvSmem& sm = *(GemvSmem*)md_smem;
  GemvJob j;
  j.nm = 1;
  j.W[0] = p.lm_head;
  j.N[0] = p.V;
  j.K = p.H;
  j.u_off = p.off_u;
  j.B = p.B;
  j.pair = false;
  const int B = p.B;
  build_slots(j, sm);
  load_inv_rms(p, sm.inv, p.H);
  sub_stamp(p, 0);
  run_gemv(j, p.ws, p.ws_bytes, p.off_zero, [=](int slot0, int n) {
    for (int e = threadIdx.x; e < n * 16 * B; e += NT) {
      int t = e % B, rr = (e / B) % 16, i = e / (B * 16);
      GSM.out[(slot0 + i) * 16 + rr][t] = GSM.y[i][rr][t] * GSM.inv[t];
    }
  });
  sub_stamp(p, 2);
  static_assert(sizeof(GemvSmem::in) >= 2 * sizeof(float) * NT * MAXB, "argmax scratch reuses the input staging");
  float* bv = &sm.in[0][0];              // [NT][MAXB] best value (the input staging is unused here)
  int* bi = (int*)(bv + NT * MAXB);      // [NT][MAXB] best index
  for (int t = 0; t < MAXB; ++t) { bv[threadIdx.x * MAXB + t] = -INFINITY; bi[threadIdx.x * MAXB + t] = 0x7FFFFFFF; }
  for (int e = threadIdx.x; e < sm.nslots * 16 * B; e += NT) {
    int t = e % B, sr = e / B;
    int m, v;
    if (!slot_row(sm.slots[sr >> 4], sr & 15, j.N, m, v)) continue;
    float lg = sm.out[sr][t];
    p.logits[(size_t)t * p.V + v] = lg;
    float& cb = bv[threadIdx.x * MAXB + t];
    int& ci = bi[threadIdx.x * MAXB + t];
    if (lg > cb || (lg == cb && v < ci)) { cb = lg; ci = v; }
  }
  __syncthreads();
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  if (threadIdx.x < B) {
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
  if (p.B < 1 || p.B > MAXB) return;
  if (p.trace && threadIdx.x == 0 && p.trace_n > 0) p.trace[(size_t)blockIdx.x * p.trace_n + p.trace_n - 1] = wall_clock64();
  clear_next_bank(p);
  int sidx = 0;
  if (threadIdx.x == 0) md_cur_phase = 0;
  phase_embed(p);
  grid_sync(p, sidx);
  for (int l = 0; l < p.n_layers; ++l) {
    const LayerDesc& L = p.layers[l];
    const uint16_t* g_next = (l + 1 < p.n_layers) ? p.layers[l + 1].attn_norm : p.final_norm;
    phase_qkv(p, L);
    grid_sync(p, sidx);
    phase_attn_gqa(p, L, l);
    grid_sync(p, sidx);
    phase_residual_gemv(p, L.wo, p.nq * p.hd, p.off_ou, L.ffn_norm);
    grid_sync(p, sidx);
    phase_gateup(p, L.w_gate, L.w_up, p.ffn);
    grid_sync(p, sidx);
    phase_residual_gemv(p, L.w_down, p.ffn, p.off_h, g_next);
    grid_sync(p, sidx);
    if (dev_failed(p)) return;
  }
  phase_lmhead(p);
  // the last workgroup to arrive reduces the argmax candidates
  bool last = arrive(p, sidx);
  if (threadIdx.x == 0) ((int*)md_smem)[0] = last;
  __syncthreads();
  if (((int*)md_smem)[0]) final_argmax(p);
}

}  // namespace md

// ===================================================================== launch helpers
namespace md {

// Tiled weight layout (see the GEMV section): one thread per 16-byte chunk of
// the packed output.  Chunk c of block (t, s) holds row t*16 + 4*(c/16) + c%4,
// columns s*32 + 8*((c%16)/4) .. +7; rows past the matrix are zero.
__global__ void k_pack_weight(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int64_t rows,
                              int64_t cols) {
  const int64_t S = cols / 32, T = (rows + 15) / 16;
  const int64_t n = T * S * 64;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t blk = i >> 6;
    int c = (int)(i & 63);
    int64_t t = blk / S, s = blk % S;
    int rr = (c >> 4) * 4 + (c & 3), j = (c & 15) >> 2;
    int64_t r = t * 16 + rr;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rows) v = *(const uint4*)(src + r * cols + s * 32 + j * 8);
    *(uint4*)(dst + blk * 512 + c * 8) = v;
  }
}

hipError_t launch_pack(const void* src, void* dst, int64_t rows, int64_t cols, hipStream_t stream) {
  int64_t n = ((rows + 15) / 16) * (cols / 32) * 64;
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(k_pack_weight, dim3((unsigned)g), dim3(256), 0, stream, (const uint16_t*)src, (uint16_t*)dst,
                     rows, cols);
  return hipGetLastError();
}

size_t megakernel_smem_bytes() {
  size_t gemv = sizeof(GemvSmem) + (size_t)1024 * MAXB * 4 + 64;  // + partial-sum staging of up to 1024 workgroups
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
