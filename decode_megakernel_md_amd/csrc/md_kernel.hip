// The decode megakernel for gfx950 (MI355X) and the C ABI of libmd.so.
//
// One persistent cooperative launch runs a whole decode step: one workgroup
// per CU, each walking the same phase list; phases are separated by
// device-wide sync points (hierarchical counters, see the sync section below).  This is the
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

#include <mutex>
#include <string>
#include <vector>

#include "md.h"
#include "md_device.h"
#include "md_model.h"

namespace md {

// The step's parameter block is read where the launch placed it, in the
// kernel-argument segment: the kernel passes that pointer to every device
// function, which makes it wave-uniform, so the loads are scalar (no copy in
// scratch memory, no wait on the vector-memory counter that the weight
// streams use).  The kernel-argument intrinsic itself is only meaningful in
// the kernel's own body, hence the explicit argument.  The layer table is
// read the same way (it does not change during a step).
typedef const __attribute__((address_space(4))) Params KParams;
typedef const __attribute__((address_space(4))) LayerDesc KLayer;
__device__ __forceinline__ KParams& kp_uniform(KParams& r) {
  const uint64_t a = (uint64_t)&r;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return *(KParams*)(((uint64_t)hi << 32) | lo);
}
#define PARAMS KParams& p = kp_uniform(pk)
__device__ __forceinline__ KLayer& layer_ref(KParams& pk, int l) {
  PARAMS;
  return ((KLayer*)p.layers)[__builtin_amdgcn_readfirstlane(l)];
}

// GEMV inputs: one buffer per use within a step (u: 2l = attention input
// of layer l, 2l+1 = its FFN input, 2L = the final norm's input; the others
// one per layer), so that no such address is read before it is written in
// the same launch and their loads may be served by the local L2.
__device__ __forceinline__ uint32_t u_at(KParams& pk, int i) { PARAMS; return p.off_u + (uint32_t)i * p.u_stride; }
__device__ __forceinline__ uint32_t ou_at(KParams& pk, int l) { PARAMS; return p.off_ou + (uint32_t)l * p.ou_stride; }
__device__ __forceinline__ uint32_t h_at(KParams& pk, int l) { PARAMS; return p.off_h + (uint32_t)l * p.h_stride; }
__device__ __forceinline__ uint32_t hs_at(KParams& pk, int l) { PARAMS; return p.off_hs + (uint32_t)l * p.hs_stride; }
__device__ __forceinline__ uint32_t hr_at(KParams& pk, int l) { PARAMS; return p.off_hr + (uint32_t)l * p.hr_lstride; }
__device__ __forceinline__ uint32_t uq_at(KParams& pk, int l) { PARAMS; return p.off_uq + (uint32_t)l * p.uq_stride; }
// the partial sums of squares that scale u(i) (indexed as u) and uq(l)
__device__ __forceinline__ uint32_t ssq_at(KParams& pk, int i) { PARAMS; return p.off_ssq + (uint32_t)i * p.ssq_stride; }
__device__ __forceinline__ uint32_t ssq2_at(KParams& pk, int l) { PARAMS; return p.off_ssq2 + (uint32_t)l * p.ssq2_stride; }

// ===================================================================== sync
// One sync point = 8 class counters (one per workgroup class blockIdx % 8,
// which on this part is the XCD the workgroup runs on) and one extra line,
// each on its own 128-byte line.  A workgroup arrives by incrementing its
// class counter without waiting for the result; a waiter polls the 8 class
// counters at once (one lane each) until every class has fully arrived.  The
// last sync point of a decode step instead reports which workgroup arrived
// last (its class counter's last arrival increments the extra line).
// Counters live in two banks used by alternate steps; every step clears the
// bank of the next step (nobody touches it during this step).
// 9 lines of 128 B; 17 in the 64-row build, whose attention phase counts
// the finished chunks of up to 64 x 8 (row, kv head) pairs in one sync point
constexpr int SP_WORDS = WIDE ? 17 * 32 : 9 * 32;
constexpr int NGRP = 8;

__device__ __forceinline__ unsigned* sync_pt(KParams& pk, int idx) {
  PARAMS;
  return p.sync + (size_t)p.bank * p.n_sync * SP_WORDS + (size_t)idx * SP_WORDS;
}

__device__ __forceinline__ bool dev_failed(KParams& pk) {
  PARAMS;
  return __hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__device__ __forceinline__ void set_err(KParams& pk, int code) {
  PARAMS;
  __hip_atomic_fetch_or(p.err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned class_members(int grp) { return (gridDim.x - grp + NGRP - 1) / NGRP; }

// every wave: make this wave's stores complete, then the workgroup arrives
// once.  The increment returns nothing, so nobody waits for it here.  Wave 1
// makes it: the next function entry waits for its completion in the issuing
// wave, and wave 0 builds the next phase's tables right away.
constexpr int ARRIVER = 64;
__device__ void arrive(KParams& pk, int idx) {
  PARAMS;
  wait_stores();
  __builtin_amdgcn_s_barrier();
  if (threadIdx.x == ARRIVER) {
    unsigned* sp = sync_pt(p, idx);
    const int grp = blockIdx.x & (NGRP - 1);
    (void)__hip_atomic_fetch_add(sp + 32 * grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Arrival at the step's last sync point; returns (in thread 0) whether this
// workgroup was the last of the grid to arrive.
__device__ bool arrive_last(KParams& pk, int idx) {
  PARAMS;
  wait_stores();
  __builtin_amdgcn_s_barrier();
  bool last = false;
  if (threadIdx.x == 0) {
    unsigned* sp = sync_pt(p, idx);
    const int grp = blockIdx.x & (NGRP - 1);
    const unsigned ngrp = gridDim.x < NGRP ? gridDim.x : NGRP;
    unsigned old = __hip_atomic_fetch_add(sp + 32 * grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == class_members(grp))
      last = __hip_atomic_fetch_add(sp + 32 * NGRP, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == ngrp;
  }
  return last;
}

// wait until every class has fully arrived at sync point idx (wave 0 polls,
// lane g the counter of class g)
__device__ void wait_all(KParams& pk, int idx) {
  PARAMS;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int ngrp = gridDim.x < NGRP ? gridDim.x : NGRP;
    const bool mine = lane < ngrp;
    const unsigned need = mine ? class_members(lane) : 0u;
    unsigned* c = sync_pt(p, idx) + 32 * (mine ? lane : 0);
    unsigned spins = 0;
    while (true) {
      const unsigned v = mine ? __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
      if (__all(v >= need)) break;
      __builtin_amdgcn_s_sleep(1);
      if (((++spins) & 1023u) == 0 && (spins > p.spin_limit || dev_failed(p))) {
        if (lane == 0) set_err(p, MDE_WATCHDOG);
        break;
      }
    }
  }
  __builtin_amdgcn_s_barrier();
}

// ---- trace stamps (optional, p.trace).  In the 8-row build the megakernel
// keeps them in LDS during the step, as 32-bit ticks after its start, and
// writes them out when it ends: a global store per stamp would be waited for
// at the next function entry (the calling convention waits there for every
// outstanding memory operation) and so lengthen what it measures.  Slots of
// phases past TR_PH, the 64-row build and the multi-launch step store
// directly.  LDS word i: main slot i (i < 2 TR_PH), else sub-phase slot
// trace_n/2 + (i - 2 TR_PH); 0 = not recorded, else ticks + 1.
constexpr int TR_PH = WIDE ? 0 : 640;
constexpr int TR_WORDS = WIDE ? 1 : 10 * TR_PH;
__shared__ uint32_t md_trace_lds[TR_WORDS];
__shared__ uint64_t md_trace_t0;  // the step's start (0: stamps go to memory directly)

__device__ __forceinline__ void trace_put(KParams& pk, int slot, int lds_i) {
  PARAMS;
  const uint64_t t = wall_clock64();
  if (!WIDE && lds_i >= 0 && lds_i < TR_WORDS && md_trace_t0 != 0) md_trace_lds[lds_i] = (uint32_t)(t - md_trace_t0) + 1u;
  else p.trace[(size_t)blockIdx.x * p.trace_n + slot] = t;
}
// the step's start: stamps from here on are kept in LDS
__device__ __forceinline__ void trace_begin(KParams& pk) {
  PARAMS;
  if (threadIdx.x == 0) md_trace_t0 = 0;
  if (!p.trace || p.trace_n <= 0) return;
  for (int i = threadIdx.x; i < TR_WORDS; i += NT) md_trace_lds[i] = 0u;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t t = wall_clock64();
    p.trace[(size_t)blockIdx.x * p.trace_n + p.trace_n - 1] = t;
    if (!WIDE) md_trace_t0 = t;
  }
}
// write the kept stamps out (wave 0; thread 0 wrote them, so no barrier)
__device__ void trace_flush(KParams& pk) {
  PARAMS;
  if (WIDE || !p.trace || threadIdx.x >= 64) return;
  const uint64_t t0 = md_trace_t0;
  if (t0 == 0) return;
  for (int i = threadIdx.x; i < TR_WORDS; i += 64) {
    const uint32_t v = md_trace_lds[i];
    const int slot = i < 2 * TR_PH ? i : p.trace_n / 2 + (i - 2 * TR_PH);
    if (v != 0u && slot < p.trace_n - 1) p.trace[(size_t)blockIdx.x * p.trace_n + slot] = t0 + (v - 1u);
  }
}

__device__ __forceinline__ void stamp(KParams& pk, int slot) {
  PARAMS;
  if (p.trace && threadIdx.x == 0 && slot < p.trace_n) trace_put(p, slot, slot < 2 * TR_PH ? slot : -1);
}

// Sub-phase stamps: slot trace_n/2 + 8*(phase index) + k, k < 8.  k < 4:
// the phase's own, after its wait; k = 4: its slot tables are built, k = 5:
// it starts waiting, k = 6: the previous phase's arrival is made, its stores
// completed (4 to 6 before the wait, while md_cur_phase still holds the
// previous phase's index).
__shared__ int md_cur_phase;
__device__ __forceinline__ void sub_stamp(KParams& pk, int k) {
  PARAMS;
  if (p.trace && threadIdx.x == 0) {
    const int ph = md_cur_phase, slot = p.trace_n / 2 + 8 * ph + k;
    if (slot < p.trace_n - 1) trace_put(p, slot, ph < TR_PH ? 2 * TR_PH + 8 * ph + k : -1);
  }
}
__device__ __forceinline__ void pre_stamp(KParams& pk, int k) {
  PARAMS;
  if (p.trace && threadIdx.x == 0) {
    const int ph = md_cur_phase + 1, slot = p.trace_n / 2 + 8 * ph + k;
    if (slot < p.trace_n - 1) trace_put(p, slot, ph < TR_PH ? 2 * TR_PH + 8 * ph + k : -1);
  }
}

// Sync point sidx: stamps 2*sidx (work done) and 2*sidx+1 (wait over).
__device__ __forceinline__ void grid_sync(KParams& pk, int& sidx) {
  PARAMS;
  stamp(p, 2 * sidx);
  arrive(p, sidx);
  wait_all(p, sidx);
  stamp(p, 2 * sidx + 1);
  ++sidx;
  if (threadIdx.x == 0) md_cur_phase = sidx;
}

// Split form of a sync point: grid_arrive when this workgroup's work for it is
// done; wait_point once the next phase has issued what it may issue before
// the other workgroups are done (its first weight loads).  idx < 0: no wait
// (the multi-launch step, where the kernel boundary is the barrier).
__device__ __forceinline__ void grid_arrive(KParams& pk, int sidx) {
  PARAMS;
  stamp(p, 2 * sidx);
  arrive(p, sidx);
  pre_stamp(p, 6);
}
// the phase after sync point idx begins (trace stamps only)
__device__ __forceinline__ void enter_phase(KParams& pk, int idx) {
  PARAMS;
  stamp(p, 2 * idx + 1);
  if (threadIdx.x == 0) md_cur_phase = idx + 1;
}
__device__ __forceinline__ void wait_point(KParams& pk, int idx) {
  PARAMS;
  if (idx < 0) return;
  pre_stamp(p, 5);
  wait_all(p, idx);
  enter_phase(p, idx);
}

// clear this WG's share of the other bank (used by the next step)
__device__ void clear_next_bank(KParams& pk) {
  PARAMS;
  unsigned* nb = p.sync + (size_t)(p.bank ^ 1) * p.n_sync * SP_WORDS;
  size_t n = (size_t)p.n_sync * SP_WORDS;
  size_t per = (n + gridDim.x - 1) / gridDim.x;
  size_t a = per * blockIdx.x, e = a + per < n ? a + per : n;
  for (size_t i = a + threadIdx.x; i < e; i += NT) nb[i] = 0u;
}

// Row r of a step: its sequence (cache slot) and position.  Decode: row r is
// sequence r at positions[r].  Verify: every row belongs to sequence 0 and
// row r is the token at positions[0] + r.  Out-of-range positions set the
// device error word and are clamped (the step's outputs are then undefined).
__device__ __forceinline__ int row_seq(KParams& pk, int r) {
  PARAMS; return p.verify ? 0 : r; }
__device__ __forceinline__ int row_pos(KParams& pk, int r) {
  PARAMS;
  int pos = p.verify ? p.positions[0] + r : p.positions[r];
  if (pos < 0 || pos >= p.max_ctx) {
    set_err(p, MDE_POSITION);
    pos = pos < 0 ? 0 : p.max_ctx - 1;
  }
  return pos;
}

// Where position pos of sequence slot s sits in a layer's attention cache:
// its page and the row within the page.  A contiguous cache has one page per
// slot; a paged one looks the page up in the block table (s and pos uniform
// across the wave: one scalar load).  A page id outside the pool sets the
// device error word and reads page 0 instead (the step's outputs are then
// undefined, but no access leaves the cache).
struct KvLoc {
  int page, r;
};
__device__ __forceinline__ KvLoc kv_loc(KParams& pk, int s, int pos) {
  PARAMS;
  KvLoc l;
  if (p.bt == nullptr) {
    l.page = s;
    l.r = pos;
    return l;
  }
  const int idx = __builtin_amdgcn_readfirstlane(s * p.bt_stride + (pos >> p.pg_shift));
  int pg = ((const __attribute__((address_space(4))) int32_t*)(uintptr_t)p.bt)[idx];
  if ((unsigned)pg >= (unsigned)p.n_pages) {
    set_err(p, MDE_PAGE);
    pg = 0;
  }
  l.page = pg;
  l.r = pos & (p.pg_cap - 1);
  return l;
}

// ===================================================================== GEMV
// Y[r][t] = sum_k W[r][k] * U[t][k] for this workgroup's rows of a list of
// matrices (up to MAXMAT per phase: q/k/v, the gate and up of every expert a
// step uses, the down projections of all of them, ...).
//
// Weights are in the tiled layout md_pack_weight writes: 16-row tiles, and
// within a tile one contiguous 1 KB block per 32-column k-step holding the
// matrix-core A operand (lane l: row l%16, columns 8*(l/16)..+7), the block
// ordered as four 256-byte quarters of 4 rows.  A tile's blocks are
// consecutive, so every wave instruction reads 1 KB contiguous and each tile
// is one sequential stream.
//
// U is an activation in hi/lo form, bf16[2][MAXB][K] (part, token, k): the
// B operand (32 k x 16 columns: token t hi at column 2t, lo at 2t+1) is one
// 16-byte load per lane.
//
// Work split: each matrix's rows are cut into 4-row quarters and workgroup w
// owns quarters [Q*w/G, Q*(w+1)/G), so every workgroup streams the same
// number of bytes.  Its quarters are packed four to a "slot" (one
// matrix-core tile whose lanes may read four different matrices), and slots
// are consumed in groups of two that share one B operand: a group never
// mixes inputs, so all its quarters multiply the same U.  The four waves split
// the k-steps of a group and keep GDS k-steps of loads in flight in one
// continuous stream across groups (no pipeline drain between tiles).
//
// The workgroup's LDS.  Phases address it through this symbol (not through a
// pointer argument) so that accesses compile to LDS instructions.  It is a
// static array: functions reach it at a fixed address (dynamic LDS would be
// found through a per-kernel offset table in memory, a load in the stream).
// (the 64-row build takes nearly all of the CU's 160 KB: its epilogue
// staging holds 64 tokens per row)
constexpr size_t MD_SMEM_BYTES = WIDE ? 160 * 1024 - 256 : 130 * 1024;
__shared__ __attribute__((aligned(16))) char md_smem[MD_SMEM_BYTES];

constexpr int CMAX_DEV = 256;    // largest chunk count per (sequence, kv head)
// slots per group (they share every B operand load); even: SwiGLU pairs.
// 4 in the 64-row build: twice the weight bytes per k-step for the same B
// operands (its ring is only GDS = 2 deep)
constexpr int TG = WIDE ? 4 : 2;
// k-steps in flight per wave: 8 (measured: 4 and 8 stream equally fast,
// deeper is slower); fewer in the 64-row build, whose ring holds 8 B
// operands per k-step
constexpr int GDS = WIDE ? 2 : 8;
constexpr int MAXSLOT = 96;      // slots per workgroup and phase
constexpr int MAXGRP = MAXSLOT / TG;
constexpr int MAXMAT = 72;       // matrices per phase
constexpr int STAGE_ROWS = WIDE ? 192 : 768;  // epilogue staging rows per workgroup (of MAXB tokens)
constexpr int IN_ROWS = WIDE ? 96 : 768;       // input staging rows (scratch of the MLA phases)
constexpr int MIN_KS = NW;       // every wave needs a k-step of every group

struct RowSplit {
  int r0, r1;
};
// (N * w fits in 32 bits for every split made here: N <= 2^22 quarters or
// units, w <= G <= 1024.)
__device__ __forceinline__ RowSplit rows_of(int N, int w, int G) {
  RowSplit s;
  s.r0 = (int)((uint32_t)N * (uint32_t)w / (uint32_t)G);
  s.r1 = (int)((uint32_t)N * (uint32_t)(w + 1) / (uint32_t)G);
  return s;
}

// One slot: the lanes of quarter position e read matrix m[e] (index into the
// phase's matrix table), global quarter gq[e] (rows 4*gq .. 4*gq+3).
// gq < 0: an empty quarter (its lanes read the zero block).
struct Slot {
  int8_t m[4];
  int gq[4];
};
struct MatDesc {
  uint64_t w;        // tiled weights
  uint64_t tstride;  // bytes per 16-row tile
  int N;             // rows
  int tag;           // meaning chosen by the phase (expert slot, ...)
};
enum : int { GK_SINGLE = 0, GK_PAIR = 1 };
// A group: slots TG*g .. TG*g + TG-1, which share every B operand load.
// GK_PAIR: slots TG*g + 2j hold gate rows and TG*g + 2j+1 the up rows of the
// same quarters (SwiGLU); GK_SINGLE: independent slots.
struct GroupDesc {
  uint32_t u_off;    // byte offset of U in the workspace
  int KS;            // k-steps (K / 32); U rows are K elements apart
  int kind;
  int pad_;
};

struct GemvSmem {
  float red[2][NW][TG][16][16];  // per-wave partial tiles of a group (one B tile of it), two buffers
                                 // alternating; also reused as [NT][MAXB] scratch after the stream (8-row build)
  Slot slots[MAXSLOT];
  GroupDesc grp[MAXGRP];
  MatDesc mats[MAXMAT];
  int nslots, ngroups, nmats, overflow;
  int wtot[NW];                  // k-steps of every group, per wave
  // epilogue staging: inputs read before the weight stream starts, outputs
  // written after it ends, so the stream itself issues no other memory
  // operation.  Indexed by slot row (slot*16 + row-in-slot) or, in phases
  // that own residual rows, by row - first owned row.
  float in[IN_ROWS][MAXB];
  float out[STAGE_ROWS][MAXB];
  float gain[STAGE_ROWS];
  float inv[MAXB];
};
#define GSM (*reinterpret_cast<GemvSmem*>(md_smem))

// Slot tables of a phase whose work split does not depend on the step's data
// (everything but the routed experts' phases) are the same in every layer:
// the first layer of a launch builds them, later layers copy them back and
// only re-enter the per-layer weight pointers.  They live at the end of the
// static LDS block.
enum : int {
  PL_QKV = 0, PL_OPROJ, PL_GATEUP, PL_DDOWN, PL_LMHEAD, PL_KDA_PROJ, PL_KDA_O, PL_MLA_A, PL_MLA_B, PL_MLA_O, PL_MOE_A,
  NPLAN
};
constexpr int PLAN_SLOTS = 48;
struct SlotPlan {
  int valid, nslots, overflow, pad_;
  int wtot[NW];
  Slot slots[PLAN_SLOTS];
  GroupDesc grp[PLAN_SLOTS / TG];
};
constexpr size_t PLAN_OFF = MD_SMEM_BYTES - NPLAN * sizeof(SlotPlan);
#define PLANS (reinterpret_cast<SlotPlan*>(md_smem + PLAN_OFF))
static_assert(sizeof(Slot) % 4 == 0 && sizeof(GroupDesc) % 4 == 0 && PLAN_OFF % 16 == 0, "plans are copied as words");

// wave-parallel copy of n 32-bit words (wave 0 calls it)
__device__ __forceinline__ void copy_words(void* dst, const void* src, int n) {
  for (int i = __lane_id(); i < n; i += 64) ((int*)dst)[i] = ((const int*)src)[i];
}

// Slot-list builder, run by wave 0 on wave-uniform values (scalar
// arithmetic; every lane writes the same table entries).  Groups are opened
// with begin(U, K, kind); quarters are appended with single() or pair() and
// written straight into the LDS slot table; a group never spans two begin()
// calls.
struct SlotBuilder {
  int ns, fill, pfill, nm;  // slots, quarters in the open slot, pending pairs, matrices (all in registers:
                            // the builder only writes LDS, so its stores pipeline)
  int tot[NW];              // k-steps of the groups so far, per wave
  GroupDesc gd;
  __device__ void new_group() {
    GSM.grp[ns / TG] = gd;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot[w] += (gd.KS - w + NW - 1) / NW;
  }
  __device__ void empty_slot(int si) {
    for (int e = 0; e < 4; ++e) { GSM.slots[si].m[e] = 0; GSM.slots[si].gq[e] = -1; }
  }
  bool ovf;
  int plan;     // cached plan of this phase (built or replayed), or -1
  bool replay;  // the plan is valid: only matrices are entered
  __device__ void start(int plan_id = -1) {
    plan = plan_id;
    replay = plan_id >= 0 && __builtin_amdgcn_readfirstlane(PLANS[plan_id].valid) != 0;
    if (replay) {  // the cached tables; begin() enters this use's input
      SlotPlan& P = PLANS[plan_id];
      const int pns = __builtin_amdgcn_readfirstlane(P.nslots);
      copy_words(GSM.slots, P.slots, pns * (int)(sizeof(Slot) / 4));
      copy_words(GSM.grp, P.grp, (pns / TG) * (int)(sizeof(GroupDesc) / 4));
    }
    ns = 0; fill = 0; pfill = 0; nm = 0; ovf = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot[w] = 0;
    gd.u_off = 0; gd.KS = MIN_KS; gd.kind = GK_SINGLE; gd.pad_ = 0;
  }
  // Matrices of the chosen experts, one lane per matrix: for expert j of
  // U, its weights RSM.ex[j][c0 .. c0+nc-1] (N x K), entered at m0 + nc*j + c;
  // tag j when tag_j, else 0.  Returns m0.
  template <int NC>
  __device__ int expert_mats(const uint16_t* const (*ex)[3], int nu, int c0, int N, int K, bool tag_j) {
    const int m0 = nm;
    if (m0 + NC * nu > MAXMAT) { ovf = true; return 0; }
    for (int i = __lane_id(); i < NC * nu; i += 64) {
      const int j = i / NC, c = i - j * NC;
      MatDesc d;
      d.w = (uint64_t)ex[j][c0 + c]; d.tstride = (uint64_t)(K >> 5) * 1024u; d.N = N; d.tag = tag_j ? j : 0;
      GSM.mats[m0 + i] = d;
    }
    nm = m0 + NC * nu;
    return m0;
  }
  __device__ int mat(const void* w, int N, int K, int tag) {
    int i = nm;
    if (i >= MAXMAT) { ovf = true; return 0; }
    MatDesc d;
    d.w = (uint64_t)w; d.tstride = (uint64_t)(K >> 5) * 1024u; d.N = N; d.tag = tag;
    GSM.mats[i] = d;
    nm = i + 1;
    return i;
  }
  // open slot ns (and its group when ns is even)
  __device__ bool open_slot() {
    if (ns >= MAXSLOT) { ovf = true; return false; }
    empty_slot(ns);
    if (ns % TG == 0) new_group();
    return true;
  }
  __device__ void flush() {
    if (fill) { ++ns; fill = 0; }
  }
  __device__ void pflush() {
    if (pfill) { ns += 2; pfill = 0; }
  }
  __device__ void close() {
    flush();
    pflush();
    while (ns % TG) {
      if (!open_slot()) break;
      ++ns;
    }
  }
  __device__ void begin(uint32_t u_off, int K, int kind) {
    if (replay) {  // a replayed plan's groups all take this use's input
      const int ng = __builtin_amdgcn_readfirstlane(PLANS[plan].nslots) / TG;
      for (int i = __lane_id(); i < ng; i += 64) GSM.grp[i].u_off = u_off;
      return;
    }
    close();
    if (K < 32 * MIN_KS || (K & 31)) ovf = true;
    gd.u_off = u_off; gd.KS = K >> 5; gd.kind = kind; gd.pad_ = 0;
  }
  __device__ void single(int m, int gq) {
    if (fill == 0 && !open_slot()) return;
    GSM.slots[ns].m[fill] = (int8_t)m;
    GSM.slots[ns].gq[fill] = gq;
    if (++fill == 4) flush();
  }
  __device__ void pair(int mg, int mu, int gq) {
    if (pfill == 0) {
      if (ns + 1 >= MAXSLOT) { ovf = true; return; }
      empty_slot(ns);
      empty_slot(ns + 1);
      if (ns % TG == 0) new_group();
    }
    GSM.slots[ns].m[pfill] = (int8_t)mg;
    GSM.slots[ns].gq[pfill] = gq;
    GSM.slots[ns + 1].m[pfill] = (int8_t)mu;
    GSM.slots[ns + 1].gq[pfill] = gq;
    if (++pfill == 4) pflush();
  }
  // this workgroup's quarters of an N-row matrix (the split of the last N is kept)
  int lastN = -1;
  RowSplit lastq;
  __device__ RowSplit quarters(int N) {
    if (N != lastN) { lastq = rows_of((N + 3) >> 2, blockIdx.x, gridDim.x); lastN = N; }
    return lastq;
  }
  // Whole slots of a run, one lane per slot: slots ns .. ns+n-1 hold
  // quarters gq0 + 4k .. +3 of matrix m (and, for pairs, slots ns+2k /
  // ns+2k+1 the gate / up quarters of the same rows).  Opens their groups.
  __device__ void bulk(int m, int mu, int gq0, int n, bool pairs) {
    const int per = pairs ? 2 : 1;
    if (ns + per * n > MAXSLOT) { ovf = true; return; }
    for (int k = __lane_id(); k < n; k += 64) {
      const int si = ns + per * k;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        GSM.slots[si].m[e] = (int8_t)m;
        GSM.slots[si].gq[e] = gq0 + 4 * k + e;
        if (pairs) {
          GSM.slots[si + 1].m[e] = (int8_t)mu;
          GSM.slots[si + 1].gq[e] = gq0 + 4 * k + e;
        }
      }
      if (si % TG == 0) GSM.grp[si / TG] = gd;
    }
    // groups opened: slot indices in [ns, ns + per*n) that are multiples of TG
    const int first = (ns + TG - 1) / TG, last = (ns + per * n - 1) / TG;
    const int ng = last - first + 1;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot[w] += ng * ((gd.KS - w + NW - 1) / NW);
    ns += per * n;
  }
  __device__ void singles_of(int m, int N) { singles_in(m, quarters(N)); }
  __device__ void pairs_of(int mg, int mu, int N) { pairs_in(mg, mu, quarters(N)); }
  // quarters q.r0 .. q.r1-1 of matrix m (of gate/up matrices mg, mu)
  __device__ void singles_in(int m, RowSplit q) {
    if (replay) return;
    int gq = q.r0;
    while (fill != 0 && gq < q.r1) single(m, gq++);
    if (fill == 0 && q.r1 - gq >= 4) {
      const int n = (q.r1 - gq) >> 2;
      bulk(m, 0, gq, n, false);
      gq += 4 * n;
    }
    for (; gq < q.r1; ++gq) single(m, gq);
  }
  __device__ void pairs_in(int mg, int mu, RowSplit q) {
    if (replay) return;
    int gq = q.r0;
    while (pfill != 0 && gq < q.r1) pair(mg, mu, gq++);
    if (pfill == 0 && q.r1 - gq >= 4) {
      const int n = (q.r1 - gq) >> 2;
      bulk(mg, mu, gq, n, true);
      gq += 4 * n;
    }
    for (; gq < q.r1; ++gq) pair(mg, mu, gq);
  }
  // Gate/up pairs of nu experts entered as matrices m0 + 2j (gate) and
  // m0 + 2j + 1 (up), all N rows: this workgroup's quarters of each, expert
  // after expert, four to a pair of slots (one lane per quarter); the last
  // pair of slots is closed.  Same tables as pairs_of expert by expert.
  __device__ void expert_pairs(int m0, int nu, int N) {
    if (replay) return;
    pflush();
    RowSplit q = quarters(N);
    const int npq = q.r1 - q.r0, E = nu * npq, P = (E + 3) >> 2;
    if (ns + 2 * P > MAXSLOT) { ovf = true; return; }
    // When every workgroup owns the same number of quarters, workgroups 2k
    // and 2k+1 trade places on every other expert: the two halves of a tile's
    // blocks then alternate between them instead of one of them always
    // reading the first half (measured: with a fixed order, the workgroups
    // of one parity streamed the routed experts up to 20% slower at batch 8).
    const int Q = (N + 3) >> 2, G = gridDim.x, wx = blockIdx.x ^ 1;
    const bool trade = Q % G == 0 && wx < G;
    const int r0x = trade ? rows_of(Q, wx, G).r0 : q.r0;
    for (int i = __lane_id(); i < 4 * P; i += 64) {
      const int ps = i >> 2, e = i & 3, si = ns + 2 * ps;
      const bool v = i < E;
      const int j = v ? i / npq : 0;
      const int gq = v ? ((j & 1) ? r0x : q.r0) + (i - j * npq) : -1;
      GSM.slots[si].m[e] = (int8_t)(v ? m0 + 2 * j : 0);
      GSM.slots[si].gq[e] = gq;
      GSM.slots[si + 1].m[e] = (int8_t)(v ? m0 + 2 * j + 1 : 0);
      GSM.slots[si + 1].gq[e] = gq;
      if (e == 0 && si % TG == 0) GSM.grp[si / TG] = gd;
    }
    if (P > 0) {
      const int ng = (ns + 2 * P - 1) / TG - (ns + TG - 1) / TG + 1;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot[w] += ng * ((gd.KS - w + NW - 1) / NW);
    }
    ns += 2 * P;
  }
  // Singles of nu experts entered as matrices m0 + j, all N rows, expert j
  // reading U at u0 + j * ustride (K columns): each expert's quarters fill
  // whole groups of their own (one lane per slot).  Same tables as begin()
  // plus singles_of expert by expert.
  __device__ void expert_singles(int m0, int nu, int N, uint32_t u0, uint32_t ustride, int K) {
    if (replay) return;
    close();
    if (K < 32 * MIN_KS || (K & 31)) ovf = true;
    RowSplit q = quarters(N);
    const int nq = q.r1 - q.r0;
    if (nq <= 0 || nu <= 0) return;
    const int S = ((nq + 3) / 4 + TG - 1) / TG * TG;  // slots per expert
    if (ns + nu * S > MAXSLOT) { ovf = true; return; }
    for (int i = __lane_id(); i < nu * S; i += 64) {
      const int j = i / S, k = i - j * S, si = ns + i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int qi = 4 * k + e;
        const bool v = qi < nq;
        GSM.slots[si].m[e] = (int8_t)(v ? m0 + j : 0);
        GSM.slots[si].gq[e] = v ? q.r0 + qi : -1;
      }
      if (k % TG == 0) {
        GroupDesc g;
        g.u_off = u0 + (uint32_t)j * ustride; g.KS = K >> 5; g.kind = GK_SINGLE; g.pad_ = 0;
        GSM.grp[si / TG] = g;
      }
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) tot[w] += nu * (S / TG) * (((K >> 5) - w + NW - 1) / NW);
    ns += nu * S;
  }
  __device__ void finish() {
    if (replay) {
      SlotPlan& P = PLANS[plan];
      ns = __builtin_amdgcn_readfirstlane(P.nslots);
      ovf = ovf || __builtin_amdgcn_readfirstlane(P.overflow) != 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot[w] = __builtin_amdgcn_readfirstlane(P.wtot[w]);
    } else {
      close();
    }
    GSM.nslots = ns;
    GSM.ngroups = ns / TG;
    GSM.nmats = nm;
    GSM.overflow = ovf ? 1 : 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) GSM.wtot[w] = tot[w];
    // a plan is kept only when all its groups read one input (replays give
    // them this use's input, which differs from layer to layer)
    bool one_u = true;
    for (int i = __lane_id(); i < ns / TG; i += 64) one_u = one_u && GSM.grp[i].u_off == GSM.grp[0].u_off;
    one_u = __all(one_u);
    if (!replay && plan >= 0 && !ovf && ns <= PLAN_SLOTS && one_u) {
      SlotPlan& P = PLANS[plan];
      copy_words(P.slots, GSM.slots, ns * (int)(sizeof(Slot) / 4));
      copy_words(P.grp, GSM.grp, (ns / TG) * (int)(sizeof(GroupDesc) / 4));
      P.nslots = ns;
      P.overflow = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) P.wtot[w] = tot[w];
      P.valid = 1;
    }
  }
};

// Per-lane source of one slot.
__device__ __forceinline__ void slot_src(int si, int lq, uint32_t lchunk, int wv, uint64_t zero_addr, uint64_t& pa,
                                         uint32_t& pstep) {
  int gq = GSM.slots[si].gq[lq];
  int m = GSM.slots[si].m[lq];
  if (gq < 0) {
    // An empty quarter's lanes read the bytes of a filled quarter of the same
    // k-step: the slot's first (quarters fill in order), or, for an empty
    // slot, the first of its group (never empty).  Its rows are never
    // stored, and the lines are those its instruction or the group's other
    // instruction reads anyway: no extra traffic, and no single line that
    // every workgroup's empty lanes would read (a hot cache channel).
    const int s2 = GSM.slots[si].gq[0] >= 0 ? si : si - si % TG;
    gq = GSM.slots[s2].gq[0];
    m = GSM.slots[s2].m[0];
  }
  bool lv = gq >= 0;
  uint64_t W = GSM.mats[m].w, ts = GSM.mats[m].tstride;
  pa = lv ? W + (uint64_t)(gq >> 2) * ts + (uint64_t)((gq & 3) * 256) + lchunk + (uint64_t)wv * 1024u : zero_addr;
  pstep = lv ? (uint32_t)(NW * 1024) : 0u;
}

// Output (token t of the tile, row rr of slot TG*g + i) of a finished
// group: the four waves' partials (8-row build: hi and lo columns) summed in
// a fixed order.
__device__ __forceinline__ float gy(int rb, int i, int rr, int t) {
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if constexpr (WIDE) s += GSM.red[rb][w][i][rr][t];
    else s += GSM.red[rb][w][i][rr][2 * t] + GSM.red[rb][w][i][rr][2 * t + 1];
  }
  return s;
}

__device__ __forceinline__ int group_nks(int g, int wv) {
  int KS = __builtin_amdgcn_readfirstlane(GSM.grp[g].KS);
  return (KS - wv + NW - 1) / NW;
}

// 1/rms per token from the partial sums of squares of every workgroup (this
// thread holds those of workgroups tid and tid + NT), summed in a fixed
// order: identical in every workgroup.
__device__ __forceinline__ void inv_finish(KParams& pk, float* inv, int n_feat, i32x4 a0, i32x4 b0, i32x4 a1, i32x4 b1) {
  PARAMS;
  float* stage = (float*)(md_smem + sizeof(GemvSmem));  // [2*NT][MAXB]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    stage[threadIdx.x * MAXB + k] = __int_as_float(a0[k]);
    stage[threadIdx.x * MAXB + 4 + k] = __int_as_float(b0[k]);
    stage[(threadIdx.x + NT) * MAXB + k] = __int_as_float(a1[k]);
    stage[(threadIdx.x + NT) * MAXB + 4 + k] = __int_as_float(b1[k]);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    int t = 2 * wv + k;
    float sum = 0.f;
    for (int g = lane; g < (int)gridDim.x; g += 64) sum += stage[g * MAXB + t];
    sum = wave_sum(sum);
    if (lane == 0) inv[t] = 1.0f / sqrtf(sum / (float)n_feat + p.eps);
  }
  __syncthreads();
}

// The per-wave weight stream over a range of GSM's group list.  gemv_begin
// issues the weight loads of the first GDS k-steps (they depend on no other
// workgroup, so a phase issues them before it waits at its sync point);
// gemv_run then issues the matching activation (B operand) loads and streams
// the rest, GDS k-steps ahead of the matrix cores, continuously across
// groups.  Each weight block is multiplied by every B tile of the step (NB
// tiles, NPART operands each), so a step's weights are read once whatever
// the batch.
template <int NB>
struct GemvStream {
  int wv, lq, tok, part, B, ngroups, total;
  int gfirst;           // the range's first group (ig runs ahead of the matrix cores)
  uint32_t lchunk, lane16;
  uint64_t zero_addr;
  rsrc_t urs;
  int ig, is, nks_i;
  uint32_t boff;        // B operand offset of this lane's row in tile 0 (OOB: a token past B)
  uint32_t btile;       // bytes between the B tiles of the group
  uint32_t bpart;       // bytes between a tile's operands (the high parts and the rests)
  uint32_t bmask;       // bit j: this lane's token of tile j is a row of the step
  uint64_t pa[TG];
  uint32_t ps[TG];
  i32x4 ra[GDS][TG];
  i32x4 rb[GDS][NB * NPART];
  uint32_t bo[GDS];
  uint32_t btd[GDS], bpd[GDS];  // btile and bpart of the k-step's group (the first GDS k-steps may span groups)
};

template <int NB>
__device__ __forceinline__ void gs_group(GemvStream<NB>& s, int g) {
  const int ks = __builtin_amdgcn_readfirstlane(GSM.grp[g].KS);
  const uint32_t uo = __builtin_amdgcn_readfirstlane(GSM.grp[g].u_off);
  s.nks_i = (ks - s.wv + NW - 1) / NW;
  s.boff = uo + (uint32_t)((s.part * MAXB + s.tok) * ks * 32) * 2u + s.lane16;
  s.btile = (uint32_t)(TTILE * ks * 32) * 2u;
  s.bpart = (uint32_t)(MAXB * ks * 32) * 2u;
#pragma unroll
  for (int i = 0; i < TG; ++i) slot_src(TG * g + i, s.lq, s.lchunk, s.wv, s.zero_addr, s.pa[i], s.ps[i]);
}

// Weight loads of one k-step (ring entry d); past the last group they read
// the zero block.  Records the k-step's B-operand offset (tile 0).
template <int NB>
__device__ __forceinline__ void gs_issue_a(GemvStream<NB>& s, int d) {
  const bool ok = s.ig < s.ngroups;
#pragma unroll
  for (int i = 0; i < TG; ++i) {
    s.ra[d][i] = __builtin_nontemporal_load((const __attribute__((address_space(1))) i32x4*)(ok ? s.pa[i] : s.zero_addr));
    s.pa[i] += s.ps[i];
  }
  s.bo[d] = ok ? s.boff + (uint32_t)(s.is * NW + s.wv) * 64u : OOB;
  s.btd[d] = s.btile;
  s.bpd[d] = s.bpart;
  if (++s.is == s.nks_i) {
    s.is = 0;
    ++s.ig;
    if (s.ig < s.ngroups) gs_group(s, s.ig);
  }
}
// Activation (B operand) loads of one k-step, every tile: cache policy sc0
// (not kept in the CU's L1, served by the XCD's L2).  Every activation buffer
// is used once per launch (one buffer per use, see u_at), so the L2 never
// holds an older copy of it: the first read in an XCD fetches what the
// producers wrote through to memory before the sync point, later reads in
// that XCD hit.  (On a buffer reused within a launch such loads would return
// stale lines: measured.)  Lanes whose token of a tile is past the step's
// rows read nothing (offset past the resource: zeros).
template <int NB>
__device__ __forceinline__ void gs_issue_b(GemvStream<NB>& s, int d, uint32_t bo, uint32_t btile, uint32_t bpart) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const uint32_t o = (bo != OOB && ((s.bmask >> j) & 1u)) ? bo + (uint32_t)j * btile : OOB;
#pragma unroll
    for (int q = 0; q < NPART; ++q) s.rb[d][j * NPART + q] = ld_x4<CP_SC0>(s.urs, o == OOB ? OOB : o + (uint32_t)q * bpart);
  }
}

// Steady state: weight and activation loads of one k-step, then the group
// switch (loads before the branch, so the compiler sees one load sequence).
template <int NB>
__device__ __forceinline__ void gs_issue(GemvStream<NB>& s, int d) {
  const bool ok = s.ig < s.ngroups;
#pragma unroll
  for (int i = 0; i < TG; ++i) {
    s.ra[d][i] = __builtin_nontemporal_load((const __attribute__((address_space(1))) i32x4*)(ok ? s.pa[i] : s.zero_addr));
    s.pa[i] += s.ps[i];
  }
  gs_issue_b(s, d, ok ? s.boff + (uint32_t)(s.is * NW + s.wv) * 64u : OOB, s.btile, s.bpart);
  if (++s.is == s.nks_i) {
    s.is = 0;
    ++s.ig;
    if (s.ig < s.ngroups) gs_group(s, s.ig);
  }
}

// Groups [g0, g1) of the tables (one staging pass).
template <int NB>
__device__ __forceinline__ void gemv_begin(GemvStream<NB>& s, const uint8_t* ws, uint32_t ws_bytes, uint32_t off_zero,
                                           int B, int g0, int g1) {
  const int lane = threadIdx.x & 63;
  s.wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  s.ngroups = g1;
  if (g0 == 0 && g1 == __builtin_amdgcn_readfirstlane(GSM.ngroups)) {
    s.total = __builtin_amdgcn_readfirstlane(GSM.wtot[s.wv]);
  } else {
    int t = 0;
    for (int g = g0; g < g1; ++g) t += group_nks(g, s.wv);
    s.total = t;
  }
  s.urs = make_rsrc_u(ws, ws_bytes);
  s.lq = (lane & 15) >> 2;
  s.lchunk = (uint32_t)(((lane >> 4) * 4 + (lane & 3)) * 16);
  s.lane16 = (uint32_t)(lane >> 4) * 16u;
  // B column lane & 15: 8-row build token (lane & 15) / 2, hi or lo by the
  // lane's parity; 64-row build token lane & 15 of the tile (hi and lo are
  // separate operands)
  s.tok = WIDE ? (lane & 15) : (lane & 15) >> 1;
  s.part = WIDE ? 0 : lane & 1;
  s.B = B;
  s.bmask = 0;
#pragma unroll
  for (int j = 0; j < NB; ++j) s.bmask |= (TTILE * j + s.tok < B) ? (1u << j) : 0u;
  s.zero_addr = (uint64_t)(ws + off_zero);
  s.ig = g0;
  s.gfirst = g0;
  s.is = 0;
  s.nks_i = 1;
  s.boff = OOB;
  s.btile = 0;
  s.bpart = 0;
#pragma unroll
  for (int i = 0; i < TG; ++i) {
    s.pa[i] = s.zero_addr;
    s.ps[i] = 0;
  }
  if (g0 < g1) gs_group(s, g0);
#pragma unroll
  for (int d = 0; d < GDS; ++d) gs_issue_a(s, d);
}

// 1/rms of every token of a 64-row step (the wide build): wave w sums
// tokens 16w .. 16w+15 over all workgroups' partials, lane l taking
// workgroups l, l + 64, ... in order, then a fixed-order wave reduction (the
// same order as inv_finish).
__device__ __forceinline__ void inv_finish_wide(KParams& pk, float* inv, int n_feat, uint32_t inv_off, int B) {
  PARAMS;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  const int G = gridDim.x;
  constexpr int TPW = MAXB / NW;  // tokens per wave
  float acc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) acc[k] = 0.f;
  for (int g = lane; g < G; g += 64) {
    float v[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) v[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        r, (TPW * wv + k < B) ? inv_off + (uint32_t)(g * MAXB + TPW * wv + k) * 4u : OOB, 0, CP_SC0));
#pragma unroll
    for (int k = 0; k < TPW; ++k) acc[k] += v[k];
  }
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const float sum = wave_sum(acc[k]);
    if (lane == 0) inv[TPW * wv + k] = 1.0f / sqrtf(sum / (float)n_feat + p.eps);
  }
  __syncthreads();
}

// Stream everything.  After each finished group g, epi(g, rb, j) reads the
// outputs of its B tile j with gy(rb, i, row-in-slot, token) (LDS only).
// One barrier per tile of a group: the partials of consecutive tiles go to
// alternating buffers.  inv_n > 0: first fill GSM.inv with 1/rms over inv_n
// features from the per-workgroup partial sums of squares at inv_off.  Those
// loads are issued before the ring's activation loads, so waiting for them
// never waits for the ring.
template <int NB, class Epi>
__device__ __forceinline__ void gemv_run(KParams& pk, GemvStream<NB>& s, int inv_n, uint32_t inv_off, Epi epi) {
  PARAMS;
  static_assert(TG % 2 == 0, "SwiGLU groups hold gate/up slot pairs");
  const int lane = threadIdx.x & 63;
  if constexpr (!WIDE) {
    i32x4 ia0, ib0, ia1, ib1;
    if (inv_n > 0) {
      const rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
      const int g0 = threadIdx.x, g1 = threadIdx.x + NT;
      const int G = gridDim.x;
      ia0 = ld_x4<CP_SC0>(r, g0 < G ? inv_off + (uint32_t)(g0 * MAXB) * 4u : OOB);
      ib0 = ld_x4<CP_SC0>(r, g0 < G ? inv_off + (uint32_t)(g0 * MAXB + 4) * 4u : OOB);
      ia1 = ld_x4<CP_SC0>(r, g1 < G ? inv_off + (uint32_t)(g1 * MAXB) * 4u : OOB);
      ib1 = ld_x4<CP_SC0>(r, g1 < G ? inv_off + (uint32_t)(g1 * MAXB + 4) * 4u : OOB);
    }
#pragma unroll
    for (int d = 0; d < GDS; ++d) gs_issue_b(s, d, s.bo[d], s.btd[d], s.bpd[d]);
    if (inv_n > 0) inv_finish(p, GSM.inv, inv_n, ia0, ib0, ia1, ib1);
  } else {
    if (inv_n > 0) inv_finish_wide(p, GSM.inv, inv_n, inv_off, s.B);
#pragma unroll
    for (int d = 0; d < GDS; ++d) gs_issue_b(s, d, s.bo[d], s.btd[d], s.bpd[d]);
  }
  f32x4 acc[TG][NB];
#pragma unroll
  for (int i = 0; i < TG; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int cg = s.gfirst, cs = 0, rbuf = 0;
  int nks_c = cg < s.ngroups ? group_nks(cg, s.wv) : 1;
  // One k-step: matrix-core work on ring entry d, its refill, and at the end
  // of a group its tiles' partials to LDS, one barrier each, and the epilogue.
#define GEMV_STEP(J0, D)                                                                                        \
  {                                                                                                             \
    _Pragma("unroll") for (int j = 0; j < NB; ++j) _Pragma("unroll") for (int q = 0; q < NPART; ++q) {          \
      bf16x8 bop = __builtin_bit_cast(bf16x8, s.rb[D][j * NPART + q]);                                          \
      _Pragma("unroll") for (int i = 0; i < TG; ++i) acc[i][j] =                                                \
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, s.ra[D][i]), bop, acc[i][j], 0, 0, 0); \
    }                                                                                                           \
    gs_issue(s, D);                                                                                             \
    if ((J0) + (D) < s.total) {                                                                                 \
      if (++cs == nks_c) {                                                                                      \
        cs = 0;                                                                                                 \
        _Pragma("unroll") for (int j = 0; j < NB; ++j) {                                                        \
          if (TTILE * j < s.B) {                                                                                \
            _Pragma("unroll") for (int i = 0; i < TG; ++i) _Pragma("unroll") for (int r = 0; r < 4; ++r)        \
                GSM.red[rbuf][s.wv][i][4 * (lane >> 4) + r][lane & 15] = acc[i][j][r];                          \
            __syncthreads();                                                                                    \
            _Pragma("unroll") for (int i = 0; i < TG; ++i) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};               \
            epi(cg, rbuf, j);                                                                                   \
            rbuf ^= 1;                                                                                          \
          }                                                                                                     \
        }                                                                                                       \
        ++cg;                                                                                                   \
        if (cg < s.ngroups) nks_c = group_nks(cg, s.wv);                                                        \
      }                                                                                                         \
    }                                                                                                           \
  }
  // The first round is peeled: its ring was filled in two parts (weights
  // before the sync point, activations after), and a loop entered from that
  // state would get the first round's conservative load waits in every round.
  // The bodies are unconditional: steps past the end read the zero block and
  // add nothing.  (A guarded body would make the compiler assume the later
  // loads of the previous round may be missing and wait for all of them.)
#pragma unroll
  for (int d = 0; d < GDS; ++d) GEMV_STEP(0, d)
  for (int j0 = GDS; j0 < s.total; j0 += GDS) {
#pragma unroll
    for (int d = 0; d < GDS; ++d) GEMV_STEP(j0, d)
  }
#undef GEMV_STEP
  __syncthreads();
}

// Row rr (0..15) of a slot: matrix and global row; false for an empty
// quarter or a row past the matrix end.
__device__ __forceinline__ bool slot_row(int si, int rr, int& m, int& row) {
  int gq = GSM.slots[si].gq[rr >> 2];
  if (gq < 0) return false;
  m = GSM.slots[si].m[rr >> 2];
  row = gq * 4 + (rr & 3);
  return row < GSM.mats[m].N;
}

// Post-stream writer over 4-row quarters, for slots [s0, s1) of a staging
// pass: fn(si, sr0, t, m, row0, n) for every quarter of slot si that holds
// rows (rows row0 .. row0+n-1 of matrix m, n <= 4, staged at rows sr0 ..
// sr0+n-1) and every token t < B.  Consecutive threads take consecutive
// quarters of one token, so their stores are consecutive in memory.
template <class F>
__device__ __forceinline__ void for_quarters(int s0, int s1, int B, F fn) {
  const int nq = (s1 - s0) * 4;
  for (int e = threadIdx.x; e < nq * B; e += NT) {
    const int sq = e % nq, t = e / nq;
    const int si = s0 + (sq >> 2), qq = sq & 3;
    const int gq = GSM.slots[si].gq[qq];
    if (gq < 0) continue;
    const int m = GSM.slots[si].m[qq];
    const int row0 = gq * 4, n = GSM.mats[m].N - row0;
    if (n <= 0) continue;
    fn(si, 4 * sq, t, m, row0, n < 4 ? n : 4);
  }
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

// Finish slot building; on overflow (more slots, matrices or staging rows
// than the LDS tables hold) report it and make the phase compute nothing.
// stage_rows < 0: the phase stages by slot row (16 per slot).
__device__ __forceinline__ bool builder_done(KParams& pk, SlotBuilder& sb, int stage_rows) {
  PARAMS;
  if (threadIdx.x < 64) {
    sb.finish();
    // (slot-staged phases of the 64-row build run in staging passes)
    const bool ovf = sb.ovf || (stage_rows < 0 ? (WIDE ? 0 : sb.ns * 16) : stage_rows) > STAGE_ROWS;
    if (ovf) {
      if (threadIdx.x == 0) set_err(p, MDE_CAPACITY);
      GSM.overflow = 1;
      GSM.nslots = 0;
      GSM.ngroups = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) GSM.wtot[w] = 0;
    }
  }
  __syncthreads();
  pre_stamp(p, 4);
  return GSM.ngroups > 0;
}


// ===================================================================== phases
// The weight-streaming phases.  8-row build: functions of their own (one copy
// each, the stream function called from them).  64-row build: inlined into
// the kernel, because as functions they must save every callee-saved vector
// register they touch, which there goes to scratch memory (there are no free
// accumulation registers to park them in) at every phase of every layer.
#if MD_MAXB == 8
#define MD_PHASE_FN __device__ __noinline__
#else
#define MD_PHASE_FN __device__ __forceinline__
#endif

// Write U[part][t][k] = hilo(v) for one element.
__device__ __forceinline__ void put_hilo(rsrc_t r, uint32_t u_off, int K, int t, int k, float v) {
  uint16_t hi, lo;
  split_hilo(v, hi, lo);
  st_u16(r, u_off + (uint32_t)((0 * MAXB + t) * K + k) * 2u, hi);
  st_u16(r, u_off + (uint32_t)((1 * MAXB + t) * K + k) * 2u, lo);
}
// The same for elements k0 .. k0+n-1 (n <= 4; k0 a multiple of 4): one
// 8-byte store per part when n = 4.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void put_hilo4(rsrc_t r, uint32_t u_off, int K, int t, int k0, const float (&v)[4], int n) {
  if (n == 4) {
    uint16_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_hilo(v[i], h[i], l[i]);
    const u32x2 hv = {(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    const u32x2 lv = {(uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
    __builtin_amdgcn_raw_buffer_store_b64(hv, r, u_off + (uint32_t)((0 * MAXB + t) * K + k0) * 2u, 0, CP_SC1);
    __builtin_amdgcn_raw_buffer_store_b64(lv, r, u_off + (uint32_t)((1 * MAXB + t) * K + k0) * 2u, 0, CP_SC1);
  } else {
    for (int i = 0; i < n; ++i) put_hilo(r, u_off, K, t, k0 + i, v[i]);
  }
}

// This workgroup's sum of squares of x per token (partials [NT][MAXB] in
// the reduction scratch, one per thread) -> ssq[w][t]: wave sums, then the
// four waves in order (a fixed order: deterministic).
__device__ __forceinline__ void store_ssq(KParams& pk, rsrc_t r, float* part, uint32_t off_ssq) {
  PARAMS;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float* wsum = part + NT * MAXB;  // [NW][MAXB]
#pragma unroll
  for (int t = 0; t < MAXB; ++t) {
    float v = wave_sum(part[threadIdx.x * MAXB + t]);
    if (lane == 0) wsum[wv * MAXB + t] = v;
  }
  __syncthreads();
  if (threadIdx.x < MAXB) {
    const int t = threadIdx.x;
    float a = wsum[t] + wsum[MAXB + t] + wsum[2 * MAXB + t] + wsum[3 * MAXB + t];
    st_f32(r, off_ssq + (uint32_t)(blockIdx.x * MAXB + t) * 4u, a);
  }
}

// The same for the 64-row build: thread tid holds the partial of token
// tid % 64 over its rows (acc); the four waves' partials are added in order.
__device__ __forceinline__ void store_ssq_wide(KParams& pk, rsrc_t r, float acc, uint32_t off_ssq) {
  float* part = (float*)GSM.red;  // [NT]
  __syncthreads();
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < MAXB) {
    const int t = threadIdx.x;
    const float a = part[t] + part[64 + t] + part[128 + t] + part[192 + t];
    st_f32(r, off_ssq + (uint32_t)(blockIdx.x * MAXB + t) * 4u, a);
  }
}

// --- embedding: x[t] = E[tok_t] on this WG's hidden rows
__device__ __noinline__ void phase_embed(KParams& pk) {
  PARAMS;
  RowSplit s = owned_rows(p.H, blockIdx.x, gridDim.x);
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  const uint16_t* g = p.layers[0].attn_norm;
  auto elem = [&](int t, int i) -> float {
    int tok = p.tokens[t];
    if (tok < 0 || tok >= p.V) {
      set_err(p, MDE_TOKEN);
      tok = tok < 0 ? 0 : p.V - 1;
    }
    float x = bf16_f32(p.embed[(size_t)tok * p.H + i]);
    p.x[t * p.H + i] = x;
    put_hilo(r, u_at(p, 0), p.H, t, i, bf16_f32(g[i]) * x);
    return x * x;
  };
  if constexpr (WIDE) {
    float acc = 0.f;
    const int t = threadIdx.x & 63;
    if (t < p.B)
      for (int i = s.r0 + (threadIdx.x >> 6); i < s.r1; i += NT / 64) acc += elem(t, i);
    store_ssq_wide(p, r, acc, ssq_at(p, 0));
  } else {
    float* part = (float*)md_smem;  // [NT][MAXB]
    for (int t = 0; t < MAXB; ++t) part[threadIdx.x * MAXB + t] = 0.f;
    for (int e = threadIdx.x; e < (s.r1 - s.r0) * p.B; e += NT) {
      int t = e / (s.r1 - s.r0), i = s.r0 + e % (s.r1 - s.r0);
      part[threadIdx.x * MAXB + t] += elem(t, i);
    }
    store_ssq(p, r, part, ssq_at(p, 0));
  }
}

// Router logit entries: {f32 logit, u32 tag}, tag = 2 (step_seq * n_layers
// + layer) + 1 (odd: a cleared entry never matches).  One 8-byte atomic store
// each, so a reader never sees a logit with another entry's tag.
__device__ __forceinline__ uint32_t rl_tag(KParams& pk, int layer) {
  PARAMS;
  return ((p.step_seq * (uint32_t)p.n_layers + (uint32_t)layer) << 1) | 1u;
}
__device__ __forceinline__ uint64_t* rl_entry(KParams& pk, int t, int e) {
  PARAMS;
  return (uint64_t*)(p.ws + p.off_rl + (size_t)(t * p.n_experts + e) * 8u);
}
__device__ __forceinline__ void put_logit(KParams& pk, int layer, int t, int e, float v) {
  PARAMS;
  const uint64_t x = (uint64_t)__float_as_uint(v) | ((uint64_t)rl_tag(p, layer) << 32);
  __hip_atomic_store(rl_entry(p, t, e), x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The entries a routing wave reads: tokens wv, wv + NW, ... (lane = expert).
constexpr int RTPW = MAXB / NW;
struct RouteIn {
  uint64_t v[RTPW];
};
__device__ __forceinline__ void route_load(KParams& pk, RouteIn& in) {
  PARAMS;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < RTPW; ++i) {
    const int t = wv + NW * i;
    in.v[i] = (t < p.B && lane < p.n_experts)
                  ? __hip_atomic_load(rl_entry(p, t, lane), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                  : 0ull;
  }
}

// ------------------------------------------------------------ shared stream
// Every weight-streaming phase runs through gemv_phase: one copy of the
// stream loop and of the group epilogue, shared by all of them, so that the
// code stays in the instruction cache from phase to phase and layer to layer.
enum : int { EPI_BY_KIND = 0, EPI_RESIDUAL = 1 };

// Epilogue of finished group g (the waves' partials in GSM.red[rb]).
// EPI_BY_KIND: a GK_SINGLE group stores y * inv_rms per slot row, a GK_PAIR
// group silu(inv*gate) * (inv*up) at the gate slots' rows; EPI_RESIDUAL adds
// y to the owned residual rows staged at GSM.out[row - r0].
// (B tile j of the group: tokens TTILE*j .. TTILE*(j+1) - 1, those below B; slot
// rows are staged relative to s0, the first slot of the staging pass.)
__device__ __forceinline__ void gemv_epi(int g, int rb, int j, int kind, int B, int r0, int s0) {
  const int t0 = TTILE * j;
  const int Bt = B - t0 < TTILE ? B - t0 : TTILE;
  if (kind == EPI_RESIDUAL) {
    for (int e = threadIdx.x; e < TG * 16 * Bt; e += NT) {
      int t = e % Bt, rr = (e / Bt) % 16, i = e / (Bt * 16);
      int m, row;
      if (slot_row(TG * g + i, rr, m, row)) GSM.out[row - r0][t0 + t] += gy(rb, i, rr, t);
    }
  } else if (GSM.grp[g].kind == GK_PAIR) {
    for (int e = threadIdx.x; e < (TG / 2) * 16 * Bt; e += NT) {
      int t = e % Bt, rr = (e / Bt) % 16, jj = e / (Bt * 16);
      float a = gy(rb, 2 * jj, rr, t) * GSM.inv[t0 + t];
      float u = gy(rb, 2 * jj + 1, rr, t) * GSM.inv[t0 + t];
      GSM.out[(TG * g + 2 * jj - s0) * 16 + rr][t0 + t] = silu(a) * u;
    }
  } else {
    for (int e = threadIdx.x; e < TG * 16 * Bt; e += NT) {
      int t = e % Bt, rr = (e / Bt) % 16, i = e / (Bt * 16);
      GSM.out[(TG * g + i - s0) * 16 + rr][t0 + t] = gy(rb, i, rr, t) * GSM.inv[t0 + t];
    }
  }
}

// The weight stream of a phase whose slot tables are built: its first
// k-steps are requested, then the phase waits at sync point wait_idx, then
// everything streams.  inv_n > 0: outputs are scaled by 1/rms over inv_n
// features (partial sums of squares at inv_off).  EPI_RESIDUAL: the owned
// residual rows [r0, r0 + nrow) of x and the gains g_next of the next norm
// are staged in GSM.out / GSM.gain (requested behind the first weight loads,
// written once the wait is over).
// Groups [g0, g1) only (g1 < 0: to the end): one pass of a phase whose
// slot rows do not all fit the staging at once (64-row steps).
__device__ __noinline__ RouteIn gemv_phase(KParams& pk, int wait_idx, int inv_n, uint32_t inv_off, int kind, int r0,
                                           int nrow, const uint16_t* g_next, int g0 = 0, int g1 = -1,
                                           bool route_in = false) {
  PARAMS;
  const int B = p.B, H = p.H;
  if (g1 < 0) g1 = __builtin_amdgcn_readfirstlane(GSM.ngroups);
  const int s0 = TG * g0;
  GemvStream<NBT> gs;
  gemv_begin(gs, p.ws, p.ws_bytes, p.off_zero, B, g0, g1);
  // route_in: the router logits too, behind the first weight loads (they
  // arrive while the stream runs and are returned after it)
  RouteIn rin = {};
  if (route_in) route_load(p, rin);
  float xv[4], gv[4];
  if (kind == EPI_RESIDUAL) {
    // buffer loads: an offset past the resource reads 0, so no load is
    // conditional (a conditional load would be waited for on its own, and
    // with it the weight loads above)
    const rsrc_t xr = make_rsrc_u(p.x, (uint32_t)(MAXB * H * 4));
    const rsrc_t gr = make_rsrc_u(g_next, (uint32_t)(H * 2));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = threadIdx.x + k * NT;
      const bool in = e < nrow * B;
      const int t = e % B, lr = e / B;
      xv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, in ? (uint32_t)(t * H + r0 + lr) * 4u : OOB, 0, 0));
      gv[k] = bf16_f32(__builtin_amdgcn_raw_buffer_load_b16(gr, (in && t == 0) ? (uint32_t)(r0 + lr) * 2u : OOB, 0, 0));
    }
  }
  wait_point(p, wait_idx);
  if (kind == EPI_RESIDUAL) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = threadIdx.x + k * NT;
      if (e < nrow * B) {
        const int t = e % B, lr = e / B;
        GSM.out[lr][t] = xv[k];
        if (t == 0) GSM.gain[lr] = gv[k];
      }
    }
    for (int e = threadIdx.x + 4 * NT; e < nrow * B; e += NT) {  // more rows than 4 per thread
      int t = e % B, lr = e / B;
      GSM.out[lr][t] = p.x[t * H + r0 + lr];
      if (t == 0) GSM.gain[lr] = bf16_f32(g_next[r0 + lr]);
    }
    __syncthreads();
  }
  sub_stamp(p, 0);
  gemv_run(p, gs, inv_n, inv_off, [=](int g, int rb, int j) { gemv_epi(g, rb, j, kind, B, r0, s0); });
  sub_stamp(p, 2);
  return rin;
}

// A slot-staged phase in staging passes: groups [g0, g1) per pass (one pass
// unless the slot rows of MAXB tokens exceed the staging), every pass after
// the first without a wait; post(s0, s1) writes out the staged outputs of
// slots [s0, s1) (staging row (si - s0) * 16 + row-in-slot).
template <class Post>
__device__ __forceinline__ void gemv_passes(KParams& pk, int wait_idx, int inv_n, uint32_t inv_off, Post post) {
  if constexpr (!WIDE) {  // the slot tables' rows always fit: one pass
    gemv_phase(pk, wait_idx, inv_n, inv_off, EPI_BY_KIND, 0, 0, nullptr);
    post(0, __builtin_amdgcn_readfirstlane(GSM.nslots));
  } else {
    constexpr int PER = STAGE_ROWS / (16 * TG);
    const int ng = __builtin_amdgcn_readfirstlane(GSM.ngroups);
    int g0 = 0;
    do {
      const int g1 = ng - g0 < PER ? ng : g0 + PER;
      gemv_phase(pk, g0 == 0 ? wait_idx : -1, inv_n, inv_off, EPI_BY_KIND, 0, 0, nullptr, g0, g1);
      post(TG * g0, TG * g1);
      g0 = g1;
    } while (g0 < ng);
  }
}

// --- QKV projection (GQA): raw q, k, v (RMS-normalised input) -> qkv[t][row]
MD_PHASE_FN void phase_qkv(KParams& pk, int l_layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int B = p.B;
  SlotBuilder sb;
  if (threadIdx.x < 64) {
    sb.start(PL_QKV);
    int mq = sb.mat(L.wq, p.nq * p.hd, p.H, 0);
    int mk = sb.mat(L.wk, p.nkv * p.hd, p.H, p.nq * p.hd);
    int mv = sb.mat(L.wv, p.nkv * p.hd, p.H, (p.nq + p.nkv) * p.hd);
    sb.begin(u_at(p, 2 * l_layer), p.H, GK_SINGLE);
    sb.singles_of(mq, p.nq * p.hd);
    sb.singles_of(mk, p.nkv * p.hd);
    sb.singles_of(mv, p.nkv * p.hd);
  }
  builder_done(p, sb, -1);
  const int nqkv = (p.nq + 2 * p.nkv) * p.hd;
  gemv_passes(p, wait_idx, p.H, ssq_at(p, 2 * l_layer), [&](int s0, int s1) {
    rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
    for (int e = threadIdx.x; e < (s1 - s0) * 16 * B; e += NT) {
      int t = e % B, sr = e / B;
      int m, row;
      if (!slot_row(s0 + (sr >> 4), sr & 15, m, row)) continue;
      st_f32(r, p.off_qkv + (uint32_t)(t * nqkv + GSM.mats[m].tag + row) * 4u, GSM.out[sr][t]);
    }
  });
}

// RoPE rotation of pair i at position pos: (cos, sin) from the table the
// host fills at init (angles pos * theta^(-2i/d) evaluated in fp64, rounded
// to fp32), fp32[max_ctx][d/2][2].
__device__ __forceinline__ void rope_cs(KParams& pk, int pos, int i, float& c, float& s) {
  PARAMS;
  const float* t = p.rope + ((size_t)pos * (p.rope_d / 2) + i) * 2;
  c = t[0];
  s = t[1];
}

// --- GQA decode attention.  Task (b, kv head g, chunk c) covers cached
// positions [a0, a1) of sequence b, chunk boundaries on 32-position tiles.
// Each wave takes a quarter of the chunk's tiles, one 32-position block per
// tile, with the next block's K and V in flight while the current one is
// used.  Both products run on the matrix cores:
//   scores S^T = K . Q: K rows are the A operand, the group's rotated q heads
//     the B columns (head h: column 2h its bf16 high part, 2h+1 the rest);
//   output O^T = V^T . P: the V tile (stored dimension-major) is the A
//     operand, the probabilities the B columns (column 2h the high bf16 part
//     of head h's, 2h+1 the rest).
// The score tile's rows are permuted (row 4i+j of K tile tt is position
// 8i+4tt+j of the block) so that each lane's scores are exactly the eight
// positions its B column of P needs: the online softmax runs in registers,
// per column, with cross-row swaps only.  The task's partial (max, sum, o)
// per head goes to the workspace; the last workgroup to finish a (b, g)
// combines the chunks.
struct AttnSmem {
  float q[GSMAX][128];          // rotated, scaled q of the group's heads
  float wm[NW + 1][GSMAX], wl[NW + 1][GSMAX];  // entry NW: the new row (decode, last chunk)
  alignas(16) float wo[NW][GSMAX][128];
  float knew[128], vnew[128];   // the new row, as the cache stores it
  int last;
};

template <int HD>
struct KVBlock {
  i32x4 k[2][HD / 32];          // 2 tiles of 16 positions x HD/32 k-steps
  i32x4 v[HD / 16];             // the V tile: HD/16 slices of 16 dims x 32 positions
};

// Block at blk (a multiple of 32) of a wave share ending at w1: its 32 K
// rows (row-major [32][HD]) at kb and its V tile ([HD][32]) at vb.
template <int HD, int CP>
__device__ __forceinline__ void load_block(KVBlock<HD>& r, const uint16_t* kb, const uint16_t* vb, int blk, int w1,
                                           int lane) {
  const int m = lane & 15, g = lane >> 4;
  const rsrc_t krs = make_rsrc_u(kb, 32 * HD * 2), vrs = make_rsrc_u(vb, 32 * HD * 2);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int prow = blk + 8 * (m >> 2) + 4 * tt + (m & 3);
#pragma unroll
    for (int s = 0; s < HD / 32; ++s) {
      uint32_t off = (prow < w1) ? (uint32_t)((prow - blk) * HD + s * 32 + g * 8) * 2u : OOB;
      r.k[tt][s] = ld_x4<CP>(krs, off);
    }
  }
#pragma unroll
  for (int q = 0; q < HD / 16; ++q) {
    uint32_t off = blk < w1 ? (uint32_t)((q * 16 + m) * 32 + g * 8) * 2u : OOB;
    r.v[q] = ld_x4<CP>(vrs, off);
  }
}

#define ASM (*reinterpret_cast<AttnSmem*>(md_smem))

// bf16 pairs of (x0, x1) as one 32-bit word (round to nearest even)
__device__ __forceinline__ uint32_t cvt_bf16x2(float x0, float x1) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  f32x2 v = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// One wave's share [w0, w1) of a task.  Its first two blocks (w0, w0 + 32)
// are in flight in ba, bb on entry; each block used is refilled two blocks
// ahead.  Leaves the wave's (max, sum, o) per head in ASM.wm/wl/wo[wv].
struct AttnTask;
template <int HD, int CP>
__device__ __forceinline__ void load_kv_block(KParams& pk, KVBlock<HD>& r, const AttnTask& t, int blk, int lane);
template <int HD, int CP>
__device__ __forceinline__ void attn_wave(KParams& pk, KVBlock<HD>& ba, KVBlock<HD>& bb, const AttnTask& t, int w0,
                                          int w1, int gs) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nn = lane & 15, hh = nn >> 1, pp = nn & 1, g = lane >> 4;
  bf16x8 qb[HD / 32];
#pragma unroll
  for (int s = 0; s < HD / 32; ++s) {
    uint32_t u[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = s * 32 + g * 8 + 2 * k;
      const float v0 = hh < gs ? ASM.q[hh][d] : 0.f, v1 = hh < gs ? ASM.q[hh][d + 1] : 0.f;
      const uint32_t hi = cvt_bf16x2(v0, v1);
      // column 2h+1 carries q minus its bf16 high part
      const float r0 = v0 - __uint_as_float(hi << 16), r1 = v1 - __uint_as_float(hi & 0xFFFF0000u);
      u[k] = pp ? cvt_bf16x2(r0, r1) : hi;
    }
    qb[s] = __builtin_bit_cast(bf16x8, u);
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[HD / 16];
#pragma unroll
  for (int q = 0; q < HD / 16; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto block = [&](const KVBlock<HD>& cur, int blk) __attribute__((always_inline)) {
    // scores: lane holds positions blk + 8g + j (j < 8) of column nn
    float sc[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < HD / 32; ++s)
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[tt][s]), qb[s], a, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * tt + i] = a[i] + dpp_f<DPP_QXOR1>(a[i]);
    }
    if (blk + 32 > w1) {  // the share's last, partial block
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (blk + 8 * g + j >= w1) sc[j] = -INFINITY;
    }
    float mb = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mb = fmaxf(mb, sc[j]);
    mb = rows_max(mb);
    const float mn = fmaxf(m_run, mb);  // finite: position blk is always valid
    const float corr = __expf(m_run - mn);
    float pr[8], ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pr[j] = __expf(sc[j] - mn);
      ps += pr[j];
    }
    l_run = l_run * corr + rows_sum(ps);
    m_run = mn;
    uint32_t u[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t hi = cvt_bf16x2(pr[2 * k], pr[2 * k + 1]);
      const float r0 = pr[2 * k] - __uint_as_float(hi << 16);
      const float r1 = pr[2 * k + 1] - __uint_as_float(hi & 0xFFFF0000u);
      u[k] = pp ? cvt_bf16x2(r0, r1) : hi;
    }
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u);
    if (blk + 32 > w1) {
      // V rows past the share may hold anything (even non-finite values):
      // zero this lane's positions >= w1 so that 0 * V cannot poison O
      const int nv = w1 - blk - 8 * g;  // valid positions of this lane's eight
#pragma unroll
      for (int q = 0; q < HD / 16; ++q) {
        i32x4 v = cur.v[q];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t keep = (2 * k + 1 < nv) ? 0xFFFFFFFFu : (2 * k < nv ? 0x0000FFFFu : 0u);
          v[k] = (int)((uint32_t)v[k] & keep);
        }
        acc[q] *= corr;
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pb, acc[q], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int q = 0; q < HD / 16; ++q) {
        acc[q] *= corr;
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.v[q]), pb, acc[q], 0, 0, 0);
      }
    }
  };
  for (int blk = w0; blk < w1; blk += 64) {
    block(ba, blk);
    if (blk + 32 >= w1) break;
    load_kv_block<HD, CP>(pk, ba, t, blk + 64, lane);
    block(bb, blk + 32);
    if (blk + 64 >= w1) break;
    load_kv_block<HD, CP>(pk, bb, t, blk + 96, lane);
  }
  // head hh's output = column 2hh + column 2hh+1; lane holds dims 16q + 4g + i
  if (hh < gs) {
#pragma unroll
    for (int q = 0; q < HD / 16; ++q) {
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc[q][i] + dpp_f<DPP_QXOR1>(acc[q][i]);
      if (!pp) *(f32x4*)&ASM.wo[wv][hh][16 * q + 4 * g] = o;
    }
    if (g == 0 && !pp) {
      ASM.wm[wv][hh] = m_run;
      ASM.wl[wv][hh] = l_run;
    }
  }
}

// Verify: the new K/V rows of all rows (positions p..p+B-1 of sequence 0)
// go to the cache before attention, device-coherently, because row r
// attends the rows of the tokens before it, computed by other workgroups.
__device__ __noinline__ void phase_gqa_kv_write(KParams& pk, int l_layer) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int hd = p.hd, nqkv = (p.nq + 2 * p.nkv) * hd;
  rsrc_t wr = make_rsrc_u(p.ws, p.ws_bytes);
  for (int task = blockIdx.x; task < p.B * p.nkv; task += gridDim.x) {
    const int g = task % p.nkv, b = task / p.nkv;
    const int pos = row_pos(p, b);
    const KvLoc l = kv_loc(p, row_seq(p, b), pos);
    const size_t pstride = (size_t)p.nkv * p.pg_cap * hd;
    uint16_t* kc = (uint16_t*)(p.kv + L.kv_off) + (size_t)l.page * pstride + (size_t)g * p.pg_cap * hd;
    uint16_t* vc = kc + (size_t)p.n_pages * pstride;
    rsrc_t krs = make_rsrc_u(kc + (size_t)l.r * hd, hd * 2);
    rsrc_t vrs = make_rsrc_u(vc + (size_t)(l.r & ~31) * hd, hd * 64);  // the V tile holding pos
    for (int i = threadIdx.x; i < hd / 2; i += NT) {
      int colk = p.nq * hd + g * hd;
      float a = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colk + i) * 4u);
      float bb = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colk + i + hd / 2) * 4u);
      float cs, sn;
      rope_cs(p, pos, i, cs, sn);
      st_u16(krs, (uint32_t)i * 2u, bf16_rne(a * cs - bb * sn));
      st_u16(krs, (uint32_t)(i + hd / 2) * 2u, bf16_rne(a * sn + bb * cs));
    }
    for (int i = threadIdx.x; i < hd; i += NT) {
      int colv = (p.nq + p.nkv) * hd + g * hd;
      st_u16(vrs, (uint32_t)(i * 32 + (l.r & 31)) * 2u,
             bf16_rne(ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colv + i) * 4u)));
    }
  }
}

// One task of the GQA attention phase: (sequence b, kv head g, chunk c) of
// the cached rows, and this wave's share [w0, w1) of the chunk.  Decode: the
// cached rows are 0..pos-1 (the new row is folded in by the combine); verify:
// 0..pos (the new rows were written by phase_gqa_kv_write).  Chunks are
// whole 32-position tiles (the last one ragged); waves split a chunk's tiles.
struct AttnTask {
  int b, g, c, pos, n, a0, a1, w0, w1;
  int s;                // the sequence's cache slot
  const uint16_t* kh;   // K rows of kv head g in page 0 (page q: + q * pstride)
  const uint16_t* vh;   // V tiles of kv head g in page 0
  size_t pstride;       // elements per page (all kv heads)
};
__device__ __forceinline__ AttnTask attn_task(KParams& pk, int l_layer, int task) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  AttnTask t;
  const int C = p.attn_chunks, hd = p.hd;
  t.c = task % C;
  t.g = (task / C) % p.nkv;
  t.b = task / (C * p.nkv);
  t.pos = row_pos(p, t.b);
  t.n = p.verify ? t.pos + 1 : t.pos;
  const int P = ((t.n + C - 1) / C + 31) & ~31;
  t.a0 = t.c * P < t.n ? t.c * P : t.n;
  t.a1 = (t.c + 1) * P < t.n ? (t.c + 1) * P : t.n;
  const int wv = threadIdx.x >> 6, nt = (t.a1 - t.a0 + 31) >> 5;
  t.w0 = t.a0 + 32 * (nt * wv / NW);
  const int e = t.a0 + 32 * (nt * (wv + 1) / NW);
  t.w1 = e < t.a1 ? e : t.a1;
  t.s = row_seq(p, t.b);
  t.pstride = (size_t)p.nkv * p.pg_cap * hd;
  t.kh = (const uint16_t*)(p.kv + L.kv_off) + (size_t)t.g * p.pg_cap * hd;
  t.vh = t.kh + (size_t)p.n_pages * t.pstride;
  return t;
}

// K rows and V tile of block blk (a multiple of 32) of a task's sequence:
// one page holds the whole block.  Blocks past the wave's share load nothing
// (every offset is out of range) and look nothing up.
template <int HD>
__device__ __forceinline__ void kv_block_ptrs(KParams& pk, const AttnTask& t, int blk, const uint16_t*& kb,
                                              const uint16_t*& vb) {
  kb = t.kh;
  vb = t.vh;
  if (blk < t.w1) {
    const KvLoc l = kv_loc(pk, t.s, blk);
    const size_t o = (size_t)l.page * t.pstride + (size_t)l.r * HD;
    kb += o;
    vb += o;
  }
}
template <int HD, int CP>
__device__ __forceinline__ void load_kv_block(KParams& pk, KVBlock<HD>& r, const AttnTask& t, int blk, int lane) {
  const uint16_t *kb, *vb;
  kv_block_ptrs<HD>(pk, t, blk, kb, vb);
  load_block<HD, CP>(r, kb, vb, blk, t.w1, lane);
}

// GQA decode attention.  Each task's partial (max, sum, o) per head goes to
// the workspace; when decoding, the task of the last chunk also folds in the
// new row, computed in place (q . k_new, v_new) rather than read back from
// the cache it writes.  The last workgroup to finish a (b, g) combines the
// chunks with one round of loads (a running max over the chunks).  When
// decoding, the first task's first K/V blocks are requested before the wait
// for the q/k/v projections (the cached rows do not depend on them).
// Inlined into the kernel: as a called function it would save and restore
// the callee-saved registers its live values occupy.
template <int HD, bool VERIFY>
__device__ __forceinline__ void attn_phase(KParams& pk, int l_layer, int layer, int wait_idx) {
  PARAMS;
  constexpr int CP = VERIFY ? CP_SC1 : 0;
  AttnSmem& sm = *(AttnSmem*)md_smem;
  const int lane = threadIdx.x & 63;
  const int gs = p.nq / p.nkv, B = p.B;
  const int C = p.attn_chunks;
  const int ntask = B * p.nkv * C;
  const int nqkv = (p.nq + 2 * p.nkv) * HD;
  rsrc_t wr = make_rsrc_u(p.ws, p.ws_bytes);
  const float scale = 1.0f / sqrtf((float)HD);
  KVBlock<HD> ba, bb;
  AttnTask t;
  auto start = [&](int task) __attribute__((always_inline)) {
    t = attn_task(p, l_layer, task);
    load_kv_block<HD, CP>(p, ba, t, t.w0, lane);
    load_kv_block<HD, CP>(p, bb, t, t.w0 + 32, lane);
  };
  if (!VERIFY && (int)blockIdx.x < ntask) start(blockIdx.x);
  wait_point(p, wait_idx);
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    if (VERIFY || task != (int)blockIdx.x) start(task);
    const int b = t.b, g = t.g, c = t.c, pos = t.pos;
    for (int e = threadIdx.x; e < gs * (HD / 2); e += NT) {
      int h = e / (HD / 2), i = e % (HD / 2);
      int col = (g * gs + h) * HD;
      float a = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + col + i) * 4u);
      float bq = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + col + i + HD / 2) * 4u);
      float cs, sn;
      rope_cs(p, pos, i, cs, sn);
      sm.q[h][i] = (a * cs - bq * sn) * scale;
      sm.q[h][i + HD / 2] = (a * sn + bq * cs) * scale;
    }
    // decode: the task of the last chunk folds the new row into its partial
    // (and writes it to the cache; nothing reads it back in this step)
    const bool newrow = !VERIFY && c == C - 1;
    if (newrow) {
      const KvLoc nl = kv_loc(p, t.s, pos);
      const size_t po = (size_t)nl.page * t.pstride;
      uint16_t* kc = const_cast<uint16_t*>(t.kh) + po + (size_t)nl.r * HD;                          // K row of pos
      uint16_t* vt = const_cast<uint16_t*>(t.vh) + po + (size_t)(nl.r & ~31) * HD + (nl.r & 31);  // V tile of pos
      for (int i = threadIdx.x; i < HD / 2; i += NT) {
        int colk = p.nq * HD + g * HD;
        float a = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colk + i) * 4u);
        float bk = ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colk + i + HD / 2) * 4u);
        float cs, sn;
        rope_cs(p, pos, i, cs, sn);
        uint16_t k0 = bf16_rne(a * cs - bk * sn), k1 = bf16_rne(a * sn + bk * cs);
        kc[i] = k0;
        kc[i + HD / 2] = k1;
        sm.knew[i] = bf16_f32(k0);
        sm.knew[i + HD / 2] = bf16_f32(k1);
      }
      for (int i = threadIdx.x; i < HD; i += NT) {
        int colv = (p.nq + p.nkv) * HD + g * HD;
        uint16_t v0 = bf16_rne(ld_f32(wr, p.off_qkv + (uint32_t)(b * nqkv + colv + i) * 4u));
        vt[i * 32] = v0;
        sm.vnew[i] = bf16_f32(v0);
      }
    }
    __syncthreads();
    if (newrow) {  // q_h . k_new, one head per wave at a time
      const int ln = threadIdx.x & 63;
      for (int h = threadIdx.x >> 6; h < gs; h += NW) {
        float sp = 0.f;
        for (int d = ln; d < HD; d += 64) sp += sm.q[h][d] * sm.knew[d];
        sp = wave_sum(sp);
        if (ln == 0) { sm.wm[NW][h] = sp; sm.wl[NW][h] = 1.f; }
      }
    }
    sub_stamp(p, 0);
    attn_wave<HD, CP>(p, ba, bb, t, t.w0, t.w1, gs);
    __syncthreads();
    sub_stamp(p, 3);
    // this task's partial: (m, l) in part_ml[b][head][c]; o in part_o[b][head][c][hd]
    for (int e = threadIdx.x; e < gs * HD; e += NT) {
      int h = e / HD, d = e % HD;
      float M = -INFINITY;
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.wm[w][h]);
      if (newrow) M = fmaxf(M, sm.wm[NW][h]);
      float o = 0.f, l = 0.f;
      for (int w = 0; w < NW; ++w) {
        float f = sm.wm[w][h] == -INFINITY ? 0.f : __expf(sm.wm[w][h] - M);
        o += f * sm.wo[w][h][d];
        l += f * sm.wl[w][h];
      }
      if (newrow) {
        float f = __expf(sm.wm[NW][h] - M);
        o += f * sm.vnew[d];
        l += f;
      }
      uint32_t head = (uint32_t)((b * p.nq + g * gs + h) * C + c);
      if (d == 0) {
        st_f32(wr, p.off_attn_ml + head * 8u, M);
        st_f32(wr, p.off_attn_ml + head * 8u + 4u, l);
      }
      st_f32(wr, p.off_attn + (head * (uint32_t)HD + d) * 4u, o);
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
      // thread per (head, 4 dims): running-max combine over the chunks, 8 in flight
      constexpr int TPH = HD / 4;  // threads per head
      for (int e = threadIdx.x; e < gs * TPH; e += NT) {
        const int h = e / TPH, d4 = (e % TPH) * 4;
        const uint32_t hb = (uint32_t)((b * p.nq + g * gs + h) * C);
        float M = -INFINITY, den = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
        for (int c0 = 0; c0 < C; c0 += 8) {
          float mc[8], lc[8];
          i32x4 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const bool ok = c0 + u < C;
            mc[u] = ok ? ld_f32(wr, p.off_attn_ml + (hb + c0 + u) * 8u) : -INFINITY;
            lc[u] = ok ? ld_f32(wr, p.off_attn_ml + (hb + c0 + u) * 8u + 4u) : 0.f;
            v[u] = ld_x4<CP_SC1>(wr, ok ? p.off_attn + ((hb + c0 + u) * (uint32_t)HD + d4) * 4u : OOB);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (mc[u] == -INFINITY) continue;
            const float mn = fmaxf(M, mc[u]);
            const float fo = M == -INFINITY ? 0.f : __expf(M - mn), fc = __expf(mc[u] - mn);
            den = den * fo + lc[u] * fc;
            o0 = o0 * fo + __int_as_float(v[u][0]) * fc;
            o1 = o1 * fo + __int_as_float(v[u][1]) * fc;
            o2 = o2 * fo + __int_as_float(v[u][2]) * fc;
            o3 = o3 * fo + __int_as_float(v[u][3]) * fc;
            M = mn;
          }
        }
        const float il = 1.0f / den;
        const int col = (g * gs + h) * HD + d4;
        put_hilo(wr, ou_at(p, l_layer), p.nq * HD, b, col + 0, o0 * il);
        put_hilo(wr, ou_at(p, l_layer), p.nq * HD, b, col + 1, o1 * il);
        put_hilo(wr, ou_at(p, l_layer), p.nq * HD, b, col + 2, o2 * il);
        put_hilo(wr, ou_at(p, l_layer), p.nq * HD, b, col + 3, o3 * il);
      }
    }
    __syncthreads();
    sub_stamp(p, 2);
  }
}

__device__ __forceinline__ void phase_attn_gqa(KParams& pk, int l_layer, int layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  if (p.verify) {
    if (p.hd == 128) attn_phase<128, true>(p, l_layer, layer, wait_idx);
    else attn_phase<64, true>(p, l_layer, layer, wait_idx);
  } else {
    if (p.hd == 128) attn_phase<128, false>(p, l_layer, layer, wait_idx);
    else attn_phase<64, false>(p, l_layer, layer, wait_idx);
  }
}

// ------------------------------------------------------------------ gated delta rule
// Layers that are not MLA in the hybrid model (section "Our Kimi K3
// megakernel": the attention kind is chosen by layer index).  Per head h,
// with q and k L2-normalised and alpha, beta the sigmoid gates:
//   u = S^T k;  S <- alpha S + beta k (v - u)^T;  o = S^T q (updated S).
// Projection phase: q, k, v and the two gate logits per head, one GEMV
// over five matrices; kda[t] = [q (nh*dk) | k (nh*dk) | v (nh*dv) | a (nh) | b (nh)].
MD_PHASE_FN void phase_kda_proj(KParams& pk, int l_layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int B = p.B, nh = p.kda_h, dk = p.kda_dk, dv = p.kda_dv;
  const int width = 2 * nh * dk + nh * dv + 2 * nh;
  SlotBuilder sb;
  if (threadIdx.x < 64) {
    sb.start(PL_KDA_PROJ);
    int m0 = sb.mat(L.kda_wq, nh * dk, p.H, 0);
    int m1 = sb.mat(L.kda_wk, nh * dk, p.H, nh * dk);
    int m2 = sb.mat(L.kda_wv, nh * dv, p.H, 2 * nh * dk);
    int m3 = sb.mat(L.kda_wa, nh, p.H, 2 * nh * dk + nh * dv);
    int m4 = sb.mat(L.kda_wb, nh, p.H, 2 * nh * dk + nh * dv + nh);
    sb.begin(u_at(p, 2 * l_layer), p.H, GK_SINGLE);
    sb.singles_of(m0, nh * dk);
    sb.singles_of(m1, nh * dk);
    sb.singles_of(m2, nh * dv);
    sb.singles_of(m3, nh);
    sb.singles_of(m4, nh);
  }
  builder_done(p, sb, -1);
  gemv_passes(p, wait_idx, p.H, ssq_at(p, 2 * l_layer), [&](int s0, int s1) {
    rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
    for (int e = threadIdx.x; e < (s1 - s0) * 16 * B; e += NT) {
      int t = e % B, sr = e / B;
      int m, row;
      if (!slot_row(s0 + (sr >> 4), sr & 15, m, row)) continue;
      st_f32(r, p.off_kda + (uint32_t)(t * width + GSM.mats[m].tag + row) * 4u, GSM.out[sr][t]);
    }
  });
}

struct KdaSmem {
  float q[128], k[128], v[32];
  float qs, ks, a, b;
  float red[8][32];
  float red2[8][32];
};

// Recurrence phase: task (b, h, 32-column slice of the state).  The slice
// (dk x 32 fp32) is read once into registers -- thread (rg, j) holds rows
// rg, rg+8, ... of column j -- updated there and written back in place.
// The first task's state slice is requested before the wait: the state is
// only read and written here, so it is final from the previous step.
__device__ __noinline__ void phase_kda_rec(KParams& pk, int l_layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  KdaSmem& sm = *(KdaSmem*)md_smem;
  const int B = p.B, nh = p.kda_h, dk = p.kda_dk, dv = p.kda_dv;
  const int width = 2 * nh * dk + nh * dv + 2 * nh;
  const int ns = dv / 32;
  const int ntask = B * nh * ns;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rg = threadIdx.x >> 5, jj = threadIdx.x & 31;
  rsrc_t wr = make_rsrc_u(p.ws, p.ws_bytes);
  float s[16];
  auto load_state = [&](int task) __attribute__((always_inline)) {
    const int js = task % ns, h = (task / ns) % nh, b = task / (ns * nh);
    float* S = (float*)(p.kv + L.kv_off) + (size_t)(b * nh + h) * dk * dv;
    rsrc_t srs = make_rsrc_u(S, (uint32_t)(dk * dv * 4));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int i = rg + 8 * r;
      s[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          srs, i < dk ? (uint32_t)(i * dv + 32 * js + jj) * 4u : OOB, 0, 0));
    }
  };
  if ((int)blockIdx.x < ntask) load_state(blockIdx.x);
  wait_point(p, wait_idx);
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int js = task % ns, h = (task / ns) % nh, b = task / (ns * nh);
    const uint32_t base = p.off_kda + (uint32_t)(b * width) * 4u;
    float* S = (float*)(p.kv + L.kv_off) + (size_t)(b * nh + h) * dk * dv;
    rsrc_t srs = make_rsrc_u(S, (uint32_t)(dk * dv * 4));
    if (task != (int)blockIdx.x) load_state(task);
    if (threadIdx.x < dk) {
      sm.q[threadIdx.x] = ld_f32(wr, base + (uint32_t)(h * dk + threadIdx.x) * 4u);
      sm.k[threadIdx.x] = ld_f32(wr, base + (uint32_t)(nh * dk + h * dk + threadIdx.x) * 4u);
    }
    if (threadIdx.x < 32) sm.v[threadIdx.x] = ld_f32(wr, base + (uint32_t)(2 * nh * dk + h * dv + 32 * js + threadIdx.x) * 4u);
    if (threadIdx.x == 0) {
      sm.a = sigmoid(ld_f32(wr, base + (uint32_t)(2 * nh * dk + nh * dv + h) * 4u));
      sm.b = sigmoid(ld_f32(wr, base + (uint32_t)(2 * nh * dk + nh * dv + nh + h) * 4u));
    }
    __syncthreads();
    if (wv < 2) {  // wave 0: 1/||q||, wave 1: 1/||k|| (1 without normalisation)
      const float* vec = wv == 0 ? sm.q : sm.k;
      float a0 = lane < dk ? vec[lane] : 0.f, a1 = lane + 64 < dk ? vec[lane + 64] : 0.f;
      float n2 = wave_sum(a0 * a0 + a1 * a1);
      float sc = p.kda_l2 ? 1.0f / fmaxf(sqrtf(n2), 1e-6f) : 1.0f;
      if (lane == 0) { if (wv == 0) sm.qs = sc; else sm.ks = sc; }
    }
    __syncthreads();
    const float qs = sm.qs, ks = sm.ks;
    float up = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int i = rg + 8 * r;
      if (i < dk) up += s[r] * (sm.k[i] * ks);
    }
    sm.red[rg][jj] = up;
    __syncthreads();
    float u = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) u += sm.red[g][jj];
    const float delta = sm.b * (sm.v[jj] - u), al = sm.a;
    float op = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int i = rg + 8 * r;
      float kn = sm.k[i < dk ? i : 0] * ks;
      s[r] = al * s[r] + kn * delta;
      if (i < dk) op += s[r] * (sm.q[i] * qs);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s[r]), srs,
                                            i < dk ? (uint32_t)(i * dv + 32 * js + jj) * 4u : OOB, 0, 0);
    }
    sm.red2[rg][jj] = op;
    __syncthreads();
    if (threadIdx.x < 32) {
      float o = 0.f;
#pragma unroll
      for (int g = 0; g < 8; ++g) o += sm.red2[g][threadIdx.x];
      put_hilo(wr, ou_at(p, l_layer), nh * dv, b, h * dv + 32 * js + threadIdx.x, o);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ verify
// Section "DSpark" of the pages: one launch scores an anchor and its proposed
// continuations.  The rows are the tokens t_0..t_{B-1} of sequence 0 at
// positions p..p+B-1, each attending the cache up to its own position.  The
// delta-rule state advances token by token: task (h, 32-column slice) runs
// the B updates in registers, emits o for every row, and stores the state
// after every row in the snapshot ring; the state itself is rewritten only
// once the accepted length is known (verify_finish).
__device__ __noinline__ void phase_kda_rec_verify(KParams& pk, int l_layer) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  KdaSmem& sm = *(KdaSmem*)md_smem;
  const int B = p.B, nh = p.kda_h, dk = p.kda_dk, dv = p.kda_dv;
  const int width = 2 * nh * dk + nh * dv + 2 * nh;
  const int ns = dv / 32;
  const int ntask = nh * ns;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rg = threadIdx.x >> 5, jj = threadIdx.x & 31;
  const size_t sbytes = (size_t)nh * dk * dv * 4;
  rsrc_t wr = make_rsrc_u(p.ws, p.ws_bytes);
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int js = task % ns, h = task / ns;
    const float* S = (const float*)(p.kv + L.kv_off) + (size_t)h * dk * dv;  // sequence 0
    rsrc_t srs = make_rsrc_u(S, (uint32_t)(dk * dv * 4));
    float s[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int i = rg + 8 * r;
      s[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          srs, i < dk ? (uint32_t)(i * dv + 32 * js + jj) * 4u : OOB, 0, 0));
    }
    for (int j = 0; j < B; ++j) {
      const uint32_t base = p.off_kda + (uint32_t)(j * width) * 4u;
      if (threadIdx.x < dk) {
        sm.q[threadIdx.x] = ld_f32(wr, base + (uint32_t)(h * dk + threadIdx.x) * 4u);
        sm.k[threadIdx.x] = ld_f32(wr, base + (uint32_t)(nh * dk + h * dk + threadIdx.x) * 4u);
      }
      if (threadIdx.x < 32) sm.v[threadIdx.x] = ld_f32(wr, base + (uint32_t)(2 * nh * dk + h * dv + 32 * js + threadIdx.x) * 4u);
      if (threadIdx.x == 0) {
        sm.a = sigmoid(ld_f32(wr, base + (uint32_t)(2 * nh * dk + nh * dv + h) * 4u));
        sm.b = sigmoid(ld_f32(wr, base + (uint32_t)(2 * nh * dk + nh * dv + nh + h) * 4u));
      }
      __syncthreads();
      if (wv < 2) {
        const float* vec = wv == 0 ? sm.q : sm.k;
        float a0 = lane < dk ? vec[lane] : 0.f, a1 = lane + 64 < dk ? vec[lane + 64] : 0.f;
        float n2 = wave_sum(a0 * a0 + a1 * a1);
        float sc = p.kda_l2 ? 1.0f / fmaxf(sqrtf(n2), 1e-6f) : 1.0f;
        if (lane == 0) { if (wv == 0) sm.qs = sc; else sm.ks = sc; }
      }
      __syncthreads();
      const float qs = sm.qs, ks = sm.ks;
      float up = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int i = rg + 8 * r;
        if (i < dk) up += s[r] * (sm.k[i] * ks);
      }
      sm.red[rg][jj] = up;
      __syncthreads();
      float u = 0.f;
#pragma unroll
      for (int g = 0; g < 8; ++g) u += sm.red[g][jj];
      const float delta = sm.b * (sm.v[jj] - u), al = sm.a;
      rsrc_t snap = make_rsrc_u(p.kda_ring + ((size_t)L.kda_idx * MAXB + j) * sbytes + (size_t)h * dk * dv * 4,
                                (uint32_t)(dk * dv * 4));
      float op = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int i = rg + 8 * r;
        float kn = sm.k[i < dk ? i : 0] * ks;
        s[r] = al * s[r] + kn * delta;
        if (i < dk) op += s[r] * (sm.q[i] * qs);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s[r]), snap,
                                              i < dk ? (uint32_t)(i * dv + 32 * js + jj) * 4u : OOB, 0, CP_SC1);
      }
      sm.red2[rg][jj] = op;
      __syncthreads();
      if (threadIdx.x < 32) {
        float o = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) o += sm.red2[g][threadIdx.x];
        put_hilo(wr, ou_at(p, l_layer), nh * dv, j, h * dv + 32 * js + threadIdx.x, o);
      }
      __syncthreads();
    }
  }
}

// After the LM head: every workgroup takes the argmax of every row from the
// candidates (the same fixed order as the decode path), derives the accepted
// length a = 1 + m (m: the largest j with t_i == argmax(row i-1) for all
// 1 <= i <= j), and copies its share of each delta-rule layer's snapshot m
// into the state.  Workgroup 0 reports a and argmax(row a-1).
constexpr int MAX_KDA_LAYERS = 512;
__device__ __noinline__ void verify_finish(KParams& pk) {
  PARAMS;
  int* arg = (int*)md_smem;                 // [MAXB]
  int* acc = arg + MAXB;                    // [1]
  uint64_t* koff = (uint64_t*)(md_smem + 64);  // [MAX_KDA_LAYERS] state offsets of the delta-rule layers
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int t = wv; t < p.B; t += NW) {
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
    if (lane == 0) arg[t] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int m = 0;
    for (int j = 1; j < p.B; ++j) {
      if (p.tokens[j] == arg[j - 1]) m = j;
      else break;
    }
    acc[0] = m + 1;
    if (blockIdx.x == 0) {
      p.out_accept[0] = m + 1;
      p.out_next[0] = arg[m];
    }
  }
  for (int l = threadIdx.x; l < p.n_layers; l += NT) {
    const LayerDesc& d = p.layers[l];
    if (d.kind == LK_KDA && d.kda_idx < MAX_KDA_LAYERS) koff[d.kda_idx] = d.kv_off;
  }
  __syncthreads();
  const int m = acc[0] - 1, n = p.n_kda < MAX_KDA_LAYERS ? p.n_kda : MAX_KDA_LAYERS;
  const size_t sbytes = (size_t)p.kda_h * p.kda_dk * p.kda_dv * 4;
  const uint32_t units = (uint32_t)(sbytes / 16);
  const RowSplit my = rows_of((int)units, blockIdx.x, gridDim.x);
  for (int k = 0; k < n; ++k) {
    rsrc_t src = make_rsrc_u(p.kda_ring + ((size_t)k * MAXB + m) * sbytes, (uint32_t)sbytes);
    rsrc_t dst = make_rsrc_u(p.kv + koff[k], (uint32_t)sbytes);
    for (int u = my.r0 + threadIdx.x; u < my.r1; u += NT) {
      i32x4 v = ld_x4<CP_SC1>(src, (uint32_t)u * 16u);
      __builtin_amdgcn_raw_buffer_store_b128(v, dst, (uint32_t)u * 16u, 0, 0);
    }
  }
}

// ------------------------------------------------------------------ MLA
// Multi-head latent attention (the other layer kind of the hybrid model), in
// the absorbed form: the cache holds per position the RMS-normalised latent
// c (kv_lora = 512) and the rotated key part k_pe (64).  Per head h:
//   q~_h = W_uk,h^T q_nope,h;  s_t = (q~_h . c_t + q_pe,h . kpe_t) / sqrt(nope + rope);
//   z_h = sum_t softmax(s)_t c_t;  o_h = W_uv,h z_h;  x += W_o o.
constexpr int MLA_KL = 512, MLA_RD = 64, MLA_QA = MLA_KL + MLA_RD, MLA_KS = MLA_QA / 32;

// M1: c_q0 = W_qa xn (q_lora) and ckv = W_kva xn (kv_lora + rope).  c_q0 goes
// out as U = hilo(g_q * c_q0) plus its partial sums of squares (the q norm),
// ckv as fp32.
MD_PHASE_FN void phase_mla_a(KParams& pk, int l_layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int B = p.B, QL = p.q_lora, KVR = MLA_QA;
  SlotBuilder sb;
  if (threadIdx.x < 64) {
    sb.start(PL_MLA_A);
    int ma = sb.mat(L.mla_wqa, QL, p.H, 0);
    int mk = sb.mat(L.mla_wkva, KVR, p.H, 1);
    sb.begin(u_at(p, 2 * l_layer), p.H, GK_SINGLE);
    sb.singles_of(ma, QL);
    sb.singles_of(mk, KVR);
  }
  builder_done(p, sb, -1);
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  // staged output (token t, staging row sr of a pass from slot s0); returns
  // its square for c_q0's norm, 0 for the latent part
  auto elem = [&](int t, int sr, int s0) -> float {
    int m, row;
    if (!slot_row(s0 + (sr >> 4), sr & 15, m, row)) return 0.f;
    float v = GSM.out[sr][t];
    if (GSM.mats[m].tag == 0) {
      put_hilo(r, uq_at(p, l_layer), QL, t, row, bf16_f32(L.mla_qnorm[row]) * v);
      return v * v;
    }
    st_f32(r, p.off_ckv + (uint32_t)(t * KVR + row) * 4u, v);
    return 0.f;
  };
  if constexpr (WIDE) {
    float acc = 0.f;
    const int t = threadIdx.x & 63;
    gemv_passes(p, wait_idx, p.H, ssq_at(p, 2 * l_layer), [&](int s0, int s1) {
      if (t < B)
        for (int sr = threadIdx.x >> 6; sr < (s1 - s0) * 16; sr += NT / 64) acc += elem(t, sr, s0);
    });
    store_ssq_wide(p, r, acc, ssq2_at(p, l_layer));
  } else {
    gemv_phase(p, wait_idx, p.H, ssq_at(p, 2 * l_layer), EPI_BY_KIND, 0, 0, nullptr);
    float* part = (float*)GSM.red;  // [NT][MAXB]
    for (int t = 0; t < MAXB; ++t) part[threadIdx.x * MAXB + t] = 0.f;
    for (int e = threadIdx.x; e < GSM.nslots * 16 * B; e += NT) {
      int t = e % B, sr = e / B;
      part[threadIdx.x * MAXB + t] += elem(t, sr, 0);
    }
    store_ssq(p, r, part, ssq2_at(p, l_layer));
  }
}

// The new latent cache row of sequence b: RMSNorm(c) * g_kv and the rotated
// k_pe, rounded to bf16, written device-coherently (another workgroup reads
// it in this same step).
__device__ void mla_cache_row(KParams& pk, int l_layer, int b) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  float* c = &GSM.in[0][0];  // [576] (the staging area is free before the stream)
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  const int pos = row_pos(p, b);
  for (int i = threadIdx.x; i < MLA_QA; i += NT) c[i] = ld_f32(r, p.off_ckv + (uint32_t)(b * MLA_QA + i) * 4u);
  __syncthreads();
  float* red = &GSM.in[80][0];  // [NW]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float ss = 0.f;
  for (int i = threadIdx.x; i < MLA_KL; i += NT) ss += c[i] * c[i];
  ss = wave_sum(ss);
  if (lane == 0) red[wv] = ss;
  __syncthreads();
  float tot = red[0] + red[1] + red[2] + red[3];
  float inv = 1.0f / sqrtf(tot / (float)MLA_KL + p.eps);
  const KvLoc l = kv_loc(p, row_seq(p, b), pos);
  uint16_t* row = (uint16_t*)(p.kv + L.kv_off) + ((size_t)l.page * p.pg_cap + l.r) * MLA_QA;
  rsrc_t cr = make_rsrc_u(row, MLA_QA * 2);
  for (int i = threadIdx.x; i < MLA_KL; i += NT) st_u16(cr, (uint32_t)i * 2u, bf16_rne(bf16_f32(L.mla_kvnorm[i]) * (c[i] * inv)));
  for (int i = threadIdx.x; i < MLA_RD / 2; i += NT) {
    float cs, sn;
    rope_cs(p, pos, i, cs, sn);
    float a = c[MLA_KL + i], bb = c[MLA_KL + i + MLA_RD / 2];
    st_u16(cr, (uint32_t)(MLA_KL + i) * 2u, bf16_rne(a * cs - bb * sn));
    st_u16(cr, (uint32_t)(MLA_KL + i + MLA_RD / 2) * 2u, bf16_rne(a * sn + bb * cs));
  }
  wait_stores();
  __syncthreads();
}

// M2: q = W_qb RMSNorm(c_q0) (nh x (nope + rope)), and the new cache rows
// (workgroup G-1-b writes sequence b's).
MD_PHASE_FN void phase_mla_b(KParams& pk, int l_layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int B = p.B, nh = p.mla_h, QW = p.nope + MLA_RD;
  const int cb = (int)gridDim.x - 1 - (int)blockIdx.x;
  SlotBuilder sb;
  if (threadIdx.x < 64) {
    sb.start(PL_MLA_B);
    int m = sb.mat(L.mla_wqb, nh * QW, p.q_lora, 0);
    sb.begin(uq_at(p, l_layer), p.q_lora, GK_SINGLE);
    sb.singles_of(m, nh * QW);
  }
  builder_done(p, sb, -1);
  bool row_done = false;
  gemv_passes(p, wait_idx, p.q_lora, ssq2_at(p, l_layer), [&](int s0, int s1) {
    if (!row_done && cb < B) mla_cache_row(p, l_layer, cb);  // (in the input staging, which the stream leaves alone)
    row_done = true;
    rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
    for (int e = threadIdx.x; e < (s1 - s0) * 16 * B; e += NT) {
      int t = e % B, sr = e / B;
      int m, row;
      if (!slot_row(s0 + (sr >> 4), sr & 15, m, row)) continue;
      st_f32(r, p.off_qm + (uint32_t)(t * nh * QW + row) * 4u, GSM.out[sr][t]);
    }
  });
}

// M3: absorbed queries qabs[t][h] = [W_uk,h^T q_nope,h | RoPE(q_pe,h)] / sqrt(nope + rope).
// Task (h, 128-column block of the latent); the tokens in tiles of 8 (one
// tile up to 8 rows), so each slice of W_uk is read from memory once.  W_kvb is row-major [nh*(nope+v)][512]: head
// h's rows are [W_uk,h (nope rows) | W_uv,h (v rows)].
MD_PHASE_FN void phase_mla_absorb(KParams& pk, int l_layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int B = p.B, nh = p.mla_h, nope = p.nope, QW = nope + MLA_RD, VW = nope + p.vdim;
  constexpr int NCB = MLA_KL / 128;
  const int ntask = nh * NCB;
  const float scale = 1.0f / sqrtf((float)QW);
  constexpr int AT = 8;                    // tokens per tile
  float* qn = &GSM.in[0][0];               // [AT][nope <= 128]
  float* red = &GSM.out[0][0];             // [NW][AT][128]
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  rsrc_t wrs = make_rsrc_u(L.mla_wkvb, (uint32_t)((size_t)nh * VW * MLA_KL * 2));
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int cg = lane & 15, rg = wv * 4 + (lane >> 4);  // 16 row groups x 16 column groups of 8
  // this thread's rows rg, rg + 16, ... (nope <= 128: at most 8) of the
  // task's W_uk slice, requested before the wait (the weights depend on no
  // other workgroup) and used by every token tile
  i32x4 wk[8];
  auto load_w = [&](int task) __attribute__((always_inline)) {
    const int h = task / NCB, cbk = task % NCB;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = rg + 16 * k;
      wk[k] = ld_x4<0>(wrs, i < nope ? (uint32_t)(((h * VW + i) * MLA_KL) + 128 * cbk + 8 * cg) * 2u : OOB);
    }
  };
  if ((int)blockIdx.x < ntask) load_w(blockIdx.x);
  wait_point(p, wait_idx);
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int h = task / NCB, cbk = task % NCB;
    if (task != (int)blockIdx.x) load_w(task);
    for (int t0 = 0; t0 < B; t0 += AT) {
    const int Bt = B - t0 < AT ? B - t0 : AT;
    if (t0 > 0) __syncthreads();  // the previous tile's reads of qn and red are done
    for (int e = threadIdx.x; e < Bt * nope; e += NT) {
      int t = e / nope, i = e % nope;
      qn[t * 128 + i] = ld_f32(r, p.off_qm + (uint32_t)((t0 + t) * nh * QW + h * QW + i) * 4u);
    }
    __syncthreads();
    float acc[AT][8];
#pragma unroll
    for (int t = 0; t < AT; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[t][j] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = rg + 16 * k;
      if (i >= nope) break;
      const i32x4 w = wk[k];
      float wf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wf[2 * j] = __uint_as_float((uint32_t)w[j] << 16);
        wf[2 * j + 1] = __uint_as_float((uint32_t)w[j] & 0xFFFF0000u);
      }
#pragma unroll
      for (int t = 0; t < AT; ++t) {
        float qv = t < Bt ? qn[t * 128 + i] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t][j] += wf[j] * qv;
      }
    }
    // sum the 4 row groups of this wave, then the 4 waves
#pragma unroll
    for (int t = 0; t < AT; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[t][j] = rows_sum(acc[t][j]);
    if (lane < 16) {
#pragma unroll
      for (int t = 0; t < AT; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) red[(wv * AT + t) * 128 + 8 * cg + j] = acc[t][j];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < Bt * 128; e += NT) {
      int t = e / 128, c = e % 128;
      float v = red[(0 * AT + t) * 128 + c] + red[(1 * AT + t) * 128 + c] + red[(2 * AT + t) * 128 + c] +
                red[(3 * AT + t) * 128 + c];
      st_f32(r, p.off_qabs + (uint32_t)(((t0 + t) * nh + h) * MLA_QA + 128 * cbk + c) * 4u, v * scale);
    }
    }
    if (cbk == 0) {
      for (int e = threadIdx.x; e < B * (MLA_RD / 2); e += NT) {
        int t = e / (MLA_RD / 2), i = e % (MLA_RD / 2);
        const int pos = row_pos(p, t);
        float a = ld_f32(r, p.off_qm + (uint32_t)(t * nh * QW + h * QW + nope + i) * 4u);
        float bb = ld_f32(r, p.off_qm + (uint32_t)(t * nh * QW + h * QW + nope + i + MLA_RD / 2) * 4u);
        float cs, sn;
        rope_cs(p, pos, i, cs, sn);
        st_f32(r, p.off_qabs + (uint32_t)((t * nh + h) * MLA_QA + MLA_KL + i) * 4u, (a * cs - bb * sn) * scale);
        st_f32(r, p.off_qabs + (uint32_t)((t * nh + h) * MLA_QA + MLA_KL + i + MLA_RD / 2) * 4u, (a * sn + bb * cs) * scale);
      }
    }
    __syncthreads();
  }
}

// M4: attention over the latent cache.  Task (b, chunk c) covers positions
// [c*P, (c+1)*P) of 0..pos for every head at once, so each cache row is read
// once per step.  Blocks of 32 rows are staged in LDS twice: row-major (the A
// operand of the scores) and transposed, latent dims by positions (the A
// operand of P.C); the next block is in flight while the current one is
// used.  Scores: wave w serves heads 8w..8w+7 on the matrix cores (rows as
// the A operand, the heads' absorbed queries as hi/lo B columns), then an
// online softmax per head; the probabilities go to LDS as hi/lo bf16 (about
// 16 bits).  z_h += sum_t p_t c_t on the matrix cores too: wave w serves
// heads 16(w%2)..+15 and latent dims 256(w/2)..+255, the hi and lo halves
// of P accumulating into the same 16 dims x 16 heads tiles.  Partial
// (max, sum, z) per head go to the workspace.  Inlined into the kernel: as a
// called function it would save and restore the callee-saved registers its
// live values occupy (about 116 per lane, through scratch memory, on every
// call).
constexpr int MLA_ROWP = MLA_QA + 8;  // LDS row pitch in bf16 (pads rows off the same banks)
constexpr int MLA_TP = 32 + 8;        // pitch of the transposed block and of P, in bf16 (20 dwords:
                                      // conflict-free transposed writes and operand reads)
struct MlaSmem {
  uint16_t rows[32][MLA_ROWP];        // the block, row-major: [position][latent | rope]
  uint16_t ct[MLA_KL][MLA_TP];        // its latent part transposed: [dim][position]
  uint16_t pb[2][32][MLA_TP];         // probabilities [hi, lo][head][position]
  float s[32][32];                    // [position][head] scores
  float corr[32];                     // per head: rescale of z for this block
};

// Thread tid loads chunk c16 = tid/32 + 8k (16 bytes) of row tid%32, k < 9;
// rows past the chunk end are loaded as zeros.  crs covers the layer's whole
// cache; the block's 32 rows of sequence slot sq lie in at most two pages.
__device__ __forceinline__ void mla_load_block(KParams& pk, i32x4 (&pf)[9], rsrc_t crs, int sq, int blk, int a1) {
  PARAMS;
  const int rr = threadIdx.x & 31, t = blk + rr;
  const KvLoc l0 = kv_loc(p, sq, blk);
  KvLoc l1 = l0;
  const int last = blk + 31 < a1 ? blk + 31 : a1 - 1;  // the block's last row in the chunk (a partial block too)
  if (p.bt != nullptr && (last >> p.pg_shift) != (blk >> p.pg_shift)) l1 = kv_loc(p, sq, last);
  // this thread's row: contiguous, row t of page sq; paged, row t % pg_cap of
  // the first page or, past its end, of the second
  const bool second = p.bt != nullptr && (t >> p.pg_shift) != (blk >> p.pg_shift);
  const int pg = second ? l1.page : l0.page;
  const int r = p.bt != nullptr ? (t & (p.pg_cap - 1)) : t;
  const uint32_t row = (uint32_t)pg * (uint32_t)p.pg_cap + (uint32_t)r;
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int c16 = (threadIdx.x >> 5) + 8 * k;
    pf[k] = ld_x4<0>(crs, t < a1 ? (row * MLA_QA + c16 * 8) * 2u : OOB);
  }
}
// Row-major copy, and the transposed copy of the latent chunks (k < 8): the
// lanes of rows 2i and 2i+1 (adjacent lanes) swap halves so that each writes
// whole dwords (two positions) of four dims, even lane dims 0..3, odd lane 4..7.
__device__ __forceinline__ void mla_store_block(const i32x4 (&pf)[9]) {
  MlaSmem& sm = *(MlaSmem*)md_smem;
  const int rr = threadIdx.x & 31, odd = rr & 1, r0 = rr & ~1;
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int c16 = (threadIdx.x >> 5) + 8 * k;
    *(i32x4*)&sm.rows[rr][c16 * 8] = pf[k];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c16 = (threadIdx.x >> 5) + 8 * k;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = t + 2 * odd;  // this lane's dword of the chunk: dims 2q, 2q+1
      const uint32_t send = (uint32_t)(odd ? pf[k][t] : pf[k][t + 2]);
      const uint32_t par = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, DPP_QXOR1, 0xF, 0xF, false);
      const uint32_t own = (uint32_t)pf[k][q];
      const uint32_t lo = odd ? par : own, hi = odd ? own : par;  // position r0 in the low half
      *(uint32_t*)&sm.ct[c16 * 8 + 2 * q][r0] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      *(uint32_t*)&sm.ct[c16 * 8 + 2 * q + 1][r0] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
    }
  }
}

// The cache rows are read with the default policy (kept in the XCD's L2):
// the rows of earlier steps were written in earlier launches, and this
// step's new rows were written (written through) before the previous sync
// point and read by nobody before, so no L2 holds an older copy of them.
// The task's first two blocks are requested before the wait for the
// absorbed queries (the rows are final by then); two blocks stay in flight.
__device__ __forceinline__ void phase_mla_attn(KParams& pk, int l_layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  MlaSmem& sm = *(MlaSmem*)md_smem;
  const int B = p.B, nh = p.mla_h, C = p.mla_chunks;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nn = lane & 15, hh = nn >> 1, pp = nn & 1;
  const int h0 = 8 * wv;                      // scores and softmax: heads h0..h0+7
  const int hb = 16 * (wv & 1), db = 256 * (wv >> 1);  // P.C: heads hb..hb+15, dims db..db+255
  rsrc_t wr = make_rsrc_u(p.ws, p.ws_bytes);
  const rsrc_t crs = make_rsrc_u(p.kv + L.kv_off, (uint32_t)((size_t)p.n_pages * p.pg_cap * MLA_QA * 2));
  i32x4 pfA[9], pfB[9];  // blocks in flight
  // task geometry: chunk c of row b, cache rows [a0, a1)
  int b = 0, c = 0, pos = 0, a0 = 0, a1 = 0, sq = 0;
  auto task_of = [&](int task) __attribute__((always_inline)) {
    c = task % C;
    b = task / C;
    pos = row_pos(p, b);
    const int n = pos + 1;
    const int P = (n + C - 1) / C;
    a0 = c * P < n ? c * P : n;
    a1 = (c + 1) * P < n ? (c + 1) * P : n;
    sq = row_seq(p, b);
    if (a0 < a1) mla_load_block(p, pfA, crs, sq, a0, a1);
    if (a0 + 32 < a1) mla_load_block(p, pfB, crs, sq, a0 + 32, a1);
  };
  if ((int)blockIdx.x < B * C) task_of(blockIdx.x);
  wait_point(p, wait_idx);
  for (int task = blockIdx.x; task < B * C; task += gridDim.x) {
    if (task != (int)blockIdx.x) task_of(task);
    // this wave's heads' absorbed queries as hi/lo B operands
    bf16x8 qb[MLA_KS];
    {
      const int h = h0 + hh;
#pragma unroll
      for (int s = 0; s < MLA_KS; ++s) {
        i32x4 v0 = ld_x4<CP_SC1>(wr, h < nh ? p.off_qabs + (uint32_t)((b * nh + h) * MLA_QA + s * 32 + (lane >> 4) * 8) * 4u : OOB);
        i32x4 v1 = ld_x4<CP_SC1>(wr, h < nh ? p.off_qabs + (uint32_t)((b * nh + h) * MLA_QA + s * 32 + (lane >> 4) * 8 + 4) * 4u : OOB);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float v = __int_as_float(k < 4 ? v0[k] : v1[k - 4]);
          uint16_t hi, lo;
          split_hilo(v, hi, lo);
          qb[s][k] = __builtin_bit_cast(__bf16, pp ? lo : hi);
        }
      }
    }
    float m_run[8], l_run[8];
    f32x4 z[16];  // tile j: dims db + 16j + 4*(lane/16) + i, head hb + nn
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      m_run[h] = -INFINITY;
      l_run[h] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a0 < a1) mla_store_block(pfA);
    __syncthreads();
    // block blk (in LDS): its scores, softmax and P.C; nxt holds block
    // blk + 32 (in flight), spare is free and takes block blk + 64
    auto step = [&](const i32x4 (&nxt)[9], i32x4 (&spare)[9], int blk) __attribute__((always_inline)) {
      if (blk + 64 < a1) mla_load_block(p, spare, crs, sq, blk + 64, a1);
      // scores of 32 positions x this wave's 8 heads
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < MLA_KS; ++s) {
          i32x4 kv = *(const i32x4*)&sm.rows[tt * 16 + (lane & 15)][s * 32 + (lane >> 4) * 8];
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qb[s], a, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = a[i] + dpp_f<DPP_QXOR1>(a[i]);
          int pr = tt * 16 + 4 * (lane >> 4) + i;
          if (!pp) sm.s[pr][h0 + hh] = (blk + pr < a1) ? v : -INFINITY;
        }
      }
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      __builtin_amdgcn_wave_barrier();
      // online softmax per head (positions past the chunk end have p = 0)
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        float sv = lane < 32 ? sm.s[lane][h0 + h] : -INFINITY;
        float mb = wave_max(sv);
        float mn = fmaxf(m_run[h], mb);
        const float corr = __expf(m_run[h] - mn);
        float pv = lane < 32 ? __expf(sv - mn) : 0.f;
        l_run[h] = l_run[h] * corr + wave_sum(pv);
        m_run[h] = mn;
        if (lane < 32) {
          uint16_t hi, lo;
          split_hilo(pv, hi, lo);
          sm.pb[0][h0 + h][lane] = hi;
          sm.pb[1][h0 + h][lane] = lo;
        }
        if (lane == 0) sm.corr[h0 + h] = corr;
      }
      __syncthreads();  // P and the rescales of every head
      // z += P.C for heads hb..hb+15, dims db..db+255
      {
        const float cr = sm.corr[hb + nn];
        const bf16x8 ph = *(const bf16x8*)&sm.pb[0][hb + nn][8 * (lane >> 4)];
        const bf16x8 pl = *(const bf16x8*)&sm.pb[1][hb + nn][8 * (lane >> 4)];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const i32x4 cv = *(const i32x4*)&sm.ct[db + 16 * j + (lane & 15)][8 * (lane >> 4)];
          f32x4 acc = z[j] * cr;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cv), ph, acc, 0, 0, 0);
          z[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cv), pl, acc, 0, 0, 0);
        }
      }
      __syncthreads();  // every wave is done with this block's rows, transposed copy and P
      if (blk + 32 < a1) {
        mla_store_block(nxt);
        __syncthreads();
      }
    };
    for (int blk = a0; blk < a1; blk += 64) {
      step(pfB, pfA, blk);
      if (blk + 32 < a1) step(pfA, pfB, blk + 32);
    }
    // partials: (m, l) of the softmax heads by lane 0; z of the P.C heads, 4 dims per tile
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const int hg = h0 + h;
      if (hg >= nh) break;
      const uint32_t idx = (uint32_t)((b * C + c) * nh + hg);
      if (lane == 0) {
        st_f32(wr, p.off_mml + idx * 8u, m_run[h]);
        st_f32(wr, p.off_mml + idx * 8u + 4u, l_run[h]);
      }
    }
    {
      const int hg = hb + nn;
      const uint32_t idx = (uint32_t)((b * C + c) * nh + (hg < nh ? hg : 0));
#pragma unroll
      for (int j = 0; j < 16; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, z[j]), wr,
                                               hg < nh ? p.off_mz + (idx * MLA_KL + db + 16 * j + 4 * (lane >> 4)) * 4u : OOB,
                                               0, CP_SC1);
    }
    __syncthreads();
  }
}

// M5: combine the chunks of each head and un-absorb: o_h = W_uv,h z_h.
// The nsl = v_dim/32 tasks of a head first split its 512 latent dims for the
// combine (each reads a quarter of the chunk partials when nsl = 4, with the
// chunks shared out over all threads so that one round of loads covers them),
// publish the combined z to the workspace and count themselves in a per-head
// word; then task (h, sl) waits for that count and multiplies the whole z by
// its 32-row slice of W_uv,h, whose loads were issued before the wait.
// parts: 1 = the combine, 2 = the rows, 3 = both (the multi-launch step runs
// them as two launches).  Inlined into the kernel, as the attention phases
// are, so that those registers are not saved and restored through scratch.
__device__ __forceinline__ void phase_mla_out(KParams& pk, int l_layer, int parts) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int B = p.B, nh = p.mla_h, nope = p.nope, vd = p.vdim, VW = nope + vd, C = p.mla_chunks;
  const int nsl = vd / 32;
  const int ntask = nh * nsl;
  constexpr int OT = 8;          // tokens per tile (one tile up to 8 rows)
  float* z = &GSM.in[0][0];      // [OT][512]
  float* cw = &GSM.out[0][0];    // [OT][256] combine weights
  float* cl = cw + OT * 256;     // [OT] 1 / denominator
  float* cs = cl + OT;           // [OT][256] chunk sums
  float* zp = &GSM.red[0][0][0][0][0];  // [NT][4] sums over a share of the chunks
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  rsrc_t wrs = make_rsrc_u(L.mla_wkvb, (uint32_t)((size_t)nh * VW * MLA_KL * 2));
  unsigned* ready = sync_pt(p, p.sync_attn_base + l_layer);  // per head: parts of z published
  // Part 1: task (h, q) combines dims [d0, d1) of head h's z over the chunks
  // and publishes them; the nsl tasks of a head split the 512 dims.
  for (int task = blockIdx.x; (parts & 1) && task < ntask; task += gridDim.x) {
    const int h = task / nsl, q = task % nsl;
    const int d0 = 4 * ((q * (MLA_KL / 4)) / nsl), nd4 = ((q + 1) * (MLA_KL / 4)) / nsl - d0 / 4;
    for (int t0 = 0; t0 < B; t0 += OT) {
    const int Bt = B - t0 < OT ? B - t0 : OT;
    if (t0 > 0) __syncthreads();  // the previous tile is done with cw, cs, cl and zp
    for (int e = threadIdx.x; e < Bt * C; e += NT) {
      int t = e / C, cc = e % C;
      cw[t * 256 + cc] = ld_f32(r, p.off_mml + (uint32_t)(((t0 + t) * C + cc) * nh + h) * 8u);
      cs[t * 256 + cc] = ld_f32(r, p.off_mml + (uint32_t)(((t0 + t) * C + cc) * nh + h) * 8u + 4u);
    }
    __syncthreads();
    for (int t = threadIdx.x >> 6; t < Bt; t += NW) {  // one wave per token: max, weights, denominator
      const int ln = threadIdx.x & 63;
      float M = -INFINITY;
      for (int cc = ln; cc < C; cc += 64) M = fmaxf(M, cw[t * 256 + cc]);
      M = wave_max(M);
      float den = 0.f;
      for (int cc = ln; cc < C; cc += 64) {
        float f = cw[t * 256 + cc] == -INFINITY ? 0.f : __expf(cw[t * 256 + cc] - M);
        cw[t * 256 + cc] = f;
        den += f * cs[t * 256 + cc];
      }
      den = wave_sum(den);
      if (ln == 0) cl[t] = 1.0f / den;
    }
    __syncthreads();
    // thread per (share s of the chunks, token, 4 dims), MZU chunk loads in flight
    constexpr int MZU = 32;
    const int items = Bt * nd4;
    const int S = items < NT ? NT / items : 1;
    const int per = (C + S - 1) / S;
    for (int e = threadIdx.x; e < items * S; e += NT) {
      const int sh = e / items, it = e % items;
      const int t = it / nd4, d4 = d0 + (it % nd4) * 4;
      const int ca = sh * per, cb = ca + per < C ? ca + per : C;
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
      for (int c0 = ca; c0 < cb; c0 += MZU) {
        i32x4 v[MZU];
#pragma unroll
        for (int u = 0; u < MZU; ++u)
          v[u] = ld_x4<CP_SC1>(r, c0 + u < cb ? p.off_mz + ((uint32_t)(((t0 + t) * C + c0 + u) * nh + h) * MLA_KL + d4) * 4u : OOB);
#pragma unroll
        for (int u = 0; u < MZU; ++u) {
          float f = c0 + u < cb ? cw[t * 256 + c0 + u] : 0.f;
          o0 += f * __int_as_float(v[u][0]);
          o1 += f * __int_as_float(v[u][1]);
          o2 += f * __int_as_float(v[u][2]);
          o3 += f * __int_as_float(v[u][3]);
        }
      }
      if (S == 1) {
        const float il = cl[t];
        const uint32_t at = p.off_mzc + ((uint32_t)((t0 + t) * nh + h) * MLA_KL + d4) * 4u;
        st_f32(r, at, o0 * il);
        st_f32(r, at + 4u, o1 * il);
        st_f32(r, at + 8u, o2 * il);
        st_f32(r, at + 12u, o3 * il);
      } else {
        zp[e * 4 + 0] = o0;
        zp[e * 4 + 1] = o1;
        zp[e * 4 + 2] = o2;
        zp[e * 4 + 3] = o3;
      }
    }
    if (S > 1) {  // add the shares (e < items * S <= NT above)
      __syncthreads();
      for (int it = threadIdx.x; it < items; it += NT) {
        const int t = it / nd4, d4 = d0 + (it % nd4) * 4;
        float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
        for (int sh = 0; sh < S; ++sh) {
          o0 += zp[(sh * items + it) * 4 + 0];
          o1 += zp[(sh * items + it) * 4 + 1];
          o2 += zp[(sh * items + it) * 4 + 2];
          o3 += zp[(sh * items + it) * 4 + 3];
        }
        const float il = cl[t];
        const uint32_t at = p.off_mzc + ((uint32_t)((t0 + t) * nh + h) * MLA_KL + d4) * 4u;
        st_f32(r, at, o0 * il);
        st_f32(r, at + 4u, o1 * il);
        st_f32(r, at + 8u, o2 * il);
        st_f32(r, at + 12u, o3 * il);
      }
    }
    }
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) (void)__hip_atomic_fetch_add(ready + h, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Part 2: task (h, sl) computes o rows sl*32 .. sl*32+31 of head h from
  // the whole combined z, once the nsl parts of it are published.  Every
  // workgroup publishes all of its parts before it waits for any, so the
  // wait ends whatever the grid size.
  for (int task = blockIdx.x; (parts & 2) && task < ntask; task += gridDim.x) {
    const int h = task / nsl, sl = task % nsl;
    const int row = sl * 32 + (threadIdx.x >> 3), part = threadIdx.x & 7;
    i32x4 wv[8];  // this lane's 64 dims of its row, requested before the wait
#pragma unroll
    for (int k = 0; k < 8; ++k) wv[k] = ld_x4<0>(wrs, (uint32_t)((h * VW + nope + row) * MLA_KL + part * 64 + k * 8) * 2u);
    if (threadIdx.x < 64) {
      unsigned spins = 0;
      while (true) {
        const unsigned v = __hip_atomic_load(ready + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v >= (unsigned)nsl) break;
        __builtin_amdgcn_s_sleep(1);
        if (((++spins) & 1023u) == 0 && (spins > p.spin_limit || dev_failed(p))) {
          if (threadIdx.x == 0) set_err(p, MDE_WATCHDOG);
          break;
        }
      }
    }
    __syncthreads();
    for (int t0 = 0; t0 < B; t0 += OT) {
    const int Bt = B - t0 < OT ? B - t0 : OT;
    if (t0 > 0) __syncthreads();  // the previous tile is done with z
    for (int e = threadIdx.x; e < Bt * (MLA_KL / 4); e += NT) {
      const int t = e / (MLA_KL / 4), d4 = (e % (MLA_KL / 4)) * 4;
      const i32x4 v = ld_x4<CP_SC1>(r, p.off_mzc + ((uint32_t)((t0 + t) * nh + h) * MLA_KL + d4) * 4u);
      z[t * MLA_KL + d4 + 0] = __int_as_float(v[0]);
      z[t * MLA_KL + d4 + 1] = __int_as_float(v[1]);
      z[t * MLA_KL + d4 + 2] = __int_as_float(v[2]);
      z[t * MLA_KL + d4 + 3] = __int_as_float(v[3]);
    }
    __syncthreads();
    // o[t][row]: 8 lanes per row, 64 dims each
    {
      float ot[OT];
#pragma unroll
      for (int t = 0; t < OT; ++t) ot[t] = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        int d = part * 64 + k * 8;
        float wf[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wf[2 * j] = __uint_as_float((uint32_t)wv[k][j] << 16);
          wf[2 * j + 1] = __uint_as_float((uint32_t)wv[k][j] & 0xFFFF0000u);
        }
#pragma unroll
        for (int t = 0; t < OT; ++t) {
          if (t < Bt) {
#pragma unroll
            for (int j = 0; j < 8; ++j) ot[t] += wf[j] * z[t * MLA_KL + d + j];
          }
        }
      }
#pragma unroll
      for (int t = 0; t < OT; ++t) {
        float v = ot[t];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        ot[t] = v;
      }
      if (part == 0) {
        for (int t = 0; t < Bt; ++t) put_hilo(r, ou_at(p, l_layer), nh * vd, t0 + t, h * vd + row, ot[t]);
      }
    }
    }
    __syncthreads();
  }
}

// Routing state of the current MoE layer (section "Our Kimi K3 megakernel":
// router, then shared and routed experts).  It lives in LDS past every
// phase's own block, so it survives from the routed gate/up phase to the
// down projections.
struct RouteSmem {
  int nu;                 // |U|
  int u[64];              // U, ascending expert id
  int pos[64];            // expert id -> index in U, or -1
  int ids[MAXB][8];       // chosen experts per token, in descending router order
  float w[MAXB][8];       // their weights
  float wt[MAXB][64];     // weight of U entry j for token t (0: not chosen)
  const uint16_t* ex[64][3];  // gate, up, down weights of U entry j
  const uint16_t* exall[64][3];  // every expert's (fetched before the routing is known)
  uint64_t mask[MAXB];    // experts each token chose
};
constexpr size_t cmax_(size_t a, size_t b) { return a > b ? a : b; }
constexpr size_t ROUTE_OFF =
    (cmax_(cmax_(sizeof(GemvSmem) + (WIDE ? 0 : (size_t)1024 * MAXB * 4), sizeof(AttnSmem)), cmax_(sizeof(MlaSmem), sizeof(KdaSmem))) + 63) /
    64 * 64;
#define RSM (*reinterpret_cast<RouteSmem*>(md_smem + ROUTE_OFF))
static_assert(ROUTE_OFF + sizeof(RouteSmem) <= PLAN_OFF, "LDS layout exceeds the static LDS block");

// --- residual-owning projections: x[t][r] += sum over the phase's matrices
// of W . U (the O-projection; the dense down projection; the shared and
// routed expert down projections, whose inputs already carry the routing
// weights), then the next norm's input U = hilo(g_next * x) and this WG's
// sum of squares of x.
enum : int { RES_OPROJ = 0, RES_DENSE_DOWN = 1, RES_MOE_DOWN = 2, RES_MLA_O = 3, RES_KDA_O = 4 };

MD_PHASE_FN void phase_residual(KParams& pk, int l_layer, int mode, const uint16_t* g_next, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int B = p.B, H = p.H;
  const RowSplit own = owned_rows(H, blockIdx.x, gridDim.x);
  const int nrow = own.r1 - own.r0;
  SlotBuilder sb;
  if (threadIdx.x < 64) {
    sb.start(mode == RES_OPROJ ? PL_OPROJ : mode == RES_DENSE_DOWN ? PL_DDOWN : mode == RES_MLA_O ? PL_MLA_O : mode == RES_KDA_O ? PL_KDA_O : -1);
    if (mode == RES_OPROJ) {
      int m = sb.mat(L.wo, H, p.nq * p.hd, 0);
      sb.begin(ou_at(p, l_layer), p.nq * p.hd, GK_SINGLE);
      sb.singles_of(m, H);
    } else if (mode == RES_MLA_O) {
      int m = sb.mat(L.mla_wo, H, p.mla_h * p.vdim, 0);
      sb.begin(ou_at(p, l_layer), p.mla_h * p.vdim, GK_SINGLE);
      sb.singles_of(m, H);
    } else if (mode == RES_KDA_O) {
      int m = sb.mat(L.kda_wo, H, p.kda_h * p.kda_dv, 0);
      sb.begin(ou_at(p, l_layer), p.kda_h * p.kda_dv, GK_SINGLE);
      sb.singles_of(m, H);
    } else if (mode == RES_DENSE_DOWN) {
      int m = sb.mat(L.w_down, H, p.ffn, 0);
      sb.begin(h_at(p, l_layer), p.ffn, GK_SINGLE);
      sb.singles_of(m, H);
    } else {
      if (p.n_shared > 0) {
        int m = sb.mat(L.sh_down, H, p.shared_ffn, 0);
        sb.begin(hs_at(p, l_layer), p.shared_ffn, GK_SINGLE);
        sb.singles_of(m, H);
      }
      const int nu = __builtin_amdgcn_readfirstlane(RSM.nu);
      const int m0 = sb.expert_mats<1>(RSM.ex, nu, 2, H, p.expert_ffn, false);
      sb.expert_singles(m0, nu, H, hr_at(p, l_layer), p.hr_stride, p.expert_ffn);
    }
  }
  builder_done(p, sb, nrow);
  const int r0 = own.r0;
  // the next norm's input: this layer's FFN input after an attention block,
  // the next layer's attention input (or the final norm's) after the FFN
  const bool attn_block = mode == RES_OPROJ || mode == RES_MLA_O || mode == RES_KDA_O;
  const int nxt = 2 * l_layer + (attn_block ? 1 : 2);
  const uint32_t u_next = u_at(p, nxt);
  gemv_phase(p, wait_idx, 0, 0u, EPI_RESIDUAL, r0, nrow, g_next);
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  auto elem = [&](int t, int lr) -> float {
    float x = GSM.out[lr][t];
    p.x[t * H + r0 + lr] = x;
    put_hilo(r, u_next, H, t, r0 + lr, GSM.gain[lr] * x);
    return x * x;
  };
  if constexpr (WIDE) {
    float acc = 0.f;
    const int t = threadIdx.x & 63;
    if (t < B)
      for (int lr = threadIdx.x >> 6; lr < nrow; lr += NT / 64) acc += elem(t, lr);
    store_ssq_wide(p, r, acc, ssq_at(p, nxt));
  } else {
    static_assert(WIDE || sizeof(GemvSmem::red) >= sizeof(float) * (NT + NW) * MAXB, "partial sums reuse the reduction scratch");
    float* part = (float*)GSM.red;  // [NT][MAXB]
    for (int t = 0; t < MAXB; ++t) part[threadIdx.x * MAXB + t] = 0.f;
    for (int e = threadIdx.x; e < nrow * B; e += NT) {
      int t = e % B, lr = e / B;
      part[threadIdx.x * MAXB + t] += elem(t, lr);
    }
    store_ssq(p, r, part, ssq_at(p, nxt));
  }
}

// --- dense SwiGLU gate/up: h = silu(inv*Wg U) * (inv*Wu U) -> hi/lo
MD_PHASE_FN void phase_gateup(KParams& pk, int l_layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int B = p.B, F = p.ffn;
  SlotBuilder sb;
  if (threadIdx.x < 64) {
    sb.start(PL_GATEUP);
    int mg = sb.mat(L.w_gate, F, p.H, 0);
    int mu = sb.mat(L.w_up, F, p.H, 0);
    sb.begin(u_at(p, 2 * l_layer + 1), p.H, GK_PAIR);
    sb.pairs_of(mg, mu, F);
  }
  builder_done(p, sb, -1);
  gemv_passes(p, wait_idx, p.H, ssq_at(p, 2 * l_layer + 1), [&](int s0, int s1) {
    rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
    for_quarters(s0, s1, B, [&](int si, int sr0, int t, int m, int row0, int n) {
      if (si & 1) return;  // up slots carry no output (passes start on even slots)
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = GSM.out[sr0 + i][t];
      put_hilo4(r, h_at(p, l_layer), F, t, row0, v, n);
    });
  });
}

// ------------------------------------------------------------------ MoE
// Section "Our Kimi K3 megakernel" of the pages orders a MoE layer as router,
// shared expert, routed experts.  Phase A streams the router (E rows) and the
// shared expert's gate/up; after the sync every workgroup derives the
// routing from the fp32 router logits itself (same data, same fixed order,
// so every copy is identical and no further sync is needed); phase B streams
// the gate/up of the experts any token chose (their union U, ascending id),
// scaling each token's h by its routing weight (0 when it did not choose the
// expert); the down projections of the shared and the routed experts then
// run as one residual phase.
// Phase B reads the same input as phase A and none of A's shared-expert
// outputs (those are read by the down projection, whose wait for phase B's
// arrivals covers them: every workgroup arrives at B after A).  It needs
// only the router logits, and those carry their own proof of freshness: each
// 8-byte entry holds the logit and a tag naming the step and the layer, so a
// reader checks the tags of what it read (and reads again until they match)
// instead of waiting at a sync point.  Phase A has no arrival.

// Workgroups that hold the router alone (the last ones, one 4-row quarter
// each), or 0 when every workgroup holds router rows: the router's few
// quarters go apart when there is a shared expert and the grid is more than
// twice their count (a router quarter is a whole group of k-steps, which on
// top of a shared-expert group would double that workgroup's stream).
__device__ __forceinline__ int router_wgs(KParams& pk) {
  PARAMS;
  const int rq = (p.n_experts + 3) >> 2;
  return p.n_shared > 0 && (int)gridDim.x > 2 * rq ? rq : 0;
}

MD_PHASE_FN void phase_moe_a(KParams& pk, int l_layer, int wait_idx) {
  PARAMS;
  KLayer& L = layer_ref(p, l_layer);
  const int B = p.B;
  // every expert's weight pointers for phase B: requested now, entered into
  // LDS once wave 0 has built the tables (the load hides behind the builder;
  // phase B needs no load before its own tables)
  const int nep = 3 * p.n_experts;
  const uint16_t* ep = (int)threadIdx.x < nep ? L.experts[threadIdx.x] : nullptr;
  SlotBuilder sb;
  if (threadIdx.x < 64) {
    sb.start(PL_MOE_A);
    const int G = gridDim.x, w = blockIdx.x, rq = (p.n_experts + 3) >> 2;
    const bool apart = router_wgs(p) > 0;
    if (p.n_shared > 0) {
      int mg = sb.mat(L.sh_gate, p.shared_ffn, p.H, 0);
      int mu = sb.mat(L.sh_up, p.shared_ffn, p.H, 0);
      sb.begin(u_at(p, 2 * l_layer + 1), p.H, GK_PAIR);
      const int nq = (p.shared_ffn + 3) >> 2;
      if (!apart) sb.pairs_of(mg, mu, p.shared_ffn);
      else if (w < G - rq) sb.pairs_in(mg, mu, rows_of(nq, w, G - rq));
    }
    int mr = sb.mat(L.router, p.n_experts, p.H, -1);
    sb.begin(u_at(p, 2 * l_layer + 1), p.H, GK_SINGLE);
    if (!apart) {
      sb.singles_of(mr, p.n_experts);
    } else if (w >= G - rq) {
      RowSplit q;
      q.r0 = w - (G - rq);
      q.r1 = q.r0 + 1;
      sb.singles_in(mr, q);
    }
  }
  if ((int)threadIdx.x < nep) RSM.exall[threadIdx.x / 3][threadIdx.x % 3] = ep;
  builder_done(p, sb, -1);
  gemv_passes(p, wait_idx, p.H, ssq_at(p, 2 * l_layer + 1), [&](int s0, int s1) {
    rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
    for_quarters(s0, s1, B, [&](int si, int sr0, int t, int m, int row0, int n) {
      const bool pair = GSM.grp[si / TG].kind == GK_PAIR;
      if (pair && (si & 1)) return;  // up slots carry no output
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = GSM.out[sr0 + i][t];
      if (pair) {
        put_hilo4(r, hs_at(p, l_layer), p.shared_ffn, t, row0, v, n);
      } else {
        for (int i = 0; i < n; ++i) put_logit(p, l_layer, t, row0 + i, v[i]);
      }
    });
  });
}

// Routing of every token from the router logits (fp32, written by phase A):
// the top_k experts by logit, larger first and the lower id on ties;
// weights softmax(logits) over all experts at the chosen ones, renormalised
// over the chosen ones when norm_topk.  Every workgroup runs this on the same
// data in the same order.  Workgroup 0 reports the choices.
// Every expert's weight pointers of the layer into LDS.  They do not depend
// on the routing, so this runs before the wait for the router logits.
__device__ __forceinline__ void prefetch_experts(KParams& pk, int layer) {
  PARAMS;
  KLayer& L = layer_ref(p, layer);
  for (int i = threadIdx.x; i < p.n_experts * 3; i += NT) RSM.exall[i / 3][i % 3] = L.experts[i];
}

// in: this wave's entries as route_load read them (requested earlier, so
// their latency overlaps other work); read again until every tag is this
// layer's.
__device__ __noinline__ void compute_routes(KParams& pk, int layer, RouteIn in) {
  PARAMS;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int E = p.n_experts, k = p.top_k, B = p.B;
  const uint32_t tag = rl_tag(p, layer);
  for (unsigned spins = 0;; ++spins) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < RTPW; ++i) {
      const int t = wv + NW * i;
      if (t < B && lane < E && (uint32_t)(in.v[i] >> 32) != tag) ok = false;
    }
    if (__all(ok)) break;
    if (((spins + 1) & 1023u) == 0 && (spins > p.spin_limit || dev_failed(p))) {
      if (lane == 0) set_err(p, MDE_WATCHDOG);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    route_load(p, in);
  }
  float lgs[RTPW];
#pragma unroll
  for (int i = 0; i < RTPW; ++i) lgs[i] = __uint_as_float((uint32_t)in.v[i]);
#pragma unroll
  for (int i = 0; i < RTPW; ++i) {
    const int t = wv + NW * i;
    if (t >= B) break;
    // lane e holds expert e (a NaN logit counts as -inf, so that the ranks
    // below are a permutation)
    const float lg = (lane < E && lgs[i] == lgs[i]) ? lgs[i] : -INFINITY;
    const float mx0 = wave_max(lg);
    const float pe = lane < E ? __expf(lg - mx0) : 0.f;
    const float all = wave_sum(pe);
    // rank of expert e: the experts with a larger logit, or an equal one and
    // a lower id; the chosen are ranks 0 .. k-1, in that order
    int rank = 0;
    for (int j = 0; j < E; ++j) {
      const float lj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lg), j));
      rank += (lj > lg || (lj == lg && j < lane)) ? 1 : 0;
    }
    const bool taken = lane < E && rank < k;
    if (taken) { RSM.ids[t][rank] = lane; RSM.w[t][rank] = pe; }
    const uint64_t chosen = __ballot(taken);
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_wave_barrier();
    float sel = 0.f;  // the chosen probabilities, larger first
    for (int j = 0; j < k; ++j) sel += RSM.w[t][j];
    const float den = p.norm_topk ? sel : all;
    const float wj = lane < k ? RSM.w[t][lane] : 0.f;
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_wave_barrier();
    if (lane < k) RSM.w[t][lane] = wj / den;
    if (lane == 0) RSM.mask[t] = chosen;
  }
  for (int i = threadIdx.x; i < MAXB * 64; i += NT) RSM.wt[i >> 6][i & 63] = 0.f;
  __syncthreads();
  if (threadIdx.x < 64) {  // U = the union, ascending; expert e (lane e) sits at popcount of the ids below it
    uint64_t mask = 0;
    for (int t = 0; t < B; ++t) mask |= RSM.mask[t];
    if (p.moe_all) mask = E == 64 ? ~0ull : (1ull << E) - 1ull;  // every expert streams (weight 0 if unchosen)
    const bool in = (mask >> lane) & 1ull;
    const int at = __popcll(mask & ((1ull << lane) - 1ull));
    if (in) RSM.u[at] = lane;
    RSM.pos[lane] = in ? at : -1;
    if (lane == 0) RSM.nu = __popcll(mask);
  }
  __syncthreads();
  // the chosen experts' weight pointers (the slot builders read them here)
  for (int i = threadIdx.x; i < RSM.nu * 3; i += NT) RSM.ex[i / 3][i % 3] = RSM.exall[RSM.u[i / 3]][i % 3];
  for (int e = threadIdx.x; e < B * k; e += NT) {
    int t = e / k, j = e % k;
    RSM.wt[t][RSM.pos[RSM.ids[t][j]]] = RSM.w[t][j];
    if (blockIdx.x == 0 && p.out_ids) p.out_ids[((size_t)layer * B + t) * k + j] = RSM.ids[t][j];
  }
  __syncthreads();
}

// route_after (p.moe_all): every expert's gate/up streams, so the tables
// need no routing and the stream waits for nobody (its input and scales were
// ready for phase A); the router logits are requested behind the stream's
// first weight loads (8-row build) and the routing runs after the stream,
// before the outputs are scaled (experts no token chose get weight 0).
// Otherwise the routing is done and the chosen experts' union is streamed.
MD_PHASE_FN void phase_moe_b(KParams& pk, int l_layer, bool route_after) {
  PARAMS;
  const int B = p.B;
  SlotBuilder sb;
  if (route_after) __syncthreads();  // every expert's pointers (loaded in phase A) are in LDS
  if (threadIdx.x < 64) {
    sb.start();
    sb.begin(u_at(p, 2 * l_layer + 1), p.H, GK_PAIR);
    const int nu = route_after ? p.n_experts : __builtin_amdgcn_readfirstlane(RSM.nu);
    const int m0 = sb.expert_mats<2>(route_after ? RSM.exall : RSM.ex, nu, 0, p.expert_ffn, p.H, true);
    sb.expert_pairs(m0, nu, p.expert_ffn);
  }
  builder_done(p, sb, -1);
  auto post = [&](int s0, int s1) {
    rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
    for_quarters(s0, s1, B, [&](int si, int sr0, int t, int m, int row0, int n) {
      if (si & 1) return;  // up slots carry no output
      const int j = GSM.mats[m].tag;
      const float wj = RSM.wt[t][j];
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = GSM.out[sr0 + i][t] * wj;
      put_hilo4(r, hr_at(p, l_layer) + (uint32_t)j * p.hr_stride, p.expert_ffn, t, row0, v, n);
    });
  };
  if constexpr (!WIDE) {
    if (route_after) {
      const RouteIn in = gemv_phase(p, -1, p.H, ssq_at(p, 2 * l_layer + 1), EPI_BY_KIND, 0, 0, nullptr, 0, -1, true);
      compute_routes(p, l_layer, in);
      post(0, __builtin_amdgcn_readfirstlane(GSM.nslots));
      return;
    }
  }
  gemv_passes(p, -1, p.H, ssq_at(p, 2 * l_layer + 1), [&](int s0, int s1) {
    if (route_after && s0 == 0) {
      RouteIn in;
      route_load(p, in);
      compute_routes(p, l_layer, in);
    }
    post(s0, s1);
  });
}

// --- final norm + LM head: logits, per-WG argmax candidates
MD_PHASE_FN void phase_lmhead(KParams& pk, int wait_idx) {
  PARAMS;
  const int B = p.B;
  SlotBuilder sb;
  if (threadIdx.x < 64) {
    sb.start(PL_LMHEAD);
    int m = sb.mat(p.lm_head, p.V, p.H, 0);
    sb.begin(u_at(p, p.n_layers * 2), p.H, GK_SINGLE);
    sb.singles_of(m, p.V);
  }
  builder_done(p, sb, -1);
  rsrc_t r = make_rsrc_u(p.ws, p.ws_bytes);
  if constexpr (WIDE) {
    // thread tid keeps the best logit of token tid % 64 over its rows of
    // every pass; then the four waves' candidates of a token, in order
    float cb = -INFINITY;
    int ci = 0x7FFFFFFF;
    const int t = threadIdx.x & 63;
    gemv_passes(p, wait_idx, p.H, ssq_at(p, 2 * p.n_layers), [&](int s0, int s1) {
      if (t >= B) return;
      for (int sr = threadIdx.x >> 6; sr < (s1 - s0) * 16; sr += NT / 64) {
        int m, v;
        if (!slot_row(s0 + (sr >> 4), sr & 15, m, v)) continue;
        const float lg = GSM.out[sr][t];
        p.logits[(size_t)t * p.V + v] = lg;
        if (lg > cb || (lg == cb && v < ci)) { cb = lg; ci = v; }
      }
    });
    float* bv = (float*)GSM.red;  // [NT]
    int* bi = (int*)(bv + NT);    // [NT]
    __syncthreads();
    bv[threadIdx.x] = cb;
    bi[threadIdx.x] = ci;
    __syncthreads();
    if (threadIdx.x < B) {
      float best = -INFINITY;
      int idx = 0x7FFFFFFF;
      for (int w = 0; w < NW; ++w) {
        const float v = bv[64 * w + t];
        const int k = bi[64 * w + t];
        if (v > best || (v == best && k < idx)) { best = v; idx = k; }
      }
      st_f32(r, p.off_cand + (uint32_t)(blockIdx.x * MAXB + t) * 8u, best);
      st_u32(r, p.off_cand + (uint32_t)(blockIdx.x * MAXB + t) * 8u + 4u, (uint32_t)idx);
    }
  } else {
    gemv_phase(p, wait_idx, p.H, ssq_at(p, 2 * p.n_layers), EPI_BY_KIND, 0, 0, nullptr);
    static_assert(WIDE || sizeof(GemvSmem::in) >= 2 * sizeof(float) * NT * MAXB, "argmax scratch reuses the input staging");
    float* bv = &GSM.in[0][0];             // [NT][MAXB] best value (the input staging is unused here)
    int* bi = (int*)(bv + NT * MAXB);      // [NT][MAXB] best index
    for (int t = 0; t < MAXB; ++t) { bv[threadIdx.x * MAXB + t] = -INFINITY; bi[threadIdx.x * MAXB + t] = 0x7FFFFFFF; }
    for (int e = threadIdx.x; e < GSM.nslots * 16 * B; e += NT) {
      int t = e % B, sr = e / B;
      int m, v;
      if (!slot_row(sr >> 4, sr & 15, m, v)) continue;
      float lg = GSM.out[sr][t];
      p.logits[(size_t)t * p.V + v] = lg;
      float& cb = bv[threadIdx.x * MAXB + t];
      int& ci = bi[threadIdx.x * MAXB + t];
      if (lg > cb || (lg == cb && v < ci)) { cb = lg; ci = v; }
    }
    __syncthreads();
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
}

// final argmax over the WG candidates (one workgroup)
__device__ __noinline__ void final_argmax(KParams& pk) {
  PARAMS;
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

// ===================================================================== multi-launch
// The same step as one kernel launch per phase (the kernel boundary is the
// barrier): the baseline whose inter-kernel gaps the megakernel removes.
// Every launch is md_megakernel itself in its one-phase mode (a second kernel
// calling the same phase functions would make every LDS access in them go
// through a per-kernel address table in memory), on the same grid, so the
// results are identical.  LDS does not survive a launch, so the routed
// experts' down projection recomputes the routing (same data, same result).
enum : int {
  PH_EMBED = 0, PH_QKV, PH_KV_WRITE, PH_ATTN, PH_OPROJ, PH_GATEUP, PH_DOWN, PH_MOE_A, PH_MOE_B, PH_MOE_C,
  PH_KDA_PROJ, PH_KDA_REC, PH_KDA_O, PH_MLA_A, PH_MLA_B, PH_MLA_ABS, PH_MLA_ATTN, PH_MLA_OUT, PH_MLA_O,
  PH_LMHEAD, PH_ARGMAX, PH_MLA_OUT2
};

__device__ __forceinline__ void run_one_phase(KParams& pk, int layer, int phase) {
  PARAMS;
  const int l = layer < 0 ? 0 : layer;
  const int l_layer = l;
  KLayer& L = layer_ref(p, l);
  const uint16_t* g_next = (l + 1 < p.n_layers) ? layer_ref(p, l + 1).attn_norm : p.final_norm;
  switch (phase) {
    case PH_EMBED: clear_next_bank(p); phase_embed(p); break;
    case PH_QKV: phase_qkv(p, l_layer, -1); break;
    case PH_KV_WRITE: phase_gqa_kv_write(p, l_layer); break;
    case PH_ATTN: phase_attn_gqa(p, l_layer, l, -1); break;
    case PH_OPROJ: phase_residual(p, l_layer, RES_OPROJ, L.ffn_norm, -1); break;
    case PH_GATEUP: phase_gateup(p, l_layer, -1); break;
    case PH_DOWN: phase_residual(p, l_layer, RES_DENSE_DOWN, g_next, -1); break;
    case PH_MOE_A: phase_moe_a(p, l_layer, -1); break;
    case PH_MOE_B: {
      prefetch_experts(p, l);
      RouteIn in;
      route_load(p, in);
      compute_routes(p, l, in);
      phase_moe_b(p, l_layer, false);
      break;
    }
    case PH_MOE_C: {
      prefetch_experts(p, l);
      RouteIn in;
      route_load(p, in);
      compute_routes(p, l, in);
      phase_residual(p, l_layer, RES_MOE_DOWN, g_next, -1);
      break;
    }
    case PH_KDA_PROJ: phase_kda_proj(p, l_layer, -1); break;
    case PH_KDA_REC: phase_kda_rec(p, l_layer, -1); break;
    case PH_KDA_O: phase_residual(p, l_layer, RES_KDA_O, L.ffn_norm, -1); break;
    case PH_MLA_A: phase_mla_a(p, l_layer, -1); break;
    case PH_MLA_B: phase_mla_b(p, l_layer, -1); break;
    case PH_MLA_ABS: phase_mla_absorb(p, l_layer, -1); break;
    case PH_MLA_ATTN: phase_mla_attn(p, l_layer, -1); break;
    case PH_MLA_OUT: phase_mla_out(p, l_layer, 1); break;
    case PH_MLA_OUT2: phase_mla_out(p, l_layer, 2); break;
    case PH_MLA_O: phase_residual(p, l_layer, RES_MLA_O, L.ffn_norm, -1); break;
    case PH_LMHEAD: phase_lmhead(p, -1); break;
    case PH_ARGMAX: if (blockIdx.x == 0) final_argmax(p); break;
    default: break;
  }
}

// ===================================================================== kernel
extern "C" __global__ __launch_bounds__(NT) void MD_KERNEL(Params p_arg) {
  KParams& p = *(KParams*)__builtin_amdgcn_kernarg_segment_ptr();
  (void)p_arg;
  if (p.B < 1 || p.B > MAXB) return;
  if (threadIdx.x < NPLAN) PLANS[threadIdx.x].valid = 0;
  __syncthreads();
  if (p.ml_phase >= 0) {  // one phase of the multi-launch step
    if (threadIdx.x == 0) {
      md_cur_phase = 0;
      md_trace_t0 = 0;
    }
    run_one_phase(p, p.ml_layer, p.ml_phase);
    return;
  }
  trace_begin(p);
  clear_next_bank(p);
  int sidx = 0;
  if (threadIdx.x == 0) md_cur_phase = 0;
  // Every sync point s is split: grid_arrive(p, s) when this workgroup's share
  // is done; the next phase waits for s itself -- a weight-streaming phase
  // after issuing its first weight loads (they depend on nobody), any other
  // phase first thing (WAIT).
#define WAIT() wait_point(p, sidx++)
#define ARRIVE() grid_arrive(p, sidx)
  phase_embed(p);
  ARRIVE();
  for (int l = 0; l < p.n_layers; ++l) {
    const int l_layer = l;
    KLayer& L = layer_ref(p, l);
    const uint16_t* g_next = (l + 1 < p.n_layers) ? layer_ref(p, l + 1).attn_norm : p.final_norm;
    const int kind = L.kind;
    if (kind == LK_GQA) {
      phase_qkv(p, l_layer, sidx++);
      ARRIVE();
      if (p.verify) {
        WAIT();
        phase_gqa_kv_write(p, l_layer);
        ARRIVE();
      }
      phase_attn_gqa(p, l_layer, l, sidx++);
      ARRIVE();
      phase_residual(p, l_layer, RES_OPROJ, L.ffn_norm, sidx++);
      ARRIVE();
    } else if (kind == LK_KDA) {
      phase_kda_proj(p, l_layer, sidx++);
      ARRIVE();
      if (p.verify) {
        WAIT();
        phase_kda_rec_verify(p, l_layer);
      } else {
        phase_kda_rec(p, l_layer, sidx++);
      }
      ARRIVE();
      phase_residual(p, l_layer, RES_KDA_O, L.ffn_norm, sidx++);
      ARRIVE();
    } else {
      phase_mla_a(p, l_layer, sidx++);
      ARRIVE();
      phase_mla_b(p, l_layer, sidx++);
      ARRIVE();
      phase_mla_absorb(p, l_layer, sidx++);
      ARRIVE();
      phase_mla_attn(p, l_layer, sidx++);
      ARRIVE();
      WAIT();
      phase_mla_out(p, l_layer, 3);
      ARRIVE();
      phase_residual(p, l_layer, RES_MLA_O, L.ffn_norm, sidx++);
      ARRIVE();
    }
    if (p.n_experts == 0) {
      phase_gateup(p, l_layer, sidx++);
      ARRIVE();
      phase_residual(p, l_layer, RES_DENSE_DOWN, g_next, sidx++);
      ARRIVE();
    } else {
      phase_moe_a(p, l_layer, sidx++);
      // no arrival, no wait: phase B validates the router logits' tags, and
      // the down projection, which reads phase A's outputs, waits for phase
      // B's arrivals (each made after this workgroup's A stores completed)
      stamp(p, 2 * sidx);
      enter_phase(p, sidx++);
      if (p.moe_all) {
        phase_moe_b(p, l_layer, true);
      } else {
        RouteIn in;
        route_load(p, in);
        compute_routes(p, l, in);
        phase_moe_b(p, l_layer, false);
      }
      ARRIVE();
      phase_residual(p, l_layer, RES_MOE_DOWN, g_next, sidx++);
      ARRIVE();
    }
    if (dev_failed(p)) {
      trace_flush(p);
      return;
    }
  }
  phase_lmhead(p, sidx++);
  if (p.verify) {
    ARRIVE();
    WAIT();
    verify_finish(p);
    trace_flush(p);
    return;
  }
#undef WAIT
#undef ARRIVE
  // the last workgroup to arrive reduces the argmax candidates
  stamp(p, 2 * sidx);
  bool last = arrive_last(p, sidx);
  if (threadIdx.x == 0) ((int*)md_smem)[0] = last;
  __syncthreads();
  if (((int*)md_smem)[0]) final_argmax(p);
  trace_flush(p);
}

}  // namespace md

// ===================================================================== launch helpers
namespace md {

#if MD_MAXB == 8
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
#endif

// All of the kernel's LDS is static (md_smem): launches ask for no dynamic LDS.
hipError_t MD_BUILD_NAME(launch_megakernel)(const Params& p, int grid, hipStream_t stream) {
  void* args[] = {(void*)&p};
  return hipLaunchCooperativeKernel((const void*)MD_KERNEL, dim3(grid), dim3(NT), args, 0u, stream);
}

// One decode step as a sequence of phase launches on `stream`.
hipError_t MD_BUILD_NAME(launch_multilaunch)(const Params& p, const int* kinds, int grid, hipStream_t stream) {
  const unsigned smem = 0u;
  Params q = p;
  auto go = [&](int layer, int phase, int g) {
    q.ml_layer = layer;
    q.ml_phase = phase;
    hipLaunchKernelGGL(MD_KERNEL, dim3(g), dim3(NT), smem, stream, q);
  };
  go(-1, PH_EMBED, grid);
  for (int l = 0; l < p.n_layers; ++l) {
    if (kinds[l] == LK_GQA) {
      go(l, PH_QKV, grid);
      go(l, PH_ATTN, grid);
      go(l, PH_OPROJ, grid);
    } else if (kinds[l] == LK_KDA) {
      go(l, PH_KDA_PROJ, grid);
      go(l, PH_KDA_REC, grid);
      go(l, PH_KDA_O, grid);
    } else {
      go(l, PH_MLA_A, grid);
      go(l, PH_MLA_B, grid);
      go(l, PH_MLA_ABS, grid);
      go(l, PH_MLA_ATTN, grid);
      go(l, PH_MLA_OUT, grid);
      go(l, PH_MLA_OUT2, grid);
      go(l, PH_MLA_O, grid);
    }
    if (p.n_experts == 0) {
      go(l, PH_GATEUP, grid);
      go(l, PH_DOWN, grid);
    } else {
      go(l, PH_MOE_A, grid);
      go(l, PH_MOE_B, grid);
      go(l, PH_MOE_C, grid);
    }
  }
  go(-1, PH_LMHEAD, grid);
  go(-1, PH_ARGMAX, grid);  // workgroup 0 reduces all grid candidates
  return hipGetLastError();
}

#if MD_MAXB == 8
// ===================================================================== KV movement
// Copies between attention-cache pages and between sequence slots, for
// callers that fork a sequence or move its cache (copy-on-write of a shared
// last page, prefix reuse).  Block (i, l) copies item i of layer l with
// 16-byte loads and stores.
//   pages (src, dst non-null): page src[i] -> dst[i] of every GQA layer (its
//     K page and its V page) and every MLA layer; ids outside the pool set
//     the error word and are skipped;
//   slot (src, dst null): slot src_slot -> dst_slot of every delta-rule
//     layer's state and, where the attention caches are contiguous (one page
//     per slot; bt_stride == 0), of every GQA and MLA layer too.
__device__ __forceinline__ void copy_bytes(uint8_t* dst, const uint8_t* src, size_t n) {
  for (size_t i = (size_t)threadIdx.x * 16; i < n; i += (size_t)blockDim.x * 16)
    *(i32x4*)(dst + i) = *(const i32x4*)(src + i);
}

__global__ void k_kv_copy(Params p, const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int src_slot,
                          int dst_slot) {
  const int i = blockIdx.x, l = blockIdx.y;
  const LayerDesc& L = p.layers[l];
  uint8_t* base = p.kv + L.kv_off;
  const bool pages = src != nullptr;
  if (L.kind == LK_KDA) {
    if (pages) return;
    const size_t sb = (size_t)p.kda_h * p.kda_dk * p.kda_dv * 4;
    copy_bytes(base + (size_t)dst_slot * sb, base + (size_t)src_slot * sb, sb);
    return;
  }
  if (!pages && p.bt_stride > 0) return;  // paged: the block table maps the slot's pages
  const int a = pages ? src[i] : src_slot, b = pages ? dst[i] : dst_slot;
  if ((unsigned)a >= (unsigned)p.n_pages || (unsigned)b >= (unsigned)p.n_pages) {
    if (threadIdx.x == 0) __hip_atomic_fetch_or(p.err, (int)MDE_PAGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (a == b) return;
  if (L.kind == LK_GQA) {
    const size_t pb = (size_t)p.nkv * p.pg_cap * p.hd * 2;
    uint8_t* vbase = base + (size_t)p.n_pages * pb;
    copy_bytes(base + (size_t)b * pb, base + (size_t)a * pb, pb);
    copy_bytes(vbase + (size_t)b * pb, vbase + (size_t)a * pb, pb);
  } else {
    const size_t pb = (size_t)p.pg_cap * 576 * 2;
    copy_bytes(base + (size_t)b * pb, base + (size_t)a * pb, pb);
  }
}

hipError_t launch_kv_copy(const Params& p, const int32_t* src, const int32_t* dst, int n, int src_slot, int dst_slot,
                          hipStream_t stream) {
  if (n <= 0 || p.n_layers <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_kv_copy, dim3(n, p.n_layers), dim3(256), 0, stream, p, src, dst, src_slot, dst_slot);
  return hipGetLastError();
}

// ===================================================================== static scratch
// The allocation-free decode step (md_decode_step_noalloc) takes its per-step
// buffers from this file-scope array instead of the model's workspace: one
// copy per device, held from the library's load until the process ends.  In
// host code its name is only a stand-in; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept per device.
constexpr size_t MD_SCRATCH_BYTES = (size_t)128 << 20;
static __device__ __align__(256) uint8_t scratch[MD_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static void* g_scratch_addr[MAX_DEVICES];
static std::mutex g_scratch_mu;

size_t scratch_bytes() { return MD_SCRATCH_BYTES; }

// Device address of `scratch` on device dev, which must be the current device.
hipError_t scratch_address(int dev, void** out) {
  *out = nullptr;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

// n 32-bit words at dst set to v (a kernel, not a memset, so that the fill is
// an ordinary kernel node where the call is captured into a graph).
__global__ void k_fill_u32(uint32_t* __restrict__ dst, uint32_t v, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) dst[i] = v;
}

hipError_t launch_fill_u32(void* dst, uint32_t v, uint32_t n_words, hipStream_t stream) {
  uint32_t g = (n_words + 255) / 256;
  if (g > 1024) g = 1024;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(k_fill_u32, dim3(g), dim3(256), 0, stream, (uint32_t*)dst, v, n_words);
  return hipGetLastError();
}

#endif

hipError_t MD_BUILD_NAME(megakernel_occupancy)(int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)MD_KERNEL, NT, 0);
}

}  // namespace md
