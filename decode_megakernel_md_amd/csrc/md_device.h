// Device-side building blocks of the decode megakernel (gfx950 / CDNA4).
//
//  * buffer-resource loads and stores with explicit cache policy;
//  * the cross-workgroup visibility protocol;
//  * hierarchical sync counters with a bounded wait;
//  * the MFMA weight-streaming GEMV engine.
//
// Cross-workgroup data protocol.  Every value that one workgroup produces
// for another (normalised activations, partial sums of squares, q/k/v,
// attention partials, argmax candidates, router results) is written with a
// device-coherent store (cache policy sc1: written through to the device
// coherence point) and read with a device-coherent load (sc1: never served
// from a stale copy in another XCD's L2).  A producer waits until its stores
// have completed (s_waitcnt vmcnt(0)) before it increments a sync counter;
// a consumer reads the data only after it has observed the counter.  Because
// no cross-workgroup value ever sits dirty in an L2, no L2 write-back or
// invalidate (the costly part of an agent-scope fence on this part) is needed.
// One exception: the weight stream's activations (the B operands of its
// matrix-core tiles) are read with cache policy sc0, served by the XCD's L2.
// That is safe because each activation buffer is written and read once per
// launch (one buffer per use) and the L2s start every launch without copies
// of the workspace: an XCD's first read misses and fetches the written-through
// data, later reads of the same lines hit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef MD_MAXB
#define MD_MAXB 8
#endif
// Names of the two builds' kernel and launch functions
#if MD_MAXB == 8
#define MD_KERNEL md_megakernel
#define MD_BUILD_NAME(x) x
#else
#define MD_KERNEL md_megakernel_w64
#define MD_BUILD_NAME(x) x##_w64
#endif

namespace md {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int NT = 256;      // threads per workgroup (4 waves of 64)
constexpr int NW = 4;        // waves per workgroup
// Token rows a step can carry: the library builds this file twice, with 8
// (batches up to 8 and the verify step) and with 64 (wide batches, up to 64
// sequences).  Activation buffers are laid out [..][MAXB][..].
constexpr int MAXB = MD_MAXB;
static_assert(MAXB == 8 || MAXB == 64, "the two builds: 8 and 64 rows");
constexpr bool WIDE = MAXB > 8;       // the 64-row build (decode only)
// The matrix cores' B operand is 16 columns.  8-row build: a tile is 8
// tokens, token t's bf16 high part in column 2t and the rest in 2t+1 (one
// operand, one instruction per tile).  64-row build: a tile is 16 tokens,
// one per column, with the high parts and the rests as two operands whose
// products go to the same accumulators (half the accumulator registers per
// token).
constexpr int TTILE = WIDE ? 16 : 8;  // tokens per B tile
constexpr int NPART = WIDE ? 2 : 1;   // B operands per tile
constexpr int NBT = MAXB / TTILE;     // B tiles of a full step
constexpr int VMAX = 8;               // rows of a verify step (anchor + 7 drafts)
constexpr int GSMAX = 8;              // query heads per kv head
constexpr unsigned OOB = 0xFFFFFFF0u;  // buffer offset beyond any resource: loads return 0

// cache-policy bits of buffer instructions on gfx950
constexpr int CP_SC0 = 1;    // not kept in the CU's L1
constexpr int CP_NT = 2;     // streaming (non-temporal)
constexpr int CP_SC1 = 16;   // device scope: coherent across XCDs

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0]|expcnt[6:4]|lgkmcnt[11:8]|vmcnt_hi[15:14])
constexpr int WAIT_VM0 = 0x0F70;
constexpr int WAIT_LGKM0 = 0xC07F;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Resource from values the compiler cannot prove uniform (function
// arguments, values loaded from memory): force them into scalar registers so
// buffer instructions take the resource directly instead of looping over lanes.
__device__ __forceinline__ rsrc_t make_rsrc_u(const void* base, uint32_t bytes) {
  uint64_t a = (uint64_t)base;
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return make_rsrc((const void*)(((uint64_t)hi << 32) | lo), n);
}

// ---- coherent scalar access (32-bit) through a resource
__device__ __forceinline__ float ld_f32(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP_SC1));
}
__device__ __forceinline__ void st_f32(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, CP_SC1);
}
__device__ __forceinline__ uint32_t ld_u32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP_SC1);
}
__device__ __forceinline__ void st_u32(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, CP_SC1);
}
__device__ __forceinline__ void st_u16(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, CP_SC1);
}
template <int CP>
__device__ __forceinline__ i32x4 ld_x4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
}

// ---- bf16 helpers
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): about 16 significant bits.
__device__ __forceinline__ void split_hilo(float x, uint16_t& hi, uint16_t& lo) {
  hi = bf16_rne(x);
  lo = bf16_rne(x - bf16_f32(hi));
}

// ---- cross-lane moves without LDS: DPP within a 16-lane row, and gfx950's
// permlane16/32 swaps across rows.  permlane16_swap(v, v) yields
// (rows 0,0,2,2) and (rows 1,1,3,3); permlane32_swap(v, v) yields (low half
// twice) and (high half twice).
constexpr int DPP_QXOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QXOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROR4 = 0x124;   // row_ror:4
constexpr int DPP_ROR8 = 0x128;   // row_ror:8 (within a row: lane i <-> i^8)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// The swaps are written as inline assembly: the compiler builtins fold the two
// results of a swap whose inputs are equal into one value, which is wrong.
// Both registers start as copies of v; two wait states separate the VALU
// writes of the copies from the cross-lane read.
__device__ __forceinline__ void swap16(float v, float& x, float& y) {
  x = v;
  y = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void swap32(float v, float& x, float& y) {
  x = v;
  y = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}

// sum over the 4 rows of each column (lanes c, c+16, c+32, c+48)
__device__ __forceinline__ float rows_sum(float v) {
  float x, y;
  swap16(v, x, y);
  swap32(x + y, x, y);
  return x + y;
}
__device__ __forceinline__ float rows_max(float v) {
  float x, y;
  swap16(v, x, y);
  swap32(fmaxf(x, y), x, y);
  return fmaxf(x, y);
}

// ---- wave reductions: every lane gets the result; the combination order is
// fixed, so the result is deterministic
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<DPP_QXOR1>(v);
  v += dpp_f<DPP_QXOR2>(v);
  v += dpp_f<DPP_ROR4>(v);
  v += dpp_f<DPP_ROR8>(v);
  return rows_sum(v);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QXOR1>(v));
  v = fmaxf(v, dpp_f<DPP_QXOR2>(v));
  v = fmaxf(v, dpp_f<DPP_ROR4>(v));
  v = fmaxf(v, dpp_f<DPP_ROR8>(v));
  return rows_max(v);
}

__device__ __forceinline__ void wait_stores() {
  __builtin_amdgcn_s_waitcnt(WAIT_VM0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }
__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

}  // namespace md
