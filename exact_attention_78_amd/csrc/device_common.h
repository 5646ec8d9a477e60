// Device-side helpers shared by the gfx950 attention kernels: vector types, MFMA and
// LDS-transpose wrappers, cross-half lane exchange and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Element type tags for the 16-bit paths.
struct Bf16Tag {};
struct F16Tag {};

// 32x32x16 MFMA, fp32 accumulate. Lane l holds A[l%32][(l/32)*8 + s] and
// B[(l/32)*8 + s][l%32] (s = 0..7); the result lane l holds C[(r/4)*8 + (l/32)*4 + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(Bf16Tag, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(F16Tag, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values to one packed 16-bit pair, round to nearest even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack2(Bf16Tag, float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint32_t pack2(F16Tag, float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Combine a value held by lane l with the one held by lane l^32. v_permlane32_swap
// exchanges the upper 32 lanes of its first register with the lower 32 lanes of its
// second; with both registers holding x, one ends up with this lane's own value and
// the other with its partner's, in an order that depends on the half, so only a
// symmetric combination of the two is used. (Inline asm keeps the two registers
// distinct: the builtin's result is folded wrongly when both operands are the same.)
__device__ __forceinline__ void permlane32_swap_pair(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// IEEE-754 2019 maximum (NaN-propagating) of three values: one v_maximum3_f32, with no
// canonicalising v_max of each input as fmaxf needs. Written as the instruction itself:
// from nested two-input maxima the compiler re-balances a chain of these into pairs
// (v_maximum3 with a repeated operand) and a tree over them, 24 instructions for the 32
// scores of a tile where 16 do. (Its inputs here are MFMA results of an earlier step or
// VALU results, far outside the MFMA-to-VALU read hazard window.)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_maximum3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_halves(float x) {
  float a = x, b = x;
  permlane32_swap_pair(a, b);
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float add_halves(float x) {
  float a = x, b = x;
  permlane32_swap_pair(a, b);
  return a + b;
}

// LDS transpose read of 4 x 16-bit elements. Within each 16-lane group, lane i receives
// element (i % 4) of the 8-byte segments addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on XCD w % 8).
// Renumber them so that each XCD walks one contiguous range of logical ids: consecutive
// logical ids share a (batch, head) and therefore its K/V in that XCD's L2.
__device__ __forceinline__ int xcd_logical_id(int w, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = w % 8, loc = w / 8;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + loc;
}

// Orders of the query tiles over the workgroup ids of a 1D grid. kOrderXcdPairs is the one
// every kernel uses; the others are kept as launch variants of the 16-bit forward pass so
// that the orders can be measured against each other.
enum TileOrder : int {
  kOrderXcdPairs = 0,        // per XCD, each pair of its heads, longest query tile first
  kOrderXcdAllHeads = 1,     // per XCD, all its heads' tiles together, longest first
  kOrderXcdHead = 2,         // per XCD, one head at a time, longest first
  kOrderXcdNatural = 3,      // per XCD, one head at a time, natural order
  kOrderLinearLongest = 4,   // no XCD remap (consecutive ids share a head), longest first
  kOrderLinearNatural = 5,   // no XCD remap, natural order
};

// Query tile (bh, mt) of workgroup w in a grid of total = BH * n_mtiles workgroups.
// The XCD orders give each XCD a contiguous set of heads, so their K/V stay in its L2.
// Causal grids go longest query tile first, over groups of g heads of the XCD when BH is
// a multiple of 8 (the XCD starts all the group's longest tiles before any shorter one:
// the tail of short tiles shrinks, while only g heads' K/V compete for the L2), else per
// head. Non-causal tiles all have one length, so only the XCD remap matters there.
__device__ __forceinline__ void query_tile_ordered(int order, int w, int total, int n_mtiles, bool causal, int& bh,
                                                   int& mt) {
  const int n_bh = total / n_mtiles;
  if (order >= kOrderLinearLongest) {
    bh = w / n_mtiles;
    const int m = w % n_mtiles;
    mt = causal && order == kOrderLinearLongest ? n_mtiles - 1 - m : m;
    return;
  }
  if (causal && order != kOrderXcdNatural && n_bh % 8 == 0) {
    const int nh = n_bh / 8, loc = w / 8;
    const int g = order == kOrderXcdAllHeads ? nh : order == kOrderXcdHead ? 1 : (nh % 2 == 0 ? 2 : 1);
    const int grp = loc / (g * n_mtiles), r = loc % (g * n_mtiles);
    bh = (w % 8) * nh + grp * g + r % g;
    mt = n_mtiles - 1 - r / g;
  } else {
    const int logical = xcd_logical_id(w, total);
    const int m = logical % n_mtiles;
    bh = logical / n_mtiles;
    mt = causal && order != kOrderXcdNatural ? n_mtiles - 1 - m : m;
  }
}

// The order all kernels use by default (per XCD, pairs of heads, longest first).
__device__ __forceinline__ void xcd_query_tile(int w, int total, int n_mtiles, bool causal, int& bh, int& mt) {
  query_tile_ordered(kOrderXcdPairs, w, total, n_mtiles, causal, bh, mt);
}

// Wait until at most N vector-memory loads of this wave are outstanding.
// (s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at
// their maxima; the builtin keeps the compiler's own counter tracking informed.)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Byte address of a __shared__ object in the LDS aperture.
__device__ __forceinline__ uint32_t lds_u32(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// One 16-byte-per-lane global->LDS DMA (global_load_lds_dwordx4): lane i's 16 bytes land
// at LDS byte lds_base + 16*i; lds_base must be wave-uniform. The LDS base goes through
// M0, which the operand constraint binds, so the compiler itself writes M0 before the
// instruction and knows what M0 holds afterwards. The load is written as inline assembly
// so that the compiler does not see an LDS write it would guard with a full vmcnt(0)
// drain before every later LDS read: completion is tracked by hand with wait_vmcnt<>()
// and barrier_lds(). (The s_nop separates the M0 write from the instruction that reads it.)
__device__ __forceinline__ void dma_load16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(gptr), "{m0}"(lds_base) : "memory");
}

// The 4-byte form (global_load_lds_dword): lane i's 4 bytes land at lds_base + 4*i (lanes
// with exec clear write nothing).
__device__ __forceinline__ void dma_load4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(gptr), "{m0}"(lds_base) : "memory");
}

// Both forms with a wave-uniform base address (an SGPR pair) and a 32-bit per-lane byte
// offset from it: a loop then keeps one offset register per lane instead of a 64-bit
// address.
__device__ __forceinline__ void dma_load16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void dma_load4_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" :: "v"(voff), "s"(sbase), "{m0}"(lds_base) : "memory");
}

// Workgroup barrier for LDS hand-over only: LDS reads of this wave are complete, then
// s_barrier. Unlike __syncthreads() it does not drain this wave's outstanding global
// loads, so a load for a later tile can stay in flight across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int I>
using IC = std::integral_constant<int, I>;

}  // namespace attn
