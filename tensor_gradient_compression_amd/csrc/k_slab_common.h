// Helpers shared by the slab kernels (k_slab2.hip, k_rec3.hip): LDS-qualified types,
// wait and fence wrappers, the 16-byte HBM -> LDS transfer of a wave, and the Omega
// range pipeline of a slab (a slab's sparse entries are one contiguous range of the
// ascending Omega, found from the membership bitmask and word ranks at its two ends).
#pragma once
#include <type_traits>

#include "tg_common.h"

namespace tg {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
// LDS-qualified pointers: accesses through them compile to ds_* instructions (a
// generic pointer would give flat accesses, which also count against vmcnt)
#define LDS __attribute__((address_space(3)))

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void wave_fence() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
}

// The two 16-bit weights of a 32-bit word as floats (element 2i in the low half), and
// two floats rounded to the weight type and packed the same way.
template <typename WT> __device__ __forceinline__ float wlo(uint32_t w);
template <typename WT> __device__ __forceinline__ float whi(uint32_t w);
template <typename WT> __device__ __forceinline__ uint32_t wpack(float lo, float hi);
template <> __device__ __forceinline__ float wlo<bf16_t>(uint32_t w) { return __uint_as_float(w << 16); }
template <> __device__ __forceinline__ float whi<bf16_t>(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
template <> __device__ __forceinline__ float wlo<_Float16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
template <> __device__ __forceinline__ float whi<_Float16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}
// (round to nearest even, as from_f32; one v_cvt_pk_bf16_f32 for bf16)
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
template <> __device__ __forceinline__ uint32_t wpack<bf16_t>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, bf16x2v));
}
template <> __device__ __forceinline__ uint32_t wpack<_Float16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, f16x2v));
}

// nchunks 16-byte pieces from src to dst (wave-uniform), one per lane per instruction
__device__ __forceinline__ void wave_dma(const void* src, uint32_t nchunks, LDS unsigned char* dst,
                                        uint32_t lane) {
  for (uint32_t q0 = 0; q0 < nchunks; q0 += 64)
    if (q0 + lane < nchunks)
      __builtin_amdgcn_global_load_lds((const unsigned char*)src + (size_t)(q0 + lane) * 16,
                                       (lds_void*)(dst + (size_t)q0 * 16), 16, 0, 0);
}

// A slab transfer of exactly ND loads a wave, nchunks in (64 (ND - 1), 64 ND], through a
// buffer resource over the slab: the lane's byte offset is the one vector operand and
// each group's base a scalar one, so the transfer needs no 64-bit address registers.
// With nchunks >= 64 every lane is active: the last group of 64 chunks is shifted back
// to end at the slab's end, so it writes some chunks the group before it wrote, with
// the same data. A fixed count lets the caller wait for all but the last transfer with
// one immediate wait count, and lets the compiler see that count too.
template <int ND>
__device__ __forceinline__ void wave_dma_n(const void* src, uint32_t nchunks,
                                          LDS unsigned char* dst, uint32_t lane) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, (int)(nchunks * 16u), 0x00020000);
  const uint32_t lo = lane * 16u;
  if (ND > 1 || nchunks == 64) {
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const uint32_t b = i + 1 < ND ? 64u * i : nchunks - 64;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + b * 16u), 16, lo,
                                               (int)(b * 16u), 0, 0);
    }
  } else if (lane < nchunks) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, lo, 0, 0, 0);
  }
}

// Omega rank of element e from its bitmask word and word rank; kS past the end
__device__ __forceinline__ uint64_t rank_at(uint64_t word, uint32_t wr, uint64_t e, uint64_t N,
                                            uint64_t kS) {
  if (e >= N) return kS;
  return wr + (uint64_t)__popcll(word & ((1ull << (e & 63)) - 1ull));
}

// Omega range of slab s: [J(s), J(s + 1)) with J(s) = Omega rank of element s * slab_e.
// A wave keeps the current slab's range, the next slab's range, the first NOM * 64
// indices (and N_S) of the next slab's range, and the bitmask words and ranks that
// bound the slab after it; entries past NOM * 64 in one slab are read directly.
constexpr int NOM = 3;

// Two slots, used alternately by consecutive slabs of a wave; the slab loops are unrolled
// by two so that a slot index is a compile-time constant and the prefetched entries are
// never copied between registers (a copy would have to wait for every load in flight,
// the next slab's transfer included).
// Bitmask words and word ranks at the start (lane 0) and the end (lane 1) of a slab,
// fetched with vector loads: they retire on vmcnt with the slab transfers (scalar loads
// would retire on lgkmcnt, out of order, so every wait on LDS traffic after them would
// also wait for their memory round trip). Read out with lane_u64 / readlane after the
// next vmcnt wait.
struct BoundsV {
  uint64_t m = 0;
  uint32_t r = 0;
};
template <typename MaskPtr, typename RankPtr>
__device__ __forceinline__ BoundsV load_bounds(MaskPtr mask, RankPtr rank, uint64_t elo,
                                               uint64_t slab_e, uint64_t N, uint32_t lane) {
  const uint64_t ehi = elo + slab_e;
  const uint64_t wl = elo >> 6, wh = ehi < N ? ehi >> 6 : 0;
  const uint64_t idx = lane == 0 ? wl : wh;
  BoundsV b;
  b.m = mask[idx];
  b.r = rank[idx];
  return b;
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// A wave-uniform value held in vector registers. The compiler keeps uniform values in
// scalar registers; where a kernel runs out of those it spills them into lanes of a
// vector register and reads each one back (v_readlane) at every use. Values whose uses
// are all vector operations (addresses of per-lane loads, per-lane compares) lose
// nothing by living in a vector register instead.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x) {
  uint32_t y;
  __asm__("v_mov_b32 %0, %1" : "=v"(y) : "s"(x));
  return y;
}
__device__ __forceinline__ uint64_t in_vgpr64(uint64_t x) {
  return ((uint64_t)in_vgpr((uint32_t)(x >> 32)) << 32) | in_vgpr((uint32_t)x);
}
// a global-memory pointer held so (its loads stay global loads: a generic pointer's
// would be flat loads, which also count against the LDS wait counter)
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* in_vgpr_ptr(T* p) {
  return (__attribute__((address_space(1))) T*)in_vgpr64((uint64_t)(uintptr_t)p);
}

struct OmegaPipe {
  uint64_t lo[2] = {0, 0}, hi[2] = {0, 0};   // Omega ranges of the slabs in the two slots
  BoundsV bw;                     // the slab after: bounds (lane 0: start, lane 1: end)
  uint32_t om[2][NOM];
  float us[2][NOM];
};
template <int V>
using Slot = std::integral_constant<int, V>;

}  // namespace
}  // namespace tg
