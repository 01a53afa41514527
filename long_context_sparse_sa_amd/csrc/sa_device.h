// Device-side helpers shared by the gfx950 kernels of the sparse-attention path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWave = 64;

// ---- storage decoding --------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals at exponent 0.
__device__ __forceinline__ float e4m3_bits_to_f32(uint8_t u) {
  const uint32_t sign = ((uint32_t)u & 0x80u) << 24;
  const uint32_t e = ((uint32_t)u >> 3) & 0xFu;
  const uint32_t m = (uint32_t)u & 0x7u;
  if (e == 0) {
    const float v = (float)m * 0.001953125f;  // m * 2^-9
    return __uint_as_float(__float_as_uint(v) | sign);
  }
  return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t i);
template <>
__device__ __forceinline__ float load_elem<0>(const void* base, int64_t i) {
  return reinterpret_cast<const float*>(base)[i];
}
template <>
__device__ __forceinline__ float load_elem<1>(const void* base, int64_t i) {
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
}
template <>
__device__ __forceinline__ float load_elem<2>(const void* base, int64_t i) {
  return e4m3_bits_to_f32(reinterpret_cast<const uint8_t*>(base)[i]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- order-preserving image of an fp32 score ---------------------------------------------------------------------
// Larger float -> larger key; -0.0 is folded onto +0.0 so that equal scores compare equal. 0 is below every key
// of a finite score and serves as the "accept everything" threshold.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // +-0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---- wave helpers ------------------------------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

// Lane swaps inside each row of 16 lanes as DPP operand modifiers (no LDS round trip). Each is an xor of the lane
// index: 0xB1 = quad_perm [1, 0, 3, 2] (lane ^ 1), 0x4E = quad_perm [2, 3, 0, 1] (lane ^ 2), 0x141 =
// row_half_mirror (lane ^ 7), 0x140 = row_mirror (lane ^ 15).
template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_swap(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, Ctrl, 0xF, 0xF, false);
}
template <int Ctrl>
__device__ __forceinline__ float dpp_swap(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
}
// The value of lane ^ s (s a power of two below 64). Strides up to 8 stay inside a row of 16 lanes and come through
// DPP swaps, composed where one swap is not enough: lane ^ 4 = (lane ^ 7) ^ 3 and lane ^ 8 = (lane ^ 15) ^ 7
// (0x1B = quad_perm [3, 2, 1, 0], lane ^ 3). Every lane takes the same swaps, so no lane-dependent choice can turn
// into a branch under which a swap would read a lane switched off. Strides 16 and 32 use a lane permute.
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int s) {
  switch (s) {
    case 1: return dpp_swap<0xB1>(x);
    case 2: return dpp_swap<0x4E>(x);
    case 4: return dpp_swap<0x1B>(dpp_swap<0x141>(x));
    case 8: return dpp_swap<0x141>(dpp_swap<0x140>(x));
    default: return (uint32_t)__shfl_xor((int)x, s, kWave);
  }
}
__device__ __forceinline__ uint64_t lane_xor64(uint64_t x, int s) {
  return ((uint64_t)lane_xor((uint32_t)(x >> 32), s) << 32) | lane_xor((uint32_t)x, s);
}
// Sum over each aligned quad of lanes, in every lane of it; the pairing of an xor-shuffle tree (lane ^ 1, then
// lane ^ 2), so the rounding is the same.
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp_swap<0xB1>(x);
  x += dpp_swap<0x4E>(x);
  return x;
}
// Sum over each aligned group of n lanes (n a power of two, at most 64), in every lane of it. Up to 16 lanes the
// partner sums come through DPP: after the quad sum, lane ^ 7 and then lane ^ 15 lie in the other quad and the other
// half-row, which by then hold their own sums, so the pairing is again that of an xor-shuffle tree.
__device__ __forceinline__ float group_sum(float x, int n) {
  if (n >= 2) x += dpp_swap<0xB1>(x);
  if (n >= 4) x += dpp_swap<0x4E>(x);
  if (n >= 8) x += dpp_swap<0x141>(x);
  if (n >= 16) x += dpp_swap<0x140>(x);
  if (n >= 32) x += __shfl_xor(x, 16, kWave);
  if (n >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}

// One VALU lane exchange (v_permlane32_swap: lanes 32..63 of the first operand trade places with lanes 0..31 of
// the second). The sum of the two results is, in lane l < 32, a_l + a_{l+32} and, in lane l >= 32, b_{l-32} + b_l:
// two half-wave pair sums in one register.
__device__ __forceinline__ float fold_halves(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same over rows of 16 lanes (v_permlane16_swap: the odd rows of the first operand trade places with the even
// rows of the second). The sum of the two results is, in the even rows, a_l + a_{l+16} and, in the odd rows,
// b_{l-16} + b_l.
__device__ __forceinline__ float fold_rows(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of `mask` below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Waits until at most N vector-memory operations of this wave are outstanding (loads complete in issue order).
// Emitted as a real s_waitcnt (vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their no-wait maxima) so
// that the compiler's own wait bookkeeping sees it and does not add waits of its own for older loads; the empty
// asm with a memory clobber keeps memory accesses from moving across it.
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_vmem() { wait_vmem_below<0>(); }

// Workgroup barrier for an LDS hand-off: this wave's LDS operations complete, then s_barrier. Unlike
// __syncthreads() it does not wait for outstanding global-memory operations, so asynchronous copies issued for
// later tiles stay in flight; the asm memory clobber keeps the compiler from moving memory accesses across it.
// Data copied into LDS asynchronously must be waited for (wait_vmem*) by each wave before the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// This wave's LDS (and scalar-memory) operations complete; the memory clobber keeps accesses from moving across.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16-byte asynchronous copy global -> LDS: lane i of the wave writes lds_base + 16 * i.
//
// Issued from inline asm on purpose. When the compiler sees a global->LDS copy it cannot tell which LDS bytes
// it writes, so it drains every outstanding vector-memory operation (s_waitcnt vmcnt(0)) before the next LDS
// read, which serialises a multi-buffered pipeline on the copies just issued for later tiles. Hidden in asm, the
// copy is ordered only by the waits the caller places (wait_vmem_below / wait_vmem, then lds_barrier) before
// reading the tile. Loads return in issue order, so "at most N outstanding" means every copy older than the
// newest N has landed, whatever other loads the compiler interleaves. M0 (the LDS base of the copy) is saved
// and restored so that no compiler-held M0 value is disturbed; the s_nop covers the M0-write -> LDS-DMA hazard.
// The copy has no register result: the address registers are consumed at issue.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(m0)
      : "memory");
}

// LDS transpose read of four 16-bit values (gfx950 ds_read_b64_tr_b16). Within each group of 16 lanes, output
// lane i receives element (i % 4) of the 8-byte rows addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_addr));
}

}  // namespace sa
