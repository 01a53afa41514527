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

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of `mask` below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Waits until at most N vector-memory operations of this wave are outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for an LDS hand-off: this wave's LDS operations complete, then s_barrier. Unlike
// __syncthreads() it does not wait for outstanding global-memory operations, so asynchronous copies issued for
// later tiles stay in flight; the asm memory clobber keeps the compiler from moving memory accesses across it.
// Data copied into LDS asynchronously must be waited for (wait_vmem*) by each wave before the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16-byte asynchronous copy global -> LDS: lane i of the wave writes lds_base + 16 * i.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

// LDS transpose read of four 16-bit values (gfx950 ds_read_b64_tr_b16). Within each group of 16 lanes, output
// lane i receives element (i % 4) of the 8-byte rows addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_addr));
}

}  // namespace sa
