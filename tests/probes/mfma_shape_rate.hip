// Issue rate of the two gfx950 bf16 MFMA shapes on random operands, alone and inside the indexer's tile scorer.
// This is the measurement behind scoring 64-head queries on the 16x16x32 MFMA instead of the 32x32x16 one.
//
// Four loops, each run on 2048 workgroups of four waves with about 70 KB of LDS reserved per workgroup, so that two
// workgroups (two waves per SIMD) share each CU as in the scorers:
//   * MFMA only: 32x32x16 with four accumulator chains, or 16x16x32 with eight, cycling over eight operand
//     registers that hold seeded random bf16 values in [-2, 2);
//   * the scorer of a 64-position key tile for a 64-head query (the library's score_tile<2> on the 32x32x16 MFMA,
//     or score_tile16 on the 16x16x32 MFMA): key fragments read from an LDS tile of random keys, the ReLU-weighted
//     head sum, and one workgroup barrier per tile, as in the scoring loops (no key copies, no candidate output).
// Each loop runs twice, interleaved, since the clock drifts over a run. Rates are reported against the 2.5 PFLOP/s
// bf16 peak.
//
// Build and run (one MI355X):
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       -mllvm -amdgpu-mfma-vgpr-form tests/probes/mfma_shape_rate.hip -o _build/mfma_shape_rate && \
//       ./_build/mfma_shape_rate
#include <cstdio>

#include "../../long_context_sparse_sa_amd/csrc/sa_score_tile.h"

using namespace sa;
using namespace sa::tile;

#define CK(x)                                                                       \
  do {                                                                              \
    if ((x) != hipSuccess) {                                                        \
      printf("HIP error at line %d\n", __LINE__);                                   \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

constexpr int kBlocks = 256 * 2 * 4;
constexpr size_t kPadLds = 54 * 1024;  // with the 16 KB tile: about 70 KB per workgroup, two per CU

__device__ float hash_unit(unsigned x) {  // uniform in [-2, 2)
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return ((float)(x & 0xFFFFu) / 65536.f - 0.5f) * 4.f;
}

// V 0: 32x32x16 only; 1: 16x16x32 only; 2: scorer on 32x32x16; 3: scorer on 16x16x32
template <int V>
__global__ __launch_bounds__(256) void k_rate(float* __restrict__ out, int iters) {
  __shared__ __attribute__((aligned(1024))) char tile[kTileBytes];
  extern __shared__ char pad[];
  if (iters < 0) pad[threadIdx.x] = 0;
  const int lane = lane_id();
  const unsigned seed = (blockIdx.x * 256 + threadIdx.x) * 977u;
  for (int i = threadIdx.x; i < kTileBytes / 2; i += 256)
    reinterpret_cast<__bf16*>(tile)[i] = (__bf16)hash_unit(0x9e3779b9u + 7u * i);
  __syncthreads();
  float r = 0.f;
  if constexpr (V <= 1) {
    bf16x8 a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[j][i] = (__bf16)hash_unit(seed + 2 * (8 * j + i) + 1);
        b[j][i] = (__bf16)hash_unit(seed + 2 * (8 * j + i) + 12345);
      }
    if constexpr (V == 0) {
      f32x16 acc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
      for (int it = 0; it < iters; ++it) {
        asm volatile("" : "+v"(a[0]));
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int j = (k + c) & 7;
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(3 * j) & 7], acc[c], 0, 0, 0);
          }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) r += acc[c][i];
    } else {
      f32x4 acc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = f32x4{};
      for (int it = 0; it < iters; ++it) {
        asm volatile("" : "+v"(a[0]));
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const int j = (k + c) & 7;
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[(3 * j) & 7], acc[c], 0, 0, 0);
          }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) r += acc[c][i];
    }
  } else {
    // one random 64-head query per wave, weights in [-2, 2)
    if constexpr (V == 2) {
      bf16x8 qa[2][kSteps];
      float wv[2][16];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
          for (int i = 0; i < 8; ++i) qa[mt][ks][i] = (__bf16)hash_unit(seed + 64 * mt + 8 * ks + i);
#pragma unroll
        for (int e = 0; e < 16; ++e) wv[mt][e] = hash_unit(seed + 999 + 16 * mt + e);
      }
      for (int it = 0; it < iters; ++it) {
        lds_barrier();
        r += score_tile<2>(tile, lane, qa, wv);
      }
    } else {
      bf16x8 qa[4][kSteps16];
      float wv[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int ks = 0; ks < kSteps16; ++ks)
#pragma unroll
          for (int i = 0; i < 8; ++i) qa[mt][ks][i] = (__bf16)hash_unit(seed + 32 * mt + 8 * ks + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[mt][e] = hash_unit(seed + 999 + 4 * mt + e);
      }
      for (int it = 0; it < iters; ++it) {
        lds_barrier();
        r += score_tile16(tile, lane, qa, wv);
      }
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = r;
}

template <int V>
int run(float* dout, const char* name) {
  // MFMA-only loops: 32 (or 64) MFMAs per iteration; scorers: one 64x64x128 tile (1 MFLOP per wave) per iteration
  const double flop_per_iter = V == 0 ? 32.0 * 32768 : V == 1 ? 64.0 * 16384 : 64.0 * 64 * 128 * 2;
  const int iters = V <= 1 ? 512 : 256;
  CK(hipFuncSetAttribute(reinterpret_cast<const void*>(k_rate<V>), hipFuncAttributeMaxDynamicSharedMemorySize,
                         (int)kPadLds));
  k_rate<V><<<kBlocks, 256, kPadLds>>>(dout, iters);
  CK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  CK(hipEventRecord(e0));
  for (int rep = 0; rep < 3; ++rep) k_rate<V><<<kBlocks, 256, kPadLds>>>(dout, iters);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  float ms = 0.f;
  CK(hipEventElapsedTime(&ms, e0, e1));
  const double tflops = 3.0 * kBlocks * 4 * iters * flop_per_iter / (ms * 1e-3) / 1e12;
  printf("%-34s %8.3f ms  %7.1f TFLOP/s  %.3f of 2.5 PFLOP/s\n", name, ms, tflops, tflops / 2500.0);
  fflush(stdout);
  CK(hipEventDestroy(e0));
  CK(hipEventDestroy(e1));
  return 0;
}

int main() {
  float* dout = nullptr;
  CK(hipMalloc(&dout, (size_t)kBlocks * 256 * sizeof(float)));
  for (int pass = 0; pass < 2; ++pass) {
    if (run<0>(dout, "MFMA 32x32x16 only") || run<1>(dout, "MFMA 16x16x32 only") ||
        run<2>(dout, "scorer on 32x32x16 (LDS, barrier)") || run<3>(dout, "scorer on 16x16x32 (LDS, barrier)"))
      return 1;
  }
  CK(hipFree(dout));
  return 0;
}
