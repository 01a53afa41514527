// Accumulation error of the gfx950 fp8 (e4m3) 32x32x16 MFMA against the bf16 32x32x16 MFMA fed the same e4m3
// values converted exactly to bf16, on 128-long dot products (8 chained k-steps of 16), measured against the exact
// fp64 result and expressed relative to the sum of |products| of each output. This is the measurement behind
// contracting the fp8 index keys on the bf16 MFMA. Inputs: seeded LCG codes with random sign, exponent field
// 1..14 and any mantissa (normal values, no NaN); 256 trials of one 32x32 output tile (262,144 outputs).
//
// Build and run (one MI355X):
//   hipcc --offload-arch=gfx950 -O2 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       tests/probes/mfma_fp8_precision.hip -o _build/mfma_fp8_precision && ./_build/mfma_fp8_precision
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;

#define CK(x)                                                          \
  do {                                                                 \
    if ((x) != hipSuccess) { printf("HIP error at line %d\n", __LINE__); return 1; } \
  } while (0)

constexpr int K = 128, KS = K / 16, TRIALS = 256;

// a8/b8: [trial][64 lanes][KS] packed 8 fp8 codes; a16/b16: [trial][64][KS][8] bf16 bits
__global__ void k_probe(const long* a8, const long* b8, const uint16_t* a16, const uint16_t* b16, float* c8,
                        float* c16) {
  const int t = blockIdx.x, l = threadIdx.x;
  f32x16 x = {}, y = {};
  for (int ks = 0; ks < KS; ++ks) {
    const int i = (t * 64 + l) * KS + ks;
    x = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a8[i], b8[i], x, 0, 0, 0);
    const bf16x8 av = *reinterpret_cast<const bf16x8*>(a16 + (size_t)i * 8);
    const bf16x8 bv = *reinterpret_cast<const bf16x8*>(b16 + (size_t)i * 8);
    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, y, 0, 0, 0);
  }
  for (int r = 0; r < 16; ++r) {
    c8[(t * 64 + l) * 16 + r] = x[r];
    c16[(t * 64 + l) * 16 + r] = y[r];
  }
}

static double e4m3(uint8_t u) {
  const int s = u >> 7, e = (u >> 3) & 15, m = u & 7;
  const double v = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}
static uint16_t bf16_of(double v) {  // exact for e4m3 values
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int main() {
  uint64_t seed = 12345;
  auto rnd = [&]() { seed = seed * 6364136223846793005ull + 1442695040888963407ull; return (uint32_t)(seed >> 33); };
  // codes: random sign, exponent field 1..14 (normal values, no NaN), any mantissa
  std::vector<uint8_t> A((size_t)TRIALS * 32 * K), B((size_t)TRIALS * K * 32);
  for (auto& c : A) c = (uint8_t)((rnd() & 0x80) | ((1 + rnd() % 14) << 3) | (rnd() & 7));
  for (auto& c : B) c = (uint8_t)((rnd() & 0x80) | ((1 + rnd() % 14) << 3) | (rnd() & 7));
  std::vector<long> a8((size_t)TRIALS * 64 * KS), b8(a8.size());
  std::vector<uint16_t> a16(a8.size() * 8), b16(a8.size() * 8);
  for (int t = 0; t < TRIALS; ++t)
    for (int l = 0; l < 64; ++l)
      for (int ks = 0; ks < KS; ++ks) {
        const size_t i = ((size_t)t * 64 + l) * KS + ks;
        uint64_t pa = 0, pb = 0;
        for (int j = 0; j < 8; ++j) {
          const int k = 16 * ks + 8 * (l / 32) + j, m = l % 32, n = l % 32;
          const uint8_t ca = A[((size_t)t * 32 + m) * K + k], cb = B[((size_t)t * K + k) * 32 + n];
          pa |= (uint64_t)ca << (8 * j);
          pb |= (uint64_t)cb << (8 * j);
          a16[i * 8 + j] = bf16_of(e4m3(ca));
          b16[i * 8 + j] = bf16_of(e4m3(cb));
        }
        a8[i] = (long)pa;
        b8[i] = (long)pb;
      }
  long *da8, *db8;
  uint16_t *da16, *db16;
  float *dc8, *dc16;
  CK(hipMalloc(&da8, a8.size() * 8));
  CK(hipMalloc(&db8, b8.size() * 8));
  CK(hipMalloc(&da16, a16.size() * 2));
  CK(hipMalloc(&db16, b16.size() * 2));
  CK(hipMalloc(&dc8, (size_t)TRIALS * 64 * 16 * 4));
  CK(hipMalloc(&dc16, (size_t)TRIALS * 64 * 16 * 4));
  CK(hipMemcpy(da8, a8.data(), a8.size() * 8, hipMemcpyHostToDevice));
  CK(hipMemcpy(db8, b8.data(), b8.size() * 8, hipMemcpyHostToDevice));
  CK(hipMemcpy(da16, a16.data(), a16.size() * 2, hipMemcpyHostToDevice));
  CK(hipMemcpy(db16, b16.data(), b16.size() * 2, hipMemcpyHostToDevice));
  hipLaunchKernelGGL(k_probe, dim3(TRIALS), dim3(64), 0, 0, da8, db8, da16, db16, dc8, dc16);
  if (hipDeviceSynchronize() != hipSuccess) { printf("launch failed\n"); return 1; }
  std::vector<float> c8((size_t)TRIALS * 64 * 16), c16(c8.size());
  CK(hipMemcpy(c8.data(), dc8, c8.size() * 4, hipMemcpyDeviceToHost));
  CK(hipMemcpy(c16.data(), dc16, c16.size() * 4, hipMemcpyDeviceToHost));
  double max8 = 0, max16 = 0, sum8 = 0, sum16 = 0, maxrel32_16 = 0;
  long nz8 = 0, nz16 = 0, n = 0;
  for (int t = 0; t < TRIALS; ++t)
    for (int l = 0; l < 64; ++l)
      for (int r = 0; r < 16; ++r) {
        const int m = 8 * (r / 4) + 4 * (l / 32) + (r % 4), col = l % 32;
        double exact = 0, mag = 0;
        for (int k = 0; k < K; ++k) {
          const double p = e4m3(A[((size_t)t * 32 + m) * K + k]) * e4m3(B[((size_t)t * K + k) * 32 + col]);
          exact += p;
          mag += std::fabs(p);
        }
        const size_t i = ((size_t)t * 64 + l) * 16 + r;
        const double e8 = std::fabs(c8[i] - exact) / mag, e16 = std::fabs(c16[i] - exact) / mag;
        // the fp32 rounding of the exact value, the floor any fp32 result has
        const double e32 = std::fabs((double)(float)exact - exact) / mag;
        max8 = std::fmax(max8, e8); max16 = std::fmax(max16, e16); maxrel32_16 = std::fmax(maxrel32_16, e16 - e32);
        sum8 += e8; sum16 += e16; nz8 += e8 > 0; nz16 += e16 > 0; ++n;
      }
  printf("outputs %ld, K = %d\n", n, K);
  printf("fp8 MFMA : max |err|/sum|prod| = %.3g (2^%.1f), mean %.3g, nonzero %.1f%%\n", max8, std::log2(max8),
         sum8 / n, 100.0 * nz8 / n);
  printf("bf16 MFMA: max |err|/sum|prod| = %.3g (2^%.1f), mean %.3g, nonzero %.1f%%\n", max16,
         max16 > 0 ? std::log2(max16) : -999.0, sum16 / n, 100.0 * nz16 / n);
  return 0;
}
