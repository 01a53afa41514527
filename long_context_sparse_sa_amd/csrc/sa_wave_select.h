// Exact radix selection helpers (wave level) for the top-k of (key desc, position asc).
//
// Candidates are (key, pos) pairs where key is the order-preserving image of an fp32 score. The k best are found
// with four 8-bit radix passes over the key (most significant digit first); when several candidates share the
// k-th key, four more passes over the position pick the lowest positions among them (ties go to the lower
// position, as the selection rule requires). Positions are unique, so the result is exactly k candidates.
#pragma once

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

// Inclusive prefix sum over the 64 lanes with DPP row operations (no LDS round trips): shifts by 1, 2, 4 and 8
// inside each row of 16 lanes, then row 0's total is broadcast into row 1 (and row 2's into row 3), then the
// total of rows 0-1 into rows 2-3. Lanes a shift moves past the row start read `old` = 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
  (void)lane;
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2 and 3
  return (uint32_t)x;
}

// One wave scans 256 histogram bins in the order of selection (descending digit for keys, ascending for
// positions) and finds the bin in which the running count first reaches `need`. Returns the digit; `before` is
// the number of candidates in bins ahead of it. All lanes return the same values.
__device__ __forceinline__ uint32_t find_digit(const uint32_t* hist, uint32_t need, bool descending, int lane,
                                               uint32_t* before, uint32_t* in_bin) {
  uint32_t c[4];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = 4 * lane + i;
    c[i] = hist[descending ? 255 - o : o];
    local += c[i];
  }
  const uint32_t incl = wave_inclusive_scan(local, lane);
  uint32_t run = incl - local;
  int found = -1;
  uint32_t fb = 0, fc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (found < 0 && run < need && run + c[i] >= need) {
      found = 4 * lane + i;
      fb = run;
      fc = c[i];
    }
    run += c[i];
  }
  const uint64_t m = ballot(found >= 0);
  const int src = m ? (int)__builtin_ctzll(m) : 0;  // uniform: the values are read as scalars
  const int o = __builtin_amdgcn_readlane(found, src);
  *before = (uint32_t)__builtin_amdgcn_readlane((int)fb, src);
  *in_bin = (uint32_t)__builtin_amdgcn_readlane((int)fc, src);
  return (uint32_t)(descending ? 255 - o : o);
}

// Wave-level exact top-k of buf[0, n) (n > k is not required). Afterwards buf[0, min(n, k)) holds the selected
// candidates (in their original relative order) and the return value is the k-th key (0 when n < k).
// `hist` is 256 words of LDS private to this wave. Every lane must call it with the same n.
// Every pass reads the buffer kBatchW entries per lane at a time, so the loads of a batch are in flight together;
// the key passes cover only the bits below the prefix that every key shares.
constexpr int kBatchW = 16;

template <typename F>
__device__ __forceinline__ void wave_batched(const Cand* buf, int n, int lane, F f) {
  for (int base = 0; base < n; base += kWave * kBatchW) {
    Cand c[kBatchW];
#pragma unroll
    for (int j = 0; j < kBatchW; ++j) {
      const int i = base + j * kWave + lane;
      c[j] = i < n ? buf[i] : Cand{0u, -1};
    }
#pragma unroll
    for (int j = 0; j < kBatchW; ++j)
      if (base + j * kWave + lane < n) f(c[j]);
  }
}

// Minimum / maximum over the wave, the same in every lane: DPP swaps reduce each row of 16 lanes, then the four
// row results are read as scalars.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_swap<0xB1>(v));
  v = min(v, dpp_swap<0x4E>(v));
  v = min(v, dpp_swap<0x141>(v));
  v = min(v, dpp_swap<0x140>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(r0, r1), min(r2, r3));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_swap<0xB1>(v));
  v = max(v, dpp_swap<0x4E>(v));
  v = max(v, dpp_swap<0x141>(v));
  v = max(v, dpp_swap<0x140>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

__device__ __noinline__ uint32_t wave_select_compact(Cand* buf, int n, int k, uint32_t* hist, int lane) {
  if (n < k) return 0u;
  // ---- bits shared by every key
  uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
  wave_batched(buf, n, lane, [&](const Cand& e) {
    lmin = e.key < lmin ? e.key : lmin;
    lmax = e.key > lmax ? e.key : lmax;
  });
  const uint32_t kmin = wave_min_u32(lmin), kmax = wave_max_u32(lmax);
  int bits = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);
  uint32_t mask = bits == 32 ? 0u : ~((1u << bits) - 1u);
  uint32_t prefix = kmin & mask, need = (uint32_t)k, ties = (uint32_t)n;
  // ---- key passes over the differing bits
  while (bits > 0) {
    const int d = bits < 8 ? bits : 8;
    const int shift = bits - d;
    for (int i = lane; i < 256; i += kWave) hist[i] = 0;
    __builtin_amdgcn_wave_barrier();
    wave_batched(buf, n, lane, [&](const Cand& e) {
      if ((e.key & mask) == prefix) atomicAdd(&hist[(e.key >> shift) & 255u], 1u);
    });
    __builtin_amdgcn_wave_barrier();
    uint32_t before, in_bin;
    const uint32_t dg = find_digit(hist, need, true, lane, &before, &in_bin);
    need -= before;
    ties = in_bin;
    prefix |= dg << shift;
    mask |= ((1u << d) - 1u) << shift;
    bits -= d;
    __builtin_amdgcn_wave_barrier();
  }
  const uint32_t kstar = prefix;
  // ---- position passes among the candidates tied at the k-th key
  int32_t pstar = 0x7FFFFFFF;
  if (need < ties) {
    uint32_t pprefix = 0, pmask = 0, pneed = need;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = lane; i < 256; i += kWave) hist[i] = 0;
      __builtin_amdgcn_wave_barrier();
      wave_batched(buf, n, lane, [&](const Cand& e) {
        const uint32_t p = (uint32_t)e.pos;
        if (e.key == kstar && (p & pmask) == pprefix) atomicAdd(&hist[(p >> shift) & 255u], 1u);
      });
      __builtin_amdgcn_wave_barrier();
      uint32_t before, in_bin;
      const uint32_t dg = find_digit(hist, pneed, false, lane, &before, &in_bin);
      pneed -= before;
      pprefix |= dg << shift;
      pmask |= 255u << shift;
      __builtin_amdgcn_wave_barrier();
    }
    pstar = (int32_t)pprefix;
  }
  // ---- in-place stable compaction; a batch is loaded whole before any of it is written back, and writes never
  // pass the read front
  int out = 0;
  for (int base = 0; base < n; base += kWave * kBatchW) {
    Cand c[kBatchW];
#pragma unroll
    for (int j = 0; j < kBatchW; ++j) {
      const int i = base + j * kWave + lane;
      c[j] = i < n ? buf[i] : Cand{0u, -1};
    }
#pragma unroll
    for (int j = 0; j < kBatchW; ++j) {
      const int i = base + j * kWave + lane;
      const bool keep = i < n && (c[j].key > kstar || (c[j].key == kstar && c[j].pos <= pstar));
      const uint64_t m = ballot(keep);
      if (keep) buf[out + lanes_below(m)] = c[j];
      out += __popcll(m);
    }
  }
  return kstar;
}

}  // namespace sa
