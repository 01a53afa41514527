// Exact top-k merge for the selection step (LongCat Sparse Attention deep-dive: DSA baseline section, arg-topK
// equation; SI section, the sparse part is the top-K over positions outside sink and window).
//
// One workgroup (1024 threads) per query gathers its candidates -- the k kept from earlier key ranges plus the
// ones the scoring kernels emitted -- and keeps exactly the k best by (score desc, position asc):
//   * candidate keys are staged in LDS; a min/max pass finds the bits all of them share, and radix passes (8-bit
//     digits, privatized histograms) run only over the bits below that common prefix;
//   * when several candidates share the k-th key, radix passes over their positions keep the lowest ones.
// Intermediate calls keep the k best and publish the k-th key as the next threshold; the final call sorts the k
// positions ascending (final_mode 1) or in (key desc, position asc) order (final_mode 2, used for bucket ids) with
// a bitonic sort in LDS whose stages of stride <= 64 run inside one wave, and writes idx / n_sel.
#include "sa_device.h"
#include "sa_internal.h"
#include "sa_wave_select.h"

namespace sa {
namespace {

constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kHistCopies = 4;        // private histograms, one per 4 waves
constexpr int kMaxSortK = 16384;
constexpr int kBatch = 8;             // candidates loaded per thread before they are processed
constexpr int kLdsBytes = 163840;     // LDS per workgroup on gfx950

struct MergeShared {
  uint32_t hist[kHistCopies][256];
  uint32_t tot[256];
  uint32_t digit, before, in_bin;
  uint32_t kmin, kmax;
  int n, out;
};

__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Ascending bitonic sort of a[0, n2) in LDS (n2 a power of two, >= 2), all threads of the block. Thread t handles
// pair indices t, t + 1024, ...; for strides <= 64 the 64 pairs of a wave touch 128 consecutive elements that no
// other wave touches, so those stages need no block barrier.
template <typename T>
__device__ __forceinline__ void bitonic_sort(T* a, int n2, int tid) {
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += kMergeThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const T x = a[lo], y = a[hi];
        if ((x > y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      const int next = stride > 1 ? stride >> 1 : size;
      if (stride > 64 || next > 64)
        __syncthreads();
      else
        wave_lds_fence();
    }
  }
  __syncthreads();
}

// Block-wide histogram pass over the candidates matching (prefix, mask) on digit (v >> shift) & 255, then the
// digit search. `src(i, &v)` gives the radix value of candidate i, or false when the candidate does not take part.
template <typename Src>
__device__ __forceinline__ void radix_pass(MergeShared& sh, int n, Src src, uint32_t prefix, uint32_t mask,
                                           int shift, uint32_t need, bool descending, int tid, int wave) {
  for (int i = tid; i < kHistCopies * 256; i += kMergeThreads) (&sh.hist[0][0])[i] = 0;
  __syncthreads();
  uint32_t* h = sh.hist[wave % kHistCopies];
  for (int i = tid; i < n; i += kMergeThreads) {
    uint32_t v;
    if (src(i, &v) && (v & mask) == prefix) atomicAdd(&h[(v >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (tid < 256) {
    uint32_t s = 0;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) s += sh.hist[c][tid];
    sh.tot[tid] = s;
  }
  __syncthreads();
  if (tid < kWave) {
    uint32_t before, in_bin;
    const uint32_t dg = find_digit(sh.tot, need, descending, tid, &before, &in_bin);
    if (tid == 0) {
      sh.digit = dg;
      sh.before = before;
      sh.in_bin = in_bin;
    }
  }
  __syncthreads();
}

// Dynamic LDS: [sort area: sort_bytes][candidate keys: up to key_cap]. The gather buffer always holds every
// candidate; when they do not all fit in LDS the keys are read from it instead.
__global__ __launch_bounds__(kMergeThreads) void k_merge(int k, const Cand* __restrict__ kept_in, int kept_ld,
                                                         const int32_t* __restrict__ kept_n_in,
                                                         const Cand* __restrict__ cand, int64_t cand_ld,
                                                         const uint32_t* __restrict__ cand_cnt, int64_t cand_n,
                                                         uint32_t* __restrict__ zero_cnt,
                                                         Cand* __restrict__ gather, int64_t gather_cap,
                                                         Cand* __restrict__ kept_out, int32_t* __restrict__ kept_n_out,
                                                         uint32_t* __restrict__ thr_out, int final_mode,
                                                         int32_t* __restrict__ idx, int idx_ld,
                                                         int32_t* __restrict__ n_sel, int sort_bytes, int key_cap) {
  __shared__ MergeShared sh;
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  int32_t* sorted = reinterpret_cast<int32_t*>(dyn);
  uint32_t* keys_s = reinterpret_cast<uint32_t*>(dyn + sort_bytes);
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  Cand* g = gather + (int64_t)b * gather_cap;

  const int nk = kept_in ? kept_n_in[b] : 0;
  const int64_t nc = cand ? (cand_cnt ? (int64_t)cand_cnt[b] : cand_n) : 0;
  const bool fits = nk + nc <= key_cap;
  if (tid == 0) {
    sh.n = 0;
    sh.out = 0;
    sh.kmin = 0xFFFFFFFFu;
    sh.kmax = 0u;
  }
  __syncthreads();

  // ---- gather: kBatch independent loads per thread, then one LDS atomic per wave for the slots
  auto gather_from = [&](const Cand* src, int64_t cnt) {
    for (int64_t base = 0; base < cnt; base += (int64_t)kMergeThreads * kBatch) {
      Cand c[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t i = base + j * kMergeThreads + tid;
        c[j] = i < cnt ? src[i] : Cand{0u, -1};
      }
      uint64_t m[kBatch];
      int tot = 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        m[j] = ballot(c[j].key != 0u);  // key 0 marks an empty slot
        tot += __popcll(m[j]);
      }
      int wb = 0;
      if (lane == 0 && tot) wb = atomicAdd(&sh.n, tot);
      wb = __shfl(wb, 0, kWave);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (c[j].key != 0u) {
          const int slot = wb + lanes_below(m[j]);
          g[slot] = c[j];
          if (fits) keys_s[slot] = c[j].key;
        }
        wb += __popcll(m[j]);
      }
    }
  };
  if (nk) gather_from(kept_in + (int64_t)b * kept_ld, nk);
  if (nc) gather_from(cand + (int64_t)b * cand_ld, nc);
  __syncthreads();
  const int n = sh.n;
  if (zero_cnt && tid == 0) zero_cnt[b] = 0u;  // the next key range counts its candidates from zero
  auto key_at = [&](int i) -> uint32_t { return fits ? keys_s[i] : g[i].key; };

  // ---- exact selection of min(k, n)
  uint32_t kstar = 0;
  int32_t pstar = 0x7FFFFFFF;
  if (n >= k) {
    // bits shared by every candidate key
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
    for (int i = tid; i < n; i += kMergeThreads) {
      const uint32_t v = key_at(i);
      lmin = v < lmin ? v : lmin;
      lmax = v > lmax ? v : lmax;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t x = __shfl_xor(lmin, off, kWave), y = __shfl_xor(lmax, off, kWave);
      lmin = x < lmin ? x : lmin;
      lmax = y > lmax ? y : lmax;
    }
    if (lane == 0) {
      atomicMin(&sh.kmin, lmin);
      atomicMax(&sh.kmax, lmax);
    }
    __syncthreads();
    const uint32_t kmin = sh.kmin, kmax = sh.kmax;
    uint32_t need = (uint32_t)k, ties = (uint32_t)n;
    int bits = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);  // low bits that still differ
    uint32_t mask = bits == 32 ? 0u : ~((1u << bits) - 1u);
    uint32_t prefix = kmin & mask;
    auto key_src = [&](int i, uint32_t* v) {
      *v = key_at(i);
      return true;
    };
    while (bits > 0) {
      const int d = bits < 8 ? bits : 8;
      const int shift = bits - d;
      radix_pass(sh, n, key_src, prefix, mask, shift, need, true, tid, wave);
      need -= sh.before;
      ties = sh.in_bin;
      prefix |= sh.digit << shift;
      mask |= ((1u << d) - 1u) << shift;
      bits -= d;
    }
    kstar = prefix;
    if (need < ties) {
      // several candidates share the k-th key: keep the `need` lowest positions among them
      uint32_t pprefix = 0, pmask = 0, pneed = need;
      auto pos_src = [&](int i, uint32_t* v) {
        if (key_at(i) != kstar) return false;
        *v = (uint32_t)g[i].pos;
        return true;
      };
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        radix_pass(sh, n, pos_src, pprefix, pmask, shift, pneed, false, tid, wave);
        pneed -= sh.before;
        pprefix |= sh.digit << shift;
        pmask |= 255u << shift;
      }
      pstar = (int32_t)pprefix;
    }
  }
  const int take = n < k ? n : k;

  // ---- output, phase A: indices of the selected candidates into the sort area (wave-aggregated slots)
  for (int base = 0; base < n; base += kMergeThreads) {
    const int i = base + tid;
    bool sel = false;
    if (i < n) {
      const uint32_t key = key_at(i);
      sel = n < k || key > kstar || (key == kstar && g[i].pos <= pstar);
    }
    const uint64_t m = ballot(sel);
    int wb = 0;
    if (lane == 0 && m) wb = atomicAdd(&sh.out, __popcll(m));
    wb = __shfl(wb, 0, kWave);
    if (sel) sorted[wb + lanes_below(m)] = i;
  }
  __syncthreads();
  // phase B: independent loads of the selected candidates
  if (!final_mode) {
    for (int s2 = tid; s2 < take; s2 += kMergeThreads) kept_out[(int64_t)b * k + s2] = g[sorted[s2]];
    if (tid == 0) {
      kept_n_out[b] = take;
      thr_out[b] = n >= k ? kstar : 0u;
    }
    return;
  }
  int n2 = 2;
  while (n2 < take) n2 <<= 1;
  if (final_mode == 1) {
    for (int s2 = tid; s2 < n2; s2 += kMergeThreads) sorted[s2] = s2 < take ? g[sorted[s2]].pos : 0x7FFFFFFF;
    __syncthreads();
    bitonic_sort(sorted, n2, tid);
    for (int i = tid; i < idx_ld; i += kMergeThreads) idx[(int64_t)b * idx_ld + i] = i < take ? sorted[i] : -1;
  } else {
    // (key desc, position asc): sort ascending on (~key << 32 | position); the index list is read first
    uint64_t* sorted64 = reinterpret_cast<uint64_t*>(dyn);
    uint64_t v[kMaxSortK / 2 / kMergeThreads];
#pragma unroll
    for (int j = 0; j < kMaxSortK / 2 / kMergeThreads; ++j) {
      const int s2 = j * kMergeThreads + tid;
      v[j] = ~0ull;
      if (s2 < take) {
        const Cand e = g[sorted[s2]];
        v[j] = ((uint64_t)(~e.key) << 32) | (uint32_t)e.pos;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxSortK / 2 / kMergeThreads; ++j) {
      const int s2 = j * kMergeThreads + tid;
      if (s2 < n2) sorted64[s2] = v[j];
    }
    __syncthreads();
    bitonic_sort(sorted64, n2, tid);
    for (int i = tid; i < idx_ld; i += kMergeThreads)
      idx[(int64_t)b * idx_ld + i] = i < take ? (int32_t)(uint32_t)sorted64[i] : -1;
  }
  if (tid == 0) n_sel[b] = take;
}

}  // namespace

hipError_t launch_merge(int B, int k, const Cand* kept_in, int kept_ld, const int32_t* kept_n_in, const Cand* cand,
                        int64_t cand_ld, const uint32_t* cand_cnt, int64_t cand_n, uint32_t* zero_cnt, Cand* gather,
                        int64_t gather_cap, Cand* kept_out, int32_t* kept_n_out, uint32_t* thr_out, int final_mode,
                        int32_t* idx, int idx_ld, int32_t* n_sel, hipStream_t st) {
  if (k < 1 || (final_mode == 1 && k > kMaxSortK) || (final_mode == 2 && k > kMaxSortK / 2)) return hipErrorInvalidValue;
  int n2 = 2;
  while (n2 < k) n2 <<= 1;
  const int sort_bytes = n2 * (final_mode == 2 ? 8 : 4);
  const int dyn = kLdsBytes - (int)sizeof(MergeShared) - 256;
  const int key_cap = (dyn - sort_bytes) / 4;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_merge), hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_merge, dim3((unsigned)B), dim3(kMergeThreads), (size_t)dyn, st, k, kept_in, kept_ld, kept_n_in,
                     cand, cand_ld, cand_cnt, cand_n, zero_cnt, gather, gather_cap, kept_out, kept_n_out, thr_out,
                     final_mode, idx, idx_ld, n_sel, sort_bytes, key_cap);
  return hipGetLastError();
}

int merge_max_k() { return kMaxSortK; }

namespace {
__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}
}  // namespace

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks64 = (n + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 1024 ? blocks64 : 1024);
  hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace sa
