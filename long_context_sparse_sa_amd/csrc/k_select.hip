// Exact top-k merge for the selection step (LongCat Sparse Attention deep-dive: DSA baseline section, arg-topK
// equation; SI section, the sparse part is the top-K over positions outside sink and window).
//
// One workgroup (1024 threads) per query gathers its candidates -- the k kept from earlier key ranges plus the
// ones the scoring kernels emitted -- and keeps exactly the k best by (score desc, position asc): four 8-bit radix
// passes on the order-preserving key find the k-th key, and four passes on the position resolve ties at that key
// towards lower positions. Intermediate calls keep the k best and publish the k-th key as the next threshold;
// the final call sorts the k positions ascending (final_mode 1) or in (key desc, position asc) order
// (final_mode 2, used for bucket ids) with a bitonic sort in LDS and writes idx / n_sel.
#include "sa_device.h"
#include "sa_internal.h"
#include "sa_wave_select.h"

namespace sa {
namespace {

constexpr int kMergeThreads = 1024;
constexpr int kMaxSortK = 16384;

struct MergeShared {
  uint32_t hist[256];
  uint32_t digit, before, in_bin;
  int n;
  int out;
};

// Block-wide digit search: wave 0 scans, everyone reads the result.
__device__ __forceinline__ void block_find_digit(MergeShared& sh, uint32_t need, bool descending) {
  __syncthreads();
  if (threadIdx.x < kWave) {
    uint32_t before, in_bin;
    const uint32_t dg = find_digit(sh.hist, need, descending, (int)threadIdx.x, &before, &in_bin);
    if (threadIdx.x == 0) {
      sh.digit = dg;
      sh.before = before;
      sh.in_bin = in_bin;
    }
  }
  __syncthreads();
}

// Ascending bitonic sort of a[0, n2) in LDS (n2 a power of two), all threads of the block.
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
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kMergeThreads) void k_merge(int k, const Cand* __restrict__ kept_in, int kept_ld,
                                                         const int32_t* __restrict__ kept_n_in,
                                                         const uint32_t* __restrict__ seg_cnt,
                                                         const Cand* __restrict__ seg_data, int n_seg, int seg_cap,
                                                         Cand* __restrict__ gather, int64_t gather_cap,
                                                         Cand* __restrict__ kept_out, int32_t* __restrict__ kept_n_out,
                                                         uint32_t* __restrict__ thr_out, int final_mode,
                                                         int32_t* __restrict__ idx, int idx_ld,
                                                         int32_t* __restrict__ n_sel) {
  __shared__ MergeShared sh;
  __shared__ int32_t sorted[kMaxSortK];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  constexpr int n_waves = kMergeThreads / kWave;
  Cand* g = gather + (int64_t)b * gather_cap;

  // ---- gather
  const int nk = kept_in ? kept_n_in[b] : 0;
  if (tid == 0) sh.n = nk;
  for (int i = tid; i < nk; i += kMergeThreads) g[i] = kept_in[(int64_t)b * kept_ld + i];
  __syncthreads();
  for (int s = wave; s < n_seg; s += n_waves) {
    const int c = (int)seg_cnt[(int64_t)b * n_seg + s];
    if (c == 0) continue;
    int base = 0;
    if (lane == 0) base = atomicAdd(&sh.n, c);
    base = __shfl(base, 0, kWave);
    const Cand* src = seg_data + ((int64_t)b * n_seg + s) * seg_cap;
    for (int i = lane; i < c; i += kWave) g[base + i] = src[i];
  }
  __syncthreads();
  const int n = sh.n;

  // ---- exact selection of min(k, n)
  uint32_t kstar = 0;
  int32_t pstar = 0x7FFFFFFF;
  if (n >= k) {
    uint32_t prefix = 0, mask = 0, need = (uint32_t)k, ties = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += kMergeThreads) sh.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kMergeThreads) {
        const uint32_t key = g[i].key;
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
      }
      block_find_digit(sh, need, true);
      need -= sh.before;
      ties = sh.in_bin;
      prefix |= sh.digit << shift;
      mask |= 255u << shift;
    }
    kstar = prefix;
    if (need < ties) {
      uint32_t pprefix = 0, pmask = 0, pneed = need;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += kMergeThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kMergeThreads) {
          const Cand e = g[i];
          const uint32_t p = (uint32_t)e.pos;
          if (e.key == kstar && (p & pmask) == pprefix) atomicAdd(&sh.hist[(p >> shift) & 255u], 1u);
        }
        block_find_digit(sh, pneed, false);
        pneed -= sh.before;
        pprefix |= sh.digit << shift;
        pmask |= 255u << shift;
      }
      pstar = (int32_t)pprefix;
    }
  }
  const int take = n < k ? n : k;

  // ---- output
  if (tid == 0) sh.out = 0;
  __syncthreads();
  if (!final_mode) {
    for (int i = tid; i < n; i += kMergeThreads) {
      const Cand e = g[i];
      if (n < k || e.key > kstar || (e.key == kstar && e.pos <= pstar)) {
        const int slot = atomicAdd(&sh.out, 1);
        kept_out[(int64_t)b * k + slot] = e;
      }
    }
    if (tid == 0) {
      kept_n_out[b] = take;
      thr_out[b] = n >= k ? kstar : 0u;
    }
    return;
  }
  int n2 = 1;
  while (n2 < take) n2 <<= 1;
  if (final_mode == 1) {
    // positions ascending
    for (int i = tid; i < n2; i += kMergeThreads) sorted[i] = 0x7FFFFFFF;
    __syncthreads();
    for (int i = tid; i < n; i += kMergeThreads) {
      const Cand e = g[i];
      if (n < k || e.key > kstar || (e.key == kstar && e.pos <= pstar)) sorted[atomicAdd(&sh.out, 1)] = e.pos;
    }
    __syncthreads();
    bitonic_sort(sorted, n2, tid);
    for (int i = tid; i < idx_ld; i += kMergeThreads) idx[(int64_t)b * idx_ld + i] = i < take ? sorted[i] : -1;
  } else {
    // (key desc, position asc): sort ascending on (~key << 32 | position)
    uint64_t* sorted64 = reinterpret_cast<uint64_t*>(sorted);
    for (int i = tid; i < n2; i += kMergeThreads) sorted64[i] = ~0ull;
    __syncthreads();
    for (int i = tid; i < n; i += kMergeThreads) {
      const Cand e = g[i];
      if (n < k || e.key > kstar || (e.key == kstar && e.pos <= pstar))
        sorted64[atomicAdd(&sh.out, 1)] = ((uint64_t)(~e.key) << 32) | (uint32_t)e.pos;
    }
    __syncthreads();
    bitonic_sort(sorted64, n2, tid);
    for (int i = tid; i < idx_ld; i += kMergeThreads)
      idx[(int64_t)b * idx_ld + i] = i < take ? (int32_t)(uint32_t)sorted64[i] : -1;
  }
  if (tid == 0) n_sel[b] = take;
}

}  // namespace

hipError_t launch_merge(int B, int k, const Cand* kept_in, int kept_ld, const int32_t* kept_n_in,
                        const uint32_t* seg_cnt, const Cand* seg_data, int n_seg, int seg_cap, Cand* gather,
                        int64_t gather_cap, Cand* kept_out, int32_t* kept_n_out, uint32_t* thr_out, int final_mode,
                        int32_t* idx, int idx_ld, int32_t* n_sel, hipStream_t st) {
  if ((final_mode == 1 && k > kMaxSortK) || (final_mode == 2 && k > kMaxSortK / 2)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_merge, dim3((unsigned)B), dim3(kMergeThreads), 0, st, k, kept_in, kept_ld, kept_n_in, seg_cnt,
                     seg_data, n_seg, seg_cap, gather, gather_cap, kept_out, kept_n_out, thr_out, final_mode, idx,
                     idx_ld, n_sel);
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
