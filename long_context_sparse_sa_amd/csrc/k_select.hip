// Exact top-k merge for the selection step (LongCat Sparse Attention deep-dive: DSA baseline section, arg-topK
// equation; SI section, the sparse part is the top-K over positions outside sink and window).
//
// One workgroup (1024 threads) per query gathers its candidates -- the k kept from earlier key ranges plus the
// slots or segments a scoring launch wrote -- and keeps exactly the k best by (score desc, position asc):
//   * the gather and the output are order-preserving (ballot masks of 16 rounds of 1024 entries, one scan per
//     batch), so inputs in ascending position order give outputs in ascending position order without a sort;
//   * keys and positions live in LDS, or in the gather buffer in global memory when they do not fit; the storage
//     is a compile-time choice, so every access is a plain LDS or global load;
//   * segments are gathered a chunk at a time, every entry located by a binary search over the segment offsets, so
//     that all loads of a chunk are in flight together;
//   * the bits all keys share are skipped; 12-bit radix passes find the k-th key;
//     when several candidates share it, radix passes over their positions keep the lowest ones.
// Intermediate calls keep the k best and publish the k-th key as the next threshold. Bucket ranking (final_mode
// 2) is the one caller that needs (key desc, position asc) order; it sorts its at most top_b ids in LDS.
#include <atomic>

#include "sa_device.h"
#include "sa_internal.h"
#include "sa_wave_select.h"

namespace sa {
namespace {

constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kHistCopies = 1;
constexpr int kDigitBits = 12;  // radix digit width: two passes cover the 24 bits that keys near one binade differ in
constexpr int kBins = 1 << kDigitBits;
constexpr int kBinsPerThread = kBins / 1024;
static_assert(kBinsPerThread * 1024 == kBins, "the digit search gives each of the 1024 threads whole bins");
constexpr int kRounds = 16;  // rounds of 1024 entries compacted per batch
constexpr int kBatch = kRounds * kMergeThreads;
constexpr int kMaxSortK = 16384;
constexpr int kLdsBytes = 163840;  // LDS per workgroup on gfx950

struct MergeShared {
  union {
    uint32_t hist[kHistCopies][kBins];  // selection passes
    struct {
      int32_t off[kMergeThreads];  // gather: offset of each segment of a chunk in the chunk's concatenation
    } seg;
  } u;
  uint64_t masks[kRounds][kMergeWaves];
  int32_t moff[kRounds * kMergeWaves];
  int32_t wsum[kMergeWaves];
  int32_t batch_total;
  uint32_t digit, before, in_bin;
  uint32_t kmin, kmax;
  uint32_t small_n, small_key;  // small-bin finish: entries listed, the k-th key and position found
  int32_t small_pos;
};

// Order-preserving compaction of one batch: entry r * 1024 + tid (r < kRounds) is flagged by f[r]. Returns the
// number of flagged entries; slot[r] receives the rank of entry r among them. All threads must call.
__device__ __forceinline__ int batch_slots(MergeShared& sh, const bool (&f)[kRounds], int (&slot)[kRounds], int tid) {
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  uint64_t m[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    m[r] = ballot(f[r]);
    if (lane == 0) sh.masks[r][wave] = m[r];
  }
  __syncthreads();
  if (wave == 0) {  // the 256 (round, wave) counts in entry order, four per lane
    int c[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      c[j] = __popcll(sh.masks[e / kMergeWaves][e % kMergeWaves]);
      local += c[j];
    }
    const int incl = (int)wave_inclusive_scan((uint32_t)local, lane);
    int run = incl - local;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sh.moff[4 * lane + j] = run;
      run += c[j];
    }
    if (lane == kWave - 1) sh.batch_total = incl;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r) slot[r] = sh.moff[r * kMergeWaves + wave] + lanes_below(m[r]);
  return sh.batch_total;
}

// Block-wide exclusive scan of one int per thread; *total receives the sum. All threads must call.
__device__ __forceinline__ int block_scan(MergeShared& sh, int v, int tid, int* total) {
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int incl = (int)wave_inclusive_scan((uint32_t)v, lane);
  if (lane == kWave - 1) sh.wsum[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    const int x = sh.wsum[w];
    before += w < wave ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__device__ __forceinline__ void note_minmax(uint32_t& lmin, uint32_t& lmax, uint32_t key) {
  lmin = key < lmin ? key : lmin;
  lmax = key > lmax ? key : lmax;
}

// One radix pass over a digit of d <= kDigitBits bits at `shift`, then the digit search in the order of selection
// (descending for keys, ascending for positions). Key passes (kPos false) count the keys matching (prefix, mask);
// position passes count the positions matching (prefix, mask) among entries whose key equals kstar. Loads are
// unconditional (clamped index) and batched four per thread, so they are in flight together; only the counting
// is predicated. Every thread then takes kBinsPerThread bins of the digit search.
template <bool kPos>
__device__ __forceinline__ void radix_pass(MergeShared& sh, int n, const uint32_t* K, const int32_t* P, uint32_t kstar,
                                           uint32_t prefix, uint32_t mask, int shift, int d, uint32_t need, int tid) {
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t dmask = (1u << d) - 1u;
  for (int i = tid; i < kHistCopies * kBins; i += kMergeThreads) (&sh.u.hist[0][0])[i] = 0;
  __syncthreads();
  uint32_t* h = sh.u.hist[wave % kHistCopies];
  for (int base = 0; base < n; base += 4 * kMergeThreads) {
    uint32_t kv[4], pv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + j * kMergeThreads + tid;
      const int ic = i < n ? i : n - 1;
      kv[j] = K[ic];
      if (kPos) pv[j] = (uint32_t)P[ic];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = base + j * kMergeThreads + tid < n;
      const uint32_t v = kPos ? pv[j] : kv[j];
      const bool ok = in && (!kPos || kv[j] == kstar) && (v & mask) == prefix;
      if (ok) atomicAdd(&h[(v >> shift) & dmask], 1u);
    }
  }
  __syncthreads();
  // digit search with every thread: thread t owns selection-order bins kBinsPerThread * t .. + kBinsPerThread - 1
  const bool descending = !kPos;
  const int nb = 1 << d;
  uint32_t c[kBinsPerThread], local = 0;
  int binof[kBinsPerThread];
#pragma unroll
  for (int e = 0; e < kBinsPerThread; ++e) {
    const int o = kBinsPerThread * tid + e;
    binof[e] = descending ? nb - 1 - o : o;
    c[e] = 0;
    if (o < nb)
#pragma unroll
      for (int cp = 0; cp < kHistCopies; ++cp) c[e] += sh.u.hist[cp][binof[e]];
    local += c[e];
  }
  const uint32_t winc = wave_inclusive_scan(local, lane);
  if (lane == kWave - 1) sh.wsum[wave] = (int32_t)winc;
  __syncthreads();
  uint32_t before_w = 0;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) before_w += w < wave ? (uint32_t)sh.wsum[w] : 0u;
  const uint32_t incl = before_w + winc, excl = incl - local;
  if (excl < need && incl >= need) {
    uint32_t run = excl;
    bool found = false;
#pragma unroll
    for (int e = 0; e < kBinsPerThread; ++e) {
      if (!found && run + c[e] >= need) {
        found = true;
        sh.digit = (uint32_t)binof[e];
        sh.before = run;
        sh.in_bin = c[e];
      }
      run += c[e];
    }
  }
  __syncthreads();
}

// The k-th entry when at most 64 entries are left in its bin: the `ties` entries whose key matches (prefix, mask)
// are listed in LDS (in the histogram area, free after a pass) and one wave ranks them exactly in (key desc,
// position asc) order; positions are distinct, so exactly one entry has rank need - 1. Its key and position are
// kstar and pstar: every entry above it in that order, and no other, is kept. All threads must call.
__device__ __forceinline__ void small_bin_finish(MergeShared& sh, int n, const uint32_t* K, const int32_t* P,
                                                 uint32_t prefix, uint32_t mask, uint32_t need, int tid,
                                                 uint32_t* kstar, int32_t* pstar) {
  uint32_t* lk = &sh.u.hist[0][0];
  int32_t* lp = reinterpret_cast<int32_t*>(&sh.u.hist[0][kWave]);
  if (tid == 0) sh.small_n = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 4 * kMergeThreads) {
    uint32_t kv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + j * kMergeThreads + tid;
      kv[j] = K[i < n ? i : n - 1];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + j * kMergeThreads + tid;
      if (i < n && (kv[j] & mask) == prefix) {
        const uint32_t o = atomicAdd(&sh.small_n, 1u);
        lk[o] = kv[j];
        lp[o] = P[i];
      }
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const int m = (int)sh.small_n;
    const uint32_t mk = tid < m ? lk[tid] : 0u;
    const int32_t mp = tid < m ? lp[tid] : 0x7FFFFFFF;
    int rank = 0;
    for (int j = 0; j < m; ++j) {
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mk, j);
      const int32_t pj = __builtin_amdgcn_readlane(mp, j);
      rank += (kj > mk || (kj == mk && pj < mp)) ? 1 : 0;
    }
    if (tid < m && rank == (int)need - 1) {
      sh.small_key = mk;
      sh.small_pos = mp;
    }
  }
  __syncthreads();
  *kstar = sh.small_key;
  *pstar = sh.small_pos;
}

// Ascending bitonic sort of a[0, n2) in LDS (n2 a power of two, >= 2), all threads of the block.
__device__ __forceinline__ void bitonic_sort(uint64_t* a, int n2, int tid) {
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += kMergeThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t x = a[lo], y = a[hi];
        if ((x > y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Gather, select and write one query's result, with keys K[] and positions P[] in LDS (kLds) or in the gather
// buffer in global memory.
template <bool kLds>
__device__ __forceinline__ void merge_body(MergeShared& sh, int b, int k, const MergeIn& in, const MergeOut& out,
                                           uint32_t* __restrict__ K, int32_t* __restrict__ P, int nk,
                                           uint64_t* sort_area) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;

  // ---- gather: the kept entries, then the slots (compacted) or the segments, all in input order
  if (nk) {
    const Cand* src = in.kept + (int64_t)b * in.kept_ld;
    for (int base = 0; base < nk; base += 4 * kMergeThreads) {
      Cand c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + j * kMergeThreads + tid;
        c[j] = i < nk ? src[i] : Cand{0u, 0};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + j * kMergeThreads + tid;
        if (i < nk) {
          K[i] = c[j].key;
          P[i] = c[j].pos;
          note_minmax(lmin, lmax, c[j].key);
        }
      }
    }
  }
  int n = nk;
  const Cand* cb = in.cand ? in.cand + (int64_t)b * in.cand_ld : nullptr;
  if (in.slot_key) {
    const uint32_t* kb = in.slot_key + (int64_t)b * in.slot_ld;
    for (int64_t base = 0; base < in.n_slots; base += kBatch) {
      uint32_t c[kRounds];
      bool f[kRounds];
      int slot[kRounds];
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        const int64_t i = base + r * kMergeThreads + tid;
        c[r] = i < in.n_slots ? kb[i] : 0u;
      }
#pragma unroll
      for (int r = 0; r < kRounds; ++r) f[r] = c[r] != 0u;
      const int got = batch_slots(sh, f, slot, tid);
#pragma unroll
      for (int r = 0; r < kRounds; ++r)
        if (f[r]) {
          K[n + slot[r]] = c[r];
          P[n + slot[r]] = in.slot_pos0 + (int32_t)(base + r * kMergeThreads + tid);
          note_minmax(lmin, lmax, c[r]);
        }
      n += got;
    }
  }
  if (cb) {
    // segments are taken 1024 at a time. The segment of each entry of a chunk's concatenation is first written
    // into that entry's position slot (one wave per segment); then every thread requests its entries eight at once,
    // from unconditional addresses (entries past the end read entry 0 of the chunk's first segment), so that the
    // whole chunk arrives in one round trip instead of one per segment. Each entry's slot is read and then
    // overwritten by the one thread that owns the entry.
    for (int w0 = 0; w0 < in.n_seg; w0 += kMergeThreads) {
      const int w = w0 + tid;
      const int c = w < in.n_seg ? (int)in.seg_cnt[(int64_t)b * in.n_seg + w] : 0;
      int total;
      const int ex = block_scan(sh, c, tid, &total);
      sh.u.seg.off[tid] = ex;
      __syncthreads();
      const int nw = in.n_seg - w0 < kMergeThreads ? in.n_seg - w0 : kMergeThreads;
      for (int j = wave; j < nw; j += kMergeWaves) {
        const int o = sh.u.seg.off[j];
        const int cnt = (j + 1 < nw ? sh.u.seg.off[j + 1] : total) - o;
        for (int e = lane; e < cnt; e += kWave) P[n + o + e] = j;
      }
      __syncthreads();
      const Cand* chunk = cb + (int64_t)w0 * in.seg_cap;
      constexpr int kPer = 8;  // entries per thread in flight together
      for (int e0 = 0; e0 < total; e0 += kPer * kMergeThreads) {
        Cand c8[kPer];
        int js[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int e = e0 + u * kMergeThreads + tid;
          const int v = P[n + (e < total ? e : total - 1)];
          js[u] = e < total ? v : 0;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int e = e0 + u * kMergeThreads + tid;
          const int within = e < total ? e - sh.u.seg.off[js[u]] : 0;
          c8[u] = chunk[(int64_t)js[u] * in.seg_cap + within];
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int e = e0 + u * kMergeThreads + tid;
          if (e < total) {
            K[n + e] = c8[u].key;
            P[n + e] = c8[u].pos;
            note_minmax(lmin, lmax, c8[u].key);
          }
        }
      }
      n += total;
      __syncthreads();
    }
  }
  lmin = wave_min_u32(lmin);
  lmax = wave_max_u32(lmax);
  if (lane == 0) {
    atomicMin(&sh.kmin, lmin);
    atomicMax(&sh.kmax, lmax);
  }
  __syncthreads();

  // ---- exact selection of min(k, n)
  uint32_t kstar = 0;
  int32_t pstar = 0x7FFFFFFF;
  if (n >= k) {
    const uint32_t kmin = sh.kmin, kmax = sh.kmax;
    uint32_t need = (uint32_t)k, ties = (uint32_t)n;
    int bits = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);  // low bits that still differ
    uint32_t mask = bits == 32 ? 0u : ~((1u << bits) - 1u);
    uint32_t prefix = kmin & mask;
    bool small = false;
    while (bits > 0) {
      const int d = bits < kDigitBits ? bits : kDigitBits;
      const int shift = bits - d;
      radix_pass<false>(sh, n, K, P, 0u, prefix, mask, shift, d, need, tid);
      need -= sh.before;
      ties = sh.in_bin;
      prefix |= sh.digit << shift;
      mask |= ((1u << d) - 1u) << shift;
      bits -= d;
      // few entries left in the k-th key's bin: rank them in one wave instead of more passes over all entries
      if (ties <= (uint32_t)kWave && (bits > 0 || need < ties)) {
        small_bin_finish(sh, n, K, P, prefix, mask, need, tid, &kstar, &pstar);
        small = true;
        break;
      }
    }
    if (!small) kstar = prefix;
    if (!small && need < ties) {
      // several candidates share the k-th key: keep the `need` lowest positions among them
      uint32_t pprefix = 0, pmask = 0, pneed = need;
      // positions are below 2^31: digits of bits 30..19, 18..7 and 6..0
      for (int pbits = 31; pbits > 0;) {
        const int d = pbits < kDigitBits ? pbits : kDigitBits;
        const int shift = pbits - d;
        radix_pass<true>(sh, n, K, P, kstar, pprefix, pmask, shift, d, pneed, tid);
        pneed -= sh.before;
        pprefix |= sh.digit << shift;
        pmask |= ((1u << d) - 1u) << shift;
        pbits -= d;
      }
      pstar = (int32_t)pprefix;
    }
  }
  const int take = n < k ? n : k;

  // ---- the selected entries, in input order
  int done = 0;
  for (int base = 0; base < n; base += kBatch) {
    bool f[kRounds];
    int slot[kRounds];
    uint32_t kv[kRounds];
    int32_t pv[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {  // unconditional (clamped) reads, all in flight together
      const int i = base + r * kMergeThreads + tid;
      const int ic = i < n ? i : n - 1;
      kv[r] = K[ic];
      pv[r] = P[ic];
      f[r] = i < n && (n < k || kv[r] > kstar || (kv[r] == kstar && pv[r] <= pstar));
    }
    const int got = batch_slots(sh, f, slot, tid);
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      if (!f[r]) continue;
      const int o = done + slot[r];
      if (out.final_mode == 0) out.kept_out[(int64_t)b * k + o] = Cand{kv[r], pv[r]};
      else if (out.final_mode == 1) out.idx[(int64_t)b * out.idx_ld + o] = pv[r];
      else sort_area[o] = ((uint64_t)(~kv[r]) << 32) | (uint32_t)pv[r];
    }
    done += got;
  }
  if (out.final_mode == 0) {
    if (tid == 0) {
      out.kept_n_out[b] = take;
      out.thr_out[b] = n >= k ? kstar : 0u;
    }
    return;
  }
  if (out.final_mode == 2 && take > 1) {
    int n2 = 2;
    while (n2 < take) n2 <<= 1;
    __syncthreads();
    for (int i = take + tid; i < n2; i += kMergeThreads) sort_area[i] = ~0ull;
    __syncthreads();
    bitonic_sort(sort_area, n2, tid);
    for (int i = tid; i < take; i += kMergeThreads) out.idx[(int64_t)b * out.idx_ld + i] = (int32_t)(uint32_t)sort_area[i];
  } else if (out.final_mode == 2 && take == 1) {
    __syncthreads();
    if (tid == 0) out.idx[(int64_t)b * out.idx_ld] = (int32_t)(uint32_t)sort_area[0];
  }
  for (int i = take + tid; i < out.idx_ld; i += kMergeThreads) out.idx[(int64_t)b * out.idx_ld + i] = -1;
  if (tid == 0) out.n_sel[b] = take;
}

// Dynamic LDS: [keys: cap x 4 B][positions: cap x 4 B][bucket-rank sort area: sort_bytes].
__global__ __launch_bounds__(kMergeThreads) void k_merge(int k, MergeIn in, Cand* __restrict__ gather,
                                                         int64_t gather_cap, MergeOut out, int cap) {
  __shared__ MergeShared sh;
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) {
    sh.kmin = 0xFFFFFFFFu;
    sh.kmax = 0u;
  }
  const int nk = in.kept ? in.kept_n[b] : 0;
  int64_t n_in = in.slot_key ? in.n_slots : 0;
  if (in.cand && in.seg_cnt) {
    int s = 0;
    for (int w = tid; w < in.n_seg; w += kMergeThreads) s += (int)in.seg_cnt[(int64_t)b * in.n_seg + w];
    int total;
    block_scan(sh, s, tid, &total);
    n_in += total;
  }
  __syncthreads();
  uint64_t* sort_area = reinterpret_cast<uint64_t*>(dyn + (size_t)8 * cap);
  if (nk + n_in <= cap) {
    merge_body<true>(sh, b, k, in, out, reinterpret_cast<uint32_t*>(dyn), reinterpret_cast<int32_t*>(dyn + 4 * cap),
                     nk, sort_area);
  } else {
    Cand* g = gather + (int64_t)b * gather_cap;
    merge_body<false>(sh, b, k, in, out, reinterpret_cast<uint32_t*>(g), reinterpret_cast<int32_t*>(g) + gather_cap,
                      nk, sort_area);
  }
}

}  // namespace

hipError_t launch_merge(int B, int k, const MergeIn& in, Cand* gather, int64_t gather_cap, const MergeOut& out,
                        hipStream_t st) {
  if (k < 1 || k > kMaxSortK || (out.final_mode == 2 && k > kMaxSortK / 2)) return hipErrorInvalidValue;
  if (B == 0) return hipSuccess;
  int n2 = 2;
  while (n2 < k) n2 <<= 1;
  const int sort_bytes = out.final_mode == 2 ? 8 * n2 : 0;
  const int dyn = kLdsBytes - (int)sizeof(MergeShared) - 256;
  const int cap = (dyn - sort_bytes) / 8;
  // the dynamic LDS limit is raised once per device (host threads may race here: the call is idempotent)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
  if (bit == 0 || !(attr_set.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_merge), hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  SA_LAUNCH(k_merge, dim3((unsigned)B), dim3(kMergeThreads), (size_t)dyn, st, k, in, gather, gather_cap,
                     out, cap);
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
  SA_LAUNCH(k_fill_u32, dim3(blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace sa
