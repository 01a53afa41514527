// Exact top-k for few queries by a radix select spread over many workgroups (LongCat Sparse Attention deep-dive:
// DSA baseline section, arg-topK equation; SI section, the sparse part is the top-K over positions outside sink
// and window).
//
// Input: one order-preserving key per position, keys[b * keys_ld + s] for s < L, 0 for positions that are not
// candidates (the scoring kernel's all-slots mode writes them). Each query's positions are cut into G chunks and
// every (chunk, query) pair is one workgroup of every launch, so a handful of queries still fills the chip:
//   pass 0, 1, 2  histograms of digits 31..21, 20..10 and 9..0 of the keys that match the digits found so far,
//                 added into a global histogram per query and pass. Pass p >= 1 finds digit p - 1 in the
//                 histogram of pass p - 1 (a 2048-bin scan) and reads the digits before it from a per-query
//                 record that the first chunk's workgroup of each earlier launch extended;
//   count         the last digit, hence the k-th key kstar (recorded), then per chunk the keys above kstar and
//                 the keys equal to it;
//   write         per chunk (kstar from the record), an order-preserving compaction of the selected positions at
//                 the chunk's offset (the
//                 counts of the chunks before it). Among keys equal to kstar the lowest positions are kept: chunk j
//                 keeps the first min(eq_j, need_eq - ties in chunks before j) of its ties.
// The selected positions come out in ascending order, padded with -1 to idx_ld; n_sel = min(k, candidates).
#include "sa_device.h"
#include "sa_internal.h"
#include "sa_wave_select.h"

namespace sa {
namespace {

constexpr int kRThreads = 256;
constexpr int kRWaves = kRThreads / kWave;
constexpr int kRBins = 2048;
constexpr int kChunkAlign = 1024;  // chunk starts are multiples of this many positions (aligned vector loads)
constexpr int kTargetWgs = 1024;

__device__ __forceinline__ int pass_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ int pass_bins(int p) { return p == 2 ? 1024 : 2048; }

struct RadixShared {
  uint32_t hist[kRBins];
  uint32_t wsum[kRWaves];
  uint32_t wsum2[kRWaves];
  uint32_t digit, before, total;
};

// Exclusive scan over the block of one value per thread; *total receives the block sum. All threads must call.
__device__ __forceinline__ uint32_t block_excl_scan(RadixShared& sh, uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint32_t incl = wave_inclusive_scan(v, lane);
  if (lane == kWave - 1) sh.wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kRWaves; ++w) {
    const uint32_t x = sh.wsum[w];
    before += w < wave ? x : 0u;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Block-wide search of one query's global histogram h (nbins bins) in descending bin order: the bin in which the
// running count from the top first reaches need (>= 1). Returns false (digit 0) when all bins together hold
// fewer than need. *before = count in the bins above the digit; *total = sum of all bins. All threads must call.
__device__ bool find_desc(RadixShared& sh, const uint32_t* __restrict__ h, int nbins, uint32_t need, uint32_t* digit,
                          uint32_t* before, uint32_t* total) {
  const int tid = threadIdx.x;
  const int per = nbins / kRThreads;  // 8 or 4 bins per thread, thread t takes descending ranks per*t ..
  uint32_t c[8], local = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    c[e] = e < per ? h[nbins - 1 - (per * tid + e)] : 0u;
    local += c[e];
  }
  uint32_t all;
  const uint32_t excl = block_excl_scan(sh, local, &all);
  if (excl < need && excl + local >= need) {
    uint32_t run = excl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e < per && run < need && run + c[e] >= need) {
        sh.digit = (uint32_t)(nbins - 1 - (per * tid + e));
        sh.before = run;
      }
      run += c[e];
    }
  }
  __syncthreads();
  const bool ok = all >= need;
  *digit = ok ? sh.digit : 0u;
  *before = ok ? sh.before : 0u;
  *total = all;
  __syncthreads();
  return ok;
}

// The k-th key of query b from the three pass histograms: kstar, the number of keys to keep among those equal to
// it (need_eq >= 1), and the number of candidates. ok = false when there are fewer than k candidates (then every
// candidate is kept: kstar = 0, need_eq = 0).
struct KStar {
  bool ok;
  uint32_t kstar, need_eq, n_cand;
};

// Per-query record of the digits found so far, kRecWords words: written by the workgroup of chunk 0 of the launch
// that finds them, read by every workgroup of the later launches (a launch boundary orders the two).
constexpr int kRecWords = 8;
enum : int { kRecOk = 0, kRecNCand, kRecD0, kRecB0, kRecD1, kRecB1, kRecKStar, kRecNeedEq };

__device__ __forceinline__ void store_rec(uint32_t* rec, int i, uint32_t v) {
  if (blockIdx.x == 0 && threadIdx.x == 0) rec[i] = v;
}

// Chunk j of query b: positions [s0, s1).
struct Chunk {
  int64_t s0, s1;
};
__device__ __forceinline__ Chunk chunk_of(int64_t L, int64_t chunk) {
  Chunk c;
  c.s0 = (int64_t)blockIdx.x * chunk;
  c.s1 = c.s0 + chunk < L ? c.s0 + chunk : L;
  return c;
}

// Key scans. A chunk is read in batches of 4 * kRThreads keys, four per thread (s a multiple of 4; the row is
// padded to a multiple of 4 so the vector load stays inside it). Loads are never predicated: an address past the
// chunk's end is clamped to the chunk's start and the value masked to 0 afterwards, so that all loads of a round
// are in flight together (a load under a branch makes the compiler wait for it at the branch's end). The first
// kPre batches are issued at kernel entry, before the record and histogram reads that precede the scan; later
// batches go kRound per round trip. A chunk of at most kPre batches (the usual size) needs no second round.
constexpr int kBatch = 4 * kRThreads;
constexpr int kPre = 2;
constexpr int kRound = 8;

__device__ __forceinline__ uint4 load_batch(const uint32_t* __restrict__ row, const Chunk& c, int64_t bs) {
  const int64_t s = bs + 4 * (int64_t)threadIdx.x;
  return *reinterpret_cast<const uint4*>(row + (s < c.s1 ? s : c.s0));
}
__device__ __forceinline__ void unpack(const uint4& x, const Chunk& c, int64_t bs, uint32_t (&v)[4]) {
  const int64_t s = bs + 4 * (int64_t)threadIdx.x;
  v[0] = s + 0 < c.s1 ? x.x : 0u;
  v[1] = s + 1 < c.s1 ? x.y : 0u;
  v[2] = s + 2 < c.s1 ? x.z : 0u;
  v[3] = s + 3 < c.s1 ? x.w : 0u;
}
struct PreKeys {
  uint4 x[kPre];
};
__device__ __forceinline__ PreKeys preload(const uint32_t* __restrict__ row, const Chunk& c) {
  PreKeys p;
#pragma unroll
  for (int h = 0; h < kPre; ++h) p.x[h] = load_batch(row, c, c.s0 + (int64_t)h * kBatch);
  return p;
}
// f(bs, v) for every batch of the chunk in order (block-uniform calls: f may hold barriers).
template <typename F>
__device__ __forceinline__ void scan_chunk(const uint32_t* __restrict__ row, const Chunk& c, const PreKeys& p,
                                           F&& f) {
#pragma unroll
  for (int h = 0; h < kPre; ++h) {
    const int64_t bs = c.s0 + (int64_t)h * kBatch;
    if (bs < c.s1) {
      uint32_t v[4];
      unpack(p.x[h], c, bs, v);
      f(bs, v);
    }
  }
  for (int64_t base = c.s0 + (int64_t)kPre * kBatch; base < c.s1; base += (int64_t)kRound * kBatch) {
    uint4 x[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) x[u] = load_batch(row, c, base + (int64_t)u * kBatch);
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int64_t bs = base + (int64_t)u * kBatch;
      if (bs < c.s1) {
        uint32_t v[4];
        unpack(x[u], c, bs, v);
        f(bs, v);
      }
    }
  }
}

template <int PASS>
__global__ __launch_bounds__(kRThreads) void k_radix_hist(const uint32_t* __restrict__ keys, int64_t keys_ld,
                                                          int64_t L, int64_t chunk, int k, int B,
                                                          uint32_t* __restrict__ hist, uint32_t* __restrict__ recs) {
  __shared__ RadixShared sh;
  const int b = blockIdx.y, tid = threadIdx.x;
  constexpr int nb = PASS == 2 ? 1024 : 2048;
  constexpr int shift = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  uint32_t* rec = recs + (size_t)b * kRecWords;
  const Chunk c = chunk_of(L, chunk);
  const uint32_t* row = keys + (int64_t)b * keys_ld;
  const PreKeys pre = preload(row, c);
  for (int i = tid; i < kRBins; i += kRThreads) sh.hist[i] = 0u;
  uint32_t prefix = 0u, pmask = 0u;
  if (PASS == 1) {
    uint32_t d0, b0, tot;
    const bool ok = find_desc(sh, hist + (size_t)b * kRBins, 2048, (uint32_t)k, &d0, &b0, &tot);
    store_rec(rec, kRecOk, ok ? 1u : 0u);
    store_rec(rec, kRecNCand, tot);
    store_rec(rec, kRecD0, d0);
    store_rec(rec, kRecB0, b0);
    if (!ok) return;  // block-uniform: fewer than k candidates, every one is kept
    prefix = d0 << 21;
    pmask = 0x7FFu << 21;
  } else if (PASS == 2) {
    if (rec[kRecOk] == 0u) return;
    const uint32_t d0 = rec[kRecD0], b0 = rec[kRecB0];
    uint32_t d1, b1, t1;
    find_desc(sh, hist + ((size_t)B + b) * kRBins, 2048, (uint32_t)k - b0, &d1, &b1, &t1);
    store_rec(rec, kRecD1, d1);
    store_rec(rec, kRecB1, b1);
    prefix = (d0 << 21) | (d1 << 10);
    pmask = (0x7FFu << 21) | (0x7FFu << 10);
  }
  __syncthreads();
  scan_chunk(row, c, pre, [&](int64_t, const uint32_t (&v)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (v[e] != 0u && (v[e] & pmask) == prefix) atomicAdd(&sh.hist[(v[e] >> shift) & (nb - 1)], 1u);
  });
  __syncthreads();
  uint32_t* g = hist + ((size_t)PASS * B + b) * kRBins;
  for (int i = tid; i < nb; i += kRThreads) {
    const uint32_t x = sh.hist[i];
    if (x) atomicAdd(&g[i], x);
  }
}

__global__ __launch_bounds__(kRThreads) void k_radix_count(const uint32_t* __restrict__ keys, int64_t keys_ld,
                                                           int64_t L, int64_t chunk, int k, int B,
                                                           const uint32_t* __restrict__ hist,
                                                           uint32_t* __restrict__ recs, uint32_t* __restrict__ cnt) {
  __shared__ RadixShared sh;
  const int b = blockIdx.y, tid = threadIdx.x;
  uint32_t* rec = recs + (size_t)b * kRecWords;
  const Chunk c = chunk_of(L, chunk);
  const uint32_t* row = keys + (int64_t)b * keys_ld;
  const PreKeys pre = preload(row, c);
  KStar ks{rec[kRecOk] != 0u, 0u, 0u, rec[kRecNCand]};
  if (ks.ok) {
    const uint32_t need = (uint32_t)k - rec[kRecB0] - rec[kRecB1];
    uint32_t d2, b2, t2;
    find_desc(sh, hist + ((size_t)2 * B + b) * kRBins, 1024, need, &d2, &b2, &t2);
    ks.kstar = (rec[kRecD0] << 21) | (rec[kRecD1] << 10) | d2;
    ks.need_eq = need - b2;
  }
  store_rec(rec, kRecKStar, ks.kstar);
  store_rec(rec, kRecNeedEq, ks.need_eq);
  uint32_t gt = 0, eq = 0;
  scan_chunk(row, c, pre, [&](int64_t, const uint32_t (&v)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gt += v[e] > ks.kstar ? 1u : 0u;
      eq += (ks.ok && v[e] == ks.kstar) ? 1u : 0u;
    }
  });
  uint32_t tg, te;
  block_excl_scan(sh, gt, &tg);
  block_excl_scan(sh, eq, &te);
  if (tid == 0) {
    cnt[((int64_t)b * gridDim.x + blockIdx.x) * 2 + 0] = tg;
    cnt[((int64_t)b * gridDim.x + blockIdx.x) * 2 + 1] = te;
  }
}

__global__ __launch_bounds__(kRThreads) void k_radix_write(const uint32_t* __restrict__ keys, int64_t keys_ld,
                                                           int64_t L, int64_t chunk, int k, int B,
                                                           const uint32_t* __restrict__ recs,
                                                           const uint32_t* __restrict__ cnt,
                                                           int32_t* __restrict__ idx, int idx_ld,
                                                           int32_t* __restrict__ n_sel, Cand* __restrict__ kept,
                                                           uint32_t* __restrict__ thr_out) {
  __shared__ RadixShared sh;
  const int b = blockIdx.y, j = blockIdx.x, tid = threadIdx.x;
  const int G = gridDim.x;
  const uint32_t* rec = recs + (size_t)b * kRecWords;
  const Chunk c = chunk_of(L, chunk);
  const uint32_t* row = keys + (int64_t)b * keys_ld;
  const PreKeys pre = preload(row, c);
  const KStar ks{rec[kRecOk] != 0u, rec[kRecKStar], rec[kRecNeedEq], rec[kRecNCand]};
  // counts of the chunks before this one
  const uint32_t* cb = cnt + (int64_t)b * G * 2;
  uint32_t pg = 0, pe = 0;
  for (int i = tid; i < j; i += kRThreads) {
    pg += cb[2 * i];
    pe += cb[2 * i + 1];
  }
  uint32_t pre_gt, pre_eq;
  block_excl_scan(sh, pg, &pre_gt);
  block_excl_scan(sh, pe, &pre_eq);
  const uint32_t my_eq = cb[2 * j + 1];
  const uint32_t ties_before = pre_eq < ks.need_eq ? pre_eq : ks.need_eq;
  const uint32_t quota = ks.need_eq > pre_eq ? (my_eq < ks.need_eq - pre_eq ? my_eq : ks.need_eq - pre_eq) : 0u;
  const int64_t off = (int64_t)pre_gt + ties_before;
  // rank r of the selection: position into idx, (key, position) into kept, whichever is given
  int32_t* out = idx ? idx + (int64_t)b * idx_ld : nullptr;
  Cand* kp = kept ? kept + (int64_t)b * k : nullptr;
  auto put = [&](int64_t r, uint32_t key, int64_t pos) {
    if (out) out[r] = (int32_t)pos;
    if (kp) kp[r] = Cand{key, (int32_t)pos};
  };

  uint32_t run_gt = 0, run_eq = 0;  // entries of this chunk before the current batch
  scan_chunk(row, c, pre, [&](int64_t base, const uint32_t (&v)[4]) {
    const int64_t s = base + 4 * tid;
    bool g[4], t[4];
    uint32_t lg = 0, lt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g[e] = v[e] > ks.kstar;
      t[e] = ks.ok && v[e] == ks.kstar;
      lg += g[e] ? 1u : 0u;
      lt += t[e] ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan(sh, (lg << 16) | lt, &tot);  // at most 1024 of each per batch
    uint32_t gb = run_gt + (ex >> 16), eb = run_eq + (ex & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (g[e]) {
        put(off + gb + (eb < quota ? eb : quota), v[e], s + e);
        ++gb;
      } else if (t[e]) {
        if (eb < quota) put(off + gb + eb, v[e], s + e);
        ++eb;
      }
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xFFFFu;
  });
  if (j == 0) {
    const int take = ks.ok ? k : (int)ks.n_cand;
    if (out)
      for (int i = take + tid; i < idx_ld; i += kRThreads) out[i] = -1;
    if (tid == 0) {
      n_sel[b] = take;
      if (thr_out) thr_out[b] = ks.ok ? ks.kstar : 0u;  // later keys must beat the k-th key to enter
    }
  }
}

// Keys of caller-given fp32 scores: grid (key blocks, queries); also zeroes the select's control words.
__global__ __launch_bounds__(256) void k_keys_from_scores(const float* __restrict__ scores, int64_t scores_ld,
                                                          int64_t L, const int32_t* __restrict__ t, int n_sink,
                                                          int n_window, int64_t keys_ld, uint32_t* __restrict__ keys,
                                                          uint32_t* __restrict__ ctl, int64_t ctl_words,
                                                          int64_t t_default, int t_div) {
  const int b = blockIdx.y;
  const int64_t nthr = (int64_t)gridDim.x * gridDim.y * blockDim.x;
  for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; i < ctl_words; i += nthr)
    ctl[i] = 0u;
  const int64_t tb = (t ? (int64_t)t[b] : t_default) / t_div;
  const float* row = scores + (int64_t)b * scores_ld;
  uint32_t* out = keys + (int64_t)b * keys_ld;
  for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < keys_ld; s += (int64_t)gridDim.x * blockDim.x) {
    const bool cand = s < L && s >= n_sink && s <= tb - n_window;
    out[s] = cand ? score_key(row[s]) : 0u;
  }
}

}  // namespace

hipError_t launch_keys_from_scores(const float* scores, int64_t scores_ld, int64_t L, int B, const int32_t* t,
                                   int n_sink, int n_window, const RadixPlan& p, uint32_t* keys, uint32_t* ctl,
                                   int64_t ctl_words, hipStream_t st, int64_t t_default, int t_div) {
  if (B == 0) return hipSuccess;
  int64_t blocks = (p.keys_ld + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  SA_LAUNCH(k_keys_from_scores, dim3((unsigned)blocks, (unsigned)B), dim3(256), 0, st, scores, scores_ld, L, t,
            n_sink, n_window, p.keys_ld, keys, ctl, ctl_words, t_default < 0 ? L - 1 : t_default,
            t_div < 1 ? 1 : t_div);
  return hipGetLastError();
}

RadixPlan radix_plan(int B, int64_t L) {
  RadixPlan p{};
  p.keys_ld = (L + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  int64_t g = B > 0 ? (kTargetWgs + B - 1) / B : 1;
  int64_t chunk = (L + g - 1) / g;
  if (chunk < 2 * kChunkAlign) chunk = 2 * kChunkAlign;
  chunk = (chunk + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  p.chunk = chunk;
  p.n_chunks = (int)((L + chunk - 1) / chunk);
  if (p.n_chunks < 1) p.n_chunks = 1;
  return p;
}

// ctl layout: pass histograms [3, B, 2048] words, per-chunk counts [B, n_chunks, 2] words, then the per-query
// digit records [B, kRecWords] words.
size_t radix_ctl_words(int B, const RadixPlan& p) {
  return (size_t)3 * B * kRBins + (size_t)2 * B * p.n_chunks + (size_t)kRecWords * B;
}

hipError_t launch_radix_select(int B, int64_t L, int k, const RadixPlan& p, const uint32_t* keys, uint32_t* ctl,
                               int32_t* idx, int idx_ld, int32_t* n_sel, Cand* kept, uint32_t* thr_out,
                               hipStream_t st) {
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_chunks, (unsigned)B);
  uint32_t* hist = ctl;
  uint32_t* cnt = ctl + (size_t)3 * B * kRBins;
  uint32_t* recs = cnt + (size_t)2 * B * p.n_chunks;
  SA_LAUNCH(k_radix_hist<0>, grid, dim3(kRThreads), 0, st, keys, p.keys_ld, L, p.chunk, k, B, hist, recs);
  SA_LAUNCH(k_radix_hist<1>, grid, dim3(kRThreads), 0, st, keys, p.keys_ld, L, p.chunk, k, B, hist, recs);
  SA_LAUNCH(k_radix_hist<2>, grid, dim3(kRThreads), 0, st, keys, p.keys_ld, L, p.chunk, k, B, hist, recs);
  SA_LAUNCH(k_radix_count, grid, dim3(kRThreads), 0, st, keys, p.keys_ld, L, p.chunk, k, B, hist, recs,
                     cnt);
  SA_LAUNCH(k_radix_write, grid, dim3(kRThreads), 0, st, keys, p.keys_ld, L, p.chunk, k, B, recs, cnt, idx,
                     idx_ld, n_sel, kept, thr_out);
  return hipGetLastError();
}

}  // namespace sa
