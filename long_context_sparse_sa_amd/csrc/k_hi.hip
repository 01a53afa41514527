// Hierarchical (coarse-to-fine) indexing (LongCat Sparse Attention deep-dive, section "Mechanism 3: hierarchical
// indexing (HI)"): the cache is cut into pages of P positions and each page into sub-blocks of B positions; each
// sub-block keeps the mean of its index keys (computed once per cache); a page's score is the indexer equation
// summed over its sub-blocks' mean keys; the best M pages are recalled and the token-level top-k runs only over
// their positions.
//
// Kernels here: the mean keys (k_hi_means) and the token stage (k_hi_fine). The page scores are the MFMA
// scorer's page mode (k_index.hip); the top-M pages are the radix select over them (k_radix.hip).
#include "sa_device.h"
#include "sa_internal.h"
#include "sa_score_tile.h"
#include "sa_wave_select.h"

namespace sa {
namespace {

using namespace tile;

// One thread per (sub-block, dimension): the fp64 sum of the block's cached keys (exact for bf16 inputs of
// moderate spread), divided by their count in fp64, rounded to fp32 and then to bf16 (nearest even both times).
__global__ __launch_bounds__(256) void k_hi_means(const uint16_t* __restrict__ k, int64_t k_ld, int64_t L, int d,
                                                  int sub, uint16_t* __restrict__ means, int64_t n_sub) {
  const int64_t n_all = n_sub * d;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_all; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i / d;
    const int x = (int)(i % d);
    const int64_t s0 = n * sub;
    const int cnt = (int)(L - s0 < sub ? L - s0 : sub);
    double acc = 0.0;
    for (int j = 0; j < cnt; ++j) acc += (double)bf16_bits_to_f32(k[(s0 + j) * k_ld + x]);
    means[i] = f32_to_bf16_bits((float)(acc / (double)cnt));
  }
}

constexpr int kFineQ = 4;                              // queries per workgroup
constexpr int kBitmapWords = (int)(kHiMaxCachePages / 32);

// Token stage. Workgroup = four waves = four queries. The union of their recalled pages is formed in LDS (a bitmap
// over the cache's pages, then its set bits in ascending order); the workgroup walks the union's 64-position tiles
// (bf16 keys by DMA, as the flat scorers do), and each wave scores only the tiles of its own pages (a cursor into
// its ascending page list), keeping candidates above its running threshold in its buffer and compacting the buffer
// to the exact top-k when it is full. Positions arrive in ascending order, so the buffer stays in position order.
template <int NMT>
__global__ __launch_bounds__(64 * kFineQ) void k_hi_fine(const void* __restrict__ q, const float* __restrict__ w,
                                                         const void* __restrict__ k, int64_t k_ld, int64_t L, int B,
                                                         const int32_t* __restrict__ t,
                                                         const int32_t* __restrict__ pages, int pages_ld,
                                                         const int32_t* __restrict__ n_pages, int page_len,
                                                         int64_t n_cache_pages, int kk, int n_sink, int n_window,
                                                         Cand* __restrict__ buf, int32_t* __restrict__ buf_n,
                                                         int cap) {
  constexpr int kNBuf = 4;
  __shared__ __attribute__((aligned(1024))) char tiles[kNBuf][kTileBytes];
  __shared__ uint32_t bitmap[kBitmapWords];
  __shared__ int32_t own[kFineQ][kHiMaxPages];
  __shared__ int32_t uni[kFineQ * kHiMaxPages];
  __shared__ uint32_t hist[kFineQ][256];
  __shared__ int32_t wsum[kFineQ];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int tid = threadIdx.x;
  const int b = blockIdx.x * kFineQ + wave;
  const bool active = b < B;
  const int n_words = (int)((n_cache_pages + 31) / 32);

  // the queries and weights, then the page lists and their union
  bf16x8 qa[NMT][kSteps];
  float wv[NMT][16];
  int64_t tb = -1;
  int n_own = 0;
  if (active) {
    tb = t ? (int64_t)t[b] : L - 1;
    load_query<NMT, false>(q, w, b, lane, qa, wv);
    wait_vmem();  // known complete before the tile loop (whose waits would otherwise drain the tile copies)
    n_own = n_pages[b];
    n_own = n_own < 0 ? 0 : (n_own > kHiMaxPages ? kHiMaxPages : n_own);
  }
  for (int i = tid; i < n_words; i += blockDim.x) bitmap[i] = 0u;
  __syncthreads();
  for (int i = lane; i < n_own; i += kWave) {
    const int32_t p = pages[(int64_t)b * pages_ld + i];
    own[wave][i] = p;
    atomicOr(&bitmap[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  // set bits in ascending order: each thread owns a contiguous run of bitmap words
  const int per = (n_words + (int)blockDim.x - 1) / (int)blockDim.x;
  const int w0 = tid * per;
  int cnt = 0;
  for (int i = 0; i < per; ++i)
    if (w0 + i < n_words) cnt += __popc(bitmap[w0 + i]);
  const int incl = (int)wave_inclusive_scan((uint32_t)cnt, lane);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = incl - cnt, n_union = 0;
#pragma unroll
  for (int v = 0; v < kFineQ; ++v) {
    before += v < wave ? wsum[v] : 0;
    n_union += wsum[v];
  }
  for (int i = 0; i < per; ++i) {
    if (w0 + i >= n_words) break;
    uint32_t m = bitmap[w0 + i];
    while (m) {
      const int bit = __builtin_ctz(m);
      m &= m - 1u;
      uni[before++] = (w0 + i) * 32 + bit;
    }
  }
  __syncthreads();

  const int tiles_per_page = page_len / kTileKeys;
  const int64_t n_tiles = (int64_t)n_union * tiles_per_page;
  auto tile_start = [&](int64_t i) {
    return (int64_t)uni[i / tiles_per_page] * page_len + (i % tiles_per_page) * kTileKeys;
  };
  const char* kbytes = reinterpret_cast<const char*>(k);
  const int64_t ld_bytes = k_ld * 2;
  Cand* mybuf = buf + (int64_t)(active ? b : 0) * cap;
  int n = 0, cur = 0;
  uint32_t thr = 0;
  const int64_t cand_end = tb - n_window;  // last candidate position
  walk_tiles<false, kFineQ, kNBuf>(kbytes, ld_bytes, L, n_tiles, tile_start, tiles, wave, lane,
                                   [&](const char* tile, int64_t i) {
                                     if (!active) return;
                                     const int32_t page = uni[i / tiles_per_page];
                                     while (cur < n_own && own[wave][cur] < page) ++cur;
                                     if (cur >= n_own || own[wave][cur] != page) return;  // not this query's page
                                     const int64_t s0 = tile_start(i);
                                     if (s0 > cand_end) return;
                                     const float score = score_tile<NMT>(tile, lane, qa, wv);
                                     const int64_t s = s0 + lane;
                                     const bool cand = s < L && s >= n_sink && s <= cand_end;
                                     const uint32_t key = score_key(score);
                                     if (n + kWave > cap) {
                                       wait_vmem();
                                       thr = wave_select_compact(mybuf, n, kk, hist[wave], lane);
                                       n = n < kk ? n : kk;
                                     }
                                     const bool emit = cand && key > thr;
                                     const uint64_t mk = ballot(emit);
                                     if (emit) mybuf[n + lanes_below(mk)] = Cand{key, (int32_t)s};
                                     n += __popcll(mk);
                                   });
  if (active && lane == 0) buf_n[b] = n;
}

}  // namespace

hipError_t launch_hi_means(const uint16_t* k, int64_t k_ld, int64_t L, int d, int sub, uint16_t* means,
                           hipStream_t st) {
  if (L < 1 || d < 1 || sub < 1) return hipSuccess;
  const int64_t n_sub = (L + sub - 1) / sub;
  int64_t blocks = (n_sub * d + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  SA_LAUNCH(k_hi_means, dim3((unsigned)blocks), dim3(256), 0, st, k, k_ld, L, d, sub, means, n_sub);
  return hipGetLastError();
}

bool hi_fine_supported(const IndexerArgs& a) {
  return a.d == 128 && (a.H == 32 || a.H == 64) && a.q_dtype == 1 && a.k_dtype == 1;
}

hipError_t launch_hi_fine(const IndexerArgs& a, const int32_t* pages, int pages_ld, const int32_t* n_pages,
                          int page_len, int64_t n_cache_pages, int k, int n_sink, int n_window, Cand* buf,
                          int32_t* buf_n, int cap, hipStream_t st) {
  if (!hi_fine_supported(a) || page_len % kTileKeys != 0 || n_cache_pages > kHiMaxCachePages || cap < k + kWave)
    return hipErrorInvalidValue;
  if (a.B < 1) return hipSuccess;
  const dim3 grid((unsigned)((a.B + kFineQ - 1) / kFineQ));
  if (a.H == 64)
    SA_LAUNCH(k_hi_fine<2>, grid, dim3(64 * kFineQ), 0, st, a.q, a.w, a.k, a.k_ld, a.L, a.B, a.t, pages, pages_ld,
              n_pages, page_len, n_cache_pages, k, n_sink, n_window, buf, buf_n, cap);
  else
    SA_LAUNCH(k_hi_fine<1>, grid, dim3(64 * kFineQ), 0, st, a.q, a.w, a.k, a.k_ld, a.L, a.B, a.t, pages, pages_ld,
              n_pages, page_len, n_cache_pages, k, n_sink, n_window, buf, buf_n, cap);
  return hipGetLastError();
}

}  // namespace sa
