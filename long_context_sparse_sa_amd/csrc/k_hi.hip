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

#include <type_traits>

namespace sa {
namespace {

using namespace tile;

// f(integral_constant<J>) for J = I .. N-1, unrolled.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFineRing = 3;  // key tiles per wave held in registers: kFineRing - 1 in flight while one is scored

// A 64-position key tile as 16 coalesced 1 KB loads: load j brings positions 4 j .. 4 j + 3 (this lane: position
// 4 j + lane / 16, 16-byte chunk lane % 16). The tile's base is uniform (scalar), the lane's part a constant 32-bit
// offset, so a load costs no vector address arithmetic. A tile that runs past L - 1 clamps its rows (never scored).
__device__ __forceinline__ void load_tile_regs(const char* kbytes, int64_t ld_bytes, int64_t L, int64_t s0, int lane,
                                               uint32_t lane_off, u32x4 (&r)[16]) {
  const char* base = kbytes + s0 * ld_bytes;
  if (s0 + kTileKeys <= L) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      r[j] = *reinterpret_cast<const u32x4*>(base + (uint32_t)(4 * j * ld_bytes) + lane_off);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      int64_t row = s0 + 4 * j + (lane >> 4);
      row = row < L ? row : L - 1;
      r[j] = *reinterpret_cast<const u32x4*>(kbytes + row * ld_bytes + 16 * (lane & 15));
    }
  }
}

// ... and into the LDS tile layout the scorer reads (chunk c of position n at chunk c ^ (n % 16)).
__device__ __forceinline__ void store_tile_lds(char* tile, int lane, const u32x4 (&r)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) *reinterpret_cast<u32x4*>(tile + tile_off(4 * j + (lane >> 4), lane & 15)) = r[j];
}

// Token stage. Workgroup = one wave = (query b, part p): the part is a range of page ids, [p G, (p + 1) G) (one
// part per query unless there are too few queries to fill the chip), and the wave walks the query's recalled pages
// inside it in ascending order. The recalled pages of different queries rarely coincide, so a key tile is scored
// for one query only: many key bytes must be in flight per compute unit, and they must arrive in whole cache
// lines. Each wave therefore loads its tiles with coalesced 1 KB loads into a register ring (kFineRing - 1 tiles in
// flight, one wave on every SIMD), and copies the current tile through a private 16 KB LDS tile into the MFMA
// fragment layout, where the same scorer as the flat paths reads it (bit-identical scores). Candidates above the
// wave's running threshold go to its segment, compacted to the exact top-k when full and once more at the end.
// Positions arrive in ascending order, so a segment stays in position order and a later candidate that only ties
// the k-th key never displaces it; the segments of a query ascend with p.
template <int NMT>
__global__ __launch_bounds__(64) void k_hi_fine(const void* __restrict__ q, const float* __restrict__ w,
                                                const void* __restrict__ k, int64_t k_ld, int64_t L,
                                                const int32_t* __restrict__ t, const int32_t* __restrict__ pages,
                                                int pages_ld, const int32_t* __restrict__ n_pages, int page_len,
                                                int part_pages, int kk, int n_sink, int n_window,
                                                Cand* __restrict__ seg, int64_t seg_cap,
                                                uint32_t* __restrict__ seg_cnt) {
  __shared__ __attribute__((aligned(1024))) char tile[kTileBytes];
  __shared__ uint32_t hist[256];
  const int lane = lane_id();
  const int b = blockIdx.x;
  const int part = blockIdx.y;
  const int n_parts = gridDim.y;
  const int64_t tb = t ? (int64_t)t[b] : L - 1;
  const int64_t cand_end = tb - n_window;  // last candidate position
  uint32_t* cnt_out = seg_cnt + (int64_t)b * n_parts + part;
  // this query's recalled pages inside [first_page, last_page]: a binary search of the ascending list
  const int64_t first_page = (int64_t)part * part_pages;
  int64_t last_page = first_page + part_pages - 1;
  if (cand_end < 0 || first_page * page_len > cand_end) {
    if (lane == 0) *cnt_out = 0u;
    return;
  }
  if (last_page * page_len > cand_end) last_page = cand_end / page_len;
  const int32_t* own = pages + (int64_t)b * pages_ld;
  int n_own = n_pages[b];
  n_own = n_own < 0 ? 0 : n_own;
  auto lower_bound = [&](int64_t v) {
    int lo = 0, hi = n_own;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)own[mid] < v) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  const int i0 = lower_bound(first_page);
  const int i1 = lower_bound(last_page + 1);
  if (i1 <= i0) {
    if (lane == 0) *cnt_out = 0u;
    return;
  }
  QueryFrags<NMT> qf;
  qf.template load<false>(q, w, b, lane);
  const int tiles_per_page = page_len / kTileKeys;
  const int n_tiles = (i1 - i0) * tiles_per_page;
  const char* kbytes = reinterpret_cast<const char*>(k);
  const int64_t ld_bytes = k_ld * 2;
  const uint32_t lane_off = (uint32_t)((lane >> 4) * ld_bytes + 16 * (lane & 15));
  Cand* mybuf = seg + ((int64_t)b * n_parts + part) * seg_cap;
  const int cap = (int)seg_cap;
  int n = 0;
  uint32_t thr = 0;
  // Load-ahead cursor over (recalled page, tile in page), advanced once per tile; past the last tile it keeps
  // returning the last one. Every step issues its loads, past the end too: with the same number of loads on every
  // path, the compiler's wait before a tile's first use counts exactly the newer tiles' loads and leaves them in
  // flight (a conditional load makes it wait for all of them).
  int la_page = i0, la_tile = 0;
  int64_t la_base = (int64_t)own[i0] * page_len;
  auto next_start = [&]() __attribute__((always_inline)) {
    const int64_t s0 = la_base + (int64_t)la_tile * kTileKeys;
    if (++la_tile == tiles_per_page) {
      if (la_page + 1 < i1) {
        la_tile = 0;
        ++la_page;
        la_base = (int64_t)own[la_page] * page_len;
      } else {
        la_tile = tiles_per_page - 1;  // stay on the last tile
      }
    }
    return s0;
  };
  u32x4 ring[kFineRing][16];
  int64_t ring_s0[kFineRing];
  static_for<0, kFineRing - 1>([&](auto R) __attribute__((always_inline)) {
    constexpr int r = decltype(R)::value;
    ring_s0[r] = next_start();
    load_tile_regs(kbytes, ld_bytes, L, ring_s0[r], lane, lane_off, ring[r]);
  });
  // tile i sits in ring slot i % kFineRing; slots are compile-time (the loop is unrolled by the ring size)
  auto step = [&](auto S) __attribute__((always_inline)) {
    constexpr int sl = decltype(S)::value;
    constexpr int ahead = (sl + kFineRing - 1) % kFineRing;
    ring_s0[ahead] = next_start();
    load_tile_regs(kbytes, ld_bytes, L, ring_s0[ahead], lane, lane_off, ring[ahead]);
    const int64_t s0 = ring_s0[sl];
    if (s0 > cand_end) return;
    // the previous tile's fragment reads are complete (their MFMAs consumed them); LDS operations of one wave
    // complete in order, and the wait makes the copy visible to the fragment reads in any case
    store_tile_lds(tile, lane, ring[sl]);
    wait_lds();
    const float score = qf.score(tile, lane);
    const int64_t s = s0 + lane;
    const bool cand = s < L && s >= n_sink && s <= cand_end;
    const uint32_t key = score_key(score);
    if (n + kWave > cap) {
      wait_vmem();  // the segment's stores have landed before the compaction reads them back
      thr = wave_select_compact(mybuf, n, kk, hist, lane);
      n = n < kk ? n : kk;
    }
    const bool emit = cand && key > thr;
    const uint64_t mk = ballot(emit);
    if (emit) mybuf[n + lanes_below(mk)] = Cand{key, (int32_t)s};
    n += __popcll(mk);
  };
  // whole groups of kFineRing tiles, then the remainder: a loop body without skipped steps gives every path to
  // the loop header the same loads in flight
  int i = 0;
  for (; i + kFineRing <= n_tiles; i += kFineRing)
    static_for<0, kFineRing>([&](auto J) __attribute__((always_inline)) { step(J); });
  static_for<0, kFineRing - 1>([&](auto J) __attribute__((always_inline)) {
    if (i + decltype(J)::value < n_tiles) step(J);
  });
  wait_vmem();  // the loads past the end land before the wave exits
  if (n > kk) {
    wait_vmem();
    wave_select_compact(mybuf, n, kk, hist, lane);
    n = kk;
  }
  if (lane == 0) *cnt_out = (uint32_t)n;
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

HiFinePlan hi_fine_plan(int64_t L, int B, int page_len, int k) {
  HiFinePlan p{};
  const int64_t n_cache_pages = (L + page_len - 1) / page_len;
  // one part per query, or enough parts to give every compute unit several waves when there are few queries
  int64_t parts = B > 0 ? (kHiTargetWaves + B - 1) / B : 1;
  if (parts > n_cache_pages) parts = n_cache_pages;
  if (parts > 65535) parts = 65535;  // the grid's y extent
  if (parts < 1) parts = 1;
  p.part_pages = (int)((n_cache_pages + parts - 1) / parts);
  p.n_parts = (int)((n_cache_pages + p.part_pages - 1) / p.part_pages);
  // a segment holds the part's candidates up to a compaction; never more than the part's positions (plus a tile)
  int64_t cap = 2 * (int64_t)k + kWave;
  const int64_t most = (int64_t)p.part_pages * page_len + kWave;
  if (cap > most) cap = most;
  if (cap < k + kWave) cap = k + kWave;
  p.seg_cap = (cap + kWave - 1) / kWave * kWave;
  return p;
}

hipError_t launch_hi_fine(const IndexerArgs& a, const int32_t* pages, int pages_ld, const int32_t* n_pages,
                          int page_len, int k, int n_sink, int n_window, const HiFinePlan& p, Cand* seg,
                          uint32_t* seg_cnt, hipStream_t st) {
  if (!hi_fine_supported(a) || page_len % kTileKeys != 0 || p.seg_cap < k + kWave || p.n_parts < 1)
    return hipErrorInvalidValue;
  if (a.B < 1) return hipSuccess;
  const dim3 grid((unsigned)a.B, (unsigned)p.n_parts);
  if (a.H == 64)
    SA_LAUNCH(k_hi_fine<2>, grid, dim3(64), 0, st, a.q, a.w, a.k, a.k_ld, a.L, a.t, pages, pages_ld, n_pages,
              page_len, p.part_pages, k, n_sink, n_window, seg, p.seg_cap, seg_cnt);
  else
    SA_LAUNCH(k_hi_fine<1>, grid, dim3(64), 0, st, a.q, a.w, a.k, a.k_ld, a.L, a.t, pages, pages_ld, n_pages,
              page_len, p.part_pages, k, n_sink, n_window, seg, p.seg_cap, seg_cnt);
  return hipGetLastError();
}

}  // namespace sa
