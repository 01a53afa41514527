// Lightning-indexer scoring for gfx950 (LongCat Sparse Attention deep-dive, DSA baseline section, indexer
// equation): I(b, s) = sum_j w[b, j] * ReLU(q[b, j, :] . k[s, :]), one key row shared by all heads, no scale.
//
// Two kernels:
//  * k_score_valu  -- any head count, width and dtype; one thread per position, fp32 accumulation.
//  * k_score_mfma  -- d = 128 and H in {32, 64}: the (query-head x position) dot products are a dense contraction
//    and run on the bf16 32x32x16 MFMA, one wave per query so that the ReLU-weighted head sum stays inside the
//    wave. Key tiles of 64 positions are staged in LDS (bf16 rows by asynchronous DMA; e4m3 rows converted exactly
//    to bf16 on the way in) and shared by the workgroup's waves (four or eight queries: eight when B >= 8).
// Both kernels either write the dense score row or emit only candidates whose score beats the caller's running
// threshold, so a decode step never writes the [B, L] score matrix.
#include <atomic>
#include <type_traits>

#include "sa_device.h"
#include "sa_internal.h"
#include "sa_score_tile.h"
#include "sa_wave_select.h"

namespace sa {
namespace {

using namespace tile;

constexpr int kValuKeysPerWg = 256;
constexpr int kMfmaKeysPerWg = 512;

// Zeroes clear[0, n) with every thread of the grid (a no-op for n = 0).
__device__ __forceinline__ void clear_region(uint32_t* clear, int64_t n) {
  if (n <= 0) return;
  const int64_t nthr = (int64_t)gridDim.x * gridDim.y * blockDim.x;
  for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += nthr)
    clear[i] = 0u;
}

__device__ __forceinline__ bool is_candidate(int64_t s, int64_t t, int n_sink, int n_window) {
  return s >= n_sink && s <= t - n_window;
}

template <int QT, int KT>
__global__ __launch_bounds__(256) void k_score_valu(const void* __restrict__ q, const float* __restrict__ w,
                                                    const void* __restrict__ k, int64_t k_ld, int64_t L, int H,
                                                    int d, const int32_t* __restrict__ t, int64_t lo, int64_t hi,
                                                    int mode, float* __restrict__ scores, int64_t scores_ld,
                                                    int n_sink, int n_window, const uint32_t* __restrict__ thr_key,
                                                    Cand* __restrict__ cand, int64_t cand_ld,
                                                    uint32_t* __restrict__ seg_cnt, uint32_t* __restrict__ clear,
                                                    int64_t clear_n) {
  clear_region(clear, clear_n);
  extern __shared__ float smem[];
  float* qs = smem;            // [H * d]
  float* ws = smem + H * d;    // [H]
  __shared__ int wave_n[kValuKeysPerWg / kWave];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  for (int i = tid; i < H * d; i += blockDim.x) qs[i] = load_elem<QT>(q, (int64_t)b * H * d + i);
  for (int i = tid; i < H; i += blockDim.x) ws[i] = w[(int64_t)b * H + i];
  __syncthreads();

  const int64_t s = lo + (int64_t)blockIdx.x * kValuKeysPerWg + tid;
  const int64_t tb = t ? (int64_t)t[b] : L - 1;
  float score = 0.f;
  if (s < hi) {
    const int64_t row = s * k_ld;
    for (int j = 0; j < H; ++j) {
      float dot = 0.f;
      for (int x = 0; x < d; ++x) dot = fmaf(qs[j * d + x], load_elem<KT>(k, row + x), dot);
      score = fmaf(ws[j], fmaxf(dot, 0.f), score);
    }
  }
  if (mode == kScoreDense) {
    if (s < hi) scores[(int64_t)b * scores_ld + (s - lo)] = (s <= tb) ? score : -INFINITY;
    return;
  }
  const uint32_t key = score_key(score);
  const bool is_cand = s < hi && is_candidate(s, tb, n_sink, n_window);
  if (mode == kScoreAll) {
    if (s < hi) reinterpret_cast<uint32_t*>(cand)[(int64_t)b * cand_ld + (s - lo)] = is_cand ? key : 0u;
    return;
  }
  // emission in position order: this workgroup's segment holds its candidates above the threshold
  const bool emit = is_cand && key > (thr_key ? thr_key[b] : 0u);
  const uint64_t m = ballot(emit);
  const int wave = tid / kWave;
  if (lane_id() == 0) wave_n[wave] = __popcll(m);
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kValuKeysPerWg / kWave; ++i) {
    before += i < wave ? wave_n[i] : 0;
    total += wave_n[i];
  }
  Cand* seg = cand + (int64_t)b * cand_ld + (int64_t)blockIdx.x * kValuKeysPerWg;
  if (emit) seg[before + lanes_below(m)] = Cand{key, (int32_t)s};
  if (tid == 0) seg_cnt[(int64_t)b * gridDim.x + blockIdx.x] = (uint32_t)total;
}

// Split-L scoring: workgroup = NQ waves = NQ queries. Each of the gridDim.x workgroups of a query group scores a
// contiguous run of the 64-position tiles of [lo, hi), with its queries in registers. bf16 keys arrive by
// asynchronous DMA into four LDS buffers (three tiles in flight); e4m3 keys are loaded two tiles ahead into a
// register ring, converted and committed to two LDS buffers. Emitted candidates are staged per wave in LDS and
// flushed, in position order, to the workgroup's own segment whenever the stage could overflow and at the end;
// the segment's count is stored last.
// G2: block maxima of the two 32-head groups of each 64-head query in one wave (row 2 b + g of the keys; t holds
// one entry per (query, group) and the query's is read at 2 b).
template <int NMT, bool E4M3, int NQ, bool G2 = false>
__global__ __launch_bounds__(64 * NQ) void k_score_mfma(const void* __restrict__ q, const float* __restrict__ w,
                                                        const void* __restrict__ k, int64_t k_ld, int64_t L, int B,
                                                        const int32_t* __restrict__ t, int64_t lo, int64_t hi,
                                                        int mode, float* __restrict__ scores, int64_t scores_ld,
                                                        int n_sink, int n_window,
                                                        const uint32_t* __restrict__ thr_key,
                                                        Cand* __restrict__ cand, int64_t cand_ld,
                                                        uint32_t* __restrict__ seg_cnt,
                                                        uint32_t* __restrict__ clear, int64_t clear_n,
                                                        int page_subs, int page_len, int64_t tok_L) {
  clear_region(clear, clear_n);
  typedef KeyLoader<E4M3, NQ> KL;
  constexpr int kNBuf = E4M3 ? 2 : 4;
  constexpr int kStage = 512;
  __shared__ __attribute__((aligned(1024))) char tiles[kNBuf][kTileBytes];
  __shared__ Cand staged[NQ][kStage];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: addresses stay scalar
  const int b = blockIdx.y * NQ + wave;
  const bool active = b < B;
  // this workgroup scores the contiguous run of tiles [first_tile, first_tile + n_tiles)
  const int64_t tiles_total = (hi - lo + kTileKeys - 1) / kTileKeys;
  const int64_t run = (tiles_total + gridDim.x - 1) / gridDim.x;
  const int64_t first_tile = (int64_t)blockIdx.x * run;
  const int64_t left = tiles_total - first_tile;
  const int64_t n_tiles = left < 0 ? 0 : (left < run ? left : run);
  auto tile_start = [&](int64_t i) { return lo + (first_tile + i) * kTileKeys; };
  const char* kbytes = reinterpret_cast<const char*>(k);
  const int64_t ld_bytes = k_ld * (E4M3 ? 1 : 2);

  QueryFrags<NMT> qf;
  uint32_t thr = 0;
  int64_t tb = L - 1;
  if (active) {
    tb = t ? (int64_t)t[G2 ? 2 * b : b] : L - 1;
    if (mode == kScoreEmit && thr_key) thr = thr_key[b];
    qf.template load<E4M3>(q, w, b, lane);
  }
  // no wait here: the query loads are older than every tile copy and loads complete in issue order, so the first
  // tile's wait (at most two tiles of copies outstanding) also covers them

  int n_emit = 0;     // staged in LDS
  int64_t n_out = 0;  // already in this workgroup's segment
  Cand* seg = cand + (int64_t)b * cand_ld + first_tile * kTileKeys;
  auto flush = [&]() {
    for (int j = lane; j < n_emit; j += kWave) seg[n_out + j] = staged[wave][j];
    n_out += n_emit;
    n_emit = 0;
  };
  auto process_tile = [&](const char* tile, int64_t s0) {
    if (!active || s0 >= hi) return;
    if constexpr (G2) {
      static_assert(NMT == 2, "two 32-head groups per 64-head query");
      if (s0 / page_len >= tb / page_len) return;  // only the blocks before the local one are ranked
      const float2 sc = qf.score_groups(tile, lane);
      const bool in_range = s0 + lane < hi;
      const uint32_t k0 = wave_max_u32(in_range ? score_key(sc.x) : 0u);
      const uint32_t k1 = wave_max_u32(in_range ? score_key(sc.y) : 0u);
      if (lane == 0) {
        uint32_t* row = reinterpret_cast<uint32_t*>(scores) + (int64_t)(2 * b) * scores_ld + s0 / page_len;
        atomicMax(row, k0);
        atomicMax(row + scores_ld, k1);
      }
      return;
    }
    // block maxima rank only the blocks before the one holding t (page_len is the block length, a multiple of 64,
    // so a tile lies in one block)
    if (mode == kScoreBlockMax && s0 / page_len >= tb / page_len) return;
    if (mode == kScoreEmit && n_emit > kStage - kTileKeys) flush();
    const float score = qf.score(tile, lane);
    const int64_t s = s0 + lane;  // lane order is position order
    const bool in_range = s < hi;
    if (mode == kScoreBlockMax) {
      // every position of a block before the local one is visible; the block's key is the max of its scores'
      // keys (score_key is order-preserving), combined over its tiles with an atomic max
      const uint32_t kv = wave_max_u32(in_range ? score_key(score) : 0u);
      if (lane == 0) atomicMax(reinterpret_cast<uint32_t*>(scores) + (int64_t)b * scores_ld + s0 / page_len, kv);
    } else if (mode == kScorePage) {
      // the rows are the sub-block mean keys of the hierarchical index; page p = rows [p G, (p + 1) G) (G divides
      // the 64 rows of a tile, tiles start at multiples of 64): its score sums theirs, rows past the last add 0
      const float v = group_sum(in_range ? score : 0.f, page_subs);
      if ((lane & (page_subs - 1)) == 0 && in_range) {
        const int64_t page = s / page_subs;
        const int64_t tq = t ? tb : tok_L - 1;
        scores[(int64_t)b * scores_ld + page - lo / page_subs] = page * page_len <= tq ? v : -INFINITY;
      }
    } else if (mode == kScoreDense) {
      if (in_range) scores[(int64_t)b * scores_ld + (s - lo)] = (s <= tb) ? score : -INFINITY;
    } else {
      const uint32_t key = score_key(score);
      const bool is_cand = in_range && is_candidate(s, tb, n_sink, n_window);
      if (mode == kScoreAll) {
        if (in_range) reinterpret_cast<uint32_t*>(cand)[(int64_t)b * cand_ld + (s - lo)] = is_cand ? key : 0u;
      } else {
        const bool emit = is_cand && key > thr;
        const uint64_t m = ballot(emit);
        if (emit) staged[wave][n_emit + lanes_below(m)] = Cand{key, (int32_t)s};
        n_emit += __popcll(m);
      }
    }
  };

  walk_tiles<E4M3, NQ, kNBuf>(kbytes, ld_bytes, L, n_tiles, tile_start, tiles, wave, lane,
                              [&](const char* tile, int64_t i) { process_tile(tile, tile_start(i)); });
  if (active && mode == kScoreEmit) {
    if (n_emit > 0) flush();
    if (lane == 0) seg_cnt[(int64_t)b * gridDim.x + blockIdx.x] = (uint32_t)n_out;
  }
}

// Streaming selection for many queries (prefill chunk): workgroup = NQ waves = NQ queries, each wave streams its
// query's candidate positions in ascending order, appends candidates that beat its running threshold to a
// private buffer in global memory, and when the buffer is full keeps only the exact top-k (raising the threshold
// to the k-th key). Positions arrive in ascending order, so a later candidate that only ties the k-th key can
// never displace it: appending requires a strictly larger key.
template <int NMT, bool E4M3, int NQ>
__global__ __launch_bounds__(64 * NQ) void k_stream_select(const void* __restrict__ q, const float* __restrict__ w,
                                                       const void* __restrict__ k, int64_t k_ld, int64_t L, int B,
                                                       const int32_t* __restrict__ t, int kk, int n_sink,
                                                       int n_window, Cand* __restrict__ buf,
                                                       int32_t* __restrict__ buf_n, int cap) {
  typedef KeyLoader<E4M3, NQ> KL;
  constexpr int kNBufS = E4M3 ? 2 : 4;
  __shared__ __attribute__((aligned(1024))) char tiles[kNBufS][kTileBytes];
  __shared__ uint32_t hist[NQ][256];
  __shared__ int64_t wave_end[NQ];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: addresses stay scalar
  const int b = blockIdx.x * NQ + wave;
  const bool active = b < B;
  const char* kbytes = reinterpret_cast<const char*>(k);
  const int64_t ld_bytes = k_ld * (E4M3 ? 1 : 2);

  const int64_t tb = active ? (t ? (int64_t)t[b] : L - 1) : -1;
  const int64_t cand_end = active ? tb - n_window : -1;  // last candidate position (inclusive)
  if (lane == 0) wave_end[wave] = cand_end;
  QueryFrags<NMT> qf;
  if (active) qf.template load<E4M3>(q, w, b, lane);
  __syncthreads();
  int64_t end = wave_end[0];
  for (int i = 1; i < NQ; ++i) end = wave_end[i] > end ? wave_end[i] : end;
  const int64_t s_begin = ((int64_t)n_sink / kTileKeys) * kTileKeys;
  const int n_tiles = end >= s_begin ? (int)((end - s_begin) / kTileKeys + 1) : 0;

  Cand* mybuf = buf + (int64_t)(active ? b : 0) * cap;
  int n = 0;
  uint32_t thr = 0;
  const int cend = (int)cand_end;  // positions fit in 32 bits
  auto score_and_emit = [&](const char* tile, int64_t s0) {
    if (!active || s0 > cand_end) return;
    const float score = qf.score(tile, lane);
    const int s = (int)s0 + lane;  // lane order is position order
    const uint32_t key = score_key(score);
    const bool cand = s >= n_sink && s <= cend;
    if (n + kWave > cap) {
      wait_vmem();
      thr = wave_select_compact(mybuf, n, kk, hist[wave], lane);
      n = n < kk ? n : kk;
    }
    const bool emit = cand && key > thr;
    const uint64_t m = ballot(emit);
    if (emit) mybuf[n + lanes_below(m)] = Cand{key, s};
    n += __popcll(m);
  };
  if constexpr (!E4M3) {
    // bf16 keys: asynchronous DMA into four LDS buffers, three tiles in flight
    typename KL::Regs none;
    KL::init(none, ld_bytes, wave, lane);
    const int n_pre = n_tiles < kNBufS - 1 ? n_tiles : kNBufS - 1;
    for (int p = 0; p < n_pre; ++p)
      KL::fetch(kbytes, ld_bytes, L, s_begin + (int64_t)p * kTileKeys, tiles[p], wave, lane, none);
    for (int tile = 0; tile < n_tiles; ++tile) {
      const int newer = n_tiles - 1 - tile;
      if (newer >= 2) wait_vmem_below<2 * KL::kPerWave>();
      else if (newer == 1) wait_vmem_below<KL::kPerWave>();
      else wait_vmem_below<0>();
      lds_barrier();
      if (tile + kNBufS - 1 < n_tiles)
        KL::fetch(kbytes, ld_bytes, L, s_begin + (int64_t)(tile + kNBufS - 1) * kTileKeys,
                  tiles[(tile + kNBufS - 1) % kNBufS], wave, lane, none);
      score_and_emit(tiles[tile % kNBufS], s_begin + (int64_t)tile * kTileKeys);
    }
  } else {
    typename KL::Regs regs;
    if (n_tiles > 0) {
      KL::fetch(kbytes, ld_bytes, L, s_begin, tiles[0], wave, lane, regs);
      KL::commit(regs, tiles[0], threadIdx.x);
    }
    for (int tile = 0; tile < n_tiles; ++tile) {
      wait_vmem();
      __syncthreads();
      const bool more = tile + 1 < n_tiles;
      if (more)
        KL::fetch(kbytes, ld_bytes, L, s_begin + (int64_t)(tile + 1) * kTileKeys, tiles[(tile + 1) & 1], wave, lane,
                  regs);
      score_and_emit(tiles[tile & 1], s_begin + (int64_t)tile * kTileKeys);
      if (more) KL::commit(regs, tiles[(tile + 1) & 1], threadIdx.x);
    }
  }
  if (active && lane == 0) buf_n[b] = n;
}


// ---- streaming selection for few queries ---------------------------------------------------------------------------
// One launch scores a range of positions for every query. Workgroup = NQ waves = NQ queries scoring a run of at most
// stream_wg_keys / NQ positions, whose keys stay in LDS (the score matrix never leaves the chip). Each query wave then
//   1. publishes one statistic of its chunk: x = the m-th largest of its 64 per-lane maxima, so that at least m keys
//      of the chunk are >= x;
//   2. polls its query's slots, a bounded number of times, until the other workgroups of the launch have published
//      theirs (the grid is sized to be co-resident, so they normally have; after the last poll it goes on with
//      whatever is published);
//   3. takes T = the r-th largest published x with r = ceil(k / m): r chunks hold at least m keys >= T each, so at
//      least k candidates score >= T and T is a lower bound of the k-th key, whatever subset was seen. The bound of
//      the earlier launches of the call (thr[b]) is a lower bound too; the larger one is used;
//   4. emits its keys >= T, in position order, to its own segment of the merge's input.
// Workgroup 0 of each query group also takes the same statistic over every slot of the call so far and stores it in
// thr[b] for the next launch. No key per (query, position) is written to memory.
// keys per workgroup in LDS, over its NQ queries: 32 KB, or 16 KB where four bf16 DMA buffers (64 KB) are staged
// for only four queries, so that two such workgroups share a CU
constexpr int stream_wg_keys(bool e4m3, int nq) { return (!e4m3 && nq == 4) ? 4096 : 8192; }
constexpr int kStreamMaxWgs = 512;    // workgroups per query group and launch (eight slots per lane)
constexpr int kStreamTopCap = 1024;   // kept statistics of earlier launches per query (r <= 512 of them are needed)
constexpr int kStreamTargetWgs = 256;  // workgroups a launch aims for, over all its query groups

struct StreamArgs {
  int64_t lo, hi;        // positions of this launch
  int n_sink, n_window;
  int k, m;              // k of the selection; m of the published statistic (1..64)
  uint32_t* pub;         // [B, pub_ld], zero at the first launch: slots (this launch's workgroup w owns slot slot0 + w)
  int64_t pub_ld;
  int slot0;
  uint32_t* thr;         // [B] lower bound carried between launches
  uint32_t* top;         // [B, kStreamTopCap + 1]: count, then the largest statistics of the earlier launches
  int first;             // first launch of the call: thr and top are not read
  int last;              // last launch of the call: thr and top are not written
  Cand* cand;            // [B, cand_ld]: segment j at cand + j * seg_cap
  int64_t cand_ld, seg_cap;
  uint32_t* seg_cnt;     // [B, seg_ld]
  int64_t seg_ld;
  int spin_limit;        // polls of the other workgroups' slots before going on without them
};

// The r-th largest (r >= 1) of the values v[j] (j < NV, lanes x registers) of the wave, or 0 when fewer than r are
// nonzero: the largest x with at least r values >= x, found bit by bit.
// Branch-free: zero values never count (every candidate threshold c is >= 1).
template <int NV>
__device__ __forceinline__ uint32_t wave_rth_largest(const uint32_t (&v)[NV], int r) {
  uint32_t prefix = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) cnt += __popcll(ballot(v[j] >= c));
    prefix = cnt >= r ? c : prefix;
  }
  return prefix;
}

template <int NMT, bool E4M3, int NQ>
__global__ __launch_bounds__(64 * NQ) void k_score_stream(const void* __restrict__ q, const float* __restrict__ w,
                                                          const void* __restrict__ k, int64_t k_ld, int64_t L, int B,
                                                          const int32_t* __restrict__ t, StreamArgs a) {
  constexpr int kNBuf = E4M3 ? 2 : 4;
  constexpr int kRun = stream_wg_keys(E4M3, NQ) / NQ;  // keys of one query in LDS
  constexpr int kSlotRegs = kStreamMaxWgs / kWave;
  __shared__ __attribute__((aligned(1024))) char tiles[kNBuf][kTileBytes];
  __shared__ uint32_t keys_s[NQ][kRun];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int b = blockIdx.y * NQ + wave;
  const bool active = b < B;
  const int n_wg = gridDim.x, wg = blockIdx.x;
  const int64_t tiles_total = (a.hi - a.lo + kTileKeys - 1) / kTileKeys;
  const int64_t run = (tiles_total + n_wg - 1) / n_wg;  // <= kRun / 64 (the host plans it so)
  const int64_t first_tile = (int64_t)wg * run;
  const int64_t left = tiles_total - first_tile;
  const int n_tiles = (int)(left < 0 ? 0 : (left < run ? left : run));
  auto tile_start = [&](int64_t i) { return a.lo + (first_tile + i) * kTileKeys; };
  const char* kbytes = reinterpret_cast<const char*>(k);
  const int64_t ld_bytes = k_ld * (E4M3 ? 1 : 2);

  QueryFrags<NMT> qf;
  int64_t tb = L - 1;
  if (active) {
    tb = t ? (int64_t)t[b] : L - 1;
    qf.template load<E4M3>(q, w, b, lane);
  }
  // the query and weight loads complete before the first tile copy is issued: the compiler then knows them done,
  // instead of waiting for them inside the tile loop, where its vmcnt waits would also drain the copies in flight
  wait_vmem();
  walk_tiles<E4M3, NQ, kNBuf>(kbytes, ld_bytes, L, n_tiles, tile_start, tiles, wave, lane,
                              [&](const char* tile, int64_t i) {
                                if (!active) return;
                                const float score = qf.score(tile, lane);
                                const int64_t s = tile_start(i) + lane;
                                const bool cand = s < a.hi && is_candidate(s, tb, a.n_sink, a.n_window);
                                keys_s[wave][i * kTileKeys + lane] = cand ? score_key(score) : 0u;
                              });
  // 1. the chunk's statistic (each lane reads back only the keys it wrote itself, all requested at once). It is
  // published as at least 1, so that a written slot is never 0: a published 1 only lowers the bound to 1, which no
  // candidate's key is below (key 0 marks "no candidate"), so every candidate is then emitted and the result is
  // still exact.
  constexpr int kKeysPerLane = kRun / kTileKeys;
  uint32_t mine[kKeysPerLane];
#pragma unroll
  for (int i = 0; i < kKeysPerLane; ++i) mine[i] = i < n_tiles ? keys_s[wave][i * kTileKeys + lane] : 0u;
  uint32_t lmax = 0;
#pragma unroll
  for (int i = 0; i < kKeysPerLane; ++i) lmax = mine[i] > lmax ? mine[i] : lmax;
  const uint32_t lm[1] = {lmax};
  uint32_t x = wave_rth_largest(lm, a.m);
  x = x > 1u ? x : 1u;
  if (!active) return;  // no barrier follows

  // 2. this wave's query row: publish the statistic, then poll the launch's slots (a bounded number of times) until
  // every workgroup's is written; slots still unwritten read 0, which the bound ignores (the slots of a call start
  // at zero). Cross-workgroup data goes through device-coherent single accesses (agent-scope atomics: they bypass
  // the per-XCD L2 caches, which are not coherent with one another), never through fences, which would write back
  // and invalidate a whole L2 under the other workgroups' tile copies. The wave's own slot is taken from x.
  uint32_t* slots = a.pub + (int64_t)b * a.pub_ld + a.slot0;
  if (lane == 0) __hip_atomic_store(slots + wg, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // Launches of at most 128 workgroups (the usual case) keep their slots in two registers per lane; the loads of one
  // poll are issued together (clamped addresses) and slots past the launch's count are 0.
  constexpr int kFewRegs = 2;
  const bool few = n_wg <= kFewRegs * kWave;
  uint32_t xs[kSlotRegs];
  for (int it = 0;; ++it) {
    uint32_t v[kSlotRegs];
#pragma unroll
    for (int j = 0; j < kFewRegs; ++j) {
      const int i = j * kWave + lane;
      v[j] = __hip_atomic_load(slots + (i < n_wg ? i : n_wg - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!few) {
#pragma unroll
      for (int j = kFewRegs; j < kSlotRegs; ++j) {
        const int i = j * kWave + lane;
        v[j] = __hip_atomic_load(slots + (i < n_wg ? i : n_wg - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    bool up = true;
#pragma unroll
    for (int j = 0; j < kSlotRegs; ++j) {
      const int i = j * kWave + lane;
      xs[j] = (i >= n_wg || (few && j >= kFewRegs)) ? 0u : (i == wg ? x : v[j]);
      up = up && (i >= n_wg || xs[j] != 0u);
    }
    if (__all(up) || it >= a.spin_limit) break;
    __builtin_amdgcn_s_sleep(4);
  }

  // 3. the lower bound of the k-th key
  const int r = (a.k + a.m - 1) / a.m;
  uint32_t T;
  if (few) {
    const uint32_t x2[kFewRegs] = {xs[0], xs[1]};
    T = wave_rth_largest(x2, r);
  } else {
    T = wave_rth_largest(xs, r);
  }
  if (!a.first) {
    const uint32_t prev = __hip_atomic_load(a.thr + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    T = prev > T ? prev : T;
  }
  if (wg == 0 && !a.last) {
    // the same statistic over every slot of the call so far, for the next launch: the r-th largest of the union is
    // the r-th largest of (the r largest of the earlier launches' slots, kept in top[b]) and this launch's slots;
    // the values >= it are kept as the new top[b] (only this wave touches top[b])
    constexpr int kTopRegs = kStreamTopCap / kWave;
    uint32_t* tp = a.top + (int64_t)b * (kStreamTopCap + 1);
    const int tn = a.first ? 0 : (int)tp[0];
    uint32_t ys[kTopRegs];
#pragma unroll
    for (int j = 0; j < kTopRegs; ++j) {
      const int i = j * kWave + lane;
      ys[j] = i < tn ? tp[1 + i] : 0u;
    }
    uint32_t u = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = u | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < kSlotRegs; ++j) cnt += __popcll(ballot(xs[j] >= c));
#pragma unroll
      for (int j = 0; j < kTopRegs; ++j) cnt += __popcll(ballot(ys[j] >= c));
      u = cnt >= r ? c : u;
    }
    wait_vmem();  // every load of top[b] has returned before it is overwritten
    int n = 0;
    auto keep = [&](uint32_t v) {
      const bool f = v != 0u && v >= u;
      const uint64_t mk = ballot(f);
      const int o = n + lanes_below(mk);
      if (f && o < kStreamTopCap) tp[1 + o] = v;
      n += __popcll(mk);
    };
#pragma unroll
    for (int j = 0; j < kSlotRegs; ++j) keep(xs[j]);
#pragma unroll
    for (int j = 0; j < kTopRegs; ++j) keep(ys[j]);
    if (lane == 0) {
      tp[0] = (uint32_t)(n < kStreamTopCap ? n : kStreamTopCap);  // ties beyond the cap change no r-th value
      __hip_atomic_store(a.thr + b, u > T ? u : T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // 4. emission of the keys >= T in position order
  Cand* seg = a.cand + (int64_t)b * a.cand_ld + (int64_t)(a.slot0 + wg) * a.seg_cap;
  int n_out = 0;
#pragma unroll
  for (int i = 0; i < kKeysPerLane; ++i) {
    const uint32_t key = mine[i];  // 0 past the last tile
    const bool emit = key != 0u && key >= T;
    const uint64_t mk = ballot(emit);
    if (emit) seg[n_out + lanes_below(mk)] = Cand{key, (int32_t)(tile_start(i) + lane)};
    n_out += __popcll(mk);
  }
  if (lane == 0) a.seg_cnt[(int64_t)b * a.seg_ld + a.slot0 + wg] = (uint32_t)n_out;
}

template <int QT, int KT>
hipError_t launch_valu(const IndexerArgs& a, int64_t lo, int64_t hi, int mode, float* scores, int64_t scores_ld,
                       int n_sink, int n_window, const uint32_t* thr, Cand* cand, int64_t cand_ld,
                       uint32_t* seg_cnt, hipStream_t st) {
  const int64_t n = hi - lo;
  dim3 grid((unsigned)((n + kValuKeysPerWg - 1) / kValuKeysPerWg), (unsigned)a.B);
  const size_t lds = sizeof(float) * ((size_t)a.H * a.d + a.H);
  SA_LAUNCH((k_score_valu<QT, KT>), grid, dim3(256), lds, st, a.q, a.w, a.k, a.k_ld, a.L, a.H, a.d, a.t,
                     lo, hi, mode, scores, scores_ld, n_sink, n_window, thr, cand, cand_ld, seg_cnt, a.clear,
                     a.clear_n);
  return hipGetLastError();
}

// Workgroups per launch: about one per CU for 8-query workgroups (two per CU for 4-query ones), each walking
// many tiles when the range is long.
constexpr int kScoreTargetThreads = 256 * 512;

// Workgroups per query group, and the tiles of each contiguous run, for n_tiles tiles: about kScoreTargetThreads
// threads in flight, and no workgroup left without tiles.
void mfma_grid(int B, int NQ, int64_t n_tiles, int64_t* n_wg, int64_t* run) {
  const int groups = B > NQ ? (B + NQ - 1) / NQ : 1;
  const int64_t target = kScoreTargetThreads / (64 * NQ);
  int64_t per_group = (target + groups - 1) / groups;
  if (per_group > n_tiles) per_group = n_tiles;
  if (per_group < 1) per_group = 1;
  if (n_tiles < 1) n_tiles = 1;
  const int64_t r0 = (n_tiles + per_group - 1) / per_group;
  *n_wg = (n_tiles + r0 - 1) / r0;
  *run = (n_tiles + *n_wg - 1) / *n_wg;
}

template <int NMT, bool FP8, int NQ, bool G2 = false>
hipError_t launch_mfma(const IndexerArgs& a, int64_t lo, int64_t hi, int mode, float* scores, int64_t scores_ld,
                       int n_sink, int n_window, const uint32_t* thr, Cand* cand, int64_t cand_ld,
                       uint32_t* seg_cnt, hipStream_t st, int page_subs = 1, int page_len = 1, int64_t tok_L = 0) {
  const int64_t n_tiles = (hi - lo + kTileKeys - 1) / kTileKeys;
  int64_t n_wg, run;
  mfma_grid(a.B, NQ, n_tiles, &n_wg, &run);
  if (n_tiles < 1 || a.B < 1) return hipSuccess;
  dim3 grid((unsigned)n_wg, (unsigned)((a.B + NQ - 1) / NQ));
  SA_LAUNCH((k_score_mfma<NMT, FP8, NQ, G2>), grid, dim3(64 * NQ), 0, st, a.q, a.w, a.k, a.k_ld, a.L, a.B, a.t,
                     lo, hi, mode, scores, scores_ld, n_sink, n_window, thr, cand, cand_ld, seg_cnt, a.clear, a.clear_n,
                     page_subs, page_len, tok_L);
  return hipGetLastError();
}

}  // namespace

bool score_uses_mfma(const IndexerArgs& a) {
  const bool shape = a.d == 128 && (a.H == 32 || a.H == 64);
  const bool types = (a.q_dtype == 1 && a.k_dtype == 1) || (a.q_dtype == 2 && a.k_dtype == 2);
  return shape && types;
}

int score_keys_per_wg(const IndexerArgs& a) { return score_uses_mfma(a) ? kMfmaKeysPerWg : kValuKeysPerWg; }

EmitPlan score_emit_plan(const IndexerArgs& a, int64_t lo, int64_t hi) {
  EmitPlan p{0, 0};
  if (hi <= lo) return p;
  if (score_uses_mfma(a)) {
    int64_t n_wg, run;
    mfma_grid(a.B, a.B >= 8 ? 8 : 4, (hi - lo + kTileKeys - 1) / kTileKeys, &n_wg, &run);
    p.n_seg = (int)n_wg;
    p.seg_cap = run * kTileKeys;
  } else {
    p.n_seg = (int)((hi - lo + kValuKeysPerWg - 1) / kValuKeysPerWg);
    p.seg_cap = kValuKeysPerWg;
  }
  return p;
}

hipError_t launch_score(const IndexerArgs& a, int64_t lo, int64_t hi, int mode, float* scores, int64_t scores_ld,
                        int n_sink, int n_window, const uint32_t* thr, Cand* cand, int64_t cand_ld,
                        uint32_t* seg_cnt, hipStream_t st) {
  if (hi <= lo) return hipSuccess;
  if (score_uses_mfma(a)) {
    const bool fp8 = a.q_dtype == 2;
    const bool wide = a.B >= 8;
#define SA_SCORE(NMT, F8, NQ) \
  return launch_mfma<NMT, F8, NQ>(a, lo, hi, mode, scores, scores_ld, n_sink, n_window, thr, cand, cand_ld, seg_cnt, st)
    if (a.H == 64) {
      if (fp8) { if (wide) SA_SCORE(2, true, 8); else SA_SCORE(2, true, 4); }
      else { if (wide) SA_SCORE(2, false, 8); else SA_SCORE(2, false, 4); }
    } else {
      if (fp8) { if (wide) SA_SCORE(1, true, 8); else SA_SCORE(1, true, 4); }
      else { if (wide) SA_SCORE(1, false, 8); else SA_SCORE(1, false, 4); }
    }
#undef SA_SCORE
  }
  const int qt = a.q_dtype, kt = a.k_dtype;
  if (qt == 0 && kt == 0) return launch_valu<0, 0>(a, lo, hi, mode, scores, scores_ld, n_sink, n_window, thr, cand, cand_ld, seg_cnt, st);
  if (qt == 1 && kt == 1) return launch_valu<1, 1>(a, lo, hi, mode, scores, scores_ld, n_sink, n_window, thr, cand, cand_ld, seg_cnt, st);
  if (qt == 2 && kt == 2) return launch_valu<2, 2>(a, lo, hi, mode, scores, scores_ld, n_sink, n_window, thr, cand, cand_ld, seg_cnt, st);
  return hipErrorInvalidValue;
}

bool stream_select_supported(const IndexerArgs& a) { return score_uses_mfma(a); }

hipError_t launch_page_scores(const IndexerArgs& m, int page_subs, int page_len, int64_t tok_L, float* scores,
                              int64_t scores_ld, hipStream_t st) {
  if (!score_uses_mfma(m) || m.q_dtype != 1 || page_subs < 1 || page_subs > 64 || (page_subs & (page_subs - 1)))
    return hipErrorInvalidValue;
  if (m.B < 1 || m.L < 1) return hipSuccess;
  // eight queries per workgroup share each key tile for mid-sized batches; many queries (a prefill chunk) take
  // four, so that two workgroups share a CU (measured faster there, as for the per-query streaming select)
  const bool wide = m.B >= 8 && m.B < 64;
  if (m.H == 64) {
    if (wide) return launch_mfma<2, false, 8>(m, 0, m.L, kScorePage, scores, scores_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, page_subs, page_len, tok_L);
    return launch_mfma<2, false, 4>(m, 0, m.L, kScorePage, scores, scores_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, page_subs, page_len, tok_L);
  }
  if (wide) return launch_mfma<1, false, 8>(m, 0, m.L, kScorePage, scores, scores_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, page_subs, page_len, tok_L);
  return launch_mfma<1, false, 4>(m, 0, m.L, kScorePage, scores, scores_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, page_subs, page_len, tok_L);
}

hipError_t launch_block_max(const IndexerArgs& a, int block, uint32_t* keys, int64_t keys_ld, hipStream_t st) {
  if (!score_uses_mfma(a) || block < kTileKeys || block % kTileKeys != 0) return hipErrorInvalidValue;
  if (a.B < 1 || a.L < 1) return hipSuccess;
  float* out = reinterpret_cast<float*>(keys);  // the block-max mode writes uint32 keys through the scores pointer
  const bool wide = a.B >= 8;
  const bool fp8 = a.q_dtype == 2;
  if (a.groups2) {
    // rows are (query, group) pairs of 32 heads; one wave takes both groups of a query (a 64-head query)
    IndexerArgs aq = a;
    aq.B = a.B / 2;
    aq.H = 64;
    const bool wq = aq.B >= 32;  // four queries per workgroup below 32 (16 queries at 128K: 41.8 against 44.0 us)
    if (fp8) return wq ? launch_mfma<2, true, 8, true>(aq, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L)
                       : launch_mfma<2, true, 4, true>(aq, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L);
    return wq ? launch_mfma<2, false, 8, true>(aq, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L)
              : launch_mfma<2, false, 4, true>(aq, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L);
  }
  if (a.H == 64) {
    if (fp8) return wide ? launch_mfma<2, true, 8>(a, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L)
                         : launch_mfma<2, true, 4>(a, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L);
    return wide ? launch_mfma<2, false, 8>(a, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L)
                : launch_mfma<2, false, 4>(a, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L);
  }
  if (fp8) return wide ? launch_mfma<1, true, 8>(a, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L)
                       : launch_mfma<1, true, 4>(a, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L);
  return wide ? launch_mfma<1, false, 8>(a, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L)
              : launch_mfma<1, false, 4>(a, 0, a.L, kScoreBlockMax, out, keys_ld, 0, 0, nullptr, nullptr, 0, nullptr, st, 1, block, a.L);
}

bool stream_supported(const IndexerArgs& a) { return score_uses_mfma(a); }

StreamPlan stream_plan(const IndexerArgs& a, int64_t end) {
  StreamPlan p{};
  // four queries per workgroup (two workgroups per CU) up to 31 queries: at 16 queries the scorer takes 42 us
  // against 45 us with eight
  p.nq = a.B >= 32 ? 8 : 4;
  // positions per workgroup: enough workgroups for the whole chip (about kStreamTargetWgs over all query groups),
  // at most the workgroup's LDS capacity, a whole number of tiles
  const int64_t cap_keys = stream_wg_keys(a.q_dtype == 2, p.nq) / p.nq;
  const int64_t groups = a.B > p.nq ? (a.B + p.nq - 1) / p.nq : 1;
  const int64_t target = kStreamTargetWgs / groups > 1 ? kStreamTargetWgs / groups : 1;
  int64_t run = (end + target - 1) / target;
  run = (run + kTileKeys - 1) / kTileKeys * kTileKeys;
  run = run < kTileKeys ? kTileKeys : (run > cap_keys ? cap_keys : run);
  p.run_keys = (int)run;
  p.end = end;
  // launch ranges hold whole runs, so the workgroup count of all launches together does not depend on how many
  // workgroups one launch has
  p.slots = (end + p.run_keys - 1) / p.run_keys;
  p.pub_ld = p.slots;
  p.top_words = kStreamTopCap + 1;
  return p;
}

namespace {
// Workgroups of one k_score_stream instance resident on the current device at once (cached per device).
template <int NMT, bool E4M3, int NQ>
hipError_t stream_resident(int* out) {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return hipSuccess;
    }
  }
  int per_cu = 0, cus = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k_score_stream<NMT, E4M3, NQ>),
                                                   64 * NQ, 0);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int r = per_cu * cus > 0 ? per_cu * cus : 1;
  if (dev >= 0 && dev < 64) cache[dev].store(r, std::memory_order_relaxed);
  *out = r;
  return hipSuccess;
}

template <int NMT, bool E4M3, int NQ>
hipError_t launch_stream_t(const IndexerArgs& a, int k, int n_sink, int n_window, const StreamPlan& p, uint32_t* pub,
                           uint32_t* thr, uint32_t* top, uint32_t* seg_cnt, Cand* cand, int spin_limit,
                           hipStream_t st) {
  int resident = 0;
  hipError_t e = stream_resident<NMT, E4M3, NQ>(&resident);
  if (e != hipSuccess) return e;
  const int groups = (a.B + NQ - 1) / NQ;
  int n_wg = resident / groups;
  n_wg = n_wg < 1 ? 1 : (n_wg > kStreamMaxWgs ? kStreamMaxWgs : n_wg);
  const int64_t range = (int64_t)n_wg * p.run_keys;
  StreamArgs sa{};
  sa.n_sink = n_sink;
  sa.n_window = n_window;
  sa.k = k;
  sa.pub = pub;
  sa.pub_ld = p.pub_ld;
  sa.thr = thr;
  sa.top = top;
  sa.cand = cand;
  sa.cand_ld = p.slots * (int64_t)p.run_keys;
  sa.seg_cap = p.run_keys;
  sa.seg_cnt = seg_cnt;
  sa.seg_ld = p.slots;
  sa.spin_limit = spin_limit;
  e = launch_fill_u32(pub, (int64_t)a.B * p.pub_ld, 0u, st);  // slots and counters of the call start at zero
  if (e != hipSuccess) return e;
  int slot0 = 0;
  for (int64_t lo = 0; lo < p.end; lo += range) {
    const int64_t hi = lo + range < p.end ? lo + range : p.end;
    const int wgs = (int)((hi - lo + p.run_keys - 1) / p.run_keys);
    // statistic: the m-th largest lane maximum of each chunk, m chosen from this launch's workgroup count so that
    // about 2k keys of its range reach the bound (at most 64 lanes; at least k / wgs so that r = ceil(k / m)
    // chunks can exist)
    int m = (int)((2 * (int64_t)k + wgs - 1) / wgs);
    m = m < 1 ? 1 : (m > 64 ? 64 : m);
    sa.m = m;
    sa.lo = lo;
    sa.hi = hi;
    sa.slot0 = slot0;
    sa.first = lo == 0;
    sa.last = hi >= p.end;
    SA_LAUNCH((k_score_stream<NMT, E4M3, NQ>), dim3((unsigned)wgs, (unsigned)groups), dim3(64 * NQ), 0, st, a.q, a.w,
              a.k, a.k_ld, a.L, a.B, a.t, sa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    slot0 += wgs;
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_stream_decode(const IndexerArgs& a, int k, int n_sink, int n_window, const StreamPlan& p,
                                uint32_t* pub, uint32_t* thr, uint32_t* top, uint32_t* seg_cnt, Cand* cand,
                                int spin_limit, hipStream_t st) {
  if (!score_uses_mfma(a) || a.B < 1) return a.B < 1 ? hipSuccess : hipErrorInvalidValue;
  const bool fp8 = a.q_dtype == 2;
#define SA_STREAMD(NMT, F8, NQ) \
  return launch_stream_t<NMT, F8, NQ>(a, k, n_sink, n_window, p, pub, thr, top, seg_cnt, cand, spin_limit, st)
  if (p.nq == 8) {
    if (a.H == 64) { if (fp8) SA_STREAMD(2, true, 8); else SA_STREAMD(2, false, 8); }
    else { if (fp8) SA_STREAMD(1, true, 8); else SA_STREAMD(1, false, 8); }
  } else {
    if (a.H == 64) { if (fp8) SA_STREAMD(2, true, 4); else SA_STREAMD(2, false, 4); }
    else { if (fp8) SA_STREAMD(1, true, 4); else SA_STREAMD(1, false, 4); }
  }
#undef SA_STREAMD
}

hipError_t launch_stream_select(const IndexerArgs& a, int k, int n_sink, int n_window, Cand* buf, int32_t* buf_n,
                                int cap, hipStream_t st) {
  if (!score_uses_mfma(a) || cap < k + 32) return hipErrorInvalidValue;
  // four queries per workgroup: two workgroups share each CU, so one's MFMA work overlaps the other's epilogue
  // (eight queries per workgroup halve the key traffic but measured slower: the waves of a workgroup move in
  // lockstep between tile barriers)
  const bool fp8 = a.q_dtype == 2;
  const int nq = 4;
  dim3 grid((unsigned)((a.B + nq - 1) / nq));
#define SA_STREAM(NMT, F8, NQ)                                                                                  \
  SA_LAUNCH((k_stream_select<NMT, F8, NQ>), grid, dim3(64 * NQ), 0, st, a.q, a.w, a.k, a.k_ld, a.L, a.B, \
                     a.t, k, n_sink, n_window, buf, buf_n, cap)
  if (a.H == 64) {
    if (fp8) SA_STREAM(2, true, 4); else SA_STREAM(2, false, 4);
  } else {
    if (fp8) SA_STREAM(1, true, 4); else SA_STREAM(1, false, 4);
  }
#undef SA_STREAM
  return hipGetLastError();
}

}  // namespace sa
