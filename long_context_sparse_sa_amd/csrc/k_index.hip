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
#include <type_traits>

#include "sa_device.h"
#include "sa_internal.h"
#include "sa_wave_select.h"

namespace sa {
namespace {

constexpr int kValuKeysPerWg = 256;
constexpr int kMfmaKeysPerWg = 512;
constexpr int kTileKeys = 64;

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

// ---- MFMA scoring building blocks ---------------------------------------------------------------------------------
// NMT = H / 32 head tiles per query, d = 128. The dot products always run on the bf16 32x32x16 MFMA, whose sums
// are exact for these operands. E4M3-stored keys and queries are converted exactly to bf16 on the way into LDS
// and registers: the fp8 MFMA is not used because its internal accumulation loses about 2^-15 of the sum of
// |products|, which would move scores by more than the selection tolerance.
//
// LDS key tile: 64 positions x 256 bytes of bf16; the 16-byte chunk c of position n is stored at chunk
// c ^ (n % 16) so that the 32 lanes reading one chunk column spread over the banks.
constexpr int kTileRowBytes = 256;
constexpr int kTileChunks = 16;
constexpr int kTileBytes = kTileKeys * kTileRowBytes;
constexpr int kSteps = 8;  // MFMA k-steps of 16 dims

__device__ __forceinline__ int tile_off(int n, int c) { return n * kTileRowBytes + 16 * (c ^ (n % kTileChunks)); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

// Exact E4M3 -> bf16 of the four bytes of `packed`.
__device__ __forceinline__ bf16x4 e4m3x4_to_bf16(int packed) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, true);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(int a, int b) {
  return __builtin_shufflevector(e4m3x4_to_bf16(a), e4m3x4_to_bf16(b), 0, 1, 2, 3, 4, 5, 6, 7);
}

template <bool E4M3, int NW>
struct KeyLoader;

// bf16 keys: the stored 256-byte rows go straight to LDS by asynchronous DMA (16 KB = 16 wave instructions).
// Each lane's byte offset inside a tile is computed once (init); a tile then costs one address add per copy,
// except a tile that runs past row L - 1, which clamps its rows (rows past the end are never scored, the clamp
// keeps the copy in bounds).
template <int NW>
struct KeyLoader<false, NW> {
  static constexpr int kPerWave = 16 / NW;
  struct Regs {
    int64_t off[kPerWave];
  };
  static __device__ __forceinline__ void init(Regs& r, int64_t ld_bytes, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int slot = (wave * kPerWave + j) * 64 + lane;
      const int n = slot / kTileChunks;
      const int c = (slot % kTileChunks) ^ (n % kTileChunks);
      r.off[j] = n * ld_bytes + c * 16;
    }
  }
  static __device__ __forceinline__ void fetch(const char* kbytes, int64_t ld_bytes, int64_t L, int64_t s0,
                                               char* tile, int wave, int lane, Regs& r) {
    const char* base = kbytes + s0 * ld_bytes;
    if (s0 + kTileKeys <= L) {
#pragma unroll
      for (int j = 0; j < kPerWave; ++j) dma16(base + r.off[j], tile + (wave * kPerWave + j) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < kPerWave; ++j) {
        const int slot = (wave * kPerWave + j) * 64 + lane;
        const int n = slot / kTileChunks;
        const int c = (slot % kTileChunks) ^ (n % kTileChunks);
        const int64_t row = (s0 + n < L ? s0 + n : L - 1) - s0;
        dma16(base + row * ld_bytes + c * 16, tile + (wave * kPerWave + j) * 1024);
      }
    }
  }
  static __device__ __forceinline__ void commit(const Regs&, char*, int) {}
};

// e4m3 keys: each thread loads BPT stored bytes of one position and writes them as 2 BPT bytes of bf16.
template <int NW>
struct KeyLoader<true, NW> {
  static constexpr int BPT = 8192 / (64 * NW);      // raw bytes per thread (32 or 16)
  static constexpr int TPK = 128 / BPT;             // threads per position
  struct Regs {
    int4 part[BPT / 16];
  };
  static __device__ __forceinline__ void init(Regs&, int64_t, int, int) {}
  static __device__ __forceinline__ void fetch(const char* kbytes, int64_t ld_bytes, int64_t L, int64_t s0, char*,
                                               int, int, Regs& r) {
    const int tid = threadIdx.x;
    int64_t s = s0 + tid / TPK;
    s = s < L ? s : L - 1;
    const int4* src = reinterpret_cast<const int4*>(kbytes + s * ld_bytes + BPT * (tid % TPK));
#pragma unroll
    for (int p = 0; p < BPT / 16; ++p) r.part[p] = src[p];
  }
  static __device__ __forceinline__ void commit(const Regs& r, char* tile, int tid) {
    const int n = tid / TPK, c0 = (BPT / 8) * (tid % TPK);
#pragma unroll
    for (int p = 0; p < BPT / 16; ++p) {
      *reinterpret_cast<bf16x8*>(tile + tile_off(n, c0 + 2 * p)) = e4m3x8_to_bf16(r.part[p].x, r.part[p].y);
      *reinterpret_cast<bf16x8*>(tile + tile_off(n, c0 + 2 * p + 1)) = e4m3x8_to_bf16(r.part[p].z, r.part[p].w);
    }
  }
};

// Query fragments (A operand, head = 32 * mt + lane % 32, dims 16 ks + 8 (lane / 32) ..) and the head weights in
// the accumulator layout (this lane's 16 values of tile mt belong to heads 32 mt + 8 (r / 4) + 4 (lane / 32) + r % 4).
template <int NMT, bool E4M3>
__device__ __forceinline__ void load_query(const void* q, const float* w, int64_t b, int lane,
                                           bf16x8 (&qa)[NMT][kSteps], float (&wv)[NMT][16]) {
  constexpr int H = 32 * NMT;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int64_t e0 = (b * H + 32 * mt + (lane & 31)) * 128 + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      if constexpr (E4M3) {
        const int2 raw = *reinterpret_cast<const int2*>(reinterpret_cast<const char*>(q) + e0 + ks * 16);
        qa[mt][ks] = e4m3x8_to_bf16(raw.x, raw.y);
      } else {
        qa[mt][ks] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(q) + e0 + ks * 16);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[mt][r] = w[b * H + 32 * mt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)];
  }
}

// ReLU as one integer max: a negative float (or -0) has a negative int image and becomes +0; other values pass.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Scores of the 64 positions of a tile: lane l returns the score of position l of the tile.
// The eight key fragments of a 32-position half sit in a register ring: the half-0 fragments are read up front
// and each slot is refilled with the matching half-1 fragment as soon as its MFMAs are issued, so every LDS read
// has eight MFMA pairs to land. The half-1 MFMAs are interleaved with the half-0 ReLU-weighted head sum (two MFMAs,
// then eight VALU instructions, per k-step), so the matrix unit and the VALU work at the same time.
template <int NMT>
__device__ __forceinline__ float score_tile(const char* tile, int lane, const bf16x8 (&qa)[NMT][kSteps],
                                           const float (&wv)[NMT][16]) {
  static_assert(NMT * 16 % kSteps == 0, "head-sum chunks must divide evenly over the k-steps");
  constexpr int kChunk = NMT * 16 / kSteps;  // half-0 accumulator elements folded per half-1 k-step
  const int hs = lane >> 5;
  auto frag = [&](int nt, int ks) {
    return *reinterpret_cast<const bf16x8*>(tile + tile_off(32 * nt + (lane & 31), 2 * ks + hs));
  };
  bf16x8 fr[kSteps];
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) fr[ks] = frag(0, ks);
  f32x16 acc0[NMT], acc1[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    acc0[mt] = f32x16{};
    acc1[mt] = f32x16{};
  }
  // half 0
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) {
    const bf16x8 bk = fr[ks];
    fr[ks] = frag(1, ks);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc0[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][ks], bk, acc0[mt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // half 1, with the half-0 head sum in the MFMA shadow
  float part0 = 0.f;
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc1[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][ks], fr[ks], acc1[mt], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < kChunk; ++e) {
      const int idx = ks * kChunk + e;
      part0 = fmaf(wv[idx / 16][idx % 16], relu(acc0[idx / 16][idx % 16]), part0);
    }
  }
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) {
    __builtin_amdgcn_sched_group_barrier(0x008, NMT, 0);       // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 2 * kChunk, 0);  // VALU
  }
  __builtin_amdgcn_sched_barrier(0);
  float part1 = 0.f;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) part1 = fmaf(wv[mt][r], relu(acc1[mt][r]), part1);
  // part0 / part1 hold the half-0 / half-1 sums over this lane's heads; lanes l and l ^ 32 cover the two head
  // halves of the same position
  return fold_halves(part0, part1);
}

// Split-L scoring: workgroup = NQ waves = NQ queries. Each of the gridDim.x workgroups of a query group scores a
// contiguous run of the 64-position tiles of [lo, hi), with its queries in registers. bf16 keys arrive by
// asynchronous DMA into four LDS buffers (three tiles in flight); e4m3 keys are loaded two tiles ahead into a
// register ring, converted and committed to two LDS buffers. Emitted candidates are staged per wave in LDS and
// flushed, in position order, to the workgroup's own segment whenever the stage could overflow and at the end;
// the segment's count is stored last.
template <int NMT, bool E4M3, int NQ>
__global__ __launch_bounds__(64 * NQ) void k_score_mfma(const void* __restrict__ q, const float* __restrict__ w,
                                                        const void* __restrict__ k, int64_t k_ld, int64_t L, int B,
                                                        const int32_t* __restrict__ t, int64_t lo, int64_t hi,
                                                        int mode, float* __restrict__ scores, int64_t scores_ld,
                                                        int n_sink, int n_window,
                                                        const uint32_t* __restrict__ thr_key,
                                                        Cand* __restrict__ cand, int64_t cand_ld,
                                                        uint32_t* __restrict__ seg_cnt,
                                                        uint32_t* __restrict__ clear, int64_t clear_n) {
  clear_region(clear, clear_n);
  typedef KeyLoader<E4M3, NQ> KL;
  constexpr int kNBuf = E4M3 ? 2 : 4;
  constexpr int kStage = 512;
  constexpr int kDmaPerWave = KeyLoader<false, NQ>::kPerWave;
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

  bf16x8 qa[NMT][kSteps];
  float wv[NMT][16];
  uint32_t thr = 0;
  int64_t tb = L - 1;
  if (active) {
    tb = t ? (int64_t)t[b] : L - 1;
    if (mode == kScoreEmit && thr_key) thr = thr_key[b];
    load_query<NMT, E4M3>(q, w, b, lane, qa, wv);
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
    if (mode == kScoreEmit && n_emit > kStage - kTileKeys) flush();
    const float score = score_tile<NMT>(tile, lane, qa, wv);
    const int64_t s = s0 + lane;  // lane order is position order
    const bool in_range = s < hi;
    if (mode == kScoreDense) {
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

  if constexpr (!E4M3) {
    typename KL::Regs none;
    KL::init(none, ld_bytes, wave, lane);
    const int64_t n_pre = n_tiles < kNBuf - 1 ? n_tiles : kNBuf - 1;
    for (int64_t p = 0; p < n_pre; ++p) KL::fetch(kbytes, ld_bytes, L, tile_start(p), tiles[p], wave, lane, none);
    for (int64_t i = 0; i < n_tiles; ++i) {
      const int64_t newer = n_tiles - 1 - i;
      if (newer >= 2) wait_vmem_below<2 * kDmaPerWave>();
      else if (newer == 1) wait_vmem_below<kDmaPerWave>();
      else wait_vmem_below<0>();
      lds_barrier();
      if (i + kNBuf - 1 < n_tiles)
        KL::fetch(kbytes, ld_bytes, L, tile_start(i + kNBuf - 1), tiles[(i + kNBuf - 1) % kNBuf], wave, lane, none);
      process_tile(tiles[i % kNBuf], tile_start(i));
    }
  } else {
    typename KL::Regs ring[2];
    if (n_tiles > 0) {
      KL::fetch(kbytes, ld_bytes, L, tile_start(0), nullptr, wave, lane, ring[0]);
      if (n_tiles > 1) KL::fetch(kbytes, ld_bytes, L, tile_start(1), nullptr, wave, lane, ring[1]);
      KL::commit(ring[0], tiles[0], threadIdx.x);
      if (n_tiles > 2) KL::fetch(kbytes, ld_bytes, L, tile_start(2), nullptr, wave, lane, ring[0]);
    }
    // tile i + 1 (ring slot (i + 1) % 2) goes to LDS while tile i is scored; its slot then takes tile i + 3.
    // Unrolled by two so that ring slots and LDS buffers are compile-time (a runtime-indexed ring would live in
    // scratch memory).
    auto step = [&](int64_t i, auto P) {
      constexpr int p = decltype(P)::value;
      lds_barrier();
      if (i + 1 < n_tiles) {
        KL::commit(ring[1 - p], tiles[1 - p], threadIdx.x);
        if (i + 3 < n_tiles) KL::fetch(kbytes, ld_bytes, L, tile_start(i + 3), nullptr, wave, lane, ring[1 - p]);
      }
      process_tile(tiles[p], tile_start(i));
    };
    for (int64_t i = 0; i < n_tiles; i += 2) {
      step(i, std::integral_constant<int, 0>{});
      if (i + 1 < n_tiles) step(i + 1, std::integral_constant<int, 1>{});
    }
  }
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
  bf16x8 qa[NMT][kSteps];
  float wv[NMT][16];
  if (active) load_query<NMT, E4M3>(q, w, b, lane, qa, wv);
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
    const float score = score_tile<NMT>(tile, lane, qa, wv);
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

template <int QT, int KT>
hipError_t launch_valu(const IndexerArgs& a, int64_t lo, int64_t hi, int mode, float* scores, int64_t scores_ld,
                       int n_sink, int n_window, const uint32_t* thr, Cand* cand, int64_t cand_ld,
                       uint32_t* seg_cnt, hipStream_t st) {
  const int64_t n = hi - lo;
  dim3 grid((unsigned)((n + kValuKeysPerWg - 1) / kValuKeysPerWg), (unsigned)a.B);
  const size_t lds = sizeof(float) * ((size_t)a.H * a.d + a.H);
  hipLaunchKernelGGL((k_score_valu<QT, KT>), grid, dim3(256), lds, st, a.q, a.w, a.k, a.k_ld, a.L, a.H, a.d, a.t,
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

template <int NMT, bool FP8, int NQ>
hipError_t launch_mfma(const IndexerArgs& a, int64_t lo, int64_t hi, int mode, float* scores, int64_t scores_ld,
                       int n_sink, int n_window, const uint32_t* thr, Cand* cand, int64_t cand_ld,
                       uint32_t* seg_cnt, hipStream_t st) {
  const int64_t n_tiles = (hi - lo + kTileKeys - 1) / kTileKeys;
  int64_t n_wg, run;
  mfma_grid(a.B, NQ, n_tiles, &n_wg, &run);
  if (n_tiles < 1 || a.B < 1) return hipSuccess;
  dim3 grid((unsigned)n_wg, (unsigned)((a.B + NQ - 1) / NQ));
  hipLaunchKernelGGL((k_score_mfma<NMT, FP8, NQ>), grid, dim3(64 * NQ), 0, st, a.q, a.w, a.k, a.k_ld, a.L, a.B, a.t,
                     lo, hi, mode, scores, scores_ld, n_sink, n_window, thr, cand, cand_ld, seg_cnt, a.clear, a.clear_n);
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
  hipLaunchKernelGGL((k_stream_select<NMT, F8, NQ>), grid, dim3(64 * NQ), 0, st, a.q, a.w, a.k, a.k_ld, a.L, a.B, \
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
