// MFMA building blocks of the lightning-indexer scorers (LongCat Sparse Attention deep-dive, DSA baseline section,
// indexer equation): staged key tiles, register-resident query fragments, and the score of a 64-position tile,
// I(b, s) = sum_j w[b, j] * ReLU(q[b, j, :] . k[s, :]), for d = 128 and 32 * NMT heads.
#pragma once

#include <type_traits>

#include "sa_device.h"

namespace sa {
namespace tile {

constexpr int kTileKeys = 64;

// NMT = H / 32 head tiles per query, d = 128. The dot products always run on a bf16 MFMA (32x32x16 for 32 heads,
// 16x16x32 for 64 heads, below): products of bf16 operands are exact in fp32 and are summed in fp32. E4M3-stored
// keys and queries are converted exactly to bf16 on the way into LDS and registers. The fp8 MFMA is not used: on
// 128-long dot products its internal accumulation was measured to lose up to 1.8e-4 (mean 1.7e-5) of the sum of
// |products|, against 2.6e-7 for the bf16 MFMA on the converted values, and that would move scores by more than
// the selection tolerance.
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
//
// frag(nt, ks) gives this lane's B fragment of k-step ks in half nt: position 32 nt + lane % 32, dims
// 16 ks + 8 (lane / 32) .. + 7. score_tile reads them from an LDS tile; score_frags takes any source.
template <int NMT, typename FR>
__device__ __forceinline__ float score_frags(FR&& frag, const bf16x8 (&qa)[NMT][kSteps],
                                            const float (&wv)[NMT][16]) {
  static_assert(NMT * 16 % kSteps == 0, "head-sum chunks must divide evenly over the k-steps");
  constexpr int kChunk = NMT * 16 / kSteps;  // half-0 accumulator elements folded per half-1 k-step
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

template <int NMT>
__device__ __forceinline__ float score_tile(const char* tile, int lane, const bf16x8 (&qa)[NMT][kSteps],
                                           const float (&wv)[NMT][16]) {
  const int hs = lane >> 5;
  return score_frags<NMT>(
      [&](int nt, int ks) {
        return *reinterpret_cast<const bf16x8*>(tile + tile_off(32 * nt + (lane & 31), 2 * ks + hs));
      },
      qa, wv);
}

// ---- 64 heads on the 16x16x32 MFMA ----------------------------------------------------------------------------
// The same scores for 64 heads with four M-tiles of 16 heads, four N-tiles of 16 positions and four k-steps of 32
// dims: as many MFMA flops and LDS fragment bytes per tile, a quarter of the accumulator registers per instruction,
// and half the head-weight registers. On random bf16 operands this shape sustains a higher issue rate than the
// 32x32x16 one (a loop of each on random operands, two waves per SIMD: 0.76-0.79 against 0.62-0.70 of the peak),
// and the scorer loop with its ReLU-weighted head sum and LDS fragment reads goes from about 0.56 to 0.60.
//
// Operands: A (queries) lane l holds head 16 mt + l % 16, dims 32 ks + 8 (l / 16) .. + 7; B (keys) lane l holds
// position 16 nt + l % 16, the same dims; the accumulator of (mt, nt) holds, in lane l, position 16 nt + l % 16
// for heads 16 mt + 4 (l / 16) + r, r < 4. The key tile in LDS is the one above (chunk c of position n at chunk
// slot c ^ (n % 16)): the 16 lanes of a row read 16 positions at one chunk, spread over every bank.
constexpr int kSteps16 = 4;

template <bool E4M3>
__device__ __forceinline__ void load_query16(const void* q, const float* w, int64_t b, int lane,
                                             bf16x8 (&qa)[4][kSteps16], float (&wv)[4][4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t e0 = (b * 64 + 16 * mt + (lane & 15)) * 128 + (lane >> 4) * 8;
#pragma unroll
    for (int ks = 0; ks < kSteps16; ++ks) {
      if constexpr (E4M3) {
        const int2 raw = *reinterpret_cast<const int2*>(reinterpret_cast<const char*>(q) + e0 + ks * 32);
        qa[mt][ks] = e4m3x8_to_bf16(raw.x, raw.y);
      } else {
        qa[mt][ks] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(q) + e0 + ks * 32);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = w[b * 64 + 16 * mt + 4 * (lane >> 4) + r];
  }
}

// Scores of the 64 positions of a tile (lane l: position l). Half 0 (N-tiles 0, 1) runs first with its eight key
// fragments read up front; each ring slot is refilled with the matching half-1 fragment once its MFMAs are issued.
// The half-1 MFMAs are interleaved with the half-0 ReLU-weighted head sum (four MFMAs, then eight VALU
// instructions, per fragment). Each lane sums its 16 heads of each N-tile; two lane exchanges then add the four
// lane rows that hold the other heads of the same position.
// NG = 1: one sum over the 64 heads; NG = 2: the two 32-head groups (head tiles 0-1 and 2-3) summed on their own,
// returned as (group 0, group 1).
template <int NG, typename FR>
__device__ __forceinline__ auto score_frags16(FR&& frag, const bf16x8 (&qa)[4][kSteps16], const float (&wv)[4][4]) {
  static_assert(NG == 1 || NG == 2, "one or two head groups");
  bf16x8 fr[8];  // slot i = 4 n + ks: N-tile n of the half being multiplied, k-step ks
#pragma unroll
  for (int i = 0; i < 8; ++i) fr[i] = frag(i >> 2, i & 3);
  f32x4 acc0[2][4], acc1[2][4];  // [N-tile within the half][mt]
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      acc0[n][mt] = f32x4{};
      acc1[n][mt] = f32x4{};
    }
  // half 0
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bf16x8 bk = fr[i];
    fr[i] = frag(2 + (i >> 2), i & 3);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      acc0[i >> 2][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][i & 3], bk, acc0[i >> 2][mt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // half 1, with the half-0 head sum in the MFMA shadow (32 products over the eight fragments)
  float p[NG][4];  // this lane's head sums of N-tiles 0..3, per group
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int n = 0; n < 4; ++n) p[g][n] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      acc1[i >> 2][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][i & 3], fr[i], acc1[i >> 2][mt], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = 4 * i + e, n = idx >> 4, mt = (idx >> 2) & 3, r = idx & 3;
      float& acc = p[mt * NG / 4][n];
      acc = fmaf(wv[mt][r], relu(acc0[n][mt][r]), acc);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float& acc = p[mt * NG / 4][2 + n];
        acc = fmaf(wv[mt][r], relu(acc1[n][mt][r]), acc);
      }
  // lanes l and l ^ 32 hold heads of rows {0, 2} and {1, 3} of the same positions: the first exchange leaves
  // N-tiles 0 and 1 in lanes 0..31 and N-tiles 2 and 3 in lanes 32..63 (rows 0 + 2 or 1 + 3 added); the second
  // adds rows l and l ^ 16, so that lane l holds all the group's heads of position l
  auto fold = [&](const float (&q)[4]) { return fold_rows(fold_halves(q[0], q[2]), fold_halves(q[1], q[3])); };
  if constexpr (NG == 1) return fold(p[0]);
  else return float2{fold(p[0]), fold(p[1])};
}

__device__ __forceinline__ float score_tile16(const char* tile, int lane, const bf16x8 (&qa)[4][kSteps16],
                                              const float (&wv)[4][4]) {
  const int row = lane >> 4;
  return score_frags16<1>(
      [&](int nt, int ks) {
        return *reinterpret_cast<const bf16x8*>(tile + tile_off(16 * nt + (lane & 15), 4 * ks + row));
      },
      qa, wv);
}

// The two 32-head groups of a 64-head query, summed on their own: lane l returns (group 0, group 1) of position l.
__device__ __forceinline__ float2 score_tile16_groups(const char* tile, int lane, const bf16x8 (&qa)[4][kSteps16],
                                                      const float (&wv)[4][4]) {
  const int row = lane >> 4;
  return score_frags16<2>(
      [&](int nt, int ks) {
        return *reinterpret_cast<const bf16x8*>(tile + tile_off(16 * nt + (lane & 15), 4 * ks + row));
      },
      qa, wv);
}

// A query's register-resident fragments and head weights, and the score of an LDS key tile: 32 heads on the
// 32x32x16 MFMA, 64 heads on the 16x16x32 one.
template <int NMT>
struct QueryFrags {
  bf16x8 qa[NMT][kSteps];
  float wv[NMT][16];
  template <bool E4M3>
  __device__ __forceinline__ void load(const void* q, const float* w, int64_t b, int lane) {
    load_query<NMT, E4M3>(q, w, b, lane, qa, wv);
  }
  __device__ __forceinline__ float score(const char* tile, int lane) const { return score_tile<NMT>(tile, lane, qa, wv); }
};
template <>
struct QueryFrags<2> {
  bf16x8 qa[4][kSteps16];
  float wv[4][4];
  template <bool E4M3>
  __device__ __forceinline__ void load(const void* q, const float* w, int64_t b, int lane) {
    load_query16<E4M3>(q, w, b, lane, qa, wv);
  }
  __device__ __forceinline__ float score(const char* tile, int lane) const { return score_tile16(tile, lane, qa, wv); }
  __device__ __forceinline__ float2 score_groups(const char* tile, int lane) const {
    return score_tile16_groups(tile, lane, qa, wv);
  }
};

// The B fragments of the 64-position tile at s0 straight from global memory into registers (rows past L - 1 are
// clamped to it; they are never scored). Plain loads: the compiler places the waits before their first use.
__device__ __forceinline__ void load_frags(const char* kbytes, int64_t ld_bytes, int64_t L, int64_t s0, int lane,
                                           bf16x8 (&f)[2][kSteps]) {
  const int hs = lane >> 5;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    int64_t row = s0 + 32 * nt + (lane & 31);
    row = row < L ? row : L - 1;
    const char* p = kbytes + row * ld_bytes + 16 * hs;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) f[nt][ks] = *reinterpret_cast<const bf16x8*>(p + 32 * ks);
  }
}

// Waits until at most min(newer, MAXN) tiles of PER copies each are outstanding (vmcnt takes an immediate).
template <int MAXN, int PER>
__device__ __forceinline__ void wait_tiles_newer(int64_t newer) {
  if constexpr (MAXN > 0) {
    if (newer >= MAXN) {
      wait_vmem_below<MAXN * PER>();
      return;
    }
    wait_tiles_newer<MAXN - 1, PER>(newer);
  } else {
    wait_vmem_below<0>();
  }
}

// Walks the tiles 0 .. n_tiles-1 of a workgroup's run (tile i covers positions tile_start(i) .. + 63): every wave
// calls on_tile(tile_in_lds, i) once per tile, in order, after the tile's keys have landed in LDS. bf16 keys arrive
// by asynchronous DMA into NBUF >= 3 LDS buffers (NBUF - 1 tiles in flight); e4m3 keys are loaded two tiles ahead into a
// register ring, converted and committed to two LDS buffers. All waves of the workgroup must call it.
template <bool E4M3, int NQ, int NBUF, typename TS, typename F>
__device__ __forceinline__ void walk_tiles(const char* kbytes, int64_t ld_bytes, int64_t L, int64_t n_tiles,
                                           TS tile_start, char (*tiles)[kTileBytes], int wave, int lane,
                                           F&& on_tile) {
  typedef KeyLoader<E4M3, NQ> KL;
  constexpr int kDmaPerWave = KeyLoader<false, NQ>::kPerWave;
  if constexpr (!E4M3) {
    // at tile i's wait, tiles i+1 .. i+NBUF-2 may still be in flight; after the barrier (every wave is done with
    // tile i-1) tile i+NBUF-1 goes into tile i-1's buffer, so NBUF-1 tiles are in flight while tile i is scored
    static_assert(NBUF >= 3 && (NBUF - 2) * kDmaPerWave < 64, "the wait counts must fit the vmcnt field");
    typename KL::Regs none;
    KL::init(none, ld_bytes, wave, lane);
    const int64_t n_pre = n_tiles < NBUF - 1 ? n_tiles : NBUF - 1;
    for (int64_t p = 0; p < n_pre; ++p) KL::fetch(kbytes, ld_bytes, L, tile_start(p), tiles[p], wave, lane, none);
    for (int64_t i = 0; i < n_tiles; ++i) {
      const int64_t newer = n_tiles - 1 - i;
      wait_tiles_newer<NBUF - 2, kDmaPerWave>(newer);
      lds_barrier();
      if (i + NBUF - 1 < n_tiles)
        KL::fetch(kbytes, ld_bytes, L, tile_start(i + NBUF - 1), tiles[(i + NBUF - 1) % NBUF], wave, lane, none);
      on_tile(tiles[i % NBUF], i);
    }
  } else {
    static_assert(NBUF == 2, "e4m3 tiles alternate between two LDS buffers");
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
      on_tile(tiles[p], i);
    };
    for (int64_t i = 0; i < n_tiles; i += 2) {
      step(i, std::integral_constant<int, 0>{});
      if (i + 1 < n_tiles) step(i + 1, std::integral_constant<int, 1>{});
    }
  }
}

}  // namespace tile
}  // namespace sa
