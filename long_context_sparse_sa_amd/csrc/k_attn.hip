// Sparse attention over the read set (LongCat Sparse Attention deep-dive: DSA baseline section, attention over the
// selected latent rows c_s, MLA absorbed-MQA form with one latent row shared by every query head; SI section, HFA:
// partial attentions over disjoint row sets merge exactly by log-sum-exp rescaling).
//
// The read set of query b is a virtual row list: the sink [0, ns), the window [w0, t] (w0 >= ns so the two never
// overlap), then the sparse positions idx[b, 0:n_sel[b]].
//
// Kernels:
//  * k_attn_generic -- any widths, fp32 or bf16, one workgroup per (query, head), two passes (max/sum, then
//    weighted V), fp32 throughout.
//  * k_attn_mfma    -- bf16 latent of width 576 (V = first 512 or all 576 columns), 64 heads per workgroup
//    (4 waves = 2 head blocks of 32 heads x 2 halves of the 576 dims). Rows are gathered 32 at a time into LDS
//    by asynchronous DMA (72 x 16-byte chunks per 1152-byte row), S^T = K Q^T runs on the 32x32x16 bf16 MFMA with
//    each wave's 32 query heads register-resident over its 288 dims (the two halves add their partial scores
//    through LDS), the online softmax runs in the log2 domain, and O^T = V^T P^T takes V through LDS transpose
//    reads so that P never leaves registers. Rows are split over workgroups when queries are few; each split's
//    partial rows go to the workspace in fp16, scaled per (head, column half) by a power of two into [-1, 1], and
//    k_attn_combine merges the splits by their (max, sum).
#include <math.h>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Split partials: floats per (query, head, split) after the fp16 row: max, sum, and the power-of-two factor of each
// half of the value columns.
constexpr int kMlWords = 4;

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)u);
}

struct RowList {
  int ns, nw, nsel, w0;
  const int32_t* idx;
  __device__ __forceinline__ int count() const { return ns + nw + nsel; }
  __device__ __forceinline__ int pos(int r) const {
    if (r < ns) return r;
    if (r < ns + nw) return w0 + (r - ns);
    return idx[r - ns - nw];
  }
};

__device__ __forceinline__ RowList make_rows(int b, int64_t L, const int32_t* t, const int32_t* idx, int idx_ld,
                                             const int32_t* n_sel, int n_sink, int n_window) {
  RowList R;
  const int tb = t ? t[b] : (int)(L - 1);
  R.ns = n_sink < tb + 1 ? n_sink : tb + 1;
  int w0 = tb - n_window + 1;
  w0 = w0 > R.ns ? w0 : R.ns;
  R.w0 = w0;
  R.nw = tb + 1 - w0 > 0 ? tb + 1 - w0 : 0;
  int ns = 0;
  if (idx && n_sel) {
    ns = n_sel[b];
    ns = ns < 0 ? 0 : (ns > idx_ld ? idx_ld : ns);
  }
  R.nsel = ns;
  R.idx = idx ? idx + (int64_t)b * idx_ld : nullptr;
  return R;
}

// ---------------------------------------------------------------------------------------------------------------
// Generic path
// ---------------------------------------------------------------------------------------------------------------
constexpr int kGenThreads = 256;
constexpr int kGenMaxDv = 1024;

template <int DT>
__device__ __forceinline__ void store_out(void* out, int64_t i, float v) {
  if constexpr (DT == 0)
    reinterpret_cast<float*>(out)[i] = v;
  else
    reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(v);
}

template <int DT>
__global__ __launch_bounds__(kGenThreads) void k_attn_generic(const void* __restrict__ q, const void* __restrict__ kv,
                                                               const void* __restrict__ v, int64_t kv_ld, int64_t v_ld,
                                                               int64_t L, int H, int d_qk, int d_v,
                                                               const int32_t* __restrict__ t,
                                                               const int32_t* __restrict__ idx, int idx_ld,
                                                               const int32_t* __restrict__ n_sel, int n_sink,
                                                               int n_window, float scale, void* __restrict__ out,
                                                               float* __restrict__ lse) {
  extern __shared__ float gsm[];
  float* qs = gsm;                       // [d_qk]
  float* zb = gsm + d_qk;                // [kGenThreads]
  int* pb = reinterpret_cast<int*>(zb + kGenThreads);  // [kGenThreads]
  __shared__ float red_m[kGenThreads / kWave], red_l[kGenThreads / kWave];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const RowList R = make_rows(b, L, t, idx, idx_ld, n_sel, n_sink, n_window);
  const int n = R.count();
  const int64_t qoff = ((int64_t)b * H + h) * d_qk;
  for (int i = tid; i < d_qk; i += kGenThreads) qs[i] = load_elem<DT>(q, qoff + i);
  __syncthreads();
  const void* vsrc = v ? v : kv;
  const int64_t vld = v ? v_ld : kv_ld;

  auto logit = [&](int s) {
    float acc = 0.f;
    const int64_t row = (int64_t)s * kv_ld;
    for (int x = 0; x < d_qk; ++x) acc = fmaf(qs[x], load_elem<DT>(kv, row + x), acc);
    return acc * scale;
  };

  // pass 1: running (max, sum) per thread, then a block reduction
  float m = -INFINITY, l = 0.f;
  for (int r = tid; r < n; r += kGenThreads) {
    const float z = logit(R.pos(r));
    const float mn = fmaxf(m, z);
    l = l * expf(m - mn) + expf(z - mn);
    m = mn;
  }
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const float mo = __shfl_xor(m, off, kWave), lo = __shfl_xor(l, off, kWave);
    const float mn = fmaxf(m, mo);
    l = (mn == -INFINITY) ? 0.f : l * expf(m - mn) + lo * expf(mo - mn);
    m = mn;
  }
  if ((tid & (kWave - 1)) == 0) {
    red_m[tid / kWave] = m;
    red_l[tid / kWave] = l;
  }
  __syncthreads();
  float M = -INFINITY, Ls = 0.f;
  for (int i = 0; i < kGenThreads / kWave; ++i) {
    const float mn = fmaxf(M, red_m[i]);
    Ls = (mn == -INFINITY) ? 0.f : Ls * expf(M - mn) + red_l[i] * expf(red_m[i] - mn);
    M = mn;
  }

  // pass 2: o = sum_s exp(z_s - M) V_s / Ls, threads own output columns
  float acc[kGenMaxDv / kGenThreads];
#pragma unroll
  for (int j = 0; j < kGenMaxDv / kGenThreads; ++j) acc[j] = 0.f;
  for (int r0 = 0; r0 < n; r0 += kGenThreads) {
    const int r = r0 + tid;
    if (r < n) {
      const int s = R.pos(r);
      zb[tid] = expf(logit(s) - M);
      pb[tid] = s;
    }
    __syncthreads();
    const int cnt = n - r0 < kGenThreads ? n - r0 : kGenThreads;
    for (int j = 0; j < cnt; ++j) {
      const float p = zb[j];
      const int64_t row = (int64_t)pb[j] * vld;
#pragma unroll
      for (int c = 0; c < kGenMaxDv / kGenThreads; ++c) {
        const int dv = tid + c * kGenThreads;
        if (dv < d_v) acc[c] = fmaf(p, load_elem<DT>(vsrc, row + dv), acc[c]);
      }
    }
    __syncthreads();
  }
  const int64_t ooff = ((int64_t)b * H + h) * d_v;
#pragma unroll
  for (int c = 0; c < kGenMaxDv / kGenThreads; ++c) {
    const int dv = tid + c * kGenThreads;
    if (dv < d_v) store_out<DT>(out, ooff + dv, n > 0 ? acc[c] / Ls : 0.f);
  }
  if (lse && tid == 0) lse[(int64_t)b * H + h] = n > 0 ? M + logf(Ls) : -INFINITY;
}

// ---------------------------------------------------------------------------------------------------------------
// MFMA path: bf16 latent rows of 576 values (1152 bytes = 72 chunks of 16 bytes), 64 heads per workgroup
// ---------------------------------------------------------------------------------------------------------------
constexpr int kRowElems = 576;
constexpr int kRowChunks = 72;
constexpr int kRowBytes = 1152;
constexpr int kTileRows = 32;
constexpr int kTileBytes = kTileRows * kRowBytes;        // 36864
constexpr int kDmaPerWave = kTileBytes / 1024 / 4;       // 9 wave instructions of 1 KB per tile
constexpr int kNBuf = 3;                                 // LDS tiles: up to 2 in flight while one is consumed
constexpr int kMaxRowsPerSplit = 4096;                   // positions of one split staged in LDS
constexpr int kQSteps = kRowElems / 2 / 16;              // 18 k-steps of 16 dims: each wave takes half the dims
constexpr float kRescaleSlack = 8.f;                     // log2 headroom before the running max is raised
constexpr int kPrefK = 4;                                // K fragments in flight ahead of the S^T MFMAs
constexpr int kPrefV = 3;                                // V^T fragments in flight ahead of the O^T MFMAs

// Chunk c of row n lives at chunk slot c ^ f(n), f(n) = ((n >> 2) & 3) | (((n >> 1) & 1) << 2) (the XOR stays
// inside the aligned group of 8 chunks; f has period 16). With 1152-byte rows this keeps both LDS read patterns
// free of bank conflicts: 16 consecutive rows reading one chunk (K fragments), and 4 consecutive rows reading 4
// consecutive chunks in 8-byte halves (V transpose reads of two lane groups).
__device__ __forceinline__ int chunk_slot(int n, int c) { return c ^ (((n >> 2) & 3) | (((n >> 1) & 1) << 2)); }

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

__device__ __forceinline__ bf16x8 lds_load_b128(uint32_t lds_addr) {
  return *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(lds_addr);
}
__device__ __forceinline__ i16x4 lds_read_tr16_at(uint32_t lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>(lds_addr));
}

// Lanes l and l ^ 32 exchanged in one VALU instruction: the pair returned holds this lane's value and the partner's
// (which is which depends on the half), so only symmetric combinations of the two are used.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_min(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Grid: 1-D, a multiple of 8 blocks. A unit is (query b, row split); every unit has H / 64 head groups. Blocks are
// dealt to the 8 XCDs by block id mod 8, so XCD x takes the x-th eighth of the (unit, head group) list in order:
// all head groups of a unit, and normally every split of a query, share one XCD's L2. The second gather of a
// tile's rows and the query rows of every split after the first are then served by that L2.
__device__ __forceinline__ void attn_block(int HG, int* u, int* hg) {
  const int blk = (int)blockIdx.x;
  const int g = (blk % 8) * (int)(gridDim.x / 8) + blk / 8;
  *u = g / HG;
  *hg = g % HG;
}

// Workgroup = 4 waves = 2 head blocks of 32 heads x 2 halves. The two waves of a head block each compute S^T = K Q^T
// for their 32 heads over one half of the 576 dims (32x32x16 MFMA, their half of the query heads in registers),
// add each other's partial through LDS (both get the same sum), run the same online softmax, and each accumulates
// O^T = V^T P^T for its half of the value columns. P stays in the registers S^T produced it in: the C layout of
// S^T holds, per lane, 8 rows of one head for each 16-row k-step, and the V^T fragments are read (LDS transpose
// reads) in that same row order.
template <int DV>
__global__ __launch_bounds__(256) void k_attn_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                                   int64_t kv_ld, int64_t L, int H, const int32_t* __restrict__ t,
                                                   const int32_t* __restrict__ idx, int idx_ld,
                                                   const int32_t* __restrict__ n_sel, int n_sink, int n_window,
                                                   float scale_log2, int n_splits, int n_units,
                                                   uint16_t* __restrict__ part_o, float* __restrict__ part_ml,
                                                   uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int DVH = DV / 2;   // value columns per wave
  constexpr int NT = DVH / 32;  // 32-wide output tiles per wave
  __shared__ __attribute__((aligned(1024))) char tiles[kNBuf][kTileBytes];
  __shared__ int32_t pos_s[kMaxRowsPerSplit];
  // partial S^T of each wave, by tile parity, register group and lane: with one barrier per tile a wave may write
  // the next tile's scores before its partner has read this tile's, so consecutive tiles use different halves
  __shared__ f32x4 exch[2][4][4][kWave];
  const int HG = H / 64;
  int u, hg;
  attn_block(HG, &u, &hg);
  if (u >= n_units) return;
  const int b = u / n_splits, split = u % n_splits;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: DMA destinations stay scalar
  const int hsel = lane >> 5;       // which 8 of each 16 dims / rows this lane carries
  const int j = lane & 31;
  const int hb = wave >> 1, dh = wave & 1;
  const int head = 64 * hg + 32 * hb + j;
  const int64_t bh = (int64_t)b * H + head;
  const int dv0 = dh * DVH;

  // Q^T fragments (B operand): head `head`, dims 288 dh + 16 ks + 8 hsel .. +8, requested first: they depend on
  // nothing, so their latency overlaps the read-set bounds and position loads below (loads complete in issue
  // order, so every later wait also covers them)
  bf16x8 qf[kQSteps];
#pragma unroll
  for (int ks = 0; ks < kQSteps; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(q + bh * kRowElems + 288 * dh + 16 * ks + 8 * hsel);

  const RowList R = make_rows(b, L, t, idx, idx_ld, n_sel, n_sink, n_window);
  const int n_rows = R.count();
  // the query's own read set is cut into n_splits tile-aligned parts of nearly equal size, so that read sets far
  // below the bound the grid was planned for still spread over every split; since n_rows never exceeds that bound,
  // no part exceeds the plan's rows per split (at most kMaxRowsPerSplit, the positions staged below)
  const int n_row_tiles = (n_rows + kTileRows - 1) / kTileRows;
  const int r_begin = (int)((int64_t)split * n_row_tiles / n_splits) * kTileRows;
  int r_end = (int)((int64_t)(split + 1) * n_row_tiles / n_splits) * kTileRows;
  r_end = r_end < n_rows ? r_end : n_rows;
  const int n_my = r_end - r_begin;

  if (n_my <= 0) {
    if (n_splits == 1) {
      for (int i = tid; i < 64 * DV; i += 256) out[((int64_t)b * H + 64 * hg) * DV + i] = 0;
      if (lse && tid < 64) lse[(int64_t)b * H + 64 * hg + tid] = -INFINITY;
    } else if (tid < 64) {
      const int64_t bh0 = (int64_t)b * H + 64 * hg + tid;
      part_ml[(bh0 * n_splits + split) * kMlWords + 0] = -INFINITY;
      part_ml[(bh0 * n_splits + split) * kMlWords + 1] = 0.f;
    }
    return;
  }
  const int n_tiles = (n_my + kTileRows - 1) / kTileRows;
  // positions of this split's rows into LDS: the selected-index loads of a thread are issued eight at a time
  // (unconditional, clamped into the list) so that their latencies overlap
  {
    constexpr int kStageBatch = 8;
    const int n_stage = n_tiles * kTileRows;
    const int first_sel = R.ns + R.nw;  // read-set rows from here on come from the selected list
    for (int r0 = 0; r0 < n_stage; r0 += 256 * kStageBatch) {
      int32_t v[kStageBatch];
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        int js = r_begin + r0 + u * 256 + tid - first_sel;
        js = js < 0 ? 0 : (js < R.nsel ? js : R.nsel - 1);
        v[u] = R.nsel > 0 ? R.idx[js] : 0;
      }
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const int r = r0 + u * 256 + tid;
        const int rr = r_begin + r;
        if (r < n_stage)
          pos_s[r] = r >= n_my ? 0 : (rr < R.ns ? rr : (rr < first_sel ? R.w0 + (rr - R.ns) : v[u]));
      }
    }
  }
  __syncthreads();

  // DMA plan of this lane, the same for every tile: its chunk jj of the wave's share lands in row drow[jj] of the
  // tile at chunk slot dcol[jj]; the source row address is gbase[jj] + position * row bytes (one 32x32->64 multiply-add
  // per copy: positions are non-negative and a row is far below 4 GB).
  const uint32_t ld_bytes = (uint32_t)(kv_ld * 2);
  uint32_t drow[kDmaPerWave];
  uint64_t gbase[kDmaPerWave];
#pragma unroll
  for (int jj = 0; jj < kDmaPerWave; ++jj) {
    const int slot = (wave * kDmaPerWave + jj) * 64 + lane;
    const int n = slot / kRowChunks;
    drow[jj] = 4u * n;
    gbase[jj] = (uint64_t)(uintptr_t)kv + 16u * chunk_slot(n, slot % kRowChunks);
  }
  auto dma_rows = [&](int tile, uint32_t* s) {  // source positions of this lane's copies (LDS reads, one wait)
#pragma unroll
    for (int jj = 0; jj < kDmaPerWave; ++jj)
      s[jj] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(pos_s) + tile * 4 * kTileRows + drow[jj]);
  };
  auto dma_one = [&](int jj, const uint32_t* s, int buf) {
    dma16(reinterpret_cast<const void*>(gbase[jj] + (uint64_t)s[jj] * ld_bytes),
          &tiles[buf][(wave * kDmaPerWave + jj) * 1024]);
  };
  auto issue = [&](int tile, int buf) {
    uint32_t s[kDmaPerWave];
    dma_rows(tile, s);
#pragma unroll
    for (int jj = 0; jj < kDmaPerWave; ++jj) dma_one(jj, s, buf);
  };

  f32x16 o[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) o[i] = f32x16{};
  float m_use = -INFINITY, l_run = 0.f;  // exponents are taken relative to m_use (log2 domain)

  // Per-lane LDS byte offsets inside a tile (each unrolled access below is one of these plus a compile-time offset).
  // K fragment (A operand of S^T): row j, chunk 36 dh + 2 ks + hsel at its chunk slot: kofs[ks & 3] + 128 (ks >> 2).
  uint32_t kofs[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) kofs[qq] = j * kRowBytes + 16 * chunk_slot(j, 36 * dh + 2 * qq + hsel);
  // V^T fragment (A operand of O^T) through transpose reads: in each 16-lane group gq = lane / 16, lane
  // a + 4 r4 addresses row 4 hv + r4 (hv = gq / 2) at columns dv0 + 32 nt + 16 (gq & 1) + 4 a; the second read
  // takes rows + 8 (its own base: the swizzle differs), the second k-step rows + 16 (same swizzle). Columns
  // 4 a .. 4 a + 3 sit in chunk C0 + 4 nt at byte 8 (a & 1).
  const int gq = lane >> 4, qa = lane & 3, r4 = (lane >> 2) & 3;
  const int hv = gq >> 1;
  const int vrow = 4 * hv + r4;
  const int C0 = dv0 / 8 + 2 * (gq & 1) + (qa >> 1);
  uint32_t vofs[4];  // [2 * (rows + 8 for the second read) + parity of nt]
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = vrow + 8 * rd;
      vofs[2 * rd + par] = row * kRowBytes + 16 * chunk_slot(row, C0 + 4 * par) + 8 * (qa & 1);
    }
  const uint32_t tiles_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&tiles[0][0];

  // One tile: S^T, the online softmax, O^T. kPartial: the split's last tile is not full (rows past its end are
  // masked to -inf); only that tile pays for the mask.
  auto process = [&](int tile, auto partial) __attribute__((always_inline)) {
    // this tile's fragment bases, made opaque so that the compiler keeps one register per base and folds every
    // constant into the instruction offset (instead of hoisting base + constant sums out of the loop)
    const uint32_t tbase = tiles_lds + (uint32_t)((tile % kNBuf) * kTileBytes);
    uint32_t kb[4], vb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kb[i] = tbase + kofs[i];
      vb[i] = tbase + vofs[i];
      asm volatile("" : "+v"(kb[i]), "+v"(vb[i]));
    }

    // partial S^T (32 rows x 32 heads) over this wave's 288 dims, then the partner's half through LDS. The K
    // fragments run kPrefK steps ahead of the MFMAs in a register ring; the scheduling fences keep the compiler
    // from pulling each read next to its MFMA, which would expose the LDS latency on every step.
    auto k_frag = [&](int ks) { return lds_load_b128(kb[ks & 3] + 128 * (ks >> 2)); };
    bf16x8 kr[kPrefK];
#pragma unroll
    for (int i = 0; i < kPrefK; ++i) kr[i] = k_frag(i);
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      const bf16x8 cur = kr[ks % kPrefK];
      if (ks + kPrefK < kQSteps) kr[ks % kPrefK] = k_frag(ks + kPrefK);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[ks], s, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      exch[tile & 1][wave][g4][lane] = f32x4{s[4 * g4], s[4 * g4 + 1], s[4 * g4 + 2], s[4 * g4 + 3]};
    // one barrier per tile: it hands over the partial scores, shows the next tile's copies landed (every wave
    // waits for its own first), and shows every wave done with the previous tile's buffer, which the copies of
    // tile + kNBuf - 1 then refill
    wait_vmem_below<0>();
    lds_barrier();
    if (tile + kNBuf - 1 < n_tiles) issue(tile + kNBuf - 1, (tile + kNBuf - 1) % kNBuf);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 other = exch[tile & 1][wave ^ 1][g4][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * g4 + e] += other[e];
    }
    auto v_frag = [&](int i) {  // V^T fragment of step i = kk * NT + nt
      const int nt = i % NT, kk = i / NT;
      const i16x4 v0 = lds_read_tr16_at(vb[nt & 1] + 128 * (nt >> 1) + 18432 * kk);
      const i16x4 v1 = lds_read_tr16_at(vb[2 + (nt & 1)] + 128 * (nt >> 1) + 18432 * kk);
      // whole-vector shuffle + bit_cast (a bit_cast of a single ext-vector element is not used here: clang lowers
      // it to element 0 for every index)
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vr[kPrefV];
#pragma unroll
    for (int i = 0; i < kPrefV; ++i) vr[i] = v_frag(i);

    // register r of this lane holds row 8 (r / 4) + 4 hsel + r % 4 of head `head`. The softmax works on raw
    // scores: log2-domain exponent = score * scale_log2 - m_use. The tile's largest scaled score is the scale
    // times the largest raw score, or times the smallest one when the scale is negative (a uniform choice).
    // Rows past the split's end are pushed to the extreme that never wins, and their weights are zeroed below
    // (so that a zero scale never meets an infinity).
    const bool neg = scale_log2 < 0.f;
    const int valid = decltype(partial)::value ? n_my - tile * kTileRows : kTileRows;
    if constexpr (decltype(partial)::value) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * hsel + (r & 3) >= valid) s[r] = neg ? INFINITY : -INFINITY;
    }
    float mt = s[0];
    if (!neg) {
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
      mt = halves_max(mt);
    } else {
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fminf(mt, s[r]);
      mt = halves_min(mt);
    }
    mt *= scale_log2;  // finite: row 0 of a tile is always valid
    // raise the reference only when this tile would exceed it by more than 2^kRescaleSlack
    const bool raise = mt > m_use + kRescaleSlack;
    if (__any(raise)) {
      const float m_new = raise ? mt : m_use;
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);  // 1 where not raised, 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] = o[nt] * alpha;
      m_use = m_new;
    }
    bf16x8 pf[2];
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // exponents are <= kRescaleSlack; results below 2^-126 flush to zero, far below bf16 resolution of the sum
        float p = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + e], scale_log2, -m_use));
        if constexpr (decltype(partial)::value) {
          const int r = 8 * kk + e;
          p = 8 * (r >> 2) + 4 * hsel + (r & 3) >= valid ? 0.f : p;
        }
        psum += p;
        pf[kk][e] = (__bf16)p;
      }
    l_run += psum;

    // O^T (value columns x heads) += V^T P^T; k-step kk covers rows 16 kk + {4 hsel .. +3, 8 + 4 hsel .. +3}.
    // Step i = kk * NT + nt (both k-steps of a tile are NT MFMAs apart); its V^T fragment (two transpose reads)
    // is fetched kPrefV steps ahead.
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      const bf16x8 cur = vr[i % kPrefV];
      if (i + kPrefV < 2 * NT) vr[i % kPrefV] = v_frag(i + kPrefV);
      o[i % NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pf[i / NT], o[i % NT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int n_pre = n_tiles < kNBuf - 1 ? n_tiles : kNBuf - 1;
  for (int p = 0; p < n_pre; ++p) issue(p, p);
  // the first tile's copies landed and are visible to every wave; later tiles are waited for at the barrier of the
  // tile before them
  if (n_pre > 1) wait_vmem_below<kDmaPerWave>();
  else wait_vmem_below<0>();
  lds_barrier();
  const int n_full = n_my / kTileRows;
  for (int tile = 0; tile < n_full; ++tile) process(tile, BoolTag<false>{});
  if (n_full < n_tiles) process(n_full, BoolTag<true>{});

  // lanes j and j + 32 hold disjoint rows of the same head: add their sums
  l_run = halves_sum(l_run);
  // register r of tile nt holds column dv0 + 32 nt + 8 (r / 4) + 4 hsel + r % 4 of head `head`
  if (n_splits == 1) {
    // the bf16 output rows leave through LDS (the tile buffers are free now) as whole rows
    const float inv = 1.f / l_run;
    constexpr int kOutLd = DV + 8;  // padded row of bf16 (16 bytes) so that the lanes of a column spread over banks
    uint16_t* ostage = reinterpret_cast<uint16_t*>(&tiles[0][0]);
    static_assert(64 * kOutLd * 2 <= kNBuf * kTileBytes, "the workgroup's output rows fit in the tile buffers");
    __syncthreads();  // every wave is done with the tile buffers
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint32_t lo = f32_to_bf16_bits(o[nt][4 * g4 + 0] * inv) | ((uint32_t)f32_to_bf16_bits(o[nt][4 * g4 + 1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_bits(o[nt][4 * g4 + 2] * inv) | ((uint32_t)f32_to_bf16_bits(o[nt][4 * g4 + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(ostage + (32 * hb + j) * kOutLd + dv0 + 32 * nt + 8 * g4 + 4 * hsel) = uint2{lo, hi};
      }
    __syncthreads();
    // 64 rows of DV / 8 16-byte chunks: a whole number per thread, all read before any is stored
    constexpr int kPerT = 64 * (DV / 8) / 256;
    static_assert(kPerT * 256 == 64 * (DV / 8), "the output chunks divide evenly over the threads");
    uint16_t* obase = out + ((int64_t)b * H + 64 * hg) * DV;
    uint4 oc[kPerT];
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int e = tid + 256 * i, h = e / (DV / 8), c = 8 * (e % (DV / 8));
      oc[i] = *reinterpret_cast<const uint4*>(ostage + h * kOutLd + c);
    }
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int e = tid + 256 * i;
      *reinterpret_cast<uint4*>(obase + e * 8) = oc[i];  // rows of one workgroup are contiguous in out
    }
    if (lse && dh == 0 && hsel == 0) lse[bh] = (m_use + log2f(l_run)) * kLn2;
  } else {
    // Split partials in fp16: each (head, half of the value columns) is scaled by a power of two 2^-e with
    // 2^e > its largest |o| (exact in fp32), so that its values lie in [-1, 1] where fp16 keeps 11 significant bits;
    // 2^e goes with (m, l). The rows of both head blocks leave through LDS together (the tile buffers are free
    // now), so that every row is written by consecutive threads as whole lines.
    float amax = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(o[nt][r]));
    amax = halves_max(amax);  // lanes j and j + 32 hold the same head
    int ex = 0;
    (void)frexpf(amax, &ex);  // amax < 2^ex (ex = 0 for amax = 0)
    const float down = ldexpf(1.f, -ex);
    constexpr int kStageLd = DV + 8;  // padded row of fp16: the lanes of a column write land in different banks
    static_assert(64 * kStageLd * 2 <= kNBuf * kTileBytes, "the workgroup's partial rows fit in the tile buffers");
    uint16_t* stage = reinterpret_cast<uint16_t*>(&tiles[0][0]);
    __syncthreads();  // every wave is done with the tile buffers
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint32_t lo = f32_to_f16_bits(o[nt][4 * g4 + 0] * down) | (f32_to_f16_bits(o[nt][4 * g4 + 1] * down) << 16);
        const uint32_t hi = f32_to_f16_bits(o[nt][4 * g4 + 2] * down) | (f32_to_f16_bits(o[nt][4 * g4 + 3] * down) << 16);
        *reinterpret_cast<uint2*>(stage + (32 * hb + j) * kStageLd + dv0 + 32 * nt + 8 * g4 + 4 * hsel) = uint2{lo, hi};
      }
    __syncthreads();
    // 64 rows of DV / 8 16-byte chunks, a whole number per thread, all read before any is stored; row h of the
    // workgroup sits h * n_splits rows after its first row
    constexpr int kPerT = 64 * (DV / 8) / 256;
    static_assert(kPerT * 256 == 64 * (DV / 8), "the partial chunks divide evenly over the threads");
    uint16_t* pbase = part_o + (((int64_t)b * H + 64 * hg) * n_splits + split) * DV;
    const int row_step = n_splits * DV;
    uint4 pc[kPerT];
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int e = tid + 256 * i, h = e / (DV / 8), c = 8 * (e % (DV / 8));
      pc[i] = *reinterpret_cast<const uint4*>(stage + h * kStageLd + c);
    }
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int e = tid + 256 * i, h = e / (DV / 8), c = 8 * (e % (DV / 8));
      *reinterpret_cast<uint4*>(pbase + h * row_step + c) = pc[i];
    }
    if (hsel == 0) {
      float* ml = part_ml + (bh * n_splits + split) * kMlWords;
      if (dh == 0) {
        ml[0] = m_use;
        ml[1] = l_run;
      }
      ml[2 + dh] = ldexpf(1.f, ex);
    }
  }
}

// Exact merge of the row splits of one (query, head): o = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i, where split
// i's row O_i is its fp16 row times the power of two stored for its half of the columns. One block per (query,
// head); thread i owns four value columns. Its first eight split rows are requested before anything else, and
// every thread derives the split weights itself from the (max, sum) pairs, which are the same for the whole block
// (uniform loads), so the block needs no barrier. A split with no rows has max -inf and no value row (its
// workspace row is never written): its weight is 0 and its row is skipped, not multiplied.
constexpr int kCombineThreads = 192;  // four columns each: d_v <= 768
constexpr int kCombineBatch = 8;

__device__ __forceinline__ f32x4 f16x4_to_f32(uint2 v) {
  return f32x4{f16_bits_to_f32(v.x & 0xFFFFu), f16_bits_to_f32(v.x >> 16), f16_bits_to_f32(v.y & 0xFFFFu),
               f16_bits_to_f32(v.y >> 16)};
}

template <int DT>
__global__ __launch_bounds__(kCombineThreads) void k_attn_combine(const uint16_t* __restrict__ part_o,
                                                                  const float* __restrict__ part_ml, int n_splits,
                                                                  int d_v, void* __restrict__ out,
                                                                  float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;
  const int dv = 4 * (int)threadIdx.x;
  const bool act = dv < d_v;
  const int half = dv < d_v / 2 ? 0 : 1;  // d_v / 2 is a multiple of 4: the four columns share a half
  const float* ml = part_ml + bh * n_splits * kMlWords;
  const uint16_t* po = part_o + bh * n_splits * d_v + (act ? dv : 0);
  // the first kCombineBatch splits' partials and (max, sum, factor) triples, all requested before any is used:
  // indices past the last split are clamped to it (loads are never predicated, so that they stay in flight
  // together) and the duplicates are skipped below
  uint2 v[kCombineBatch];
  float mv[kCombineBatch], lv[kCombineBatch], fv[kCombineBatch];
#pragma unroll
  for (int u = 0; u < kCombineBatch; ++u) {
    const int i = u < n_splits ? u : n_splits - 1;
    v[u] = *reinterpret_cast<const uint2*>(po + (int64_t)i * d_v);
    mv[u] = ml[kMlWords * i];
    lv[u] = ml[kMlWords * i + 1];
    fv[u] = ml[kMlWords * i + 2 + half];
  }
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kCombineBatch; ++u) M = u < n_splits ? fmaxf(M, mv[u]) : M;
  for (int i = kCombineBatch; i < n_splits; ++i) M = fmaxf(M, ml[kMlWords * i]);
  float Ls = 0.f;
  f32x4 acc = f32x4{};
  if (M != -INFINITY) {
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const float w = u < n_splits ? exp2f(mv[u] - M) : 0.f;
      Ls += w * lv[u];
      if (w > 0.f) acc += (w * fv[u]) * f16x4_to_f32(v[u]);  // a split without rows has weight 0
    }
    for (int i0 = kCombineBatch; i0 < n_splits; i0 += kCombineBatch) {
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        const int i = i0 + u < n_splits ? i0 + u : n_splits - 1;
        v[u] = *reinterpret_cast<const uint2*>(po + (int64_t)i * d_v);
        mv[u] = ml[kMlWords * i];
        lv[u] = ml[kMlWords * i + 1];
        fv[u] = ml[kMlWords * i + 2 + half];
      }
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        const float w = i0 + u < n_splits ? exp2f(mv[u] - M) : 0.f;
        Ls += w * lv[u];
        if (w > 0.f) acc += (w * fv[u]) * f16x4_to_f32(v[u]);
      }
    }
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  if (act) {
    if constexpr (DT == 1) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16_bits(acc[0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16_bits(acc[2] * inv) | ((uint32_t)f32_to_bf16_bits(acc[3] * inv) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + bh * d_v + dv) = pk;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) store_out<DT>(out, bh * d_v + dv + r, acc[r] * inv);
    }
  }
  if (lse && threadIdx.x == 0) lse[bh] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

}  // namespace

AttnPlan attn_plan(int B, int H, int d_qk, int d_v, int64_t max_rows, int dtype, bool separate_v) {
  AttnPlan p{};
  p.mfma = dtype == 1 && !separate_v && d_qk == kRowElems && (d_v == 512 || d_v == 576) && H % 64 == 0;
  if (!p.mfma) {
    p.n_splits = 1;
    p.rows_per_split = 0;
    return p;
  }
  // splits and tiles per split for the largest read set; a smaller one is cut into the same number of parts,
  // each of at most ceil(tiles / splits) <= tps tiles
  const int64_t units = B > 0 ? (int64_t)B * (H / 64) : 1;
  const int64_t tiles = max_rows > 0 ? (max_rows + kTileRows - 1) / kTileRows : 1;
  int64_t splits = (256 + units - 1) / units;
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  int64_t tps = (tiles + splits - 1) / splits;
  if (tps > kMaxRowsPerSplit / kTileRows) {
    tps = kMaxRowsPerSplit / kTileRows;
    splits = (tiles + tps - 1) / tps;
  }
  const int64_t rps = tps * kTileRows;
  p.n_splits = (int)splits;
  p.rows_per_split = (int)rps;
  return p;
}

// Per (query, head, split): d_v fp16 partial values, then kMlWords floats (max, sum, one factor per column half).
size_t attn_workspace_bytes(const AttnPlan& p, int B, int H, int d_v) {
  if (!p.mfma || p.n_splits <= 1) return 0;
  return (size_t)B * H * p.n_splits * ((size_t)d_v * sizeof(uint16_t) + kMlWords * sizeof(float));
}

// attn_plan never uses more than max(ceil(256 / units), ceil(tiles / (kMaxRowsPerSplit / kTileRows))) splits,
// which grows with the tile count, so this bound covers every call whose read sets are bounded by max_rows.
size_t attn_workspace_bound(int B, int H, int d_qk, int d_v, int64_t max_rows, int dtype) {
  const AttnPlan p = attn_plan(B, H, d_qk, d_v, max_rows, dtype, false);
  if (!p.mfma) return 0;
  const int64_t units = B > 0 ? (int64_t)B * (H / 64) : 1;
  const int64_t tiles = max_rows > 0 ? (max_rows + kTileRows - 1) / kTileRows : 1;
  const int64_t s1 = (256 + units - 1) / units;
  const int64_t s2 = (tiles + kMaxRowsPerSplit / kTileRows - 1) / (kMaxRowsPerSplit / kTileRows);
  const int64_t s = s1 > s2 ? s1 : s2;
  return (size_t)B * H * s * ((size_t)d_v * sizeof(uint16_t) + kMlWords * sizeof(float));
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& p, void* ws, hipStream_t st) {
  if (!p.mfma) {
    if (a.d_v > kGenMaxDv) return hipErrorInvalidValue;
    const size_t lds = sizeof(float) * ((size_t)a.d_qk + 2 * kGenThreads);
    dim3 grid((unsigned)a.H, (unsigned)a.B);
    if (a.dtype == 0)
      SA_LAUNCH(k_attn_generic<0>, grid, dim3(kGenThreads), lds, st, a.q, a.kv, a.v, a.kv_ld, a.v_ld, a.L,
                         a.H, a.d_qk, a.d_v, a.t, a.idx, a.idx_ld, a.n_sel, a.n_sink, a.n_window, a.scale, a.out,
                         a.lse);
    else
      SA_LAUNCH(k_attn_generic<1>, grid, dim3(kGenThreads), lds, st, a.q, a.kv, a.v, a.kv_ld, a.v_ld, a.L,
                         a.H, a.d_qk, a.d_v, a.t, a.idx, a.idx_ld, a.n_sel, a.n_sink, a.n_window, a.scale, a.out,
                         a.lse);
    return hipGetLastError();
  }
  if ((uint64_t)a.kv_ld * 2 > 0xffffffffull) return hipErrorInvalidValue;  // row byte stride is a 32-bit multiplier
  uint16_t* part_o = reinterpret_cast<uint16_t*>(ws);
  float* part_ml = part_o ? reinterpret_cast<float*>(part_o + (size_t)a.B * a.H * p.n_splits * a.d_v) : nullptr;
  const int HG = a.H / 64;
  const int n_units = a.B * p.n_splits;
  dim3 grid((unsigned)((n_units + 7) / 8 * 8 * HG));
  const float sl2 = a.scale * kLog2e;
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  if (a.d_v == 576)
    SA_LAUNCH(k_attn_mfma<576>, grid, dim3(256), 0, st, q, kv, a.kv_ld, a.L, a.H, a.t, a.idx, a.idx_ld,
                       a.n_sel, a.n_sink, a.n_window, sl2, p.n_splits, n_units, part_o, part_ml, out,
                       a.lse);
  else
    SA_LAUNCH(k_attn_mfma<512>, grid, dim3(256), 0, st, q, kv, a.kv_ld, a.L, a.H, a.t, a.idx, a.idx_ld,
                       a.n_sel, a.n_sink, a.n_window, sl2, p.n_splits, n_units, part_o, part_ml, out,
                       a.lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  SA_LAUNCH(k_attn_combine<1>, dim3((unsigned)(a.B * a.H)), dim3(kCombineThreads), 0, st, part_o, part_ml,
                     p.n_splits, a.d_v, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace sa
