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
//    (4 waves x 16 heads). Rows are gathered 32 at a time into LDS by asynchronous DMA (72 x 16-byte chunks per
//    1152-byte row), S^T = K Q^T runs on 16x16x32 MFMA with the query heads register-resident, the online
//    softmax runs in the log2 domain, and O^T = V^T P^T takes V through LDS transpose reads so that P never
//    leaves registers. Rows are split over workgroups; k_attn_combine merges the splits by their (max, sum).
#include <math.h>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
constexpr int kNBuf = 4;                                 // LDS tiles: up to 3 in flight while one is consumed
constexpr int kMaxRowsPerSplit = 512;
constexpr int kQSteps = kRowElems / 32;                  // 18 k-steps of 32 dims
constexpr float kRescaleSlack = 8.f;                     // log2 headroom before the running max is raised

// chunk c of row n lives at chunk slot c ^ (n & 7) (the XOR stays inside the aligned group of 8 chunks)
__device__ __forceinline__ int chunk_slot(int n, int c) { return c ^ (n & 7); }

// Grid: 1-D, block id = group + n_groups * split with group = (query, 64-head group). When n_groups is a multiple
// of 8, every split of a group (and the combine blocks of its heads) runs on the same XCD and shares its L2.
template <int DV>
__global__ __launch_bounds__(256) void k_attn_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                                   int64_t kv_ld, int64_t L, int H, const int32_t* __restrict__ t,
                                                   const int32_t* __restrict__ idx, int idx_ld,
                                                   const int32_t* __restrict__ n_sel, int n_sink, int n_window,
                                                   float scale_log2, int rows_per_split, int n_splits,
                                                   float* __restrict__ part_o, float* __restrict__ part_ml,
                                                   uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int NT = DV / 16;  // 16-wide output tiles per head group
  __shared__ __attribute__((aligned(1024))) char tiles[kNBuf][kTileBytes];
  __shared__ int32_t pos_s[kMaxRowsPerSplit];
  const int n_groups = (int)gridDim.x / n_splits;
  const int group = (int)blockIdx.x % n_groups, split = (int)blockIdx.x / n_groups;
  const int HG = H / 64;
  const int b = group / HG, hg = group % HG;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int g = lane >> 4;         // lane group 0..3
  const int li = lane & 15;        // lane in group
  const int h = 64 * hg + 16 * wave + li;  // the head this lane works for
  const int64_t bh = (int64_t)b * H + h;

  // Q^T fragments (B operand): head h, dims 32 ks + 8 g .. +8
  bf16x8 qf[kQSteps];
#pragma unroll
  for (int ks = 0; ks < kQSteps; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(q + bh * kRowElems + 32 * ks + 8 * g);

  const RowList R = make_rows(b, L, t, idx, idx_ld, n_sel, n_sink, n_window);
  const int n_rows = R.count();
  const int r_begin = split * rows_per_split;
  int r_end = r_begin + rows_per_split;
  r_end = r_end < n_rows ? r_end : n_rows;
  const int n_my = r_end - r_begin;

  if (n_my <= 0) {
    if (n_splits == 1) {
      for (int i = g; i < DV; i += 4) out[bh * DV + i] = 0;
      if (lse && g == 0) lse[bh] = -INFINITY;
    } else if (g == 0) {
      part_ml[(bh * n_splits + split) * 2 + 0] = -INFINITY;
      part_ml[(bh * n_splits + split) * 2 + 1] = 0.f;
    }
    return;
  }
  const int n_tiles = (n_my + kTileRows - 1) / kTileRows;
  for (int r = tid; r < n_tiles * kTileRows; r += 256) pos_s[r] = r < n_my ? R.pos(r_begin + r) : 0;
  __syncthreads();

  const char* kvb = reinterpret_cast<const char*>(kv);
  const int64_t ld_bytes = kv_ld * 2;
  auto issue = [&](int tile, int buf) {
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const int slot = (wave * kDmaPerWave + j) * 64 + lane;
      const int n = slot / kRowChunks;
      const int c = chunk_slot(n, slot % kRowChunks);
      const int s = pos_s[tile * kTileRows + n];
      dma16(kvb + (int64_t)s * ld_bytes + c * 16, &tiles[buf][(wave * kDmaPerWave + j) * 1024]);
    }
  };

  f32x4 o[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) o[i] = f32x4{};
  float m_use = -INFINITY, l_run = 0.f;  // exponents are taken relative to m_use (log2 domain)

  // Per-lane LDS offsets. K fragment of row n = 16 mt + li, chunk 4 ks + g sits at
  //   n * 1152 + 16 * ((4 ks + g) ^ (n & 7)) = li * 1152 + kofs[ks & 1] + 128 (ks >> 1) + 18432 mt,
  // and the transpose-read source of row r0 (+16), chunk 2 nt + h at r0 * 1152 + vofs[nt & 3] + 128 (nt >> 2) (+18432),
  // so every unrolled access is a base register plus a compile-time offset.
  const int mk = li & 7;
  const int kofs0 = li * kRowBytes + 16 * (g ^ mk);
  const int kofs1 = li * kRowBytes + 16 * ((g ^ mk) ^ 4);
  const int row0 = 4 * g + (li >> 2);
  const int mv = row0 & 7;
  const int hsel = (li & 3) >> 1;
  int vofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vofs[j] = row0 * kRowBytes + 16 * ((2 * j + hsel) ^ mv) + 8 * (li & 1);

  wait_vmem();  // the Q fragments are in registers before the tile copies start counting
  const int n_pre = n_tiles < kNBuf - 1 ? n_tiles : kNBuf - 1;
  for (int p = 0; p < n_pre; ++p) issue(p, p);
  for (int tile = 0; tile < n_tiles; ++tile) {
    // wait for this tile's copies; the (at most two) later tiles may stay in flight
    const int newer = n_tiles - 1 - tile;
    if (newer >= 2) wait_vmem_below<2 * kDmaPerWave>();
    else if (newer == 1) wait_vmem_below<kDmaPerWave>();
    else wait_vmem_below<0>();
    lds_barrier();
    if (tile + kNBuf - 1 < n_tiles) issue(tile + kNBuf - 1, (tile + kNBuf - 1) % kNBuf);
    const char* tb = tiles[tile % kNBuf];

    // S^T (rows x heads): two 16-row halves
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks) {
        const char* kp = tb + ((ks & 1) ? kofs1 : kofs0) + 128 * (ks >> 1) + 18432 * mt;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kp);
        s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[mt], 0, 0, 0);
      }
    }
    // this lane holds head h at tile rows 16 mt + 4 g + r
    const int valid = n_my - tile * kTileRows;
    float x[2][4];
    float mt_max = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mt + 4 * g + r;
        x[mt][r] = row < valid ? s[mt][r] * scale_log2 : -INFINITY;
        mt_max = fmaxf(mt_max, x[mt][r]);
      }
    mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 16, kWave));
    mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 32, kWave));
    // raise the reference only when this tile would exceed it by more than 2^kRescaleSlack
    const bool raise = mt_max > m_use + kRescaleSlack;
    if (__any(raise)) {
      const float m_new = raise ? mt_max : m_use;
      const float alpha = exp2f(m_use - m_new);  // 1 where not raised, 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] = o[nt] * alpha;
      m_use = m_new;
    }
    bf16x8 pf;
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(x[mt][r] - m_use);
        psum += p;
        pf[4 * mt + r] = (__bf16)p;
      }
    l_run += psum;

    // O^T (dv x heads) += V^T P^T; V^T fragments through LDS transpose reads.
    // A operand slots e = 0..3 -> tile rows 4 g + e, e = 4..7 -> rows 16 + 4 g + (e - 4), matching pf.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const char* vp = tb + vofs[nt & 3] + 128 * (nt >> 2);
      const i16x4 v0 = lds_read_tr16(vp);
      const i16x4 v1 = lds_read_tr16(vp + 18432);
      // whole-vector shuffle + bit_cast (a bit_cast of a single ext-vector element is not used here: clang lowers
      // it to element 0 for every index)
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[nt], 0, 0, 0);
    }
  }

  // lanes h, h^16, h^32, h^48 hold disjoint rows of head h: reduce the sum
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (n_splits == 1) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint16_t* dst = out + bh * DV + 16 * nt + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r] = f32_to_bf16_bits(o[nt][r] * inv);
    }
    if (lse && g == 0) lse[bh] = (m_use + log2f(l_run)) * kLn2;
  } else {
    float* dst = part_o + (bh * n_splits + split) * DV;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4*>(dst + 16 * nt + 4 * g) = o[nt];
    if (g == 0) {
      part_ml[(bh * n_splits + split) * 2 + 0] = m_use;
      part_ml[(bh * n_splits + split) * 2 + 1] = l_run;
    }
  }
}

// Exact merge of the splits of one (query, head): o = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i.
// Block id = group + n_groups * j, head = 64 hg + j, matching the XCD of the attention blocks of that group.
template <int DT>
__global__ __launch_bounds__(64) void k_attn_combine(const float* __restrict__ part_o,
                                                     const float* __restrict__ part_ml, int n_splits, int n_groups,
                                                     int H, int d_v, void* __restrict__ out, float* __restrict__ lse) {
  const int group = (int)blockIdx.x % n_groups, j = (int)blockIdx.x / n_groups;
  const int HG = H / 64;
  const int64_t bh = (int64_t)(group / HG) * H + 64 * (group % HG) + j;
  const float* ml = part_ml + bh * n_splits * 2;
  float M = -INFINITY;
  for (int i = 0; i < n_splits; ++i) M = fmaxf(M, ml[2 * i]);
  float Ls = 0.f;
  if (M != -INFINITY)
    for (int i = 0; i < n_splits; ++i) Ls += exp2f(ml[2 * i] - M) * ml[2 * i + 1];
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  for (int dv = 4 * threadIdx.x; dv < d_v; dv += 4 * blockDim.x) {
    f32x4 acc = f32x4{};
    if (M != -INFINITY)
      for (int i = 0; i < n_splits; ++i) {
        const float wgt = exp2f(ml[2 * i] - M);
        if (wgt != 0.f) acc += wgt * *reinterpret_cast<const f32x4*>(part_o + (bh * n_splits + i) * d_v + dv);
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) store_out<DT>(out, bh * d_v + dv + r, acc[r] * inv);
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
  const int64_t units = B > 0 ? (int64_t)B * (H / 64) : 1;
  const int64_t rows = max_rows > 0 ? max_rows : 1;
  int64_t splits = (256 + units - 1) / units;
  const int64_t max_splits = (rows + kTileRows - 1) / kTileRows;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t rps = (rows + splits - 1) / splits;
  rps = (rps + kTileRows - 1) / kTileRows * kTileRows;
  if (rps > kMaxRowsPerSplit) rps = kMaxRowsPerSplit;
  splits = (rows + rps - 1) / rps;
  p.n_splits = (int)splits;
  p.rows_per_split = (int)rps;
  return p;
}

size_t attn_workspace_bytes(const AttnPlan& p, int B, int H, int d_v) {
  if (!p.mfma || p.n_splits <= 1) return 0;
  return (size_t)B * H * p.n_splits * ((size_t)d_v + 2) * sizeof(float);
}

// attn_plan never uses more than max(ceil(256 / units), ceil(rows / kMaxRowsPerSplit)) splits, which grows with
// rows, so this bound covers every call whose read sets are bounded by max_rows.
size_t attn_workspace_bound(int B, int H, int d_qk, int d_v, int64_t max_rows, int dtype) {
  const AttnPlan p = attn_plan(B, H, d_qk, d_v, max_rows, dtype, false);
  if (!p.mfma) return 0;
  const int64_t units = B > 0 ? (int64_t)B * (H / 64) : 1;
  const int64_t rows = max_rows > 0 ? max_rows : 1;
  const int64_t s1 = (256 + units - 1) / units;
  const int64_t s2 = (rows + kMaxRowsPerSplit - 1) / kMaxRowsPerSplit;
  const int64_t s = s1 > s2 ? s1 : s2;
  return (size_t)B * H * s * ((size_t)d_v + 2) * sizeof(float);
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& p, void* ws, hipStream_t st) {
  if (!p.mfma) {
    if (a.d_v > kGenMaxDv) return hipErrorInvalidValue;
    const size_t lds = sizeof(float) * ((size_t)a.d_qk + 2 * kGenThreads);
    dim3 grid((unsigned)a.H, (unsigned)a.B);
    if (a.dtype == 0)
      hipLaunchKernelGGL(k_attn_generic<0>, grid, dim3(kGenThreads), lds, st, a.q, a.kv, a.v, a.kv_ld, a.v_ld, a.L,
                         a.H, a.d_qk, a.d_v, a.t, a.idx, a.idx_ld, a.n_sel, a.n_sink, a.n_window, a.scale, a.out,
                         a.lse);
    else
      hipLaunchKernelGGL(k_attn_generic<1>, grid, dim3(kGenThreads), lds, st, a.q, a.kv, a.v, a.kv_ld, a.v_ld, a.L,
                         a.H, a.d_qk, a.d_v, a.t, a.idx, a.idx_ld, a.n_sel, a.n_sink, a.n_window, a.scale, a.out,
                         a.lse);
    return hipGetLastError();
  }
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_ml = part_o ? part_o + (size_t)a.B * a.H * p.n_splits * a.d_v : nullptr;
  const int n_groups = a.B * (a.H / 64);
  dim3 grid((unsigned)(n_groups * p.n_splits));
  const float sl2 = a.scale * kLog2e;
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  if (a.d_v == 576)
    hipLaunchKernelGGL(k_attn_mfma<576>, grid, dim3(256), 0, st, q, kv, a.kv_ld, a.L, a.H, a.t, a.idx, a.idx_ld,
                       a.n_sel, a.n_sink, a.n_window, sl2, p.rows_per_split, p.n_splits, part_o, part_ml, out, a.lse);
  else
    hipLaunchKernelGGL(k_attn_mfma<512>, grid, dim3(256), 0, st, q, kv, a.kv_ld, a.L, a.H, a.t, a.idx, a.idx_ld,
                       a.n_sel, a.n_sink, a.n_window, sl2, p.rows_per_split, p.n_splits, part_o, part_ml, out, a.lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  hipLaunchKernelGGL(k_attn_combine<1>, dim3((unsigned)(a.B * a.H)), dim3(64), 0, st, part_o, part_ml, p.n_splits,
                     n_groups, a.H, a.d_v, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace sa
