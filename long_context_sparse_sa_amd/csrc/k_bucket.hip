// Bucket directory and Flat bucket search of Latent Sparse Attention (LSA eight-entry page, section 2: index keys
// are grouped into buckets that keep a representative vector and their member positions; the Flat variant compares
// the query with every representative; the chosen buckets expand to their positions, and sink and window positions
// are read in addition).
//
// Build (once per cache):
//   per-chunk bucket histograms -> column scan (each bucket's count in earlier chunks, and its total) -> offsets
//   (exclusive scan of the totals) -> stable scatter (positions in ascending order within each bucket) ->
//   representatives (fp64 sums, rounded once to fp32).
// Select (per step):
//   four lanes per bucket score q . rep for every query and write one key per (query, bucket) -> one workgroup per
//   query chooses the exact top-b (ties to the lower bucket id) and expands the chosen buckets' members inside
//   [sink end, window start): all members are fetched in one round trip, compacted, and sorted ascending by
//   binning the positions (a bitonic sort when the bins crowd).
#include <mutex>

#include "sa_device.h"
#include "sa_internal.h"
#include "sa_wave_select.h"

namespace sa {
namespace {

constexpr int kChunkMin = 4096;
constexpr int64_t kTableBudget = 1 << 24;  // entries of the (chunk x bucket) table
constexpr int kMaxExpand = 16384;
constexpr int kBinMax = 16;  // entries per position bin sorted in registers by the expansion
constexpr int kFastCand = 256;  // candidates ranked directly when the first digit pass leaves at most this many

// Ascending sort of the n <= N entries at src into dst by an odd-even transposition network in registers.
template <int N>
__device__ __forceinline__ void sort_bin(const int32_t* src, int n, int32_t* dst) {
  int32_t e[N];
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = i < n ? src[i] : 0x7FFFFFFF;
#pragma unroll
  for (int r = 0; r < N; ++r)
#pragma unroll
    for (int i = r & 1; i + 1 < N; i += 2) {
      const int32_t x = e[i], y = e[i + 1];
      e[i] = x < y ? x : y;
      e[i + 1] = x < y ? y : x;
    }
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < n) dst[i] = e[i];
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// Single-workgroup exclusive scan: offsets[c] = sum_{c' < c} counts[c'], offsets[nb] = total. Each thread takes a
// contiguous run of counts (up to kRun of them held in registers, all loaded before any is used), the run sums are
// scanned in LDS, and each thread writes its run's offsets from the registers.
constexpr int kRun = 32;

__global__ __launch_bounds__(1024) void k_offsets(const int32_t* __restrict__ counts, int nb, int32_t* __restrict__ offsets) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (nb + 1023) / 1024;
  const int lo = tid * per, hi = lo + per < nb ? lo + per : nb;
  int32_t v[kRun];
  int32_t s = 0;
  if (per <= kRun) {
#pragma unroll
    for (int u = 0; u < kRun; ++u) v[u] = lo + u < hi ? counts[lo + u] : 0;
#pragma unroll
    for (int u = 0; u < kRun; ++u) s += v[u];
  } else {
    for (int i = lo; i < hi; ++i) s += counts[i];
  }
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int32_t run = tid > 0 ? part[tid - 1] : 0;
  if (per <= kRun) {
#pragma unroll
    for (int u = 0; u < kRun; ++u)
      if (lo + u < hi) {
        offsets[lo + u] = run;
        run += v[u];
      }
  } else {
    for (int i = lo; i < hi; ++i) {
      offsets[i] = run;
      run += counts[i];
    }
  }
  if (tid == 1023) offsets[nb] = part[1023];
}

// Per-chunk bucket histogram: table[chunk][c] = number of positions of the chunk in bucket c. With nb <= kLdsBuckets
// the histogram is built with LDS atomics and the row is written whole (no clearing needed); otherwise with global
// atomics into a row the caller zeroed.
constexpr int kLdsBuckets = 16384;

template <bool LDS>
__global__ __launch_bounds__(256) void k_chunk_hist(const int32_t* __restrict__ assign, int64_t L, int64_t chunk, int nb,
                                                    int32_t* __restrict__ table) {
  const int64_t c = blockIdx.x;
  const int64_t lo = c * chunk, hi = lo + chunk < L ? lo + chunk : L;
  int32_t* row = table + c * nb;
  if constexpr (LDS) {
    __shared__ int32_t hist[kLdsBuckets];
    for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    constexpr int kStage = 16;
    for (int64_t i0 = lo; i0 < hi; i0 += kStage * (int64_t)blockDim.x) {
      int32_t v[kStage];
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int64_t i = i0 + u * (int64_t)blockDim.x + threadIdx.x;
        v[u] = i < hi ? assign[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < kStage; ++u)
        if (v[u] >= 0) atomicAdd(&hist[v[u]], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += blockDim.x) row[i] = hist[i];
  } else {
    for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x) atomicAdd(&row[assign[i]], 1);
  }
}

// Column scan, one thread per bucket: table[chunk][c] <- the bucket's count in earlier chunks (exclusive), and
// counts[c] <- its total. Sixteen rows are loaded before any is used, so that the loads overlap.
__global__ __launch_bounds__(256) void k_chunk_scan(int nb, int64_t n_chunks, int32_t* __restrict__ table,
                                                    int32_t* __restrict__ counts) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nb) return;
  constexpr int kBatch = 16;
  int32_t run = 0;
  for (int64_t ch0 = 0; ch0 < n_chunks; ch0 += kBatch) {
    int32_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = ch0 + u < n_chunks ? table[(ch0 + u) * nb + c] : 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (ch0 + u < n_chunks) table[(ch0 + u) * nb + c] = run;
      run += v[u];
    }
  }
  counts[c] = run;
}

constexpr int kScatterStage = 4096;  // positions of a chunk staged in LDS (the LDS path requires chunk <= this)

// Stable scatter: one workgroup per chunk. With nb <= kLdsBuckets the chunk's cursors (offsets[c] + the bucket's
// count in earlier chunks) sit in LDS; one wave then walks the chunk in ascending position order, 64 positions at a
// time: a lane's slot in its bucket is the cursor plus the number of lower lanes with the same bucket, and the
// highest such lane advances the cursor. Otherwise the cursors stay in the table row (global memory).
template <bool LDS>
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ assign, int64_t L, int64_t chunk, int nb,
                                                 const int32_t* __restrict__ offsets, int32_t* __restrict__ table,
                                                 int32_t* __restrict__ members) {
  const int64_t c = blockIdx.x;
  const int64_t lo = c * chunk, hi = lo + chunk < L ? lo + chunk : L;
  int32_t* row = table + c * nb;
  __shared__ int32_t cur_lds[LDS ? kLdsBuckets : 1];
  __shared__ int32_t asg[LDS ? kScatterStage : 1];  // the chunk's assignments, so the ordered walk never waits on HBM
  __shared__ int32_t tag[LDS ? kLdsBuckets : 1];    // per-bucket scratch of the duplicate test below
  if constexpr (LDS) {
    // staged sixteen entries per thread at a time: every load of a batch is in flight before any is stored
    constexpr int kStage = 16;
    const int n_pos = (int)(hi - lo);
    for (int i0 = 0; i0 < nb; i0 += kStage * (int)blockDim.x) {
      int32_t v[kStage];
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int i = i0 + u * (int)blockDim.x + (int)threadIdx.x;
        const int ic = i < nb ? i : nb - 1;
        v[u] = offsets[ic] + row[ic];
      }
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int i = i0 + u * (int)blockDim.x + (int)threadIdx.x;
        if (i < nb) cur_lds[i] = v[u];
      }
    }
    for (int i0 = 0; i0 < n_pos; i0 += kStage * (int)blockDim.x) {
      int32_t v[kStage];
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int i = i0 + u * (int)blockDim.x + (int)threadIdx.x;
        v[u] = assign[lo + (i < n_pos ? i : n_pos - 1)];
      }
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int i = i0 + u * (int)blockDim.x + (int)threadIdx.x;
        if (i < n_pos) asg[i] = v[u];
      }
    }
    __syncthreads();
  } else {
    for (int i = threadIdx.x; i < nb; i += blockDim.x) row[i] += offsets[i];
    __syncthreads();
  }
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const uint64_t below = (1ull << lane) - 1ull;
  // (the cursors are addressed through the arrays themselves, not a pointer that may point to either memory: a
  // generic pointer makes every cursor access a flat instruction that waits for the member stores)
  for (int64_t base = lo; base < hi; base += kWave) {
    const int64_t s = base + lane;
    const bool valid = s < hi;
    const int a = valid ? (LDS ? asg[s - lo] : assign[s]) : -1;
    // rank among the lanes of this step with the same bucket: a lane whose bucket no other lane holds has rank 0
    // and is the last. Duplicates are found by each lane writing its id to its bucket's tag and reading it back
    // (one writer per bucket wins); only the buckets of the lanes that lost are then matched lane by lane.
    int rank = 0;
    bool last = valid;
    uint64_t dup;
    if constexpr (LDS) {
      if (valid) tag[a] = lane;
      __builtin_amdgcn_wave_barrier();
      const int w = valid ? tag[a] : lane;
      dup = ballot(w != lane);
    } else {
      dup = ballot(valid);  // without the LDS tags every bucket of the step is matched
    }
    while (dup) {
      const int leader = __builtin_ctzll(dup);
      const int v = __builtin_amdgcn_readlane(a, leader);
      const bool same = valid && a == v;
      const uint64_t m = ballot(same);
      if (same) {
        rank = __popcll(m & below);
        last = (m >> lane) == 1ull;
      }
      dup &= ~m;
    }
    int32_t start = 0;
    if (valid) start = LDS ? cur_lds[a] : row[a];
    if (valid) members[start + rank] = (int32_t)s;
    if constexpr (!LDS) wait_vmem();
    __builtin_amdgcn_wave_barrier();
    if (last) {
      if constexpr (LDS) cur_lds[a] = start + rank + 1;
      else row[a] = start + rank + 1;
    }
    if constexpr (!LDS) wait_vmem();
    __builtin_amdgcn_wave_barrier();
  }
}

// One wave per bucket: rep = (float)(sum of member keys in fp64 / count). Each lane owns two dims of a 128-dim
// slice (one 4-byte load per bf16 member row, two for fp32). The member positions come 64 at a time in one load
// and are broadcast with readlane, so sixteen member rows are requested before any is summed, none waiting on an
// index load.
template <int KT>
__global__ __launch_bounds__(256) void k_reps(const void* __restrict__ k, int64_t k_ld, int d,
                                              const int32_t* __restrict__ offsets, const int32_t* __restrict__ members,
                                              int nb, float* __restrict__ reps) {
  const int bucket = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = lane_id();
  if (bucket >= nb) return;
  const int lo = offsets[bucket], hi = offsets[bucket + 1];
  constexpr int kBatch = 16;
  for (int x0 = 0; x0 < d; x0 += 2 * kWave) {
    const int x = x0 + 2 * lane;
    const bool has0 = x < d, has1 = x + 1 < d;
    double s0 = 0.0, s1 = 0.0;
    for (int i0 = lo; i0 < hi; i0 += kWave) {
      const int nm = hi - i0 < kWave ? hi - i0 : kWave;
      const int mi = members[i0 + (lane < nm ? lane : 0)];
      for (int u0 = 0; u0 < nm; u0 += kBatch) {
        float a0[kBatch], a1[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int m = __builtin_amdgcn_readlane(mi, u0 + u < nm ? u0 + u : 0);  // clamped; not summed
          const int64_t e = (int64_t)m * k_ld + (has0 ? x : 0);
          if constexpr (KT == 1) {
            if (has1 && ((k_ld | x) & 1) == 0) {  // both bf16 of the pair in one aligned 4-byte load
              const uint32_t pr = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(k) + e);
              a0[u] = __uint_as_float(pr << 16);
              a1[u] = __uint_as_float(pr & 0xFFFF0000u);
            } else {
              a0[u] = load_elem<KT>(k, e);
              a1[u] = has1 ? load_elem<KT>(k, e + 1) : 0.f;
            }
          } else {
            a0[u] = load_elem<KT>(k, e);
            a1[u] = has1 ? load_elem<KT>(k, e + 1) : 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (u0 + u < nm) {
            s0 += (double)a0[u];
            s1 += (double)a1[u];
          }
      }
    }
    const double n = (double)(hi - lo);
    if (has0) reps[(int64_t)bucket * d + x] = hi > lo ? (float)(s0 / n) : 0.f;
    if (has1) reps[(int64_t)bucket * d + x + 1] = hi > lo ? (float)(s1 / n) : 0.f;
  }
}

// Scores every query against every representative (fp32 dot) and writes the slot keys[b * nb + bucket]: the
// order-preserving key of the score for a non-empty bucket, 0 (empty slot) otherwise.
template <int QT>
__global__ __launch_bounds__(256) void k_bucket_scores(const void* __restrict__ q, int B, int d,
                                                       const float* __restrict__ reps,
                                                       const int32_t* __restrict__ offsets, int nb,
                                                       uint32_t* __restrict__ keys) {
  extern __shared__ __attribute__((aligned(16))) float qs[];  // [B * d]
  // four lanes per bucket, sixteen buckets per wave: each lane takes every fourth group of four dims of its
  // bucket's representative, keeps it for all queries, and the four partial dot products meet in two lane swaps
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int qtr = lane & 3;
  const int bucket = (blockIdx.x * 4 + wave) * 16 + (lane >> 2);
  const bool in = bucket < nb;
  const int bc = in ? bucket : 0;  // loads clamped to bucket 0 rather than predicated (no branch around them)
  const int32_t o0 = offsets[bc], o1 = offsets[bc + 1];
  const float* r = reps + (int64_t)bc * d;
  // for d a multiple of 16 up to 16 * kRepRegs the lane's slice (dims 16 c + 4 qtr .. + 3) is loaded into registers
  // here, before the queries are staged, so that the two loads overlap
  constexpr int kRepRegs = 16;
  const bool in_regs = (d & 15) == 0 && d <= 16 * kRepRegs;
  float4 rv[kRepRegs];
  if (in_regs) {  // uniform; slices past d repeat the first one (never used), so every load stays in the row
#pragma unroll
    for (int c = 0; c < kRepRegs; ++c)
      rv[c] = *reinterpret_cast<const float4*>(r + (16 * c < d ? 16 * c + 4 * qtr : 4 * qtr));
  }
  // the queries into LDS: up to kStageRegs elements per thread are all loaded before any is stored, so their
  // latencies overlap
  constexpr int kStageRegs = 16;
  const int n_q = B * d;
  if (n_q <= kStageRegs * (int)blockDim.x) {
    float v[kStageRegs];
#pragma unroll
    for (int m = 0; m < kStageRegs; ++m) {
      const int i = threadIdx.x + m * blockDim.x;
      v[m] = load_elem<QT>(q, i < n_q ? i : n_q - 1);  // clamped, not predicated: no branch, no wait per load
    }
#pragma unroll
    for (int m = 0; m < kStageRegs; ++m) {
      const int i = threadIdx.x + m * blockDim.x;
      if (i < n_q) qs[i] = v[m];
    }
  } else {
    for (int i = threadIdx.x; i < n_q; i += blockDim.x) qs[i] = load_elem<QT>(q, i);
  }
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += 8) {
    float acc[8];
    const float* qrow[8];  // rows past the last query repeat it; their sums are not stored (no branches inside)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc[u] = 0.f;
      qrow[u] = qs + (b0 + u < B ? b0 + u : B - 1) * d;
    }
    if (in_regs) {
#pragma unroll
      for (int c = 0; c < kRepRegs; ++c) {
        if (16 * c < d) {
          float4 qv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) qv[u] = *reinterpret_cast<const float4*>(qrow[u] + 16 * c + 4 * qtr);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            acc[u] = fmaf(qv[u].x, rv[c].x, acc[u]);
            acc[u] = fmaf(qv[u].y, rv[c].y, acc[u]);
            acc[u] = fmaf(qv[u].z, rv[c].z, acc[u]);
            acc[u] = fmaf(qv[u].w, rv[c].w, acc[u]);
          }
        }
      }
    } else if ((d & 3) == 0) {
#pragma unroll 4
      for (int x = 4 * qtr; x < d; x += 16) {
        const float4 rv = *reinterpret_cast<const float4*>(r + x);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float4 qv = *reinterpret_cast<const float4*>(qrow[u] + x);
          acc[u] = fmaf(qv.x, rv.x, acc[u]);
          acc[u] = fmaf(qv.y, rv.y, acc[u]);
          acc[u] = fmaf(qv.z, rv.z, acc[u]);
          acc[u] = fmaf(qv.w, rv.w, acc[u]);
        }
      }
    } else {
#pragma unroll 4
      for (int x = qtr; x < d; x += 4) {
        const float rv = r[x];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = fmaf(qrow[u][x], rv, acc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc[u] = quad_sum(acc[u]);
    }
    if (qtr == 0 && in) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b0 + u < B) keys[(int64_t)(b0 + u) * nb + bucket] = o1 > o0 ? score_key(acc[u]) : 0u;
    }
  }
}

// Tree search, one level down: for query b and its kept node kept[b, i] (i < n_kept[b]), scores every child
// (the next level's nodes child_off[node] .. child_off[node + 1] - 1) and writes its slot key into keys[b * n_next
// + child] (0 for a child without members or children); slots of children of unkept nodes keep their (zero) value.
// Four lanes per child; each lane sums the same dims in the same order as k_bucket_scores (dims 16 c + 4 quarter
// .. + 3, ascending c, then two lane swaps), so a node's score is bit-identical to the Flat search's.
template <int QT>
__global__ __launch_bounds__(256) void k_tree_children(const void* __restrict__ q, int d,
                                                       const int32_t* __restrict__ kept, int keep_ld,
                                                       const int32_t* __restrict__ n_kept,
                                                       const int32_t* __restrict__ child_off,
                                                       const float* __restrict__ reps,
                                                       const int32_t* __restrict__ offsets, int n_next,
                                                       uint32_t* __restrict__ keys) {
  extern __shared__ __attribute__((aligned(16))) float qrow[];  // [d]
  const int b = blockIdx.y, i = blockIdx.x;
  int nk = n_kept[b];
  nk = nk < 0 ? 0 : (nk > keep_ld ? keep_ld : nk);
  if (i >= nk) return;
  const int node = kept[(int64_t)b * keep_ld + i];
  const int c0 = child_off[node], c1 = child_off[node + 1];
  for (int x = threadIdx.x; x < d; x += blockDim.x) qrow[x] = load_elem<QT>(q, (int64_t)b * d + x);
  __syncthreads();
  const int qtr = threadIdx.x & 3;
  for (int base = c0; base < c1; base += (int)blockDim.x / 4) {
    const int child = base + (int)threadIdx.x / 4;
    const bool in = child < c1;
    const int cc = in ? child : c0;  // every lane of a quad takes part in the swaps below
    const float* r = reps + (int64_t)cc * d;
    float acc = 0.f;
    if ((d & 3) == 0) {
      for (int x = 4 * qtr; x < d; x += 16) {
        const float4 rv = *reinterpret_cast<const float4*>(r + x);
        const float4 qv = *reinterpret_cast<const float4*>(qrow + x);
        acc = fmaf(qv.x, rv.x, acc);
        acc = fmaf(qv.y, rv.y, acc);
        acc = fmaf(qv.z, rv.z, acc);
        acc = fmaf(qv.w, rv.w, acc);
      }
    } else {
      for (int x = qtr; x < d; x += 4) acc = fmaf(qrow[x], r[x], acc);
    }
    acc = quad_sum(acc);
    if (qtr == 0 && in)
      keys[(int64_t)b * n_next + child] = offsets[child + 1] > offsets[child] ? score_key(acc) : 0u;
  }
}

// Expansion: the kept positions of a chosen bucket form the sub-range of its (ascending) member list inside
// [lo, hi) with lo = end of the sink and hi = start of the window (which also excludes positions after t).
__device__ __forceinline__ int lower_bound(const int32_t* a, int n, int32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// One workgroup per query: the choice of its top_b buckets, then their expansion.
//
// Choice: the query's slot keys (16 per thread in registers; a longer row is re-read per pass) go through an LDS
// histogram of their top 11 bits, which gives the bin of the top_b-th largest non-empty slot. When that bin and
// the bins above it hold at most kFastCand slots (the usual case: the top of the score distribution is thin),
// those candidates are collected and each one's rank in (score desc, id asc) order is counted directly. Otherwise
// two more passes (digits 20..10 and 9..0) find kstar, the top_b-th largest key; chosen are the slots above kstar
// and, among the slots equal to it, the lowest bucket ids (an id limit is searched only when there are more ties
// than places left), sorted into rank order by a bitonic sort (in one wave's registers when at most 64 are
// chosen). With fewer than top_b non-empty buckets every one is chosen.
__global__ __launch_bounds__(1024) void k_choose_expand(const uint32_t* __restrict__ keys, int nb, int top_b,
                                                        int32_t* __restrict__ buckets_out,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ members, int64_t L,
                                                        const int32_t* __restrict__ t, int n_sink, int n_window,
                                                        int32_t* __restrict__ idx, int cap,
                                                        int32_t* __restrict__ n_sel) {
  constexpr int kWaves = 1024 / kWave;
  constexpr int kKeyRegs = 16;  // slots tid + 1024 m (m < kKeyRegs) stay in registers
  __shared__ int32_t rng_lo[1024], rng_n[1024], rng_base[1024];
  __shared__ int32_t chosen[1024];
  __shared__ int32_t buf[kMaxExpand];
  __shared__ int32_t tmp[kMaxExpand];
  __shared__ int32_t bin_cnt[1024], bin_cur[1024];
  __shared__ int32_t wsum[kWaves];
  __shared__ int overflow;
  __shared__ uint32_t sel_digit, sel_before, sel_n;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;

  // ---- choice of the buckets
  const uint32_t* kr = keys + (int64_t)b * nb;
  uint32_t kv[kKeyRegs];
#pragma unroll
  for (int m = 0; m < kKeyRegs; ++m) kv[m] = tid + 1024 * m < nb ? kr[tid + 1024 * m] : 0u;
  auto for_keys = [&](auto&& f) {  // f(bucket id, slot key); slots past nb hold key 0 (empty)
#pragma unroll
    for (int m = 0; m < kKeyRegs; ++m) f(tid + 1024 * m, kv[m]);
    for (int i = tid + 1024 * kKeyRegs; i < nb; i += 1024) f(i, kr[i]);
  };
  // block sum of one value per thread, with this thread's exclusive prefix
  auto block_scan = [&](int v, int* total) {
    const int incl = (int)wave_inclusive_scan((uint32_t)v, lane);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      before += w < wave ? wsum[w] : 0;
      all += wsum[w];
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
  };
  uint64_t* sorted = reinterpret_cast<uint64_t*>(buf);  // buf is free until the expansion
  int nc = 0;
  bool have_rng = false;  // rng_lo / rng_n of the chosen buckets are already set (block-uniform)
  {
  uint32_t* hist = reinterpret_cast<uint32_t*>(tmp);  // tmp is free until the expansion sorts
  uint32_t need = (uint32_t)top_b, prefix = 0u, pmask = 0u;
  int n_valid = 0;
  bool full = true;   // at least top_b non-empty buckets
  bool fast = false;  // the candidates of the first pass are ranked directly
  uint32_t fast_lo = 0u;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < 2048; i += 1024) hist[i] = 0u;
    __syncthreads();
    for_keys([&](int, uint32_t v) {
      if (v != 0u && (v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & (uint32_t)(nbins - 1)], 1u);
    });
    __syncthreads();
    // descending search: thread t takes bins nbins - 1 - per t and (per = 2) the one below it
    const int per = nbins / 1024;
    const uint32_t c0 = hist[nbins - 1 - per * tid], c1 = per > 1 ? hist[nbins - 2 - per * tid] : 0u;
    int tot;
    const uint32_t ex = (uint32_t)block_scan((int)(c0 + c1), &tot);
    if (ex < need && ex + c0 + c1 >= need) {
      const bool first = ex + c0 >= need;
      sel_digit = (uint32_t)(nbins - 1 - per * tid - (first ? 0 : 1));
      sel_before = first ? ex : ex + c0;
    }
    __syncthreads();
    if (pass == 0) {
      n_valid = tot;
      if ((uint32_t)tot < need) {  // block-uniform
        full = false;
        break;
      }
      if (sel_before + hist[sel_digit] <= (uint32_t)kFastCand) {  // block-uniform
        fast = true;
        fast_lo = sel_digit << 21;  // the candidates: keys whose top 11 bits are at least the digit
        break;
      }
    }
    prefix |= sel_digit << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
    need -= sel_before;
    __syncthreads();
  }
  nc = full ? top_b : n_valid;
  if (fast) {
    // the n <= kFastCand candidates as ascending (~key, id) = score desc, id asc; the rank of each is the number
    // of candidates before it, and ranks below top_b are the chosen buckets in rank order
    if (tid == 0) sel_n = 0u;
    __syncthreads();
    for_keys([&](int i, uint32_t v) {
      if (v != 0u && v >= fast_lo) sorted[atomicAdd(&sel_n, 1u)] = ((uint64_t)~v << 32) | (uint32_t)i;
    });
    __syncthreads();
    const int n = (int)sel_n;
    if (tid < n) {
      // each candidate also requests its bucket's member-list bounds before ranking, so that the expansion finds
      // them ready
      const uint64_t me = sorted[tid];
      const int id = (int)(uint32_t)me;
      const int o0 = offsets[id], o1 = offsets[id + 1];
      int r = 0;
#pragma unroll 8
      for (int j = 0; j < n; ++j) r += sorted[j] < me ? 1 : 0;
      if (r < top_b) {
        chosen[r] = id;
        rng_lo[r] = o0;
        rng_n[r] = o1 - o0;
        if (buckets_out) buckets_out[(int64_t)b * top_b + r] = id;
      }
    }
    have_rng = true;
  } else {
    const uint32_t kstar = prefix;  // with full: chosen = slots above kstar + `need` of the slots equal to it
    uint32_t id_lim = 0xFFFFFFFFu;  // slots equal to kstar are chosen when their id is below this
    if (full) {
      int my_ties = 0, n_ties;
      for_keys([&](int, uint32_t v) { my_ties += v == kstar ? 1 : 0; });
      block_scan(my_ties, &n_ties);
      if ((uint32_t)n_ties > need) {  // block-uniform: the smallest limit that admits `need` ties
        int lo = 0, hi = nb;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          int mine = 0, cnt;
          for_keys([&](int i, uint32_t v) { mine += (v == kstar && i < mid) ? 1 : 0; });
          block_scan(mine, &cnt);
          if ((uint32_t)cnt >= need) hi = mid;
          else lo = mid + 1;
        }
        id_lim = (uint32_t)lo;
      }
    }
    // the chosen (key, id) pairs, unordered, then sorted: ascending (~key, id) = score desc, id asc
    if (tid == 0) sel_n = 0u;
    __syncthreads();
    for_keys([&](int i, uint32_t v) {
      const bool take = full ? (v > kstar || (v == kstar && (uint32_t)i < id_lim)) : v != 0u;
      if (take) sorted[atomicAdd(&sel_n, 1u)] = ((uint64_t)~v << 32) | (uint32_t)i;
    });
    __syncthreads();
    if (nc <= kWave) {
      // up to 64 chosen: wave 0 sorts them in registers (lane l holds entry l), a bitonic network over lane pairs
      // exchanged by shuffles, with no workgroup barrier
      if (wave == 0) {
        uint64_t v = lane < nc ? sorted[lane] : ~0ull;
#pragma unroll
        for (int size = 2; size <= kWave; size <<= 1)
#pragma unroll
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t o = lane_xor64(v, stride);
            const bool keep_min = ((lane & stride) == 0) == ((lane & size) == 0);  // lower lane of an ascending pair
            v = keep_min ? (o < v ? o : v) : (o > v ? o : v);
          }
        if (lane < nc) chosen[lane] = (int32_t)(uint32_t)v;
        if (buckets_out && lane < top_b) buckets_out[(int64_t)b * top_b + lane] = lane < nc ? (int32_t)(uint32_t)v : -1;
      }
      if (buckets_out)
        for (int i = kWave + tid; i < top_b; i += 1024) buckets_out[(int64_t)b * top_b + i] = -1;
    } else {
      int n2 = 2;
      while (n2 < nc) n2 <<= 1;
      for (int i = nc + tid; i < n2; i += 1024) sorted[i] = ~0ull;
      __syncthreads();
      for (int size = 2; size <= n2; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int i = tid; i < (n2 >> 1); i += 1024) {
            const int lo = 2 * i - (i & (stride - 1));
            const int hi = lo + stride;
            const bool up = (lo & size) == 0;
            const uint64_t x = sorted[lo], y = sorted[hi];
            if ((x > y) == up) {
              sorted[lo] = y;
              sorted[hi] = x;
            }
          }
          __syncthreads();
        }
      if (tid < nc) chosen[tid] = (int32_t)(uint32_t)sorted[tid];
      if (buckets_out && tid < top_b)
        buckets_out[(int64_t)b * top_b + tid] = tid < nc ? (int32_t)(uint32_t)sorted[tid] : -1;
    }
  }
  }
  __syncthreads();

  // ---- expansion
  const int tb = t ? t[b] : (int)(L - 1);
  const int ns = n_sink < tb + 1 ? n_sink : tb + 1;
  int w0 = tb - n_window + 1;
  w0 = w0 > ns ? w0 : ns;
  int32_t* out = idx + (int64_t)b * cap;
  // member-list bounds of every chosen bucket, one thread per bucket (a single round trip), unless the choice
  // already fetched them
  if (!have_rng) {
    if (tid < nc) {
      const int c = chosen[tid];
      const int o0 = offsets[c];
      rng_lo[tid] = o0;
      rng_n[tid] = offsets[c + 1] - o0;
    }
    __syncthreads();
  }
  int total_all;
  const int all_base = block_scan(tid < nc ? rng_n[tid] : 0, &total_all);
  int total = 0;
  if (total_all <= kMaxExpand) {  // block-uniform
    // every member of the chosen buckets at once: the bucket of each entry of their concatenation is written into
    // tmp (one wave per bucket), then every thread requests eight entries together (clamped, unconditional
    // loads); the members inside [ns, w0) are compacted into buf in any order (the sort below orders them)
    if (tid < nc) rng_base[tid] = all_base;
    if (tid == 0) sel_n = 0u;
    __syncthreads();
    for (int i = wave; i < nc; i += kWaves) {
      const int base = rng_base[i], n = rng_n[i];
      for (int j = lane; j < n; j += kWave) tmp[base + j] = i;
    }
    __syncthreads();
    constexpr int kPer = 8;
    for (int e0 = 0; e0 < total_all; e0 += kPer * 1024) {
      int32_t mv[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = e0 + u * 1024 + tid;
        const int ec = e < total_all ? e : total_all - 1;
        const int seg = tmp[ec];
        mv[u] = members[rng_lo[seg] + (ec - rng_base[seg])];
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = e0 + u * 1024 + tid;
        const bool keep = e < total_all && mv[u] >= ns && mv[u] < w0;
        const uint64_t mk = ballot(keep);
        uint32_t base = 0u;
        if (lane == 0 && mk) base = atomicAdd(&sel_n, (uint32_t)__popcll(mk));
        base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
        if (keep) buf[base + lanes_below(mk)] = mv[u];
      }
    }
    __syncthreads();
    total = (int)sel_n;
    if (total > cap) {
      for (int i = tid; i < cap; i += 1024) out[i] = -1;
      if (tid == 0) n_sel[b] = -total;
      return;
    }
  } else {
  // each chosen bucket's members in [ns, w0): one wave per bucket counts, 64 members per load, how many lie below
  // ns and below w0 (members are ascending, so the counts are the range's bounds)
  for (int i = wave; i < nc; i += kWaves) {
    const int c = chosen[i];
    const int o0 = offsets[c], o1 = offsets[c + 1];
    int below_ns = 0, below_w0 = 0;
#pragma unroll 4
    for (int e0 = o0; e0 < o1; e0 += kWave) {
      const int e = e0 + lane;
      const int32_t m = e < o1 ? members[e] : 0x7FFFFFFF;
      below_ns += __popcll(ballot(m < ns));
      below_w0 += __popcll(ballot(m < w0));
    }
    if (lane == 0) {
      rng_lo[i] = o0 + below_ns;
      rng_n[i] = below_w0 - below_ns;
    }
  }
  __syncthreads();
  // output offsets of the ranges (exclusive scan over the chosen buckets, one per thread)
  const int v = tid < nc ? rng_n[tid] : 0;
  const int incl = (int)wave_inclusive_scan((uint32_t)v, lane);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    before += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  if (tid < nc) rng_base[tid] = before + incl - v;
  if (total > cap) {
    for (int i = tid; i < cap; i += 1024) out[i] = -1;
    if (tid == 0) n_sel[b] = -total;
    return;
  }
  __syncthreads();
  // the ranges into LDS, one wave per bucket
  for (int i = wave; i < nc; i += kWaves) {
    const int lo = rng_lo[i], n = rng_n[i], base = rng_base[i];
    for (int j = lane; j < n; j += kWave) buf[base + j] = members[lo + j];
  }
  __syncthreads();
  }
  // sort the positions (distinct: a position belongs to one bucket only) by binning them over [ns, w0) into 1024
  // bins of equal width, one per thread, then sorting each bin's few entries in registers; a bin that gets more
  // than kBinMax entries (clustered positions) sends the whole query to a bitonic sort instead
  // bin = floor((v - ns) * 1024 / span) in double: monotone in v, below 1024 for v < w0 (the product stays far
  // more than one double ulp under 1024), and the same rounding for the count and the scatter
  const int64_t span = (int64_t)w0 - ns > 0 ? (int64_t)w0 - ns : 1;
  const double bin_scale = 1024.0 / (double)span;
  auto bin_of = [&](int32_t v) {
    const int bn = (int)((double)(v - ns) * bin_scale);
    return bn < 1023 ? bn : 1023;
  };
  bin_cnt[tid] = 0;
  if (tid == 0) overflow = 0;
  __syncthreads();
  for (int g = tid; g < total; g += 1024) atomicAdd(&bin_cnt[bin_of(buf[g])], 1);
  __syncthreads();
  const int my_cnt = bin_cnt[tid];
  if (my_cnt > kBinMax) overflow = 1;
  const int incl2 = (int)wave_inclusive_scan((uint32_t)my_cnt, lane);
  if (lane == kWave - 1) wsum[wave] = incl2;
  __syncthreads();
  int before2 = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) before2 += w < wave ? wsum[w] : 0;
  const int my_start = before2 + incl2 - my_cnt;
  bin_cur[tid] = my_start;
  __syncthreads();
  if (!overflow) {
    for (int g = tid; g < total; g += 1024) {
      const int32_t v = buf[g];
      tmp[atomicAdd(&bin_cur[bin_of(v)], 1)] = v;
    }
    __syncthreads();
    // each bin sorted in registers, by a network as wide as the fullest bin of the wave needs
    if (ballot(my_cnt > 8)) sort_bin<kBinMax>(tmp + my_start, my_cnt, out + my_start);
    else if (ballot(my_cnt > 4)) sort_bin<8>(tmp + my_start, my_cnt, out + my_start);
    else sort_bin<4>(tmp + my_start, my_cnt, out + my_start);
  } else {
    int n2 = 1;
    while (n2 < total) n2 <<= 1;
    for (int i = total + tid; i < n2; i += 1024) buf[i] = 0x7FFFFFFF;
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < (n2 >> 1); i += 1024) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int32_t x = buf[lo], y = buf[hi];
          if ((x > y) == up) {
            buf[lo] = y;
            buf[hi] = x;
          }
        }
        __syncthreads();
      }
    for (int i = tid; i < total; i += 1024) out[i] = buf[i];
  }
  for (int i = total + tid; i < cap; i += 1024) out[i] = -1;
  if (tid == 0) n_sel[b] = total;
}

}  // namespace

BucketBuildPlan bucket_build_plan(int64_t L, int32_t nb) {
  BucketBuildPlan p;
  int64_t max_chunks = kTableBudget / (nb > 0 ? nb : 1);
  if (max_chunks < 1) max_chunks = 1;
  int64_t chunk = (L + max_chunks - 1) / max_chunks;
  if (chunk < kChunkMin) chunk = kChunkMin;
  chunk = (chunk + kWave - 1) / kWave * kWave;
  p.chunk = chunk;
  p.n_chunks = L > 0 ? (L + chunk - 1) / chunk : 0;
  return p;
}

hipError_t launch_bucket_build(const void* k, int k_dtype, int64_t k_ld, int64_t L, int d, const int32_t* assign,
                               int nb, float* reps, int32_t* offsets, int32_t* members, int32_t* counts,
                               int32_t* table, const BucketBuildPlan& p, hipStream_t st) {
  const int64_t tbl = p.n_chunks * (int64_t)nb;
  const bool lds = nb <= kLdsBuckets && p.chunk <= kScatterStage;
  if (L > 0) {
    if (lds) {
      SA_LAUNCH(k_chunk_hist<true>, dim3((unsigned)p.n_chunks), dim3(256), 0, st, assign, L, p.chunk, nb, table);
    } else {
      SA_LAUNCH(k_fill_i32, dim3(1024), dim3(256), 0, st, table, tbl, 0);
      SA_LAUNCH(k_chunk_hist<false>, dim3((unsigned)p.n_chunks), dim3(256), 0, st, assign, L, p.chunk, nb, table);
    }
    SA_LAUNCH(k_chunk_scan, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, nb, p.n_chunks, table, counts);
  } else {
    SA_LAUNCH(k_fill_i32, dim3(256), dim3(256), 0, st, counts, (int64_t)nb, 0);
  }
  SA_LAUNCH(k_offsets, dim3(1), dim3(1024), 0, st, counts, nb, offsets);
  if (L > 0) {
    if (lds)
      SA_LAUNCH(k_scatter<true>, dim3((unsigned)p.n_chunks), dim3(256), 0, st, assign, L, p.chunk, nb, offsets, table,
                members);
    else
      SA_LAUNCH(k_scatter<false>, dim3((unsigned)p.n_chunks), dim3(256), 0, st, assign, L, p.chunk, nb, offsets,
                table, members);
  }
  if (k_dtype == 0)
    SA_LAUNCH(k_reps<0>, dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, st, k, k_ld, d, offsets, members, nb, reps);
  else
    SA_LAUNCH(k_reps<1>, dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, st, k, k_ld, d, offsets, members, nb, reps);
  return hipGetLastError();
}

int bucket_expand_max() { return kMaxExpand; }

// ---- scratch of the no-allocation variant of the bucket search ---------------------------------------------------
// One key per (query, bucket) in a static device array: each device that loads the library holds its own copy
// until the process ends. Host code never passes `scratch` itself to a kernel (on the host it only names the
// symbol): the device address comes from hipGetSymbolAddress, looked up once per device with that device current.
constexpr int64_t kScratchWords = (int64_t)1 << 21;  // 8 MiB
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint32_t scratch[kScratchWords];

int64_t bucket_scratch_words() { return kScratchWords; }

hipError_t bucket_scratch(hipStream_t st, uint32_t** out) {
  static std::mutex mu;
  static uint32_t* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e;
  if (st) {
    hipDevice_t d;
    e = hipStreamGetDevice(st, &d);
    if (e != hipSuccess) return e;
    dev = (int)d;
  } else {
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = static_cast<uint32_t*>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

hipError_t launch_bucket_scores(const void* q, int q_dtype, int B, int d, const float* reps, const int32_t* offsets,
                                int nb, uint32_t* keys, hipStream_t st) {
  const unsigned n_wg = (unsigned)((nb + 63) / 64);  // 64 buckets per workgroup
  const size_t lds = sizeof(float) * (size_t)B * d;
  if (q_dtype == 0)
    SA_LAUNCH(k_bucket_scores<0>, dim3(n_wg), dim3(256), lds, st, q, B, d, reps, offsets, nb, keys);
  else
    SA_LAUNCH(k_bucket_scores<1>, dim3(n_wg), dim3(256), lds, st, q, B, d, reps, offsets, nb, keys);
  return hipGetLastError();
}

hipError_t launch_tree_children(const void* q, int q_dtype, int B, int d, const int32_t* kept, int keep_ld,
                                const int32_t* n_kept, const int32_t* child_off, const float* reps,
                                const int32_t* offsets, int n_next, uint32_t* keys, hipStream_t st) {
  if (B < 1 || keep_ld < 1) return hipSuccess;
  const dim3 grid((unsigned)keep_ld, (unsigned)B);
  const size_t lds = sizeof(float) * (size_t)d;
  if (q_dtype == 0)
    SA_LAUNCH(k_tree_children<0>, grid, dim3(256), lds, st, q, d, kept, keep_ld, n_kept, child_off, reps, offsets,
              n_next, keys);
  else
    SA_LAUNCH(k_tree_children<1>, grid, dim3(256), lds, st, q, d, kept, keep_ld, n_kept, child_off, reps, offsets,
              n_next, keys);
  return hipGetLastError();
}

hipError_t launch_bucket_choose(const uint32_t* keys, int B, int nb, int top_b, int32_t* buckets_out,
                                const int32_t* offsets, const int32_t* members, int64_t L, const int32_t* t,
                                int n_sink, int n_window, int32_t* idx, int cap, int32_t* n_sel, hipStream_t st) {
  if (B < 1) return hipSuccess;
  SA_LAUNCH(k_choose_expand, dim3((unsigned)B), dim3(1024), 0, st, keys, nb, top_b, buckets_out, offsets,
                     members, L, t, n_sink, n_window, idx, cap, n_sel);
  return hipGetLastError();
}

hipError_t launch_bucket_select(const void* q, int q_dtype, int B, int d, const float* reps, const int32_t* offsets,
                                const int32_t* members, int nb, int64_t L, const int32_t* t, int top_b, int n_sink,
                                int n_window, int32_t* idx, int cap, int32_t* n_sel, int32_t* buckets_out,
                                uint32_t* keys, hipStream_t st) {
  const unsigned n_wg = (unsigned)((nb + 63) / 64);  // 64 buckets per workgroup
  const size_t lds = sizeof(float) * (size_t)B * d;
  if (q_dtype == 0)
    SA_LAUNCH(k_bucket_scores<0>, dim3(n_wg), dim3(256), lds, st, q, B, d, reps, offsets, nb, keys);
  else
    SA_LAUNCH(k_bucket_scores<1>, dim3(n_wg), dim3(256), lds, st, q, B, d, reps, offsets, nb, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SA_LAUNCH(k_choose_expand, dim3((unsigned)B), dim3(1024), 0, st, keys, nb, top_b, buckets_out, offsets,
                     members, L, t, n_sink, n_window, idx, cap, n_sel);
  return hipGetLastError();
}

}  // namespace sa
