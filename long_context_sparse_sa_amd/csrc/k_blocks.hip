// Block-granular indexers ("long-context attention" lecture, sections "Qwen Sparse Attention" and "MiniMax Sparse
// Attention"): the small kernels around the shared scorers and selects.
//  * QSA ranks micro-blocks of b positions by the indexer equation on their pooled (mean) keys: the pooled keys are
//    the mean-key kernel's output (k_hi.hip), the ranking is the flat selection over them with each query's last
//    complete micro-block as its visible bound (k_block_t), and k_qsa_expand turns the chosen micro-blocks into
//    positions and appends the unfinished micro-block's visible positions.
//  * MSA scores tokens per group of indexer heads (each group a query of the flat scorer), keeps each block's
//    largest score (the MFMA scorer's block-max mode), ranks the blocks before the local one with the radix select,
//    and k_msa_expand turns the chosen blocks plus the local block into positions.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

__global__ __launch_bounds__(256) void k_block_t(const int32_t* __restrict__ t, int B, int reps, int64_t L, int div,
                                                 int32_t* __restrict__ t_out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * reps) return;
  int64_t tb = t ? (int64_t)t[i / reps] : L - 1;
  if (div > 1) {
    tb = (tb + 1) / div - 1;
    tb = tb < 0 ? 0 : tb;
  }
  t_out[i] = (int32_t)tb;
}

// One workgroup per query; entry j of the output row: block j / b (of the chosen ones) at offset j % b, then the
// tail, then -1 padding.
__global__ __launch_bounds__(256) void k_qsa_expand(const int32_t* __restrict__ blk, int kb,
                                                    const int32_t* __restrict__ n_blk, const int32_t* __restrict__ t,
                                                    int64_t L, int b, int32_t* __restrict__ idx, int idx_ld,
                                                    int32_t* __restrict__ n_sel) {
  const int q = blockIdx.x;
  const int64_t tq = t ? (int64_t)t[q] : L - 1;
  const int64_t n_complete = (tq + 1) / b;
  int nb = n_complete > 0 ? n_blk[q] : 0;
  nb = nb < 0 ? 0 : (nb > kb ? kb : nb);
  const int n_exp = nb * b;
  const int tail = (int)(tq + 1 - n_complete * b);
  const int total = n_exp + tail;
  const int32_t* my = blk + (int64_t)q * kb;
  int32_t* out = idx + (int64_t)q * idx_ld;
  for (int j = threadIdx.x; j < idx_ld; j += blockDim.x) {
    int32_t v = -1;
    if (j < n_exp) v = my[j / b] * b + j % b;
    else if (j < total) v = (int32_t)(n_complete * b + (j - n_exp));
    out[j] = v;
  }
  if (threadIdx.x == 0) n_sel[q] = total;
}

__global__ __launch_bounds__(256) void k_msa_expand(const int32_t* __restrict__ blk, int blk_ld,
                                                    const int32_t* __restrict__ n_blk, const int32_t* __restrict__ t,
                                                    int c, int32_t* __restrict__ idx, int idx_ld,
                                                    int32_t* __restrict__ n_sel) {
  const int q = blockIdx.x;
  const int64_t tq = t[q];
  const int64_t local = tq / c;
  int nb = n_blk ? n_blk[q] : 0;
  nb = nb < 0 ? 0 : (nb > blk_ld ? blk_ld : nb);
  const int n_exp = nb * c;
  const int total = n_exp + (int)(tq - local * c + 1);
  const int32_t* my = blk ? blk + (int64_t)q * blk_ld : nullptr;
  int32_t* out = idx + (int64_t)q * idx_ld;
  for (int j = threadIdx.x; j < idx_ld; j += blockDim.x) {
    int32_t v = -1;
    if (j < n_exp) v = my[j / c] * c + j % c;
    else if (j < total) v = (int32_t)(local * c + (j - n_exp));
    out[j] = v;
  }
  if (threadIdx.x == 0) n_sel[q] = total;
}

}  // namespace

hipError_t launch_block_t(const int32_t* t, int B, int reps, int64_t L, int div, int32_t* t_out, hipStream_t st) {
  const int n = B * reps;
  if (n < 1) return hipSuccess;
  SA_LAUNCH(k_block_t, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, t, B, reps, L, div, t_out);
  return hipGetLastError();
}

hipError_t launch_qsa_expand(const int32_t* blk, int kb, const int32_t* n_blk, const int32_t* t, int B, int64_t L,
                             int b, int32_t* idx, int idx_ld, int32_t* n_sel, hipStream_t st) {
  if (B < 1) return hipSuccess;
  SA_LAUNCH(k_qsa_expand, dim3((unsigned)B), dim3(256), 0, st, blk, kb, n_blk, t, L, b, idx, idx_ld, n_sel);
  return hipGetLastError();
}

hipError_t launch_msa_expand(const int32_t* blk, int blk_ld, const int32_t* n_blk, const int32_t* t, int B, int c,
                             int32_t* idx, int idx_ld, int32_t* n_sel, hipStream_t st) {
  if (B < 1) return hipSuccess;
  SA_LAUNCH(k_msa_expand, dim3((unsigned)B), dim3(256), 0, st, blk, blk_ld, n_blk, t, c, idx, idx_ld, n_sel);
  return hipGetLastError();
}

}  // namespace sa
