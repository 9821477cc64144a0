// attn_merge_results: merge of results computed over disjoint shares of the
// keys -- the exchange step of a sequence-sharded decode, where each device
// decodes its share of every sequence's tokens and the devices' (O, lse)
// pairs are combined per row (Star Attention article, phase 2: the query host
// combines the hosts' local outputs by their softmax statistics; Tree
// Attention article, an energy view of attention: the local energies are
// reduced across devices).
//
// A result (O_p, lse_p) is the record (m = lse_p, l = 1, o = O_p) in
// natural-log units, so the associative merge rule combines them:
//   M = max_p lse_p,  w_p = e^(lse_p - M),
//   O = sum_p w_p O_p / sum_p w_p,  lse = M + ln sum_p w_p.
#include <hip/hip_runtime.h>

#include "attn_decode.h"
#include "device_common.h"
#include "plan.h"

namespace attn {
namespace {

// A wave per row: the parts' maximum lse first (lane l reads parts l, l + 64,
// ...), then every part weighted by e^(lse_p - M) in part order (fixed order:
// deterministic); lane l holds D/64 of the outputs.  A part with lse = -inf
// saw no key: it adds nothing and its O is not read.  ENERGY: lse only (the
// logsumexp of the parts' lse; no O is read or written).
constexpr int kRowsPerBlock = 4;
constexpr int kBatch = 8;  // parts loaded together

template <int D, bool ENERGY>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void merge_results(
    int n, int64_t rows, const float *__restrict__ o_parts, const float *__restrict__ lse_parts,
    float *__restrict__ o, float *__restrict__ lse) {
  constexpr int EPL = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= rows) return;  // whole waves; no barrier follows
  float M = -INFINITY;
  for (int p = lane; p < n; p += kWave) M = fmaxf(M, lse_parts[(int64_t)p * rows + row]);
  M = wave_max(M);
  float acc[EPL], wsum = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  if (M != -INFINITY) {
    for (int p0 = 0; p0 < n; p0 += kBatch) {
      float wgt[kBatch], ov[kBatch][EPL];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int p = p0 + k;
        wgt[k] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) ov[k][e] = 0.0f;
        if (p < n) {
          const float lp = lse_parts[(int64_t)p * rows + row];
          if (lp != -INFINITY) {
            wgt[k] = fast_exp2((lp - M) * kLog2e);
            if constexpr (!ENERGY) {
              const float *src = o_parts + ((int64_t)p * rows + row) * D + lane * EPL;
#pragma unroll
              for (int e = 0; e < EPL; ++e) ov[k][e] = src[e];
            }
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        wsum += wgt[k];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wgt[k], ov[k][e], acc[e]);
      }
    }
  }
  const bool empty = M == -INFINITY || !(wsum > 0.0f);
  if (lane == 0) lse[row] = empty ? -INFINITY : M + log2f(wsum) * kLn2;
  if constexpr (ENERGY) return;
  const float inv = empty ? 0.0f : 1.0f / wsum;
  float *dst = o + row * D + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[e] = acc[e] * inv;
}

// Rows per call: a wave per row, so 2^25 rows are 2^31 work-items, below the
// 2^32 that one launch dimension can count.
constexpr int64_t kMaxResultRows = (int64_t)1 << 25;

}  // namespace
}  // namespace attn

attn_status_t attn_merge_results(int32_t n_parts, int64_t rows, int32_t head_dim,
                                 const float *o_parts, const float *lse_parts, float *o,
                                 float *lse, void *stream) {
  using namespace attn;
  try {
    if (n_parts < 1 || rows < 0 || rows > kMaxResultRows) return ATTN_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
    if (rows == 0) return ATTN_OK;
    const bool energy = o_parts == nullptr && o == nullptr;  // lse only
    if (!lse_parts || !lse || (!energy && (!o_parts || !o))) return ATTN_ERR_NULL;
    if (!aligned(o_parts, 4) || !aligned(lse_parts, 4) || !aligned(o, 4) || !aligned(lse, 4))
      return ATTN_ERR_ALIGN;
    (void)hipGetLastError();
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    const dim3 block(kRowsPerBlock * kWave);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (energy)
      hipLaunchKernelGGL((merge_results<64, true>), grid, block, 0, s, n_parts, rows, o_parts,
                         lse_parts, o, lse);
    else if (head_dim == 64)
      hipLaunchKernelGGL((merge_results<64, false>), grid, block, 0, s, n_parts, rows, o_parts,
                         lse_parts, o, lse);
    else
      hipLaunchKernelGGL((merge_results<128, false>), grid, block, 0, s, n_parts, rows, o_parts,
                         lse_parts, o, lse);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}
