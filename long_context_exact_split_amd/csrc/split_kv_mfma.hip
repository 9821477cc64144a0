// Split-KV decode for dense query blocks on the matrix cores (gfx950 MFMA).
//
// Used when one KV head serves many query rows at once (R = G * q_len > 8):
// a speculative-style block of query tokens, or the samples of a shared
// prefix.  The contraction is then dense enough (32 flop per KV byte for 32
// rows) that the vector ALUs could not keep up with HBM.  Each work item is
// (sequence b, KV head, block of 32 query rows, chunk of KV); its four waves
// take 32-key tiles of the chunk in turn and each keeps an online softmax
// ("attention acceleration" concept page, section 2.1) for all 32 rows.
//
// Per 32-key tile, in one wave:
//   S^T[32 keys x 32 rows] = K_tile . Q^T   v_mfma_f32_32x32x16_bf16, K as the A
//        operand, so lane l owns query row l % 32 and 16 of the tile's keys;
//        row max / row sum need one exchange between lanes l and l + 32.
//   P = 2^(S*scale*log2e - m): fp32, rounded once to fp16 (11 significant
//        bits) for the product; the row sums l use the fp32 values.
//   O^T[D x 32 rows] += V_tile^T . P^T   v_mfma_f32_32x32x16_f16.  P^T is the
//        B operand taken straight from the S^T accumulator registers; V is
//        converted from bf16 to fp16 when its tile is stored into LDS (exact:
//        bf16 has 8 significant bits, fp16 11), and V^T is read from LDS with
//        the gfx950 transpose read ds_read_b64_tr_b16, which hands each lane
//        four consecutive keys of one column.  Lane l again owns row l % 32,
//        so rescaling O when the running max grows is lane-local.
//        Range: fp16 spans 2^-14 .. 65504, bf16 much more, so the product
//        carries P * 2^7 (P <= 2^8 with the lazy rescale, so P * 2^7 <= 2^15)
//        and V * 2^-7 (exact for 2^-7 <= |v| <= 8.3e6; smaller values keep
//        an absolute precision of 2^-18), which leaves O unchanged.
// K and V tiles are loaded coalesced (LPK lanes per key row, 16 bytes each,
// non-temporal) and staged in wave-private LDS; the next tile's loads are in
// flight while the current one is computed.  The four waves' (m, l, o) are
// merged through LDS at the end of each piece of work (work_map.h), giving
// one record per (piece, row) in the same layout as the vector-ALU kernel, so
// the same merge kernel follows.
#include "mfma_piece.h"

#ifdef ATTN_WG_STAMPS
#define ATTN_WG_STAMPS_READBACK attn_probe_wg_stamps_mfma
#include "probe/wg_stamps.h"  // per-workgroup clocks: measurement builds only
#else
#define ATTN_WG_STAMP()
#endif

namespace attn {
namespace {

using namespace mfma;

template <int D, bool ENERGY, bool PAGED>
__global__ __launch_bounds__(kThreads) void split_kv_mfma(SplitArgs a) {
  ATTN_WG_STAMP();
  __shared__ MfmaSmem<D, ENERGY> sh;
  WorkMap m = a.map;
  m.causal_rows = 0;  // one row block: never set for this kernel's maps
  if (m.mode == 0) {
    const int w = blockIdx.x;
    const int sigma = w / m.n_chunks, c = w - sigma * m.n_chunks;
    const int group = sigma / m.row_blocks, rb = sigma - group * m.row_blocks;
    const int b = group / m.Hkv, kvh = group - b * m.Hkv;
    const int L = (int)seq_len(m, b);
    const int c0 = c * m.chunk_len;
    if (c0 >= L) return;
    mfma_piece<D, ENERGY, PAGED>(a, b, kvh, rb, c0, min(c0 + m.chunk_len, L), w, sh);
  } else {
    const int64_t U = total_units(m);
    PieceCursor cur = first_piece(m, U, blockIdx.x);
    Piece p;
    while (next_piece(m, blockIdx.x, cur, &p))
      mfma_piece<D, ENERGY, PAGED>(a, p.b, p.kvh, p.rb, (int)p.t0, (int)p.t1, p.slot, sh);
  }
}

// FIN: the finalising epilogue (a.fin set; full mode, dense caches only).
template <int D, int RW, bool ENERGY, bool PAGED, bool CAUSAL_ROWS, bool FIN = false>
__global__ __launch_bounds__(RW * kWave) void split_kv_mfma_rows(SplitArgs a) {
  __shared__ RowsSmem<D, RW, ENERGY> sh;
  WorkMap m = a.map;
  m.causal_rows = CAUSAL_ROWS ? 1 : 0;  // as the launcher checked; known at compile time
  if (m.mode == 0) {
    const int w = blockIdx.x;
    const int sigma = w / m.n_chunks, c = w - sigma * m.n_chunks;
    const int group = sigma / m.row_blocks, rb = sigma - group * m.row_blocks;
    const int b = group / m.Hkv, kvh = group - b * m.Hkv;
    const int L = (int)seq_len(m, b);
    const int c0 = c * m.chunk_len;
    if (c0 >= L) return;
    rows_piece<D, RW, ENERGY, PAGED, FIN>(a, b, kvh, rb, c0, min(c0 + m.chunk_len, L), w, sh);
  } else if constexpr (CAUSAL_ROWS) {
    // The causal layout's arithmetic (closed-form sums, a binary search per
    // piece) runs on one lane, a batch of pieces at a time, into LDS; the
    // tile loop then runs with none of its state held in registers (inlined
    // next to the loop it cost SGPR spills and ~5% more VALU per tile).
    constexpr int kBatch = 16;
    __shared__ PieceCursor cur_s;
    __shared__ Piece list[kBatch];
    __shared__ int count;
    const int wl = xcd_local_index(blockIdx.x, m.n_wg, m.row_blocks > 1);
    if (threadIdx.x == 0) cur_s = first_piece(m, total_units(m), wl);
    for (;;) {
      __syncthreads();  // every wave is done with the previous batch
      if (threadIdx.x == 0) {
        PieceCursor c = cur_s;
        int n = 0;
        Piece p;
        while (n < kBatch && next_piece(m, wl, c, &p)) list[n++] = p;
        cur_s = c;
        count = n;
      }
      __syncthreads();
      const int n = __builtin_amdgcn_readfirstlane(count);
      if (n == 0) break;
      for (int k = 0; k < n; ++k) {
        const Piece &p = list[k];
        const int b = __builtin_amdgcn_readfirstlane(p.b);
        const int kvh = __builtin_amdgcn_readfirstlane(p.kvh);
        const int rb = __builtin_amdgcn_readfirstlane(p.rb);
        const int t0 = __builtin_amdgcn_readfirstlane((int)p.t0);
        const int t1 = __builtin_amdgcn_readfirstlane((int)p.t1);
        const int64_t slot = ((int64_t)__builtin_amdgcn_readfirstlane((int)(p.slot >> 32)) << 32) |
                             (uint32_t)__builtin_amdgcn_readfirstlane((int)(p.slot & 0xffffffff));
        rows_piece<D, RW, ENERGY, PAGED, FIN>(a, b, kvh, rb, t0, t1, slot, sh);
      }
    }
  } else {
    const int64_t U = total_units(m);
    const int wl = xcd_local_index(blockIdx.x, m.n_wg, m.row_blocks > 1);
    PieceCursor cur = first_piece(m, U, wl);
    Piece p;
    while (next_piece(m, wl, cur, &p))
      rows_piece<D, RW, ENERGY, PAGED, FIN>(a, p.b, p.kvh, p.rb, (int)p.t0, (int)p.t1, p.slot, sh);
  }
}

template <int D, int RW, bool ENERGY, bool PAGED>
hipError_t launch_rows(const attn_plan_t &plan, const SplitArgs &a, hipStream_t stream) {
  if (a.fin) {
    if constexpr (!ENERGY && !PAGED) {
      if (a.map.causal_rows)
        hipLaunchKernelGGL((split_kv_mfma_rows<D, RW, false, false, true, true>),
                           dim3((unsigned)plan.work_items), dim3(RW * kWave), 0, stream, a);
      else
        hipLaunchKernelGGL((split_kv_mfma_rows<D, RW, false, false, false, true>),
                           dim3((unsigned)plan.work_items), dim3(RW * kWave), 0, stream, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (a.map.causal_rows)
    hipLaunchKernelGGL((split_kv_mfma_rows<D, RW, ENERGY, PAGED, true>),
                       dim3((unsigned)plan.work_items), dim3(RW * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((split_kv_mfma_rows<D, RW, ENERGY, PAGED, false>),
                       dim3((unsigned)plan.work_items), dim3(RW * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool ENERGY, bool PAGED>
hipError_t launch_rows_rw(const attn_plan_t &plan, const SplitArgs &a, hipStream_t stream) {
  switch (plan.rows_per_block) {
    case 2 * kRows: return launch_rows<D, 2, ENERGY, PAGED>(plan, a, stream);
    case 4 * kRows: return launch_rows<D, 4, ENERGY, PAGED>(plan, a, stream);
    case 8 * kRows: return launch_rows<D, 8, ENERGY, PAGED>(plan, a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D, bool ENERGY, bool PAGED>
hipError_t launch_kernel(const attn_plan_t &plan, const SplitArgs &a, hipStream_t stream) {
  if (plan.kernel == 2) return launch_rows_rw<D, ENERGY, PAGED>(plan, a, stream);
  if (plan.rows_per_block != kRows || a.map.causal_rows) return hipErrorInvalidValue;
  hipLaunchKernelGGL((split_kv_mfma<D, ENERGY, PAGED>), dim3((unsigned)plan.work_items),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const attn_plan_t &plan, const SplitArgs &a, bool energy, hipStream_t stream) {
  const bool paged = a.pg.block_table != nullptr;
  if (energy)
    return paged ? launch_kernel<D, true, true>(plan, a, stream)
                 : launch_kernel<D, true, false>(plan, a, stream);
  return paged ? launch_kernel<D, false, true>(plan, a, stream)
               : launch_kernel<D, false, false>(plan, a, stream);
}

}  // namespace

hipError_t launch_split_mfma(const attn_plan_t &plan, const SplitArgs &a, int head_dim,
                             bool energy_only, hipStream_t stream) {
  if (plan.work_items <= 0) return hipSuccess;
  if (head_dim == 64) return launch_d<64>(plan, a, energy_only, stream);
  if (head_dim == 128) return launch_d<128>(plan, a, energy_only, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn

