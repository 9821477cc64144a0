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
//   P = 2^(S*scale*log2e - m): fp32, split into bf16 hi + lo parts (the
//        product then carries ~16 significant bits of P).
//   O^T[D x 32 rows] += V_tile^T . P^T   P^T is the B operand taken straight
//        from the S^T accumulator registers; V^T is read from LDS with the
//        gfx950 transpose read ds_read_b64_tr_b16, which hands each lane four
//        consecutive keys of one column.  Lane l again owns row l % 32, so
//        rescaling O when the running max grows is lane-local.
// K and V tiles are loaded coalesced (LPK lanes per key row, 16 bytes each,
// non-temporal) and staged in wave-private LDS; the next tile's loads are in
// flight while the current one is computed.  The four waves' (m, l, o) are
// merged through LDS at the end, giving one record per (item, row) in the
// same layout as the vector-ALU kernel, so the same merge kernel follows.
#include "device_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 32;   // query rows per work item
constexpr int kTile = 32;   // keys per tile
constexpr float kLazyRescale = 8.0f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

template <int D>
struct Tiles {
  static constexpr int LPK = D / 8;          // lanes per key row (16 bytes each)
  static constexpr int KPI = kWave / LPK;    // keys per load instruction
  static constexpr int NL = kTile / KPI;     // load instructions per tile and tensor
  static constexpr int KS = D / 16;          // MFMA k-steps of Q.K (8 dims per lane half)
  static constexpr int NT = D / 32;          // 32-dim output tiles of O^T
  static constexpr int KROW = D + 8;         // LDS row pitch of the K tile (bf16 elements)
  static constexpr int VROW = D + 16;        // LDS row pitch of the V tile (bf16 elements)
};

template <int D, bool ENERGY>
struct Smem {
  uint16_t k[kWaves][kTile * Tiles<D>::KROW];
  uint16_t v[kWaves][ENERGY ? 1 : kTile * Tiles<D>::VROW];
};

template <int D, bool ENERGY>
struct SmemOut {
  float m[kWaves][kRows];
  float l[kWaves][kRows];
  float o[ENERGY ? 1 : kWaves][ENERGY ? 1 : kRows][ENERGY ? 1 : D + 4];
};

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int D, bool ENERGY>
__global__ __launch_bounds__(kThreads) void split_kv_mfma(SplitArgs a) {
  using T = Tiles<D>;
  constexpr int LPK = T::LPK, KPI = T::KPI, NL = T::NL, KS = T::KS, NT = T::NT;
  __shared__ union {
    Smem<D, ENERGY> t;
    SmemOut<D, ENERGY> out;
  } sh;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int h = lane >> 5;   // lane half
  const int j = lane & 31;   // query row owned by this lane (and key slot in A layouts)

  int item = blockIdx.x;
  const int chunk = item % a.n_chunks;
  item /= a.n_chunks;
  const int rb = item % a.row_blocks;
  const int group = item / a.row_blocks;
  const int b = group / a.Hkv;
  const int kvh = group - b * a.Hkv;

  int Lb = a.kv_lens ? a.kv_lens[b] : (int)a.L_max;
  Lb = Lb < 0 ? 0 : (Lb > (int)a.L_max ? (int)a.L_max : Lb);
  const int c0 = chunk * a.chunk_len;
  if (c0 >= Lb) return;
  const int c1 = min(c0 + a.chunk_len, Lb);

  // This lane's query row and its visibility limit (keys t < lim).
  const int row = rb * kRows + j;
  const bool valid = row < a.R;
  int lim = c0;
  bf16x8_t qf[KS];
  if (valid) {
    const int i = row / a.G;
    const int head = kvh * a.G + (row - i * a.G);
    lim = a.causal ? Lb - a.q_len + i + 1 : Lb;
    lim = lim < c0 ? c0 : (lim > c1 ? c1 : lim);
    const uint16_t *q = static_cast<const uint16_t *>(a.q) +
                        (((int64_t)b * a.q_len + i) * a.Hq + head) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4 *>(q + 8 * s));
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8_t, u32x4{0, 0, 0, 0});
  }
  // Last visible key over the block's rows (row limits grow with the token index).
  int hi;
  {
    const int last = min(a.R, (rb + 1) * kRows) - 1;
    const int ilast = last / a.G;
    hi = a.causal ? Lb - a.q_len + ilast + 1 : Lb;
    hi = hi < c0 ? c0 : (hi > c1 ? c1 : hi);
  }

  float m = -INFINITY, lsum = 0.0f;
  f32x16_t oacc[ENERGY ? 1 : NT];
#pragma unroll
  for (int n = 0; n < (ENERGY ? 1 : NT); ++n)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[n][e] = 0.0f;

  const int64_t base = (int64_t)group * a.L_max * D;
  const uint16_t *kg = static_cast<const uint16_t *>(a.k) + base + (lane % LPK) * 8;
  const uint16_t *vg = ENERGY ? nullptr : static_cast<const uint16_t *>(a.v) + base + (lane % LPK) * 8;
  uint16_t *ks = sh.t.k[wave];
  uint16_t *vs = sh.t.v[wave];
  const int n_tiles = (hi - c0 + kTile - 1) / kTile;

  u32x4 kr[NL], vr[ENERGY ? 1 : NL];
  auto load = [&](int tile) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      int t = c0 + tile * kTile + i * KPI + lane / LPK;
      t = t < hi ? t : hi - 1;
      kr[i] = load_nt(kg + (int64_t)t * D);
      if constexpr (!ENERGY) vr[i] = load_nt(vg + (int64_t)t * D);
    }
  };

  int tile = wave;
  if (tile < n_tiles) load(tile);
  for (; tile < n_tiles; tile += kWaves) {
    // Stage this tile in LDS (the wave's previous LDS reads are complete:
    // LDS instructions of one wave execute in order).
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int key = i * KPI + lane / LPK;
      *reinterpret_cast<u32x4 *>(ks + key * T::KROW + (lane % LPK) * 8) = kr[i];
      if constexpr (!ENERGY) *reinterpret_cast<u32x4 *>(vs + key * T::VROW + (lane % LPK) * 8) = vr[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int t0 = c0 + tile * kTile;
    if (tile + kWaves < n_tiles) load(tile + kWaves);

    // S^T = K . Q^T
    f32x16_t sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t kf = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4 *>(ks + j * T::KROW + h * (D / 2) + 8 * s));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
    }
    // Scale, mask, online softmax (lane l: row j, keys 8(e/4) + 4h + e%4).
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = t0 + 8 * (e >> 2) + 4 * h + (e & 3);
      sacc[e] = t < lim ? sacc[e] * a.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sacc[e]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (__any(tmax > m + kLazyRescale)) {
      const float mn = fmaxf(m, tmax);
      const float alpha = rescale_factor(m, mn);
      lsum *= alpha;
      if constexpr (!ENERGY) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[n][e] *= alpha;
      }
      m = mn;
    }
    const float mref = m == -INFINITY ? 0.0f : m;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sacc[e] = fast_exp2(sacc[e] - mref);
      lsum += sacc[e];
    }
    if constexpr (!ENERGY) {
      // P^T fragments (B operand): k-step s holds accumulator entries 8s..8s+7.
      bf16x8_t phi[2], plo[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 wh, wl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = sacc[8 * s + 2 * e], p1 = sacc[8 * s + 2 * e + 1];
          const uint32_t hw = pack_bf16(p0, p1);
          wh[e] = hw;
          const float h0 = __builtin_bit_cast(float, hw << 16);
          const float h1 = __builtin_bit_cast(float, hw & 0xFFFF0000u);
          wl[e] = pack_bf16(p0 - h0, p1 - h1);
        }
        phi[s] = __builtin_bit_cast(bf16x8_t, wh);
        plo[s] = __builtin_bit_cast(bf16x8_t, wl);
      }
      // V^T fragments (A operand) by transpose reads: in 16-lane group g,
      // lane lg points at key k0 + lg/4, column n0 + 4(lg%4); it receives
      // the four keys k0..k0+3 of column n0 + lg.
      const int g = lane >> 4, lg = lane & 15;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          s16x4_t part[2];
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int key = 16 * s + 8 * r + 4 * (g >> 1) + (lg >> 2);
            const int col = 32 * n + 16 * (g & 1) + 4 * (lg & 3);
            part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t *)(vs + key * T::VROW + col));
          }
          const bf16x8_t vf = __builtin_bit_cast(
              bf16x8_t, u32x4{(uint32_t)(uint16_t)part[0][0] | ((uint32_t)(uint16_t)part[0][1] << 16),
                              (uint32_t)(uint16_t)part[0][2] | ((uint32_t)(uint16_t)part[0][3] << 16),
                              (uint32_t)(uint16_t)part[1][0] | ((uint32_t)(uint16_t)part[1][1] << 16),
                              (uint32_t)(uint16_t)part[1][2] | ((uint32_t)(uint16_t)part[1][3] << 16)});
          oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, phi[s], oacc[n], 0, 0, 0);
          oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, plo[s], oacc[n], 0, 0, 0);
        }
      }
    }
  }

  // Per-wave row statistics: lanes l and l + 32 hold the same m and halves of l.
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // every wave is done with its tile buffers
  if (h == 0) {
    sh.out.m[wave][j] = m;
    sh.out.l[wave][j] = lsum;
  }
  if constexpr (!ENERGY) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sh.out.o[wave][j][32 * n + 8 * (e >> 2) + 4 * h + (e & 3)] = oacc[n][e];
  }
  __syncthreads();
  const int64_t rec0 = ((int64_t)group * a.part.chunks + chunk) * a.part.rows + rb * kRows;
  constexpr int kOut = ENERGY ? kRows : kRows * D;
  for (int idx = threadIdx.x; idx < kOut; idx += kThreads) {
    const int r = ENERGY ? idx : idx / D;
    const int d = ENERGY ? 0 : idx - r * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sh.out.m[w][r]);
    float acc = 0.0f, ls = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = rescale_factor(sh.out.m[w][r], M);
      if constexpr (!ENERGY) acc += sh.out.o[w][r][d] * f;
      ls += sh.out.l[w][r] * f;
    }
    if constexpr (!ENERGY) a.part.o[(rec0 + r) * D + d] = acc;
    if (d == 0) {
      a.part.m[rec0 + r] = M;
      a.part.l[rec0 + r] = ls;
    }
  }
}

template <int D, bool ENERGY>
hipError_t launch(const attn_plan_t &plan, const SplitArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((split_kv_mfma<D, ENERGY>), dim3((unsigned)plan.work_items), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_mfma(const attn_plan_t &plan, const SplitArgs &a, int head_dim,
                             bool energy_only, hipStream_t stream) {
  if (plan.work_items <= 0) return hipSuccess;
  if (plan.rows_per_block != kRows) return hipErrorInvalidValue;
  if (head_dim == 64)
    return energy_only ? launch<64, true>(plan, a, stream) : launch<64, false>(plan, a, stream);
  if (head_dim == 128)
    return energy_only ? launch<128, true>(plan, a, stream) : launch<128, false>(plan, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
