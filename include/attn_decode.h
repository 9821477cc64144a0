/*
 * attn_decode.h -- exact split-KV softmax attention decoding on AMD Instinct
 * MI355X (gfx950).  C ABI: plain pointers, sizes and status codes.
 *
 * What is computed.  For every query row (sequence b, query token i, query
 * head h) the library returns the attention output
 *     O = sum_t softmax_t(scale * q . k_t) v_t
 * and its logsumexp ("energy")
 *     lse = ln sum_t exp(scale * q . k_t)
 * over the visible keys t of KV head h / (Hq / Hkv).  This is the plain
 * definition S = Q K^T / sqrt(d_k), P = softmax(S), O = P V of the "attention
 * acceleration" concept page (technical principles, section 1).  The cache is
 * cut into chunks; each chunk yields the statistics m = max, l = sum e^(s-m)
 * and the unnormalised partial output o (same page, section 2.1, online
 * softmax), and the partials are combined by the associative merge
 *     m = max(m_a, m_b), l = l_a e^(m_a-m) + l_b e^(m_b-m), o likewise,
 * which is exact in any order because max and logsumexp are associative
 * (Tree Attention article, "an energy view of attention").  Star Attention's
 * phase 2 (query encoding and token generation) aggregates the same softmax
 * statistics across hosts; here the chunks of one GPU play the hosts.
 *
 * Layouts (row-major, last axis contiguous, 16-byte aligned base pointers):
 *     Q    [B][q_len][Hq][D]      element type attn_dtype_t
 *     K, V [B][Hkv][L_max][D]     element type attn_dtype_t
 *     O    [B][q_len][Hq][D]      float32
 *     lse  [B][q_len][Hq]         float32 (natural log)
 * Query head h reads KV head h / G with G = Hq / Hkv (contiguous groups).
 * kv_lens[b] is the number of cached tokens of sequence b (tokens at or past
 * kv_lens[b] are never read, so they may hold anything, NaN included).  With
 * causal = 1 the q_len new tokens are the last q_len cached positions and
 * query token i sees keys t <= kv_lens[b] - q_len + i.  A row that sees no
 * key gets O = 0 and lse = -inf.
 *
 * Ownership and streams.  The caller allocates every buffer (device memory
 * for tensors, kv_lens and the workspace) and keeps it alive until the work
 * on the stream completes.  The library allocates nothing, keeps no device
 * state, never synchronises, and caches only the CU count per device.  All
 * work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 * The calls enqueue kernel launches only (no memset, copy or allocation), so
 * a call may be captured into a HIP graph on a capturing stream and the
 * graph replayed, as long as every buffer it names stays alive.
 *
 * Null tensors are accepted where they would hold no element (K and V when
 * max_kv_len == 0, every tensor when B == 0).
 *
 * Errors.  Arguments are validated on the host before anything is launched;
 * on error nothing is enqueued or written and a status other than ATTN_OK is
 * returned.  ATTN_ERR_HIP reports a failed launch.  No C++ exception crosses
 * the ABI.  Non-finite inputs propagate into the outputs unchecked.  The
 * values of kv_lens live on the device and cannot be checked on the host:
 * they are clamped to [0, max_kv_len] inside the kernels.
 * Thread safety: every function is reentrant.
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>

/* Exported symbols: the library is built with hidden default visibility and
 * exports exactly the functions declared with ATTN_API. */
#if defined(__GNUC__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL                         */
  ATTN_ERR_SHAPE = 2,       /* a size is out of range or Hq % Hkv != 0            */
  ATTN_ERR_DTYPE = 3,       /* unknown element type                               */
  ATTN_ERR_ALIGN = 4,       /* a tensor base is not 16-byte (4-byte for fp32 out) aligned */
  ATTN_ERR_WORKSPACE = 5,   /* workspace smaller than the size query returned     */
  ATTN_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed          */
  ATTN_ERR_UNSUPPORTED = 7, /* head_dim other than 64 or 128, or a shape the kernels do not cover */
  ATTN_ERR_VALUE = 8,       /* non-finite scale, chunk_len not a multiple of 64, or a bad */
                            /* paging description (page size, strides, table extent)     */
  ATTN_ERR_SCRATCH = 9      /* attn_decode_static: the call's records exceed the static   */
                            /* scratch array (ATTN_STATIC_SCRATCH_BYTES)                   */
} attn_status_t;

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1 } attn_dtype_t;

/* One decode call.  B = batch >= 0, q_len >= 1, Hq % Hkv == 0, D in {64, 128},
 * 0 <= max_kv_len <= 2^31 - 2^16.  kv_lens: device int32[B], or NULL for "every
 * sequence holds max_kv_len tokens".  scale: logit multiplier, normally
 * 1/sqrt(D).  chunk_len: 0 lets the partitioner choose the chunk length; a
 * positive multiple of 64 forces it. */
typedef struct {
  int32_t batch;
  int32_t q_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t causal;
  int64_t max_kv_len;
  const int32_t *kv_lens;
  float scale;
  int32_t chunk_len;
  attn_dtype_t dtype;
} attn_desc_t;

/* The partitioner's decision for a descriptor (introspection and tests).
 * Segments are the (sequence, KV head, row block) triples; each is one KV
 * head's L_b cached tokens read for one block of query rows. */
typedef struct {
  int32_t kernel;            /* 0: VALU split-KV kernel, 1: MFMA query-block kernel (32    */
                             /*    rows), 2: MFMA shared-tile kernel (64-256 rows)          */
  int32_t rows;              /* R = (Hq / Hkv) * q_len query rows per (b, KV head)          */
  int32_t rows_per_block;    /* query rows one segment carries                              */
  int32_t row_blocks;        /* ceil(R / rows_per_block)                                    */
  int32_t balanced;          /* 1: every workgroup streams an equal share of all segments'  */
                             /*    tokens (lengths read on the device); 0: fixed chunks     */
  int32_t chunk_len;         /* fixed: C; balanced: tokens per workgroup if all L_b = L_max */
  int32_t chunks_per_seq;    /* fixed: ceil(max_kv_len / C); balanced: 0                    */
  int32_t threads_per_item;  /* threads per workgroup                                       */
  int64_t work_items;        /* workgroups launched                                         */
  int64_t record_slots;      /* partial-record slots (each holds rows_per_block rows)       */
  int32_t cu_count;          /* compute units the plan was sized for                        */
  size_t workspace_bytes;    /* partial (m, l, o) records                                   */
} attn_plan_t;

/* Partition a decode call for `cu_count` compute units (<= 0: those of the
 * current device).  Splits each sequence's KV into chunks of C tokens so that
 * the work items fill the GPU (Tree Attention's per-device local energies and
 * Star Attention's per-host context blocks, placed on CUs).  Pure host code
 * when cu_count > 0. */
ATTN_API attn_status_t attn_decode_plan(const attn_desc_t *desc, int32_t cu_count, attn_plan_t *plan);

/* Bytes of device workspace that attn_decode, attn_decode_energy,
 * attn_decode_energy_zeta and the paged variants need for `desc` on the
 * current device (0 is possible for an empty call). */
ATTN_API attn_status_t attn_workspace_bytes(const attn_desc_t *desc, size_t *bytes);

/* lse only: the energy F at zeta = 0, i.e. the logsumexp of every row, read
 * from K alone (Tree Attention article, "an energy view of attention": the
 * local energies are computed in parallel and combined by an associative
 * reduction).  lse: float32 [B][q_len][Hq]. */
ATTN_API attn_status_t attn_decode_energy(const attn_desc_t *desc, const void *q, const void *k,
                                 float *lse, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* O and lse (definition above).  v has the layout of k. */
ATTN_API attn_status_t attn_decode(const attn_desc_t *desc, const void *q, const void *k, const void *v,
                          float *o, float *lse, void *workspace, size_t workspace_bytes,
                          void *stream);

/* The two phases of attn_decode / attn_decode_energy, for callers that time
 * them separately or move the records between devices before merging (Tree
 * Attention computes local energies per device and then reduces them; Star
 * Attention's query host aggregates the hosts' softmax statistics).
 *
 * attn_decode_partials: (m, l, o) records for every piece of work into
 * `workspace` (sized by attn_workspace_bytes).  With v == NULL only (m, l)
 * are produced (energy only).  For the plan P of attn_decode_plan, with
 * Nr = P.record_slots * P.rows_per_block and X = roundup(4 * Nr, 256) bytes:
 *   float m[Nr] at byte 0        -- piece max of the scaled logits, log2 units
 *   float l[Nr] at byte X        -- sum of 2^(s * log2e - m) over the piece
 *   float o[Nr][D] at byte 2X    -- unnormalised output of the piece
 * Record slot k holds rows k*rows_per_block .. +rows_per_block-1 of one piece.
 * Fixed chunks: slot = segment * chunks_per_seq + c covers tokens
 * [c*C, (c+1)*C) and exists for c < ceil(L_b / C).  Balanced: the segments
 * (segment = (b*Hkv + kvh)*row_blocks + row block) are laid end to end into
 * U = Hkv*row_blocks*sum(L_b) tokens; workgroup w covers [floor(wU/W),
 * floor((w+1)U/W)) and its piece of segment s sits at slot w + s.
 * Row r of a row block is query token r / G, head kvh*G + r % G.
 *
 * attn_decode_merge: merges each row's records (exact in any order), then
 * O = o / l and lse = (m + log2 l) * ln 2.  o == NULL gives lse only; o !=
 * NULL requires records produced with v != NULL.  Same desc and workspace as
 * the attn_decode_partials call that filled it; errors as above. */
ATTN_API attn_status_t attn_decode_partials(const attn_desc_t *desc, const void *q, const void *k,
                                   const void *v, void *workspace, size_t workspace_bytes,
                                   void *stream);
ATTN_API attn_status_t attn_decode_merge(const attn_desc_t *desc, float *o, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Energy at a given zeta (Tree Attention article, "an energy view of
 * attention"): for every row, with the row's auxiliary vector zeta,
 *     F(zeta) = ln sum_t exp(scale * q . k_t + zeta . v_t)
 * over the row's visible keys.  F(0) is the row's lse, and the gradient of F
 * in zeta at 0 is the row's attention output O, so central differences of
 * this call reproduce attn_decode's O.  zeta: [B][q_len][Hq][D], element
 * type and alignment of q.  lse receives F(zeta), float32 [B][q_len][Hq].
 * Runs on the vector-ALU kernel for every row count; dense caches only. */
ATTN_API attn_status_t attn_decode_energy_zeta(const attn_desc_t *desc, const void *q, const void *k,
                                      const void *v, const void *zeta, float *lse,
                                      void *workspace, size_t workspace_bytes, void *stream);

/* Paged KV caches ("attention acceleration" concept page, section 3,
 * PagedAttention): K and V live in pools of fixed-size pages of P tokens; a
 * block table maps logical page j of sequence b (tokens [jP, (j+1)P)) to a
 * physical page.  Pages need not be contiguous or in order, and several
 * sequences may map the same page (a shared prompt prefix).  Element e of
 * the row of token t, KV head kvh, sequence b is
 *     pool[block_table[b * pages_per_seq + t / P] * page_stride
 *          + kvh * head_stride + (t % P) * token_stride + e].
 * Two common layouts: head-major pages [num_pages][Hkv][P][D]
 * (page_stride = Hkv*P*D, head_stride = P*D, token_stride = D) and
 * token-major pages [num_pages][P][Hkv][D] (P*Hkv*D, D, Hkv*D).
 *   block_table     device int32 [B][pages_per_seq]; only the entries of pages
 *                   that hold tokens t < kv_lens[b] are read; an entry outside
 *                   [0, num_pages) is read as page 0 (memory-safe, result
 *                   unspecified)
 *   pages_per_seq   >= 1 and pages_per_seq * P >= max_kv_len
 *   page_size       P, a power of two in [1, 2^20]
 *   num_pages       pages in each pool (>= 1 when any token is cached)
 *   strides         in elements, >= 0, each a multiple of 16 bytes; D
 *                   consecutive elements per row; num_pages * page_stride
 *                   below 2^48
 * Everything else (descriptor, q, outputs, workspace, errors) is as for the
 * dense entry points; desc->max_kv_len is the logical extent of the token
 * axis.  Identical results to the dense call on the cache the table
 * describes: paging changes where rows are read, not the arithmetic. */
typedef struct {
  const int32_t *block_table;
  int32_t pages_per_seq;
  int32_t page_size;
  int64_t num_pages;
  int64_t page_stride;
  int64_t head_stride;
  int64_t token_stride;
} attn_paged_kv_t;

ATTN_API attn_status_t attn_decode_paged(const attn_desc_t *desc, const attn_paged_kv_t *paged,
                                const void *q, const void *k_pool, const void *v_pool, float *o,
                                float *lse, void *workspace, size_t workspace_bytes, void *stream);
ATTN_API attn_status_t attn_decode_energy_paged(const attn_desc_t *desc, const attn_paged_kv_t *paged,
                                       const void *q, const void *k_pool, float *lse,
                                       void *workspace, size_t workspace_bytes, void *stream);
/* The split phase alone on a paged cache (records as attn_decode_partials;
 * attn_decode_merge then finishes the call). */
ATTN_API attn_status_t attn_decode_partials_paged(const attn_desc_t *desc, const attn_paged_kv_t *paged,
                                         const void *q, const void *k_pool, const void *v_pool,
                                         void *workspace, size_t workspace_bytes, void *stream);

/* Shared-prefix batch sampling (Bifurcated Attention, TL;DR): S samples of
 * one query token each attend over one shared prefix KV followed by their
 * own decoded KV.  The prefix part runs as one multi-row contraction per KV
 * head, so the prefix is read once for all samples; prefix and suffix
 * partials are then merged exactly.  bf16 only; D in {64, 128}.
 *     Q  [S][Hq][D]; Kp, Vp [Hkv][Lp][D]; Ks, Vs [S][Hkv][Ls][D]  (bf16)
 *     O  [S][Hq][D] float32;  lse [S][Hq] float32
 * Lp >= 0 and Ls >= 0; when both are 0 every row is empty. */
typedef struct {
  int32_t num_samples;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int64_t prefix_len;
  int64_t suffix_len;
  float scale;
  attn_dtype_t dtype;
} attn_bifurcated_desc_t;

ATTN_API attn_status_t attn_bifurcated_workspace_bytes(const attn_bifurcated_desc_t *desc, size_t *bytes);

ATTN_API attn_status_t attn_decode_bifurcated(const attn_bifurcated_desc_t *desc, const void *q,
                                     const void *k_prefix, const void *v_prefix,
                                     const void *k_suffix, const void *v_suffix, float *o,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* Context encoding with an anchor block (Star Attention, phase 1: the
 * context is cut into blocks, and every block after the first is processed
 * with the first block, the anchor, placed in front of it).  Block b's query
 * token i attends over [anchor ; block b]: every anchor key, and the block's
 * own keys t <= i (causal within the block).  The anchor is read in place
 * by every block (no copy), its part of each row is merged exactly with the
 * block's own part.  bf16 only; D in {64, 128}; (Hq/Hkv) * block_len <=
 * 65536.  The first block itself is the case anchor_len = 0.
 *     Q  [N][Lb][Hq][D]; Ka, Va [Hkv][A][D]; Kb, Vb [N][Hkv][Lb][D]  (bf16)
 *     O  [N][Lb][Hq][D] float32;  lse [N][Lb][Hq] float32
 * Errors as for the decode entry points. */
typedef struct {
  int32_t num_blocks;
  int32_t block_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int64_t anchor_len;
  float scale;
  attn_dtype_t dtype;
} attn_anchor_desc_t;

ATTN_API attn_status_t attn_anchor_workspace_bytes(const attn_anchor_desc_t *desc, size_t *bytes);

ATTN_API attn_status_t attn_prefill_anchor(const attn_anchor_desc_t *desc, const void *q,
                                  const void *k_anchor, const void *v_anchor,
                                  const void *k_blocks, const void *v_blocks, float *o,
                                  float *lse, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* attn_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The partial records go to a device
 * array the library holds, ATTN_STATIC_SCRATCH_BYTES bytes on every GPU it
 * runs on, kept until the process ends; its address is looked up on the
 * first call on each device.  The call allocates nothing.  Same arguments
 * (minus the workspace), results and errors as attn_decode, plus
 * ATTN_ERR_SCRATCH when the call needs more record space than the array
 * holds (attn_workspace_bytes tells; 16 MiB covers, e.g., the 5.12M-token
 * GQA decode and a 16-sequence batch of 4-token query blocks over 128K
 * tokens each).  Every call on one GPU uses the same array: calls that
 * overlap on one GPU (on different streams, or from different threads
 * without ordering) race and give wrong results.  Each call writes every
 * record it reads, so nothing needs clearing between calls. */
#define ATTN_STATIC_SCRATCH_BYTES (16u << 20)
ATTN_API attn_status_t attn_decode_static(const attn_desc_t *desc, const void *q, const void *k,
                                          const void *v, float *o, float *lse, void *stream);

/* Merge of results computed over disjoint shares of the keys -- the
 * exchange step of a sequence-sharded decode.  When each of N devices holds
 * a share of every sequence's tokens, each runs attn_decode on its share,
 * and the N (O, lse) pairs of every row (gathered on one device) give the
 * row's result over all its keys: (O_p, lse_p) is the record (m = lse_p,
 * l = 1, o = O_p), so with M = max_p lse_p and w_p = e^(lse_p - M)
 *     O = sum_p w_p O_p / sum_p w_p,   lse = M + ln sum_p w_p
 * (Star Attention article, phase 2: the query host combines the hosts'
 * local outputs by their softmax statistics; Tree Attention article, "an
 * energy view of attention": the local energies are reduced across
 * devices).  Exact up to rounding for any cut of the keys into shares.
 *     o_parts   float32 [n_parts][rows][D]   (part p, row r at (p*rows + r)*D)
 *     lse_parts float32 [n_parts][rows]      natural log
 *     o         float32 [rows][D];  lse float32 [rows]
 * n_parts >= 1, 0 <= rows <= 2^25, D = head_dim in {64, 128}; 4-byte
 * aligned pointers; the outputs must not overlap the inputs.  A part with
 * lse_p = -inf (it saw no key) adds nothing and its O_p is not read; a row
 * whose every part is -inf gets O = 0 and lse = -inf.  With o_parts and o
 * both NULL only lse is merged (lse = ln sum_p e^(lse_p): the energies of
 * attn_decode_energy on each share reduced to the energy over all keys).
 * One launch on `stream`, nothing allocated; errors as above
 * (ATTN_ERR_SHAPE for n_parts or rows out of range, ATTN_ERR_UNSUPPORTED
 * for head_dim, ATTN_ERR_NULL when only one of o_parts and o is NULL). */
ATTN_API attn_status_t attn_merge_results(int32_t n_parts, int64_t rows, int32_t head_dim,
                                          const float *o_parts, const float *lse_parts, float *o,
                                          float *lse, void *stream);

/* Static text for a status code. */
ATTN_API const char *attn_status_string(attn_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_H */
