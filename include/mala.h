/*
 * mala.h - C ABI of libmala, MassAlloc Attention (MALA) for AMD MI355X (gfx950).
 *
 * The operator is the one defined in "MassAlloc Attention: Let Attention
 * Allocate Its Own Compute" (arXiv 2609.32712):
 *   - forward: every legal causal Q K^T tile is scored; the post-score work
 *     (softmax update, V load, P V) runs only for tiles whose largest
 *     contribution ratio against the running normalizer clears tau / L_q
 *     (Sec. 2.2, Eq. 1-3, Algorithm 1);
 *   - backward: S is recomputed and each tile is tested against the saved
 *     log-normalizer (Sec. 2.2, Eq. 4, Algorithm 2);
 *   - split-KV decode: each split tests its tiles against its own partial
 *     normalizer with L counting the full context; partials are merged by
 *     the normalizer-aware reduction (Sec. 2.4, App. A.1).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, head-major: Q, O, dO, dQ are
 *     [batch, n_q_heads, n_q, head_dim]; K, V, dK, dV are
 *     [batch, n_kv_heads, n_k, head_dim]; LSE is [batch, n_q_heads, n_q].
 *     Query head h reads KV head h / (n_q_heads / n_kv_heads) (grouped-query
 *     attention). Base pointers must be 16-byte aligned.
 *   - Element type: MALA_BF16 (bfloat16 Q/K/V/O/dO/dQ/dK/dV) or MALA_F32.
 *     LSE, workspaces and all internal accumulation are fp32.
 *   - Scores are s = softmax_scale * <q, k>; logarithms are natural (Sec. 2.1).
 *   - Causal legality is bottom-right aligned: key k is visible to query row q
 *     iff k <= q + (n_k - n_q); L_q = q + (n_k - n_q) + 1 (L_q = n_k when not
 *     causal). tau must be finite and >= 0; tau = 0 skips nothing, which is
 *     dense softmax attention (Sec. 2.3).
 *   - All pointers except `p` and the tiling outputs are device pointers.
 *     The caller owns every buffer; the library allocates nothing, keeps no
 *     state between calls (mala_decode_noalloc's fixed device scratch aside)
 *     and never synchronizes: work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and the call returns.
 *   - Errors: a non-MALA_OK status means nothing was enqueued and no output
 *     was written; mala_last_error() describes it (thread-local). A fault
 *     inside a kernel surfaces at the caller's next synchronization.
 *   - Optional diagnostics (pass NULL to disable) report the decisions, which
 *     the operator itself never materializes (Sec. 2.4): an int8 tile mask
 *     (1 kept, 0 skipped, -1 not a legal tile) and int32 kept-tile counters.
 */
#ifndef MALA_H_
#define MALA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MALA_OK = 0,
  MALA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, bad tau  */
  MALA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. head_dim)   */
  MALA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required  */
  MALA_ERR_HIP = 4            /* a HIP launch reported an error              */
} mala_status;

typedef enum { MALA_F32 = 0, MALA_BF16 = 1 } mala_dtype;

typedef enum { MALA_OP_FWD = 0, MALA_OP_BWD = 1, MALA_OP_DECODE = 2 } mala_op;

/* Problem flags. */
enum {
  /* bf16 backward: multiply dS into dQ as one bf16 operand (as dK always
   * takes it) instead of a hi + lo pair of bf16 operands. Faster (one fewer
   * matrix product per kept tile and key column) and less accurate: dQ errors
   * grow to ~2^-9 of the summed terms, which can exceed 1% of the result
   * where the terms of a row cancel. */
  MALA_FLAG_FAST_GRAD = 1,
  /* bf16 backward: take the offline gate (Eq. 4) of every legal tile in a
   * separate score pass before dK/dV, and let dK/dV stage and process only
   * the 64-row steps that hold a kept tile, so that a skipped tile costs no
   * dO load (App. A.1, "Fused backward execution"). Every legal score is
   * still formed, unless mala_bwd_nested passes the forward's tile mask:
   * then only the forward's kept tiles are scored. Pays off when few tiles
   * are kept (trained attention, larger tau); on inputs where every tile is
   * kept the score pass costs about a tenth of the backward and the walks
   * gain part of it back (+4% in all at 32K). The decisions may differ from
   * those of the default path only for tiles whose margin is within fp32
   * rounding of the threshold. Ignored for MALA_F32. */
  MALA_FLAG_GATE_PASS = 2
};

/* One prefill/training attention problem. */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;      /* divides n_q_heads                              */
  int32_t n_q;             /* query rows per head (>= 0)                     */
  int32_t n_k;             /* key rows per head (>= 0; >= n_q when causal)   */
  int32_t head_dim;        /* 64 or 128                                      */
  int32_t dtype;           /* mala_dtype                                     */
  int32_t causal;          /* nonzero: causal mask (bottom-right aligned)    */
  float tau;               /* tolerance, finite, >= 0                        */
  float softmax_scale;     /* finite, > 0; usually 1/sqrt(head_dim)          */
  int32_t flags;           /* MALA_FLAG_* (0 = defaults)                     */
} mala_problem;

/* One split-KV decode step: a single query token per sequence.
 * batch * n_kv_heads must not exceed 65535 (MALA_ERR_UNSUPPORTED), and a
 * KV head groups at most 16 query heads. */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;        /* 128 for MALA_BF16; 64 or 128 for MALA_F32      */
  int32_t cache_capacity;  /* rows per (sequence, KV head) in the caches     */
  int32_t max_n_k;         /* upper bound of seqlens_k; sizes the launch     */
  int32_t dtype;           /* mala_dtype                                     */
  float tau;
  float softmax_scale;
  int32_t split_keys;      /* keys per split: 0 = the default (256),
                              MALA_DECODE_SPLIT_AUTO = chosen from the problem
                              size, else a positive multiple of 64; a split
                              longer than max_n_k is one split per sequence.
                              mala_decode_split_keys() reports the value used. */
} mala_decode_problem;

/* split_keys: pick the split length from the problem (see mala_decode_split_keys). */
enum { MALA_DECODE_SPLIT_AUTO = -1 };

/*
 * Decision partition used by an operation (the pages leave B_q and B_k open,
 * Sec. 2.1; the realized support depends on it).
 *   op = MALA_OP_FWD:    *bq x *bk query x key tiles, both tiled from 0.
 *   op = MALA_OP_BWD:    *bq x *bk tiles; they refine the forward tiles, so a
 *                        forward-skipped tile is backward-skipped (Sec. 2.2).
 *   op = MALA_OP_DECODE: *bq = 1 (one decision per query head), *bk keys per
 *                        tile, *chunk the default keys per split (a problem
 *                        may choose another length: mala_decode_split_keys);
 *                        splits are aligned to position 0 and tiles to the
 *                        split start; the newest tile of a split is tested
 *                        first.
 * *chunk is 0 for FWD/BWD. Returns MALA_ERR_INVALID_ARG for an unknown op or
 * a null output pointer.
 */
mala_status mala_get_tiling(int32_t op, int32_t dtype, int32_t head_dim,
                            int32_t* bq, int32_t* bk, int32_t* chunk);

/*
 * Forward (Algorithm 1; Sec. 2.2 "Online Sparse Softmax").
 *   q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d]  inputs
 *   o [B,Hq,Nq,d]                     output: softmax over the retained keys
 *   lse [B,Hq,Nq] fp32                output: z_q = log Z_{R,q} (natural log),
 *                                     the state the backward needs
 *   tile_mask  int8 [B,Hq,Tr,Tc] or NULL, Tr = ceil(Nq/bq), Tc = ceil(Nk/bk)
 *   kept_tiles int32 [B,Hq,Tr] or NULL: kept tiles per query block; the
 *              post-score key slots of each row are bk * kept_tiles (Eq. 11).
 */
mala_status mala_fwd(const mala_problem* p, const void* q, const void* k, const void* v,
                     void* o, float* lse, int8_t* tile_mask, int32_t* kept_tiles,
                     void* stream);

/* Bytes of device workspace mala_bwd needs for problem p (the per-row
 * D = rowsum(O o dO) in fp32 and one decision bit per backward tile; with
 * MALA_FLAG_GATE_PASS on a bf16 problem also fp32 dK, dV partials per query
 * head, 8 * B * Hq * Nk * d bytes, and 4 bytes per batch, KV head and
 * 128-key block); 0 if p is invalid. The size depends on p->flags. */
size_t mala_bwd_workspace_size(const mala_problem* p);

/*
 * Backward (Algorithm 2; Sec. 2.2 "Offline Sparse Probability").
 *   q, k, v, o, lse  as produced/consumed by mala_fwd (o and lse from the
 *                    forward call on the same q, k, v, tau)
 *   d_o [B,Hq,Nq,d]  upstream gradient
 *   dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d]  outputs (dk, dv summed over the
 *                    query heads sharing a KV head)
 *   workspace, ws_bytes  >= mala_bwd_workspace_size(p), 256-byte aligned
 *   tile_mask  int8 [B,Hq,Tr,Tcb] or NULL with the backward tiling
 *   kept_tiles int32 [B,Hq,Tr] or NULL: kept backward tiles per query block
 */
mala_status mala_bwd(const mala_problem* p, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* d_o,
                     void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                     int8_t* tile_mask, int32_t* kept_tiles, void* stream);

/*
 * Backward on the forward's retained support (Sec. 2.2, "Offline Sparse
 * Probability": the finalized normalizer is at least every partial one the
 * forward tested against, so with the same tile partition a tile the forward
 * skipped also meets the backward skip condition, and the backward support
 * nests in the forward's). This is mala_bwd in the MALA_FLAG_GATE_PASS mode
 * whose score pass forms only the scores of the forward's kept tiles: the
 * cost of the decisions then follows the forward's kept fraction instead of
 * the number of legal tiles.
 *   fwd_tile_mask  int8 [B,Hq,Tr,Tc] (device) with the forward tiling
 *                  (mala_get_tiling(MALA_OP_FWD)): the tile_mask mala_fwd
 *                  wrote for the same problem, q, k and v. A tile is scored
 *                  iff its entry is 1; its contents are not checked.
 *   the other arguments as for mala_bwd; p->flags must include
 *                  MALA_FLAG_GATE_PASS (else MALA_ERR_INVALID_ARG), and the
 *                  workspace is mala_bwd_workspace_size(p).
 * The decisions are those of mala_bwd with the same flags except for a tile
 * that the gate pass would keep while the forward skipped it, which exact
 * arithmetic rules out: both margins then lie within fp32 rounding of the
 * threshold. For MALA_F32 the forward mask is not read and the call is
 * mala_bwd.
 */
mala_status mala_bwd_nested(const mala_problem* p, const void* q, const void* k, const void* v,
                            const void* o, const float* lse, const void* d_o,
                            const int8_t* fwd_tile_mask, void* dq, void* dk, void* dv,
                            void* workspace, size_t ws_bytes, int8_t* tile_mask,
                            int32_t* kept_tiles, void* stream);

/*
 * The backward with its dK/dV walk chosen on the device: the gate-pass walks
 * (MALA_FLAG_GATE_PASS: the Eq. 4 decisions of every legal tile in a
 * separate score pass, then only the steps that hold a kept tile) or the
 * default walk, whichever the step's sparsity favours. Both recompute every
 * legal score before its decision (Sec. 2.2 "Offline Sparse Probability";
 * App. A.1 "Fused backward execution"); the result is, bit for bit, that of
 * mala_bwd with MALA_FLAG_GATE_PASS when the gate-pass walks are taken and
 * that of mala_bwd without it otherwise.
 * The rule: the Eq. 4 decisions are first taken on a sample: about 256 of
 * the blocks of 256 query rows over all heads, and about 8 key tiles of each
 * block's walk (the whole backward gate when there are fewer than 512 such
 * blocks and at most 1,984 keys, fewer than 32 tiles of 64). If it holds at least 256 legal 16-key
 * columns, the
 * gate-pass walks run when fewer than 60% of them are kept. Otherwise the
 * forward's counters decide: the gate-pass walks when the forward kept fewer
 * than 70% of its legal tiles. The choice needs no host round trip: a
 * one-workgroup kernel reduces the counts, both walks' kernels are launched,
 * and the workgroups of the walk not taken return at once.
 *   fwd_kept_tiles int32 [B,Hq,Tr] (device), Tr = ceil(Nq/bq) with the
 *                  forward tiling: the kept_tiles mala_fwd wrote for the same
 *                  problem, q, k and v. Required when n_q > 0.
 *   the other arguments as for mala_bwd; p->flags must not include
 *                  MALA_FLAG_GATE_PASS (MALA_ERR_INVALID_ARG), and the
 *                  workspace is mala_bwd_workspace_size of p with
 *                  MALA_FLAG_GATE_PASS added to p->flags (MALA_ERR_WORKSPACE
 *                  if smaller).
 * For MALA_F32 nothing is sampled, the counters are not read and the call
 * is mala_bwd.
 */
mala_status mala_bwd_auto(const mala_problem* p, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* d_o,
                          const int32_t* fwd_kept_tiles, void* dq, void* dk, void* dv,
                          void* workspace, size_t ws_bytes, int8_t* tile_mask,
                          int32_t* kept_tiles, void* stream);

/*
 * The backward as three stages, for callers that schedule or time them
 * separately. Calling MALA_BWD_PREP, MALA_BWD_DKDV, MALA_BWD_DQ in this order
 * on one stream with the same arguments and workspace is mala_bwd.
 *   PREP: D = rowsum(O o dO) into the workspace; clears the decision bits and
 *         kept_tiles, and sets tile_mask to -1.
 *   DKDV: key-major pass: recomputes S, applies the offline gate (Eq. 4),
 *         writes the decisions (bits, tile_mask), dK and dV.
 *   DQ:   query-major pass over the kept tiles recorded by DKDV: writes dQ;
 *         kept_tiles is complete once this stage has run.
 * Same argument checks and errors as mala_bwd; an unknown stage is
 * MALA_ERR_INVALID_ARG.
 */
enum { MALA_BWD_PREP = 0, MALA_BWD_DKDV = 1, MALA_BWD_DQ = 2 };
mala_status mala_bwd_stage(int32_t stage, const mala_problem* p, const void* q, const void* k,
                           const void* v, const void* o, const float* lse, const void* d_o,
                           void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                           int8_t* tile_mask, int32_t* kept_tiles, void* stream);

/* Bytes of device workspace mala_decode needs (per-split partial states and
 * decision bits). */
size_t mala_decode_workspace_size(const mala_decode_problem* p);

/*
 * Keys per split that mala_decode uses for problem p, or 0 if p is invalid.
 * Each split starts with an empty running state and tests its tiles against
 * its own partial normalizer (Sec. 2.2, split-KV decoding; App. A.1 "Fused
 * decoding execution"), so the retained support depends on this length:
 * longer splits test more tiles against a more complete normalizer (fewer
 * forced first tiles) but leave fewer splits to run in parallel.
 *   split_keys = 0:                      256
 *   split_keys = MALA_DECODE_SPLIT_AUTO: the shortest multiple of 256 (at
 *       least 256) that gives at most 1024 splits over batch x KV heads:
 *       256 * ceil(max_n_k / (256 * max(1, 1024 / (batch * n_kv_heads))))
 *   split_keys > 0:                      split_keys (a multiple of 64)
 * The result is then capped at max_n_k rounded up to 64 (one split per
 * sequence). n_chunks = ceil(max_n_k / split) splits of split / 64 tiles.
 */
int32_t mala_decode_split_keys(const mala_decode_problem* p);

/*
 * Split-KV decode (Sec. 2.4; App. A.1 "Fused decoding execution").
 *   q [B,Hq,d]                     the query token of each sequence, at
 *                                  position seqlens_k[b] - 1
 *   k_cache, v_cache [B,Hkv,cache_capacity,d]  persistent caches (read only;
 *                                  the current token's K/V already written)
 *   seqlens_k int32 [B] (device)   N_k per sequence, 1 <= N_k <= max_n_k
 *                                  <= cache_capacity (checked on the device:
 *                                  out-of-range lengths are clamped)
 *   o [B,Hq,d], lse [B,Hq] fp32    outputs
 *   workspace, ws_bytes            >= mala_decode_workspace_size(p)
 *   tile_mask  int8 [B,Hq,n_chunks,split/bk] or NULL (split =
 *              mala_decode_split_keys(p), n_chunks = ceil(max_n_k/split));
 *              entries past a sequence's end are -1
 *   kept_tiles int32 [B,Hq+Hkv] or NULL: [b][h] kept tiles of query head h,
 *              [b][Hq+g] tiles of KV head g whose V was read (kept by at least
 *              one query head of the group)
 */
mala_status mala_decode(const mala_decode_problem* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* seqlens_k, void* o, float* lse,
                        void* workspace, size_t ws_bytes, int8_t* tile_mask,
                        int32_t* kept_tiles, void* stream);

/*
 * Split-KV decode as two stages (MALA_DECODE_SPLIT then MALA_DECODE_COMBINE,
 * same arguments and workspace, one stream) is mala_decode. SPLIT scores every
 * key, gates the tiles of each split and writes the partial states, the
 * decision bits and tile_mask; COMBINE merges the partial states into o and
 * lse and counts the decision bits into kept_tiles.
 */
enum { MALA_DECODE_SPLIT = 0, MALA_DECODE_COMBINE = 1 };
mala_status mala_decode_stage(int32_t stage, const mala_decode_problem* p, const void* q,
                              const void* k_cache, const void* v_cache, const int32_t* seqlens_k,
                              void* o, float* lse, void* workspace, size_t ws_bytes,
                              int8_t* tile_mask, int32_t* kept_tiles, void* stream);

/*
 * Split-KV decode that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. It is mala_decode without the workspace
 * argument (same problem, inputs, outputs, diagnostics and results): the
 * partial states and decision bits go to a scratch array of
 * MALA_DECODE_NOALLOC_SCRATCH_BYTES of device memory that the library holds
 * in each GPU it runs on, until the process ends.
 *   - A problem whose mala_decode_workspace_size exceeds that size is
 *     rejected with MALA_ERR_UNSUPPORTED (the 128K decode batch of 8
 *     sequences x 8 query heads with 256-key splits needs about 17 MB).
 *   - All calls on one GPU share that GPU's scratch. Calls that overlap on
 *     one GPU (several streams, several threads) race on it: the caller
 *     serializes them. The kernels write every scratch word they read, so
 *     nothing needs clearing between calls.
 *   - `stream` must belong to the calling thread's current device; the first
 *     call on a device looks up that device's scratch address.
 */
#define MALA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
mala_status mala_decode_noalloc(const mala_decode_problem* p, const void* q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* seqlens_k, void* o, float* lse,
                                int8_t* tile_mask, int32_t* kept_tiles, void* stream);

/* Description of the last error on the calling thread ("" if none). */
const char* mala_last_error(void);

/* Library version string. */
const char* mala_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MALA_H_ */
