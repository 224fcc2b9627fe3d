/*
 * moba.h -- C ABI of the MoBA (Mixture of Block Attention) prefill forward
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (deep-dive report on "MoBA: Mixture of Block Attention for
 * Long-Context LLMs", sections 2.1-2.3, and the course page "Paper: MoBA
 * (Moonshot)", summary):
 *   - the length-S context is cut into n = S / B blocks of B keys (report 2.1);
 *   - block i is summarised by the mean of its keys mu_i (report 2.2);
 *   - each query row scores every block by s_i = <q, mu_i> (report 2.2);
 *   - causal mode: blocks after the query's own block j = t / B are excluded,
 *     block j is always chosen, and min(topk - 1, j) further past blocks with
 *     the highest scores are chosen, ties going to the lower block index
 *     (report 2.3; topk counts the own block, as the report's sparsity figures
 *     81.25 % for 3 of 16 blocks and 95.31 % for 3 of 64 and 12 of 256 fix);
 *   - the output is softmax(q K^T / sqrt(D)) V over the union of the chosen
 *     blocks, with a causal mask inside the own block (report 2.2, 2.3).
 *   With topk >= n every causal block is chosen and the result is dense causal
 *   attention (course page summary).
 *   Non-causal mode (causal = 0): no exclusion, no forced block, the top
 *   min(topk, n) of all n blocks are chosen and attended in full.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Layouts are dense row-major:
 *       q, out : [batch, seqlen, num_q_heads,  head_dim]
 *       k, v   : [batch, seqlen, num_kv_heads, head_dim]
 *       mu     : [batch, num_kv_heads, seqlen / block_size, head_dim] fp32
 *       sel_idx: [batch, num_q_heads, seqlen, topk] int32; the chosen block
 *                indices of each row in ascending order, padded with -1.
 *   - Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   - dtype is MOBA_DTYPE_BF16 (q, k, v, out bf16; head_dim 128) or
 *     MOBA_DTYPE_F32 (all fp32; head_dim 64 or 128).  Gate scores and all
 *     accumulations are fp32 in both cases.
 *   - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *     stream).  Work is enqueued asynchronously on it; nothing synchronises.
 *     A kernel fault surfaces at the caller's next synchronisation.
 *   - Every argument is validated on the host before anything is enqueued;
 *     on an error status nothing has been launched and nothing written.
 *   - The functions are stateless and may be called from several threads;
 *     concurrent calls need distinct workspaces.
 */
#ifndef MOBA_H_
#define MOBA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moba_status {
  MOBA_OK = 0,
  MOBA_ERR_NULL = -1,               /* a required pointer is NULL */
  MOBA_ERR_DTYPE = -2,              /* unknown dtype */
  MOBA_ERR_HEAD_DIM = -3,           /* head_dim not supported for this dtype */
  MOBA_ERR_SEQ_NOT_DIVISIBLE = -4,  /* seqlen % block_size != 0 (no padding is defined) */
  MOBA_ERR_TOPK = -5,               /* topk < 1 (decode: also topk above its maximum) */
  MOBA_ERR_GQA = -6,                /* num_q_heads % num_kv_heads != 0 or group too large */
  MOBA_ERR_WORKSPACE = -7,          /* workspace NULL or smaller than the call accepts */
  MOBA_ERR_HIP = -8,                /* a HIP runtime call or kernel launch failed */
  MOBA_ERR_SHAPE = -9,              /* non-positive or overflowing sizes */
  MOBA_ERR_ALIGN = -10              /* a pointer is not 16-byte aligned */
};

enum moba_dtype { MOBA_DTYPE_F32 = 0, MOBA_DTYPE_BF16 = 1 };

/* Library version, major * 10000 + minor * 100 + patch. */
int moba_version(void);

/* Human-readable text for a status code (static storage, never NULL). */
const char* moba_status_string(int status);

/*
 * moba_workspace_bytes: the size of the device workspace moba_attn_fwd needs
 * for these shapes (block means, per-block row lists, tile list and the
 * per-(row, past block) partial results, sized for the query chunk the
 * library processes at a time; for bf16 with long per-block row lists, or
 * with no past block and blocks of at least 1024 keys, also a copy of K and
 * V re-laid out per 64-key slice, as large as K and V).
 * Pure host arithmetic; touches no device.
 * Returns a status; on MOBA_OK *bytes holds the size.
 */
int moba_workspace_bytes(int64_t batch, int64_t seqlen, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                         int32_t block_size, int32_t topk, int32_t causal,
                         size_t* bytes);

/*
 * Query chunks.  The forward processes the query positions in chunks of
 * whole blocks; the per-(row, past block) partial results, selection rows
 * and row lists of one chunk live in the workspace at a time.  By default a
 * chunk is as long as keeps its partials within 8 GiB (the whole sequence up
 * to that size).  moba_attn_fwd accepts any workspace at least as large as
 * moba_workspace_bytes_chunked(..., max_chunk_blocks = 1, ...) and then runs
 * with the longest chunk whose workspace fits (fewer, longer chunks are
 * faster); the result does not depend on the chunking.
 *
 * moba_workspace_bytes_chunked: the workspace for chunks of at most
 *   max_chunk_blocks query blocks (0 = the default; 1 = the smallest
 *   workspace the forward accepts: one block per chunk and K, V read as they
 *   are, not re-laid out as slice images).  Pure host arithmetic.
 * moba_plan_info: the plan the forward uses with a workspace of
 *   workspace_bytes (MOBA_ERR_WORKSPACE if it is too small): *chunk_blocks
 *   query blocks per chunk, *tile_rows rows per past-block attention tile
 *   (128, 256, or 384 for tiles read from K/V slice images), *slice_images
 *   1 if K and V are re-laid out as per-64-key slice images.  Host only.
 */
int moba_workspace_bytes_chunked(int64_t batch, int64_t seqlen, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                 int32_t block_size, int32_t topk, int32_t causal,
                                 int64_t max_chunk_blocks, size_t* bytes);
int moba_plan_info(int64_t batch, int64_t seqlen, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                   int32_t block_size, int32_t topk, int32_t causal,
                   size_t workspace_bytes, int64_t* chunk_blocks,
                   int32_t* tile_rows, int32_t* slice_images);

/*
 * moba_attn_fwd: the whole MoBA prefill forward (block means, gate, top-k,
 * block-sparse attention with the own-block causal mask).
 *   q, k, v   : inputs, layouts above, same dtype.
 *   out       : output, same shape and dtype as q.
 *   sel_idx   : optional output of the chosen blocks (may be NULL).
 *   workspace : device scratch owned by the caller, at least
 *               moba_workspace_bytes_chunked(..., 1, ...) bytes (see "Query
 *               chunks" above; moba_workspace_bytes() gives the fastest
 *               plan); its contents on entry do not matter.
 * topk >= n is clamped to n (dense causal attention).  Any topk >= 1 is
 * accepted: when more than 32 past blocks must be ranked (topk - 1 > 32, or
 * topk > 32 non-causal) the gate finds the cut-off score in rounds, each a
 * further pass over the row's blocks.  Returns a status.
 */
int moba_attn_fwd(const void* q, const void* k, const void* v,
                  int64_t batch, int64_t seqlen, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                  int32_t block_size, int32_t topk, int32_t causal,
                  void* out, int32_t* sel_idx,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * moba_attn_fwd_noalloc: moba_attn_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument, and the call
 * allocates nothing.  Its scratch is a static device array of
 * MOBA_NOALLOC_SCRATCH_BYTES (512 MiB) in the library, one per GPU the
 * library runs on, held until the process ends; its address is looked up on
 * the first call on a device.  The forward runs with the longest query chunk
 * whose workspace fits in it (see "Query chunks"); shapes whose smallest
 * workspace (moba_workspace_bytes_chunked(..., 1, ...)) exceeds it return
 * MOBA_ERR_WORKSPACE (all five benchmark shapes of this library fit, up to
 * 1M positions with 32/8 heads, block 4096, top-12).  Nothing in the scratch
 * has to start at zero: every call writes what it reads.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  `stream` must belong
 * to the current device (MOBA_ERR_HIP otherwise).  Other arguments, layouts,
 * results and errors as moba_attn_fwd (mean gate).
 */
#define MOBA_NOALLOC_SCRATCH_BYTES (512ull << 20)
int moba_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                          int64_t batch, int64_t seqlen, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                          int32_t block_size, int32_t topk, int32_t causal,
                          void* out, int32_t* sel_idx, void* stream);

/*
 * Block summary and gate score (the method's gate, report 2.2, or the
 * Quest-style variant the report places in the same family, report 1.3:
 * min/max pooling of the block's keys).
 */
enum moba_gate_kind {
  MOBA_GATE_MEAN = 0,   /* mu_i = mean of block i's keys; s_i = <q, mu_i> */
  MOBA_GATE_MINMAX = 1  /* lo_i / hi_i = element-wise min / max of block i's keys;
                           s_i = sum_d max(q_d lo_id, q_d hi_id), the largest q.k
                           over the box [lo_i, hi_i] */
};

/*
 * moba_attn_fwd_gate: moba_attn_fwd with the gate chosen by gate_kind (a
 * moba_gate_kind; moba_attn_fwd is this call with MOBA_GATE_MEAN).  The causal
 * rules, the forced own block, the top-k and the attention are unchanged.
 * Same arguments, workspace size (moba_workspace_bytes covers both gates),
 * ownership and errors as moba_attn_fwd; an unknown gate_kind returns
 * MOBA_ERR_SHAPE.
 */
int moba_attn_fwd_gate(const void* q, const void* k, const void* v,
                       int64_t batch, int64_t seqlen, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                       int32_t block_size, int32_t topk, int32_t causal,
                       int32_t gate_kind, void* out, int32_t* sel_idx,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moba_minmaxpool: the min/max gate's pooling alone: lohi[b, hk, i, 0, :] =
 * element-wise minimum and lohi[b, hk, i, 1, :] = maximum of the B keys of
 * block i (exact: they are input values), fp32 [b, Hkv, n, 2, D], written in
 * full.  k and its layout as for moba_attn_fwd.
 */
int moba_minmaxpool(const void* k, int64_t batch, int64_t seqlen,
                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                    int32_t block_size, float* lohi, void* stream);

/*
 * moba_meanpool: stage 1 alone (report 2.2): mu[b, hk, i, :] = mean of the B
 * keys of block i, summed in fp32.  k as above; mu is written in full.
 */
int moba_meanpool(const void* k, int64_t batch, int64_t seqlen,
                  int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                  int32_t block_size, float* mu, void* stream);

/*
 * moba_gate: stage 2 alone (report 2.2, 2.3): fp32 scores <q, mu_i>, the
 * causal exclusion and forced own block, and the top-k with ties to the
 * lower index.  mu as written by moba_meanpool; sel_idx is written in full.
 */
int moba_gate(const void* q, const float* mu, int64_t batch, int64_t seqlen,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
              int32_t dtype, int32_t block_size, int32_t topk, int32_t causal,
              int32_t* sel_idx, void* stream);

/*
 * moba_attn_fwd_train: moba_attn_fwd (mean gate) that also writes, for the
 * backward, lse[b, h, t] = log sum_{attended keys s} exp(q.k_s / sqrt(D))
 * (natural log), fp32 [batch, Hq, seqlen].  sel_idx and lse are required.
 */
int moba_attn_fwd_train(const void* q, const void* k, const void* v,
                        int64_t batch, int64_t seqlen, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                        int32_t block_size, int32_t topk, int32_t causal,
                        void* out, int32_t* sel_idx, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward.  The gate is a hard top-k with no parameters (report §2.2): it
 * only picks each row's keys, and no gradient flows through the choice.  With
 * the forward's choice (sel_idx) held fixed each row is softmax attention over
 * its keys, and the gradients of sum(dout * out) are (p = exp(q.k_s / sqrt(D)
 * - lse), delta = dout . out):
 *   dv_s += p_s dout,  ds_s = p_s (dout . v_s - delta),
 *   dq = sum_s ds_s k_s / sqrt(D),  dk_s += ds_s q / sqrt(D).
 * The pages train with MoBA (report §3.3) but print no backward; this is the
 * gradient of the forward as computed.
 *
 * Inputs: q, k, v, out, dout as for moba_attn_fwd (out and dout like q); lse
 * and sel_idx as written by moba_attn_fwd_train with the same shapes.  A
 * selection entry that can never be chosen (beyond the last block, or after
 * the row's own block) is skipped, so no memory outside the given buffers is
 * touched; any other departure from a forward's selection (repeated blocks,
 * fewer past blocks than min(topk - 1, own block)) gives unspecified
 * gradients.
 * Outputs: dq like q, dk and dv like k, written in full (every key gets its
 * gradient, zero for a key no row attends).  bf16 only (MOBA_ERR_DTYPE for
 * fp32), head_dim 128, block_size a multiple of 64 (MOBA_ERR_SHAPE).
 * dk and dv are summed over rows in an order that can vary between runs
 * (fp32 accumulation, then one bf16 rounding).  Workspace: at least
 * moba_bwd_workspace_bytes(); nothing is allocated.  Stream-ordered.
 */
int moba_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                             int32_t block_size, int32_t topk, int32_t causal,
                             size_t* bytes);
int moba_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                  const void* dout, const float* lse, const int32_t* sel_idx,
                  int64_t batch, int64_t seqlen, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                  int32_t block_size, int32_t topk, int32_t causal,
                  void* dq, void* dk, void* dv,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-time MoBA: one new query per sequence against its key/value cache.
 * The pages evaluate generation with full attention and name sparse decode
 * as future work (report §4.4, §6.3); here the new token of sequence b, at
 * position t = L_b - 1 of a cache of L_b positions (its own key and value
 * already appended), is routed and attended exactly as prefill row t
 * (report §2.2, §2.3): own block j = t / B, cut at t; the best min(k-1, j)
 * complete past blocks 0..j-1 by <q, mean key>, ties to the lower index;
 * softmax over the union.
 *
 * Layouts (row-major, 16-byte aligned, dtype and head_dim as for
 * moba_attn_fwd):
 *   q          [batch, Hq, D]       the new tokens' queries
 *   k_cache,   [batch, max_len, Hkv, D]  positions 0 .. L_b - 1 are read;
 *   v_cache                         later positions are never touched
 *   mu_cache   fp32 [batch, Hkv, max_len / B, D]  mean key of each complete
 *              block (moba_decode_means fills it; see below)
 *   cache_lens int32 [batch] on the device: L_b, the new token included
 *   out        [batch, Hq, D]
 *   sel_idx    int32 [batch, Hq, topk] or NULL: the chosen past blocks
 *              ascending, then the own block j, then -1
 * max_len must be a multiple of block_size with max_len / block_size <=
 * 16384; Hq / Hkv <= 16; 1 <= topk <= 64.  A sequence whose L_b lies
 * outside [1, max_len] gets a zero output row and a sel row of -1 (no
 * memory is read for it).
 */

/* moba_decode_workspace_bytes: the device workspace moba_decode_fwd needs. */
int moba_decode_workspace_bytes(int64_t batch, int64_t max_len, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                int32_t block_size, int32_t topk, size_t* bytes);

/*
 * moba_decode_fwd: one decode step for every sequence of the batch.  Reads
 * mu_cache entries 0 .. j-1 of each sequence and, when L_b % block_size == 0
 * (the new token completes block j), writes entry j: the cache of means stays
 * current for the next step of a caller that appends one token per step.
 * Stream-ordered on `stream`; no allocation, no host synchronisation.
 * Errors as moba_attn_fwd (MOBA_ERR_SEQ_NOT_DIVISIBLE: max_len % block_size
 * != 0); nothing is launched on an error.
 */
int moba_decode_fwd(const void* q, const void* k_cache, const void* v_cache,
                    float* mu_cache, const int32_t* cache_lens,
                    int64_t batch, int64_t max_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                    int32_t block_size, int32_t topk, void* out, int32_t* sel_idx,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * moba_decode_means: mu_cache[b, hk, i, :] = mean of block i's keys (fp32
 * sum) for every complete block i < L_b / block_size of every sequence; other
 * entries are left as they are.  Use it once after filling a cache (after a
 * prefill, for instance); moba_decode_fwd keeps it current from then on.
 */
int moba_decode_means(const void* k_cache, const int32_t* cache_lens, int64_t batch,
                      int64_t max_len, int32_t num_kv_heads, int32_t head_dim,
                      int32_t dtype, int32_t block_size, float* mu_cache, void* stream);

/*
 * Measurement support (for benchmarks; not thread-safe).  While enabled, every
 * kernel launch made by the calls above is bracketed by two HIP events
 * recorded on the caller's stream, and the host adds the launch's
 * algorithmic work to its stage: useful FLOPs (4 * head_dim per attended key)
 * for the attention stages, compulsory HBM bytes for the others.
 * moba_profile_read waits for the recorded events, writes per stage the
 * summed kernel milliseconds, the number of launches and the summed work into
 * the caller's host arrays (n entries each, n <= MOBA_NUM_STAGES), and clears
 * the records.  The events are created by the library on first use and kept
 * for reuse.
 */
enum moba_stage {
  MOBA_STAGE_MEANPOOL = 0,  /* block means: bytes */
  MOBA_STAGE_GATE = 1,      /* gate + top-k: bytes */
  MOBA_STAGE_DISPATCH = 2,  /* per-block row lists: bytes */
  MOBA_STAGE_PAST = 3,      /* attention over non-own blocks: FLOPs */
  MOBA_STAGE_OWN = 4,       /* own block + merge: FLOPs */
  MOBA_STAGE_F32 = 5,       /* fp32 attention path: FLOPs */
  MOBA_STAGE_KVLAYOUT = 6,  /* K and V re-laid out as per-slice LDS images: bytes */
  MOBA_STAGE_DECODE_GATE = 7,   /* decode gate, top-k and union (work 0: */
  MOBA_STAGE_DECODE_ATTN = 8,   /*   the bytes read depend on the device-side cache */
  MOBA_STAGE_DECODE_MERGE = 9,  /*   lengths and are left to the caller) */
  MOBA_STAGE_BWD_PREP = 10,     /* backward: delta, base-2 lse, K/V images: bytes */
  MOBA_STAGE_BWD_DKDV = 11,     /* backward dk, dv: FLOPs (8 D per attended key) */
  MOBA_STAGE_BWD_DQ = 12,       /* backward dq: FLOPs (6 D per attended key) */
  MOBA_NUM_STAGES = 13
};
int moba_profile_enable(int on);
int moba_profile_read(double* ms, int64_t* launches, double* work, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H_ */
