/*
 * ra.h -- C ABI of libra.so: one context-parallel rank's share of Ring
 * Attention on an AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   - "超长序列并行训练技术：Ulysses与Ring-Attention详解" (intelliparadigm):
 *     section 4.1 -- attention is computed block by block, each block
 *     returning a partial output and its log-sum-exp (lse), folded into a
 *     running result; section 4.2 -- partials merge by
 *     lse_new = log(exp(lse_prev) + exp(lse_cur)), and the sequence is
 *     placed zig-zag: device i holds chunk i and chunk 2C-1-i; section 4.3
 *     -- the backward recomputes forward quantities instead of storing them;
 *     section 5.3 -- each sequence is padded on its own to a multiple of
 *     2 x world size.
 *   - "LLM Context Parallel production guide" (oh-bug): local Q is kept,
 *     KV blocks travel the ring, each step's attention is merged exactly by
 *     per-row max and exp-sum; packed varlen metadata (cumulative lengths)
 *     follows the same sequence mapping; kernels should skip dead causal
 *     blocks.
 *   - "超长上下文训练速度翻倍秘籍" (ant-ling), section 2, "踩坑一": the
 *     diagonal block (local Q x local KV) is causal; received history KV
 *     blocks are fully visible and use a non-causal call.
 *   - "seq_len 从 4K 推到 16K、CP=2 一开就慢了 20%：Ulysses Context
 *     Parallelism 的工程取舍全记录" (iqiancheng), section 1.1: KV blocks
 *     travel device 0 -> 1 -> ... -> C-1 -> 0 round the ring.
 *
 * Conventions for every entry point:
 *   - Layout: token-major packed tensors [tokens, heads, dim] with dim
 *     contiguous; lse and delta are [heads, tokens] float32.
 *   - Packed sequences: segment s covers tokens [cu[s], cu[s+1]) of a
 *     buffer.  Both a host and a device copy of every cu_seqlens array are
 *     passed and must hold the same values: the host copy is used for
 *     validation, launch sizing and the order of a launch's tiles (it is
 *     not retained), the device copy by the kernels, which locate their
 *     tiles in it.
 *   - Ownership: the caller allocates and frees every buffer, including
 *     workspaces; the library keeps no pointer after a call returns, keeps
 *     no state except a thread-local error string, never synchronises and
 *     never allocates device memory.  Work is queued on the caller's stream
 *     (a hipStream_t passed as void*; NULL = the null stream); buffers must
 *     outlive the queued work.
 *   - Empty work: zero-length segments, and descriptors whose segments are
 *     all empty, are valid; then nothing is launched for them.  Buffer
 *     pointers must still be non-NULL (any valid address will do when a
 *     buffer's size is zero).
 *   - Errors: arguments are validated before anything is queued; on
 *     RA_ERR_INVALID_ARG / RA_ERR_UNSUPPORTED nothing is launched and
 *     nothing is written.  A failed launch returns RA_ERR_HIP.  Faults of
 *     queued work surface at the caller's next synchronisation.
 *     ra_last_error() describes the last non-OK status of the thread.
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1,
  RA_ERR_UNSUPPORTED = 2,
  RA_ERR_HIP = 3
} ra_status;

typedef enum { RA_BF16 = 0, RA_FP32 = 1 } ra_dtype;

/* Which half of every segment takes part in a block (zig-zag halves). */
typedef enum {
  RA_PART_ALL = 0,
  RA_PART_FIRST_HALF = 1,  /* tokens [cu[s], cu[s] + len/2)   */
  RA_PART_SECOND_HALF = 2  /* tokens [cu[s] + len/2, cu[s+1]) */
} ra_part;

/*
 * One block of attention: local queries against one KV block.
 *
 * q [total_q, hq, dqk], k [total_k, hkv, dqk], v [total_k, hkv, dv], all of
 * `dtype`, device memory, token stride q_stride_tok / k_stride_tok /
 * v_stride_tok elements (>= heads*dim; 0 means packed).  Query head h reads
 * kv head h / (hq / hkv) (hq % hkv == 0).  Segment s of q and of k are
 * matched one to one; within a segment only the part selected by q_part /
 * k_part takes part (segment lengths must then be even).  causal = 1 masks
 * key j of the part against query i of the part unless j <= i (both counted
 * from the part's start); it requires equal q and k part lengths in every
 * segment.  causal = 0 makes every key of the segment part visible.
 * softmax_scale <= 0 selects 1/sqrt(dqk).
 *
 * Supported: bf16 with (dqk, dv) in {(64,64), (128,128), (192,128)};
 * fp32 with dqk == dv in {16, 32, 64, 128}.
 */
typedef struct ra_attn_desc {
  const void* q;
  const void* k;
  const void* v;
  ra_dtype dtype;
  int32_t hq, hkv, dqk, dv;
  int64_t q_stride_tok, k_stride_tok, v_stride_tok;
  int32_t n_seq;
  const int32_t* cu_seqlens_q;       /* device int32[n_seq + 1] */
  const int32_t* cu_seqlens_k;       /* device int32[n_seq + 1] */
  const int32_t* cu_seqlens_q_host;  /* host   int32[n_seq + 1] */
  const int32_t* cu_seqlens_k_host;  /* host   int32[n_seq + 1] */
  ra_part q_part, k_part;
  int32_t causal;
  float softmax_scale;
} ra_attn_desc;

/*
 * Partial attention of one block (intelliparadigm section 4.1: a block
 * returns (out, lse)).  out [total_q, hq, dv] float32 and lse [hq, total_q]
 * float32 (natural log) are written for the covered query rows only
 * (rows outside q_part keep their contents).  A covered row that sees no
 * key gets out = 0, lse = -inf.
 */
ra_status ra_block_attn_fwd(const ra_attn_desc* d, float* out, float* lse, void* stream);

/*
 * Same block, merged straight into a running result instead of written as
 * a partial: for the covered rows, (out_acc, lse_acc) <- merge(acc, block)
 * with the lse rule of ra_lse_merge.  Saves the partial's round trip
 * through memory (the oh-bug page's exact online-softmax merge, done in
 * the attention kernel's epilogue).
 */
ra_status ra_block_attn_fwd_merge(const ra_attn_desc* d, float* out_acc, float* lse_acc,
                                  void* stream);

/*
 * Merge a partial into a running result, for the covered rows of every
 * segment (intelliparadigm section 4.2 and the oh-bug page's exact merge):
 *   lse = m + log(exp(lse_acc - m) + exp(lse_part - m)),  m = max of the two
 *   out = exp(lse_acc - lse) out_acc + exp(lse_part - lse) out_part
 * (0, -inf) on either side is the identity; both -inf give (0, -inf).
 * out_* [total_t, h, dv] float32, lse_* [h, total_t] float32, device.
 * dv must be a multiple of 4.
 */
ra_status ra_lse_merge(float* out_acc, float* lse_acc, const float* out_part,
                       const float* lse_part, int32_t total_t, int32_t h, int32_t dv,
                       int32_t n_seq, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_host, ra_part rows, void* stream);

/*
 * Zig-zag shard map (intelliparadigm section 4.2; per-sequence splitting
 * as in its section 5.3 and the oh-bug page's varlen rule).  Host only.
 * Every sequence d of the global packed stream (length L, L % (2*cp_size)
 * == 0) is cut into 2*cp_size chunks of c = L / (2*cp_size) tokens; `rank`
 * holds chunk rank and chunk 2*cp_size-1-rank of every sequence, in that
 * order.  Writes cu_seqlens_local[n_seq+1] (= global / cp_size) and
 * src_start[2*n_seq]: the global token where local half 2d / 2d+1 starts.
 */
ra_status ra_zigzag_shard_map(int32_t cp_size, int32_t rank, int32_t n_seq,
                              const int32_t* cu_seqlens_global, int32_t* cu_seqlens_local,
                              int32_t* src_start);

/*
 * Copy a rank's rows out of a global packed buffer (gather) or back into it
 * (scatter), using the map above.  Rows are row_bytes long (a multiple of
 * 16); src_start and cu_seqlens_local are device copies of the map, host
 * copies are used for validation.  total_global bounds the global buffer.
 */
ra_status ra_zigzag_gather(const void* global_src, void* local_dst, int64_t row_bytes,
                           int32_t n_seq, const int32_t* cu_seqlens_local,
                           const int32_t* src_start, const int32_t* cu_seqlens_local_host,
                           const int32_t* src_start_host, int32_t total_global, void* stream);
ra_status ra_zigzag_scatter(const void* local_src, void* global_dst, int64_t row_bytes,
                            int32_t n_seq, const int32_t* cu_seqlens_local,
                            const int32_t* src_start, const int32_t* cu_seqlens_local_host,
                            const int32_t* src_start_host, int32_t total_global, void* stream);

/*
 * float32 -> bfloat16, round to nearest even (n elements, multiple of 4).
 */
ra_status ra_cast_f32_bf16(const float* src, void* dst, int64_t n, void* stream);

/*
 * One rank's whole forward share (the ring loop of the oh-bug page: local
 * Q against every KV block in turn, merged exactly).  `local` describes the
 * rank's local Q (k, v ignored) and the local cu_seqlens, which are the
 * same for the rank's own KV block and every received one.  At step s the
 * block of owner j = (rank - s) mod cp_size is used (KV moves rank 0 -> 1
 * -> ... as in the iqiancheng page cited above, section 1.1):
 *   s = 0      : causal, all local rows x all keys (the diagonal block);
 *   j < rank   : non-causal, all rows x FIRST half of the owner's keys;
 *   j > rank   : non-causal, SECOND half of the rows x all the owner's keys
 * (derived from the global causal rule and the zig-zag placement; the
 * other quarter of each history block is entirely masked and is skipped).
 * k_blocks / v_blocks: host arrays [cp_size] of device pointers, by owner;
 * every block uses the token strides of `local` (k_stride_tok,
 * v_stride_tok), so a block may be a head slice of a wider buffer.  With
 * cp_size = 1 the share is the single causal block: one rank's Ulysses
 * share (all tokens, a subset of the heads) is ra_rank_forward with
 * cp_size = 1 over a head slice.
 * out [total_q, hq, dv] of out_dtype, lse [hq, total_q] float32: final.
 * fuse_merge = 0: each step writes a partial to the workspace and
 * ra_lse_merge folds it; 1: steps merge in the attention epilogue;
 * 2 (bf16): the whole share in one launch, every owner's block walked in
 * ring order with the online-softmax state kept in registers and the final
 * output written by the epilogue (the pass-KV form of the oh-bug page with
 * all blocks resident).  On the 4-wave kernel a share may be split instead:
 * its key tiles (over all blocks, in ring order) are dealt round-robin over
 * several parts, each part's workgroups write a float32 partial (out, lse)
 * into the workspace, and a combine launch weights the parts by their lse
 * in part order (deterministic).  The split is taken when the share has
 * fewer than 256 workgroups (128 rows x one query head; up to 8 parts), and
 * in 2 parts when it has 256-2047 workgroups whose rows see on average 64K
 * keys or more (long shares such as 256K MLA).  A single sequence split
 * for its size deals the same number of workgroups (parts x query tiles)
 * over the query tiles by the length of their walks, at most 6 parts per
 * tile (or the split count, if larger), into 6 partial slots.  The
 * workspace is then slots x (out + lse), otherwise 0; since the rule
 * depends on the shapes, callers must always ask ra_rank_forward_workspace
 * for the size (it is the same for every rank of a ring).  The environment
 * variable RA_FWD_KV_SPLIT=<n> forces n parts (1 = none, at most 16), and
 * RA_FWD_VAR_SPLIT=0 keeps the parts uniform over the tiles.
 * fp32 falls back to fuse_merge = 1.
 * events (optional): host array of 2*cp_size hipEvent_t, recorded on the
 * stream right before / after step s's attention launch (with
 * fuse_merge = 2 only events[0], events[1], around the launch and its
 * combine).
 */
typedef struct ra_rank_desc {
  ra_attn_desc local;
  int32_t cp_size, rank;
  const void* const* k_blocks;
  const void* const* v_blocks;
  void* out;
  ra_dtype out_dtype;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  int32_t fuse_merge;
  void* const* events;
} ra_rank_desc;

ra_status ra_rank_forward_workspace(const ra_rank_desc* d, size_t* bytes);
ra_status ra_rank_forward(const ra_rank_desc* d, void* stream);

/*
 * ra_rank_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as ra_rank_forward, except that
 * d->workspace and d->workspace_bytes are ignored: the workspace is a fixed
 * array of RA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU,
 * held until the process ends (its device address is looked up once per
 * device, on the first call with that device current).  The call allocates,
 * frees and synchronises nothing.  A share whose ra_rank_forward_workspace
 * size exceeds RA_NOALLOC_SCRATCH_BYTES is rejected with RA_ERR_INVALID_ARG
 * before anything is queued.  Every call on one GPU uses that GPU's one
 * array: calls whose queued work overlaps in time on the same GPU (other
 * streams, other host threads) race on it and must be serialised by the
 * caller.  Nothing in the array needs to start at zero: every byte a call
 * reads was written earlier by the same call.
 */
#define RA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ra_status ra_rank_forward_noalloc(const ra_rank_desc* d, void* stream);

/*
 * Backward, recomputing the probabilities from the saved final lse
 * (intelliparadigm section 4.3):
 *   delta_i = dout_i . out_i                      (ra_attn_bwd_delta)
 *   P_ij = exp(scale q_i.k_j - lse_i), dV_j += sum_i P_ij dout_i,
 *   dS_ij = P_ij (dout_i . v_j - delta_i),
 *   dQ_i += scale sum_j dS_ij k_j,  dK_j += scale sum_i dS_ij q_i
 * over the block's visible pairs (ra_block_attn_bwd).  dq_acc
 * [total_q, hq, dqk], dk_acc [total_k, hkv, dqk], dv_acc [total_k, hkv, dv]
 * are float32 accumulators that are ADDED to (the caller zeroes them);
 * query heads of a group add into their kv head.  dout has the desc's
 * dtype; lse and delta are [hq, total_q] float32.  bf16 only, with
 * (dqk, dv) in {(128,128), (192,128)}.  Deterministic: no atomics.
 */
ra_status ra_attn_bwd_delta(const void* out, ra_dtype out_dtype, const void* dout,
                            ra_dtype dout_dtype, int32_t total_t, int32_t hq, int32_t dv,
                            float* delta, void* stream);
ra_status ra_block_attn_bwd(const ra_attn_desc* d, const void* dout, const float* lse,
                            const float* delta, float* dq_acc, float* dk_acc, float* dv_acc,
                            void* stream);

/*
 * One rank's whole backward share: the same step plan as ra_rank_forward;
 * dK/dV of step s are added into dk_blocks[j] / dv_blocks[j] of the owner
 * j (in a real ring they travel back to it).  out is the final forward
 * output (out_dtype), lse the final lse; delta is computed into the
 * workspace.  dq [total_q, hq, dqk] float32 is added to.
 *
 * The share runs rank-fused: one dK/dV launch over the key tiles of every
 * owner's block (each with that step's rule, added into that owner's
 * dK/dV) and one dQ launch whose query tiles walk the key tiles of all
 * blocks in ring order, dQ kept in registers; on shares with few query
 * tiles up to 4 workgroups deal a query tile's walk (on a single sequence
 * the same number of workgroups is dealt over the tiles by walk length, up
 * to 6 per tile; RA_BWD_VAR_SPLIT=0 keeps them uniform), their float32
 * partials (after delta in the workspace) added in share order.
 *
 * RA_BWD_RANK_FUSED=0 in the environment selects the per-step form
 * instead: one dK/dV and one dQ launch per ring step.  On blocks with few
 * 128-key tiles, and on the causal diagonal block, up to 4 workgroups then
 * share a key tile, each taking a contiguous share of its query iterations;
 * share 0 adds into the owner's dK/dV, shares 1.. store float32 partials in
 * the workspace, and a reduction adds them in share order.  Likewise, on
 * blocks with few 128-row query tiles, up to 4 workgroups share a query
 * tile for dQ, dealing its key tiles; share 0 adds into dq, the others'
 * float32 partials follow the dK/dV ones in the workspace.
 *
 * Both forms are deterministic (no atomics; partials added in a fixed
 * order) and give the same results up to rounding order.  The workspace
 * (device, caller-owned, ra_rank_backward_workspace bytes for the form that
 * will run; the same size for every rank of the ring) holds delta
 * [hq, total_q] and those partials; a smaller one is rejected with
 * RA_ERR_INVALID_ARG before any launch.
 * events (optional): host array of 2*cp_size hipEvent_t; events[0] is
 * recorded before the rank's first launch and events[2*cp_size-1] after its
 * last in both forms; the per-step form also records events[2s] / [2s+1]
 * around step s's launches (step 0's span includes the delta launch).
 */
typedef struct ra_rank_bwd_desc {
  ra_attn_desc local;
  int32_t cp_size, rank;
  const void* const* k_blocks;
  const void* const* v_blocks;
  const void* out;
  ra_dtype out_dtype;
  const void* dout;
  const float* lse;
  float* dq;
  float* const* dk_blocks;
  float* const* dv_blocks;
  void* workspace;
  size_t workspace_bytes;
  void* const* events;
} ra_rank_bwd_desc;

ra_status ra_rank_backward_workspace(const ra_rank_bwd_desc* d, size_t* bytes);
ra_status ra_rank_backward(const ra_rank_bwd_desc* d, void* stream);

/*
 * Accounting (the oh-bug page asks to monitor effective attention blocks
 * per rank): for one block descriptor, the number of (query, key) pairs
 * that are visible, the key tiles the forward kernel visits, and the key
 * tiles it skips as entirely masked, summed over query heads.  Host only.
 */
ra_status ra_block_attn_work(const ra_attn_desc* d, int64_t* visible_pairs,
                             int64_t* tiles_visited, int64_t* tiles_skipped);

/*
 * Other shard maps, on the same kernels (the oh-bug page's correctness
 * section on causal rank imbalance names contiguous ranges, striped /
 * interleaved tokens and the zig-zag mapping; applying the zig-zag to a
 * packed stream as a whole is the static split it warns about for varlen
 * batches):
 *   RA_MAP_ZIGZAG         per-document zig-zag (as ra_zigzag_shard_map)
 *   RA_MAP_ZIGZAG_GLOBAL  zig-zag over the packed stream: its T tokens cut
 *                         into 2C chunks regardless of documents, rank r
 *                         holding chunks r and 2C-1-r (T % 2C == 0)
 *   RA_MAP_STRIPED        token t on rank t mod C (T % C == 0)
 *   RA_MAP_CONTIGUOUS     tokens [r T/C, (r+1) T/C) on rank r (T % C == 0)
 * Every map gives each rank T/C tokens, kept in global order.
 */
typedef enum {
  RA_MAP_ZIGZAG = 0,
  RA_MAP_ZIGZAG_GLOBAL = 1,
  RA_MAP_STRIPED = 2,
  RA_MAP_CONTIGUOUS = 3
} ra_map;

/* Global token index of each local row of `rank` (host).  tokens: host
 * int32[capacity], capacity >= T / cp_size; *n_tokens receives T / cp_size. */
ra_status ra_shard_tokens(ra_map kind, int32_t cp_size, int32_t rank, int32_t n_seq,
                          const int32_t* cu_seqlens_global, int32_t* tokens, int32_t capacity,
                          int32_t* n_tokens);

/* A rectangle of one ring step: local query rows [q_lo, q_hi) of the rank
 * and local keys [k_lo, k_hi) of the KV block it holds; key j is visible to
 * row i iff (j - k_lo) <= (i - q_lo) + diag (diag >= k_hi - k_lo: every key
 * of the rectangle). */
typedef struct ra_segment {
  int32_t q_lo, q_hi, k_lo, k_hi, diag;
} ra_segment;

/* The rectangles of `rank`'s rows against the KV block of `owner` under a
 * shard map: exactly the pairs of the global rule (same document, key not
 * after query) between the two ranks' tokens, with disjoint row ranges, in
 * row order (host).  segs: host array[capacity]; *n_segs receives the
 * count (at most 2 x n_seq + 2); RA_ERR_INVALID_ARG if capacity is short. */
ra_status ra_step_segments(ra_map kind, int32_t cp_size, int32_t rank, int32_t owner,
                           int32_t n_seq, const int32_t* cu_seqlens_global, ra_segment* segs,
                           int32_t capacity, int32_t* n_segs);

/* Row gather / scatter by token index: gather writes dst row i = src row
 * tokens[i], scatter writes dst row tokens[i] = src row i, for i < n.  Rows
 * of row_bytes (a multiple of 16; buffers 16-byte aligned).  tokens_dev is
 * the device copy of tokens_host; every index must be < n_rows (the row
 * count of the indexed buffer: src for gather, dst for scatter). */
ra_status ra_gather_tokens(const void* src, void* dst, int64_t row_bytes, int32_t n_rows,
                           const int32_t* tokens_dev, const int32_t* tokens_host, int32_t n,
                           void* stream);
ra_status ra_scatter_tokens(const void* src, void* dst, int64_t row_bytes, int32_t n_rows,
                            const int32_t* tokens_dev, const int32_t* tokens_host, int32_t n,
                            void* stream);

/* Block attention (bf16) over a list of rectangles, each with its own
 * visibility rule, in one launch (the 4-wave kernel).  `d` supplies q, k,
 * v, dtype, heads, dims and token strides; d->n_seq must be 1 with
 * cu_seqlens_q_host = {0, Tq} and cu_seqlens_k_host = {0, Tk} (the buffer
 * row counts; the device cu arrays and q_part / k_part / causal are not
 * used).  segs_dev / segs_host: device array and host copy of n_seg
 * rectangles within the buffers and with disjoint row ranges.  merge = 0
 * writes the partial (out, lse) of every covered row (a row that sees no
 * key gets (0, -inf)); merge = 1 folds it into (out, lse) as
 * ra_block_attn_fwd_merge.  Rows outside every rectangle are untouched. */
ra_status ra_block_attn_fwd_segments(const ra_attn_desc* d, int32_t n_seg,
                                     const ra_segment* segs_dev, const ra_segment* segs_host,
                                     float* out, float* lse, int32_t merge, void* stream);

/* Accounting of a rectangle list for hq query heads: visible (query, key)
 * pairs, key tiles the forward kernel visits and tiles it skips as entirely
 * masked (host). */
ra_status ra_segments_work(const ra_segment* segs, int32_t n_seg, int32_t hq,
                           int64_t* visible_pairs, int64_t* tiles_visited, int64_t* tiles_skipped);

/*
 * Name of the bf16 forward kernel a launch over the rows of q_part of `d`
 * uses (ra_block_attn_fwd / _merge with d->q_part, ra_rank_forward with
 * fuse_merge = 2 and RA_PART_ALL): "attn_fwd_pp" (8 waves, 256-row query
 * tiles, matrix-core and softmax phases of the two waves of a SIMD
 * interleaved) for head dims 128/128 when the launch has at least 512 such
 * tiles over all query heads and real rows carry at least 3/4 of the tiled
 * rows' work, each segment's rows weighted by its key count (so padding in
 * the tiles of short segments counts little), "attn_fwd_bf16" (4 waves,
 * 128-row tiles) otherwise, "attn_fwd_f32" for float32.  Both bf16 kernels
 * compute the same result.  The environment variable RA_FWD_KERNEL=pp or
 * =4w forces one.  Host only; NULL (with ra_last_error set) for an invalid
 * descriptor.
 */
const char* ra_forward_kernel(const ra_attn_desc* d, ra_part q_part);

/*
 * Measurement helper (not part of the attention path): n_workgroups x 4
 * waves each run iters x 64 products v_mfma_f32_32x32x16_bf16 (8
 * independent accumulator chains, 32768 FLOP per product) on bf16 operand
 * fragments read once from `operands` (device, operand_bytes >= 16 KiB, a
 * multiple of 16, 16-byte aligned; read with wrap-around), and write one
 * float per lane to `out` (device, out_floats >= n_workgroups x 256, else
 * RA_ERR_INVALID_ARG before any launch).  Timed by
 * the caller, it gives the rate the matrix cores sustain on operands of a
 * given distribution, which bounds the attention kernels on that data.
 */
ra_status ra_mfma_ceiling(const void* operands, int64_t operand_bytes, float* out,
                          int64_t out_floats, int32_t n_workgroups, int32_t iters, void* stream);

/* Thread-local description of the last non-OK status ("" if none). */
const char* ra_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
