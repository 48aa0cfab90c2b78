/*
 * kvdecode.h -- C ABI of the paged decode-attention library (gfx950 / MI355X).
 *
 * One decode step of one attention layer is two calls: append this step's
 * K/V row into the paged cache, then attend over the whole visible history
 * with the step's query ("append, then read all history": LLM Compass
 * "KV Cache（键值缓存）", section 4 实现要点, the decode_step sketch; LLM
 * Systems Wiki "KV缓存原理与显存估算", 知识点二).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every tensor pointer is DEVICE memory owned by the caller.  The
 *   library allocates nothing, frees nothing, keeps no state between calls
 *   and never writes q, k_new, v_new, c_new, block_table or seq_lens.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Calls only enqueue work: a return of KVD_OK means "validated
 *   and launched", not "finished".  Calls on one stream run in order.
 * Errors: arguments are checked on the host before anything is launched; a
 *   negative status is returned and nothing is enqueued.  The checks read no
 *   device memory (unless KVD_VALIDATE=1, below), so contents (seq_lens,
 *   table entries) are preconditions:
 *     1 <= seq_lens[b] <= min(max_seq_len, max_blocks_per_seq * block_size);
 *     table entries of the blocks that hold positions < seq_lens[b] lie in
 *     [0, num_blocks); the block receiving an appended row is owned by that
 *     sequence alone (shared prefix blocks are copy-on-write: "KV Cache（键值
 *     缓存）", 2.3 路线二); inputs are finite.
 *   The kernels never read or write outside the buffers described here even
 *   when these are violated: lengths are clamped to the table row, and a
 *   table entry outside [0, num_blocks) is skipped (its tokens contribute
 *   nothing and no append is made to it).  A sequence with seq_lens[b] <= 0
 *   gets an all-zero output row.
 * KVD_VALIDATE=1 (environment variable, read at every call): each entry
 *   point that launches kernels first copies its seq_lens, block table (and
 *   cu_rows) and its small inputs (q, k_new, v_new) to the host, which
 *   synchronises its stream, and returns KVD_ERR_SHAPE without launching
 *   anything when one of the preconditions above fails (kvd_validate_tables,
 *   kvd_validate_finite).  The cache contents are not scanned.  Meant for
 *   debugging: it costs a round trip per call and must not be used under
 *   HIP graph capture.
 * Layouts (row-major, innermost last):
 *   paged K or V cache   [num_blocks, block_size, num_kv_heads, head_dim]
 *       token-major inside a block, the per-token [seq, heads, d_head]
 *       layout of the "单请求 KV Cache" tutorial (past_key_values 的数据结构);
 *       with an identity block table it is exactly that contiguous cache.
 *   block_table          int32 [batch, max_blocks_per_seq]: row b maps
 *       logical block j (positions 16j .. 16j+15) of sequence b to a physical
 *       block ("KV-Cache——为什么AI回复越来越快", 08 PagedAttention（vLLM）).
 *   seq_lens             int32 [batch]: length of sequence b AFTER this
 *       step's append, so the new row lands at position seq_lens[b] - 1
 *       ("KV缓存原理与显存估算", 前置知识: cache length counts the positions
 *       already forwarded).
 *   q, out               [batch, num_q_heads, head_dim]; query head h reads
 *       K/V head h / (num_q_heads / num_kv_heads) (contiguous groups: "KV-
 *       Cache——为什么AI回复越来越快", 03 三种Attention架构, GQA).
 * Types: KVD_BF16 tensors hold bfloat16, KVD_F32 tensors hold float.  The
 *   output has q's type; bf16 outputs are rounded to nearest even.  All
 *   arithmetic is fp32.
 */
#ifndef KVDECODE_H
#define KVDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KVD_F32 = 0, KVD_BF16 = 1 } kvd_dtype_t;

enum {
    KVD_OK = 0,
    KVD_ERR_NULL = -1,        /* a required pointer is NULL */
    KVD_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
    KVD_ERR_UNSUPPORTED = -3, /* dtype, head_dim, block_size or head ratio not built */
    KVD_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required */
    KVD_ERR_HIP = -5,         /* the HIP runtime reported a launch error */
    KVD_ERR_NOMEM = -6        /* block pool: too few free blocks, or host memory */
};

/* Static English text for a status code (never NULL). */
const char* kvd_status_string(int status);

/*
 * kvd_validate_tables -- the preconditions above, on HOST arrays (the checks
 * KVD_VALIDATE=1 runs).
 *   seq_lens     int32 [batch]; each must satisfy 1 <= seq_lens[b] <=
 *                min(max_seq_len, max_blocks_per_seq * 16) (max_seq_len <= 0:
 *                the table bound only)
 *   block_table  int32 [batch, max_blocks_per_seq]; the entries of blocks
 *                0 .. ceil(seq_lens[b] / 16) - 1 must lie in [0, num_blocks)
 *   new_rows     NULL, or int32 [batch]: sequence b receives its last
 *                new_rows[b] positions (0 <= new_rows[b] <= seq_lens[b]);
 *                every block holding one of them must appear exactly once
 *                among the visible entries of all sequences (owned, not
 *                shared: the copy-on-write rule of "KV Cache（键值缓存）", 2.3
 *                路线二)
 *   first_bad    NULL, or receives the first offending sequence (-1 if none)
 * Returns KVD_OK, KVD_ERR_SHAPE on a failed precondition, KVD_ERR_NULL for
 * missing arrays.  Reads only the arrays given; allocates host memory for a
 * per-block count when new_rows is given.
 */
int kvd_validate_tables(const int32_t* seq_lens, const int32_t* block_table, int batch,
                        int max_blocks_per_seq, int num_blocks, int max_seq_len,
                        const int32_t* new_rows, int* first_bad);

/*
 * kvd_validate_finite -- KVD_OK when the `count` HOST values at `data`
 * (bf16 or fp32 by dtype) are all finite, KVD_ERR_SHAPE when one is NaN or
 * infinite (the single-step attention sketch of "KV缓存原理与显存估算", 知识点二,
 * refuses non-finite inputs).
 */
int kvd_validate_finite(const void* data, size_t count, kvd_dtype_t dtype);

/*
 * kv_append_paged -- write this step's K/V rows into their cache slots.
 *
 * For each sequence b: pos = seq_lens[b] - 1, blk = block_table[b][pos / 16],
 * off = pos % 16; then K[blk][off][:][:] = k_new[b] and V[blk][off][:][:] =
 * v_new[b], an in-place O(1) slot write instead of re-concatenating the
 * history ("单请求 KV Cache", 生产系统的做法：预分配 + in-place 写入).  The
 * bytes are copied exactly; nothing else in the cache changes.
 *
 *   k_cache, v_cache  paged caches (layout above); v_cache may be NULL for a
 *                     single latent cache (MLA), then v_new must be NULL too
 *   k_new, v_new      [batch, num_kv_heads, head_dim] rows to store
 *   block_table, seq_lens  as above
 *   head_dim          any value in 1..1024 whose row size is a multiple of 4 B
 *   block_size        must be 16
 *   dtype             KVD_BF16 or KVD_F32
 * Returns KVD_OK or a negative status (nothing enqueued).
 */
int kv_append_paged(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int batch, int num_kv_heads, int head_dim, int block_size,
                    int max_blocks_per_seq, int num_blocks, kvd_dtype_t dtype, void* stream);

/*
 * decode_attn_partition_tokens -- the KV partition size (tokens) that the
 * decode calls will use for these sizes: `partition_tokens` itself when it is
 * positive (it must then be a multiple of 16), otherwise the library's
 * automatic choice.  For the paged path the automatic choice is 0, the
 * balanced split (below); for the latent path (head_dim = d_c = 512) and for
 * batches above 8191 it is a partition size.  Returns a negative status for
 * invalid sizes.
 */
int decode_attn_partition_tokens(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_seq_len, int partition_tokens);

/*
 * decode_attn_workspace_bytes -- bytes of device workspace a decode call
 * needs (fp32 partial results of every KV partition).  For MLA pass
 * num_kv_heads = 1 and head_dim = d_c.  Returns 0 for invalid sizes.
 */
size_t decode_attn_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                   int max_seq_len, int partition_tokens);

/*
 * decode_attn_paged -- single-query decode attention over a paged cache.
 *
 * For each sequence b and query head h, with g = h / (num_q_heads /
 * num_kv_heads) and L = seq_lens[b]:
 *   z_t = scale * q[b][h] . K_b[t][g]          for t in [0, L)
 *   out[b][h] = sum_t softmax(z)_t V_b[t][g]
 * where K_b[t] is the row at block_table[b][t / 16], offset t % 16 ("KV缓存原
 * 理与显存估算", 知识点二, the z / a / o equations; "KV-Cache——为什么AI回复越
 * 来越快", 02, the decode-step Attention(Q_{p+t}, K_cache, V_cache)).  All L
 * positions are visible: a single decode row has nothing in its future
 * ("单请求 KV Cache", 改动三).
 *
 * Implementation: positions are cut into pieces; a first kernel writes each
 * piece's running max, sum and unnormalised output into `workspace`, a
 * second merges the pieces by log-sum-exp into `out`.  The two phases are
 * also exported separately below.  With partition_tokens > 0 the pieces are
 * fixed partitions of that many tokens.  With partition_tokens = 0 (the
 * balanced split) every compute unit takes an equal share of all blocks of
 * the batch, whatever the mix of lengths, and a sequence is cut wherever the
 * shares end (at most ceil(ceil(max_seq_len / 16) / 16) + 1 pieces).
 *
 *   out              [batch, num_q_heads, head_dim], dtype
 *   q                [batch, num_q_heads, head_dim], dtype
 *   k_cache, v_cache [num_blocks, 16, num_kv_heads, head_dim], dtype
 *   head_dim         32, 64 or 128
 *   num_q_heads      a multiple of num_kv_heads; the ratio 1, 2 or a
 *                    multiple of 4 up to 64
 *   max_seq_len      host-known upper bound of seq_lens (sizes the grid)
 *   scale            score scale, normally 1/sqrt(head_dim)
 *   partition_tokens 0 for automatic, else a multiple of 16
 *   workspace        >= decode_attn_workspace_bytes(...) bytes, 256-B aligned
 */
int decode_attn_paged(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens,
                      int batch, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int max_blocks_per_seq, int num_blocks,
                      int max_seq_len, float scale, int partition_tokens,
                      void* workspace, size_t workspace_bytes, kvd_dtype_t dtype, void* stream);

/*
 * decode_attn_paged_partials -- first phase of decode_attn_paged only: fills
 * `workspace` with every partition's partial results.  Same arguments minus
 * `out`.  The workspace format is private to the library; pass it unchanged
 * to decode_attn_merge with the same sizes.
 */
int decode_attn_paged_partials(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               int batch, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq, int num_blocks,
                               int max_seq_len, float scale, int partition_tokens,
                               void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                               void* stream);

/*
 * decode_attn_merge -- second phase: for each (b, h), with M the largest
 * partition maximum, out = sum_p e^{m_p - M} acc_p / sum_p e^{m_p - M} l_p
 * over the partitions that hold positions of sequence b.  Sizes must equal
 * those of the partials call that filled `workspace` (for MLA: num_kv_heads =
 * 1, head_dim = d_c).
 */
int decode_attn_merge(void* out, const int32_t* seq_lens, int batch, int num_q_heads,
                      int num_kv_heads, int head_dim, int max_seq_len, int partition_tokens,
                      const void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                      void* stream);

/*
 * decode_attn_paged_window -- decode_attn_paged under a sliding window: the
 * row of sequence b attends to positions [max(0, L - window), L) only, the
 * most recent `window` tokens including this step's ("KV-Cache——为什么AI回复
 * 越来越快", Window Attention / Sliding Window; "KV缓存原理与显存估算": the
 * states outside the window may be dropped because the model's visible range
 * is different).  Blocks wholly before the window are never read, so their
 * table entries may be stale; the block holding position L - window must
 * still hold its positions.
 *   window  >= 1 (KVD_ERR_SHAPE otherwise); window >= L gives decode_attn_paged
 * Other arguments, sizes, workspace and errors as for decode_attn_paged; the
 * partials phase alone is decode_attn_paged_window_partials (finish with
 * decode_attn_merge, whose arguments do not change).
 */
int decode_attn_paged_window(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, int batch,
                             int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             int max_blocks_per_seq, int num_blocks, int max_seq_len,
                             float scale, int window, int partition_tokens, void* workspace,
                             size_t workspace_bytes, kvd_dtype_t dtype, void* stream);

int decode_attn_paged_window_partials(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      int max_seq_len, float scale, int window,
                                      int partition_tokens, void* workspace,
                                      size_t workspace_bytes, kvd_dtype_t dtype, void* stream);

/*
 * decode_attn_paged_append -- kv_append_paged followed by decode_attn_paged,
 * in one pass over the cache: the decode step of "KV-Cache——为什么AI回复越来越
 * 快" (02: this step's K/V join the cache, then the new query attends to all
 * of it) and of "单请求 KV Cache" (生产系统的做法: preallocated in-place slot
 * write).  Position seq_lens[b] - 1 takes its K/V from k_new / v_new (read
 * once, used as the last token of the softmax) and the rows are written into
 * their cache slot as kv_append_paged would write them; the other positions
 * are read from the cache.  The result equals the two separate calls up to
 * the order of floating-point accumulation.
 *   k_new, v_new  [batch, num_kv_heads, head_dim] dtype, 16-byte aligned
 *   k_cache, v_cache are written (the new rows' slots only)
 * Other arguments, sizes, workspace and errors as for decode_attn_paged.
 * Rows are written and used only for sequences with 1 <= seq_lens[b] <=
 * max_seq_len whose last block is inside the pool (the preconditions of the
 * separate calls); the block holding the new position must not be shared.
 */
int decode_attn_paged_append(void* out, const void* q, void* k_cache, void* v_cache,
                             const void* k_new, const void* v_new, const int32_t* block_table,
                             const int32_t* seq_lens, int batch, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size,
                             int max_blocks_per_seq, int num_blocks, int max_seq_len,
                             float scale, int partition_tokens, void* workspace,
                             size_t workspace_bytes, kvd_dtype_t dtype, void* stream);

/*
 * decode_attn_paged_append_partials -- first phase of decode_attn_paged_append
 * only (same arguments minus `out`); finish with decode_attn_merge.
 */
int decode_attn_paged_append_partials(const void* q, void* k_cache, void* v_cache,
                                      const void* k_new, const void* v_new,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      int max_seq_len, float scale, int partition_tokens,
                                      void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                                      void* stream);

/*
 * decode_attn_paged_append_noalloc -- decode_attn_paged_append for callers
 * that cannot allocate device memory: code recorded under HIP graph capture,
 * tight serving loops, and harnesses that forbid hipMalloc.  It takes no
 * workspace argument and calls no allocating routine: the partial results go
 * to a fixed device scratch array of KVD_NOALLOC_SCRATCH_BYTES (64 MiB) per
 * GPU, which the library holds from its first use on that GPU until the
 * process ends.
 *   Arguments, preconditions and results as for decode_attn_paged_append
 *   (the caller passes every input and `out`).
 *   Returns KVD_ERR_WORKSPACE when the call needs more than
 *   KVD_NOALLOC_SCRATCH_BYTES (decode_attn_workspace_bytes of the same sizes),
 *   KVD_ERR_HIP when the scratch address cannot be looked up.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents (nothing in it needs clearing: every value the merge
 *   reads is written by the same call first).  Calls that can overlap on one
 *   GPU -- on different streams, or from different host threads -- race on
 *   it; serialise them.
 */
#define KVD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int decode_attn_paged_append_noalloc(void* out, const void* q, void* k_cache, void* v_cache,
                                     const void* k_new, const void* v_new,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                     int block_size, int max_blocks_per_seq, int num_blocks,
                                     int max_seq_len, float scale, int partition_tokens,
                                     kvd_dtype_t dtype, void* stream);

/* Size in bytes of the scratch array of decode_attn_paged_append_noalloc. */
size_t decode_attn_noalloc_scratch_bytes(void);

/*
 * kvd_stream_read -- measurement aid, not a step of the decode: reads
 * `bytes` of device memory once (16-byte loads, each of 2048 workgroups of
 * 256 threads streaming one contiguous span) and writes almost nothing, so that its
 * duration gives the device's sustained HBM read rate, the practical ceiling
 * of a step that is bound by reading the cache ("KV-Cache——为什么AI回复越来
 * 越快", 04: decode is limited by moving the cache, not by arithmetic).
 *   src   device memory, 16-byte aligned; bytes a multiple of 16
 *   sink  device memory of at least kvd_stream_read_sink_bytes() bytes;
 *         a word of it is written only if a thread's fold of its words
 *         equals a fixed sentinel (contents otherwise untouched)
 * Returns KVD_OK, KVD_ERR_NULL, KVD_ERR_SHAPE (alignment / size),
 * KVD_ERR_WORKSPACE (sink too small) or KVD_ERR_HIP.  Asynchronous on stream.
 */
size_t kvd_stream_read_sink_bytes(void);
int kvd_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream);

/*
 * kvd_lds_read -- measurement aid, not a step of the decode: `groups`
 * workgroups of 512 threads (eight waves, the shape of the MLA kernel's
 * workgroup) each read a 64 KiB LDS array `iters` times, eight reads in
 * flight per lane, without bank conflicts, so that the rate gives one
 * compute unit's sustained LDS read bandwidth for the kinds of read that
 * feed the MLA and prefill kernels' MFMAs (context for their step times).
 *   mode    0: 16-byte reads (ds_read_b128); 1: 8-byte transposing reads of
 *           16-bit elements (ds_read_b64_tr_b16)
 *   groups  1 .. 65535 (one per compute unit measures one unit's rate)
 *   iters   1 .. 2^24; kvd_lds_read_bytes() gives the bytes read per launch
 *   cycles  device memory, 8-byte aligned, `groups` uint64 words: the shader
 *           clock cycles of each workgroup's read loop (wave 0's count)
 *   sink    device memory of at least kvd_lds_read_sink_bytes(groups)
 *           bytes; a word of it is written only if a thread's fold of its
 *           reads equals a fixed sentinel
 * Returns KVD_OK, KVD_ERR_UNSUPPORTED (mode), KVD_ERR_SHAPE, KVD_ERR_NULL,
 * KVD_ERR_WORKSPACE (sink too small) or KVD_ERR_HIP.  Asynchronous on stream.
 */
size_t kvd_lds_read_sink_bytes(int groups);
long long kvd_lds_read_bytes(int mode, int groups, int iters);
int kvd_lds_read(int mode, int groups, int iters, void* cycles, void* sink, size_t sink_bytes,
                 void* stream);

/*
 * decode_attn_mla -- absorbed multi-head latent attention decode (bf16).
 *
 * The cache keeps one row per token: the latent c_t (d_c values) followed by
 * the decoupled RoPE key k^R_t (d_rope values); the up-projections are folded
 * into the query and output projections, so each query head arrives as
 * q~ = [q~_c (d_c) ; q_R (d_rope)] ("KV Cache（键值缓存）", 2.2 路线一, the MLA
 * equations and the decoupled-RoPE note; section 4, MLA 的工程含义).
 *   z_t = scale * q~[b][h] . row_t      for t in [0, seq_lens[b])
 *   out[b][h] = sum_t softmax(z)_t c_t  (latent space, width d_c)
 * The caller chooses `scale` (the Python binding defaults to 1/sqrt(d_c/4 +
 * d_rope), the per-head width of the un-absorbed key when d_c = 4 d_h).
 * Both products run on MFMA with fp32 accumulation: the scores on bf16, the
 * value product on fp16, each softmax weight rounded to fp16 (11 bits) and
 * the latent values converted from bf16 (exact for magnitudes in [2^-14,
 * 65504], smaller ones off by at most 2^-25; latent values beyond 65504
 * overflow and the output holds inf/NaN).  The weight sum takes the fp32
 * weights.  Each partition's partial row is kept in the workspace divided by
 * its weight sum, in fp16 (its magnitudes are at most the latent values').
 *
 *   out      [batch, num_q_heads, d_c] bf16
 *   q        [batch, num_q_heads, d_c + d_rope] bf16
 *   c_cache  [num_blocks, 16, d_c + d_rope] bf16; append rows with
 *            kv_append_paged (num_kv_heads = 1, head_dim = d_c + d_rope,
 *            v_cache = v_new = NULL)
 *   d_c = 512, d_rope = 64; num_q_heads a multiple of 16
 *   partition_tokens 0 (automatic) or a multiple of 32
 *   workspace >= decode_attn_workspace_bytes(batch, num_q_heads, 1, d_c,
 *            max_seq_len, partition_tokens), 256-B aligned
 * Other arguments, errors and preconditions as for decode_attn_paged.
 */
int decode_attn_mla(void* out, const void* q, const void* c_cache,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int batch, int num_q_heads, int d_c, int d_rope, int block_size,
                    int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                    int partition_tokens, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * decode_attn_mla_partials -- first phase of decode_attn_mla only (same
 * arguments minus `out`); finish with decode_attn_merge(out, seq_lens, batch,
 * num_q_heads, 1, d_c, max_seq_len, partition_tokens, workspace, ..., KVD_BF16).
 */
int decode_attn_mla_partials(const void* q, const void* c_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int batch, int num_q_heads, int d_c, int d_rope, int block_size,
                             int max_blocks_per_seq, int num_blocks, int max_seq_len,
                             float scale, int partition_tokens, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * decode_attn_mla_append -- kv_append_paged of this step's latent rows
 * followed by decode_attn_mla, in one pass: the MLA cache of "KV Cache（键值
 * 缓存）" (2.2 路线一: one latent row per token and layer) grown by the
 * decode step's in-place slot write ("单请求 KV Cache", 生产系统的做法).
 * Position seq_lens[b] - 1 takes its row from c_new (read once, used in the
 * scores and the values like any cached row) and the row is written into its
 * cache slot as kv_append_paged would write it; the other positions are read
 * from the cache.  The result equals the two separate calls up to the order
 * of floating-point accumulation.
 *   c_new    [batch, d_c + d_rope] bf16, 16-byte aligned
 *   c_cache  is written (the new rows' slots only)
 * Other arguments, sizes, workspace and errors as for decode_attn_mla.  Rows
 * are written and used only for sequences with 1 <= seq_lens[b] <=
 * min(max_seq_len, 16 * max_blocks_per_seq) whose last block is inside the
 * pool; the block holding the new position must not be shared.
 */
int decode_attn_mla_append(void* out, const void* q, void* c_cache, const void* c_new,
                           const int32_t* block_table, const int32_t* seq_lens, int batch,
                           int num_q_heads, int d_c, int d_rope, int block_size,
                           int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                           int partition_tokens, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * decode_attn_mla_append_partials -- first phase of decode_attn_mla_append
 * only (same arguments minus `out`); finish with decode_attn_merge as after
 * decode_attn_mla_partials.
 */
int decode_attn_mla_append_partials(const void* q, void* c_cache, const void* c_new,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int batch, int num_q_heads, int d_c, int d_rope,
                                    int block_size, int max_blocks_per_seq, int num_blocks,
                                    int max_seq_len, float scale, int partition_tokens,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * INT8 KV cache ("KV-Cache——为什么AI回复越来越快", KV-Cache量化: one byte per
 * element halves the cache and the bytes a decode step reads; K is scaled per
 * channel, every dimension of a K/V head having its own scale, and V per
 * token, every token's row its own scale).
 *
 *   k_cache, v_cache [num_blocks, 16, num_kv_heads, head_dim] int8 codes in
 *                    [-127, 127], the layout of the bf16 caches
 *   k_scale          [num_kv_heads, head_dim] fp32, the per-channel K scales
 *                    (a calibration chosen by the caller)
 *   v_scale          [num_blocks, 16, num_kv_heads] fp32, one scale per token
 *                    and K/V head, addressed like the rows
 * A stored element stands for code * scale.
 */

/*
 * kv_append_paged_int8 -- the append of kv_append_paged into an INT8 cache:
 * position seq_lens[b] - 1 of sequence b gets
 *   K codes clip(round(k_new / k_scale), -127, 127) per channel,
 *   V scale s = max |v_new row| / 127 (per K/V head) and V codes
 *   clip(round(v_new / s), -127, 127) (s = 0 and codes 0 for a zero row),
 * every step in fp32 with correctly rounded divisions and round-half-to-even.
 *   k_new, v_new   [batch, num_kv_heads, head_dim] in dtype (KVD_BF16 or
 *                  KVD_F32), finite
 *   head_dim       32, 64 or 128
 * Other arguments, preconditions and errors as for kv_append_paged.
 */
int kv_append_paged_int8(int8_t* k_cache, int8_t* v_cache, float* v_scale, const void* k_new,
                         const void* v_new, const float* k_scale, const int32_t* block_table,
                         const int32_t* seq_lens, int batch, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int num_blocks,
                         kvd_dtype_t dtype, void* stream);

/*
 * decode_attn_paged_int8 -- decode_attn_paged over an INT8 cache: the same
 * attention with K[t][g][j] = k_scale[g][j] * code and V[t][g][j] =
 * v_scale[t][g] * code.  The scales are folded into the query (per channel)
 * and into the softmax weights (per token) in registers; the codes are
 * widened to fp16 exactly and the products accumulate in fp32.
 * Range: the scaled query q * k_scale and the weights times the V scales
 * (weights reach 2^8 before normalisation) are fp16 operands, so
 *   |q[b][h][j] * k_scale[g][j]| <= 65504 and v_scale[t][g] <= 255
 * (INT8: |V| up to ~32,000; FP8: up to ~114,000) keep the result finite;
 * beyond them the output holds inf or NaN.  Weight-scale products below
 * fp16's smallest normal number (6.1e-5) keep an absolute precision of
 * 6e-8 (2^-24) instead of 11 significant bits, which matters only for V
 * scales far below the 1e-2 .. 1e2 of typical activations.
 *   q, out     [batch, num_q_heads, head_dim] bf16 (dtype must be KVD_BF16)
 *   k_scale    16-byte aligned; v_scale 4-byte aligned
 * Other arguments (head_dim, ratios, partition_tokens, workspace), errors and
 * preconditions as for decode_attn_paged; the workspace is sized by
 * decode_attn_workspace_bytes with the same arguments.
 */
int decode_attn_paged_int8(void* out, const void* q, const int8_t* k_cache, const int8_t* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_table, const int32_t* seq_lens, int batch,
                           int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                           int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                           int partition_tokens, void* workspace, size_t workspace_bytes,
                           kvd_dtype_t dtype, void* stream);

/*
 * decode_attn_paged_int8_partials -- first phase of decode_attn_paged_int8
 * only (same arguments minus `out`); finish with decode_attn_merge.
 */
int decode_attn_paged_int8_partials(const void* q, const int8_t* k_cache, const int8_t* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int max_blocks_per_seq, int num_blocks,
                                    int max_seq_len, float scale, int partition_tokens,
                                    void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                                    void* stream);

/*
 * FP8 cache ("KV-Cache——为什么AI回复越来越快", KV-Cache量化: FP16 K/V stored
 * in FP8, one byte, with per-channel K and per-token V scales).  The same
 * layouts, scales and calls as the INT8 cache above, with E4M3 codes in place
 * of integers: the OCP 8-bit floating-point E4M3 format (sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 =
 * NaN, largest finite 448).
 *   append: code = E4M3(x / s) with the correctly rounded fp32 quotient, the
 *     nearest E4M3 value, ties to the even code, magnitudes beyond 448
 *     saturating to 448 (no NaN codes are written) and the quotient's sign
 *     bit kept (-0 for a negative quotient that rounds to zero); V's scale is
 *     max |v| / 448 of its own row (0 and all codes 0 for a zero row).
 *   decode: a stored value is E4M3(code) * scale.
 *   k_cache, v_cache  uint8 [num_blocks, 16, num_kv_heads, head_dim] codes
 * Other arguments, sizes, alignment and errors as for the INT8 functions.
 */
int kv_append_paged_fp8(uint8_t* k_cache, uint8_t* v_cache, float* v_scale, const void* k_new,
                        const void* v_new, const float* k_scale, const int32_t* block_table,
                        const int32_t* seq_lens, int batch, int num_kv_heads, int head_dim,
                        int block_size, int max_blocks_per_seq, int num_blocks,
                        kvd_dtype_t dtype, void* stream);

int decode_attn_paged_fp8(void* out, const void* q, const uint8_t* k_cache,
                          const uint8_t* v_cache, const float* k_scale, const float* v_scale,
                          const int32_t* block_table, const int32_t* seq_lens, int batch,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                          int partition_tokens, void* workspace, size_t workspace_bytes,
                          kvd_dtype_t dtype, void* stream);

/* decode_attn_paged_fp8_partials -- first phase of decode_attn_paged_fp8
 * (finish with decode_attn_merge, dtype KVD_BF16). */
int decode_attn_paged_fp8_partials(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, int max_blocks_per_seq, int num_blocks,
                                   int max_seq_len, float scale, int partition_tokens,
                                   void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                                   void* stream);

/*
 * Chunked prefill and multi-token decode ("单请求 KV Cache", 改动三: a row at
 * position past_len + i sees mask[i, :past_len + i + 1], the prefill triangle
 * for past_len = 0 and the decode row for one new token; "KV缓存原理与显存估算",
 * 知识点二: the new rows join the cache, then each query attends to it).
 * Sequence b has n_b = cu_rows[b + 1] - cu_rows[b] new rows, stored in row
 * order in q / k_new / v_new, and seq_lens[b] counts them.
 *
 * kv_append_paged_multi -- writes the n_b new K/V rows [N, num_kv_heads,
 * head_dim] to positions [seq_lens[b] - n_b, seq_lens[b]) through the block
 * table, as kv_append_paged does for one.  max_rows >= every n_b (sizes the
 * grid); rows of a sequence with n_b > seq_lens[b], or whose block lies
 * outside the pool, are not written.
 */
int kv_append_paged_multi(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          const int32_t* cu_rows, const int32_t* block_table,
                          const int32_t* seq_lens, int batch, int max_rows, int num_kv_heads,
                          int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                          kvd_dtype_t dtype, void* stream);

/*
 * prefill_attn_paged -- causal attention of the new rows: row i of sequence b
 * (position p = seq_lens[b] - n_b + i) gets softmax(scale q . K[0..p]) V[0..p]
 * per query head (K/V head h / (num_q_heads / num_kv_heads)).  The cache must
 * already hold all seq_lens[b] positions (kv_append_paged_multi first).
 *   q, out     [N, num_q_heads, head_dim] bf16 (dtype KVD_BF16), 16-byte aligned
 *   head_dim   64 or 128
 *   max_rows   >= every n_b, <= max_seq_len
 * Both products run on bf16 MFMA with fp32 accumulation; the softmax weights
 * enter as a bf16 value plus its bf16 remainder (~16 bits).  Other arguments
 * and errors as for decode_attn_paged (no workspace).
 */
int prefill_attn_paged(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* cu_rows, const int32_t* block_table,
                       const int32_t* seq_lens, int batch, int max_rows, int num_q_heads,
                       int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                       int num_blocks, int max_seq_len, float scale, kvd_dtype_t dtype,
                       void* stream);

/*
 * kv_copy_blocks -- copy whole physical blocks of one cache tensor: for each
 * pair i, block pairs[2 i] is copied onto block pairs[2 i + 1] (the copy a
 * copy-on-write append needs before it writes; see kvd_seq_append).
 *   cache       [num_blocks] blocks of block_bytes each (any element type;
 *               call once per tensor: K, V, and an INT8 cache's V scales)
 *   pairs       device int32 [num_pairs][2]; pairs naming a block outside
 *               [0, num_blocks) are skipped; destinations must be distinct and
 *               no destination may be another pair's source
 *   block_bytes a multiple of 4
 */
int kv_copy_blocks(void* cache, const int32_t* pairs, int num_pairs, size_t block_bytes,
                   int num_blocks, void* stream);

/*
 * Host-side paged block allocator ("KV-Cache——为什么AI回复越来越快", 08
 * PagedAttention: fixed-size pages, freed pages reused at once,
 * copy-on-write sharing of a common prefix; "KV Cache（键值缓存）", 2.3:
 * block tables, reference counts and copy-on-write between parallel samples;
 * "KV缓存原理与显存估算", 知识点三 and 源码导读: chained block hashes that
 * carry the whole prefix and a compatibility identity, reference counts for
 * who holds a block, hashes for what it holds).  Plain host memory; not
 * thread-safe (one pool per scheduler thread).  Every call succeeds
 * completely or changes nothing.
 *
 * Blocks carry a reference count.  A block whose count drops to zero is free
 * again; if it holds a registered hash it stays matchable until it is reused,
 * and blocks that never held a hash are reused first, then cached ones in
 * the order they were released.
 */
typedef struct kvd_block_pool kvd_block_pool;

/* Chained hashes of the full blocks of a token sequence: h_0 = SHA-256 of
 * (tag, identity, block tokens), h_j = SHA-256 of (tag, h_{j-1}, identity,
 * block tokens), tokens and lengths as little-endian 32-bit words.  Writes 32
 * bytes per full block to `out` and returns their number (a partial last
 * block gets none); tokens must be >= 0.  `identity` is any byte string
 * naming what makes cached states compatible (model, adapter, tokenizer,
 * dtype, salt). */
int kvd_block_hashes(const int32_t* tokens, int64_t num_tokens, int block_size,
                     const void* identity, size_t identity_bytes, uint8_t* out);

kvd_block_pool* kvd_pool_create(int num_blocks, int block_size); /* NULL on bad sizes */
void kvd_pool_destroy(kvd_block_pool* pool);
int kvd_pool_available(const kvd_block_pool* pool);  /* blocks an append may take */
int kvd_pool_used(const kvd_block_pool* pool);       /* blocks with count > 0 */
int kvd_pool_block_ref(const kvd_block_pool* pool, int block);

/* Sequences are small integers. */
int kvd_seq_create(kvd_block_pool* pool);           /* empty sequence */
int kvd_seq_fork(kvd_block_pool* pool, int seq);    /* shares every block (count + 1) */
int kvd_seq_release(kvd_block_pool* pool, int seq); /* count - 1 on each of its blocks */
int64_t kvd_seq_len(const kvd_block_pool* pool, int seq);
/* The block table; returns the number of blocks (capacity must hold them). */
int kvd_seq_table(const kvd_block_pool* pool, int seq, int32_t* out, int capacity);

/* Reserves slots for num_tokens more positions.  If the last block is partly
 * filled and shared, it is first replaced by a fresh block: the pair (old,
 * new) goes to copies[0..1] and *num_copies = 1, and the caller copies the
 * block's contents (kv_copy_blocks) before writing the new positions.  New
 * blocks are taken as needed.  KVD_ERR_NOMEM when the pool cannot supply
 * them (nothing changes). */
int kvd_seq_append(kvd_block_pool* pool, int seq, int num_tokens, int32_t* copies,
                   int max_copies, int* num_copies);

/* Registers the first num_hashes full blocks of seq under the given block
 * hashes (kvd_block_hashes of its tokens), so later sequences can reuse
 * them.  A block that already holds a hash, and a hash another block holds,
 * are left as they are. */
int kvd_seq_commit_hashes(kvd_block_pool* pool, int seq, const uint8_t* hashes, int num_hashes);

/* A new sequence that reuses the longest chain of registered blocks matching
 * hashes[0..], which is hashed, written-once state: *num_hit blocks, length
 * num_hit * block_size; the caller computes the positions after them. */
int kvd_seq_create_with_prefix(kvd_block_pool* pool, const uint8_t* hashes, int num_hashes,
                               int* num_hit);

#ifdef __cplusplus
}
#endif

#endif /* KVDECODE_H */
