/*
 * pkv.h -- C ABI of the paged-KV-cache decode library for AMD MI355X (gfx950).
 *
 * The KV cache of every sequence is split into fixed 16-token blocks that are
 * logically contiguous and physically scattered; a per-sequence block table
 * maps logical blocks to physical blocks, the decode kernel walks a
 * sequence's logical blocks through that table, and new tokens enter the
 * cache through a slot mapping.
 *   Sources: ipipp.com vLLM/PagedAttention article (2026-09-14), section 二
 *   "PagedAttention分页原理深度剖析" (16-token blocks, block table, block-wise
 *   kernel traversal); bytelighting wiki "vLLM", 核心机制 / 工作原理,
 *   "Flattened 布局与 slot_mapping" (slot mapping); ai-maas.com "vLLM 深读：
 *   用 PagedAttention 撑起高并发 LLM 推理", section 先看浪费在哪里 (physically
 *   scattered blocks, prefixes shared by pointing at the same blocks).
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers unless a comment says "host".  The caller
 *    owns and allocates every buffer; the library allocates nothing and keeps
 *    no state between calls (it is reentrant).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on that stream and returns; calls on one
 *    stream run in order (a write followed by a decode sees the write).
 *  - Arguments are validated on the host before anything is launched; the
 *    return value is a pkv_status.  The library never reads device arrays on
 *    the host (that would synchronise), so their CONTENTS are not validated
 *    up front.  Instead the kernels never touch memory outside the buffers
 *    the sizes describe: a table entry outside [0, num_blocks) makes its
 *    block count as empty, a length outside [0, max_blocks_per_seq*16] is
 *    clamped into that range, a slot outside [-1, num_blocks*16) is skipped.
 *    Results for such inputs are unspecified (but memory-safe).  This holds in
 *    every build: there is no separate debug build, no device error word and
 *    no debug-check call.  The validation entry point is pkv_check_inputs,
 *    one small launch that counts the contents the kernels would treat as
 *    invalid; a caller that wants the check runs it beside (or before) the
 *    calls whose inputs it covers.
 *  - All device pointers must be 16-byte aligned (PKV_ERR_ALIGNMENT).
 *  - block_size must be 16; head_dim must be 64 or 128; num_heads must be a
 *    multiple of num_kv_heads.  Supported (q, cache) dtype pairs for decode:
 *    (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).
 *
 * Pool layout.  K and V pools are separate, num_blocks * num_kv_heads tiles
 * of block_size * head_dim elements each; slot `sl` is offset
 * o = sl % block_size of physical block b = sl / block_size.  Inside a
 * (block, KV head) tile (the pages fix no in-block layout; this one lets the
 * decode kernel load matrix-core operands directly):
 *    k_cache[b][kv_head][d / X][o][d % X]   X = 16 / element bytes
 *            (each token row stored as 16-byte chunks of X consecutive
 *             dimensions, chunk-major: X = 4 f32, 8 bf16, 16 fp8)
 *    v_cache[b][kv_head][d][o]              (dimension-major)
 * fp8 pools hold OCP E4M3 codes (bias 7, max 448, no infinities); one fp32
 * scale per pool: value = decode(code) * k_scale (K) or * v_scale (V).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_dtype {
    PKV_DTYPE_F32 = 0,      /* IEEE binary32 */
    PKV_DTYPE_BF16 = 1,     /* bfloat16 */
    PKV_DTYPE_FP8_E4M3 = 2  /* OCP E4M3 code, one byte */
} pkv_dtype;

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = 1,  /* a size, scale or pointer argument is out of range */
    PKV_ERR_UNSUPPORTED = 2,  /* a valid but unimplemented combination (dtype pair, head_dim, block_size) */
    PKV_ERR_ALIGNMENT = 3,    /* a device pointer is not 16-byte aligned */
    PKV_ERR_WORKSPACE = 4,    /* workspace missing or smaller than paged_attention_workspace_bytes() */
    PKV_ERR_HIP = 5,          /* the HIP runtime reported an error while launching */
    PKV_ERR_OUT_OF_BLOCKS = 6, /* the block manager has too few free blocks (nothing was changed) */
    PKV_ERR_SCRATCH = 7        /* paged_attention_decode_noalloc: its static scratch is too small for these sizes */
} pkv_status;

/* Version of this ABI, incremented on any incompatible change or added
 * entry point:
 *   2 = the chunked-K / dimension-major-V pool layout, and the workspace
 *       query takes num_kv_heads;
 *   3 = the workspace must be zero-filled before its first use and is left
 *       that way by every call;
 *   4 = the block manager and paged_kv_copy_blocks;
 *   5 = paged_attention_decode_cascade;
 *   6 = paged_attention_varlen;
 *   7 = the block manager's prefix caching;
 *   8 = paged_attention_prefill;
 *   9 = paged_attention_decode_noalloc and PKV_ERR_SCRATCH;
 *  10 = the shared-prefix decode merges prefix and suffix states in a second
 *       launch: the workspace loses its meeting counters (every workspace is
 *       1 MiB smaller) and the num_seqs * runs limit of the cascade is gone;
 *  11 = pkv_tile_read (a measurement aid). */
int pkv_abi_version(void);

/* Static, NUL-terminated description of a status code (host). */
const char* pkv_status_string(int status);

/*
 * paged_kv_write -- store new tokens' K and V into the paged pools.
 *   Source: bytelighting wiki "vLLM", "Flattened 布局与 slot_mapping" (each
 *   token's logical position is sent to a physical slot); ipipp.com article
 *   §二 (16 tokens per block).
 *
 * k_new, v_new   [num_tokens][num_kv_heads][head_dim] in in_dtype.
 * k_cache,
 * v_cache        pools in cache_dtype, layouts as above.
 * slot_mapping   [num_tokens] int32: slot of token i, or -1 to skip it.
 *                Slots must be distinct (a repeated slot gives an unspecified
 *                one of the written values).
 * k_scale,
 * v_scale        used only when cache_dtype is FP8_E4M3 (must be finite and
 *                > 0 then): the code stored is the round-to-nearest-even,
 *                saturating (|y| >= 448 -> +-448, NaN -> NaN) E4M3 encoding of
 *                the fp32 quotient y = x / scale.
 * Supported: in_dtype == cache_dtype (bits copied), or cache FP8_E4M3 with
 * in_dtype F32 or BF16 (quantised).  num_tokens == 0 is a no-op.
 * Errors: PKV_ERR_INVALID_ARG (negative sizes, NULL pointers with
 * num_tokens > 0, bad scales, num_blocks*block_size >= 2^31),
 * PKV_ERR_UNSUPPORTED, PKV_ERR_ALIGNMENT, PKV_ERR_HIP.
 */
int paged_kv_write(const void* k_new, const void* v_new, int in_dtype,
                   void* k_cache, void* v_cache, int cache_dtype,
                   const int32_t* slot_mapping, int32_t num_tokens,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t num_blocks, float k_scale, float v_scale,
                   void* stream);

/*
 * paged_attention_workspace_bytes -- bytes of device workspace that
 * paged_attention_decode needs for these sizes (host; no device call).  The
 * workspace holds arrival counters and the partial softmax states of the runs
 * (sequence, group of query heads sharing a KV head) that the balanced work
 * split cuts between waves: two states per persistent wave (at most 4096
 * waves), so the size depends on the head grouping and head_dim only.  The
 * query takes num_kv_heads for that reason: a state holds one column per
 * query head of a run, and the heads per run follow from the group size
 * num_heads / num_kv_heads (the largest divisor of it that is at most 16).
 * partition_size as in paged_attention_decode.  Returns 0 for arguments
 * paged_attention_decode would reject.
 */
size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_size);

/*
 * paged_attention_decode -- one query token per sequence attends over its
 * paged context:
 *   out[s][h][:] = sum_t softmax_t(scale * q[s][h] . k_t) v_t,  t in [0, L_s)
 * with L_s = context_lens[s] and k_t, v_t read from physical block
 * block_table[s][t / 16] at offset t % 16, KV head h / (num_heads/num_kv_heads).
 *   Source: ipipp.com article §二 (for each logical block the kernel looks up
 *   the table and reads that block's K/V; the result equals attention over
 *   contiguous memory); bytelighting wiki "vLLM", 参考来源 (online softmax).
 *
 * out            [num_seqs][num_heads][head_dim] in q_dtype (round to nearest even).
 * q              [num_seqs][num_heads][head_dim] in q_dtype.
 * k_cache,
 * v_cache        pools as above, cache_dtype.
 * block_table    [num_seqs][max_blocks_per_seq] int32; entries at and after
 *                ceil(L_s/16) are never read (pad them with -1).
 * context_lens   [num_seqs] int32, each in [0, max_blocks_per_seq*block_size];
 *                L_s == 0 gives an all-zero output row.  L_s counts the token
 *                written in the current step.
 * scale          softmax scale (typically 1/sqrt(head_dim)).
 * k_scale,
 * v_scale        fp8 pool scales (ignored for F32/BF16 pools).
 * partition_size split-K granularity: 0 = balanced split only (the context
 *                blocks of all runs are cut into as many equal stretches as
 *                the chip runs waves), otherwise a positive multiple of 16:
 *                each stretch is further cut into equal partitions of at most
 *                partition_size tokens.  Every partition of a run gets its own
 *                softmax state (m, l, acc) and a run's states are merged with
 *                the rule M = max m_i, out = sum 2^(m_i-M) acc_i / sum
 *                2^(m_i-M) l_i (in registers within a wave, through the
 *                workspace between waves, by the last wave to finish its
 *                part; no second launch).  Between waves a state travels as
 *                m, l in fp32 and acc / l in the query dtype (bf16 for bf16
 *                queries: one more rounding of a partial result, as an output
 *                row would get).  The split changes rounding only; for fixed
 *                sizes and lengths the result is deterministic.
 * workspace      device buffer of >= paged_attention_workspace_bytes(...)
 *                bytes, owned by the caller, 16-byte aligned, zero-filled
 *                before its first use (every call that completes leaves its
 *                counters at zero again, so it is reused without clearing);
 *                calls that share a workspace must be ordered (same stream).
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED (also when
 * num_seqs * runs * max_blocks_per_seq >= 2^31), PKV_ERR_ALIGNMENT,
 * PKV_ERR_WORKSPACE, PKV_ERR_HIP.  num_seqs == 0 is a no-op.
 */
int paged_attention_decode(void* out,
                           const void* q, int q_dtype,
                           const void* k_cache, const void* v_cache, int cache_dtype,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           float scale, float k_scale, float v_scale,
                           int32_t partition_size,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode with no workspace
 * argument and no allocation of any kind.  For callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.
 *
 * The decode's workspace (arrival counters and the partial softmax states of
 * runs cut between waves) lives in a static device array of the library,
 * PKV_NOALLOC_SCRATCH_BYTES long, one per GPU, held from the first call on
 * that GPU until the process ends.  The first call on a device takes the
 * array's address and clears its counters with a small fill kernel on that
 * call's stream; every call that completes leaves them at zero again.
 * Arguments, results and errors as paged_attention_decode (same kernel, same
 * result bits), plus PKV_ERR_SCRATCH, returned before anything is launched,
 * when the states of the persistent waves do not fit: the counters (about
 * 64 KB) plus two states of 32 + run_heads * head_dim floats per wave, with
 * run_heads the largest divisor of num_heads / num_kv_heads that is at most
 * 16 and 2048 waves on MI355X for 16-bit and 8-bit pools.  So every shape
 * with run_heads <= 8 fits at head_dim 128 (17.4 MB at 8), and run_heads 16
 * at head_dim 128 does not (34.1 MB).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams without ordering between them, or from several
 * threads) race and give unspecified results.  Calls on one stream are
 * ordered and safe.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
int paged_attention_decode_noalloc(void* out,
                                   const void* q, int q_dtype,
                                   const void* k_cache, const void* v_cache, int cache_dtype,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   float scale, float k_scale, float v_scale,
                                   int32_t partition_size,
                                   void* stream);

/*
 * paged_attention_cascade_workspace_bytes -- workspace size for
 * paged_attention_decode_cascade: the decode workspace with merge slots wide
 * enough for a prefix run's columns, then two arrays of num_seqs * num_heads
 * state rows of head_dim + 4 floats.  Grows with num_seqs.  The state rows
 * hold data only; the counters sit where every workspace keeps them, so one
 * zero-filled buffer may serve plain and cascade calls of any shape in turn.
 * Returns 0 for arguments paged_attention_decode would reject.
 */
size_t paged_attention_cascade_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                               int32_t partition_size);

/*
 * paged_attention_decode_cascade -- the same result as paged_attention_decode
 * (up to rounding), reading each shared prefix block once for several of the
 * sequences that share it instead of once per sequence.
 *   Source: ai-maas.com article, 先看浪费在哪里 (parallel samples of one prompt
 *   share one prefix); ipipp.com article §二 (sequences of a beam search or a
 *   multi-turn chat have table entries pointing to the same physical blocks);
 *   the result is attention over each sequence's own table, so sharing only
 *   changes which reads serve which sequences.
 *
 * All arguments as in paged_attention_decode, plus:
 * prefix_leader  [num_seqs] int32 device array: the first sequence of s's
 *                sharing group.  A group is a run of consecutive sequences
 *                with the same leader; prefix_leader[s] == s for a sequence
 *                that shares nothing.
 * prefix_blocks  [num_seqs] int32 device array: the number of leading logical
 *                blocks s shares with every other member of its group (the
 *                same physical block ids in the same table positions), equal
 *                for all members; 0 = none.  Only whole blocks can be shared:
 *                the kernel uses min(prefix_blocks[s], L_s / 16).
 * The members of a group are served in chunks of 16 / (query heads per run)
 * consecutive sequences (4 for a GQA group of 4, 16 for one query head per KV
 * head): one prefix run per chunk and KV head reads the shared blocks through
 * the chunk's first table row and scores them for all the chunk's heads at
 * once.  Each sequence's remaining blocks are read by its own runs.  Both
 * kinds of run store their finished softmax state per (sequence, head) in the
 * workspace's state rows, and a second, small launch on the same stream merges
 * the two states of every head whose sequence has both (same rule as
 * partitions) and writes its output; a head whose context ends inside the
 * shared blocks is written by its prefix run directly.
 * A sequence whose entries disagree with its chunk's first sequence (another
 * leader or shared length, a leader after it) is decoded on its own; results
 * are unspecified (but memory-safe) when the shared blocks are in fact not the
 * same.  Setting prefix_blocks to all zeros gives plain decode.
 * workspace      >= paged_attention_cascade_workspace_bytes(...) bytes, with
 *                the same zero-fill and reuse contract as for
 *                paged_attention_decode.
 * Errors: as paged_attention_decode (PKV_ERR_UNSUPPORTED also when the state
 * rows need 2^31 bytes or more); PKV_ERR_INVALID_ARG for NULL prefix arrays.
 */
int paged_attention_decode_cascade(void* out,
                                   const void* q, int q_dtype,
                                   const void* k_cache, const void* v_cache, int cache_dtype,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens,
                                   const int32_t* prefix_leader, const int32_t* prefix_blocks,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   float scale, float k_scale, float v_scale,
                                   int32_t partition_size,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * paged_attention_varlen_workspace_bytes -- workspace size for
 * paged_attention_varlen: the decode workspace with merge slots 16 columns
 * wide.  Independent of the number of query rows.  Returns 0 for arguments
 * paged_attention_decode would reject.
 */
size_t paged_attention_varlen_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                              int32_t partition_size);

/*
 * paged_attention_varlen -- several new query tokens per sequence over the
 * paged cache (chunked prefill, verification of speculated tokens):
 *   out[r][h][:] = sum_{t <= p} softmax_t(scale * q[r][h] . k_t) v_t
 * for every query row r of sequence s (cu_seqlens_q[s] <= r <
 * cu_seqlens_q[s+1]), the i-th of its n = cu_seqlens_q[s+1] -
 * cu_seqlens_q[s] new tokens, which are the last n of its L_s cached tokens:
 * p = L_s - n + i (causal: a token sees its context and the new tokens up to
 * itself).  The new tokens' K/V must already be in the cache
 * (paged_kv_write takes any number of tokens per sequence).
 *   Source: bytelighting wiki "vLLM", "Flattened 布局与 slot_mapping"
 *   (cu_seqlens keeps the requests of a flattened batch apart); ai-maas.com
 *   article, 引擎的分层结构 (chunked prefill; speculative decoding verifies
 *   several guessed tokens in one pass).
 *
 * All arguments as in paged_attention_decode, except:
 * q, out         [num_q_rows][num_heads][head_dim] in q_dtype: rows are the
 *                new tokens of all sequences, sequence by sequence.
 * cu_seqlens_q   [num_seqs + 1] int32 device array: sequence s owns rows
 *                [cu_seqlens_q[s], cu_seqlens_q[s+1]); nondecreasing from 0
 *                to num_q_rows.  A sequence's count is clamped into
 *                [0, L_s]; rows a sequence does not claim, or that fall
 *                outside [0, num_q_rows), are not written (memory-safe for
 *                any contents).
 * The kernel serves 16 / (query heads per run) consecutive new tokens of a
 * sequence times the run's heads in one matrix tile (4 tokens for a GQA
 * group of 4), so each such group of tokens reads the context once, up to
 * the group's last token.
 * workspace      >= paged_attention_varlen_workspace_bytes(...) bytes, same
 *                zero-fill and reuse contract as paged_attention_decode.
 * Errors: as paged_attention_decode (PKV_ERR_UNSUPPORTED also when the units
 * or num_q_rows * num_heads * head_dim reach 2^31); PKV_ERR_INVALID_ARG for a
 * NULL cu_seqlens_q or num_q_rows < 0.  num_q_rows == 0 is a no-op.
 */
int paged_attention_varlen(void* out,
                           const void* q, int q_dtype, const int32_t* cu_seqlens_q, int32_t num_q_rows,
                           const void* k_cache, const void* v_cache, int cache_dtype,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           float scale, float k_scale, float v_scale,
                           int32_t partition_size,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * paged_attention_prefill -- the same result as paged_attention_varlen, in a
 * shape for long chunks of new tokens (chunked prefill).  One wave serves 32
 * query columns -- 32 / G consecutive new tokens of one sequence times the
 * G = num_heads / num_kv_heads query heads of one KV head -- and reads the
 * context once for all of them, up to its last token; waves serving
 * neighbouring tokens of one sequence and KV head run on one XCD, so their
 * reads meet in its L2.  There is no split over the context and no workspace.
 *   Source: as paged_attention_varlen (causal attention of a sequence's new
 *   tokens over its paged context).
 *
 * Arguments as in paged_attention_varlen, except:
 * max_q_len      an upper bound of the new tokens of any sequence (after the
 *                clamp into [0, L_s]); tokens of a sequence at index
 *                >= max_q_len are not computed and their rows not written.
 * (no partition_size, no workspace)
 * Supported: G from 1 to 32 (a wave holds floor(32 / G) tokens; when G does
 * not divide 32 the last columns stay empty), head_dim 64 or 128, the dtype
 * pairs of paged_attention_decode; otherwise PKV_ERR_UNSUPPORTED (use
 * paged_attention_varlen).  Rows no sequence claims, or outside
 * [0, num_q_rows), are not written.
 * Errors: as paged_attention_varlen; PKV_ERR_INVALID_ARG also for
 * max_q_len < 0.  num_seqs, num_q_rows or max_q_len == 0 is a no-op.
 */
int paged_attention_prefill(void* out,
                            const void* q, int q_dtype, const int32_t* cu_seqlens_q, int32_t num_q_rows,
                            int32_t max_q_len,
                            const void* k_cache, const void* v_cache, int cache_dtype,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            float scale, float k_scale, float v_scale,
                            void* stream);

/*
 * pkv_stream_read -- a plain streaming read of `bytes` bytes at `buf`
 * (16-byte nontemporal loads, each of PKV_STREAM_SINK_WORDS workgroups
 * reading one contiguous share).  `sink` is a device array of PKV_STREAM_SINK_WORDS
 * uint32 owned by the caller; the kernel may write any of them (in practice
 * none).  A measurement aid: its rate is the same-GPU reference beside the
 * decode's KV bandwidth.  Asynchronous on `stream`.
 * Errors: PKV_ERR_INVALID_ARG (NULL pointers with bytes > 0),
 * PKV_ERR_ALIGNMENT (buf or bytes not a multiple of 16, sink not 4-aligned),
 * PKV_ERR_HIP.  bytes == 0 is a no-op.
 */
#define PKV_STREAM_SINK_WORDS 8192
int pkv_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * pkv_tile_read -- the decode's read pattern without its arithmetic: 2048
 * one-wave workgroups each read an equal share of the list `ids` (n entries),
 * and for each entry the tile of `tile_bytes` at index id of `k`, then the
 * one at index id of `v`, with `depth` tiles in flight and nontemporal loads:
 * K by 16-byte lane loads, V by `v_load_bytes`-byte ones.  An id outside
 * [0, num_tiles) reads tile 0 or num_tiles - 1 (the reads stay in the
 * pools).  `sink` is a device array of PKV_TILE_SINK_WORDS uint32 owned by
 * the caller; the kernel may write any of them (in practice none).  A
 * measurement aid: it sets the V load widths, the depth and the tile size of
 * the decode's stream side by side.  Asynchronous on `stream`.
 * Supported (tile_bytes, v_load_bytes, depth): 2048 with (4, 8 or 16, 3) or
 * (4 or 16, 4) -- fp8 tiles of head_dim 128; 4096 with (4, 8 or 16, 2) --
 * bf16 tiles of head_dim 128; otherwise PKV_ERR_UNSUPPORTED.
 * Errors: PKV_ERR_INVALID_ARG (n or num_tiles < 0; NULL pointers or
 * num_tiles == 0 with n > 0), PKV_ERR_ALIGNMENT (k or v not 16-aligned, ids
 * or sink not 4-aligned), PKV_ERR_HIP.  n == 0 is a no-op.
 */
#define PKV_TILE_SINK_WORDS 2048
int pkv_tile_read(const void* k, const void* v, const int32_t* ids, int32_t n, int32_t num_tiles,
                  int32_t tile_bytes, int32_t v_load_bytes, int32_t depth, uint32_t* sink, void* stream);

/*
 * pkv_check_inputs -- count the contents of the index arrays that the kernels
 * treat as invalid.  The write and decode stay memory-safe for any contents
 * (an out-of-range table entry is an empty block, a length is clamped into
 * [0, max_blocks_per_seq*16], an out-of-range slot is skipped), so their
 * results are simply unspecified for such inputs; this call says whether that
 * happened.  It is the boundary's validation call (there is no debug build
 * or device error word).  Two launches: one workgroup for the lengths, table
 * entries and slot ranges, then ceil(num_tokens / 4096) workgroups that find
 * repeated slots through hash tables in LDS (linear in num_tokens for any
 * practical input).
 *   Source for what is valid: ipipp.com article §二 (the table maps each
 *   logical block to a physical one); bytelighting wiki "vLLM", "Flattened
 *   布局与 slot_mapping" (one slot per new token).
 *
 * block_table,
 * context_lens   as in paged_attention_decode (may be NULL when num_seqs == 0;
 *                block_table may be NULL when max_blocks_per_seq == 0).
 * slot_mapping   as in paged_kv_write (may be NULL when num_tokens == 0).
 * num_blocks     pool size in blocks.
 * counts         device int32[4], 16-byte aligned, overwritten
 *                asynchronously on `stream`:
 *                  [0] sequences whose context_lens entry is < 0 or above
 *                      max_blocks_per_seq*16;
 *                  [1] table entries the decode reads (j < ceil(L/16), L
 *                      clamped as above) outside [0, num_blocks);
 *                  [2] slot_mapping entries that are neither -1 nor in
 *                      [0, num_blocks*16);
 *                  [3] slot_mapping entries >= 0 that repeat an earlier entry.
 * Errors: PKV_ERR_INVALID_ARG (negative sizes, NULL counts or a NULL array
 * with a non-zero size, size products >= 2^31), PKV_ERR_ALIGNMENT,
 * PKV_ERR_HIP.
 */
int pkv_check_inputs(const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs,
                     const int32_t* slot_mapping, int32_t num_tokens,
                     int32_t num_blocks, int32_t* counts, void* stream);

/*
 * ---- Host block manager (no device calls) --------------------------------
 *
 * Hands out the 16-token blocks of a pool of num_blocks on demand, lets
 * sequences share blocks (fork: parallel sampling, beam search), and gives a
 * sequence a private copy of a shared, partly filled last block when it first
 * writes into it (copy-on-write).  It produces the slot_mapping entries for
 * paged_kv_write and the block_table rows and context_lens for
 * paged_attention_decode.
 *   Source: ai-maas.com vLLM article, 先看浪费在哪里 (blocks requested and
 *   returned on demand instead of a max_len reservation per request);
 *   ipipp.com article §二 (per-sequence block table; blocks shared between
 *   sequences with reference counts; a shared block is copied when written).
 *
 * Allocation is deterministic: free blocks form a stack that starts as
 * [num_blocks-1, ..., 1, 0], so block 0 is handed out first, and a block
 * returns to the top when its last reference goes (a freed sequence releases
 * its blocks in table order).  A copy-on-write queues a block copy (src ->
 * dst); pending copies keep both blocks from being handed out until
 * pkv_bm_take_copies returns them.  The caller must run the taken copies with
 * paged_kv_copy_blocks on the stream before any later paged_kv_write.
 * The manager is plain host state, owned by the caller, not thread-safe.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager for a pool of num_blocks blocks, at most max_blocks_per_seq per
 * sequence.  NULL for negative sizes, num_blocks*16 >= 2^31, or no memory. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t max_blocks_per_seq);
void pkv_bm_destroy(pkv_block_manager* m);

/* A new empty sequence.  PKV_ERR_INVALID_ARG if seq_id exists. */
int pkv_bm_add(pkv_block_manager* m, int64_t seq_id);

/* child shares every block of parent (reference counts +1) and its length.
 * PKV_ERR_INVALID_ARG if parent is unknown, child exists or they are equal. */
int pkv_bm_fork(pkv_block_manager* m, int64_t parent, int64_t child);

/* Reserve slots for n new tokens at the end of seq_id: slots_out[i] (host
 * int32[n]) = block*16 + offset of token len+i.  Allocates blocks as needed
 * and queues a copy when the last block is shared and partly filled.
 * PKV_ERR_OUT_OF_BLOCKS (state unchanged) when the pool or max_blocks_per_seq
 * is exhausted; PKV_ERR_INVALID_ARG for an unknown sequence or n < 0. */
int pkv_bm_append(pkv_block_manager* m, int64_t seq_id, int32_t n, int32_t* slots_out);

/* Drop seq_id; its blocks lose one reference each and are freed at zero. */
int pkv_bm_free(pkv_block_manager* m, int64_t seq_id);

/* Rows of the block table for n sequences: table_out (host int32
 * [n][max_blocks]) gets each sequence's blocks, -1 padded; lens_out (host
 * int32[n]) its length.  PKV_ERR_INVALID_ARG (nothing written) for an unknown
 * sequence or one with more than max_blocks blocks. */
int pkv_bm_table(const pkv_block_manager* m, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                 int32_t* table_out, int32_t* lens_out);

/* Take up to max_copies pending copies, oldest first, into src_out/dst_out
 * (host int32[max_copies]); the batch stops before a copy that reads a block
 * an earlier copy of the batch writes, so one paged_kv_copy_blocks call can
 * run it in parallel (call again for the rest).  Returns the count, -1 on bad
 * arguments. */
int32_t pkv_bm_take_copies(pkv_block_manager* m, int32_t* src_out, int32_t* dst_out, int32_t max_copies);

/* out (host int64[5]): free blocks, used blocks, live sequences, tokens held
 * by the used blocks (a shared block counted once), pending copies. */
int pkv_bm_stats(const pkv_block_manager* m, int64_t* out);

/*
 * Automatic prefix caching (off unless enabled).
 *   Source: bytelighting wiki "vLLM", paragraph on Automatic Prefix Caching
 *   (a prefix is cut into fixed blocks; each block's hash chains its parent's
 *   hash and its own content; cached blocks live in a hash table, are
 *   allocated, freed and LRU-evicted on their own; a hit matches block by
 *   block exactly and reuses only full blocks); ai-maas.com article, 引擎的分
 *   层结构 (repeated prefixes such as system prompts are computed once and
 *   shared).
 *
 * pkv_bm_enable_prefix_caching: turn caching on for an empty manager (no
 *   sequences, no pending copies); PKV_ERR_INVALID_ARG otherwise.  From then
 *   on every block a sequence with known token ids fills is registered under
 *   the chained hash of its content (the parent's hash mixed with the
 *   block's 16 token ids; a 64-bit mix that only narrows the search), unless
 *   a block with the same content after the same registered predecessor is
 *   registered already.  A registered block whose last reference goes is
 *   kept as evictable; when no never-registered block is free, the
 *   least recently released evictable block is taken (and unregistered).  A
 *   freed sequence releases its blocks deepest first.  pkv_bm_stats counts
 *   evictable blocks as free.
 * pkv_bm_add_prompt: add sequence seq_id (new) with its n prompt token ids.
 *   Its first blocks reuse the longest run of registered full blocks that
 *   match the prompt exactly (token ids, and each block's predecessor), at
 *   most (n - 1) / 16 blocks, so the last prompt token is always computed.
 *   *cached_out = the number of reused tokens (a multiple of 16); the slots
 *   of the other n - *cached_out tokens are written to slots_out, whose K/V
 *   the caller writes with paged_kv_write.  PKV_ERR_OUT_OF_BLOCKS leaves the
 *   manager unchanged.
 * pkv_bm_append_tokens: pkv_bm_append with the new tokens' ids, so the blocks
 *   they fill can be registered.  (pkv_bm_append without ids stops the
 *   registration of that sequence's later blocks.)
 * pkv_bm_cache_stats: out[0] registered blocks, out[1] of them evictable,
 *   out[2] full prompt blocks looked up, out[3] of them reused, out[4]
 *   evictions.
 */
int pkv_bm_enable_prefix_caching(pkv_block_manager* m);
int pkv_bm_add_prompt(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t n, int32_t* slots_out,
                      int32_t* cached_out);
int pkv_bm_append_tokens(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t n,
                         int32_t* slots_out);
int pkv_bm_cache_stats(const pkv_block_manager* m, int64_t* out);

/*
 * paged_kv_copy_blocks -- copy whole blocks of both pools, K and V of every
 * KV head: block dst[i] <- block src[i] for i < n (the copies of a
 * copy-on-write).  src, dst: device int32[n].  Pairs with an id outside
 * [0, num_blocks) are skipped.  The destinations must be distinct and no
 * destination may be another pair's source (pkv_bm_take_copies batches that
 * way).  Asynchronous on `stream`; n == 0 is a no-op.
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED (dtype, head_dim,
 * block_size), PKV_ERR_ALIGNMENT, PKV_ERR_HIP.
 */
int paged_kv_copy_blocks(void* k_cache, void* v_cache, int cache_dtype, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, const int32_t* src, const int32_t* dst, int32_t n,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
