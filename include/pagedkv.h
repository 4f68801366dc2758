/*
 * pagedkv.h - C ABI of the paged KV-cache attention library (MI355X, gfx950).
 *
 * The KV cache of one attention layer is a pool of fixed-size blocks,
 *
 *     kv_pool[num_blocks][block_size][2][num_kv_heads][head_size]   (fp16)
 *
 * the per-layer pool tensor of the page "vLLM 部署深度指南" (section
 * "PagedAttention 原理", code listing of the simplified KV-cache class).
 * Index 0 of the axis of size 2 holds keys, index 1 values; under
 * grouped-query attention the head axis counts KV heads. A block holds 16
 * tokens (same page, "PagedAttention 方案" and the --block-size default in the
 * launch-flag table). Sequence b reaches its tokens through row b of
 * block_tables: logical block j of the sequence lives in physical block
 * block_tables[b * max_blocks_per_seq + j], so logical position t is slot
 * block_tables[b][t / 16] * 16 + t % 16 (page "vLLM GitHub 项目 …", section 二,
 * items 1 and 4: blocks need not be contiguous and may be shared).
 *
 * Conventions for every entry point below:
 *  - Pointers named as device pointers must point to device memory the caller
 *    owns and keeps alive until the work on `stream` is done. The library
 *    allocates no memory and keeps no state except a per-thread message of the
 *    last HIP error (pa_last_error).
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream. Every
 *    device operation is asynchronous and ordered on `stream`; nothing waits
 *    for the device.
 *  - All tensors are dense, row-major, in the element types stated. fp16 is
 *    IEEE binary16; fp32 is IEEE binary32.
 *  - A status other than PA_OK means nothing was launched. Scalar arguments
 *    are checked on the host before any launch. Device-resident contents
 *    (lengths, table entries, slots) are checked by the kernels where a bad
 *    value would address memory outside the pool or the tables: such a row's
 *    output is set to NaN (decode, prefill) or the token is skipped (append).
 *  - Sizes the device work depends on (max_context_len, max_q_len) are host
 *    scalars, so no call ever reads device memory from the host.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = 1,     /* null pointer, non-positive count, inconsistent sizes      */
  PA_ERR_UNSUPPORTED = 2, /* valid request with no kernel here: block_size != 16,
                             head_size not in {64, 128}, group size not in {1,2,4,8}  */
  PA_ERR_WORKSPACE = 3,   /* workspace smaller than pa_decode_workspace_bytes         */
  PA_ERR_HIP = 4,         /* the HIP runtime refused a launch; see pa_last_error       */
  PA_ERR_EXHAUSTED = 5    /* the block manager's free list cannot cover the request     */
} pa_status;

/* Static text for a status code. Never NULL. */
const char* pa_status_string(int status);
/* Text of the last HIP error seen on this thread ("" if none). Never NULL. */
const char* pa_last_error(void);
/* ABI version, currently 1. */
int32_t pa_abi_version(void);

/* ---------------------------------------------------------------------------
 * Layout helpers: pure host arithmetic, no device access. A negative return
 * value means an argument was out of range.
 * ------------------------------------------------------------------------- */

/* Blocks held by a sequence of `len` tokens: ceil(len / block_size)
 * ("allocate" in the KV-cache listing on page "vLLM 部署深度指南"). */
int64_t pa_blocks_for_len(int64_t len, int32_t block_size);

/* Bytes of one block: block_size * 2 * num_kv_heads * head_size * elem_bytes. */
int64_t pa_block_bytes(int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                       int32_t elem_bytes);

/* Bytes of a pool of num_blocks blocks. */
int64_t pa_pool_bytes(int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                      int32_t head_size, int32_t elem_bytes);

/* Blocks that fit in floor(free_bytes * utilization) bytes; the sizing rule of
 * the --gpu-memory-utilization flag (default 0.9) on page "vLLM 部署深度指南".
 * utilization must lie in (0, 1]. */
int64_t pa_num_blocks_fit(int64_t free_bytes, double utilization, int32_t block_size,
                          int32_t num_kv_heads, int32_t head_size, int32_t elem_bytes);

/* Slot of logical position `pos` of a sequence whose block-table row (host
 * memory, at least pos / block_size + 1 entries) is `block_table_row`:
 * block_table_row[pos / block_size] * block_size + pos % block_size. Logical
 * block j of a sequence is held by whichever physical block its table names
 * (page "vLLM GitHub 项目 …", section 二, item 1; page "vLLM 部署深度指南",
 * section "PagedAttention 原理": the block-table figure maps logical to
 * physical blocks). -1 for a NULL row, pos < 0 or a negative entry. */
int64_t pa_slot(const int32_t* block_table_row, int64_t pos, int32_t block_size);

/* Element offset in the pool of (slot, kv, head, dim); kv 0 = key, 1 = value:
 * ((slot * 2 + kv) * num_kv_heads + head) * head_size + dim, the row-major index of
 * the pool tensor [num_blocks][block_size][2][num_kv_heads][head_size] of the
 * simplified KV-cache listing (page "vLLM 部署深度指南", section "PagedAttention
 * 原理"). -1 when an index is out of range. */
int64_t pa_kv_elem_offset(int64_t slot, int32_t kv, int32_t head, int32_t dim,
                          int32_t num_kv_heads, int32_t head_size);

/* Partitions of a context of max_context_len tokens: ceil(len / partition_size),
 * at least 1. */
int32_t pa_num_partitions(int32_t max_context_len, int32_t partition_size);

/* A partition size for pa_decode / pa_decode_fp8 on this library's kernels (measured on
 * MI355X): as few partitions as keep the GPU busy. A wave serves one (sequence, KV head,
 * partition), so P = ceil(W / (num_seqs * num_kv_heads)) partitions with W = 4096 waves
 * (one query head per KV head) or 2048 (grouped query heads, a kernel that holds fewer
 * waves per SIMD); the size is ceil(max_context_len / P) rounded up to a multiple of 16,
 * and at least 512 tokens when P > 16 (up to 16 partitions pa_decode schedules the
 * longest first). -1 for a negative length or count, or a head count that is not a
 * multiple of num_kv_heads. */
int32_t pa_decode_default_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t max_context_len);

/* Workspace bytes pa_decode uses. With several partitions: the partial results,
 * num_seqs * num_q_heads * partitions * (head_size + 2) * 4 bytes, plus an item list of
 * 4 * (1 + num_seqs * partitions) bytes (the order in which partitions are scheduled),
 * each part rounded up to 256 bytes; pa_decode requires them. With one partition: the
 * item list alone, 4 * (1 + num_seqs) bytes rounded up to 256; optional (pa_decode then
 * accepts a NULL or smaller workspace and runs the sequences in launch order, with the
 * same results). */
int64_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t partition_size,
                                  int32_t head_size);

/* ---------------------------------------------------------------------------
 * Device operations.
 * ------------------------------------------------------------------------- */

/* Write this step's new tokens into their slots (``append_kv`` of the listing on
 * page "vLLM 部署深度指南": new K/V go into the sequence's physical block, which
 * need not be contiguous with the others).
 *
 *   kv_pool      device fp16 [num_blocks][block_size][2][num_kv_heads][head_size], written
 *   key, value   device fp16, token t's row at key + t * key_token_stride (elements),
 *                num_kv_heads * head_size contiguous elements per row; a stride of 0
 *                means num_kv_heads * head_size
 *   slot_mapping device int64 [num_tokens]: token t goes to slot slot_mapping[t]
 *                (block * block_size + offset). A negative slot skips the token, and so
 *                does a slot >= num_blocks * block_size. Slots must be distinct; with
 *                duplicates the surviving value is unspecified.
 * Copies bits: the pool afterwards holds exactly the given fp16 values. */
pa_status pa_kv_append(void* kv_pool, const void* key, const void* value,
                       const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                       int32_t head_size, int32_t block_size, int64_t num_blocks,
                       int64_t key_token_stride, int64_t value_token_stride, void* stream);

/* One decode step of paged attention: query row b (one token per sequence, at the
 * sequence's last position) attends to the first context_lens[b] tokens of
 * sequence b, the token appended this step included. The keys and values are
 * found block by block through the sequence's table (page "vLLM GitHub 项目 …",
 * section 二, item 1: logical blocks mapped to non-contiguous physical blocks;
 * page "vLLM 部署深度指南", section "PagedAttention 原理": the pool layout), and
 * the attention is textbook softmax attention over them.
 *
 *   out           device fp16 [num_seqs][num_q_heads][head_size], written
 *   q             device fp16 [num_seqs][num_q_heads][head_size]
 *   kv_pool       device fp16 pool (layout above), read
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq], entries in [0, num_blocks)
 *                 for the first ceil(context_lens[b] / block_size) of row b; the rest
 *                 are never read
 *   context_lens  device int32 [num_seqs], each in [0, max_context_len] and at most
 *                 max_blocks_per_seq * block_size. A length of 0 gives a zero row; a
 *                 length outside these bounds, or a table entry outside
 *                 [0, num_blocks), gives a NaN row.
 *   scale         softmax scale, finite and > 0, normally 1 / sqrt(head_size)
 *                 (PA_ERR_INVALID otherwise)
 *   partition_size  tokens per split-context partition, a positive multiple of
 *                 block_size; a context longer than one partition is computed as
 *                 partitions merged by a log-sum-exp reduction
 *   workspace     device memory of at least pa_decode_workspace_bytes(...) bytes,
 *                 256-byte aligned (may be NULL when one partition covers
 *                 max_context_len); scratch only
 *   flags         0 or PA_DECODE_KV_STREAM: every block is read by one sequence only in
 *                 this call, so K/V loads carry the non-temporal cache hint (HBM
 *                 streaming rate) and the partitions are scheduled longest first. Leave
 *                 it off when sequences share prefix blocks, so shared blocks may be
 *                 served from cache (neighbouring sequences then run together). Results
 *                 are identical.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads). Arithmetic: fp16
 * inputs, fp32 products, sums and online softmax (base-2 exponentials of
 * log2(e)-scaled scores), fp16 output rounded to nearest even.
 *  - One query head per KV head: the probabilities p stay fp32 and the running max is
 *    the exact running max.
 *  - Grouped query heads (2, 4 or 8 per KV head): the scores and the P.V product run
 *    on the matrix cores, which take p rounded to fp16 (nearest even); the row sum l
 *    adds those same fp16 values in fp32, so out = sum p v / sum p holds for the values
 *    used. The reference max a row subtracts moves only when a score beats it by more
 *    than 2^8 (in base-2 units), so p <= 2^8 and the accumulator is rescaled rarely;
 *    the result is unchanged up to rounding.
 * With several partitions each writes fp32 partial results (o, m, l) that a second
 * kernel merges by log-sum-exp. */
#define PA_DECODE_KV_STREAM 1u
pa_status pa_decode(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                    float scale, int32_t partition_size, void* workspace,
                    int64_t workspace_bytes, uint32_t flags, void* stream);

/* ---- decode that allocates nothing ----------------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace of their own: code
 * being captured into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.
 * pa_decode_noalloc is pa_decode (same arguments without the workspace, same kernels,
 * bit-identical results) whose workspace is a fixed device array inside the library,
 * PA_DECODE_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from the first call on that GPU
 * until the process ends. It runs on the current device (hipGetDevice), which must be the
 * device of `stream` and of every buffer. It calls no allocator.
 *  - A call whose pa_decode_workspace_bytes(...) exceeds the array returns
 *    PA_ERR_WORKSPACE before any device access (pa_last_error gives the sizes); bad sizes
 *    return PA_ERR_INVALID.
 *  - Every call on one GPU uses that GPU's one array, which keeps the last call's
 *    contents. Nothing in it needs to start at zero. Calls whose work may overlap on one
 *    GPU (several streams, several threads) race on it: the caller serialises them. */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES (32ll << 20)
pa_status pa_decode_noalloc(void* out, const void* q, const void* kv_pool,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                            int64_t num_blocks, int32_t max_context_len, float scale,
                            int32_t partition_size, uint32_t flags, void* stream);

/* ---- shared-prefix decode ------------------------------------------------------------
 * Sequences that share a prompt point their tables at the same blocks, which avoids
 * storing and computing the prompt twice (page "vLLM GitHub 项目 …", section 二, item 4:
 * parallel sampling and beam search). pa_decode_shared_prefix computes exactly what
 * pa_decode computes, reading each group's shared prefix once: the prefix is one pass per
 * (group, KV head) whose matrix-core tile columns are the group's (sample, query head)
 * pairs (16 / (num_q_heads / num_kv_heads) samples per tile), then every sequence's own
 * tokens are one pass each, and a log-sum-exp reduction merges the two.
 *
 *   group_start     device int32 [num_groups + 1]: sequences group_start[g] ..
 *                   group_start[g + 1] - 1 form group g (non-decreasing, 0 .. num_seqs;
 *                   a sequence with nothing shared is a group of its own)
 *   prefix_lens     device int32 [num_groups]: tokens every member of group g shares, a
 *                   multiple of block_size, at most each member's context length; the
 *                   first prefix_lens[g] / block_size entries of every member's table row
 *                   are the same (the call reads them from the group's first member)
 *   max_group_size  host bound on the group sizes; max_prefix_len host bound on
 *                   prefix_lens (a multiple of block_size, at most max_context_len)
 *   workspace       pa_decode_shared_prefix_workspace_bytes(...) bytes, 256-byte aligned
 * Other arguments as pa_decode (fp16 pool; K/V loads keep the cache hint, since blocks are
 * shared). A row whose group, prefix or length breaks these bounds is NaN; a length of 0
 * gives zeros. Arithmetic as pa_decode's grouped-query path for every group size (the
 * tiles run on the matrix cores with p rounded to fp16, the reference max lagging by
 * up to 2^8), the prefix and own-token passes merged by log-sum-exp in fp32. */
pa_status pa_decode_shared_prefix(void* out, const void* q, const void* kv_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_size, int32_t block_size,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  int32_t max_context_len, float scale, int32_t partition_size,
                                  const int32_t* group_start, const int32_t* prefix_lens,
                                  int32_t num_groups, int32_t max_group_size,
                                  int32_t max_prefix_len, void* workspace,
                                  int64_t workspace_bytes, void* stream);
int64_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                int32_t max_context_len, int32_t max_prefix_len,
                                                int32_t partition_size, int32_t head_size);

/* ---- FP8 KV cache ---------------------------------------------------------------------
 * The pool may hold OCP FP8 E4M3 codes, one byte per element, in the same layout
 * [num_blocks][block_size][2][num_kv_heads][head_size] (page "vLLM 部署深度指南": the FP8
 * deployment command's --kv-cache-dtype fp8; FP8 halves memory in the quantisation
 * table). One fp32 scale per tensor: a key element x is stored as the E4M3 code of
 * fp32(x) * fp32(1 / k_scale) (the product rounded once in fp32), rounded to nearest
 * even, magnitudes of 448 and more saturated to 448, NaN kept NaN; values likewise with
 * v_scale. Attention reads code value * scale. Both scales must be finite and > 0.
 *
 * pa_kv_append_fp8: pa_kv_append into an E4M3 pool (key and value are fp16 as before;
 *   the pool's element is one byte). Writes exactly the codes above.
 * pa_decode_fp8: pa_decode over an E4M3 pool, same arguments and results plus the two
 *   scales; each code is widened exactly to fp16 and the scales applied in fp32 (the key
 *   scale with the softmax scale, the value scale with the final normalisation).
 * pa_prefill_chunk_fp8: pa_prefill_chunk over an E4M3 pool, likewise.
 * pa_decode_shared_prefix_fp8: pa_decode_shared_prefix over an E4M3 pool, likewise. */
pa_status pa_kv_append_fp8(void* kv_pool, const void* key, const void* value,
                           const int64_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                           int64_t num_blocks, int64_t key_token_stride,
                           int64_t value_token_stride, float k_scale, float v_scale,
                           void* stream);
pa_status pa_decode_fp8(void* out, const void* q, const void* kv_pool,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                        int64_t num_blocks, int32_t max_context_len, float scale,
                        float k_scale, float v_scale, int32_t partition_size, void* workspace,
                        int64_t workspace_bytes, uint32_t flags, void* stream);
pa_status pa_prefill_chunk_fp8(void* out, const void* q, const void* kv_pool,
                               const int32_t* block_tables, const int32_t* query_start_loc,
                               const int32_t* seq_lens, int32_t num_reqs, int32_t total_q,
                               int32_t max_q_len, int32_t max_seq_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                               int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                               float k_scale, float v_scale, void* workspace,
                               int64_t workspace_bytes, void* stream);
pa_status pa_decode_shared_prefix_fp8(void* out, const void* q, const void* kv_pool,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_size,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int32_t max_context_len, float scale,
                                      float k_scale, float v_scale, int32_t partition_size,
                                      const int32_t* group_start, const int32_t* prefix_lens,
                                      int32_t num_groups, int32_t max_group_size,
                                      int32_t max_prefix_len, void* workspace,
                                      int64_t workspace_bytes, void* stream);

/* Causal attention of prefill chunks over their paged context (the scheduler on
 * page "vLLM 部署深度指南" puts prefills and decodes into one step). Request r owns
 * query rows [query_start_loc[r], query_start_loc[r+1]) and seq_lens[r] tokens in
 * the pool, its own chunk already appended, so P = seq_lens[r] - chunk length
 * tokens come before the chunk; chunk row i sits at position P + i and sees
 * positions 0 .. P + i.
 *
 *   out              device fp16 [total_q][num_q_heads][head_size], written
 *   q                device fp16 [total_q][num_q_heads][head_size]
 *   block_tables     device int32 [num_reqs][max_blocks_per_seq]
 *   query_start_loc  device int32 [num_reqs + 1], non-decreasing, starts at 0, ends at
 *                    total_q; each chunk at most max_q_len rows
 *   seq_lens         device int32 [num_reqs], chunk length <= seq_lens[r] <= max_seq_len
 *                    and <= max_blocks_per_seq * block_size; rows of a request that breaks
 *                    these bounds, or whose table holds an entry outside [0, num_blocks),
 *                    are set to NaN
 *   workspace        optional device memory of pa_prefill_workspace_bytes(...) bytes,
 *                    16-byte aligned, owned by the caller, contents not kept between
 *                    calls (calls sharing one workspace must not overlap). NULL: every
 *                    128-row tile of a chunk runs over its whole context in one workgroup.
 *                    Given: the library may cut long contexts into pieces run by separate
 *                    workgroups, their fp32 partial results merged by log-sum-exp in a
 *                    second kernel (the same split-context merge as decode), so that few
 *                    or uneven requests still fill the GPU. Fewer bytes than needed:
 *                    PA_ERR_WORKSPACE.
 *   scale            finite and > 0 (PA_ERR_INVALID otherwise)
 * Arithmetic: fp16 inputs on the matrix cores with fp32 accumulation; fp32 online
 * softmax whose probabilities p are rounded to fp16 (nearest even) for the P.V product,
 * with the row sum l taken over those same fp16 values in fp32; the reference max of a
 * row moves only when a score beats it by more than 2^8 (base-2 units); fp16 output
 * rounded to nearest even. A split context merges fp32 partials by log-sum-exp. */
pa_status pa_prefill_chunk(void* out, const void* q, const void* kv_pool,
                           const int32_t* block_tables, const int32_t* query_start_loc,
                           const int32_t* seq_lens, int32_t num_reqs, int32_t total_q,
                           int32_t max_q_len, int32_t max_seq_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                           void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes that pa_prefill_chunk and pa_prefill_chunk_fp8 take for these sizes
 * on the current device (the split depends on how many workgroups it holds at once):
 * 0 when no split would help (the call then uses no workspace), -1 for bad sizes
 * (num_reqs < 0, num_q_heads <= 0, max_q_len < 0, max_seq_len < max_q_len, head_size
 * not 64 or 128). */
int64_t pa_prefill_workspace_bytes(int32_t num_reqs, int32_t num_q_heads, int32_t max_q_len,
                                   int32_t max_seq_len, int32_t head_size);

/* Copy one sequence's keys and values, in logical order, out of the pool: the
 * block-table indexing of the attention kernels, made visible bit for bit. Logical
 * position t is read from slot block_table_row[t / block_size] * block_size +
 * t % block_size (page "vLLM GitHub 项目 …", section 二, item 1; the block-table
 * figure in section "PagedAttention 原理" of page "vLLM 部署深度指南").
 *
 *   k_out, v_out     device fp16 [len][num_kv_heads][head_size], written
 *   block_table_row  device int32 [ceil(len / block_size)]; an entry outside
 *                    [0, num_blocks) leaves its tokens' rows unwritten */
pa_status pa_gather_kv(void* k_out, void* v_out, const void* kv_pool,
                       const int32_t* block_table_row, int32_t len, int32_t num_kv_heads,
                       int32_t head_size, int32_t block_size, int64_t num_blocks,
                       void* stream);

/* Read `bytes` bytes (a multiple of 16) of device memory once, as a plain HBM
 * read stream, and write one fp32 per workgroup to `sink` (device,
 * at least pa_stream_read_sink_len(bytes) floats) so the reads are not dropped.
 * A measurement aid: its rate is the read bandwidth the box reaches. */
pa_status pa_stream_read(const void* buf, int64_t bytes, float* sink, void* stream);
int64_t pa_stream_read_sink_len(int64_t bytes);

/* ---- block copies ---------------------------------------------------------------------
 * pa_copy_blocks: inside the pool, block pairs[2k+1] = block pairs[2k] for k < num_pairs:
 * the device half of copy-on-write, run before the step's appends when the block manager
 * reports copies (sequences sharing prefix blocks: page "vLLM GitHub 项目 …", section 二,
 * item 4). Whole blocks (block_size token rows of K and V for every head) are copied.
 *   pairs   device-accessible int64 [num_pairs][2] (source, destination); a pair naming a
 *           block outside [0, num_blocks) is skipped. Destinations must be distinct and
 *           must not be sources of other pairs of the same call (the pairs run
 *           concurrently), as holds for the copies of one step of the block manager.
 * pa_move_blocks: dst block d = src block s for each (s, d) pair, blocks of block_bytes
 * bytes (a multiple of 16) in two buffers of dst_blocks and src_blocks blocks: swapping
 * blocks out of the pool into a CPU swap area and back (--swap-space in the flag table of
 * page "vLLM 部署深度指南"). dst, src and pairs may each be device memory or pinned host
 * memory (hipHostMalloc; the kernel reads and writes it over the host link); any other
 * host memory is refused with PA_ERR_INVALID before a launch. Same rules on pairs.
 * pa_copy_blocks_fp8: pa_copy_blocks over an E4M3 pool (one byte per element, the
 * layout of the FP8 section above): copy-on-write for a --kv-cache-dtype fp8 cache.
 * Both are asynchronous on `stream`. */
pa_status pa_copy_blocks(void* kv_pool, const int64_t* pairs, int32_t num_pairs,
                         int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                         int64_t num_blocks, void* stream);
pa_status pa_copy_blocks_fp8(void* kv_pool, const int64_t* pairs, int32_t num_pairs,
                             int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                             int64_t num_blocks, void* stream);
pa_status pa_move_blocks(void* dst, const void* src, const int64_t* pairs, int32_t num_pairs,
                         int64_t block_bytes, int64_t dst_blocks, int64_t src_blocks,
                         void* stream);

/* ---- captured steps (HIP graphs) ----------------------------------------------------
 * A step (append, prefill, decode, reduce) is a few launches whose host-side cost rules
 * small batches; serving engines replay such a step from a captured graph (page "vLLM
 * 部署深度指南", GPTQ deployment listing and flag table: enforce_eager / --enforce-eager
 * switch the CUDA-graph path off). These calls capture whatever this library (or
 * anything else) enqueues on a stream between pa_graph_begin and pa_graph_end and
 * replay it with one launch.
 *
 *   pa_graph_begin  starts capturing `stream` (must not be the null stream; relaxed
 *                   mode). Every call enqueued on it until pa_graph_end is recorded, not
 *                   run. The device buffers and host scalars of those calls are fixed in
 *                   the graph: a replay reads the same buffers, so the caller updates
 *                   inputs in place and keeps every buffer (workspaces included) alive
 *                   until pa_graph_destroy.
 *   pa_graph_end    ends the capture and instantiates it; *graph receives a host handle
 *                   owned by the caller (NULL on error; the capture is ended either way).
 *   pa_graph_launch replays the whole capture on `stream` (stream-ordered, asynchronous).
 *   pa_graph_destroy releases the handle (NULL is ignored).
 * Capturing records no memset nodes: the library's kernels clear nothing through
 * hipMemset. */
typedef struct pa_graph pa_graph;
pa_status pa_graph_begin(void* stream);
pa_status pa_graph_end(void* stream, pa_graph** graph);
pa_status pa_graph_launch(const pa_graph* graph, void* stream);
void pa_graph_destroy(pa_graph* graph);

/* ---- host block manager --------------------------------------------------------------
 * Which pool blocks each sequence holds (page "vLLM 部署深度指南", section
 * "PagedAttention 原理", KV-cache listing: a free list that starts as 0 .. num_blocks-1
 * and is taken from the front, ceil(n / block_size) blocks per sequence, an error when it
 * runs dry; page "vLLM GitHub 项目 …", section 二: item 1, a new block only when the last
 * one is full; item 4, sequences that share a prefix point at the same blocks). Host
 * code only: no device memory, no stream. The manager owns its bookkeeping; every output
 * array belongs to the caller. Sequence ids are any int64 values; block ids are int32.
 *
 *   pa_bm_create       manager of num_blocks blocks of block_size tokens
 *   pa_bm_allocate     new sequence holding num_tokens tokens: ceil(num_tokens /
 *                      block_size) blocks from the front of the free list, all or none
 *                      (PA_ERR_EXHAUSTED, nothing taken); PA_ERR_INVALID if seq_id exists
 *   pa_bm_append_slot  reserve the slot (block * block_size + offset) of the sequence's
 *                      next token. A full last block gets a new block; a last block that
 *                      another sequence also references and that is partly filled is
 *                      replaced by a new block, and (*copy_src, *copy_dst) name the block
 *                      copy that must run on the device before the token is written
 *                      (copy-on-write; both -1 when no copy). PA_ERR_EXHAUSTED with no
 *                      change when a block is needed and none is free
 *   pa_bm_append_slots one token for each of seq_ids[0..n) in order, as above:
 *                      slot_mapping[n] receives the slots, copies[2 * k], copies[2 * k + 1]
 *                      the k-th copy pair (room for n pairs), *num_copies their count,
 *                      *num_done the tokens appended; it stops at the first failure, whose
 *                      slot and the following ones are -1
 *   pa_bm_fork         child shares every block of parent (same length)
 *   pa_bm_free         drop the sequence; each of its blocks loses a reference, in table
 *                      order, and goes to the back of the free list when none is left
 *   pa_bm_block_tables padded rows tables[n][max_blocks] (pad after the sequence's
 *                      blocks) and lengths lens[n] of the listed sequences, ready for
 *                      pa_decode / pa_prefill_chunk
 *   queries            pa_bm_seq_len (-1: unknown), pa_bm_seq_table (writes up to cap
 *                      entries, returns the count or -1), pa_bm_num_free, pa_bm_free_list
 *                      (free list in order; returns its length), pa_bm_refcount,
 *                      pa_bm_usage (fraction of blocks in use: the gpu_cache_usage_perc
 *                      gauge of the monitoring table on the deployment page),
 *                      pa_bm_slot_utilisation (fraction of slots in used blocks holding a
 *                      token)
 * Not thread-safe: one manager per thread, or the caller serialises. */
typedef struct pa_block_manager pa_block_manager;
pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);
pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, int64_t num_tokens);
pa_status pa_bm_append_slot(pa_block_manager* bm, int64_t seq_id, int64_t* slot,
                            int64_t* copy_src, int64_t* copy_dst);
pa_status pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                             int64_t* slot_mapping, int64_t* copies, int32_t* num_copies,
                             int32_t* num_done);
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);
pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id);
pa_status pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                             int32_t max_blocks, int32_t pad, int32_t* tables, int32_t* lens);
int64_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id);
int64_t pa_bm_seq_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out, int64_t cap);
int64_t pa_bm_num_free(const pa_block_manager* bm);
int64_t pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int64_t cap);
int32_t pa_bm_refcount(const pa_block_manager* bm, int64_t block);
double pa_bm_usage(const pa_block_manager* bm);
double pa_bm_slot_utilisation(const pa_block_manager* bm);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
