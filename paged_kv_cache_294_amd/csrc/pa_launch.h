// Launchers of the device kernels. Internal to the library: the C ABI in pagedkv.h checks
// every argument before calling these, so they only size grids and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_kv_append(void* pool, const void* key, const void* value, const int64_t* slots,
                            int num_tokens, int kv_row_elems, int64_t num_slots,
                            int64_t key_stride, int64_t value_stride, hipStream_t stream);
hipError_t launch_kv_append_fp8(void* pool, const void* key, const void* value,
                                const int64_t* slots, int num_tokens, int kv_row_elems,
                                int64_t num_slots, int64_t key_stride, int64_t value_stride,
                                float k_inv, float v_inv, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_o;   // [B][Hq][P][D] fp32, or null when P == 1
  float* ws_ml;  // [B][Hq][P][2] fp32 (max in log2 units, sum), or null when P == 1
  int* ws_items;  // plain decode with P > 1: (sequence, partition) items, largest first
  int num_seqs, num_q_heads, num_kv_heads, head_size;
  int max_blocks_per_seq;
  int64_t num_blocks;
  int max_context_len;
  int partition_blocks;  // partition size in blocks
  int num_partitions;    // partitions the grid covers
  int ws_parts;          // partition slots per (sequence, query head) in the workspace
  // Shared-prefix decode: sequences group_start[g] .. group_start[g + 1] - 1 share their
  // first prefix_lens[g] tokens (whole blocks, same table entries). Null: plain decode.
  const int32_t* group_start;
  const int32_t* prefix_lens;
  int num_groups;
  int group_chunks;      // prefix pass: chunks of samples per group
  int group_cap;         // samples per group the prefix pass covers (chunks * samples per tile)
  int prefix_parts;      // workspace slots 0 .. prefix_parts - 1 hold prefix partitions
  int prefix_grid;       // workgroups of the prefix pass (they come first in the launch)
  float scale_log2;      // softmax scale * log2(e), times the key scale of an FP8 cache
  float v_scale;         // value scale of an FP8 cache (1 for fp16)
  bool stream_kv;        // K/V loads carry the non-temporal hint (blocks read once per step)
  bool kv_fp8;           // the pool holds E4M3 codes (1 byte per element) instead of fp16
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_shared_prefix(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const void* pool;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  const int32_t* seq_lens;
  int num_reqs, total_q, max_q_len, max_seq_len;
  int num_q_heads, num_kv_heads, head_size;
  int max_blocks_per_seq;
  int64_t num_blocks;
  float scale_log2;  // softmax scale * log2(e), times the key scale of an FP8 cache
  float v_scale;     // value scale of an FP8 cache (1 for fp16)
  bool kv_fp8;       // the pool holds E4M3 codes (1 byte per element)
  // Context split: a request's context may be cut into up to max_pieces pieces of whole
  // stages, each piece of a row tile run by its own workgroup; split tiles leave fp32
  // partials (o, then (m, l)) in the workspace for the merge kernel. max_pieces == 1: no
  // split, no workspace.
  int max_pieces;
  int slots;         // prefill workgroups the device holds at once
  float* ws_o;       // [num_reqs][Hq][tiles][max_pieces][128 * D]
  float* ws_ml;      // [num_reqs][Hq][tiles][max_pieces][256][2]
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Pieces per request a launch may use (1: no split), the workspace it then needs, and the
// prefill workgroups the current device holds at once (fp16 and FP8 caches alike use the
// fp16 kernel's occupancy, so both take the same workspace).
int prefill_max_pieces(int num_reqs, int num_q_heads, int max_q_len, int max_seq_len,
                       int head_size);
int64_t prefill_workspace_bytes(int num_reqs, int num_q_heads, int max_q_len, int head_size,
                                int max_pieces);
int prefill_slots(int head_size);

hipError_t launch_gather_kv(void* k_out, void* v_out, const void* pool, const int32_t* table_row,
                            int len, int kv_row_elems, int64_t num_blocks, hipStream_t stream);

int64_t stream_read_groups(int64_t bytes);
hipError_t launch_stream_read(const void* buf, int64_t bytes, float* sink, hipStream_t stream);

hipError_t launch_move_blocks(void* dst, const void* src, const int64_t* pairs, int num_pairs,
                              int64_t block_bytes, int64_t dst_blocks, int64_t src_blocks,
                              hipStream_t stream);

}  // namespace pkv
