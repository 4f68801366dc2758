// C ABI of the paged KV-cache attention library: host-side argument checks, grid and
// workspace sizing, launches. Every declaration is in include/pagedkv.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/pagedkv.h"
#include "pa_launch.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kBlock = 16;
constexpr double kLog2e = 1.4426950408889634;

thread_local char g_last_error[256] = "";

pa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e),
                hipGetErrorString(e));
  return PA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by the device operations: the pool geometry this library has kernels for.
pa_status check_geometry(int32_t block_size, int32_t num_kv_heads, int32_t head_size) {
  if (block_size <= 0 || num_kv_heads <= 0 || head_size <= 0) return PA_ERR_INVALID;
  if (block_size != kBlock) return PA_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

pa_status check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return PA_ERR_INVALID;
  const int g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

}  // namespace

PA_EXPORT const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_EXHAUSTED: return "KV cache exhausted";
    default: return "unknown status";
  }
}

PA_EXPORT const char* pa_last_error(void) { return g_last_error; }

PA_EXPORT int32_t pa_abi_version(void) { return 1; }

// ---------------------------------------------------------------------------------------
// layout helpers
// ---------------------------------------------------------------------------------------

PA_EXPORT int64_t pa_blocks_for_len(int64_t len, int32_t block_size) {
  if (len < 0 || block_size <= 0) return -1;
  return (len + block_size - 1) / block_size;
}

PA_EXPORT int64_t pa_block_bytes(int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                                 int32_t elem_bytes) {
  if (block_size <= 0 || num_kv_heads <= 0 || head_size <= 0 || elem_bytes <= 0) return -1;
  return (int64_t)block_size * 2 * num_kv_heads * head_size * elem_bytes;
}

PA_EXPORT int64_t pa_pool_bytes(int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                int32_t head_size, int32_t elem_bytes) {
  const int64_t bb = pa_block_bytes(block_size, num_kv_heads, head_size, elem_bytes);
  if (bb < 0 || num_blocks < 0) return -1;
  if (num_blocks > INT64_MAX / bb) return -1;
  return num_blocks * bb;
}

PA_EXPORT int64_t pa_num_blocks_fit(int64_t free_bytes, double utilization, int32_t block_size,
                                    int32_t num_kv_heads, int32_t head_size, int32_t elem_bytes) {
  const int64_t bb = pa_block_bytes(block_size, num_kv_heads, head_size, elem_bytes);
  if (bb < 0 || free_bytes < 0 || !(utilization > 0.0 && utilization <= 1.0)) return -1;
  const double usable = std::floor((double)free_bytes * utilization);
  return (int64_t)(usable / (double)bb);
}

PA_EXPORT int64_t pa_slot(const int32_t* block_table_row, int64_t pos, int32_t block_size) {
  if (!block_table_row || pos < 0 || block_size <= 0) return -1;
  const int32_t phys = block_table_row[pos / block_size];
  if (phys < 0) return -1;
  return (int64_t)phys * block_size + pos % block_size;
}

PA_EXPORT int64_t pa_kv_elem_offset(int64_t slot, int32_t kv, int32_t head, int32_t dim,
                                    int32_t num_kv_heads, int32_t head_size) {
  if (slot < 0 || (kv != 0 && kv != 1) || head < 0 || head >= num_kv_heads || dim < 0 ||
      dim >= head_size)
    return -1;
  return ((slot * 2 + kv) * num_kv_heads + head) * (int64_t)head_size + dim;
}

PA_EXPORT int32_t pa_num_partitions(int32_t max_context_len, int32_t partition_size) {
  if (max_context_len < 0 || partition_size <= 0) return -1;
  const int32_t p = (int32_t)(((int64_t)max_context_len + partition_size - 1) / partition_size);
  return p < 1 ? 1 : p;
}

PA_EXPORT int32_t pa_decode_default_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t max_context_len) {
  if (num_seqs < 0 || max_context_len < 0 || num_kv_heads <= 0 || num_q_heads <= 0 ||
      num_q_heads % num_kv_heads)
    return -1;
  const int64_t target_waves = num_q_heads == num_kv_heads ? 4096 : 2048;
  const int64_t waves_per_part = std::max<int64_t>(1, (int64_t)num_seqs * num_kv_heads);
  const int64_t parts = (target_waves + waves_per_part - 1) / waves_per_part;
  int64_t ps = ((int64_t)max_context_len + parts - 1) / parts;
  ps = std::max<int64_t>(kBlock, (ps + kBlock - 1) / kBlock * kBlock);
  if (parts > 16) ps = std::max<int64_t>(ps, 512);
  return (int32_t)std::min<int64_t>(ps, INT32_MAX / kBlock * kBlock);
}

PA_EXPORT int64_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t max_context_len, int32_t partition_size,
                                            int32_t head_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_size <= 0) return -1;
  const int32_t p = pa_num_partitions(max_context_len, partition_size);
  if (p < 0) return -1;
  if (p == 1) return (4 * (1 + (int64_t)num_seqs) + 255) / 256 * 256;  // item list only
  const int64_t rows = (int64_t)num_seqs * num_q_heads * p;
  int64_t bytes = rows * head_size * 4;  // o
  bytes = (bytes + 255) / 256 * 256;
  bytes += rows * 2 * 4;                 // (m, l)
  bytes = (bytes + 255) / 256 * 256;
  bytes += 4 * (1 + (int64_t)num_seqs * p);  // item list of the largest-first order
  return (bytes + 255) / 256 * 256;
}

PA_EXPORT int64_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                          int32_t max_context_len,
                                                          int32_t max_prefix_len,
                                                          int32_t partition_size,
                                                          int32_t head_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || max_prefix_len < 0 ||
      max_prefix_len > max_context_len || partition_size <= 0 || head_size <= 0)
    return -1;
  const int64_t parts = (int64_t)pa_num_partitions(max_context_len, partition_size) +
                        (max_prefix_len == 0 ? 0 : pa_num_partitions(max_prefix_len, partition_size));
  const int64_t rows = (int64_t)num_seqs * num_q_heads * parts;
  const int64_t o_bytes = (rows * head_size * 4 + 255) / 256 * 256;
  return (o_bytes + rows * 8 + 255) / 256 * 256;
}

PA_EXPORT int64_t pa_prefill_workspace_bytes(int32_t num_reqs, int32_t num_q_heads,
                                             int32_t max_q_len, int32_t max_seq_len,
                                             int32_t head_size) {
  if (num_reqs < 0 || num_q_heads <= 0 || max_q_len < 0 || max_seq_len < max_q_len ||
      (head_size != 64 && head_size != 128))
    return -1;
  const int pieces = pkv::prefill_max_pieces(num_reqs, num_q_heads, max_q_len, max_seq_len, head_size);
  return pkv::prefill_workspace_bytes(num_reqs, num_q_heads, max_q_len, head_size, pieces);
}

// ---------------------------------------------------------------------------------------
// device operations
// ---------------------------------------------------------------------------------------

namespace {

pa_status kv_append_impl(void* kv_pool, const void* key, const void* value,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size, int64_t num_blocks,
                         int64_t key_token_stride, int64_t value_token_stride, bool fp8,
                         float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0) return PA_ERR_INVALID;
  if (pa_status s = check_geometry(block_size, num_kv_heads, head_size)) return s;
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
    return PA_ERR_INVALID;
  if (num_tokens == 0) return PA_OK;
  if (!kv_pool || !key || !value || !slot_mapping) return PA_ERR_INVALID;
  const int64_t row = (int64_t)num_kv_heads * head_size;
  if (key_token_stride == 0) key_token_stride = row;
  if (value_token_stride == 0) value_token_stride = row;
  if (key_token_stride < row || value_token_stride < row) return PA_ERR_INVALID;
  if (key_token_stride % 8 || value_token_stride % 8) return PA_ERR_INVALID;  // 16-byte rows
  if (!aligned16(kv_pool) || !aligned16(key) || !aligned16(value)) return PA_ERR_INVALID;
  if (row > INT32_MAX / 2) return PA_ERR_INVALID;
  if (fp8)
    return hip_status(pkv::launch_kv_append_fp8(
        kv_pool, key, value, slot_mapping, num_tokens, (int)row, num_blocks * block_size,
        key_token_stride, value_token_stride, 1.0f / k_scale, 1.0f / v_scale, (hipStream_t)stream));
  return hip_status(pkv::launch_kv_append(kv_pool, key, value, slot_mapping, num_tokens, (int)row,
                                          num_blocks * block_size, key_token_stride,
                                          value_token_stride, (hipStream_t)stream));
}

}  // namespace

PA_EXPORT pa_status pa_kv_append(void* kv_pool, const void* key, const void* value,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                 int64_t num_blocks, int64_t key_token_stride,
                                 int64_t value_token_stride, void* stream) {
  return kv_append_impl(kv_pool, key, value, slot_mapping, num_tokens, num_kv_heads, head_size,
                        block_size, num_blocks, key_token_stride, value_token_stride, false, 1.0f,
                        1.0f, stream);
}

PA_EXPORT pa_status pa_kv_append_fp8(void* kv_pool, const void* key, const void* value,
                                     const int64_t* slot_mapping, int32_t num_tokens,
                                     int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                     int64_t num_blocks, int64_t key_token_stride,
                                     int64_t value_token_stride, float k_scale, float v_scale,
                                     void* stream) {
  return kv_append_impl(kv_pool, key, value, slot_mapping, num_tokens, num_kv_heads, head_size,
                        block_size, num_blocks, key_token_stride, value_token_stride, true,
                        k_scale, v_scale, stream);
}

namespace {

pa_status decode_impl(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                      int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                      float scale, int32_t partition_size, void* workspace,
                      int64_t workspace_bytes, uint32_t flags, bool fp8, float k_scale,
                      float v_scale, void* stream, const int32_t* group_start = nullptr,
                      const int32_t* prefix_lens = nullptr, int32_t num_groups = 0,
                      int32_t max_group_size = 0, int32_t max_prefix_len = 0) {
  const bool cascade = group_start != nullptr;
  if (cascade && (prefix_lens == nullptr || num_groups <= 0 || max_group_size <= 0 ||
                  max_prefix_len < 0 || max_prefix_len % 16 || max_prefix_len > max_context_len))
    return PA_ERR_INVALID;
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
    return PA_ERR_INVALID;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0)
    return PA_ERR_INVALID;
  if (pa_status s = check_geometry(block_size, num_kv_heads, head_size)) return s;
  if (pa_status s = check_heads(num_q_heads, num_kv_heads)) return s;
  if (partition_size <= 0 || partition_size % block_size) return PA_ERR_INVALID;
  // the matrix-core kernels mask scores with -inf and track the running max in scaled
  // units, which holds only for a positive scale
  if (!std::isfinite(scale) || !(scale > 0.0f)) return PA_ERR_INVALID;
  if (flags & ~PA_DECODE_KV_STREAM) return PA_ERR_INVALID;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_INVALID;
  // the kernels address up to 16 tokens * 2 * Hkv * D elements inside a block as int32
  if ((int64_t)block_size * 2 * num_kv_heads * head_size > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !kv_pool || !block_tables || !context_lens) return PA_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(kv_pool)) return PA_ERR_INVALID;

  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.pool = kv_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.partition_blocks = partition_size / block_size;
  a.num_partitions = pa_num_partitions(max_context_len, partition_size);
  if (a.num_partitions > 65535) return PA_ERR_UNSUPPORTED;
  a.ws_parts = a.num_partitions;
  if (cascade) {
    a.group_start = group_start;
    a.prefix_lens = prefix_lens;
    a.num_groups = num_groups;
    a.group_cap = max_group_size;
    a.prefix_parts = pa_num_partitions(max_prefix_len, partition_size);
    if (max_prefix_len == 0) a.prefix_parts = 0;
    a.ws_parts = a.prefix_parts + a.num_partitions;
  }
  a.scale_log2 = (float)((double)scale * kLog2e * (double)k_scale);
  a.v_scale = v_scale;
  a.kv_fp8 = fp8;
  a.stream_kv = (flags & PA_DECODE_KV_STREAM) != 0;
  if (a.num_partitions > 1 || cascade) {
    const int64_t need =
        cascade ? pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, max_context_len,
                                                          max_prefix_len, partition_size, head_size)
                : pa_decode_workspace_bytes(num_seqs, num_q_heads, max_context_len,
                                            partition_size, head_size);
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_INVALID;
    const int64_t rows = (int64_t)num_seqs * num_q_heads * a.ws_parts;
    const int64_t o_bytes = (rows * head_size * 4 + 255) / 256 * 256;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
    if (!cascade) {  // tail of the plain layout: the item list of the largest-first order
      const int64_t ml_bytes = (rows * 2 * 4 + 255) / 256 * 256;
      a.ws_items = reinterpret_cast<int*>(static_cast<char*>(workspace) + o_bytes + ml_bytes);
    }
  } else if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0 &&
             workspace_bytes >= pa_decode_workspace_bytes(num_seqs, num_q_heads, max_context_len,
                                                          partition_size, head_size)) {
    // one partition: the workspace is optional and only holds the item list; without it the
    // sequences run in launch order
    a.ws_items = static_cast<int*>(workspace);
  }
  if (cascade) return hip_status(pkv::launch_decode_shared_prefix(a, (hipStream_t)stream));
  return hip_status(pkv::launch_decode(a, (hipStream_t)stream));
}

}  // namespace

PA_EXPORT pa_status pa_decode(void* out, const void* q, const void* kv_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int32_t max_context_len, float scale,
                              int32_t partition_size, void* workspace, int64_t workspace_bytes,
                              uint32_t flags, void* stream) {
  return decode_impl(out, q, kv_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_size, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, flags,
                     false, 1.0f, 1.0f, stream);
}

PA_EXPORT pa_status pa_decode_shared_prefix(
    void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, const int32_t* group_start,
    const int32_t* prefix_lens, int32_t num_groups, int32_t max_group_size,
    int32_t max_prefix_len, void* workspace, int64_t workspace_bytes, void* stream) {
  if (group_start == nullptr && num_seqs > 0) return PA_ERR_INVALID;
  return decode_impl(out, q, kv_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_size, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, 0u,
                     false, 1.0f, 1.0f, stream, group_start, prefix_lens, num_groups,
                     max_group_size, max_prefix_len);
}

PA_EXPORT pa_status pa_decode_shared_prefix_fp8(
    void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
    int32_t max_context_len, float scale, float k_scale, float v_scale, int32_t partition_size,
    const int32_t* group_start, const int32_t* prefix_lens, int32_t num_groups,
    int32_t max_group_size, int32_t max_prefix_len, void* workspace, int64_t workspace_bytes,
    void* stream) {
  if (group_start == nullptr && num_seqs > 0) return PA_ERR_INVALID;
  return decode_impl(out, q, kv_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_size, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, 0u,
                     true, k_scale, v_scale, stream, group_start, prefix_lens, num_groups,
                     max_group_size, max_prefix_len);
}

PA_EXPORT pa_status pa_decode_fp8(void* out, const void* q, const void* kv_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_size, int32_t block_size,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  int32_t max_context_len, float scale, float k_scale,
                                  float v_scale, int32_t partition_size, void* workspace,
                                  int64_t workspace_bytes, uint32_t flags, void* stream) {
  return decode_impl(out, q, kv_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_size, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, flags,
                     true, k_scale, v_scale, stream);
}

// ---------------------------------------------------------------------------------------
// decode with the library's own scratch (no allocation, no caller workspace)
// ---------------------------------------------------------------------------------------

namespace {

// Scratch of pa_decode_noalloc: the decode workspace (partial results and the work order)
// in a fixed device array, one copy per GPU, held until the process ends. On the host the
// name is only a stand-in for the symbol, never a device address: host code uses the
// address the runtime reports for the current device (scratch_of_current_device).
__device__ __align__(256) unsigned char scratch[PA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
pa_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (ptr == nullptr) {
      std::snprintf(g_last_error, sizeof(g_last_error), "no device address for the scratch array");
      return PA_ERR_HIP;
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

PA_EXPORT pa_status pa_decode_noalloc(void* out, const void* q, const void* kv_pool,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_size,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int32_t max_context_len, float scale,
                                      int32_t partition_size, uint32_t flags, void* stream) {
  // sizes first: a call that needs more scratch than the array holds is refused before
  // any device access
  const int64_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, max_context_len,
                                                 partition_size, head_size);
  if (need < 0) return PA_ERR_INVALID;
  if (need > (int64_t)PA_DECODE_NOALLOC_SCRATCH_BYTES) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "pa_decode_noalloc needs %lld bytes of scratch, more than its %lld",
                  (long long)need, (long long)PA_DECODE_NOALLOC_SCRATCH_BYTES);
    return PA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (num_seqs > 0) {
    if (pa_status st = scratch_of_current_device(&ws)) return st;
  }
  // nothing in the scratch has to start at zero: the work-order pre-pass writes its count
  // and list before the partition kernel reads them, and every partial result is written
  // before the reduce reads it
  return decode_impl(out, q, kv_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_size, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, partition_size, ws,
                     (int64_t)PA_DECODE_NOALLOC_SCRATCH_BYTES, flags, false, 1.0f, 1.0f, stream);
}

namespace {

pa_status prefill_impl(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                       const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_reqs,
                       int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                       int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                       float scale, bool fp8, float k_scale, float v_scale, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
    return PA_ERR_INVALID;
  if (num_reqs < 0 || total_q < 0 || max_q_len < 0 || max_seq_len < 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID;
  if (pa_status s = check_geometry(block_size, num_kv_heads, head_size)) return s;
  if (pa_status s = check_heads(num_q_heads, num_kv_heads)) return s;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return PA_ERR_INVALID;
  if (max_q_len > max_seq_len) return PA_ERR_INVALID;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_INVALID;
  if ((int64_t)block_size * 2 * num_kv_heads * head_size > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (num_reqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !kv_pool || !block_tables || !query_start_loc || !seq_lens)
    return PA_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(kv_pool)) return PA_ERR_INVALID;
  if (workspace_bytes < 0 || (workspace && !aligned16(workspace))) return PA_ERR_INVALID;
  pkv::PrefillArgs a{};
  a.max_pieces = 1;
  if (workspace) {
    const int pieces = pkv::prefill_max_pieces(num_reqs, num_q_heads, max_q_len, max_seq_len, head_size);
    const int64_t need = pkv::prefill_workspace_bytes(num_reqs, num_q_heads, max_q_len, head_size, pieces);
    if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (pieces > 1) {
      a.max_pieces = pieces;
      a.slots = pkv::prefill_slots(head_size);
      a.ws_o = static_cast<float*>(workspace);  // (m, l) after o: placed by the launcher
    }
  }
  a.out = out;
  a.q = q;
  a.pool = kv_pool;
  a.block_tables = block_tables;
  a.query_start_loc = query_start_loc;
  a.seq_lens = seq_lens;
  a.num_reqs = num_reqs;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.max_seq_len = max_seq_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.scale_log2 = (float)((double)scale * kLog2e * (double)k_scale);
  a.v_scale = v_scale;
  a.kv_fp8 = fp8;
  hipError_t e = pkv::launch_prefill(a, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  return hip_status(e);
}

}  // namespace

PA_EXPORT pa_status pa_prefill_chunk(void* out, const void* q, const void* kv_pool,
                                     const int32_t* block_tables, const int32_t* query_start_loc,
                                     const int32_t* seq_lens, int32_t num_reqs, int32_t total_q,
                                     int32_t max_q_len, int32_t max_seq_len, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                     int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                     void* workspace, int64_t workspace_bytes, void* stream) {
  return prefill_impl(out, q, kv_pool, block_tables, query_start_loc, seq_lens, num_reqs, total_q,
                      max_q_len, max_seq_len, num_q_heads, num_kv_heads, head_size, block_size,
                      max_blocks_per_seq, num_blocks, scale, false, 1.0f, 1.0f, workspace,
                      workspace_bytes, stream);
}

PA_EXPORT pa_status pa_prefill_chunk_fp8(void* out, const void* q, const void* kv_pool,
                                         const int32_t* block_tables,
                                         const int32_t* query_start_loc, const int32_t* seq_lens,
                                         int32_t num_reqs, int32_t total_q, int32_t max_q_len,
                                         int32_t max_seq_len, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_size,
                                         int32_t block_size, int32_t max_blocks_per_seq,
                                         int64_t num_blocks, float scale, float k_scale,
                                         float v_scale, void* workspace, int64_t workspace_bytes,
                                         void* stream) {
  return prefill_impl(out, q, kv_pool, block_tables, query_start_loc, seq_lens, num_reqs, total_q,
                      max_q_len, max_seq_len, num_q_heads, num_kv_heads, head_size, block_size,
                      max_blocks_per_seq, num_blocks, scale, true, k_scale, v_scale, workspace,
                      workspace_bytes, stream);
}

PA_EXPORT pa_status pa_gather_kv(void* k_out, void* v_out, const void* kv_pool,
                                 const int32_t* block_table_row, int32_t len,
                                 int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                 int64_t num_blocks, void* stream) {
  if (len < 0 || num_blocks <= 0) return PA_ERR_INVALID;
  if (pa_status s = check_geometry(block_size, num_kv_heads, head_size)) return s;
  if (len == 0) return PA_OK;
  if (!k_out || !v_out || !kv_pool || !block_table_row) return PA_ERR_INVALID;
  if (!aligned16(k_out) || !aligned16(v_out) || !aligned16(kv_pool)) return PA_ERR_INVALID;
  const int64_t row = (int64_t)num_kv_heads * head_size;
  if (row > INT32_MAX / 2) return PA_ERR_INVALID;
  return hip_status(pkv::launch_gather_kv(k_out, v_out, kv_pool, block_table_row, len, (int)row,
                                          num_blocks, (hipStream_t)stream));
}

PA_EXPORT int64_t pa_stream_read_sink_len(int64_t bytes) {
  if (bytes <= 0 || bytes % 16) return -1;
  return pkv::stream_read_groups(bytes);
}

PA_EXPORT pa_status pa_stream_read(const void* buf, int64_t bytes, float* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || !aligned16(buf)) return PA_ERR_INVALID;
  if (pkv::stream_read_groups(bytes) > INT32_MAX) return PA_ERR_UNSUPPORTED;
  return hip_status(pkv::launch_stream_read(buf, bytes, sink, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------
// block copies
// ---------------------------------------------------------------------------------------

namespace {

// The address kernels use for `p`: device memory as is, pinned host memory through its
// device mapping. Anything else (pageable host memory) is refused, since a kernel access
// to it would fault.
pa_status device_view(const void* p, const void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // do not leave the refusal for the next launch check
    return PA_ERR_INVALID;
  }
  if (attr.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || d == nullptr) {
      (void)hipGetLastError();
      return PA_ERR_INVALID;
    }
    *out = d;
    return PA_OK;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged ||
      attr.type == hipMemoryTypeUnified) {
    *out = p;
    return PA_OK;
  }
  return PA_ERR_INVALID;
}

}  // namespace

PA_EXPORT pa_status pa_move_blocks(void* dst, const void* src, const int64_t* pairs,
                                   int32_t num_pairs, int64_t block_bytes, int64_t dst_blocks,
                                   int64_t src_blocks, void* stream) {
  if (num_pairs < 0 || block_bytes <= 0 || block_bytes % 16 != 0 || dst_blocks <= 0 ||
      src_blocks <= 0)
    return PA_ERR_INVALID;
  if (num_pairs == 0) return PA_OK;
  if (!dst || !src || !pairs || !aligned16(dst) || !aligned16(src) ||
      (reinterpret_cast<uintptr_t>(pairs) & 7u))
    return PA_ERR_INVALID;
  const void *d = nullptr, *s = nullptr, *p = nullptr;
  pa_status st;
  if ((st = device_view(dst, &d)) != PA_OK || (st = device_view(src, &s)) != PA_OK ||
      (st = device_view(pairs, &p)) != PA_OK)
    return st;
  return hip_status(pkv::launch_move_blocks(const_cast<void*>(d), s,
                                            static_cast<const int64_t*>(p), num_pairs,
                                            block_bytes, dst_blocks, src_blocks,
                                            static_cast<hipStream_t>(stream)));
}

namespace {

// Copy-on-write copies inside a pool whose elements take elem_bytes bytes (2: fp16,
// 1: E4M3 codes); a block is block_size * 2 * num_kv_heads * head_size elements.
pa_status copy_blocks_impl(void* kv_pool, const int64_t* pairs, int32_t num_pairs,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                           int64_t num_blocks, int64_t elem_bytes, void* stream) {
  pa_status st = check_geometry(block_size, num_kv_heads, head_size);
  if (st != PA_OK) return st;
  if (num_blocks <= 0) return PA_ERR_INVALID;
  const int64_t block_bytes = (int64_t)block_size * 2 * num_kv_heads * head_size * elem_bytes;
  return pa_move_blocks(kv_pool, kv_pool, pairs, num_pairs, block_bytes, num_blocks, num_blocks,
                        stream);
}

}  // namespace

PA_EXPORT pa_status pa_copy_blocks(void* kv_pool, const int64_t* pairs, int32_t num_pairs,
                                   int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                                   int64_t num_blocks, void* stream) {
  return copy_blocks_impl(kv_pool, pairs, num_pairs, block_size, num_kv_heads, head_size,
                          num_blocks, 2, stream);
}

PA_EXPORT pa_status pa_copy_blocks_fp8(void* kv_pool, const int64_t* pairs, int32_t num_pairs,
                                       int32_t block_size, int32_t num_kv_heads,
                                       int32_t head_size, int64_t num_blocks, void* stream) {
  return copy_blocks_impl(kv_pool, pairs, num_pairs, block_size, num_kv_heads, head_size,
                          num_blocks, 1, stream);
}

// ---------------------------------------------------------------------------------------
// captured steps
// ---------------------------------------------------------------------------------------

struct pa_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

PA_EXPORT pa_status pa_graph_begin(void* stream) {
  if (stream == nullptr) return PA_ERR_INVALID;  // the null stream cannot be captured
  return hip_status(hipStreamBeginCapture(static_cast<hipStream_t>(stream),
                                          hipStreamCaptureModeRelaxed));
}

PA_EXPORT pa_status pa_graph_end(void* stream, pa_graph** out) {
  if (out != nullptr) *out = nullptr;
  if (stream == nullptr) return PA_ERR_INVALID;
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(static_cast<hipStream_t>(stream), &graph);
  if (e != hipSuccess) return hip_status(e);
  if (out == nullptr) {
    (void)hipGraphDestroy(graph);  // releasing on an error path: its status adds nothing
    return PA_ERR_INVALID;
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return hip_status(e);
  }
  pa_graph* g = new (std::nothrow) pa_graph{graph, exec};
  if (g == nullptr) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    std::snprintf(g_last_error, sizeof(g_last_error), "out of host memory");
    return PA_ERR_INVALID;
  }
  *out = g;
  return PA_OK;
}

PA_EXPORT pa_status pa_graph_launch(const pa_graph* g, void* stream) {
  if (g == nullptr) return PA_ERR_INVALID;
  return hip_status(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
}

PA_EXPORT void pa_graph_destroy(pa_graph* g) {
  if (g == nullptr) return;
  // a destroy call has no caller to report to: the handle is gone either way
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
}
