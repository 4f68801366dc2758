// kv_append: scatter this step's new tokens' K and V rows into their pool slots.
//
// Token t's key row (num_kv_heads * head_size fp16, contiguous) is copied to
// pool[slot][0] and its value row to pool[slot][1], where slot = slot_mapping[t]
// (page "vLLM 部署深度指南", append_kv of the KV-cache listing: new K/V go into the
// sequence's physical block). A pure copy of bits: 16-byte loads and stores, one
// thread per 16-byte piece. Bound by HBM bandwidth (read + write of 2 rows per token).
#include "pa_device.h"
#include "pa_launch.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    half_t* __restrict__ pool, const half_t* __restrict__ key, const half_t* __restrict__ value,
    const int64_t* __restrict__ slot_mapping, int kv_row_elems, int64_t num_slots,
    int64_t key_stride, int64_t value_stride) {
  const int t = blockIdx.x;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding token or a slot outside the pool
  const int pieces = kv_row_elems / 8;         // 16-byte pieces per key (or value) row
  const int c = blockIdx.y * kThreads + threadIdx.x;
  if (c >= 2 * pieces) return;
  const int kv = c >= pieces;
  const int e = (kv ? c - pieces : c) * 8;
  const half_t* src = kv ? value + t * value_stride : key + t * key_stride;
  const half8_t v = *reinterpret_cast<const half8_t*>(src + e);
  *reinterpret_cast<half8_t*>(pool + row_offset(slot, kv, kv_row_elems) + e) = v;
}

// FP8 cache: the same scatter, each 8-element piece scaled by the reciprocal of its
// tensor's scale (fp32), saturated to +-448 and rounded to E4M3 codes (8 bytes out).
__global__ __launch_bounds__(kThreads) void kv_append_fp8_kernel(
    fp8_t* __restrict__ pool, const half_t* __restrict__ key, const half_t* __restrict__ value,
    const int64_t* __restrict__ slot_mapping, int kv_row_elems, int64_t num_slots,
    int64_t key_stride, int64_t value_stride, float k_inv, float v_inv) {
  const int t = blockIdx.x;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int pieces = kv_row_elems / 8;
  const int c = blockIdx.y * kThreads + threadIdx.x;
  if (c >= 2 * pieces) return;
  const int kv = c >= pieces;
  const int e = (kv ? c - pieces : c) * 8;
  const half_t* src = kv ? value + t * value_stride : key + t * key_stride;
  const float inv = kv ? v_inv : k_inv;
  const half8_t v = *reinterpret_cast<const half8_t*>(src + e);
  unsigned int w[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    w[k] = fp8x2((float)v[4 * k] * inv, (float)v[4 * k + 1] * inv) |
           (fp8x2((float)v[4 * k + 2] * inv, (float)v[4 * k + 3] * inv) << 16);
  *reinterpret_cast<u32x2_t*>(pool + row_offset(slot, kv, kv_row_elems) + e) = u32x2_t{w[0], w[1]};
}

}  // namespace

hipError_t launch_kv_append_fp8(void* pool, const void* key, const void* value,
                                const int64_t* slots, int num_tokens, int kv_row_elems,
                                int64_t num_slots, int64_t key_stride, int64_t value_stride,
                                float k_inv, float v_inv, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int pieces2 = 2 * (kv_row_elems / 8);
  dim3 grid(num_tokens, (pieces2 + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(kv_append_fp8_kernel, grid, dim3(kThreads), 0, stream,
                     static_cast<fp8_t*>(pool), static_cast<const half_t*>(key),
                     static_cast<const half_t*>(value), slots, kv_row_elems, num_slots,
                     key_stride, value_stride, k_inv, v_inv);
  return hipGetLastError();
}

hipError_t launch_kv_append(void* pool, const void* key, const void* value, const int64_t* slots,
                            int num_tokens, int kv_row_elems, int64_t num_slots,
                            int64_t key_stride, int64_t value_stride, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int pieces2 = 2 * (kv_row_elems / 8);
  dim3 grid(num_tokens, (pieces2 + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(kThreads), 0, stream,
                     static_cast<half_t*>(pool), static_cast<const half_t*>(key),
                     static_cast<const half_t*>(value), slots, kv_row_elems, num_slots,
                     key_stride, value_stride);
  return hipGetLastError();
}

}  // namespace pkv
