// pa_gather_kv: copy one sequence's K and V rows out of the pool in logical order, through
// its block-table row (logical position t lives at slot table[t / 16] * 16 + t % 16).
// It exposes the attention kernels' block-table addressing bit for bit.
//
// stream_read: a read-only pass over a buffer, the HBM read rate the box reaches.
#include "pa_device.h"
#include "pa_launch.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gather_kv_kernel(
    half_t* __restrict__ k_out, half_t* __restrict__ v_out, const half_t* __restrict__ pool,
    const int32_t* __restrict__ table_row, int kv_row_elems, int64_t num_blocks) {
  const int t = blockIdx.x;
  const int phys = table_row[t / kBlockSize];
  if (phys < 0 || phys >= num_blocks) return;
  const int64_t slot = (int64_t)phys * kBlockSize + t % kBlockSize;
  const int pieces = kv_row_elems / 8;
  const int c = blockIdx.y * kThreads + threadIdx.x;
  if (c >= 2 * pieces) return;
  const int kv = c >= pieces;
  const int e = (kv ? c - pieces : c) * 8;
  const half8_t v = *reinterpret_cast<const half8_t*>(pool + row_offset(slot, kv, kv_row_elems) + e);
  half_t* dst = (kv ? v_out : k_out) + (int64_t)t * kv_row_elems + e;
  *reinterpret_cast<half8_t*>(dst) = v;
}

constexpr int kReadUnroll = 4;
constexpr int64_t kReadChunk = 16384;  // 16-byte pieces per workgroup (256 KiB)

// Each workgroup streams one contiguous 256 KiB chunk with non-temporal 16-byte loads,
// the fastest read shape measured on MI355X.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const half8_t* __restrict__ buf,
                                                               int64_t n16, float* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kReadChunk;
  const int64_t end = base + kReadChunk < n16 ? base + kReadChunk : n16;
  uint32_t acc = 0;
  int64_t i = base + threadIdx.x;
  for (; i + (kReadUnroll - 1) * kThreads < end; i += kReadUnroll * kThreads) {
    half8_t v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const uint4 w = __builtin_bit_cast(uint4, v[u]);
      acc ^= w.x ^ w.y ^ w.z ^ w.w;
    }
  }
  for (; i < end; i += kThreads) {
    const uint4 w = __builtin_bit_cast(uint4, buf[i]);
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  // fold the wave, then one lane per wave writes; a non-zero xor is what the caller sees
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  __shared__ uint32_t part[kThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kThreads / kWave; ++w) r ^= part[w];
    sink[blockIdx.x] = __builtin_bit_cast(float, r & 0x007FFFFFu);  // a finite float
  }
}

}  // namespace

hipError_t launch_gather_kv(void* k_out, void* v_out, const void* pool, const int32_t* table_row,
                            int len, int kv_row_elems, int64_t num_blocks, hipStream_t stream) {
  if (len == 0) return hipSuccess;
  const int pieces2 = 2 * (kv_row_elems / 8);
  dim3 grid(len, (pieces2 + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(gather_kv_kernel, grid, dim3(kThreads), 0, stream,
                     static_cast<half_t*>(k_out), static_cast<half_t*>(v_out),
                     static_cast<const half_t*>(pool), table_row, kv_row_elems, num_blocks);
  return hipGetLastError();
}

int64_t stream_read_groups(int64_t bytes) {
  const int64_t n16 = bytes / 16;
  const int64_t g = (n16 + kReadChunk - 1) / kReadChunk;
  return g < 1 ? 1 : g;
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, float* sink, hipStream_t stream) {
  const int64_t groups = stream_read_groups(bytes);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)groups), dim3(kThreads), 0, stream,
                     static_cast<const half8_t*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
