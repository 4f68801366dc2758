// Paged-attention decode on gfx950: one query token per sequence attends to the
// sequence's cached tokens, reached block by block through its block-table row
// (page "vLLM GitHub 项目 …", section 二: logical blocks map to physical blocks that
// need not be contiguous; page "vLLM 部署深度指南": 16 tokens per block in a pool
// [num_blocks][16][2][num_kv_heads][head_size]).
//
// Work split. A context is cut into partitions of `partition_blocks` blocks. One wave
// handles one (sequence, KV head, partition) and all Hq/Hkv query heads reading that KV
// head; a workgroup holds four consecutive KV heads of the same (sequence, partition),
// so its loads touch neighbouring 256-byte rows of the same tokens.
//
// Lane layout. A key (or value) row of one head is head_size fp16 = head_size/8
// 16-byte pieces. Lane (r, c) = (lane / (D/8), lane % (D/8)) holds piece c of token r of
// every group of 64/(D/8) consecutive tokens, so one wave-wide 16-byte load reads 4
// (D=128) or 8 (D=64) whole token rows, and a 16-token block is 4 (or 2) such loads for
// K and as many for V. The q.k dot of a token is summed over the D/8 lanes of its row
// with DPP moves inside the row.
//
// Softmax. Each row of lanes keeps its own running max m (log2 units), sum l and fp32
// accumulator over the tokens it sees (online softmax); the rows are merged once at the
// end of the partition. Scores use exp2 with the scale pre-multiplied by log2(e).
//
// Output. A sequence with one partition writes its fp16 row directly. Otherwise every
// partition writes (m, l, o = acc / l) to the workspace and the reduce kernel merges
// them: M = max m_p, w_p = l_p * 2^(m_p - M), out = sum w_p o_p / sum w_p.
#include "pa_device.h"
#include "pa_launch.h"

namespace pkv {
namespace {

constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWavesPerGroup * kWave;

template <int D>
struct Geo {
  static constexpr int kLanesPerToken = D / 8;                          // 16 or 8
  static constexpr int kTokensPerLoad = kWave / kLanesPerToken;         // 4 or 8
  static constexpr int kLoadsPerBlock = kBlockSize / kTokensPerLoad;    // 4 or 2
};

template <int D, int G>
__device__ __forceinline__ void write_const_rows(const DecodeArgs& a, int b, int kvh, int col,
                                                 float value) {
  half_t* out = static_cast<half_t*>(a.out);
  half8_t v;
#pragma unroll
  for (int d = 0; d < 8; ++d) v[d] = (half_t)value;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t h = (int64_t)kvh * G + g;
    *reinterpret_cast<half8_t*>(out + ((int64_t)b * a.num_q_heads + h) * D + col * 8) = v;
  }
}

template <int D, int G, bool Stream>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(const DecodeArgs a) {
  using Gm = Geo<D>;
  constexpr int LPT = Gm::kLanesPerToken;
  constexpr int TPL = Gm::kTokensPerLoad;
  constexpr int LPB = Gm::kLoadsPerBlock;

  const int lane = threadIdx.x & (kWave - 1);
  const int kvh = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const int p = blockIdx.y;
  const int b = blockIdx.z;
  if (kvh >= a.num_kv_heads) return;
  const int row = lane / LPT;
  const int col = lane % LPT;

  const int L = a.context_lens[b];
  const bool bad_len = L < 0 || L > a.max_context_len || L > a.max_blocks_per_seq * kBlockSize;
  if (bad_len || L == 0) {
    if (p == 0 && row == 0) write_const_rows<D, G>(a, b, kvh, col, bad_len ? qnan() : 0.0f);
    return;
  }
  const int part_tokens = a.partition_blocks * kBlockSize;
  const int nparts = (L + part_tokens - 1) / part_tokens;
  if (p >= nparts) return;
  const int blk_begin = p * a.partition_blocks;
  const int blk_end = min(blk_begin + a.partition_blocks, (L + kBlockSize - 1) / kBlockSize);

  const half_t* qp = static_cast<const half_t*>(a.q);
  half8_t qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qv[g] = *reinterpret_cast<const half8_t*>(
        qp + ((int64_t)b * a.num_q_heads + (int64_t)kvh * G + g) * D + col * 8);

  const int kv_row = a.num_kv_heads * D;  // elements of one K (or V) row over all heads
  const int tok_stride = 2 * kv_row;       // elements between consecutive tokens of a block
  const int64_t block_elems = (int64_t)kBlockSize * tok_stride;
  // element offset of this lane's piece of load i inside a block: + i * TPL * tok_stride
  const int lane_off = row * tok_stride + kvh * D + col * 8;
  const half_t* pool = static_cast<const half_t*>(a.pool);
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = neg_inf();
    l[g] = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[g][d] = 0.0f;
  }

  // Block-table entries of the partition, one per lane, fetched 64 at a time.
  int bt_vec = (lane < blk_end - blk_begin) ? bt[blk_begin + lane] : 0;
  bool bad_table = false;

  half8_t kc[LPB], vc[LPB];
  {
    const int phys = __builtin_amdgcn_readfirstlane(bt_vec);
    bad_table = phys < 0 || phys >= a.num_blocks;
    const half_t* base = pool + (bad_table ? 0 : (int64_t)phys * block_elems) + lane_off;
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      kc[i] = load16<Stream>(base + i * TPL * tok_stride);
      vc[i] = load16<Stream>(base + i * TPL * tok_stride + kv_row);
    }
  }

  for (int j = blk_begin; j < blk_end && !bad_table; ++j) {
    // prefetch block j+1 while block j is consumed
    half8_t kn[LPB], vn[LPB];
    const int jn = j + 1;
    if (jn < blk_end) {
      const int k64 = (jn - blk_begin) & 63;
      if (k64 == 0) bt_vec = (lane < blk_end - jn) ? bt[jn + lane] : 0;
      const int phys = __builtin_amdgcn_readlane(bt_vec, k64);
      bad_table = phys < 0 || phys >= a.num_blocks;
      const half_t* base = pool + (bad_table ? 0 : (int64_t)phys * block_elems) + lane_off;
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        kn[i] = load16<Stream>(base + i * TPL * tok_stride);
        vn[i] = load16<Stream>(base + i * TPL * tok_stride + kv_row);
      }
    }

    // scores of the LPB tokens this lane's row sees in block j, for each query head
    float s[G][LPB];
#pragma unroll
    for (int i = 0; i < LPB; ++i)
#pragma unroll
      for (int g = 0; g < G; ++g) s[g][i] = group_sum<LPT>(dot8(qv[g], kc[i], 0.0f)) * a.scale_log2;

    const int tok0 = j * kBlockSize;
    if (tok0 + kBlockSize > L) {  // the sequence's last, partly filled block
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        if (tok0 + i * TPL + row >= L) {
#pragma unroll
          for (int g = 0; g < G; ++g) s[g][i] = neg_inf();
          vc[i] = half8_t{};
        }
      }
    }

#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int i = 0; i < LPB; ++i) mx = fmaxf(mx, s[g][i]);
      const float base = (mx == neg_inf()) ? 0.0f : mx;
      const float alpha = fast_exp2(m[g] - base);
      float pr[LPB], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        pr[i] = fast_exp2(s[g][i] - base);
        psum += pr[i];
      }
      l[g] = l[g] * alpha + psum;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        float x = acc[g][d] * alpha;
#pragma unroll
        for (int i = 0; i < LPB; ++i) x = fmaf(pr[i], (float)vc[i][d], x);
        acc[g][d] = x;
      }
      m[g] = mx;
    }

#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      kc[i] = kn[i];
      vc[i] = vn[i];
    }
  }

  if (bad_table) {
    // A table entry outside the pool: the whole output row becomes NaN. With several
    // partitions the reduce kernel writes the row, so poison this partition's partial.
    if (row == 0) {
      if (nparts == 1) {
        write_const_rows<D, G>(a, b, kvh, col, qnan());
      } else if (col == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int64_t bh = (int64_t)b * a.num_q_heads + (int64_t)kvh * G + g;
          float* wml = a.ws_ml + (bh * a.num_partitions + p) * 2;
          wml[0] = qnan();
          wml[1] = qnan();
        }
      }
    }
    return;
  }

  // merge the rows' running states: M = max m_r, sum and accumulator rescaled to M
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = m[g];
#pragma unroll
    for (int o = LPT; o < kWave; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, kWave));
    const float f = (m[g] == neg_inf()) ? 0.0f : fast_exp2(m[g] - M);
    float lt = l[g] * f;
#pragma unroll
    for (int o = LPT; o < kWave; o <<= 1) lt += __shfl_xor(lt, o, kWave);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      float x = acc[g][d] * f;
#pragma unroll
      for (int o = LPT; o < kWave; o <<= 1) x += __shfl_xor(x, o, kWave);
      acc[g][d] = x;
    }
    if (row == 0) {
      const int64_t h = (int64_t)kvh * G + g;
      const int64_t bh = (int64_t)b * a.num_q_heads + h;
      const float inv = 1.0f / lt;
      if (nparts == 1) {
        half8_t o;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[d] = (half_t)(acc[g][d] * inv);
        *reinterpret_cast<half8_t*>(static_cast<half_t*>(a.out) + bh * D + col * 8) = o;
      } else {
        float4_t o0, o1;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          o0[d] = acc[g][d] * inv;
          o1[d] = acc[g][d + 4] * inv;
        }
        float* wo = a.ws_o + (bh * a.num_partitions + p) * D + col * 8;
        *reinterpret_cast<float4_t*>(wo) = o0;
        *reinterpret_cast<float4_t*>(wo + 4) = o1;
        if (col == 0) {
          float* wml = a.ws_ml + (bh * a.num_partitions + p) * 2;
          wml[0] = M;
          wml[1] = lt;
        }
      }
    }
  }
}

// Merge the partitions of every (sequence, query head) that has more than one.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(const DecodeArgs a) {
  constexpr int PER_LANE = D / kWave;  // 2 (D=128) or 1 (D=64)
  const int lane = threadIdx.x & (kWave - 1);
  const int h = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (h >= a.num_q_heads) return;
  const int L = a.context_lens[b];
  if (L < 0 || L > a.max_context_len || L > a.max_blocks_per_seq * kBlockSize) return;
  const int part_tokens = a.partition_blocks * kBlockSize;
  const int nparts = (L + part_tokens - 1) / part_tokens;
  if (nparts <= 1) return;

  const int64_t bh = (int64_t)b * a.num_q_heads + h;
  const float* ml = a.ws_ml + bh * a.num_partitions * 2;
  const float* o = a.ws_o + bh * a.num_partitions * D + lane * PER_LANE;

  float M = neg_inf();
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  float den = 0.0f, acc[PER_LANE];
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k) acc[k] = 0.0f;
#pragma unroll 8
  for (int p = 0; p < nparts; ++p) {
    const float w = ml[2 * p + 1] * fast_exp2(ml[2 * p] - M);
    den += w;
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) acc[k] = fmaf(w, o[(int64_t)p * D + k], acc[k]);
  }
  const float inv = 1.0f / den;
  half_t* out = static_cast<half_t*>(a.out) + bh * D + lane * PER_LANE;
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k) out[k] = (half_t)(acc[k] * inv);
}

template <int D, int G>
hipError_t launch_decode_dg(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid((a.num_kv_heads + kWavesPerGroup - 1) / kWavesPerGroup, a.num_partitions, a.num_seqs);
  if (a.stream_kv)
    hipLaunchKernelGGL((decode_partition_kernel<D, G, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_partition_kernel<D, G, false>), grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions == 1) return e;
  dim3 rgrid((a.num_q_heads + kWavesPerGroup - 1) / kWavesPerGroup, a.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<D>), rgrid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_decode_dg<D, 1>(a, stream);
    case 2: return launch_decode_dg<D, 2>(a, stream);
    case 4: return launch_decode_dg<D, 4>(a, stream);
    case 8: return launch_decode_dg<D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  if (a.head_size == 128) return launch_decode_d<128>(a, stream);
  if (a.head_size == 64) return launch_decode_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
