// Paged-attention decode on gfx950: one query token per sequence attends to the
// sequence's cached tokens, reached block by block through its block-table row
// (page "vLLM GitHub 项目 …", section 二: logical blocks map to physical blocks that
// need not be contiguous; page "vLLM 部署深度指南": 16 tokens per block in a pool
// [num_blocks][16][2][num_kv_heads][head_size]).
//
// Work split. A context is cut into partitions of `partition_blocks` blocks. One wave
// handles one (sequence, KV head, partition) and all Hq/Hkv query heads reading that KV
// head; a workgroup holds four consecutive KV heads of the same (sequence, partition),
// so its loads touch neighbouring 256-byte rows of the same tokens. When no block is
// shared and the items do not all fit on the GPU at once, a pre-pass lists them longest
// first and the workgroups take them in that order (order_items_kernel); otherwise they
// follow launch order (decode_item).
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
// FP8 cache. With an E4M3 pool (one byte per element) each lane loads 16 codes (16 bytes,
// as it loads 8 fp16 values) and widens them exactly to fp16 (v_cvt_scalef32_pk_f16_fp8);
// the key scale is folded into the softmax scale and the value scale into the final 1 / l,
// so the arithmetic after the load is the fp16 cache's.
//
// Output. A sequence with one partition writes its fp16 row directly. Otherwise every
// partition writes (m, l, o = acc / l) to the workspace and the reduce kernel merges
// them: M = max m_p, w_p = l_p * 2^(m_p - M), out = sum w_p o_p / sum w_p.
#include <atomic>

#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pkv {
namespace {

constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWavesPerGroup * kWave;
constexpr int kXcds = 8;  // accelerator dies of an MI355X

// Lane geometry of the MHA kernel: each lane holds EPL consecutive elements of a token row
// (one 16-byte load: 8 fp16 values or 16 E4M3 codes).
template <int D, int EPL>
struct Geo {
  static constexpr int kLanesPerToken = D / EPL;                        // 16, 8 or 4
  static constexpr int kTokensPerLoad = kWave / kLanesPerToken;         // 4, 8 or 16
  static constexpr int kLoadsPerBlock = kBlockSize / kTokensPerLoad;    // 4, 2 or 1
};

// EPL cache elements at p (16 bytes) as NV = EPL / 8 fp16 vectors.
template <typename KV, bool Stream, int NV>
__device__ __forceinline__ void load_row_piece(const KV* p, half8_t (&x)[NV]) {
  if constexpr (sizeof(KV) == 2) {
    static_assert(NV == 1, "16 bytes of fp16 are 8 elements");
    x[0] = load16<Stream>(reinterpret_cast<const half_t*>(p));
  } else {
    static_assert(NV == 2, "16 bytes of E4M3 are 16 elements");
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) const u32x4_t gconst_u32x4_t;
    gconst_u32x4_t* gp = (gconst_u32x4_t*)(p);
    u32x4_t w;
    if constexpr (Stream)
      w = __builtin_nontemporal_load(gp);
    else
      w = *gp;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * v], 1.0f, false);
      const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * v], 1.0f, true);
      const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * v + 1], 1.0f, false);
      const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * v + 1], 1.0f, true);
      x[v] = half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    }
  }
}

// Work item (KV-head group, partition, sequence) of a workgroup. Workgroups reach the 8
// XCDs round-robin in launch order (workgroup i to XCD i % 8), each XCD with its own L2.
// The items of kSeqQuad consecutive sequences for one (partition, KV-head group) read the
// same blocks when those sequences share prompt blocks, so they form a quad that runs on
// one XCD in consecutive slots; quads are dealt to the XCDs round-robin, which keeps every
// sequence's work spread over all XCDs.
constexpr int kSeqQuad = 4;

struct DecodeItem {
  int hg, p, b;
  bool valid;
};

__device__ __forceinline__ DecodeItem decode_item(const DecodeArgs& a, int num_seqs, int num_parts,
                                                  int block) {
  const int groups = (a.num_kv_heads + kWavesPerGroup - 1) / kWavesPerGroup;
  const int64_t quads = (int64_t)((num_seqs + kSeqQuad - 1) / kSeqQuad) * num_parts * groups;
  const int xcd = block % kXcds;
  const int slot = block / kXcds;
  const int64_t quad = (int64_t)(slot / kSeqQuad) * kXcds + xcd;
  DecodeItem it;
  it.hg = (int)(quad % groups);
  const int64_t rest = quad / groups;
  it.p = (int)(rest % num_parts);
  it.b = (int)(rest / num_parts) * kSeqQuad + slot % kSeqQuad;
  it.valid = quad < quads && it.b < num_seqs;
  return it;
}

template <int D, int G, int EPL>
__device__ __forceinline__ void write_const_rows(const DecodeArgs& a, int b, int kvh, int col,
                                                 float value) {
  half_t* out = static_cast<half_t*>(a.out);
  half8_t v;
#pragma unroll
  for (int d = 0; d < 8; ++d) v[d] = (half_t)value;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t h = (int64_t)kvh * G + g;
#pragma unroll
    for (int u = 0; u < EPL / 8; ++u)
      *reinterpret_cast<half8_t*>(out + ((int64_t)b * a.num_q_heads + h) * D + col * EPL + 8 * u) = v;
  }
}

// One block of the MHA kernel: scores of the LPB tokens lane row `row` sees (for each of the
// G query heads), masked past the context length L, folded into the row's online softmax.
template <int D, int G, int EPL, int LPT, int TPL, int LPB, int NV>
__device__ __forceinline__ void consume_block(const half8_t (&qv)[G][NV], const half8_t (&kc)[LPB][NV],
                                              half8_t (&vc)[LPB][NV], int tok0, int L, int row,
                                              float scale_log2, float (&m)[G], float (&l)[G],
                                              float (&acc)[G][EPL]) {
  float s[G][LPB];
#pragma unroll
  for (int i = 0; i < LPB; ++i)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float dot = 0.0f;
#pragma unroll
      for (int u = 0; u < NV; ++u) dot = dot8(qv[g][u], kc[i][u], dot);
      s[g][i] = group_sum<LPT>(dot) * scale_log2;
    }

  if (tok0 + kBlockSize > L) {  // the sequence's last, partly filled block
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      if (tok0 + i * TPL + row >= L) {
#pragma unroll
        for (int g = 0; g < G; ++g) s[g][i] = neg_inf();
#pragma unroll
        for (int u = 0; u < NV; ++u) vc[i][u] = half8_t{};
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
    for (int d = 0; d < EPL; ++d) {
      float x = acc[g][d] * alpha;
#pragma unroll
      for (int i = 0; i < LPB; ++i) x = fmaf(pr[i], (float)vc[i][d / 8][d % 8], x);
      acc[g][d] = x;
    }
    m[g] = mx;
  }
}

// End of one (sequence b, KV head kvh, partition p) of the MHA kernel. A table entry outside
// the pool (bad_table) makes the whole output row NaN: with one partition here, with
// several through a NaN partial that the reduce kernel propagates. Otherwise the lane
// rows' running states are merged (M = max m_r, sums and accumulators rescaled to M) and
// written: the fp16 row when the sequence has one partition, else (m, l, o) to the
// workspace.
template <int D, int G, int EPL, int LPT>
__device__ __forceinline__ void finish_partition(const DecodeArgs& a, int b, int kvh, int p,
                                                 int nparts, int row, int col, bool bad_table,
                                                 float (&m)[G], float (&l)[G],
                                                 float (&acc)[G][EPL]) {
  constexpr int NV = EPL / 8;
  if (bad_table) {
    if (row == 0) {
      if (nparts == 1) {
        write_const_rows<D, G, EPL>(a, b, kvh, col, qnan());
      } else if (col == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int64_t bh = (int64_t)b * a.num_q_heads + (int64_t)kvh * G + g;
          float* wml = a.ws_ml + (bh * a.ws_parts + p) * 2;
          wml[0] = qnan();
          wml[1] = qnan();
        }
      }
    }
    return;
  }
  // over the wave's rows of lanes (lane L and L ^ o for o = LPT .. 32)
  auto row_max = [](float x) {
    if constexpr (LPT <= 4) x = max_xor<4>(x);
    if constexpr (LPT <= 8) x = max_xor<8>(x);
    if constexpr (LPT <= 16) x = max_xor<16>(x);
    return max_xor<32>(x);
  };
  auto row_sum = [](float x) {
    if constexpr (LPT <= 4) x = sum_xor<4>(x);
    if constexpr (LPT <= 8) x = sum_xor<8>(x);
    if constexpr (LPT <= 16) x = sum_xor<16>(x);
    return sum_xor<32>(x);
  };
  static_assert(LPT >= 4 && LPT <= 32, "rows of 4 to 32 lanes");
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = row_max(m[g]);
    const float f = (m[g] == neg_inf()) ? 0.0f : fast_exp2(m[g] - M);
    const float lt = row_sum(l[g] * f);
#pragma unroll
    for (int d = 0; d < EPL; ++d) acc[g][d] = row_sum(acc[g][d] * f);
    if (row == 0) {
      const int64_t h = (int64_t)kvh * G + g;
      const int64_t bh = (int64_t)b * a.num_q_heads + h;
      const float inv = a.v_scale / lt;
      if (nparts == 1) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          half8_t o;
#pragma unroll
          for (int d = 0; d < 8; ++d) o[d] = (half_t)(acc[g][8 * u + d] * inv);
          *reinterpret_cast<half8_t*>(static_cast<half_t*>(a.out) + bh * D + col * EPL + 8 * u) = o;
        }
      } else {
        float* wo = a.ws_o + (bh * a.ws_parts + p) * D + col * EPL;
#pragma unroll
        for (int u = 0; u < 2 * NV; ++u) {
          float4_t o4;
#pragma unroll
          for (int d = 0; d < 4; ++d) o4[d] = acc[g][4 * u + d] * inv;
          *reinterpret_cast<float4_t*>(wo + 4 * u) = o4;
        }
        if (col == 0) {
          float* wml = a.ws_ml + (bh * a.ws_parts + p) * 2;
          wml[0] = M;
          wml[1] = lt;
        }
      }
    }
  }
}

template <int D, int G, bool Stream, typename KV>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(const DecodeArgs a,
                                                                    const int* __restrict__ items) {
  constexpr int EPL = 16 / sizeof(KV);  // elements per lane and load
  constexpr int NV = EPL / 8;           // fp16 vectors per lane
  using Gm = Geo<D, EPL>;
  constexpr int LPT = Gm::kLanesPerToken;
  constexpr int TPL = Gm::kTokensPerLoad;
  constexpr int LPB = Gm::kLoadsPerBlock;

  const int lane = threadIdx.x & (kWave - 1);
  DecodeItem item;
  if (items != nullptr) {  // largest-first list: item blockIdx / groups, KV-head group blockIdx % groups
    const int groups = (a.num_kv_heads + kWavesPerGroup - 1) / kWavesPerGroup;
    const int idx = blockIdx.x / groups;
    if (idx >= items[0]) return;
    const unsigned key = (unsigned)items[1 + idx];
    item.hg = blockIdx.x % groups;
    item.b = (int)(key >> 16);
    item.p = (int)(key & 0xffffu);
  } else {
    item = decode_item(a, a.num_seqs, a.num_partitions, blockIdx.x);
    if (!item.valid) return;
  }
  const int kvh = item.hg * kWavesPerGroup + (threadIdx.x >> 6);
  const int p = item.p;
  const int b = item.b;
  if (kvh >= a.num_kv_heads) return;
  const int row = lane / LPT;
  const int col = lane % LPT;
  // the partition's block-table entries, one per lane (64 at a time), are requested before
  // the context length arrives: the table row holds max_blocks_per_seq entries either way
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  const int first = p * a.partition_blocks;
  int bt_vec = (first + lane < a.max_blocks_per_seq) ? bt[first + lane] : 0;

  const int L = a.context_lens[b];
  const bool bad_len = L < 0 || L > a.max_context_len || L > a.max_blocks_per_seq * kBlockSize;
  if (bad_len || L == 0) {
    if (p == 0 && row == 0) write_const_rows<D, G, EPL>(a, b, kvh, col, bad_len ? qnan() : 0.0f);
    return;
  }
  const int part_tokens = a.partition_blocks * kBlockSize;
  const int nparts = (L + part_tokens - 1) / part_tokens;
  if (p >= nparts) return;
  const int blk_begin = p * a.partition_blocks;
  const int blk_end = min(blk_begin + a.partition_blocks, (L + kBlockSize - 1) / kBlockSize);

  const half_t* qp = static_cast<const half_t*>(a.q);
  half8_t qv[G][NV];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int u = 0; u < NV; ++u)
      qv[g][u] = *reinterpret_cast<const half8_t*>(
          qp + ((int64_t)b * a.num_q_heads + (int64_t)kvh * G + g) * D + col * EPL + 8 * u);

  const int kv_row = a.num_kv_heads * D;  // elements of one K (or V) row over all heads
  const int tok_stride = 2 * kv_row;       // elements between consecutive tokens of a block
  const int64_t block_elems = (int64_t)kBlockSize * tok_stride;
  // element offset of this lane's piece of load i inside a block: + i * TPL * tok_stride
  const int lane_off = row * tok_stride + kvh * D + col * EPL;
  const KV* pool = static_cast<const KV*>(a.pool);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = neg_inf();
    l[g] = 0.0f;
#pragma unroll
    for (int d = 0; d < EPL; ++d) acc[g][d] = 0.0f;
  }

  bool bad_table = false;

  half8_t kc[LPB][NV], vc[LPB][NV];
  {
    const int phys = __builtin_amdgcn_readfirstlane(bt_vec);
    bad_table = phys < 0 || phys >= a.num_blocks;
    const KV* base = pool + (bad_table ? 0 : (int64_t)phys * block_elems) + lane_off;
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      load_row_piece<KV, Stream>(base + i * TPL * tok_stride, kc[i]);
      load_row_piece<KV, Stream>(base + i * TPL * tok_stride + kv_row, vc[i]);
    }
  }

  for (int j = blk_begin; j < blk_end && !bad_table; ++j) {
    // prefetch block j+1 while block j is consumed
    half8_t kn[LPB][NV], vn[LPB][NV];
    const int jn = j + 1;
    if (jn < blk_end) {
      const int k64 = (jn - blk_begin) & 63;
      if (k64 == 0) bt_vec = (lane < blk_end - jn) ? bt[jn + lane] : 0;
      const int phys = __builtin_amdgcn_readlane(bt_vec, k64);
      bad_table = phys < 0 || phys >= a.num_blocks;
      const KV* base = pool + (bad_table ? 0 : (int64_t)phys * block_elems) + lane_off;
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        load_row_piece<KV, Stream>(base + i * TPL * tok_stride, kn[i]);
        load_row_piece<KV, Stream>(base + i * TPL * tok_stride + kv_row, vn[i]);
      }
    }

    consume_block<D, G, EPL, LPT, TPL, LPB, NV>(qv, kc, vc, j * kBlockSize, L, row, a.scale_log2,
                                                m, l, acc);

#pragma unroll
    for (int i = 0; i < LPB; ++i)
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        kc[i][u] = kn[i][u];
        vc[i][u] = vn[i][u];
      }
  }

  finish_partition<D, G, EPL, LPT>(a, b, kvh, p, nparts, row, col, bad_table, m, l, acc);
}

// ---- largest-first order ----------------------------------------------------------------
// With several partitions per sequence the work is ragged: every sequence's last partition
// is partly filled, and identical partitions take very different times under full load.
// The hardware starts workgroups in launch order as slots free up, so when the partly
// filled partitions are a sizeable share of the items (at most kOrderMaxParts partitions
// per sequence; with one partition every item is a whole, ragged context), a
// one-workgroup pre-pass lists the (sequence, partition) items by decreasing length and
// the partition kernel takes them in that order: the long items run first and the short
// ones fill the end. Only when no block is shared between sequences: otherwise launch
// order keeps the sequences of a prompt group together (see decode_item).
constexpr int kOrderMaxParts = 16;
constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = 1025;  // bucket 1024 - min(size in blocks, 1024)

// items[0] = number of (sequence, partition) items, items[1 + i] = (b << 16) | p, longest
// first; a sequence of length 0 or out of range has one item (p = 0) that writes its rows.
__device__ __forceinline__ int order_bucket(const DecodeArgs& a, int b, int p) {
  const int L = a.context_lens[b];
  const bool bad = L < 0 || L > a.max_context_len || L > a.max_blocks_per_seq * kBlockSize;
  if (bad || L == 0) return p == 0 ? kOrderBuckets - 1 : -1;  // one item writes the row
  const int size = (L + kBlockSize - 1) / kBlockSize - p * a.partition_blocks;
  if (size <= 0) return -1;
  return 1024 - min(min(size, a.partition_blocks), 1024);
}

__global__ __launch_bounds__(kOrderThreads) void order_items_kernel(const DecodeArgs a,
                                                                    int* __restrict__ items) {
  __shared__ int hist[kOrderBuckets];
  __shared__ int wsum[kOrderThreads / kWave];
  const int tid = threadIdx.x;
  for (int i = tid; i < kOrderBuckets; i += kOrderThreads) hist[i] = 0;
  __syncthreads();
  const int np = a.num_partitions;
  const int64_t pairs = (int64_t)a.num_seqs * np;
  for (int64_t i = tid; i < pairs; i += kOrderThreads) {
    const int bk = order_bucket(a, (int)(i / np), (int)(i % np));
    if (bk >= 0) atomicAdd(&hist[bk], 1);
  }
  __syncthreads();
  // exclusive prefix sum of buckets 0 .. 1023 (one per thread); bucket 1024 comes last
  const int lane = tid & (kWave - 1), w = tid / kWave;
  const int v = hist[tid];
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) wsum[w] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int k = 0; k < kOrderThreads / kWave; ++k) {
    if (k < w) before += wsum[k];
    all += wsum[k];
  }
  const int last = hist[kOrderBuckets - 1];
  __syncthreads();
  hist[tid] = before + x - v;
  if (tid == 0) {
    hist[kOrderBuckets - 1] = all;
    items[0] = all + last;
  }
  __syncthreads();
  for (int64_t i = tid; i < pairs; i += kOrderThreads) {
    const int b = (int)(i / np), p = (int)(i % np);
    const int bk = order_bucket(a, b, p);
    if (bk >= 0) items[1 + atomicAdd(&hist[bk], 1)] = (int)(((unsigned)b << 16) | (unsigned)p);
  }
}

// Grouped-query decode on the matrix cores: the G query heads that read one KV head are
// the N side of 16x16 MFMA tiles (G <= 16 columns used). Per 16-token block:
//   S^T[token][head] = K[token][:] . Q[head][:]     v_mfma_f32_16x16x32_f16, A = K rows
//                                                    loaded from HBM straight into operand
//                                                    layout, B = Q rows (zero past G)
//   O^T[dim][head]  += V^T[dim][token] . P^T[token][head]   v_mfma_f32_16x16x16f16
// Lane (n, q) = (lane % 16, lane / 16) holds S^T rows 4q..4q+3 of column n, which as fp16
// is exactly its B operand of the second product. V^T comes from the block staged in LDS
// in natural row-major order through the transposing LDS read (ds_read_b64_tr_b16): source
// lane i of a 16-lane group points at V[4q + i/4][16dt + 4(i%4)] and lane n receives
// V[4q + k][16dt + n], k = 0..3. Softmax per head (column) in fp32, base 2, with the
// reference max moved only when it is beaten by more than 2^8.
template <int D>
struct GqaGeo {
  static constexpr int KS = D / 32;          // k-steps of S^T
  static constexpr int DT = D / 16;          // 16-dim tiles of O^T
  static constexpr int PIECES = D / 8;       // 16-byte pieces per token row of one head
  static constexpr int VLOADS = PIECES / 4;  // V pieces per lane per block
  static constexpr int VPITCH = D + 16;      // LDS row pitch (halves): 8 rows fill 64 banks
};

// An FP8 cache's grouped-query loads bring 16 codes per lane (one 16-byte load); they are
// widened to fp16 where they are used.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t gconst_u32x4_t;

template <bool Stream>
__device__ __forceinline__ u32x4_t load_codes16(const fp8_t* p) {
  gconst_u32x4_t* gp = (gconst_u32x4_t*)(p);
  if constexpr (Stream)
    return __builtin_nontemporal_load(gp);
  else
    return *gp;
}

__device__ __forceinline__ half8_t widen_lo(u32x4_t w) { return widen_fp8x8(u32x2_t{w[0], w[1]}); }
__device__ __forceinline__ half8_t widen_hi(u32x4_t w) { return widen_fp8x8(u32x2_t{w[2], w[3]}); }

// The group of sequence b: g with group_start[g] <= b < group_start[g + 1], or -1.
__device__ __forceinline__ int group_of(const DecodeArgs& a, int b) {
  int lo = 0, hi = a.num_groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.group_start[mid] <= b) lo = mid; else hi = mid;
  }
  return (a.group_start[lo] <= b && b < a.group_start[lo + 1]) ? lo : -1;
}

// Shared-prefix decode splits each context at its group's prefix length P: one pass over
// the prefix per group, whose 16 tile columns are (sample, query head) pairs of the
// group's sequences (the prefix's K/V read once for all of them), and one pass over each
// sequence's own tokens P .. L - 1. Both write partitions to the workspace and the reduce
// merges them. Plain decode is mode 0.
constexpr int kModePlain = 0, kModeShared = 1;

template <int D, int G, bool Stream, typename KV, int Mode = kModePlain>
__global__ __launch_bounds__(kThreads) void decode_gqa_kernel(const DecodeArgs a,
                                                              const int* __restrict__ items) {
  static_assert(G >= 1 && G <= 16, "query heads per KV head must fit 16 columns");
  constexpr int S = 16 / G;  // samples of a group per tile in the prefix pass
  using Gm = GqaGeo<D>;
  constexpr int KS = Gm::KS, DT = Gm::DT, PIECES = Gm::PIECES, VLOADS = Gm::VLOADS;
  // FP8 cache: one 16-byte load per lane covers two k-steps of K (dims 64j + 16q4 .. +16,
  // the first 8 for k-step 2j, the next 8 for 2j + 1; the query's dims follow the same
  // order, so the products and their sum over dims are unchanged) and two 8-element pieces
  // of V; the codes stay packed until they are used
  constexpr bool kFp8 = sizeof(KV) == 1;
  constexpr int KL = kFp8 ? KS / 2 : KS;          // K loads per lane and block
  constexpr int VL = kFp8 ? VLOADS / 2 : VLOADS;  // V loads per lane and block
  constexpr int VPL = kFp8 ? 2 : 1;               // 8-element V pieces per load
  using Raw = std::conditional_t<kFp8, u32x4_t, half8_t>;  // what one load brings
  static_assert(!kFp8 || (KS % 2 == 0 && VLOADS % 2 == 0), "FP8 loads pair k-steps and pieces");
  constexpr int VPITCH = Gm::VPITCH;
  constexpr float kSlack = 8.0f;
  __shared__ __align__(16) half_t vstage[kWavesPerGroup][kBlockSize * VPITCH];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // shared-prefix decode runs both passes in one launch: the first prefix_grid workgroups
  // take the prefix items, the rest each sequence's own tokens
  const bool pre = Mode == kModeShared && (int)blockIdx.x < a.prefix_grid;
  DecodeItem item;
  if (Mode == kModePlain && items != nullptr) {  // largest-first list, as in the MHA kernel
    const int groups = (a.num_kv_heads + kWavesPerGroup - 1) / kWavesPerGroup;
    const int idx = blockIdx.x / groups;
    if (idx >= items[0]) return;
    const unsigned key = (unsigned)items[1 + idx];
    item.hg = blockIdx.x % groups;
    item.b = (int)(key >> 16);
    item.p = (int)(key & 0xffffu);
  } else {
    item = pre ? decode_item(a, a.num_groups * a.group_chunks, a.prefix_parts, blockIdx.x)
               : decode_item(a, a.num_seqs, a.num_partitions,
                             blockIdx.x - (Mode == kModeShared ? a.prefix_grid : 0));
    if (!item.valid) return;
  }
  const int kvh = item.hg * kWavesPerGroup + w;
  const int p = item.p;
  if (kvh >= a.num_kv_heads) return;
  const int n = lane & 15;   // token row of K / tile column
  const int q4 = lane >> 4;  // 16-lane group
  half_t* vs = vstage[w];

  // b: the sequence whose table the wave reads; [tok_lo, L): the tokens of this pass;
  // column n stands for query head (col_seq, col_head) when col_ok
  int b = item.b, tok_lo = 0, L, col_seq = b, col_head = kvh * G + n, slot0 = 0;
  bool col_ok = n < G;
  half_t* out = static_cast<half_t*>(a.out);
  if constexpr (Mode == kModePlain) {
    L = a.context_lens[b];
    const bool bad_len = L < 0 || L > a.max_context_len || L > a.max_blocks_per_seq * kBlockSize;
    if (bad_len || L == 0) {
      if (p == 0 && lane < G * PIECES) {
        const int h = kvh * G + lane / PIECES;
        half8_t v;
#pragma unroll
        for (int d = 0; d < 8; ++d) v[d] = (half_t)(bad_len ? qnan() : 0.0f);
        *reinterpret_cast<half8_t*>(out + ((int64_t)b * a.num_q_heads + h) * D + 8 * (lane % PIECES)) = v;
      }
      return;
    }
  } else if (pre) {
    // item.b enumerates (group, chunk of S samples)
    const int grp = b / a.group_chunks, chunk = b % a.group_chunks;
    const int seq0 = a.group_start[grp], nseq = a.group_start[grp + 1] - seq0;
    if (chunk * S >= nseq) return;
    L = a.prefix_lens[grp];
    // a prefix or group the arguments cannot hold is left out; the reduce turns its rows
    // into NaN
    if (L <= 0 || L % kBlockSize || L > a.max_context_len || L > a.max_blocks_per_seq * kBlockSize ||
        seq0 < 0 || seq0 + nseq > a.num_seqs)
      return;
    b = seq0;  // every table of the group holds the prefix blocks: read the first
    col_seq = seq0 + chunk * S + n / G;
    col_head = kvh * G + n % G;
    col_ok = n < S * G && chunk * S + n / G < nseq;
  } else {
    const int grp = group_of(a, b);
    L = a.context_lens[b];
    if (grp < 0) return;
    tok_lo = a.prefix_lens[grp];
    if (L < 0 || L > a.max_context_len || L > a.max_blocks_per_seq * kBlockSize || tok_lo < 0 ||
        tok_lo % kBlockSize || tok_lo > L)
      return;
    slot0 = a.prefix_parts;
  }
  const int part_tokens = a.partition_blocks * kBlockSize;
  const int nparts = (L - tok_lo + part_tokens - 1) / part_tokens;
  if (p >= nparts) return;
  const int blk_begin = tok_lo / kBlockSize + p * a.partition_blocks;
  const int blk_end = min(blk_begin + a.partition_blocks, (L + kBlockSize - 1) / kBlockSize);

  // B operand of S^T: column n's query dims 32ks + 8q4 .. +8, zero past the used columns
  const half_t* qp = static_cast<const half_t*>(a.q);
  half8_t qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qb[ks] = col_ok ? load16(qp + ((int64_t)col_seq * a.num_q_heads + col_head) * D +
                             (kFp8 ? 64 * (ks >> 1) + 16 * q4 + 8 * (ks & 1) : 32 * ks + 8 * q4))
                    : half8_t{};

  const int kv_row = a.num_kv_heads * D;
  const int tok_stride = 2 * kv_row;
  const int64_t block_elems = (int64_t)kBlockSize * tok_stride;
  const KV* pool = static_cast<const KV*>(a.pool);
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  // per-lane element offsets inside a block
  constexpr int KSTEP = kFp8 ? 64 : 32;  // elements between a lane's K loads
  const int koff = n * tok_stride + kvh * D + (kFp8 ? 16 : 8) * q4;  // + KSTEP j
  int voff[VL], vlds[VL];
#pragma unroll
  for (int j = 0; j < VL; ++j) {
    const int idx = lane + kWave * j;
    const int t = idx / (PIECES / VPL), c = idx % (PIECES / VPL);
    voff[j] = t * tok_stride + kv_row + kvh * D + 8 * VPL * c;
    vlds[j] = t * VPITCH + 8 * VPL * c;
  }
  auto load_raw = [&](const KV* p) -> Raw {
    if constexpr (kFp8)
      return load_codes16<Stream>(p);
    else
      return load_kv8<KV, Stream>(p);
  };
  // transposing read of V tile dt: token 4q4 + n/4, dims 16dt + 4(n%4)
  const int vtr = (4 * q4 + n / 4) * VPITCH + 4 * (n % 4);

  float m = neg_inf(), l = 0.0f;  // per column (head n); l is this lane's partial sum
  float4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  int bt_vec = (lane < blk_end - blk_begin) ? bt[blk_begin + lane] : 0;
  bool bad_table = false;
  // Loads of block jb into kr / vr: its table entry from the lane vector (refilled every 64
  // blocks); an entry outside the pool is not followed and flags the pass.
  auto request = [&](Raw (&kr)[KL], Raw (&vr)[VL], int jb) {
    const int k64 = (jb - blk_begin) & 63;
    if (k64 == 0 && jb > blk_begin) bt_vec = (lane < blk_end - jb) ? bt[jb + lane] : 0;
    const int phys = __builtin_amdgcn_readlane(bt_vec, k64);
    const bool bad = phys < 0 || phys >= a.num_blocks;
    bad_table = bad_table || bad;
    const KV* base = pool + (bad ? 0 : (int64_t)phys * block_elems);
#pragma unroll
    for (int j = 0; j < KL; ++j) kr[j] = load_raw(base + koff + KSTEP * j);
#pragma unroll
    for (int j = 0; j < VL; ++j) vr[j] = load_raw(base + voff[j]);
  };
  // Blocks in flight. fp16: the next block is requested before the current one is used
  // (two register buffers). FP8: the codes of a block are half the bytes, and two blocks
  // are kept in flight without a third buffer: block jb + 2 is requested into block jb's
  // registers as soon as its V is staged and its S^T products have read its K (C4 with
  // private copies 113.9 -> 102.7 us, shared-prefix decode 64.5 -> 60.3 us; fp16 the
  // same way took 12 more registers and was no faster)
  constexpr bool kTwoAhead = kFp8;
  auto consume = [&](Raw (&kr)[KL], Raw (&vr)[VL], int jb) {
    const int tok0 = jb * kBlockSize;
    const bool tail = tok0 + kBlockSize > L;
    // stage V (tokens past the context end as zeros: their slots may hold anything)
#pragma unroll
    for (int j = 0; j < VL; ++j) {
      const int t = (lane + kWave * j) / (PIECES / VPL);
      const bool zero = tail && tok0 + t >= L;
      if constexpr (kFp8) {
        *reinterpret_cast<half8_t*>(vs + vlds[j]) = zero ? half8_t{} : widen_lo(vr[j]);
        *reinterpret_cast<half8_t*>(vs + vlds[j] + 8) = zero ? half8_t{} : widen_hi(vr[j]);
      } else {
        *reinterpret_cast<half8_t*>(vs + vlds[j]) = zero ? half8_t{} : vr[j];
      }
    }
    // S^T of the block
    float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      half8_t ka;
      if constexpr (kFp8)
        ka = (ks & 1) ? widen_hi(kr[ks >> 1]) : widen_lo(kr[ks >> 1]);
      else
        ka = kr[ks];
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[ks], sacc, 0, 0, 0);
    }
    // the block's registers have been read: with two blocks ahead, block jb + 2 goes there
    if (kTwoAhead && jb + 2 < blk_end) request(kr, vr, jb + 2);
    // mask, column max over the block's 16 tokens, lazy rescale
    float mloc = neg_inf();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (tail && tok0 + 4 * q4 + i >= L) sacc[i] = neg_inf();
      mloc = fmaxf(mloc, sacc[i]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float mb = mloc * a.scale_log2;
    const bool move = mb > m + kSlack;
    if (__builtin_amdgcn_ballot_w64(move)) {
      asm volatile("");
      const float mnew = move ? mb : m;
      const float alpha = move ? fast_exp2(m - mnew) : 1.0f;  // a column still at -inf stays
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m = mnew;
    }
    const float base = (m == neg_inf()) ? 0.0f : m;
    half4_t pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = fast_exp2(fmaf(sacc[i], a.scale_log2, -base));
      pb[i] = (half_t)pv;
      l += (float)pb[i];
    }
    // the staged V must be visible to this wave's transposing reads
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const half4_t va = __builtin_bit_cast(
          half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                       (__attribute__((address_space(3))) short4_t*)(vs + vtr + 16 * dt)));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pb, o[dt], 0, 0, 0);
    }
    // the next block's V overwrites the stage only after these reads have returned
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  if constexpr (kTwoAhead) {
    Raw k0[KL], v0[VL], k1[KL], v1[VL];  // even and odd blocks of the pass
    request(k0, v0, blk_begin);
    if (blk_begin + 1 < blk_end) request(k1, v1, blk_begin + 1);
    for (int jb = blk_begin; jb < blk_end && !bad_table; jb += 2) {
      consume(k0, v0, jb);
      if (jb + 1 >= blk_end || bad_table) break;
      consume(k1, v1, jb + 1);
    }
  } else {
    Raw kc[KL], vc[VL];
    request(kc, vc, blk_begin);
    for (int jb = blk_begin; jb < blk_end && !bad_table; ++jb) {
      Raw kn[KL], vn[VL];
      if (jb + 1 < blk_end) request(kn, vn, jb + 1);
      consume(kc, vc, jb);
#pragma unroll
      for (int j = 0; j < KL; ++j) kc[j] = kn[j];
#pragma unroll
      for (int j = 0; j < VL; ++j) vc[j] = vn[j];
    }
  }

  // column sums over the four 16-lane groups
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  if (!col_ok) return;
  const int64_t bh = (int64_t)col_seq * a.num_q_heads + col_head;
  const int slot = slot0 + p;  // workspace partition slot
  if (bad_table) {
    if (Mode == kModePlain && nparts == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        half4_t x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (half_t)qnan();
        *reinterpret_cast<half4_t*>(out + bh * D + 16 * dt + 4 * q4) = x;
      }
    } else if (q4 == 0) {
      float* wml = a.ws_ml + (bh * a.ws_parts + slot) * 2;
      wml[0] = qnan();
      wml[1] = qnan();
    }
    return;
  }
  const float inv = a.v_scale / l;
  if (Mode == kModePlain && nparts == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      half4_t x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (half_t)(o[dt][i] * inv);
      *reinterpret_cast<half4_t*>(out + bh * D + 16 * dt + 4 * q4) = x;
    }
  } else {
    float* wo = a.ws_o + (bh * a.ws_parts + slot) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<float4_t*>(wo + 16 * dt + 4 * q4) = o[dt] * inv;
    if (q4 == 0) {
      float* wml = a.ws_ml + (bh * a.ws_parts + slot) * 2;
      wml[0] = m;
      wml[1] = l;
    }
  }
}

// Merge the partitions of every (sequence, query head) that has more than one. With
// Cascade (shared-prefix decode) every row is merged here from its prefix partitions
// (slots 0 ..) and its own partitions (slots prefix_parts ..), and rows whose length or
// group is out of bounds become NaN (no partition kernel writes rows in that mode).
template <int D, bool Cascade>
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(const DecodeArgs a) {
  constexpr int PER_LANE = D / kWave;  // 2 (D=128) or 1 (D=64)
  const int lane = threadIdx.x & (kWave - 1);
  const int h = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (h >= a.num_q_heads) return;
  const int L = a.context_lens[b];
  const bool bad_len = L < 0 || L > a.max_context_len || L > a.max_blocks_per_seq * kBlockSize;
  const int part_tokens = a.partition_blocks * kBlockSize;
  const int64_t bh = (int64_t)b * a.num_q_heads + h;
  half_t* out = static_cast<half_t*>(a.out) + bh * D + lane * PER_LANE;
  int n_pre = 0, n_own;
  if constexpr (Cascade) {
    const int grp = group_of(a, b);
    const int P = grp < 0 ? -1 : a.prefix_lens[grp];
    const bool bad = bad_len || grp < 0 || a.group_start[grp] < 0 ||
                     a.group_start[grp + 1] > a.num_seqs || b - a.group_start[grp] >= a.group_cap ||
                     P < 0 || P % kBlockSize || P > L ||
                     (P + part_tokens - 1) / part_tokens > a.prefix_parts;
    if (bad || L == 0) {
#pragma unroll
      for (int k = 0; k < PER_LANE; ++k) out[k] = (half_t)(bad ? qnan() : 0.0f);
      return;
    }
    n_pre = (P + part_tokens - 1) / part_tokens;
    n_own = (L - P + part_tokens - 1) / part_tokens;
  } else {
    if (bad_len) return;
    n_own = (L + part_tokens - 1) / part_tokens;
    if (n_own <= 1) return;
  }
  const int n_all = n_pre + n_own;
  const float* ml = a.ws_ml + bh * a.ws_parts * 2;
  const float* o = a.ws_o + bh * a.ws_parts * D + lane * PER_LANE;
  auto slot_of = [&](int k) { return k < n_pre ? k : a.prefix_parts * Cascade + (k - n_pre); };

  float M = neg_inf();
  for (int k = 0; k < n_all; ++k) M = fmaxf(M, ml[2 * slot_of(k)]);
  float den = 0.0f, acc[PER_LANE];
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k) acc[k] = 0.0f;
#pragma unroll 8
  for (int k = 0; k < n_all; ++k) {
    const int sl = slot_of(k);
    const float w = ml[2 * sl + 1] * fast_exp2(ml[2 * sl] - M);
    den += w;
#pragma unroll
    for (int e = 0; e < PER_LANE; ++e) acc[e] = fmaf(w, o[(int64_t)sl * D + e], acc[e]);
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k) out[k] = (half_t)(acc[k] * inv);
}

// Waves of the plain decode kernel for (D, G, Stream, KV) that the current device holds at
// once, from the occupancy the compiled kernel allows (0 when the runtime cannot say);
// queried once per device.
template <int D, int G, bool Stream, typename KV>
int64_t resident_waves() {
  static std::atomic<int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, cus = 0;
  hipError_t e;
  if constexpr (G == 1)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_partition_kernel<D, 1, Stream, KV>,
                                                     kThreads, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_gqa_kernel<D, G, Stream, KV>,
                                                     kThreads, 0);
  if (e != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  v = (int64_t)per_cu * cus * kWavesPerGroup;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <int D, int G, typename KV>
hipError_t launch_decode_dg(const DecodeArgs& a, hipStream_t stream) {
  const int64_t groups = (a.num_kv_heads + kWavesPerGroup - 1) / kWavesPerGroup;
  const int64_t quads = (int64_t)((a.num_seqs + kSeqQuad - 1) / kSeqQuad) * a.num_partitions * groups;
  const int64_t wgs = (quads + kXcds - 1) / kXcds * kXcds * kSeqQuad;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  const int* items = nullptr;
  dim3 pgrid = grid;
  // ordered only when no block is shared (the caller's PA_DECODE_KV_STREAM): launch order
  // keeps sequences that share prompt blocks together, so those blocks come from L2; and
  // only when the items do not all fit on the device at once (then order changes nothing)
  const int64_t waves = (int64_t)a.num_seqs * a.num_partitions * groups * kWavesPerGroup;
  if (a.stream_kv && a.num_partitions <= kOrderMaxParts && a.ws_items != nullptr &&
      waves > resident_waves<D, G, true, KV>()) {
    const int64_t owgs = (int64_t)a.num_seqs * a.num_partitions * groups;
    if (owgs > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(order_items_kernel, dim3(1), dim3(kOrderThreads), 0, stream, a, a.ws_items);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    items = a.ws_items;
    pgrid = dim3((unsigned)owgs);
  }
  if constexpr (G == 1) {  // one query head per KV head: vector ALUs
    if (a.stream_kv)
      hipLaunchKernelGGL((decode_partition_kernel<D, 1, true, KV>), pgrid, dim3(kThreads), 0, stream, a, items);
    else
      hipLaunchKernelGGL((decode_partition_kernel<D, 1, false, KV>), pgrid, dim3(kThreads), 0, stream, a, items);
  } else {  // a query-head group per KV head: matrix cores
    if (a.stream_kv)
      hipLaunchKernelGGL((decode_gqa_kernel<D, G, true, KV>), pgrid, dim3(kThreads), 0, stream, a, items);
    else
      hipLaunchKernelGGL((decode_gqa_kernel<D, G, false, KV>), pgrid, dim3(kThreads), 0, stream, a, items);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions == 1) return e;
  dim3 rgrid((a.num_q_heads + kWavesPerGroup - 1) / kWavesPerGroup, a.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<D, false>), rgrid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, typename KV>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_decode_dg<D, 1, KV>(a, stream);
    case 2: return launch_decode_dg<D, 2, KV>(a, stream);
    case 4: return launch_decode_dg<D, 4, KV>(a, stream);
    case 8: return launch_decode_dg<D, 8, KV>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int G, typename KV>
hipError_t launch_shared_prefix_dg(const DecodeArgs& a, hipStream_t stream) {
  constexpr int S = 16 / G;  // samples per prefix tile
  const int64_t hgroups = (a.num_kv_heads + kWavesPerGroup - 1) / kWavesPerGroup;
  auto grid_of = [&](int64_t seqs, int64_t parts) {
    const int64_t quads = (seqs + kSeqQuad - 1) / kSeqQuad * parts * hgroups;
    return (quads + kXcds - 1) / kXcds * kXcds * kSeqQuad;
  };
  // a.group_cap holds the caller's largest group size on entry
  DecodeArgs k = a;
  k.group_chunks = (a.group_cap + S - 1) / S;
  k.group_cap = k.group_chunks * S;
  const int64_t wpre =
      a.prefix_parts > 0 ? grid_of((int64_t)a.num_groups * k.group_chunks, a.prefix_parts) : 0;
  const int64_t wown = grid_of(a.num_seqs, a.num_partitions);
  if (wpre + wown > INT32_MAX) return hipErrorInvalidValue;
  k.prefix_grid = (int)wpre;
  // one launch: prefix items, then every sequence's own tokens (independent outputs). Each
  // physical block is read once here (the prefix once per group), so the K/V loads carry
  // the non-temporal hint (64 prompt groups x 4 samples, fp16: 103.5 -> 92.1 us; FP8,
  // after a cache flush and with two blocks in flight: 66.4 -> 64.3 us, where back to
  // back, with the whole FP8 working set in the last-level cache, plain loads were
  // faster).
  hipLaunchKernelGGL((decode_gqa_kernel<D, G, true, KV, kModeShared>), dim3((unsigned)(wpre + wown)),
                     dim3(kThreads), 0, stream, k, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DecodeArgs own = k;
  dim3 rgrid((a.num_q_heads + kWavesPerGroup - 1) / kWavesPerGroup, a.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<D, true>), rgrid, dim3(kThreads), 0, stream, own);
  return hipGetLastError();
}

template <int D, typename KV>
hipError_t launch_shared_prefix_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_shared_prefix_dg<D, 1, KV>(a, stream);
    case 2: return launch_shared_prefix_dg<D, 2, KV>(a, stream);
    case 4: return launch_shared_prefix_dg<D, 4, KV>(a, stream);
    case 8: return launch_shared_prefix_dg<D, 8, KV>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_shared_prefix(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  if (a.kv_fp8) {
    if (a.head_size == 128) return launch_shared_prefix_d<128, fp8_t>(a, stream);
    if (a.head_size == 64) return launch_shared_prefix_d<64, fp8_t>(a, stream);
  } else {
    if (a.head_size == 128) return launch_shared_prefix_d<128, half_t>(a, stream);
    if (a.head_size == 64) return launch_shared_prefix_d<64, half_t>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  if (a.kv_fp8) {
    if (a.head_size == 128) return launch_decode_d<128, fp8_t>(a, stream);
    if (a.head_size == 64) return launch_decode_d<64, fp8_t>(a, stream);
  } else {
    if (a.head_size == 128) return launch_decode_d<128, half_t>(a, stream);
    if (a.head_size == 64) return launch_decode_d<64, half_t>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
