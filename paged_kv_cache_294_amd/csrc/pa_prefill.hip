// Chunked prefill on gfx950 matrix cores: causal attention of a chunk of C query rows
// over the P tokens cached before it plus the chunk itself, all read from the paged pool
// through the request's block-table row. The scheduler on page "vLLM 部署深度指南"
// (continuous-batching listing) runs such prefills in the same step as decodes.
//
// Work split. One workgroup of four waves per (request, query head, 128-row tile of the
// chunk); each wave owns 32 query rows. The KV context is streamed in tiles of 64
// tokens (four 16-token blocks found through the table) and staged in LDS, double
// buffered, shared by the four waves. Workgroups are issued heaviest first: requests
// in decreasing order of context length (ranked inside the kernel), and within a
// request the later row tiles (which see more tokens) first.
//
// Contractions, both on v_mfma_f32_32x32x16_f16 (fp16 in, fp32 accumulate):
//   S^T[token][row] = K[token][:] . Q[row][:]   (A = K rows from LDS, B = Q rows in
//                                                registers: both in natural row-major order)
//   O^T[dim][row]  += V^T[dim][token] . P^T[token][row]
// The S^T accumulator holds, in each lane, scores of one query row for 16 tokens of a
// 32-token tile; converted to fp16 they are exactly the B operand of the second product,
// so P never leaves registers. V is transposed once per tile while it is written to LDS;
// its token order inside each 16-token group is permuted so that the 8 tokens a lane
// feeds to one product sit next to each other (one 16-byte LDS read per operand).
//
// Softmax. Online, fp32, per query row, in log2 units: p = 2^(s * scale * log2(e) - m).
// The reference max m of a row moves only when a score exceeds it by more than 2^8, so
// the accumulator rescale is rare and fp16 P stays <= 256. Causal mask: chunk row i
// (position P + i) sees tokens 0 .. P + i; only tiles crossing that diagonal or the end
// of the context are masked, and tiles past every row of a wave are skipped by it.
#include "pa_device.h"
#include "pa_launch.h"

namespace pkv {
namespace {

constexpr int kBM = 128;     // query rows per workgroup
constexpr int kWRows = 32;   // query rows per wave
constexpr int kBN = 64;      // tokens per KV tile
constexpr int kTileBlocks = kBN / kBlockSize;
constexpr int kThreads = 256;
constexpr int kXcds = 8;     // accelerator dies of an MI355X, each with its own L2
constexpr int kMaxRanked = 256;  // requests ranked by length; larger batches keep their order
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference max may lag the true max
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// An empty volatile asm statement: keeps a rarely taken branch a branch instead of letting
// the compiler run its body unconditionally behind selects.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

__device__ __forceinline__ int vt_pos(int t) {
  // token order inside a 16-token group: 0-3, 8-11, 4-7, 12-15
  const int u = t & 15;
  return (t & ~15) | (u & 3) | ((u & 4) << 1) | ((u & 8) >> 1);
}

template <int D>
struct PrefillSmem {
  static constexpr int KP = D + 8;     // K row pitch (halves)
  static constexpr int VP = kBN + 8;   // V^T row pitch (halves)
  half_t k[2][kBN * KP];
  half_t vt[2][D * VP];
};

template <int D>
__device__ __forceinline__ void write_rows(const PrefillArgs& a, int q0, int row, int h,
                                           float value) {
  half_t* out = static_cast<half_t*>(a.out) + ((int64_t)(q0 + row) * a.num_q_heads + h) * D;
  for (int d = 0; d < D; ++d) out[d] = (half_t)value;
}

// The request this workgroup serves: rank blockIdx.z in decreasing seq_len order (ties by
// index). Every thread returns the same value.
__device__ int request_of_rank(const PrefillArgs& a, int rank, int* slot) {
  if (a.num_reqs > kMaxRanked) return rank;
  if (threadIdx.x == 0) *slot = rank;
  __syncthreads();
  for (int r = threadIdx.x; r < a.num_reqs; r += kThreads) {
    const int sr = a.seq_lens[r];
    int k = 0;
    for (int u = 0; u < a.num_reqs; ++u) {
      const int su = a.seq_lens[u];
      k += (su > sr) || (su == sr && u < r);
    }
    if (k == rank) *slot = r;
  }
  __syncthreads();
  return *slot;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(const PrefillArgs a) {
  constexpr int KS = D / 16;          // k-steps of S^T (16 dims each)
  constexpr int DT = D / 32;          // 32-dim tiles of O^T
  constexpr int PIECES = D / 8;       // 16-byte pieces per K (or V) row of one head
  constexpr int K_PER_THREAD = kBN * PIECES / kThreads;
  constexpr int V_ROUNDS = PIECES / 8;  // each round: 32 token pairs x 8 pieces
  using Smem = PrefillSmem<D>;
  constexpr int KP = Smem::KP, VP = Smem::VP;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  __shared__ int s_req;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int g = lane >> 5;
  // Work item of this workgroup. Workgroups go to the 8 XCDs round-robin in launch order
  // (workgroup i to XCD i % 8), each XCD with its own L2. All row tiles of one (request,
  // head) share its K/V, so they are given to the same XCD; (request, head) groups are
  // dealt to the XCDs in heaviest-first order and each group's later row tiles go first.
  const int tiles = (a.max_q_len + kBM - 1) / kBM;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int group = (slot / tiles) * kXcds + xcd;
  if (group >= a.num_reqs * a.num_q_heads) return;  // padding of the grid (uniform per WG)
  const int h = group % a.num_q_heads;
  const int r = request_of_rank(a, group / a.num_q_heads, &s_req);
  const int i0 = (tiles - 1 - slot % tiles) * kBM;
  const int kvh = h / (a.num_q_heads / a.num_kv_heads);

  const int q0 = a.query_start_loc[r];
  const int q1 = a.query_start_loc[r + 1];
  const int C = q1 - q0;
  const int S = a.seq_lens[r];
  const int P = S - C;
  const bool rows_ok = q0 >= 0 && q1 >= q0 && q1 <= a.total_q;
  const bool bad = !rows_ok || C > a.max_q_len || S < C || S > a.max_seq_len ||
                   S > a.max_blocks_per_seq * kBlockSize;
  if (bad) {
    if (rows_ok)
      for (int i = i0 + tid; i < min(i0 + kBM, C); i += kThreads) write_rows<D>(a, q0, i, h, qnan());
    return;
  }
  if (i0 >= C) return;

  // ---- this wave's query rows: B operand of S^T, 8 dims of row (lane % 32) per k-step --
  const int row_w = i0 + kWRows * w;
  const int qrow = row_w + (lane & 31);
  const half_t* qp = static_cast<const half_t*>(a.q);
  half8_t qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qrow < C)
      qb[ks] = load16(qp + ((int64_t)(q0 + qrow) * a.num_q_heads + h) * D + 16 * ks + 8 * g);
    else
      qb[ks] = half8_t{};
  }

  const int kv_end = min(S, P + min(i0 + kBM, C));               // tokens the workgroup sees
  const int wave_end = row_w < C ? P + min(row_w + kWRows, C) : 0;  // tokens this wave sees
  const int ntiles = (kv_end + kBN - 1) / kBN;

  const int kv_row = a.num_kv_heads * D;
  const int tok_stride = 2 * kv_row;
  const int64_t block_elems = (int64_t)kBlockSize * tok_stride;
  const half_t* pool = static_cast<const half_t*>(a.pool);
  const int32_t* bt = a.block_tables + (int64_t)r * a.max_blocks_per_seq;
  const int nblk = (S + kBlockSize - 1) / kBlockSize;
  int bad_table = 0;  // uniform: set when a table entry of the context lies outside the pool

  // Staging assignment, fixed for every tile. K piece j of this thread: token
  // kt[j] = tid / PIECES + j * (256 / PIECES) of the tile, 16-byte piece tid % PIECES.
  // V: token pair (2 * (tid % 32), +1), piece tid / 32 + 8 * round.
  int koff[K_PER_THREAD], voff[V_ROUNDS][2];
#pragma unroll
  for (int j = 0; j < K_PER_THREAD; ++j) {
    const int t = tid / PIECES + j * (kThreads / PIECES);
    koff[j] = (t % kBlockSize) * tok_stride + kvh * D + 8 * (tid % PIECES);
  }
#pragma unroll
  for (int rd = 0; rd < V_ROUNDS; ++rd)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int t = 2 * (tid & 31) + e;
      voff[rd][e] = (t % kBlockSize) * tok_stride + kv_row + kvh * D + 8 * (tid / 32 + 8 * rd);
    }
  const int vblk = (2 * (tid & 31)) / kBlockSize;  // block (in the tile) of this thread's V pair

  struct Stage {
    half8_t k[K_PER_THREAD];
    half8_t v[V_ROUNDS][2];
  };
  Stage st;  // the next tile, loaded while the current one is computed

  // Loads are unconditional (a block outside the table or the pool reads block 0, which
  // exists), so the loaded registers flow straight into the LDS store after the compute;
  // tokens past the context end are zeroed at store time.
  int st_t0 = 0;  // first token of the staged tile
  auto load_tile = [&](int t0, Stage& st) {
    const half_t* base[kTileBlocks];
#pragma unroll
    for (int jb = 0; jb < kTileBlocks; ++jb) {
      const int blk = t0 / kBlockSize + jb;
      int phys = __builtin_amdgcn_readfirstlane(blk < nblk ? bt[blk] : 0);
      const int out_of_pool = phys < 0 || phys >= a.num_blocks;
      bad_table |= out_of_pool & (blk < nblk);
      phys = out_of_pool ? 0 : phys;
      base[jb] = pool + (int64_t)phys * block_elems;
    }
    bad_table = __builtin_amdgcn_readfirstlane(bad_table);
    st_t0 = t0;
#pragma unroll
    for (int j = 0; j < K_PER_THREAD; ++j)
      st.k[j] = load16(base[(tid / PIECES + j * (kThreads / PIECES)) / kBlockSize] + koff[j]);
#pragma unroll
    for (int rd = 0; rd < V_ROUNDS; ++rd)
#pragma unroll
      for (int e = 0; e < 2; ++e) st.v[rd][e] = load16(base[vblk] + voff[rd][e]);
  };

  auto store_tile = [&](Stage& st, int buf) {
    if (__builtin_amdgcn_readfirstlane(st_t0 + kBN > S || bad_table)) {
      // the context's last tile (or a bad table): tokens past the end become zeros
      keep_branch();
#pragma unroll
      for (int j = 0; j < K_PER_THREAD; ++j) {
        const int t = tid / PIECES + j * (kThreads / PIECES);
        if (st_t0 + t >= S || bad_table) st.k[j] = half8_t{};
      }
#pragma unroll
      for (int rd = 0; rd < V_ROUNDS; ++rd)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (st_t0 + 2 * (tid & 31) + e >= S || bad_table) st.v[rd][e] = half8_t{};
    }
#pragma unroll
    for (int j = 0; j < K_PER_THREAD; ++j) {
      const int t = tid / PIECES + j * (kThreads / PIECES);
      *reinterpret_cast<half8_t*>(&sm.k[buf][t * KP + 8 * (tid % PIECES)]) = st.k[j];
    }
#pragma unroll
    for (int rd = 0; rd < V_ROUNDS; ++rd) {
      const int c = tid / 32 + 8 * rd;
      const int pos = vt_pos(2 * (tid & 31));  // even; the pair's second token follows it
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        half2_t pr = {st.v[rd][0][i], st.v[rd][1][i]};
        *reinterpret_cast<half2_t*>(&sm.vt[buf][(8 * c + i) * VP + pos]) = pr;
      }
    }
  };

  const float c2 = a.scale_log2;
  float m = neg_inf(), l = 0.0f;
  float16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = float16_t{};

  // tile `it` is computed from LDS buffer it & 1 while tile it + 1 is loaded into
  // registers; it is written to the other buffer after the compute
  load_tile(0, st);
  store_tile(st, 0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int t0 = it * kBN;
    const bool has_next = it + 1 < ntiles;
    if (has_next) load_tile(t0 + kBN, st);

    if (t0 < wave_end) {
      // Per 32-token half h of the tile: S_h = S^T chain, then the softmax state update
      // and P_h = exp2(...) in fp16, then O^T += V^T_h P_h. The exps of one half are
      // interleaved with the MFMA chain of the next (S_1 or PV_0) so the matrix cores
      // keep working while the vector ALUs do the softmax.
      const int diag = __builtin_amdgcn_readfirstlane(!((t0 + kBN <= P + row_w + 1) && (t0 + kBN <= S)));
      const int lim = min(S - 1, P + qrow) - (t0 + 4 * g);  // last visible token, tile-relative
      half8_t ka[2][KS];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[tt][ks] = *reinterpret_cast<const half8_t*>(
              &sm.k[buf][(32 * tt + (lane & 31)) * KP + 16 * ks + 8 * g]);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * KS, 0);
      float16_t sacc[2];
      sacc[0] = float16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[0][ks], qb[ks], sacc[0], 0, 0, 0);

      // softmax state update of half tt: mask, row max, lazy rescale; returns the exp base
      auto update = [&](int tt) -> float {
        if (diag) {
          keep_branch();
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (32 * tt + 8 * (v >> 2) + (v & 3) > lim) sacc[tt][v] = neg_inf();
        }
        float mraw = neg_inf();
#pragma unroll
        for (int v = 0; v < 16; ++v) mraw = fmaxf(mraw, sacc[tt][v]);
        mraw = fmaxf(mraw, __shfl_xor(mraw, 32, kWave));
        const float mh = mraw * c2;  // c2 > 0; -inf stays -inf
        // move the reference max only when this half beats it by more than the slack
        const bool move = mh > m + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(move)) {
          keep_branch();
          const float mnew = move ? mh : m;
          const float alpha = fast_exp2(m - mnew);  // 0 when m was -inf, 1 when not moved
          l *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
          m = mnew;
        }
        return (m == neg_inf()) ? 0.0f : m;
      };
      // P of half tt as the fp16 B operands of two PV k-steps; adds its row sum to l
      auto probs = [&](int tt, float base, half8_t* pb) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pb[k][e] = (half_t)fast_exp2(fmaf(sacc[tt][8 * k + e], c2, -base));
        float lsum = 0.0f;
        const half2_t ones = {(half_t)1.0f, (half_t)1.0f};
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            lsum = __builtin_amdgcn_fdot2(half2_t{pb[k][e], pb[k][e + 1]}, ones, lsum, false);
        lsum += __shfl_xor(lsum, 32, kWave);
        l += lsum;
      };
      auto pv = [&](int tt, const half8_t* pb) {
        half8_t va[2][DT];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            va[k][dt] = *reinterpret_cast<const half8_t*>(
                &sm.vt[buf][(32 * dt + (lane & 31)) * VP + 16 * (2 * tt + k) + 8 * g]);
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[k][dt], pb[k], o[dt], 0, 0, 0);
      };

      half8_t pb0[2], pb1[2];
      const float base0 = update(0);
      // S_1 chain, interleaved with the exps of half 0
      sacc[1] = float16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[1][ks], qb[ks], sacc[1], 0, 0, 0);
      probs(0, base0, pb0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 1);
      }
      const float base1 = update(1);
      // PV of half 0, interleaved with the exps of half 1
      pv(0, pb0);
      probs(1, base1, pb1);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * DT, 2);
#pragma unroll
      for (int k = 0; k < 2 * DT; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 2);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 2);
      }
      pv(1, pb1);
    }

    if (has_next) store_tile(st, buf ^ 1);
    __syncthreads();
  }

  if (qrow >= C) return;
  half_t* out = static_cast<half_t*>(a.out) + ((int64_t)(q0 + qrow) * a.num_q_heads + h) * D;
  const float inv = bad_table ? qnan() : 1.0f / l;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      half4_t x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (half_t)(o[dt][4 * v4 + e] * inv);
      *reinterpret_cast<half4_t*>(out + 32 * dt + 8 * v4 + 4 * g) = x;
    }
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t stream) {
  const size_t smem = sizeof(PrefillSmem<D>);
  static bool attr_set = false;  // the attribute is per function, set once per process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t groups = (int64_t)a.num_reqs * a.num_q_heads;
  const int64_t tiles = (a.max_q_len + kBM - 1) / kBM;
  const int64_t wgs = (groups + kXcds - 1) / kXcds * kXcds * tiles;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<D>), dim3((unsigned)wgs), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.head_size == 128) return launch_prefill_d<128>(a, stream);
  if (a.head_size == 64) return launch_prefill_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
