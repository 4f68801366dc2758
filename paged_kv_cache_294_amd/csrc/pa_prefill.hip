// Chunked prefill on gfx950 matrix cores: causal attention of a chunk of C query rows
// over the P tokens cached before it plus the chunk itself, all read from the paged pool
// through the request's block-table row. The scheduler on page "vLLM 部署深度指南"
// (continuous-batching listing) runs such prefills in the same step as decodes.
//
// Work split. One workgroup of four waves per (request, query head, 128-row tile of the
// chunk); each wave owns 32 query rows. Workgroups are issued heaviest first (requests in
// decreasing order of context length, ranked inside the kernel; later row tiles first),
// and all row tiles of one (request, head) go to the same XCD so they share its L2.
//
// Staging. The KV context is streamed in stages of 32 tokens (two 16-token blocks found
// through the table). Each stage's K and V rows go from HBM straight into LDS with
// global_load_lds_dwordx4 (a wave instruction fills 1 KB of LDS, 16 bytes per lane),
// through a ring of three stages, so loads run two stages ahead of the matrix cores
// without holding registers. Ring and registers (at most 168 VGPRs) are sized for three
// workgroups per CU at 128-dim heads, whose interleaving hides the softmax behind the
// other waves' products. Within each token row the 16-byte pieces are XOR-swizzled by
// the token index to spread the operand reads over the LDS banks.
//
// Contractions, both on v_mfma_f32_32x32x16_f16 (fp16 in, fp32 accumulate):
//   S^T[token][row] = K[token][:] . Q[row][:]   (A = K rows from LDS, B = Q rows in
//                                                registers: both in natural row-major order)
//   O^T[dim][row]  += V^T[dim][token] . P^T[token][row]
// A lane's S^T accumulator holds scores of one query row for 16 tokens of the stage; as
// fp16 they are exactly its B operand of the second product, so P never leaves registers.
// V^T comes from V kept in natural row-major order through the transposing LDS read
// (ds_read_b64_tr_b16): in each 16-lane group, source lane i addresses V[t0 + i/4][d0 +
// 4 (i%4)] and lane j receives V[t0 + k][d0 + j], k = 0..3.
//
// Softmax. Online, fp32, per query row, in log2 units: p = 2^(s * scale * log2(e) - m).
// The reference max m of a row moves only when a score exceeds it by more than 2^8, so
// the accumulator rescale is rare and fp16 P stays <= 256. Causal mask: chunk row i
// (position P + i) sees tokens 0 .. P + i; only stages crossing that diagonal or the end
// of the context are masked, and stages past every row of a wave are skipped by it.
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pkv {
namespace {

constexpr int kBM = 128;     // query rows per workgroup
constexpr int kWRows = 32;   // query rows per wave
constexpr int kBN = 32;      // tokens per stage
constexpr int kStages = 3;   // ring depth (48 KB of LDS at D = 128: three workgroups per CU)
constexpr int kThreads = 256;
constexpr int kXcds = 8;     // accelerator dies of an MI355X, each with its own L2
constexpr int kMaxRanked = 256;  // requests ranked by length; larger batches keep their order
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference max may lag the true max

// One K and one V load of a stage, 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane i reads block + koff (resp. voff) and its bytes land at
// LDS byte address kdst + 16 i (resp. vdst + 16 i). The LDS destination goes through M0,
// which the statement saves and restores. Written as inline assembly so the compiler adds
// none of its conservative waits for these loads before LDS reads; the kernel waits for
// them itself with wait_vm.
__device__ __forceinline__ void load_kv_lds16(const void* block, uint32_t koff, uint32_t voff,
                                              uint32_t kdst, uint32_t vdst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "s_mov_b32 m0, %4\n\t"
      "global_load_lds_dwordx4 %2, %5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(koff), "v"(voff), "s"(kdst), "s"(vdst), "s"(block)
      : "memory");
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(size_t)((__attribute__((address_space(3))) T*)p);
}

// An empty volatile asm statement: keeps a rarely taken branch a branch instead of letting
// the compiler run its body unconditionally behind selects.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier after this wave's LDS operations have completed. Unlike
// __syncthreads() it carries no memory fence, so staging loads still in flight (tracked by
// the explicit vmcnt waits) are not drained; the "memory" clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// XOR swizzles of the 16-byte pieces of a token row in LDS (results stay below D / 8)
template <int D>
__device__ __forceinline__ int kswz(int t) { return t & 7; }
template <int D>
__device__ __forceinline__ int vswz(int t) { return D >= 128 ? 4 * (t & 3) : 4 * (t & 1); }
// K rows of an FP8 cache: 16-byte pieces of E4M3 codes (D / 16 per row)
template <int D>
__device__ __forceinline__ int kswz8(int t) { return D >= 128 ? ((t >> 1) & 7) : ((t >> 2) & 3); }

template <int D, typename KV>
struct PrefillSmem {
  static constexpr int ROW = D;                 // elements per token row (no padding)
  static constexpr int TILE = kBN * ROW;        // elements per K (or V) stage
  KV k[kStages][TILE];
  KV v[kStages][TILE];
  // FP8 cache: the current stage's V widened to fp16, in the fp16 stage layout
  half_t v16[sizeof(KV) == 1 ? TILE : 8];
};

template <int D>
__device__ __forceinline__ void write_rows(const PrefillArgs& a, int q0, int row, int h,
                                           float value) {
  half_t* out = static_cast<half_t*>(a.out) + ((int64_t)(q0 + row) * a.num_q_heads + h) * D;
  for (int d = 0; d < D; ++d) out[d] = (half_t)value;
}

// The request with rank `rank` in decreasing seq_len order (ties by index). Every thread
// returns the same value.
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

template <int D, typename KV>
__global__ __launch_bounds__(kThreads, 3) void prefill_kernel(const PrefillArgs a) {
  constexpr bool kFp8 = sizeof(KV) == 1;  // E4M3 cache: codes staged, widened on reading
  constexpr int KS = D / 16;          // k-steps of S^T (16 dims each)
  constexpr int DT = D / 32;          // 32-dim tiles of O^T
  constexpr int PIECES = D * (int)sizeof(KV) / 16;  // 16-byte pieces per token row of one head
  constexpr int TOK_PER_INST = kWave / PIECES < 8 ? kWave / PIECES : 8;  // rows per wave load
  constexpr int LANES = TOK_PER_INST * PIECES;  // lanes of a load that move data (64 or 32)
  constexpr int INST = kBN / TOK_PER_INST / (kThreads / kWave);  // K (or V) loads per wave/stage
  static_assert(INST >= 1 && INST * TOK_PER_INST * (kThreads / kWave) == kBN, "stage split");
  using Smem = PrefillSmem<D, KV>;
  constexpr int ROW = Smem::ROW;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  __shared__ int s_req;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int g = lane >> 5;

  // Work item of this workgroup (see the header comment on XCDs and order)
  const int tiles = (a.max_q_len + kBM - 1) / kBM;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int group = (slot / tiles) * kXcds + xcd;
  if (group >= a.num_reqs * a.num_q_heads) return;  // padding of the grid (uniform per WG)
  const int h = group % a.num_q_heads;
  // uniform, so the request's lengths and table entries are read with scalar loads (a vector
  // load there would have to wait for every staging load in flight)
  const int r = __builtin_amdgcn_readfirstlane(request_of_rank(a, group / a.num_q_heads, &s_req));
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

  const int kv_end = min(S, P + min(i0 + kBM, C));               // tokens the workgroup sees
  const int wave_end = row_w < C ? P + min(row_w + kWRows, C) : 0;  // tokens this wave sees
  const int nst = (kv_end + kBN - 1) / kBN;                       // stages

  const int kv_row = a.num_kv_heads * D;
  const int tok_stride = 2 * kv_row;
  const uint64_t block_bytes = (uint64_t)kBlockSize * tok_stride * sizeof(KV);
  const char* pool = static_cast<const char*>(a.pool);
  const int32_t* bt = a.block_tables + (int64_t)r * a.max_blocks_per_seq;
  const int nblk = (S + kBlockSize - 1) / kBlockSize;

  // Loads of a stage. Wave w fills token rows 8 w .. 8 w + 7 of each stage, all in block
  // 2 st + w / 2 of the context; its load j covers rows tj .. tj + TOK_PER_INST - 1 (tj =
  // (w INST + j) TOK_PER_INST), lane l writing LDS slot l % PIECES of row tj + l / PIECES
  // and reading global piece slot ^ swizzle(row). Byte offsets inside the block:
  uint32_t koff[INST], voff[INST];
#pragma unroll
  for (int j = 0; j < INST; ++j) {
    const int t = (w * INST + j) * TOK_PER_INST + (lane % LANES) / PIECES;
    const int sl = lane % PIECES;
    const int ks = kFp8 ? kswz8<D>(t) : kswz<D>(t), vs = kFp8 ? 0 : vswz<D>(t);
    koff[j] = sizeof(KV) * ((t % kBlockSize) * tok_stride + kvh * D) + 16u * (sl ^ ks);
    voff[j] = sizeof(KV) * ((t % kBlockSize) * tok_stride + kv_row + kvh * D) + 16u * (sl ^ vs);
  }
  const uint32_t lds_k0 = lds_addr(&sm.k[0][0]) + sizeof(KV) * (w * INST * TOK_PER_INST * ROW);
  constexpr uint32_t kStageBytes = sizeof(KV) * Smem::TILE;
  constexpr uint32_t kVBytes = kStages * kStageBytes;  // from sm.k to sm.v
  constexpr uint32_t kInstBytes = sizeof(KV) * TOK_PER_INST * ROW;

  // Table entries of this wave's block in each stage, one stage per lane: register v of
  // chunk c holds, in lane L, the entry for stage 64 (kTabRegs c + v) + L. Each lane also
  // checks the entries of both blocks of its stage (uniform outcome across the waves): an
  // entry of the context outside the pool makes the tile's rows NaN.
  constexpr int kTabRegs = 2;
  int tab[kTabRegs];
  int bad_lanes = 0;
  auto load_table = [&](int chunk) {
#pragma unroll
    for (int v = 0; v < kTabRegs; ++v) {
      const int sidx = 64 * (kTabRegs * chunk + v) + lane;
      int own = 0;
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int e = 2 * sidx + par;
        const int x = bt[min(e, nblk - 1)];
        const bool out_of_pool = x < 0 || x >= a.num_blocks;
        bad_lanes |= (sidx < nst && e < nblk && out_of_pool);
        if (par == (w >> 1)) own = out_of_pool ? 0 : x;
      }
      tab[v] = own;
    }
  };
  auto issue_stage = [&](int st, int ring) {
    if (st > 0 && st % (64 * kTabRegs) == 0) load_table(st / (64 * kTabRegs));  // uniform
    const int v = (st >> 6) % kTabRegs;
    int cand = tab[0];
#pragma unroll
    for (int u = 1; u < kTabRegs; ++u) cand = (v == u) ? tab[u] : cand;
    const int phys = __builtin_amdgcn_readlane(cand, st & 63);
    const char* block = pool + (uint64_t)phys * block_bytes;
    const uint32_t kdst = lds_k0 + (uint32_t)ring * kStageBytes;  // ring == st % kStages
#pragma unroll
    for (int j = 0; j < INST; ++j)
      if (LANES == kWave || lane < LANES)  // 64-dim FP8 rows fill half a wave per load
        load_kv_lds16(block, koff[j], voff[j], kdst + j * kInstBytes, kdst + kVBytes + j * kInstBytes);
  };

  const float c2 = a.scale_log2;
  float m = neg_inf(), l = 0.0f;
  float16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = float16_t{};

  // K operand row of this lane: token lane % 32 of the stage
  const int krow = lane & 31;
  // V^T operand: transposing reads of 4 tokens x 16 dims per 16-lane group
  const int li = lane & 15;         // source lane inside the 16-lane group
  const int dh = (lane >> 4) & 1;   // which 16 dims of the 32-dim tile
  const int vtok = 4 * g + li / 4;  // token (within a 16-token k-step half) of this source lane

  load_table(0);
  for (int st = 0; st < kStages - 1 && st < nst; ++st) issue_stage(st, st);
  // the query rows come in behind the first stages, and one wait covers both: the compiler
  // then knows of no load in flight inside the loop and leaves the waiting to the loop's
  // own counted waits
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qrow < C)
      qb[ks] = load16(qp + ((int64_t)(q0 + qrow) * a.num_q_heads + h) * D + 16 * ks + 8 * g);
    else
      qb[ks] = half8_t{};
  }
  wait_vm<0>();

  // One stage of the context. The ring slot is a compile-time constant (the loop below is
  // unrolled by the ring depth), so every LDS address of the stage is a per-lane base plus
  // an immediate offset.
  auto stage = [&](auto ring_c, const int it) {
    constexpr int ring = decltype(ring_c)::value;
    constexpr int kRing = ring;

    // this wave's loads of stage `it` have landed once at most the loads of the stages
    // issued after it are outstanding; the barrier makes every wave's loads visible and
    // frees ring slot (it - 1) % kStages for stage it + kStages - 1
    if (it + 1 < nst) wait_vm<2 * INST>();
    else wait_vm<0>();
    lds_barrier();
    const int t0 = it * kBN;
    if constexpr (kFp8) {
      // widen the stage's V codes to fp16 in the layout the transposing reads expect; rows
      // past the context's end become zeros (their slots may hold anything, and 0 * NaN
      // would reach the output). The previous stage's readers are past the barrier above.
      for (int e = tid; e < kBN * PIECES; e += kThreads) {
        const int t = e / PIECES, pc = e % PIECES;  // 16 codes: dims 16 pc .. 16 pc + 15
        half8_t lo = half8_t{}, hi = half8_t{};
        if (t0 + t < S) {
          const u32x2_t* src = reinterpret_cast<const u32x2_t*>(&sm.v[ring][t * ROW + 16 * pc]);
          lo = widen_fp8x8(src[0]);
          hi = widen_fp8x8(src[1]);
        }
        *reinterpret_cast<half8_t*>(&sm.v16[t * ROW + 8 * ((2 * pc) ^ vswz<D>(t))]) = lo;
        *reinterpret_cast<half8_t*>(&sm.v16[t * ROW + 8 * ((2 * pc + 1) ^ vswz<D>(t))]) = hi;
      }
      lds_barrier();
    } else if (__builtin_amdgcn_readfirstlane(t0 + kBN > S)) {
      // the context's last stage: V rows past the end become zeros (their slots may hold
      // anything, and 0 * NaN would reach the output)
      keep_branch();
      for (int e = tid; e < kBN * PIECES; e += kThreads) {
        const int t = e / PIECES;
        if (t0 + t >= S) *reinterpret_cast<half8_t*>(&sm.v[ring][t * ROW + 8 * (e % PIECES)]) = half8_t{};
      }
      lds_barrier();
    }
    if (it + kStages - 1 < nst) issue_stage(it + kStages - 1, (kRing + kStages - 1) % kStages);

    if (t0 < wave_end) {
      // S^T for the stage's 32 tokens
      half8_t ka[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (kFp8)
          ka[ks] = widen_fp8x8(*reinterpret_cast<const u32x2_t*>(
              &sm.k[ring][krow * ROW + 16 * (ks ^ kswz8<D>(krow)) + 8 * g]));
        else
          ka[ks] = *reinterpret_cast<const half8_t*>(
              &sm.k[ring][krow * ROW + 8 * ((2 * ks + g) ^ kswz<D>(krow))]);
      }
      float16_t sacc = float16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks], qb[ks], sacc, 0, 0, 0);

      // mask the diagonal / context-end stage: token t visible iff t <= min(S-1, P+qrow)
      const int diag = __builtin_amdgcn_readfirstlane(!((t0 + kBN <= P + row_w + 1) && (t0 + kBN <= S)));
      if (diag) {
        keep_branch();
        const int lim = min(S - 1, P + qrow) - (t0 + 4 * g);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (8 * (v >> 2) + (v & 3) > lim) sacc[v] = neg_inf();
      }
      float mraw = neg_inf();
#pragma unroll
      for (int v = 0; v < 16; ++v) mraw = fmaxf(mraw, sacc[v]);
      const float ms = mraw * c2;  // c2 > 0; -inf stays -inf
      // lanes l and l ^ 32 hold the same row's scores for different tokens: a row's max
      // moves iff one of its halves' maxima does, and only then do the halves exchange
      // them (so both keep the same reference max)
      if (__builtin_amdgcn_ballot_w64(ms > m + kRescaleSlack)) {
        keep_branch();
        const float mrow = fmaxf(ms, __shfl_xor(ms, 32, kWave));
        const float mnew = mrow > m + kRescaleSlack ? mrow : m;
        const float alpha = fast_exp2(m - mnew);  // 0 when m was -inf, 1 when not moved
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        m = mnew;
      }
      const float base = (m == neg_inf()) ? 0.0f : m;
      half8_t pb[2];
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[k][e] = (half_t)fast_exp2(fmaf(sacc[8 * k + e], c2, -base));
      // the row sum of exactly the fp16 values the PV product uses (products exact, fp32 sum)
      float lsum = 0.0f;
      const half2_t ones = {(half_t)1.0f, (half_t)1.0f};
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          lsum = __builtin_amdgcn_fdot2(half2_t{pb[k][e], pb[k][e + 1]}, ones, lsum, false);
      l += lsum;  // this half's tokens; the halves are added at the end

      // O^T += V^T P^T: k-step k covers stage tokens 16k .. 16k+15; the lane's 8 k-slots
      // are tokens 16k + 4g + {0..3} (first read) and 16k + 8 + 4g + {0..3} (second)
      half8_t va[2][DT];
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int t = 16 * k + 8 * hh + vtok;
            const int dim = 32 * dt + 16 * dh + 4 * (li % 4);
            const int piece = (dim / 8) ^ vswz<D>(t);
            const half_t* vsrc = kFp8 ? &sm.v16[0] : reinterpret_cast<const half_t*>(&sm.v[ring][0]);
            const short4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4_t*)(vsrc + t * ROW + 8 * piece + (dim & 4)));
            const half4_t y = __builtin_bit_cast(half4_t, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) va[k][dt][4 * hh + e] = y[e];
          }
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[k][dt], pb[k], o[dt], 0, 0, 0);
    }
    };
  using R0 = std::integral_constant<int, 0>;
  using R1 = std::integral_constant<int, 1>;
  using R2 = std::integral_constant<int, 2>;
  static_assert(kStages == 3, "the stage loop is unrolled by a ring of three");
  int it = 0;
  for (; it + 3 <= nst; it += 3) {
    stage(R0{}, it);
    stage(R1{}, it + 1);
    stage(R2{}, it + 2);
  }
  if (it < nst) stage(R0{}, it++);
  if (it < nst) stage(R1{}, it++);

  l += __shfl_xor(l, 32, kWave);
  const bool bad_table = __builtin_amdgcn_ballot_w64(bad_lanes) != 0;
  if (qrow >= C) return;
  half_t* out = static_cast<half_t*>(a.out) + ((int64_t)(q0 + qrow) * a.num_q_heads + h) * D;
  const float inv = bad_table ? qnan() : a.v_scale / l;
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

template <int D, typename KV>
hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t stream) {
  const size_t smem = sizeof(PrefillSmem<D, KV>);
  static bool attr_set = false;  // the attribute is per function, set once per process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, KV>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t groups = (int64_t)a.num_reqs * a.num_q_heads;
  const int64_t tiles = (a.max_q_len + kBM - 1) / kBM;
  const int64_t wgs = (groups + kXcds - 1) / kXcds * kXcds * tiles;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<D, KV>), dim3((unsigned)wgs), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.kv_fp8) {
    if (a.head_size == 128) return launch_prefill_d<128, fp8_t>(a, stream);
    if (a.head_size == 64) return launch_prefill_d<64, fp8_t>(a, stream);
  } else {
    if (a.head_size == 128) return launch_prefill_d<128, half_t>(a, stream);
    if (a.head_size == 64) return launch_prefill_d<64, half_t>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
