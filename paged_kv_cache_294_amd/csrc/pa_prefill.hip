// Chunked prefill on gfx950 matrix cores: causal attention of a chunk of C query rows
// over the P tokens cached before it plus the chunk itself, all read from the paged pool
// through the request's block-table row. The scheduler on page "vLLM 部署深度指南"
// (continuous-batching listing) runs such prefills in the same step as decodes.
//
// Work split. One workgroup of four waves per (request, query head, 128-row tile of the
// chunk); each wave owns 32 query rows. Workgroups are issued heaviest first (requests in
// decreasing order of context length, ranked inside the kernel; later row tiles first),
// and all row tiles of one (request, head) go to the same XCD so they share its L2.
// A launch whose tiles cannot fill the GPU may also cut each request's context into
// pieces (the context split below), one workgroup per (piece, head, tile), merged by a
// second kernel.
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
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pkv {
namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

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

// Lengths of request r and whether they are within the call's bounds.
struct Request {
  int q0, C, S, P;
  bool rows_ok;  // its query rows lie inside [0, total_q)
  bool bad;      // rows or lengths break the bounds: its rows become NaN
};

__device__ __forceinline__ Request load_request(const PrefillArgs& a, int r) {
  Request q;
  q.q0 = a.query_start_loc[r];
  const int q1 = a.query_start_loc[r + 1];
  q.C = q1 - q.q0;
  q.S = a.seq_lens[r];
  q.P = q.S - q.C;
  q.rows_ok = q.q0 >= 0 && q1 >= q.q0 && q1 <= a.total_q;
  q.bad = !q.rows_ok || q.C > a.max_q_len || q.S < q.C || q.S > a.max_seq_len ||
          q.S > a.max_blocks_per_seq * kBlockSize;
  return q;
}

// Stages of the context that the row tile starting at chunk row i0 sees: every token up
// to the tile's last row.
__device__ __forceinline__ int tile_stages(const Request& q, int i0) {
  return (min(q.S, q.P + min(i0 + kBM, q.C)) + kBN - 1) / kBN;
}

// Context split. A request whose context is long next to the launch's average load per
// resident workgroup has it cut into n equal pieces of L whole stages (the last piece
// shorter), the same cut for all its row tiles and heads; a tile that sees more than L
// stages is run piece by piece by separate workgroups and merged afterwards by
// log-sum-exp. Work is then issued by piece weight (the stages its heaviest tile runs),
// heaviest first, so that the last workgroups to start are light ones.
constexpr int kMaxPieces = 16;       // pieces per request at most
constexpr int kMinPieceStages = 16;  // a piece covers at least 512 tokens
constexpr int kCapNum = 4, kCapDen = 5;  // piece cap: 4/5 of the load per resident workgroup

// The request with rank `rank` in decreasing seq_len order (ties by index), for launches
// without a split. Every thread returns the same value.
__device__ int request_of_rank(const PrefillArgs& a, int rank, int* slot) {
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

struct PlanSmem {
  int nst[kMaxRanked];  // stages of the request's context (0 when it breaks the bounds)
  int n[kMaxRanked];    // pieces
  int L[kMaxRanked];    // stages per piece
  unsigned long long total;  // stages over all requests and row tiles (one head)
  int sel;              // picked (request, piece) as request * kMaxPieces + piece, or -1
};

// Fills the plan of every request (num_reqs <= kMaxRanked). Every thread of the workgroup
// takes part; the same plan comes out in every workgroup of a launch.
__device__ void make_plan(const PrefillArgs& a, PlanSmem& sp) {
  const int tid = threadIdx.x;
  if (tid == 0) sp.total = 0;
  __syncthreads();
  unsigned long long work = 0;
  for (int r = tid; r < a.num_reqs; r += kThreads) {
    const Request q = load_request(a, r);
    int nst = 0;
    if (!q.bad) {
      nst = (q.S + kBN - 1) / kBN;
      if (a.max_pieces > 1)
        for (int i0 = 0; i0 < q.C; i0 += kBM) work += (unsigned long long)tile_stages(q, i0);
    }
    sp.nst[r] = nst;
  }
  if (a.max_pieces > 1 && work) atomicAdd(&sp.total, work);
  __syncthreads();
  int cap = INT32_MAX;  // no split with one piece per request
  if (a.max_pieces > 1) {  // then slots >= 1
    const unsigned long long den = (unsigned long long)max(a.slots, 1) * kCapDen;
    const unsigned long long c = (sp.total * (unsigned long long)a.num_q_heads * kCapNum + den - 1) / den;
    cap = (int)max((unsigned long long)kMinPieceStages, min(c, (unsigned long long)INT32_MAX));
  }
  for (int r = tid; r < a.num_reqs; r += kThreads) {
    const int nst = sp.nst[r];
    const int n = nst == 0 ? 1 : min(a.max_pieces, (nst - 1) / cap + 1);
    sp.n[r] = n;
    sp.L[r] = (nst + n - 1) / n;
  }
  __syncthreads();
}

// Weight of piece p of a request cut into n pieces of L stages out of nst
__device__ __forceinline__ int piece_weight(int nst, int n, int L, int p) {
  return p < n - 1 ? L : nst - (n - 1) * L;
}

// The (request, piece) of rank k in decreasing piece weight (ties by request, then piece),
// as request * kMaxPieces + piece, or -1 past the last piece. Every thread returns it.
__device__ int piece_of_rank(const PrefillArgs& a, PlanSmem& sp, int k) {
  const int tid = threadIdx.x;
  if (tid == 0) sp.sel = -1;
  __syncthreads();
  const int R = a.num_reqs;
  for (int r = tid; r < R; r += kThreads) {
    const int n = sp.n[r], L = sp.L[r], nst = sp.nst[r];
    for (int p = 0; p < n; ++p) {
      const int wt = piece_weight(nst, n, L, p);
      int rank = 0;
      for (int u = 0; u < R; ++u) {
        const int nu = sp.n[u], Lu = sp.L[u];
        const int wl = piece_weight(sp.nst[u], nu, Lu, nu - 1);
        if (u < r) {
          rank += (Lu >= wt) * (nu - 1) + (wl >= wt);
        } else if (u > r) {
          rank += (Lu > wt) * (nu - 1) + (wl > wt);
        } else {
          for (int q = 0; q < nu; ++q) {
            const int wq = piece_weight(nst, nu, Lu, q);
            rank += q < p ? (wq >= wt) : q > p ? (wq > wt) : 0;
          }
        }
      }
      if (rank == k) sp.sel = r * kMaxPieces + p;
    }
  }
  __syncthreads();
  return sp.sel;
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
  __shared__ PlanSmem sp;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int g = lane >> 5;

  // Work item of this workgroup (see the header comment on XCDs and order): group k * Hq +
  // h is piece rank k of query head h
  const int tiles = (a.max_q_len + kBM - 1) / kBM;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int group = (slot / tiles) * kXcds + xcd;
  if (group >= a.num_reqs * a.max_pieces * a.num_q_heads) return;  // grid padding (uniform)
  const int h = group % a.num_q_heads;
  const int k = group / a.num_q_heads;
  // uniform, so the request's lengths and table entries are read with scalar loads (a vector
  // load there would have to wait for every staging load in flight)
  int r, p = 0, L = INT32_MAX;
  if (a.max_pieces == 1) {  // no split: requests by length (launch order above kMaxRanked)
    r = a.num_reqs <= kMaxRanked ? __builtin_amdgcn_readfirstlane(request_of_rank(a, k, &sp.sel)) : k;
  } else {  // the host splits only batches of at most kMaxRanked requests
    make_plan(a, sp);
    const int sel = __builtin_amdgcn_readfirstlane(piece_of_rank(a, sp, k));
    if (sel < 0) return;  // past the last piece
    r = sel / kMaxPieces;
    p = sel % kMaxPieces;
    L = __builtin_amdgcn_readfirstlane(sp.L[r]);
  }
  const int i0 = (tiles - 1 - slot % tiles) * kBM;
  const int kvh = h / (a.num_q_heads / a.num_kv_heads);

  const Request rq = load_request(a, r);
  const int q0 = rq.q0, C = rq.C, S = rq.S, P = rq.P;
  if (rq.bad) {
    if (rq.rows_ok && p == 0)
      for (int i = i0 + tid; i < min(i0 + kBM, C); i += kThreads) write_rows<D>(a, q0, i, h, qnan());
    return;
  }
  if (i0 >= C) return;

  // ---- this wave's query rows: B operand of S^T, 8 dims of row (lane % 32) per k-step --
  const int row_w = i0 + kWRows * w;
  const int qrow = row_w + (lane & 31);
  const half_t* qp = static_cast<const half_t*>(a.q);
  half8_t qb[KS];

  const int wave_end = row_w < C ? P + min(row_w + kWRows, C) : 0;  // tokens this wave sees
  const int nst = tile_stages(rq, i0);                            // stages the tile sees
  // this workgroup's piece: stages s0 .. s1 - 1; a tile seeing more than L stages is split
  const int s0 = p * L;
  if (s0 >= nst) return;  // the tile ends before this piece
  const int s1 = min(nst, s0 + L);
  const bool split = nst > L;
  // Where this wave's results go, fixed before the stage loop so that one pointer stays live
  // across it: the fp16 output rows of the wave, or (split tile) the wave's part of the
  // piece's partial slot, (m, l) at the same slot index of the second region.
  const int64_t pslot = (((int64_t)r * a.num_q_heads + h) * tiles + i0 / kBM) * a.max_pieces + p;
  char* const dst = split ? reinterpret_cast<char*>(a.ws_o + pslot * (kBM * D) + w * (kWRows * D))
                          : reinterpret_cast<char*>(static_cast<half_t*>(a.out) +
                                                    ((int64_t)(q0 + row_w) * a.num_q_heads + h) * D);
  const int rows_left = C - row_w;  // rows of the wave inside the chunk (may be <= 0)

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
    if (st > s0 && st % (64 * kTabRegs) == 0) load_table(st / (64 * kTabRegs));  // uniform
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

  load_table(s0 / (64 * kTabRegs));
  for (int st = s0; st < s0 + kStages - 1 && st < s1; ++st) issue_stage(st, st - s0);
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
    if (it + 1 < s1) wait_vm<2 * INST>();
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
    } else if (t0 + kBN > S) {  // uniform
      // the context's last stage: V rows past the end become zeros (their slots may hold
      // anything, and 0 * NaN would reach the output). The zero and the thread index are
      // made here, behind volatile statements, so that the compiler keeps no address or
      // zero vector of this rare path in registers across the stage loop.
      keep_branch();
      int e0 = tid, z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z) : "v"(e0));
      asm volatile("" : "+v"(e0));
      const u32x4_t zero = {(uint32_t)z, (uint32_t)z, (uint32_t)z, (uint32_t)z};
      for (int e = e0; e < kBN * PIECES; e += kThreads) {
        const int t = e / PIECES;
        if (t0 + t >= S) *reinterpret_cast<u32x4_t*>(&sm.v[ring][t * ROW + 8 * (e % PIECES)]) = zero;
      }
      lds_barrier();
    }
    if (it + kStages - 1 < s1) issue_stage(it + kStages - 1, (kRing + kStages - 1) % kStages);

    if (t0 < wave_end) {
      // S^T for the stage's 32 tokens
      half8_t ka[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (kFp8) {
          ka[ks] = widen_fp8x8(*reinterpret_cast<const u32x2_t*>(
              &sm.k[ring][krow * ROW + 16 * (ks ^ kswz8<D>(krow)) + 8 * g]));
        } else {
          // piece (2 ks + g) ^ sw with sw = kswz(krow) < 8, written as 2 (4 (ks / 4) +
          // ((ks % 4) ^ (sw / 2))) + (g ^ (sw % 2)): four lane addresses, ks / 4 an immediate
          const int sw = kswz<D>(krow);
          const int pc = 2 * (4 * (ks >> 2) + ((ks & 3) ^ (sw >> 1))) + (g ^ (sw & 1));
          ka[ks] = *reinterpret_cast<const half8_t*>(&sm.k[ring][krow * ROW + 8 * pc]);
        }
      }
      float16_t sacc = float16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks], qb[ks], sacc, 0, 0, 0);

      // O^T += V^T P^T: k-step k covers stage tokens 16k .. 16k+15; the lane's 8 k-slots
      // are tokens 16k + 4g + {0..3} (first read) and 16k + 8 + 4g + {0..3} (second)
      half8_t va[2][DT];
      auto read_v = [&](int k, int dt) {
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
      };
      if constexpr (!kFp8) {
        // K fragments read four ahead of the product that takes them (the compiler's own
        // order waits for one pair of K reads after another: an LDS round trip every two
        // products), then the first k-step's V^T fragments, which the scheduler places
        // under the S^T products
        constexpr int kAhead = KS < 4 ? KS : 4;
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // LDS reads
#pragma unroll
        for (int i = 0; i < KS - kAhead; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a matrix product
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) read_v(0, dt);
      }

      // mask the diagonal / context-end stage: token t visible iff t <= min(S-1, P+qrow)
      if (!((t0 + kBN <= P + row_w + 1) && (t0 + kBN <= S))) {  // uniform
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
        const float mrow = max_xor<32>(ms);
        const float mnew = mrow > m + kRescaleSlack ? mrow : m;
        // 0 when m was -inf; 1 when the row's max did not move, also when it stays at -inf
        // (a row that sees none of this piece's tokens while other rows of the wave do:
        // 2^(-inf - -inf) would be NaN)
        const float alpha = mnew == m ? 1.0f : fast_exp2(m - mnew);
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

#pragma unroll
      for (int k = kFp8 ? 0 : 1; k < 2; ++k)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) read_v(k, dt);
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
  int it = s0;  // ring slot (it - s0) % kStages
  for (; it + 3 <= s1; it += 3) {
    stage(R0{}, it);
    stage(R1{}, it + 1);
    stage(R2{}, it + 2);
  }
  if (it < s1) stage(R0{}, it++);
  if (it < s1) stage(R1{}, it++);

  l = sum_xor<32>(l);
  const bool bad_table = __builtin_amdgcn_ballot_w64(bad_lanes) != 0;
  if (split) {
    // fp32 partials of this piece for the merge kernel, in lane order: o (not normalised),
    // then (m, l) per lane; a bad table entry makes l NaN, which the merge carries on
    float4_t* po = reinterpret_cast<float4_t*>(dst) + lane;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        po[(dt * 4 + v4) * kWave] =
            float4_t{o[dt][4 * v4], o[dt][4 * v4 + 1], o[dt][4 * v4 + 2], o[dt][4 * v4 + 3]};
    const int64_t ps = (reinterpret_cast<float*>(dst) - a.ws_o) / (kBM * D);
    float2_t* pml = reinterpret_cast<float2_t*>(a.ws_ml + ps * (kThreads * 2));
    pml[tid] = float2_t{m, bad_table ? qnan() : l};
    return;
  }
  if ((lane & 31) >= rows_left) return;
  half_t* out = reinterpret_cast<half_t*>(dst) + (int64_t)(lane & 31) * a.num_q_heads * D;
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

// Merge of a split row tile: one workgroup per (request, query head, row tile, wave of
// the tile), its 256 threads taking a quarter of a wave lane's partial each (lane layout of
// the prefill kernel's epilogue). With M the largest of the pieces' reference maxima (log2
// units), out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, times the value scale of an
// FP8 cache. Tiles that were not split are left alone.
template <int D>
__global__ __launch_bounds__(kThreads) void prefill_merge_kernel(const PrefillArgs a) {
  constexpr int DT = D / 32;
  constexpr int J = DT;  // float4 of a lane's partial per thread (a quarter of DT * 4)
  __shared__ PlanSmem sp;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int part = tid >> 6;  // which quarter of the lane's DT * 4 float4
  const int g = lane >> 5;
  const int tiles = (a.max_q_len + kBM - 1) / kBM;
  const int w = blockIdx.x & 3;
  const int ti = (blockIdx.x >> 2) % tiles;
  const int h = (blockIdx.x >> 2) / tiles % a.num_q_heads;
  const int r = (blockIdx.x >> 2) / tiles / a.num_q_heads;
  make_plan(a, sp);
  const Request rq = load_request(a, r);
  const int i0 = ti * kBM;
  if (rq.bad || i0 >= rq.C) return;
  const int L = sp.L[r];
  const int nst = tile_stages(rq, i0);
  if (nst <= L) return;  // one piece: written by the prefill kernel itself
  const int np = (nst + L - 1) / L;
  const int64_t ps0 = (((int64_t)r * a.num_q_heads + h) * tiles + ti) * a.max_pieces;
  const float2_t* pml = reinterpret_cast<const float2_t*>(a.ws_ml + ps0 * (kThreads * 2)) + w * kWave + lane;
  float mmax = neg_inf();
  for (int p = 0; p < np; ++p) mmax = fmaxf(mmax, pml[p * kThreads][0]);
  float lsum = 0.0f;
  float4_t acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int p = 0; p < np; ++p) {
    const float2_t ml = pml[p * kThreads];
    const float wgt = fast_exp2(ml[0] - mmax);  // 0 for a piece the row saw nothing of
    lsum = fmaf(wgt, ml[1], lsum);
    const float4_t* po = reinterpret_cast<const float4_t*>(a.ws_o + (ps0 + p) * (kBM * D)) +
                         w * (DT * 4 * kWave) + part * (J * kWave) + lane;
#pragma unroll
    for (int j = 0; j < J; ++j) acc[j] += wgt * po[j * kWave];
  }
  const int row = i0 + kWRows * w + (lane & 31);
  if (row >= rq.C) return;
  half_t* out = static_cast<half_t*>(a.out) + ((int64_t)(rq.q0 + row) * a.num_q_heads + h) * D;
  const float inv = a.v_scale / lsum;
#pragma unroll
  for (int j = 0; j < J; ++j) {  // float4 index jj = dt * 4 + v4 of the epilogue's layout
    const int jj = part * J + j;
    const int dt = jj / 4, v4 = jj % 4;
    half4_t x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (half_t)(acc[j][e] * inv);
    *reinterpret_cast<half4_t*>(out + 32 * dt + 8 * v4 + 4 * g) = x;
  }
}

template <int D, typename KV>
hipError_t launch_prefill_d(PrefillArgs a, hipStream_t stream) {
  const size_t smem = sizeof(PrefillSmem<D, KV>);
  static bool attr_set = false;  // the attribute is per function, set once per process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, KV>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t groups = (int64_t)a.num_reqs * a.max_pieces * a.num_q_heads;
  const int64_t tiles = (a.max_q_len + kBM - 1) / kBM;
  if (a.max_pieces > 1)  // the workspace: o of every piece slot, then their (m, l)
    a.ws_ml = a.ws_o + (int64_t)a.num_reqs * a.num_q_heads * tiles * a.max_pieces * kBM * D;
  const int64_t wgs = (groups + kXcds - 1) / kXcds * kXcds * tiles;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<D, KV>), dim3((unsigned)wgs), dim3(kThreads), smem, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_pieces == 1) return e;
  const int64_t mwgs = (int64_t)a.num_reqs * a.num_q_heads * tiles * (kBM / kWRows);
  if (mwgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_merge_kernel<D>), dim3((unsigned)mwgs), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Prefill workgroups the current device holds at once (0 when the runtime cannot say);
// queried once per device.
template <int D, typename KV>
int64_t resident_prefill_groups() {
  static std::atomic<int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_kernel<D, KV>, kThreads,
                                                   sizeof(PrefillSmem<D, KV>)) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  v = (int64_t)per_cu * cus;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

int64_t resident_prefill(int head_size) {
  return head_size == 128 ? resident_prefill_groups<128, half_t>() : resident_prefill_groups<64, half_t>();
}

}  // namespace

// Pieces per request: only a launch whose row tiles fill at most half of the device's
// workgroup slots is split, into as many pieces as those slots take (row tiles x heads x
// pieces <= resident workgroups), each piece at least kMinPieceStages stages; no split for
// batches above kMaxRanked requests. (With more tiles than that the split measured no
// faster: at the mixed step's 1024 tiles for 768 slots it took 198 + 22 us for the merge
// against 189 us unsplit.)
int prefill_max_pieces(int num_reqs, int num_q_heads, int max_q_len, int max_seq_len,
                       int head_size) {
  if (num_reqs <= 0 || num_reqs > kMaxRanked || num_q_heads <= 0 || max_q_len <= 0) return 1;
  if (head_size != 64 && head_size != 128) return 1;
  const int64_t slots = resident_prefill(head_size);
  if (slots <= 0) return 1;
  const int64_t tiles = (int64_t)num_reqs * num_q_heads * ((max_q_len + kBM - 1) / kBM);
  int64_t n = slots / tiles;
  const int64_t max_stages = ((int64_t)max_seq_len + kBN - 1) / kBN;
  n = std::min<int64_t>(n, max_stages / kMinPieceStages);
  n = std::min<int64_t>(n, kMaxPieces);
  return n < 2 ? 1 : (int)n;
}

int64_t prefill_workspace_bytes(int num_reqs, int num_q_heads, int max_q_len, int head_size,
                                int max_pieces) {
  if (max_pieces <= 1) return 0;
  const int64_t slots_total = (int64_t)num_reqs * num_q_heads * ((max_q_len + kBM - 1) / kBM) * max_pieces;
  const int64_t o_bytes = slots_total * kBM * head_size * 4;
  const int64_t ml_bytes = slots_total * kThreads * 2 * 4;
  return o_bytes + ml_bytes;
}

int prefill_slots(int head_size) {
  const int64_t v = resident_prefill(head_size);
  return v > INT32_MAX ? INT32_MAX : (int)v;
}

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
