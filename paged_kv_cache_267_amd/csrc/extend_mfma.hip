// extend_mfma.hip -- multi-token paged attention on the gfx950 matrix cores.
//
// Each sequence brings a chunk of n new query tokens, the last n of its L
// keys (already in the paged cache).  Token i of the chunk sits at position
// p = L - n + i and attends causally to keys [lo, p], lo = max(0, p + 1 - W)
// under a sliding window W, else 0.  This is what prefix caching ("vLLM 0.5
// deep dive: PagedAttention architecture", chenxutan.com, s4.4: compute only
// the tokens after a cached shared prompt) and chunked prefill (same page,
// s5.2) run over the block tables; per token it is the decode rule of s2.3
// applied to the sequence cut after p.
//
// Columns.  The (token, query head) pairs of one (sequence, KV head) are the
// columns of the score matrix, token-major: column c is token c / G, head
// c % G.  Heads of a group and tokens of a chunk therefore share the N axis
// of the MFMA tiles, whatever G is.
//
// Work.  One workgroup of 4 waves takes one (sequence, KV head, column
// block); each wave owns CW = 16 * NCB consecutive columns.  The workgroup
// walks the keys its columns need, 32 per step, through a ring of 4 LDS
// stages: each wave moves a quarter of a step's K and V from the cache into
// LDS with DMA loads (global_load_lds: no registers held while in flight).
// Steps go in pairs: one barrier publishes a pair's two stages and retires
// the previous pair's, which then load the two steps after the pair.  Each wave then reads its MFMA operands from
// LDS (one 16-byte read per lane and fragment, fragments laid out in lane
// order, so the reads are conflict-free) and skips steps its own columns do
// not need.  Column blocks of one (sequence, KV head) are dealt to one XCD
// (workgroup j runs on XCD j % 8) so that they share its L2, pairs round
// robin over the XCDs, the last column block of a pair (the most keys,
// causally) first.  With at most 64 sequences, pairs are dealt in order of
// their sequence's work (attended keys summed over its new tokens), largest
// first, so that the last workgroups to start are short ones; every wave
// ranks the sequences itself, one lane per sequence.
//
// Per step and column block of 16 columns (v_mfma_f32_16x16x32_bf16 for both
// products, heads/tokens on N):
//   S^T = K . Q^T   A = K (16 keys x 32 dims per k-step; lane (r, c) takes key
//                   8(c/4) + c%4 (+4 for the second sub-tile) and the cache's
//                   16-byte group r + 4k), B = Q^T;
//   O^T += V^T P^T  A = V^T (16 dims x 32 keys), B = P^T: lane row r holds
//                   keys 8r .. 8r+7 in both, which is what the two S^T
//                   fragments leave in that lane, so P never moves between
//                   lanes;
//   l += 1 . P^T    one more MFMA with an all-ones A gives every column's sum
//                   of the same bf16 weights P.V used, in every lane.
// The running max is per column and lane-local (two lane swaps for the max
// over a fragment's 4 lane rows), raised lazily: accumulators are rescaled
// only when a column's max grows by more than 2^8.  It starts at a large
// finite value, so a column whose keys are all masked in a step keeps p = 0
// and no NaN.  The score scale (scale * k_scale * log2 e, positive) is folded
// into the exponent's fused multiply-add.  E4M3 codes become bf16 in
// registers (exact); v_scale is applied at the end.
#include "common.h"
#include "dispatch.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Two workgroups of 4 waves per CU (two waves per SIMD, from different
// workgroups): one wave's softmax issues while the other's matrix products
// run.  Registers per wave <= 256.
constexpr int EX_WAVES = 4;
constexpr int EX_WG_PER_CU = 2;
constexpr float EX_LAZY_LOG2 = 8.0f;
constexpr float EX_M_FLOOR = -1.0e30f;
constexpr uint32_t BF16_ONE_X2 = 0x3F803F80u;

__device__ __forceinline__ float ex_colmax4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8_t, (u32x4_t){a, b, c, d});
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; exp and lgkm counts left free).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wave priority around the matrix-product regions (1) and the softmax (0):
// when the two waves sharing a SIMD are ready together, the one issuing
// products goes first, so their phases drift apart and one wave's softmax
// fills the other's product latency (1-2 % on the prefill workloads).  The
// scheduling barriers keep the compiler from moving work across the switch.
template <int P>
__device__ __forceinline__ void wave_priority() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(P);
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier for the LDS ring: this wave's LDS reads are complete
// (lgkmcnt 0) and every wave has arrived.  No memory fence: a fence would
// also wait for the DMA loads still in flight for later steps (they count
// as outstanding LDS writes), which must stay in flight across the barrier;
// each wave waits for its own DMA of the step with an exact vmcnt instead.
// The empty asm statements keep the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4));  // lgkmcnt(0), vmcnt/expcnt free
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sequences ranked by work before dealing (at most one per lane).
constexpr int EX_RANKED_SEQS = 64;

// A sequence's length (clamped to the table's capacity) and its rows of new
// tokens, clamped as the kernel uses them.
struct ExSeq { int L, q0, n; };
__device__ __forceinline__ ExSeq ex_seq(const ExtendParams& p, int s, int Lmax) {
  const int L = min(max(p.seq_lens[s], 0), Lmax);
  const int q0 = min(max(p.qsl[s], 0), p.num_tokens);
  const int q1 = min(max(p.qsl[s + 1], q0), p.num_tokens);
  return {L, q0, q1 - q0};
}

// Work of a sequence: keys attended summed over its n new tokens (token i
// at position L - n + i attends min(L - n + i + 1, W) keys; W = 0: no
// window).  Float: only the order matters.
__device__ __forceinline__ float ex_seq_work(ExSeq q, int window) {
  const float a = (float)(q.L - q.n + 1), b = (float)q.L;   // keys of the first and last token
  if (q.n <= 0 || b <= 0.f) return 0.f;
  const float W = (float)window;
  if (window <= 0 || b <= W) return 0.5f * (float)q.n * (fmaxf(a, 1.f) + b);
  if (a >= W) return (float)q.n * W;
  // tokens below the window's width, then the rest at W keys each
  const float below = W - a;
  return 0.5f * below * (a + W - 1.f) + ((float)q.n - below) * W;
}

// The sequence of rank r when sequences are ordered by work, largest first
// (ties: lower index first), with its clamped length and rows.  Needs
// num_seqs <= 64 (lane l reads sequence l); every lane returns the same.
__device__ __forceinline__ ExSeq seq_of_rank(const ExtendParams& p, int r, int lane, int Lmax,
                                             int& s_out) {
  const int S = p.num_seqs;
  const ExSeq mine = lane < S ? ex_seq(p, lane, Lmax) : ExSeq{0, 0, 0};
  const float w = lane < S ? ex_seq_work(mine, p.window) : -1.f;
  int rank = 0;
  for (int t = 0; t < S; ++t) {
    const float wt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), t));
    rank += (wt > w || (wt == w && t < lane)) ? 1 : 0;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < S && rank == r);
  const int s = hit != 0 ? (int)__builtin_ctzll(hit) : r;
  s_out = s;
  return {__builtin_amdgcn_readlane(mine.L, s), __builtin_amdgcn_readlane(mine.q0, s),
          __builtin_amdgcn_readlane(mine.n, s)};
}

// DMA of fragments J, J+1, .. N-1 of a wave: the 16 bytes of lane l from src
// + J * S to LDS dst0 + J * 1024 + 16 l.  The instruction's immediate offset
// moves both the global and the LDS address, so it carries J * S and the LDS
// base (M0) is set J * S below the fragment.  That base must stay at or above
// dst0 (an LDS address below the workgroup's block drops the write), so only
// strides up to a fragment's 1024 bytes go into the immediate; longer ones
// are added to the global address.
template <int S, int J, int N>
__device__ __forceinline__ void dma_frags(const char* src, char* dst0) {
  if constexpr (J < N) {
    if constexpr (S <= 1024)
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(dst0 + J * (1024 - S)),
                                       16, J * S, 0);
    else
      __builtin_amdgcn_global_load_lds((const void*)(src + J * S), (lds_void_t*)(dst0 + J * 1024),
                                       16, 0, 0);
    dma_frags<S, J + 1, N>(src, dst0);
  }
}

// Steps step0 + I, .., step0 + N - 1 (those below nsteps) of the walk, step
// step0 + i in ring stage i.
template <int I, int N, class F>
__device__ __forceinline__ void ring_steps(F& f, int step0, int nsteps) {
  if constexpr (I < N) {
    if (step0 + I < nsteps) {
      f(std::integral_constant<int, I>{}, std::integral_constant<bool, I % 2 == 0>{}, step0 + I);
      ring_steps<I + 1, N>(f, step0, nsteps);
    }
  }
}

template <int KV, int D, int BS, int NCB, int NBUF>
struct ExtendTile {
  static constexpr int E = KvTraits<KV>::E;
  static constexpr int KS = D / 32;       // QK k-steps of 32 dims
  static constexpr int NB = D / 16;       // output dim blocks of 16
  static constexpr int KL = D * E / 64;   // 16-byte K granules per lane per 16-key sub-tile
  static constexpr int CW = 16 * NCB;     // columns per wave
  // A step's fragments: 64 lanes x 16 bytes each, stored in lane order.
  static constexpr int KF = 2 * KL;                       // K: (sub-tile, granule)
  static constexpr int VF = KV == KV_BF16 ? NB : NB / 2;  // V: 8 keys of a dim (bf16) or
                                                          //    16 keys of a dim (E4M3)
  static constexpr int NF = KF + VF;
  // DMA loads per moving wave per step; the first NFW waves move a step
  // (K first, then V), the others only compute
  static constexpr int FW = NF >= EX_WAVES ? NF / EX_WAVES : 1;
  static constexpr int NFW = NF / FW;
  static_assert(NF % FW == 0 && KF % FW == 0 && NFW <= EX_WAVES, "whole fragments per wave");
  static constexpr int STAGE = NF * 1024;
  static constexpr int LDS_BYTES = NBUF * STAGE;
};

template <int KV, int D, int BS, int NCB, int NBUF>
__global__ __launch_bounds__(EX_WAVES * 64, EX_WG_PER_CU) void extend_kernel(const ExtendParams p) {
  using T = ExtendTile<KV, D, BS, NCB, NBUF>;
  constexpr int KS = T::KS, NB = T::NB, KL = T::KL, CW = T::CW, KF = T::KF, FW = T::FW;
  constexpr int NFW = T::NFW;
  __shared__ __attribute__((aligned(1024))) char ring[T::LDS_BYTES];
  const int lane = threadIdx.x & 63, r = lane >> 4, c = lane & 15;
  const int wave = wave_id();

  // work item: XCD x takes pairs x, x + 8, ... of the dealing order; a
  // pair's column blocks in a row
  const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int pair = x + 8 * (k / p.cblocks);
  if (pair >= p.pairs) return;
  const int cb = p.cblocks - 1 - k % p.cblocks;
  const int hk = pair % p.num_kv_heads;
  int s = pair / p.num_kv_heads;
  const ExSeq sq = p.num_seqs <= EX_RANKED_SEQS
                       ? seq_of_rank(p, pair / p.num_kv_heads, lane, p.max_blocks * BS, s)
                       : ex_seq(p, s, p.max_blocks * BS);
  const int G = 1 << p.log2g;

  const int L = sq.L, q0 = sq.q0, n = sq.n;
  const int ncols = n << p.log2g;
  const int wg_col0 = cb * EX_WAVES * CW;
  if (wg_col0 >= ncols) return;  // the whole workgroup leaves before any barrier
  const int W = p.window;
  auto lo_of = [W](int hi) { return W > 0 ? max(0, hi - W) : 0; };

  // keys of the workgroup (the union over its waves): first and last token
  const int wg_hi_min = L - n + (wg_col0 >> p.log2g) + 1;
  const int wg_hi_max = L - n + min(n - 1, (wg_col0 + EX_WAVES * CW - 1) >> p.log2g) + 1;
  const int wg_klo = lo_of(max(wg_hi_min, 0));
  const int wg_khi = max(wg_hi_max, 0);
  const int kq0 = wg_klo >> 5;
  const int nsteps = wg_khi > wg_klo ? ((wg_khi + 31) >> 5) - kq0 : 0;

  // keys of this wave's columns (empty for a wave past the chunk)
  const int col0 = wg_col0 + wave * CW;
  const bool has_cols = col0 < ncols;
  const int t_first = min(col0 >> p.log2g, n - 1);
  const int t_last = min(n - 1, (col0 + CW - 1) >> p.log2g);
  const int hi_min = L - n + t_first + 1;
  const int hi_max = L - n + t_last + 1;
  const int lo_max = lo_of(hi_max);
  const int klo = has_cols ? lo_of(max(hi_min, 0)) : 0;
  const int khi = has_cols ? max(hi_max, 0) : 0;
  const int32_t* row_bt = p.block_tables + (size_t)s * p.max_blocks;

  // per lane: its column in each of the NCB column blocks
  int lo_c[NCB], hi_c[NCB];
  bf16x8_t qop[NCB][KS];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const int cc = col0 + 16 * j + c;
    const int t = cc >> p.log2g, g = cc & (G - 1);
    const bool valid = t < n && L - n + t >= 0;
    hi_c[j] = valid ? L - n + t + 1 : 0;
    lo_c[j] = valid ? lo_of(hi_c[j]) : 0;
    const int tq = min(t, n - 1);
    const uint16_t* qrow = p.q + ((size_t)(q0 + tq) * p.num_q_heads + hk * G + g) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = (KV == KV_BF16) ? 32 * ks + 8 * r : 16 * (r + 4 * (ks >> 1)) + 8 * (ks & 1);
      uint4 v = *(const uint4*)(qrow + d0);
      if (t >= n) v = make_uint4(0, 0, 0, 0);
      qop[j][ks] = as_bf16x8(v.x, v.y, v.z, v.w);
    }
  }

  f32x4_t acc[NCB][NB], accl[NCB];
  float m_ref[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    accl[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    m_ref[j] = EX_M_FLOOR;
  }
  bf16x8_t ones = as_bf16x8(BF16_ONE_X2, BF16_ONE_X2, BF16_ONE_X2, BF16_ONE_X2);
  asm("" : "+v"(ones));   // held in registers, not rebuilt in every step
  const float qk = p.qk_scale;
  // a raw score above thr[j] would put its weight above 2^EX_LAZY_LOG2 (qk > 0)
  float thr[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) thr[j] = (m_ref[j] + EX_LAZY_LOG2) / qk;
  const size_t tile = (size_t)D * BS * T::E;  // bytes of one (block, head) tile
  // The query operands are in registers before the first DMA load is issued:
  // from here on the only vector-memory loads in flight are the ring's, so
  // every wait in the loop can leave the later steps' loads in flight (a
  // wait for a load issued before them would drain them all, vmcnt retiring
  // in order).
  wait_vmcnt<0>();

  // Block ids come from scalar loads of the table (read-only for the whole
  // launch, hence the constant address space), issued a step before they
  // are needed; scalar loads are counted apart from the vector loads, so
  // using them never waits on the ring.
  typedef const __attribute__((address_space(4))) int32_t cbt_t;
  cbt_t* sbt = (cbt_t*)row_bt;
  auto block_id = [&](int bi) -> int { return sbt[min(bi, p.max_blocks - 1)]; };
  auto clamp_id = [&](int b) -> int { return min(max(b, 0), p.num_blocks - 1); };

  // This wave's fragments of a step are slots wave*FW .. wave*FW+FW-1 of the
  // stage (K fragments first, then V).  Per lane: the step's base address,
  // plus a per-fragment offset.
  const bool moves_k = wave * FW < KF;
  // the block ids of a step's 32 keys (two 16-token blocks, else one)
  struct StepIds { int b0, b1; };
  auto ids_of = [&](int step) -> StepIds {
    const int bi = min((kq0 + step) * 32 / BS, p.max_blocks - 1);
    const int b0 = block_id(bi);
    return {b0, BS == 16 ? block_id(bi + 1) : b0};
  };
  // A lane's source address in a step is a fixed part, set here once, plus
  // the block id times the block stride, plus (64-token blocks) the step's
  // half of the block times the bytes one key position advances; with
  // 16-token blocks a lane reads the step's first or second block.
  //   K:        lane (r, c) takes key 8(c/4) + c%4 (+4), group r (+4i)
  //   bf16 V:   dims 16v + c, keys 8r .. 8r+7
  //   E4M3 V:   dims 32v + 16(r/2) + c, keys 16(r%2) .. +15
  const uint32_t bstride = (uint32_t)(p.num_kv_heads * tile);   // below 2^32 (host check)
  const char* lane_base;
  bool lane_b1;
  int key_bytes;
  {
    const size_t head = (size_t)hk * tile;
    if (moves_k) {
      const int kk = 8 * (c >> 2) + (c & 3);
      lane_b1 = BS == 16 && kk >= 16;
      lane_base = p.kc + head + (r * BS + (BS == 16 ? kk % 16 : kk)) * 16;
      key_bytes = 16;
    } else if (KV == KV_BF16) {
      lane_b1 = BS == 16 && r >= 2;
      lane_base = p.vc + head + (c * BS + (BS == 16 ? (8 * r) % 16 : 8 * r)) * 2;
      key_bytes = 2;
    } else {
      lane_b1 = BS == 16 && (r & 1);
      lane_base = p.vc + head + ((16 * (r >> 1) + c) * BS + (BS == 16 ? 0 : 16 * (r & 1)));
      key_bytes = 1;
    }
  }
  auto step_src = [&](int step, StepIds ids) -> const char* {
    // clamped here, at use, so the loads of the ids stay in flight until
    // then; on the scalar unit, before the lane's choice between the two
    int b0 = clamp_id(ids.b0), b1 = clamp_id(ids.b1);
    asm("" : "+s"(b0), "+s"(b1));
    const uint32_t blk = (uint32_t)(lane_b1 ? b1 : b0);
    const int in_block = BS == 64 ? ((kq0 + step) * 32) % 64 : 0;
    return lane_base + (uint64_t)blk * bstride + in_block * key_bytes;
  };
  // This wave's fragments are consecutive granules of one K sub-tile, or
  // consecutive V fragments: the first one's offset joins the lane's base,
  // and the others follow at a fixed stride.
  static_assert(KL % FW == 0, "a wave's K fragments lie in one sub-tile");
  constexpr int KSTR = 4 * BS * 16;                            // next K granule
  constexpr int VSTR = KV == KV_BF16 ? 16 * BS * 2 : 32 * BS;  // next V fragment
  {
    const int f = wave * FW, v = f - KF;
    lane_base += moves_k ? (f / KL) * 64 + (f % KL) * KSTR : v * VSTR;
  }

  // DMA this wave's share of step `step` into stage `st`
  auto fetch = [&](int step, int st, StepIds ids) {
    if (wave >= NFW) return;
    const char* src = step_src(step, ids);
    char* dst0 = ring + st * T::STAGE + wave * FW * 1024;
    if (moves_k) dma_frags<KSTR, 0, FW>(src, dst0);
    else dma_frags<VSTR, 0, FW>(src, dst0);
  };
  // Steps go in pairs over a ring of 4 stages: one wait and one barrier
  // publish a pair's two steps, and after it the pair's refill loads the
  // next pair's two steps into the previous pair's stages (past the end the
  // last step is fetched again: the count of loads in flight stays fixed).
  // Two steps are in flight while two are computed.
  static_assert(NBUF == 4, "pairs of steps over a 4-stage ring");
  // block ids of the next refill (steps p + 2, p + 3 for the pair at p)
  StepIds next_a = {0, 0}, next_b = {0, 0};
  if (nsteps > 0) {
    fetch(0, 0, ids_of(0));
    fetch(min(1, nsteps - 1), 1, ids_of(min(1, nsteps - 1)));
    next_a = ids_of(min(2, nsteps - 1));
    next_b = ids_of(min(3, nsteps - 1));
  }
  auto refill = [&](int step, int st) {   // step: the pair's first, in stage st
    fetch(min(step + 2, nsteps - 1), (st + 2) % NBUF, next_a);
    fetch(min(step + 3, nsteps - 1), (st + 3) % NBUF, next_b);
  };
  // At the end of a pair's second step, once its LDS reads are consumed,
  // load the ids of the next pair's refill: scalar loads share a counter
  // with LDS reads, so issued earlier they would make the pair's LDS waits
  // wait for them too.  The next pair's barrier waits for them.
  auto load_next_ids = [&](int second) {
    asm volatile("" ::: "memory");
    next_a = ids_of(min(second + 3, nsteps - 1));
    next_b = ids_of(min(second + 4, nsteps - 1));
  };

  // One step of the walk, in ring stage `stage_c` (a compile-time constant:
  // the loop below is unrolled by the ring's depth, so the stage offsets of
  // the LDS reads are immediates); `first_c` tells the pair's first step from
  // its second.
  auto do_step = [&](auto stage_c, auto first_c, int step) {
    const int cur_st = stage_c;     // stage of `step`
    constexpr bool first = decltype(first_c)::value;
    if (first) {
      // this wave's share of the pair has landed; after the barrier
      // everyone's has, and every wave is done with the previous pair's
      // stages.  The barrier orders LDS only: a full __syncthreads would also
      // drain the DMA loads of the later steps.
      wait_vmcnt<0>();
      ring_barrier();
    }
    const int key0 = (kq0 + step) * 32;
    if (key0 + 32 <= klo || key0 >= khi) {  // no key of this wave's columns
      if (first) refill(step, cur_st);
      else load_next_ids(step);
      return;
    }
    const char* stage = ring + cur_st * T::STAGE;

    // K operands of both sub-tiles (E4M3 -> bf16 in registers)
    bf16x8_t kop[2][KS];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        const u32x4_t w = *(const u32x4_t*)(stage + (h * KL + i) * 1024 + lane * 16);
        if (KV == KV_BF16) {
          kop[h][i] = as_bf16x8(w.x, w.y, w.z, w.w);
        } else {
          kop[h][2 * i] = as_bf16x8(fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x),
                                    fp8x2_to_bf16x2<false>(w.y), fp8x2_to_bf16x2<true>(w.y));
          kop[h][2 * i + 1] = as_bf16x8(fp8x2_to_bf16x2<false>(w.z), fp8x2_to_bf16x2<true>(w.z),
                                        fp8x2_to_bf16x2<false>(w.w), fp8x2_to_bf16x2<true>(w.w));
        }
      }
    const bool full = key0 >= lo_max && key0 + 32 <= hi_min && hi_min > 0;

    wave_priority<1>();
    // scores of every column block first: the V reads below overlap them
    f32x4_t sacc[NCB][2];
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      sacc[j][0] = sacc[j][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sacc[j][0] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][ks], qop[j][ks], sacc[j][0], 0, 0, 0);
        sacc[j][1] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[1][ks], qop[j][ks], sacc[j][1], 0, 0, 0);
      }
    }

    // refill while the score products run
    if (first) refill(step, cur_st);

    // V operands: dword w holds keys 8r + 2w, 8r + 2w + 1 of dim 16nb + c
    uint32_t vq[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (KV == KV_BF16) {
        const u32x4_t w = *(const u32x4_t*)(stage + (KF + nb) * 1024 + lane * 16);
        vq[nb][0] = w.x;
        vq[nb][1] = w.y;
        vq[nb][2] = w.z;
        vq[nb][3] = w.w;
      } else {
        const int rf = 2 * (nb & 1) + (r >> 1);  // the fetching lane row
        const u32x2_t w = *(const u32x2_t*)(stage + (KF + (nb >> 1)) * 1024 +
                                            (rf * 16 + c) * 16 + 8 * (r & 1));
        vq[nb][0] = fp8x2_to_bf16x2<false>(w.x);
        vq[nb][1] = fp8x2_to_bf16x2<true>(w.x);
        vq[nb][2] = fp8x2_to_bf16x2<false>(w.y);
        vq[nb][3] = fp8x2_to_bf16x2<true>(w.y);
      }
    }
    // keys outside [klo, khi) may be unwritten or outside the window's
    // blocks: zero their V so that p = 0 never meets a NaN
    if (key0 < klo || key0 + 32 > khi) {
      // key key0 + 8r + i is kept when i is in [vlo, vhi): offsets against
      // constants, so no per-key index is formed outside the masked steps
      int k0 = key0;
      asm("" : "+s"(k0));   // formed here: not an induction variable of every step
      const int vlo = klo - k0 - 8 * r, vhi = khi - k0 - 8 * r;
      uint32_t vmask[4];
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
        vmask[w2] = ((2 * w2 >= vlo && 2 * w2 < vhi) ? 0xffffu : 0u) |
                    ((2 * w2 + 1 >= vlo && 2 * w2 + 1 < vhi) ? 0xffff0000u : 0u);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) vq[nb][w2] &= vmask[w2];
    }
    wave_priority<0>();
    // Softmax in two phases.  First, per column block: mask, running max
    // and the lazy rescale (a rare branch).  Then one branch-free run: the
    // weights of block 0, then each block's P.V products followed by the
    // next block's weights; the other wave on the SIMD fills the gaps, its
    // exponentials beside these products and the other way round.
    float scs[NCB][8];
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      const f32x4_t s0 = sacc[j][0], s1 = sacc[j][1];
      // raw scores; slot i of lane row r is key key0 + 8r + i
      float* sc = scs[j];
      sc[0] = s0[0]; sc[1] = s0[1]; sc[2] = s0[2]; sc[3] = s0[3];
      sc[4] = s1[0]; sc[5] = s1[1]; sc[6] = s1[2]; sc[7] = s1[3];
      if (!full) {   // key key0 + 8r + i is in [lo_c, hi_c) when i is in [slo, shi)
        int k0 = key0;
        asm("" : "+s"(k0));
        const int slo = lo_c[j] - k0 - 8 * r, shi = hi_c[j] - k0 - 8 * r;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (!(i >= slo && i < shi)) sc[i] = -INFINITY;
      }
      // Lazy rescale: only a score above its column's threshold calls for
      // one, so a step compares its scores and forms the column max (and the
      // new reference) only when some lane finds one.  Scaling by qk > 0 keeps
      // the order, so this is the test "column max * qk > m_ref + 2^LAZY".
      bool over = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) over |= sc[i] > thr[j];
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
        float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                         fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        mx = ex_colmax4(mx) * qk;
        const float m_new = fmaxf(m_ref[j], mx);
        const float alpha = fast_exp2(m_ref[j] - m_new);
        accl[j] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[j][nb] *= alpha;
        m_ref[j] = m_new;
        thr[j] = (m_new + EX_LAZY_LOG2) / qk;
      }
    }
    auto weights = [&](int j) -> bf16x8_t {
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pw[i] = pack_bf16x2(fast_exp2(__builtin_fmaf(scs[j][2 * i], qk, -m_ref[j])),
                            fast_exp2(__builtin_fmaf(scs[j][2 * i + 1], qk, -m_ref[j])));
      return as_bf16x8(pw[0], pw[1], pw[2], pw[3]);
    };
    bf16x8_t pop = weights(0);
    wave_priority<1>();
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      accl[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pop, accl[j], 0, 0, 0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[j][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(vq[nb][0], vq[nb][1], vq[nb][2], vq[nb][3]), pop, acc[j][nb], 0, 0, 0);
      if (j + 1 < NCB) pop = weights(j + 1);
    }
    wave_priority<0>();
    if (!first) load_next_ids(step);
  };
  // unrolled by the ring's depth: each step's stage is a constant
  for (int step0 = 0; step0 < nsteps; step0 += NBUF) ring_steps<0, NBUF>(do_step, step0, nsteps);
  // no DMA may still be writing this workgroup's LDS when it ends
  wait_vmcnt<0>();

  if (!has_cols) return;
  // normalise and store: lane (r, c) holds dims 16nb + 4r .. +3 of its column
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const float l = accl[j][0];
    const float inv = l > 0.f ? p.v_scale / l : 0.f;
    const int cc = col0 + 16 * j + c;
    const int t = cc >> p.log2g, g = cc & (G - 1);
    if (t < n) {
      uint16_t* orow = p.out + ((size_t)(q0 + t) * p.num_q_heads + hk * G + g) * D;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4_t o = acc[j][nb] * inv;
        *(u32x2_t*)(orow + 16 * nb + 4 * r) = (u32x2_t){pack_bf16x2(o[0], o[1]),
                                                        pack_bf16x2(o[2], o[3])};
      }
    }
  }
}

// Column blocks of 16 per wave, and LDS stages in the ring (a pair of steps
// in flight while a pair is computed).
template <int D> constexpr int ex_ncb() { return D == 128 ? 2 : 4; }
template <int D> constexpr int ex_nbuf() { return 4; }

template <int KV, int D, int BS>
hipError_t launch_ncb(const ExtendParams& p, hipStream_t stream) {
  constexpr int NCB = ex_ncb<D>();
  const long long grid = 8LL * ((p.pairs + 7) / 8) * p.cblocks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((extend_kernel<KV, D, BS, NCB, ex_nbuf<D>()>), dim3((unsigned)grid),
                     dim3(EX_WAVES * 64), 0, stream, p);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_bs(const ExtendParams& p, int BS, hipStream_t stream) {
  switch (BS) {
    case 16: return launch_ncb<KV, D, 16>(p, stream);
    case 32: return launch_ncb<KV, D, 32>(p, stream);
    case 64: return launch_ncb<KV, D, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <int KV>
hipError_t launch_d(const ExtendParams& p, int D, int BS, hipStream_t stream) {
  switch (D) {
    case 64: return launch_bs<KV, 64>(p, BS, stream);
    case 128: return launch_bs<KV, 128>(p, BS, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_extend(ExtendParams p, int kv_dtype, int D, int BS, int max_query_len,
                         hipStream_t stream) {
  const int CB = EX_WAVES * 16 * (D == 128 ? ex_ncb<128>() : ex_ncb<64>());  // columns per WG
  const long long cols = (long long)max_query_len << p.log2g;
  p.cblocks = (int)((cols + CB - 1) / CB);
  p.pairs = p.num_seqs * p.num_kv_heads;
  if (p.cblocks == 0 || p.pairs == 0) return hipSuccess;
  if (kv_dtype == KV_BF16) return launch_d<KV_BF16>(p, D, BS, stream);
  if (kv_dtype == KV_FP8) return launch_d<KV_FP8>(p, D, BS, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
