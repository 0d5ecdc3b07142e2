// decode_persistent.h -- paged decode attention on gfx950: the persistent,
// balanced driver shared by the two tile computations (tile_mfma.h: both
// contractions on the matrix cores; tile_valu.h: dot products on the VALU).
//
// Computation (sources: "vLLM 0.5 deep dive: PagedAttention architecture",
// chenxutan.com, s2.2-s2.3; "vLLM 0.7.2 deep dive: PagedAttention v2 with
// FlashAttention-3", jsqmd.com, s2.2-s2.3): per (sequence, query head), scaled
// dot products of the query with every in-window key, gathered block by block
// through the block table, a softmax kept stable by a running max and sum, and
// the softmax-weighted sum of the values.  The unit of output is a segment:
// one (sequence, KV head, partition) when split, one (sequence, KV head)
// otherwise; its G query heads are served from one read of each K/V tile.
//
// Schedule.  The grid is sized to the resident capacity; workgroup w serves KV
// head w % H_kv (workgroups are dealt to the 8 XCDs round-robin, so a head
// stays on one XCD and a prefix shared by many sequences stays in its L2) and
// takes that head's segments from one list, dealt to its J workgroups in
// serpentine rounds: full partitions first (by sequence), then the partial
// ones (a sequence's first or last partition, or the whole sequence when
// unsplit), largest first by a stable counting sort over size classes.  Each
// workgroup builds the list from the lengths in LDS, so all agree on it.
//
// Halves.  Where two waves per SIMD fit in registers, a workgroup is 8 waves,
// one per CU, made of two independent halves of 4 waves; otherwise it is one
// half.  The halves take the batch's segments one at a time, in list order, as
// they reach them (a claim through LDS atomics), so a half that the CU serves
// faster takes more of them and both finish together.
//
// Memory pipeline.  The workgroup walks its segments in batches.  For a batch
// it stages, in LDS, the block-table entries of every block the batch touches
// and the query rows of its segments (blocks wholly before the window are
// never listed); after that the only global loads until the batch ends are
// K/V sub-tiles (16 tokens of one block).  Each wave streams its sub-tiles
// (the 4 waves of a half take a segment's sub-tiles round-robin) NBUF - 1
// tiles ahead across segment boundaries, with a fixed number of loads per
// step (a wave past its last tile re-reads block 0), so every wait before a
// tile's first use leaves the younger tiles in flight.
//
// Merge.  At a segment end a wave deposits its (max, sum, acc) in an LDS merge
// area of its half and streams on; at its next segment end (or after the
// batch's closing barrier) it merges a quarter of that segment's output from
// the half's 4 deposits, in wave order, and writes it: the output row
// (unsplit) or the partition's output and natural-log LSE (split).  Counters
// in LDS order deposits and merges, so no wave waits at a segment end unless
// another wave of its half is a whole segment behind.  A segment longer than
// the staged table is carried into the next batch with its running state, by
// the same half.
//
// Tile policy interface (T): constants KV, D, BS, G, E (KV element bytes), EQ
// (query element bytes), OUT_F32, NBUF, QROWB (staged query row bytes), QBYTES
// (LDS for staged queries), NPAR (merge areas), HALVES (1 or 2); types Buf (one sub-tile in
// registers, with fields slot and st) and WaveLds (per-wave LDS scratch); and
// the device members reset(), load(Buf&, k_tile, v_tile, sub),
// set_query(staged rows), compute(Buf&, t0, t1, qk_scale, WaveLds&) and
// deposit(m[G], l[G], acc[G][D + 4]).
#pragma once

#include <atomic>

#include "common.h"

namespace pa {

constexpr int PD_WAVES = 4;
constexpr int PD_SEQ_CHUNK = 1024;    // sequences per launch (schedule kept in LDS)
constexpr int PD_TBL = 2048;          // block-table entries staged per batch
constexpr int PD_SORT_MAX = 512;      // partial segments ordered by size (more: by sequence)
constexpr int PD_SIZE_CLASSES = 256;  // size classes of that order (16 per octave of sub-tiles)

// Per-batch description of one segment slot.
struct SegMeta {
  int s;        // sequence (relative to the launch)
  int p;        // partition (split) or 0
  int t0, t1;   // key range of the whole segment
  int st_a;     // first sub-tile of this batch's share of the segment
  int st_b;     // end sub-tile of this batch's share
  int tbl;      // LDS table index of block st_a / SPB
  int fin;      // the segment ends in this batch
};

template <class T>
struct PdGeom {
  static constexpr int SLOTS_RAW = T::QBYTES / (T::G * T::QROWB);
  static constexpr int SLOTS = SLOTS_RAW < 64 ? SLOTS_RAW : 64;  // segments per batch (one per lane of the planner)
  static_assert(SLOTS >= 1, "query staging too small");
};

template <class T>
struct PdSmem {
  static constexpr int G = T::G, D = T::D, SLOTS = PdGeom<T>::SLOTS;
  int32_t lens[PD_SEQ_CHUNK];        // clamped lengths
  int32_t fpre[PD_SEQ_CHUNK + 1];    // full partitions before each sequence (exclusive)
  int32_t ppre[PD_SEQ_CHUNK + 1];    // partial segments before each sequence (exclusive)
  alignas(16) int32_t plist[PD_SORT_MAX];  // partial segments, largest first: (s << 20) | p
  int32_t tbl[PD_TBL];               // staged block ids of the batch
  alignas(16) uint8_t q[SLOTS][G][T::QROWB];   // staged query rows of the batch
  SegMeta meta[SLOTS];
  int32_t bcount, bnext_m, bnext_st, bused, scan[2][PD_WAVES * T::HALVES];
  int32_t next_slot;                 // slots of the batch claimed so far
  int32_t carry_half;                // half holding a segment that continues into the next batch
  int32_t hslot[T::HALVES][SLOTS + 1];   // slot of each half's k-th segment (-1 open, -2 none)
  int32_t hlock[T::HALVES][SLOTS + 1];   // claim of that entry taken
  int32_t arrived[T::HALVES][T::NPAR];   // deposits into each merge area (4 per use)
  int32_t done[T::HALVES][T::NPAR];      // quarter merges out of each area (4 per use)
  typename T::WaveLds wl[PD_WAVES * T::HALVES];  // per-wave scratch of the tile computation
  union alignas(16) {
    struct {
      float m[PD_WAVES][G];
      float l[PD_WAVES][G];
      // rows padded to a stride of 4 (mod 8) floats: the 16-byte deposits of 4
      // lane rows x G heads conflict least there (SQ_LDS_BANK_CONFLICT per LDS
      // instruction on the G = 8 workloads, stride 0 / 4 / 8 / 12 mod 32
      // floats: 2.9 / 0.11 / 0.52 / 0.11)
      float acc[PD_WAVES][G][D + 4];
    } area[T::HALVES][T::NPAR];
    struct {                          // ordering of the partial segments, before any merge
      int32_t cls[PD_SORT_MAX];
      // per chunk, class c at [c % (classes / 64)][c / (classes / 64)]: the
      // scan's lane l, which owns a run of consecutive classes, then reads
      // consecutive words with its neighbours
      int32_t cnt[PD_SORT_MAX / 64][PD_SIZE_CLASSES / 64][64];
    } srt;
  } u;
};

template <class T>
__global__ __launch_bounds__(64 * PD_WAVES * T::HALVES) void decode_persistent_kernel(DecodeParams p) {
  constexpr int D = T::D, BS = T::BS, G = T::G, E = T::E, EQ = T::EQ;
  constexpr int SPB = BS / 16;
  constexpr size_t TILE_BYTES = (size_t)D * BS * E;
  constexpr int HV = T::HALVES;         // independent 4-wave halves per workgroup
  constexpr int NTH = 64 * PD_WAVES * HV;
  constexpr int SLOTS = PdGeom<T>::SLOTS;
  constexpr int NPAR = T::NPAR;
  static_assert(G <= 16, "at most 16 query heads per KV head");

  __shared__ PdSmem<T> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int h = wave / PD_WAVES, hw = wave % PD_WAVES;   // half, wave within the half
  const int H = p.num_kv_heads, Hq = p.num_q_heads;
  const int hk = blockIdx.x % H;
  const int j = blockIdx.x / H, J = gridDim.x / H;
  const int S = p.seq_count, s0 = p.seq_begin;
  const int P = p.partition_size;     // 0: unsplit
  const int Lmax = p.max_blocks * BS;

  // ---- schedule: full partitions first (by sequence), then the partial ones --
  // (first / last partition of a sequence, or the whole sequence when unsplit)
  // largest first.
  auto seg_range = [&](int L, int pp, int& t0, int& t1) {
    const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
    if (P == 0) { t0 = lo; t1 = L; return; }
    t0 = max(lo, pp * P);
    t1 = min(L, (pp + 1) * P);
  };
  auto counts = [&](int L, int& nfull, int& npart, int& pf0) {
    // pf0: first full partition; partial ones are p_lo and/or p_hi - 1
    nfull = 0; npart = 0; pf0 = 0;
    if (P == 0) { npart = 1; return; }
    if (L <= 0) return;
    const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
    const int p_lo = lo / P, p_hi = (L + P - 1) / P;
    pf0 = (lo + P - 1) / P;
    nfull = max(0, L / P - pf0);
    npart = (p_hi - p_lo) - nfull;
  };
  {
    const int per = (S + NTH - 1) / NTH;
    const int a = min(S, tid * per), b = min(S, a + per);
    int cf = 0, cp = 0;
    for (int i = a; i < b; ++i) {
      int L = p.seq_lens[s0 + i];
      L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
      sm.lens[i] = L;
      int nf, np, f0;
      counts(L, nf, np, f0);
      cf += nf;
      cp += np;
    }
    int xf = cf, xp = cp;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int yf = __shfl_up(xf, off, 64), yp = __shfl_up(xp, off, 64);
      if (lane >= off) { xf += yf; xp += yp; }
    }
    if (lane == 63) { sm.scan[0][wave] = xf; sm.scan[1][wave] = xp; }
    __syncthreads();
    int rf = xf - cf, rp = xp - cp;
    for (int w = 0; w < wave; ++w) { rf += sm.scan[0][w]; rp += sm.scan[1][w]; }
    for (int i = a; i < b; ++i) {
      sm.fpre[i] = rf;
      sm.ppre[i] = rp;
      int nf, np, f0;
      counts(sm.lens[i], nf, np, f0);
      rf += nf;
      rp += np;
    }
    if (tid == NTH - 1) { sm.fpre[S] = rf; sm.ppre[S] = rp; }
    __syncthreads();
  }
  const int F = uniform(sm.fpre[S]), NPART = uniform(sm.ppre[S]);
  const bool sorted = NPART <= PD_SORT_MAX;
  if (sorted) {
    // list the partial segments with a size class, then order them by class
    // with a stable counting sort, so every workgroup derives the same order
    constexpr int NBK = PD_SIZE_CLASSES, SR = PD_SORT_MAX / NTH;
    constexpr int CBITS = 8, CPL = NBK / 64;   // class bits; classes per lane in the scan
    static_assert(NBK == 1 << CBITS && NBK % 64 == 0, "size classes");
    // class of a segment of sz sub-tiles: 16 classes per octave (sizes within
    // 1/16 of each other share one), larger segments in smaller classes
    auto size_class = [](int sz) -> int {
      if (sz <= 0) return NBK - 1;
      const int lz = 31 - __builtin_clz(sz);
      const int c = lz >= 4 ? 16 * lz + ((sz >> (lz - 4)) & 15) : sz;
      return NBK - 1 - min(NBK - 1, c);
    };
    for (int i = tid; i < S; i += NTH) {
      const int L = sm.lens[i];
      int nf, np, f0;
      counts(L, nf, np, f0);
      int o = sm.ppre[i];
      if (np > 0) {
        const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
        const int p_lo = P ? lo / P : 0, p_hi = P ? (L + P - 1) / P : 1;
        for (int pp = p_lo; pp < p_hi; pp = (pp == p_lo && p_hi - 1 > p_lo) ? p_hi - 1 : p_hi) {
          int t0, t1;
          seg_range(L, pp, t0, t1);
          if (P != 0 && t1 - t0 == P) continue;
          sm.plist[o] = (i << 20) | pp;
          sm.u.srt.cls[o] = size_class(t0 < t1 ? ((t1 + 15) >> 4) - (t0 >> 4) : 0);
          ++o;
        }
      }
    }
    const int nch = (NPART + 63) / 64;   // chunks holding entries
    for (int i = tid; i < nch * NBK; i += NTH) (&sm.u.srt.cnt[0][0][0])[i] = 0;
    __syncthreads();
    // entry e sits in chunk e / 64 (one wave's lanes); the lanes holding its
    // class are found bit-sliced (one ballot per bit of the 8-bit class), so
    // its rank among the chunk's entries of that class costs a fixed 9 ballots
    int mine[SR], cls[SR], wr[SR];
#pragma unroll
    for (int r = 0; r < SR; ++r) {
      const int e = tid + r * NTH, c = wave + r * (NTH / 64);
      const bool valid = e < NPART;
      mine[r] = valid ? sm.plist[e] : 0;
      cls[r] = valid ? sm.u.srt.cls[e] : 0;
      uint64_t same = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
      for (int bit = 0; bit < CBITS; ++bit) {
        const bool set = (cls[r] >> bit) & 1;
        const uint64_t bm = __builtin_amdgcn_ballot_w64(valid && set);
        same &= set ? bm : ~bm;
      }
      wr[r] = __builtin_popcountll(same & ((1ull << lane) - 1));
      if (valid && wr[r] == 0) sm.u.srt.cnt[c][cls[r] % CPL][cls[r] / CPL] = __builtin_popcountll(same);
    }
    __syncthreads();
    // class starts (exclusive scan over classes of the chunk totals; lane l
    // holds classes CPL*l ..), then each chunk's base within its class,
    // written over the counts
    if (wave == 0) {
      int tot = 0;
      for (int k = 0; k < CPL; ++k)
        for (int c = 0; c < nch; ++c) tot += sm.u.srt.cnt[c][k][lane];
      int x = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      int run = x - tot;
      for (int k = 0; k < CPL; ++k)
        for (int c = 0; c < nch; ++c) {
          const int n = sm.u.srt.cnt[c][k][lane];
          sm.u.srt.cnt[c][k][lane] = run;
          run += n;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < SR; ++r)
      if (tid + r * NTH < NPART)
        sm.plist[sm.u.srt.cnt[wave + r * (NTH / 64)][cls[r] % CPL][cls[r] / CPL] + wr[r]] = mine[r];
    __syncthreads();
  }
  if (tid < HV * NPAR) {
    (&sm.arrived[0][0])[tid] = 0;
    (&sm.done[0][0])[tid] = 0;
  }
  if (tid == 0) sm.carry_half = 0;
  __syncthreads();
  const int total = F + NPART;
  // The list is dealt to the head's J workgroups in serpentine order: round r
  // gives workgroup j entry r*J + j (r even) or r*J + J-1-j (r odd), so the
  // largest entries of one round meet the smallest of the next.
  auto list_index = [&](int m) -> int { return m * J + ((m & 1) ? J - 1 - j : j); };
  int M = total / J;  // full rounds, then possibly one entry of the last round
  if (M * J < total && list_index(M) < total) ++M;

  // k-th segment of the list -> (sequence, partition), in each lane on its
  // own: a sorted partial segment is read from the ordered list; otherwise a
  // binary search over the exclusive prefix counts finds the sequence.
  auto seg_of = [&](int k, int& si, int& pp) {
    const bool full = k < F;
    const int kk = full ? k : k - F;
    if (!full && sorted) {
      const int e = sm.plist[kk];
      si = e >> 20;
      pp = e & 0xfffff;
      return;
    }
    const int32_t* pre = full ? sm.fpre : sm.ppre;
    int lo = 0, hi = S;   // pre[lo] <= kk < pre[hi]; the sequence is the last such lo
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= kk) lo = mid;
      else hi = mid;
    }
    si = lo;
    const int L = sm.lens[si];
    int nf, np, f0;
    counts(L, nf, np, f0);
    const int r = kk - pre[si];
    if (full) {
      pp = f0 + r;
    } else {
      const int lo_t = (p.window > 0 && L > p.window) ? L - p.window : 0;
      const int p_lo = P ? lo_t / P : 0, p_hi = P ? (L + P - 1) / P : 1;
      int t0, t1;
      seg_range(L, p_lo, t0, t1);
      const bool first_partial = P == 0 || t1 - t0 != P;
      pp = (r == 0 && first_partial) ? p_lo : p_hi - 1;
    }
  };
  const char* kbase = (const char*)p.kc + (size_t)hk * TILE_BYTES;
  const char* vbase = (const char*)p.vc + (size_t)hk * TILE_BYTES;
  const size_t block_stride = (size_t)H * TILE_BYTES;
  const unsigned nb_max = (unsigned)(p.num_blocks - 1);

  using Buf = typename T::Buf;
  Buf bufs[T::NBUF];
  // running state of the segment being computed (carried across batches when a
  // segment continues)
  T tile;
  tile.reset();

  // segment ends this wave has passed (the same sequence in every wave), and
  // the last one, whose quarter merge is still to do (pend_s < 0: none)
  int uses = 0;
  int pend_s = -1, pend_pp = 0, pend_par = 0, pend_gen = 0;

  auto spin_until = [&](const int32_t* ctr, int target) {
    while (lds_load_acquire(ctr) < target)
      __builtin_amdgcn_s_sleep(1);
  };
  // Merge of the 4 states a half's waves left for a finished segment, done by
  // quarters: wave w of the half combines (in wave order) and writes outputs
  // [w, w+1) * G*D/4 of the segment's G x D block.
  auto merge_quarter = [&]() {
    if (pend_s < 0) return;
    constexpr int QN = G * D / PD_WAVES;
    const int par = pend_par;
    spin_until(&sm.arrived[h][par], PD_WAVES * (pend_gen + 1));
    auto& ar = sm.u.area[h][par];
#pragma unroll
    for (int i0 = 0; i0 < QN; i0 += 64) {
      const int e = hw * QN + i0 + lane;
      if (QN % 64 == 0 || i0 + lane < QN) {
        const int g = e / D, d = e % D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < PD_WAVES; ++w) mx = fmaxf(mx, ar.m[w][g]);
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int w = 0; w < PD_WAVES; ++w) {
          const float f =
              (mx == -INFINITY || ar.m[w][g] == -INFINITY) ? 0.f : fast_exp2(ar.m[w][g] - mx);
          den += f * ar.l[w][g];
          num += f * ar.acc[w][g][d];
        }
        const float o = den > 0.f ? num * (p.v_scale / den) : 0.f;
        const size_t r = (size_t)pend_s * Hq + hk * G + g;
        if (p.part_out == nullptr) {
          if (T::OUT_F32) ((float*)p.out)[r * D + d] = o;
          else ((uint16_t*)p.out)[r * D + d] = to_bf16_bits(o);
        } else {
          const size_t pi = r * p.max_parts + pend_pp;
          p.part_out[pi * D + d] = o;
          if (d == 0) p.part_lse[pi] = (mx + __log2f(den)) * 0.69314718055994531f;
        }
      }
    }
    if (lane == 0)
      lds_add_release(&sm.done[h][par], 1);
    pend_s = -1;
  };

  int bm = 0, bst = -1;  // next batch starts at segment bm, sub-tile bst (-1: its start)

  while (bm < M) {
    // ---- batch plan (wave 0; lane i plans slot i) -------------------------------------
    // Slot i takes list entry bm + i (slot 0 resumes a carried segment at
    // sub-tile bst).  Slots are taken in order while their blocks fit in the
    // staged table; a first slot that alone overflows it takes what fits and
    // the segment continues in the next batch.
    if (wave == 0) {
      // the lane index comes from an opaque instruction here, so the compiler
      // keeps this per-lane work inside the planner instead of hoisting
      // loop-invariant per-lane values into registers held by the main loop
      int pl;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(pl));
      const int m = bm + pl;
      const bool have = pl < SLOTS && m < M;
      int st_hi = 0, a = 0, nb = 0, row0 = 0;
      if (have) {
        int si, pp, t0, t1;
        seg_of(list_index(m), si, pp);
        seg_range(sm.lens[si], pp, t0, t1);
        const int st_lo = t0 >> 4;
        st_hi = t0 < t1 ? (t1 + 15) >> 4 : st_lo;
        a = (pl == 0 && bst >= 0) ? bst : st_lo;
        nb = st_hi > a ? (st_hi + SPB - 1) / SPB - a / SPB : 0;
        SegMeta& md = sm.meta[pl];   // rest of the slot's record once the batch is cut
        md.s = si; md.p = pp; md.t0 = t0; md.t1 = t1; md.st_a = a;
        row0 = (s0 + si) * p.max_blocks + a / SPB;   // block_tables index of the first block
      }
      int incl = nb;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (pl >= off) incl += y;
      }
      const uint64_t stop = __builtin_amdgcn_ballot_w64(!have || incl > PD_TBL);
      // first lane that takes no slot; 64 when every lane takes one (SLOTS = 64
      // and the batch's blocks all fit), where the ballot is empty
      const int f = stop != 0 ? (int)__builtin_ctzll(stop) : 64;
      const bool trunc = f == 0;                    // the first slot alone overflows the table
      const int cnt = trunc ? 1 : f;
      int b = st_hi;
      if (trunc) {
        b = (a / SPB + PD_TBL) * SPB;
        nb = PD_TBL;
        incl = PD_TBL;
      }
      if (pl < cnt) {
        SegMeta& md = sm.meta[pl];
        md.st_b = b; md.tbl = incl - nb; md.fin = b >= st_hi ? 1 : 0;
      }
      // table entries to stage: their index into block_tables for now
      for (int c = 0; c < cnt; ++c) {
        const int n = __builtin_amdgcn_readlane(nb, c), at = __builtin_amdgcn_readlane(incl, c) - n;
        const int r0 = __builtin_amdgcn_readlane(row0, c);
        for (int i = pl; i < n; i += 64) sm.tbl[at + i] = r0 + i;
      }
      // claims of the batch's slots: open, except that a segment carried over
      // from the last batch stays with the half that holds its running state
      for (int i = pl; i < HV * (SLOTS + 1); i += 64) {
        (&sm.hslot[0][0])[i] = -1;
        (&sm.hlock[0][0])[i] = 0;
      }
      if (pl == 0) {
        const int ch = sm.carry_half;
        if (bst >= 0) { sm.hslot[ch][0] = 0; sm.hlock[ch][0] = 1; }
        sm.next_slot = bst >= 0 ? 1 : 0;
        sm.bcount = cnt;
        sm.bnext_m = trunc ? bm : bm + cnt;
        sm.bnext_st = trunc ? b : -1;
      }
      if (pl == cnt - 1) sm.bused = incl;
    }
    __syncthreads();
    const int nslot = uniform(sm.bcount);
    bm = uniform(sm.bnext_m);
    bst = uniform(sm.bnext_st);

    // ---- stage block ids and queries of the batch ------------------------------------
    // Every load is issued before any is used, so staging costs one memory
    // round trip: block ids (clamped into the pool) over their table indices,
    // and the G query rows of D * EQ bytes of each slot, 16 bytes at a time.
    {
      constexpr int QV = D * EQ / 16;
      constexpr int TPT = PD_TBL / NTH;                              // table entries per thread
      constexpr int QPT = (SLOTS * G * QV + NTH - 1) / NTH;          // query pieces per thread
      static_assert(TPT >= 1 && TPT <= 8 && QPT <= 8, "staging registers");
      const int ntbl = uniform(sm.bused), nq = nslot * G * QV;
      // held in vector registers (not arrays, which the compiler would place
      // in scratch memory)
      i32x8_t tv = {};
      typename std::conditional<QPT <= 4, u32x16_t, u32x32_t>::type qv = {};
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int t = tid + k * NTH;
        if (t < ntbl) tv[k] = p.block_tables[(uint32_t)sm.tbl[t]];
      }
#pragma unroll
      for (int k = 0; k < QPT; ++k) {
        const int e = tid + k * NTH;
        if (e < nq) {
          const int c = e / (G * QV), r = e % (G * QV);
          const uint8_t* qsrc =
              (const uint8_t*)p.q + ((size_t)(s0 + sm.meta[c].s) * Hq + hk * G) * D * EQ;
          const uint4 v = *(const uint4*)(qsrc + (size_t)r * 16);
          qv[4 * k] = v.x; qv[4 * k + 1] = v.y; qv[4 * k + 2] = v.z; qv[4 * k + 3] = v.w;
        }
      }
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int t = tid + k * NTH;
        const unsigned id = (unsigned)tv[k];
        if (t < ntbl) sm.tbl[t] = (int)(id > nb_max ? nb_max : id);
      }
#pragma unroll
      for (int k = 0; k < QPT; ++k) {
        const int e = tid + k * NTH;
        if (e < nq) {
          const int c = e / (G * QV), r = e % (G * QV);
          *(uint4*)&sm.q[c][r / QV][(r % QV) * 16] =
              make_uint4(qv[4 * k], qv[4 * k + 1], qv[4 * k + 2], qv[4 * k + 3]);
        }
      }
    }
    __syncthreads();

    // ---- tile stream of this wave over its half's slots --------------------------------
    // Each half takes the batch's slots one at a time, in list order, as it
    // reaches them (the first of its waves to need its k-th slot claims the
    // next unclaimed one), so a faster half simply takes more of them.  Within
    // a slot the half's 4 waves take sub-tiles round-robin from the segment's
    // first sub-tile; first_st(c) is this wave's first sub-tile >= st_a.
    auto first_st = [&](int c) -> int {
      const int st_lo = uniform(sm.meta[c].t0) >> 4, a = uniform(sm.meta[c].st_a);
      return a + (((hw - (a - st_lo)) % PD_WAVES) + PD_WAVES) % PD_WAVES;
    };
    auto claim = [&](int k) -> int {   // slot of this half's k-th segment, or -2
      int v = -1;
      if (lane == 0) {
        v = lds_load_acquire(&sm.hslot[h][k]);
        if (v == -1) {
          if (lds_exchange_acq_rel(&sm.hlock[h][k], 1) == 0) {
            const int c = __hip_atomic_fetch_add(&sm.next_slot, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
            v = c < nslot ? c : -2;
            if (v >= 0 && !sm.meta[v].fin) sm.carry_half = h;
            lds_store_release(&sm.hslot[h][k], v);
          } else {   // another wave of the half is claiming it right now
            do {
              __builtin_amdgcn_s_sleep(1);
              v = lds_load_acquire(&sm.hslot[h][k]);
            } while (v == -1);
          }
        }
      }
      return __builtin_amdgcn_readfirstlane(v);
    };
    // load cursor: the half's k-th slot lk, which is batch slot cs (-2: none
    // left; then kend = lk slots were the half's), and its sub-tile cst
    int lk = 0, cs = claim(0), cst = cs >= 0 ? first_st(cs) : 0, kend = 1 << 30;
    auto settle = [&]() {        // move the cursor to a slot with a tile left
      while (cs >= 0 && cst >= uniform(sm.meta[cs].st_b)) {
        ++lk;
        cs = claim(lk);
        if (cs >= 0) cst = first_st(cs);
      }
      if (cs < 0) kend = lk;
    };
    settle();

    auto load_tile = [&](Buf& b) {
      int phys = 0, st = 0;
      if (cs >= 0) {
        st = cst;
        const int blk = st / SPB - uniform(sm.meta[cs].st_a) / SPB;
        phys = uniform(sm.tbl[uniform(sm.meta[cs].tbl) + blk]);
        b.slot = cs;
        b.st = st;
        cst += PD_WAVES;
        settle();
      } else {
        b.slot = -1;             // past the end: re-read block 0 (keeps the load count fixed)
        b.st = 0;
      }
      tile.load(b, kbase + (size_t)phys * block_stride, vbase + (size_t)phys * block_stride,
                st % SPB);
    };
    auto set_query = [&](int c) { tile.set_query(&sm.q[c][0][0]); };

    // ---- segment ends (slots with fin = 1) ------------------------------------------------
    // A wave first does its quarter of the previous segment's merge (all waves
    // have deposited that one once they are past it), then deposits its own
    // (max, sum, acc) in the next merge area and goes on streaming: no wave
    // waits for another unless it is a whole segment ahead.
    auto finish_slot = [&](int c) {
      if (!uniform(sm.meta[c].fin)) return;  // continues in the next batch
      merge_quarter();
      const int par = uses % NPAR, gen = uses / NPAR;
      ++uses;
      spin_until(&sm.done[h][par], PD_WAVES * gen);   // the area's previous use is merged
      auto& ar = sm.u.area[h][par];
      tile.deposit(ar.m[hw], ar.l[hw], ar.acc[hw]);
      if (lane == 0)
        lds_add_release(&sm.arrived[h][par], 1);
      tile.reset();
      pend_s = s0 + uniform(sm.meta[c].s);
      pend_pp = uniform(sm.meta[c].p);
      pend_par = par;
      pend_gen = gen;
    };

    // ---- main loop: NBUF buffers, NBUF - 1 tiles in flight --------------------------------
    constexpr int NBUF = T::NBUF;
    // A half's slots are claimed in increasing batch order, so the slot whose
    // state the wave holds (the half's ck-th, batch slot cslot) is behind a
    // tile's slot exactly when cslot is smaller.
    auto slot_of = [&](int k) -> int { return uniform(sm.hslot[h][k]); };   // claimed already
    int ck = 0, cslot = kend > 0 ? slot_of(0) : (1 << 30);
    if (kend > 0) set_query(cslot);
#pragma unroll
    for (int i = 0; i + 1 < NBUF; ++i) load_tile(bufs[i]);
    auto step = [&](Buf& cb, Buf& spare) -> bool {
      load_tile(spare);
      if (cb.slot < 0) {         // past the half's last tile: finish its remaining slots
        while (ck < kend) {
          finish_slot(cslot);
          ++ck;
          if (ck < kend) cslot = slot_of(ck);
        }
        return false;
      }
      while (cslot < cb.slot) {  // every slot of the half is visited, in order, by its waves
        finish_slot(cslot);
        ++ck;
        cslot = slot_of(ck);
        set_query(cslot);
      }
      tile.compute(cb, uniform(sm.meta[cb.slot].t0), uniform(sm.meta[cb.slot].t1), p.qk_scale,
                   sm.wl[wave]);
      return true;
    };
    // the loop is left only through the exits, so every trip through the body
    // issues the same loads and each wait leaves NBUF - 1 tiles in flight
    for (;;) {
#pragma unroll
      for (int i = 0; i < NBUF; ++i)
        if (!step(bufs[i], bufs[(i + NBUF - 1) % NBUF])) goto stream_done;
    }
  stream_done:
    __syncthreads();           // the next batch plan overwrites the staged tables
    merge_quarter();           // every wave has deposited the batch's last segment
  }
}

// Grid: resident capacity, a multiple of num_kv_heads; sequences in launches
// of PD_SEQ_CHUNK.  The resident workgroups per CU of this kernel are found
// once per device (the first launch there) and kept.
template <class T>
hipError_t launch_decode_persistent(const DecodeParams& p0, hipStream_t stream) {
  static std::atomic<int> per_cu_of[PA_MAX_DEVICES];   // 0: not yet known
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= PA_MAX_DEVICES) dev = -1;
  int per_cu = dev >= 0 ? per_cu_of[dev].load(std::memory_order_relaxed) : 0;
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_persistent_kernel<T>,
                                                     64 * PD_WAVES * T::HALVES, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    if (dev >= 0) per_cu_of[dev].store(per_cu, std::memory_order_relaxed);
  }
  const int cus = device_cu_count(dev);
  const int H = p0.num_kv_heads;
  DecodeParams p = p0;
  for (int s0 = 0; s0 < p0.num_seqs; s0 += PD_SEQ_CHUNK) {
    p.seq_begin = s0;
    p.seq_count = min(PD_SEQ_CHUNK, p0.num_seqs - s0);
    const long long work = (long long)p.seq_count * (p.partition_size > 0 ? p.max_parts : 1);
    long long J = ((long long)cus * per_cu + H - 1) / H;
    if (J > work) J = work;
    if (J < 1) J = 1;
    hipLaunchKernelGGL((decode_persistent_kernel<T>), dim3((unsigned)(J * H)),
                       dim3(64 * PD_WAVES * T::HALVES), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pa
