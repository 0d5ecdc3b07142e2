// decode_valu.h -- paged decode attention, bandwidth (VALU) path for gfx950.
//
// What it computes follows "vLLM 0.5 deep dive: PagedAttention architecture"
// (chenxutan.com) s2.2-s2.3: for each sequence the query's scaled dot products
// with every cached key, reached block by block through the block table, a
// softmax kept stable by a running max and sum, and the softmax-weighted sum
// of the values.  Grouped-query heads and the FP8 e4m3 cache are those of
// "vLLM 0.7.2 deep dive: PagedAttention v2 with FlashAttention-3" (jsqmd.com)
// s2.2; the sliding window (mask keys outside it, never load blocks wholly
// outside it) is its s2.3.
//
// Work decomposition (one workgroup per (KV head, partition, sequence)):
//   blockIdx.x = KV head  -- workgroups are dealt to the 8 XCDs round-robin, so
//                            with 8 KV heads every XCD serves one head and a
//                            prefix shared by many sequences stays in that
//                            XCD's L2;
//   blockIdx.y = partition of partition_size tokens (split) or 0 (unsplit);
//   blockIdx.z = sequence.
// The workgroup copies its slice of the block table into LDS, then its waves
// walk 16-token sub-tiles of the KV range round-robin.  Per sub-tile a wave
//   - loads the K sub-tile (16 tokens x D) and the V sub-tile with 16-byte
//     non-temporal loads, two sub-tiles ahead of the one being computed;
//   - lane (row r, column o): token o, 16-byte K groups r, r+4, ... -> partial
//     dot products for all G query heads of the KV head from one K read;
//   - folds partials over the 4 rows with two cross-row swap-adds that leave
//     each row with its own share of the G heads (transpose-reduce);
//   - masks, takes a 16-lane DPP max, updates the running max / sum (base-2
//     exponentials, log2(e) folded into the score scale);
//   - publishes p (bf16 pairs, or fp32 for f32 caches) and the rescale factors
//     to a per-wave LDS slot and accumulates p.V with bf16 dot2 (fp32 FMAs for
//     f32 caches) into per-lane fp32 accumulators.
// Waves merge (max, sum, acc) through LDS at the end and write either the
// normalised output (unsplit) or the partition's output and natural-log LSE.
#pragma once

#include "common.h"

namespace pa {

constexpr int VALU_MAX_WAVES = 4;
constexpr int TBL_CAP = 512;  // block-table entries staged in LDS per chunk

template <int KV, int D, int BS, int G>
struct ValuCfg {
  static constexpr int E = KvTraits<KV>::E;
  static constexpr int X = 16 / E;             // elements per 16-byte group
  static constexpr int C = D / X;              // 16-byte K groups per token
  static constexpr int KPL = C / 4;            // K loads per lane per sub-tile
  static constexpr int VPL = D * E / 64;       // V loads per lane per sub-tile
  static constexpr int NGL = G >= 4 ? G / 4 : 1;  // heads per lane after the fold
  static constexpr int SPB = BS / 16;          // 16-token sub-tiles per block
  // query words per (head, K group): f32 -> 4 floats; bf16 query -> X/2 pairs
  static constexpr int QW = KV == KV_F32 ? 4 : X / 2;
  static constexpr int PW = KV == KV_F32 ? 16 : 8;  // P words per head in LDS
  static_assert(C % 4 == 0, "head_dim too small for this element size");
  static_assert(VPL >= 1, "head_dim too small");
};

template <int KV, int D, int BS, int G>
struct ValuSmem {
  using Cfg = ValuCfg<KV, D, BS, G>;
  int32_t table[TBL_CAP];
  uint32_t p[VALU_MAX_WAVES][G][Cfg::PW];
  float alpha[VALU_MAX_WAVES][G];
  float m[VALU_MAX_WAVES][G];
  float l[VALU_MAX_WAVES][G];
  float acc[VALU_MAX_WAVES][G][D];
};

// Query head index held in slot kk of a lane in row r after the fold.
template <int G>
__device__ __forceinline__ int folded_head(int r, int kk) {
  if (G >= 4) return r * (G / 4) + kk;
  if (G == 2) return r >> 1;
  return 0;
}

template <int KV, int D, int BS, int G>
__global__ __launch_bounds__(64 * VALU_MAX_WAVES) void decode_valu_kernel(DecodeParams p) {
  using Cfg = ValuCfg<KV, D, BS, G>;
  constexpr int E = Cfg::E, X = Cfg::X, KPL = Cfg::KPL, VPL = Cfg::VPL, NGL = Cfg::NGL;
  constexpr int SPB = Cfg::SPB, QW = Cfg::QW, PW = Cfg::PW;
  constexpr size_t TILE_BYTES = (size_t)D * BS * E;  // one (block, head) tile

  __shared__ ValuSmem<KV, D, BS, G> sm;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int nw = uniform((int)(blockDim.x >> 6));
  const int row = lane >> 4, col = lane & 15;
  const int hk = blockIdx.x, part = blockIdx.y, s = blockIdx.z;
  const int Hq = p.num_q_heads;

  // ---- token range of this workgroup ---------------------------------------
  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.max_blocks * BS ? p.max_blocks * BS : L);
  const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
  int t0 = lo, t1 = L;
  if (p.partition_size > 0) {
    t0 = max(lo, part * p.partition_size);
    t1 = min(L, (part + 1) * p.partition_size);
  }
  if (t0 >= t1) {  // empty: zero row (unsplit) or LSE = -inf (split)
    if (p.part_out == nullptr) {
      for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
        size_t o = ((size_t)s * Hq + hk * G + i / D) * D + i % D;
        if (KV == KV_F32) ((float*)p.out)[o] = 0.f;
        else ((uint16_t*)p.out)[o] = 0;
      }
    } else if (threadIdx.x < G) {
      p.part_lse[((size_t)s * Hq + hk * G + threadIdx.x) * p.max_parts + part] = -INFINITY;
    }
    return;
  }

  // ---- query: the 16-byte groups this lane's K loads cover, for all G heads --
  uint32_t qr[G][KPL][QW];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int grp = row + 4 * i;  // K group index = head_dim / X
      if (KV == KV_F32) {
        const uint4 v = *(const uint4*)((const float*)p.q + ((size_t)s * Hq + hk * G + g) * D +
                                        grp * 4);
        qr[g][i][0] = v.x; qr[g][i][1] = v.y; qr[g][i][2] = v.z; qr[g][i][3] = v.w;
      } else {
        const uint16_t* qb = (const uint16_t*)p.q + ((size_t)s * Hq + hk * G + g) * D + grp * X;
#pragma unroll
        for (int w = 0; w < QW; w += 4) {
          const uint4 v = *(const uint4*)(qb + 2 * w);
          qr[g][i][w] = v.x; qr[g][i][w + 1] = v.y; qr[g][i][w + 2] = v.z; qr[g][i][w + 3] = v.w;
        }
      }
    }
  }

  // ---- running state ---------------------------------------------------------
  float m_run[NGL], l_run[NGL];
  float acc[G][VPL];
#pragma unroll
  for (int kk = 0; kk < NGL; ++kk) { m_run[kk] = -INFINITY; l_run[kk] = 0.f; }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int k = 0; k < VPL; ++k) acc[g][k] = 0.f;

  const char* kbase = (const char*)p.kc + (size_t)hk * TILE_BYTES;
  const char* vbase = (const char*)p.vc + (size_t)hk * TILE_BYTES;
  const size_t block_stride = (size_t)p.num_kv_heads * TILE_BYTES;
  const int32_t* table_row = p.block_tables + (size_t)s * p.max_blocks;
  const unsigned nb_max = (unsigned)(p.num_blocks - 1);

  // lane byte offsets inside a sub-tile
  uint32_t koff[KPL], voff[VPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) koff[i] = (uint32_t)(((row + 4 * i) * BS + col) * 16);
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int n = lane + 64 * k;  // 16-byte V chunk index: row d = n / E, part c = n % E
    voff[k] = (uint32_t)((n / E) * BS * E + 16 * (n % E));
  }
  const int vpart = lane % E;  // which 16-byte part of a V row (tokens vpart*X ..)

  const int st_lo = t0 >> 4, st_hi = (t1 + 15) >> 4;
  const int b_lo = st_lo / SPB, b_hi = (st_hi + SPB - 1) / SPB;

  uint4 kb0[KPL], vb0[VPL], kb1[KPL], vb1[VPL], kb2[KPL], vb2[VPL];

  auto load_tile = [&](uint4* kb, uint4* vb, int st, int tbl_base) {
    const int blk = st / SPB;
    const int phys = uniform(sm.table[blk - tbl_base]);
    const int sub = st % SPB;
    const char* kp = kbase + (size_t)phys * block_stride + sub * 256;
    const char* vp = vbase + (size_t)phys * block_stride + sub * 16 * E;
    // K/V are read once per call: non-temporal loads keep them from evicting
    // the block table, query and shared-prefix lines from L2
#pragma unroll
    for (int i = 0; i < KPL; ++i) kb[i] = load_nt16(kp + koff[i]);
#pragma unroll
    for (int k = 0; k < VPL; ++k) vb[k] = load_nt16(vp + voff[k]);
  };

  uint32_t* pw = &sm.p[wave][0][0];
  float* aw = &sm.alpha[wave][0];

  auto compute_tile = [&](const uint4* kb, uint4* vb, int st) {
    // QK^T partials for all G heads
    float part_s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) part_s[g] = 0.f;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const uint32_t kw[4] = {kb[i].x, kb[i].y, kb[i].z, kb[i].w};
      if (KV == KV_F32) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            part_s[g] = fmaf(__uint_as_float(qr[g][i][w]), __uint_as_float(kw[w]), part_s[g]);
      } else if (KV == KV_BF16) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int w = 0; w < 4; ++w) part_s[g] = dot2_bf16(qr[g][i][w], kw[w], part_s[g]);
      } else {
        uint32_t kp[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          kp[2 * w] = fp8x2_to_bf16x2<false>(kw[w]);
          kp[2 * w + 1] = fp8x2_to_bf16x2<true>(kw[w]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int w = 0; w < 8; ++w) part_s[g] = dot2_bf16(qr[g][i][w], kp[w], part_s[g]);
      }
    }
    // fold over the 4 rows: lane keeps the heads of its row, fully summed
    // (lower half keeps heads [0, G/2), upper half [G/2, G); then even rows
    //  keep the first half of those, odd rows the second)
    float f1[G >= 2 ? G / 2 : 1];
    if (G >= 2) {
#pragma unroll
      for (int k = 0; k < G / 2; ++k) f1[k] = swap_add32(part_s[k], part_s[k + G / 2]);
    } else {
      f1[0] = swap_add32(part_s[0], part_s[0]);
    }
    constexpr int N1 = G >= 2 ? G / 2 : 1;
    float sc[NGL];
    if (N1 >= 2) {
#pragma unroll
      for (int k = 0; k < N1 / 2; ++k) sc[k] = swap_add16(f1[k], f1[k + N1 / 2]);
    } else {
      sc[0] = swap_add16(f1[0], f1[0]);
    }

    // mask and online softmax (base 2)
    const int tok = st * 16 + col;
    const bool valid = tok >= t0 && tok < t1;
    float pv[NGL];
#pragma unroll
    for (int kk = 0; kk < NGL; ++kk) {
      const float x = valid ? sc[kk] * p.qk_scale : -INFINITY;
      const float tmax = row_max16(x);
      const float m_new = fmaxf(m_run[kk], tmax);
      const float alpha = fast_exp2(m_run[kk] - m_new);
      pv[kk] = fast_exp2(x - m_new);
      l_run[kk] = l_run[kk] * alpha + pv[kk];
      m_run[kk] = m_new;
      const int g = folded_head<G>(row, kk);
      if (col == 0) aw[g] = alpha;
      if (KV == KV_F32) {
        pw[g * PW + col] = __float_as_uint(pv[kk]);
      } else {
        const float nb = dpp<DPP_XOR1>(pv[kk]);
        const uint32_t pair = (col & 1) ? pack_bf16x2(nb, pv[kk]) : pack_bf16x2(pv[kk], nb);
        pw[g * PW + (col >> 1)] = pair;
      }
    }

    // zero V elements of tokens outside [t0, t1) (tail slots may hold NaN)
    const bool partial = (st * 16 < t0) || (st * 16 + 16 > t1);
    if (partial) {
      const int a = t0 - st * 16, b = t1 - st * 16;  // valid tokens: a <= u < b
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        uint32_t w[4] = {vb[k].x, vb[k].y, vb[k].z, vb[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (KV == KV_F32) {
            const int u = vpart * 4 + j;
            if (!(u >= a && u < b)) w[j] = 0u;
          } else if (KV == KV_BF16) {
            const int u = vpart * 8 + 2 * j;
            uint32_t msk = 0u;
            if (u >= a && u < b) msk |= 0x0000ffffu;
            if (u + 1 >= a && u + 1 < b) msk |= 0xffff0000u;
            w[j] &= msk;
          } else {
            const int u = 4 * j;
            uint32_t msk = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (u + q >= a && u + q < b) msk |= 0xffu << (8 * q);
            w[j] &= msk;
          }
        }
        vb[k] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }

    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // rescale and accumulate P.V
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float al = aw[g];
#pragma unroll
      for (int k = 0; k < VPL; ++k) acc[g][k] *= al;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (KV == KV_F32) {
        const float4 pp = *(const float4*)&pw[g * PW + vpart * 4];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          acc[g][k] = fmaf(pp.x, __uint_as_float(vb[k].x), acc[g][k]);
          acc[g][k] = fmaf(pp.y, __uint_as_float(vb[k].y), acc[g][k]);
          acc[g][k] = fmaf(pp.z, __uint_as_float(vb[k].z), acc[g][k]);
          acc[g][k] = fmaf(pp.w, __uint_as_float(vb[k].w), acc[g][k]);
        }
      } else if (KV == KV_BF16) {
        const uint4 pp = *(const uint4*)&pw[g * PW + vpart * 4];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          acc[g][k] = dot2_bf16(pp.x, vb[k].x, acc[g][k]);
          acc[g][k] = dot2_bf16(pp.y, vb[k].y, acc[g][k]);
          acc[g][k] = dot2_bf16(pp.z, vb[k].z, acc[g][k]);
          acc[g][k] = dot2_bf16(pp.w, vb[k].w, acc[g][k]);
        }
      } else {
        const uint4 p0 = *(const uint4*)&pw[g * PW];
        const uint4 p1 = *(const uint4*)&pw[g * PW + 4];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          acc[g][k] = dot2_bf16(p0.x, fp8x2_to_bf16x2<false>(vb[k].x), acc[g][k]);
          acc[g][k] = dot2_bf16(p0.y, fp8x2_to_bf16x2<true>(vb[k].x), acc[g][k]);
          acc[g][k] = dot2_bf16(p0.z, fp8x2_to_bf16x2<false>(vb[k].y), acc[g][k]);
          acc[g][k] = dot2_bf16(p0.w, fp8x2_to_bf16x2<true>(vb[k].y), acc[g][k]);
          acc[g][k] = dot2_bf16(p1.x, fp8x2_to_bf16x2<false>(vb[k].z), acc[g][k]);
          acc[g][k] = dot2_bf16(p1.y, fp8x2_to_bf16x2<true>(vb[k].z), acc[g][k]);
          acc[g][k] = dot2_bf16(p1.z, fp8x2_to_bf16x2<false>(vb[k].w), acc[g][k]);
          acc[g][k] = dot2_bf16(p1.w, fp8x2_to_bf16x2<true>(vb[k].w), acc[g][k]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // ---- main loop over table chunks staged in LDS ------------------------------
  for (int cb = b_lo; cb < b_hi; cb += TBL_CAP) {
    const int ce = min(b_hi, cb + TBL_CAP);
    lds_barrier();
    for (int i = threadIdx.x; i < ce - cb; i += blockDim.x) {
      const unsigned id = (unsigned)table_row[cb + i];
      sm.table[i] = (int)(id > nb_max ? nb_max : id);
    }
    lds_barrier();
    const int cs_lo = max(st_lo, cb * SPB), cs_hi = min(st_hi, ce * SPB);
    // sub-tiles are dealt to waves round-robin by their index from st_lo
    // three register buffers: two sub-tiles in flight while one is computed
    int st = cs_lo + ((wave - (cs_lo - st_lo) % nw) + nw) % nw;
    if (st < cs_hi) load_tile(kb0, vb0, st, cb);
    if (st + nw < cs_hi) load_tile(kb1, vb1, st + nw, cb);
    while (st < cs_hi) {
      if (st + 2 * nw < cs_hi) load_tile(kb2, vb2, st + 2 * nw, cb);
      compute_tile(kb0, vb0, st);
      st += nw;
      if (st >= cs_hi) break;
      if (st + 2 * nw < cs_hi) load_tile(kb0, vb0, st + 2 * nw, cb);
      compute_tile(kb1, vb1, st);
      st += nw;
      if (st >= cs_hi) break;
      if (st + 2 * nw < cs_hi) load_tile(kb1, vb1, st + 2 * nw, cb);
      compute_tile(kb2, vb2, st);
      st += nw;
    }
  }

  // ---- wave results -> LDS ------------------------------------------------------
#pragma unroll
  for (int kk = 0; kk < NGL; ++kk) {
    const float lsum = row_sum16(l_run[kk]);
    const int g = folded_head<G>(row, kk);
    if (col == 0) {
      sm.m[wave][g] = m_run[kk];
      sm.l[wave][g] = lsum;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      float a = acc[g][k];
      if (E >= 2) a += dpp<DPP_XOR1>(a);
      if (E >= 4) a += dpp<DPP_XOR2>(a);
      if (vpart == 0) sm.acc[wave][g][(lane + 64 * k) / E] = a;
    }
  lds_barrier();

  // ---- merge waves and write ------------------------------------------------------
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int g = i / D, d = i % D;
    float mx = -INFINITY;
    for (int w = 0; w < nw; ++w) mx = fmaxf(mx, sm.m[w][g]);
    float den = 0.f, num = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float f = sm.m[w][g] == -INFINITY ? 0.f : fast_exp2(sm.m[w][g] - mx);
      den += f * sm.l[w][g];
      num += f * sm.acc[w][g][d];
    }
    const float o = num / den * p.v_scale;
    const int hq = hk * G + g;
    if (p.part_out == nullptr) {
      const size_t oi = ((size_t)s * Hq + hq) * D + d;
      if (KV == KV_F32) ((float*)p.out)[oi] = o;
      else ((uint16_t*)p.out)[oi] = to_bf16_bits(o);
    } else {
      const size_t pi = ((size_t)s * Hq + hq) * p.max_parts + part;
      p.part_out[pi * D + d] = o;
      if (d == 0) p.part_lse[pi] = (mx + __log2f(den)) * 0.69314718055994531f;
    }
  }
}

// Launch for one instance; returns the hipError_t of the launch.
template <int KV, int D, int BS, int G>
hipError_t launch_decode_valu(const DecodeParams& p, int parts, int waves, hipStream_t stream) {
  dim3 grid(p.num_kv_heads, parts, p.num_seqs);
  dim3 block(64 * waves);
  hipLaunchKernelGGL((decode_valu_kernel<KV, D, BS, G>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
