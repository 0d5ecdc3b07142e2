// tile_valu.h -- one 16-token sub-tile of paged decode attention on the VALU
// (tile policy of decode_persistent.h; f32, bf16 or E4M3 caches).
//
// What it computes follows "vLLM 0.5 deep dive: PagedAttention architecture"
// (chenxutan.com) s2.3: the query's scaled dot products with the keys, a
// softmax kept stable by a running max and sum, and the softmax-weighted sum of
// the values; grouped-query heads and the E4M3 cache are those of "vLLM 0.7.2
// deep dive: PagedAttention v2 with FlashAttention-3" (jsqmd.com) s2.2.
//
// Lane (row r, column o) of a wave holds token o of the sub-tile and its
// 16-byte K groups r, r+4, ...: partial dot products for all G query heads
// come from one K read (bf16 v_dot2_f32_bf16, E4M3 converted to bf16 pairs
// first, fp32 FMA for f32 caches).  Two cross-row swap-adds fold the 4 rows so
// that each row ends with its own share of the G heads, fully summed
// (transpose-reduce).  The softmax is base-2 (log2 e folded into the score
// scale) against a per-head reference raised lazily: only when a score exceeds
// it by more than 2^8 are the 16-lane DPP row maxima and the rescale factors
// formed.  p goes to a per-wave LDS slot (bf16 pairs, fp32 for f32 caches),
// with the rescale factors when there are any, and P.V accumulates with
// v_dot2_f32_bf16 (fp32 FMA) into per-lane fp32 accumulators: lane l owns
// 16-byte pieces l, l+64, ... of the V sub-tile.
#pragma once

#include "common.h"

namespace pa {

// Query head index held in slot kk of a lane in row r after the fold.
template <int G>
__device__ __forceinline__ int folded_head(int r, int kk) {
  if (G >= 4) return r * (G / 4) + kk;
  if (G == 2) return r >> 1;
  return 0;
}

// The reference max of a head is raised only when a score exceeds it by more
// than 2^VALU_LAZY_LOG2 (base 2), so weights stay below 2^8.
constexpr float VALU_LAZY_LOG2 = 8.0f;

template <int KV_, int D_, int BS_, int G_>
struct ValuTile {
  static constexpr int KV = KV_, D = D_, BS = BS_, G = G_;
  static_assert(G <= 8, "vector-ALU path serves up to 8 query heads per KV head");
  static constexpr int E = KvTraits<KV>::E;
  static constexpr int EQ = KV == KV_F32 ? 4 : 2;          // f32 or bf16 queries
  static constexpr bool OUT_F32 = KV == KV_F32;
  static constexpr int X = 16 / E;                         // elements per 16-byte group
  static constexpr int C = D / X;                          // 16-byte K groups per token
  static constexpr int KPL = C / 4;                        // K loads per lane per sub-tile
  static constexpr int VPL = D * E / 64;                   // V loads per lane per sub-tile
  static constexpr int NGL = G >= 4 ? G / 4 : 1;           // heads per lane after the fold
  static constexpr int SPB = BS / 16;
  static constexpr int QW = KV == KV_F32 ? 4 : X / 2;      // query words per (head, K group)
  static constexpr int PW = KV == KV_F32 ? 16 : 8;         // P words per head in LDS
  // register buffers (sub-tile bytes per lane: f32 256, bf16 128, E4M3 64)
  static constexpr int NBUF = KV == KV_F32 ? 2 : KV == KV_FP8 ? 4 : 3;
  static constexpr int QROWB = D * EQ + 16;                // staged query row bytes
  static constexpr int NPAR = 2;
  // two 4-wave halves per workgroup where two waves per SIMD fit in registers
  static constexpr int HALVES = (G <= 4 && !(KV == KV_F32 && D == 128 && G > 1)) ? 2 : 1;
  // staged query bytes: E4M3 segments are cheap to stream, so a batch holds more of them
  static constexpr int QBYTES = (KV == KV_FP8 && HALVES == 2) ? 65536 : 16384;
  static_assert(C % 4 == 0 && VPL >= 1, "head_dim too small for this element size");

  struct Buf {
    uint4 k[KPL];
    uint4 v[VPL];
    int slot;   // segment slot in the batch (-1: no tile)
    int st;     // sub-tile index
  };
  struct WaveLds {
    alignas(16) uint32_t p[G][PW];   // this sub-tile's p per head
    float alpha[G];                  // rescale factor per head
  };

  uint32_t qr[G][KPL][QW];
  float m_run[NGL], l_run[NGL];
  float acc[G][VPL];

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int kk = 0; kk < NGL; ++kk) { m_run[kk] = -INFINITY; l_run[kk] = 0.f; }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int k = 0; k < VPL; ++k) acc[g][k] = 0.f;
  }

  __device__ __forceinline__ void load(Buf& b, const char* kt, const char* vt, int sub) {
    const int lane = threadIdx.x & 63, row = lane >> 4, col = lane & 15;
    const char* kp = kt + sub * 256 + (row * BS + col) * 16;
    const char* vp = vt + sub * 16 * E;
#pragma unroll
    for (int i = 0; i < KPL; ++i) b.k[i] = load_nt16(kp + i * 4 * BS * 16);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int n = lane + 64 * k;  // 16-byte V piece: row d = n / E, part n % E
      const char* a = vp + (n / E) * BS * E + 16 * (n % E);
      // a 32-token block's V row is shared by its two sub-tiles (other waves):
      // ordinary loads keep the line in L2 for the other half
      if (SPB == 1) {
        b.v[k] = load_nt16(a);
      } else {
        const u32x4_t t = *(const u32x4_t*)a;
        b.v[k] = make_uint4(t.x, t.y, t.z, t.w);
      }
    }
  }

  // The query words of this lane's K groups, for all G heads, from the staged
  // rows [G][QROWB].
  __device__ __forceinline__ void set_query(const uint8_t* qs) {
    const int row = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const uint8_t* src = qs + g * QROWB + (row + 4 * i) * X * EQ;
#pragma unroll
        for (int w = 0; w < QW; w += 4) {
          const uint4 v = *(const uint4*)(src + 4 * w);
          qr[g][i][w] = v.x; qr[g][i][w + 1] = v.y; qr[g][i][w + 2] = v.z; qr[g][i][w + 3] = v.w;
        }
      }
  }

  __device__ __forceinline__ void compute(Buf& b, int t0, int t1, float qk_scale, WaveLds& wl) {
    const int lane = threadIdx.x & 63, row = lane >> 4, col = lane & 15;
    const int vpart = lane % E;  // which 16-byte part of a V row (tokens vpart * X ..)
    const int st = b.st;
    // QK^T partials for all G heads
    float part_s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) part_s[g] = 0.f;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const uint32_t kw[4] = {b.k[i].x, b.k[i].y, b.k[i].z, b.k[i].w};
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
    constexpr int N1 = G >= 2 ? G / 2 : 1;
    float f1[N1];
    if (G >= 2) {
#pragma unroll
      for (int k = 0; k < G / 2; ++k) f1[k] = swap_add32(part_s[k], part_s[k + G / 2]);
    } else {
      f1[0] = swap_add32(part_s[0], part_s[0]);
    }
    float sc[NGL];
    if (N1 >= 2) {
#pragma unroll
      for (int k = 0; k < N1 / 2; ++k) sc[k] = swap_add16(f1[k], f1[k + N1 / 2]);
    } else {
      sc[0] = swap_add16(f1[0], f1[0]);
    }

    // mask and online softmax (base 2); every sub-tile holds a valid token.
    // The reference max is raised lazily: only when a score exceeds it by
    // more than 2^8 (one ballot over the wave) are the sub-tile's row maxima,
    // the new references and the rescale factors formed; otherwise the
    // weights are taken against the references as they stand, and the
    // accumulators keep their scale.
    const int tok = st * 16 + col;
    const bool valid = tok >= t0 && tok < t1;
    float xs[NGL];
    bool over = false;
#pragma unroll
    for (int kk = 0; kk < NGL; ++kk) {
      xs[kk] = valid ? sc[kk] * qk_scale : -INFINITY;
      over |= xs[kk] > m_run[kk] + VALU_LAZY_LOG2;
    }
    const bool rescale = __builtin_amdgcn_ballot_w64(over) != 0;
    if (rescale) {
#pragma unroll
      for (int kk = 0; kk < NGL; ++kk) {
        const float m_new = fmaxf(m_run[kk], row_max16(xs[kk]));
        const float alpha = fast_exp2(m_run[kk] - m_new);
        l_run[kk] *= alpha;
        m_run[kk] = m_new;
        if (col == 0) wl.alpha[folded_head<G>(row, kk)] = alpha;
      }
    }
#pragma unroll
    for (int kk = 0; kk < NGL; ++kk) {
      const float pv = fast_exp2(xs[kk] - m_run[kk]);
      l_run[kk] += pv;
      const int g = folded_head<G>(row, kk);
      if (KV == KV_F32) {
        wl.p[g][col] = __float_as_uint(pv);
      } else {
        const float nb = dpp<DPP_XOR1>(pv);
        const uint32_t pair = (col & 1) ? pack_bf16x2(nb, pv) : pack_bf16x2(pv, nb);
        wl.p[g][col >> 1] = pair;
      }
    }

    // zero V elements of tokens outside [t0, t1) (tail slots may hold NaN)
    if ((st * 16 < t0) || (st * 16 + 16 > t1)) {
      const int a = t0 - st * 16, e = t1 - st * 16;  // valid tokens: a <= u < e
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        uint32_t w[4] = {b.v[k].x, b.v[k].y, b.v[k].z, b.v[k].w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (KV == KV_F32) {
            const int u = vpart * 4 + jj;
            if (!(u >= a && u < e)) w[jj] = 0u;
          } else if (KV == KV_BF16) {
            const int u = vpart * 8 + 2 * jj;
            uint32_t msk = 0u;
            if (u >= a && u < e) msk |= 0x0000ffffu;
            if (u + 1 >= a && u + 1 < e) msk |= 0xffff0000u;
            w[jj] &= msk;
          } else {
            const int u = 4 * jj;
            uint32_t msk = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (u + q >= a && u + q < e) msk |= 0xffu << (8 * q);
            w[jj] &= msk;
          }
        }
        b.v[k] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }

    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // rescale (when the references moved) and accumulate P.V
    if (rescale) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float al = wl.alpha[g];
#pragma unroll
        for (int k = 0; k < VPL; ++k) acc[g][k] *= al;
      }
    }
    if (KV == KV_F32) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float4 pp = *(const float4*)&wl.p[g][vpart * 4];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          acc[g][k] = fmaf(pp.x, __uint_as_float(b.v[k].x), acc[g][k]);
          acc[g][k] = fmaf(pp.y, __uint_as_float(b.v[k].y), acc[g][k]);
          acc[g][k] = fmaf(pp.z, __uint_as_float(b.v[k].z), acc[g][k]);
          acc[g][k] = fmaf(pp.w, __uint_as_float(b.v[k].w), acc[g][k]);
        }
      }
    } else if (KV == KV_BF16) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 pp = *(const uint4*)&wl.p[g][vpart * 4];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          acc[g][k] = dot2_bf16(pp.x, b.v[k].x, acc[g][k]);
          acc[g][k] = dot2_bf16(pp.y, b.v[k].y, acc[g][k]);
          acc[g][k] = dot2_bf16(pp.z, b.v[k].z, acc[g][k]);
          acc[g][k] = dot2_bf16(pp.w, b.v[k].w, acc[g][k]);
        }
      }
    } else {
      // E4M3 V: 16 tokens of one row per piece, converted to bf16 pairs once
      uint32_t vw[VPL][8];
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        const uint32_t w[4] = {b.v[k].x, b.v[k].y, b.v[k].z, b.v[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          vw[k][2 * q] = fp8x2_to_bf16x2<false>(w[q]);
          vw[k][2 * q + 1] = fp8x2_to_bf16x2<true>(w[q]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 p0 = *(const uint4*)&wl.p[g][0];
        const uint4 p1 = *(const uint4*)&wl.p[g][4];
        const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int k = 0; k < VPL; ++k)
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[g][k] = dot2_bf16(pw[q], vw[k][q], acc[g][k]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // This wave's (max, sum, acc) of the segment into its rows of a merge area.
  __device__ __forceinline__ void deposit(float* m, float* l, float (*accw)[D + 4]) {
    const int lane = threadIdx.x & 63, row = lane >> 4, col = lane & 15;
    const int vpart = lane % E;
#pragma unroll
    for (int kk = 0; kk < NGL; ++kk) {
      const float lsum = row_sum16(l_run[kk]);
      const int g = folded_head<G>(row, kk);
      if (col == 0) {
        m[g] = m_run[kk];
        l[g] = lsum;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        float a = acc[g][k];
        if (E >= 2) a += dpp<DPP_XOR1>(a);
        if (E >= 4) a += dpp<DPP_XOR2>(a);
        if (vpart == 0) accw[g][(lane + 64 * k) / E] = a;
      }
  }
};

}  // namespace pa
