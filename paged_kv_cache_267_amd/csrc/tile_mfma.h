// tile_mfma.h -- one 16-token sub-tile of paged decode attention on the gfx950
// matrix cores (tile policy of decode_persistent.h; bf16 or E4M3 caches, bf16
// queries).
//
// Both contractions run on MFMA ("vLLM 0.5 deep dive: PagedAttention
// architecture", chenxutan.com, s2.3: scaled scores, running max and sum, the
// softmax-weighted sum of V):
//   S^T = K . Q^T     v_mfma_f32_16x16x32_bf16: A = K (16 tokens x 32 dims, the
//                     16-byte K groups exactly as they sit in the cache),
//                     B = Q^T (32 dims x 16 heads; heads >= G are zero);
//   O^T += V^T . P^T  v_mfma_f32_16x16x16_bf16: A = V^T (16 dims x 16 tokens,
//                     4 consecutive tokens of one V row per lane), B = P^T.
// Heads sit on the N axis, so lane l owns head l%16 in every fragment: the S^T
// C-fragment is bit for bit the P^T B-fragment, and a head's running max, sum
// and rescale are lane-local.  The running max is updated lazily:
// accumulators are rescaled only when a head's max grows by more than 2^8, so
// p <= 256; a sub-tile finds that by comparing its scores with the reference
// (one ballot), and only then forms the column max over the 4 lane rows (two
// permlane swaps), the only cross-lane step.  E4M3 codes are converted to bf16 in registers
// (exact; "vLLM 0.7.2 deep dive: PagedAttention v2 with FlashAttention-3",
// jsqmd.com, s2.2); k_scale is folded into the score scale, v_scale applied at
// the merge.
#pragma once

#include "common.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr float LAZY_RESCALE_LOG2 = 8.0f;

__device__ __forceinline__ float colmax4(float x) {
  // max over the 4 lane rows of a column (lanes l, l^16, l^32, l^48)
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float colsum4(float x) {
  const float y = swap_add32(x, x);
  return swap_add16(y, y);
}

template <int KV_, int D_, int BS_, int G_>
struct MfmaTile {
  static constexpr int KV = KV_, D = D_, BS = BS_, G = G_;
  static_assert(KV == KV_BF16 || KV == KV_FP8, "matrix path takes bf16 or E4M3 caches");
  static constexpr int E = KvTraits<KV>::E;
  static constexpr int EQ = 2;                 // bf16 queries
  static constexpr bool OUT_F32 = false;
  static constexpr int KS = D / 32;            // QK k-steps of 32 dims
  static constexpr int NB = D / 16;            // PV n-blocks of 16 dims
  static constexpr int KL = D * E / 64;        // 16-byte K loads per lane per sub-tile
  static constexpr int VW = E;                 // V dwords per lane per n-block (bf16 2, E4M3 1)
  static constexpr int SPB = BS / 16;
  // register buffers: NBUF - 1 sub-tiles in flight while one is computed
  // (E4M3 sub-tiles are half the bytes, so twice as many)
  static constexpr int NBUF = KV == KV_FP8 ? 5 : 3;
  // staged query row: 16 bf16 of padding make the row stride 8 (mod 32)
  // dwords, the stride at which set_query's 16-byte reads of 8 heads x 4 lane
  // rows met the fewest LDS bank conflicts (strides of 0 / 4 / 8 / 12 / 16
  // mod 32 dwords, SQ_LDS_BANK_CONFLICT per LDS instruction on the G = 8
  // workloads: 0.56 / 0.11 / 0.026 / 0.11 / 0.026)
  static constexpr int QROWB = (D + 16) * 2;
  static constexpr int QBYTES = G == 8 ? 57344 : G > 8 ? 32768 : 65536;
  static constexpr int NPAR = G <= 8 ? 2 : 1;  // merge areas that fit next to the rest
  static constexpr int HALVES = 2;             // two 4-wave halves per workgroup

  struct Buf {
    uint4 k[KL];
    uint32_t v[NB][VW];
    int slot;   // segment slot in the batch (-1: no tile)
    int st;     // sub-tile index
  };
  struct WaveLds { int unused; };

  f32x4_t acc[NB];
  float m_ref, l_run;
  bf16x8_t qop[KS];

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    m_ref = -INFINITY;
    l_run = 0.f;
  }

  // Issue the loads of sub-tile `sub` of the (block, head) tiles at kt / vt.
  __device__ __forceinline__ void load(Buf& b, const char* kt, const char* vt, int sub) {
    const int lane = threadIdx.x & 63, row = lane >> 4, col = lane & 15;
    const char* kp = kt + sub * 256 + (row * BS + col) * 16;
    const char* vp = vt + sub * 16 * E + (col * BS + 4 * row) * E;
#pragma unroll
    for (int i = 0; i < KL; ++i) b.k[i] = load_nt16(kp + i * 4 * BS * 16);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const char* a = vp + (size_t)nb * 16 * BS * E;
      // a 32-token block's V row is shared by its two sub-tiles, which run on
      // different waves: ordinary loads keep the line in L2 for the other
      // half; 16-token rows are used whole and stream past L2
      if (VW == 2) {
        const u32x2_t t = SPB == 1 ? __builtin_nontemporal_load((const u32x2_t*)a)
                                   : *(const u32x2_t*)a;
        b.v[nb][0] = t.x;
        b.v[nb][VW - 1] = t.y;
      } else {
        b.v[nb][0] = SPB == 1 ? __builtin_nontemporal_load((const uint32_t*)a)
                              : *(const uint32_t*)a;
      }
    }
  }

  // Query operand (B of S^T = K . Q^T) from the staged rows [G][QROWB].
  __device__ __forceinline__ void set_query(const uint8_t* qs) {
    const int lane = threadIdx.x & 63, row = lane >> 4, col = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = (KV == KV_BF16) ? 32 * ks + 8 * row : 16 * (row + 4 * (ks >> 1)) + 8 * (ks & 1);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < G) v = *(const uint4*)(qs + col * QROWB + d0 * 2);
      qop[ks] = __builtin_bit_cast(bf16x8_t, (u32x4_t){v.x, v.y, v.z, v.w});
    }
  }

  __device__ __forceinline__ void compute(Buf& b, int t0, int t1, float qk_scale, WaveLds&) {
    const int lane = threadIdx.x & 63, row = lane >> 4;
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      if (KV == KV_BF16) {
        const bf16x8_t kop =
            __builtin_bit_cast(bf16x8_t, (u32x4_t){b.k[i].x, b.k[i].y, b.k[i].z, b.k[i].w});
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[i], sacc, 0, 0, 0);
      } else {
        const u32x4_t lo4 = {fp8x2_to_bf16x2<false>(b.k[i].x), fp8x2_to_bf16x2<true>(b.k[i].x),
                             fp8x2_to_bf16x2<false>(b.k[i].y), fp8x2_to_bf16x2<true>(b.k[i].y)};
        const u32x4_t hi4 = {fp8x2_to_bf16x2<false>(b.k[i].z), fp8x2_to_bf16x2<true>(b.k[i].z),
                             fp8x2_to_bf16x2<false>(b.k[i].w), fp8x2_to_bf16x2<true>(b.k[i].w)};
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lo4),
                                                       qop[2 * i], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, hi4),
                                                       qop[2 * i + 1], sacc, 0, 0, 0);
      }
    }
    float sc[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sc[jj] = sacc[jj] * qk_scale;

    const int st = b.st;
    if ((st * 16 < t0) || (st * 16 + 16 > t1)) {  // partial sub-tile: mask scores, zero V
      uint32_t vmask[VW];
#pragma unroll
      for (int w = 0; w < VW; ++w) vmask[w] = 0u;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int tok = st * 16 + 4 * row + jj;
        const bool ok = tok >= t0 && tok < t1;
        if (!ok) sc[jj] = -INFINITY;
        if (ok) {
          if (KV == KV_BF16) vmask[jj >> 1] |= 0xffffu << (16 * (jj & 1));
          else vmask[0] |= 0xffu << (8 * jj);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int w = 0; w < VW; ++w) b.v[nb][w] &= vmask[w];
    }

    // only a score more than 2^8 above the reference calls for a rescale, so
    // the column max is formed only when some lane holds one
    const float thr = m_ref + LAZY_RESCALE_LOG2;
    const bool over = sc[0] > thr || sc[1] > thr || sc[2] > thr || sc[3] > thr;
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      const float cmax = colmax4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      const float m_new = fmaxf(m_ref, cmax);
      const float alpha = fast_exp2(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] *= alpha;
      m_ref = m_new;
    }
    float pr[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) pr[jj] = fast_exp2(sc[jj] - m_ref);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const s16x4_t pop = __builtin_bit_cast(
        s16x4_t, (u32x2_t){pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      u32x2_t vv;
      if (KV == KV_BF16) vv = (u32x2_t){b.v[nb][0], b.v[nb][VW - 1]};
      else vv = (u32x2_t){fp8x2_to_bf16x2<false>(b.v[nb][0]), fp8x2_to_bf16x2<true>(b.v[nb][0])};
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, vv), pop,
                                                         acc[nb], 0, 0, 0);
    }
  }

  // This wave's (max, sum, acc) of the segment into its rows of a merge area.
  __device__ __forceinline__ void deposit(float* m, float* l, float (*accw)[D + 4]) {
    const int lane = threadIdx.x & 63, row = lane >> 4, col = lane & 15;
    const float l_col = colsum4(l_run);
    if (col < G) {
      if (row == 0) {
        m[col] = m_ref;
        l[col] = l_col;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) *(f32x4_t*)&accw[col][16 * nb + 4 * row] = acc[nb];
    }
  }
};

}  // namespace pa
