// decode_mfma.h -- paged decode attention on the gfx950 matrix cores.
//
// Same computation as the bandwidth path (decode_valu.h; sources: "vLLM 0.5
// deep dive: PagedAttention architecture", chenxutan.com, s2.2-s2.3, and
// "vLLM 0.7.2 deep dive: PagedAttention v2 with FlashAttention-3", jsqmd.com,
// s2.2-s2.3), with both contractions of a 16-token sub-tile on MFMA:
//
//   S^T = K . Q^T   v_mfma_f32_16x16x32_bf16, A = K (16 tokens x 32 dims, the
//                   16-byte K groups exactly as they sit in the cache),
//                   B = Q^T (32 dims x 16 heads; heads >= G are zero)
//   O^T += V^T . P^T  v_mfma_f32_16x16x16_bf16, A = V^T (16 dims x 16 tokens:
//                   4 consecutive tokens of one V row per lane), B = P^T.
//
// With heads on the N axis, lane l owns head l%16 in every fragment: the C
// fragment of S^T (tokens 4*(l/16)+j) is bit for bit the B fragment PV needs,
// and the running max, sum and rescale of a head are lane-local.  The only
// cross-lane step per sub-tile is the column max over the 4 lane rows (two
// permlane swaps).  The running max is updated lazily: the accumulators are
// rescaled only when a column's max grows by more than 2^8, so p <= 256.
//
// E4M3 caches: K and V codes are converted to bf16 in registers (exact) with
// the hardware pair conversion; k_scale is folded into the score scale and
// v_scale applied at the end.
#pragma once

#include "common.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int MFMA_WAVES = 4;
constexpr int MFMA_TBL_CAP = 512;
constexpr float LAZY_RESCALE_LOG2 = 8.0f;

template <int KV, int D, int G>
struct MfmaSmem {
  int32_t table[MFMA_TBL_CAP];
  float m[MFMA_WAVES][G];
  float l[MFMA_WAVES][G];
  float acc[MFMA_WAVES][G][D];
};

__device__ __forceinline__ float colmax4(float x) {
  // max over the 4 lane rows of a column (lanes l, l^16, l^32, l^48)
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float colsum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int KV, int D, int BS, int G>
__global__ __launch_bounds__(64 * MFMA_WAVES) void decode_mfma_kernel(DecodeParams p) {
  static_assert(KV == KV_BF16 || KV == KV_FP8, "matrix path takes bf16 or E4M3 caches");
  static_assert(G <= 16, "at most 16 query heads per KV head");
  constexpr int E = KvTraits<KV>::E;
  constexpr int KS = D / 32;          // QK k-steps of 32 dims
  constexpr int NB = D / 16;          // PV n-blocks of 16 dims
  constexpr int KL = D * E / 64;      // 16-byte K loads per lane per sub-tile
  constexpr int VW = 4 * E / 4;       // V dwords per lane per n-block (bf16: 2, fp8: 1)
  constexpr int SPB = BS / 16;
  constexpr size_t TILE_BYTES = (size_t)D * BS * E;

  __shared__ MfmaSmem<KV, D, G> sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int row = lane >> 4, col = lane & 15;
  const int hk = blockIdx.x, part = blockIdx.y, s = blockIdx.z;
  const int Hq = p.num_q_heads;

  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.max_blocks * BS ? p.max_blocks * BS : L);
  const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
  int t0 = lo, t1 = L;
  if (p.partition_size > 0) {
    t0 = max(lo, part * p.partition_size);
    t1 = min(L, (part + 1) * p.partition_size);
  }
  if (t0 >= t1) {
    if (p.part_out == nullptr) {
      for (int i = threadIdx.x; i < G * D; i += blockDim.x)
        ((uint16_t*)p.out)[((size_t)s * Hq + hk * G + i / D) * D + i % D] = 0;
    } else if (threadIdx.x < G) {
      p.part_lse[((size_t)s * Hq + hk * G + threadIdx.x) * p.max_parts + part] = -INFINITY;
    }
    return;
  }

  // ---- Q^T as the B operand of each QK k-step (zero for heads >= G) ----------
  bf16x8_t qop[KS];
  {
    const uint16_t* qrow = (const uint16_t*)p.q + ((size_t)s * Hq + hk * G + col) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // dims of k-step ks held by lane row r: bf16 -> 32ks + 8r; E4M3 -> the
      // matching half of 16-byte group r + 4*(ks/2)
      const int d0 = (KV == KV_BF16) ? 32 * ks + 8 * row : 16 * (row + 4 * (ks >> 1)) + 8 * (ks & 1);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < G) v = *(const uint4*)(qrow + d0);
      qop[ks] = __builtin_bit_cast(bf16x8_t, (u32x4_t){v.x, v.y, v.z, v.w});
    }
  }

  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;

  const char* kbase = (const char*)p.kc + (size_t)hk * TILE_BYTES;
  const char* vbase = (const char*)p.vc + (size_t)hk * TILE_BYTES;
  const size_t block_stride = (size_t)p.num_kv_heads * TILE_BYTES;
  const int32_t* table_row = p.block_tables + (size_t)s * p.max_blocks;
  const unsigned nb_max = (unsigned)(p.num_blocks - 1);

  uint32_t koff[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) koff[i] = (uint32_t)(((row + 4 * i) * BS + col) * 16);
  // V: row d = 16*nb + col, tokens 4*row .. 4*row+3 of the sub-tile
  const uint32_t voff0 = (uint32_t)((col * BS + 4 * row) * E);

  const int st_lo = t0 >> 4, st_hi = (t1 + 15) >> 4;
  const int b_lo = st_lo / SPB, b_hi = (st_hi + SPB - 1) / SPB;

  struct Buf {
    uint4 k[KL];
    uint32_t v[NB][VW];
  };
  Buf buf0, buf1, buf2;

  auto load_tile = [&](Buf& b, int st, int tbl_base) {
    const int phys = uniform(sm.table[st / SPB - tbl_base]);
    const int sub = st % SPB;
    const char* kp = kbase + (size_t)phys * block_stride + sub * 256;
    const char* vp = vbase + (size_t)phys * block_stride + sub * 16 * E + voff0;
#pragma unroll
    for (int i = 0; i < KL; ++i) b.k[i] = load_nt16(kp + koff[i]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const char* a = vp + (size_t)nb * 16 * BS * E;
      if (VW == 2) {
        const u32x2_t t = __builtin_nontemporal_load((const u32x2_t*)a);
        b.v[nb][0] = t.x;
        b.v[nb][VW - 1] = t.y;
      } else {
        b.v[nb][0] = __builtin_nontemporal_load((const uint32_t*)a);
      }
    }
  };

  auto compute_tile = [&](Buf& b, int st) {
    // S^T for this sub-tile
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      if (KV == KV_BF16) {
        const bf16x8_t kop = __builtin_bit_cast(bf16x8_t, (u32x4_t){b.k[i].x, b.k[i].y, b.k[i].z, b.k[i].w});
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
    for (int j = 0; j < 4; ++j) sc[j] = sacc[j] * p.qk_scale;

    const bool partial = (st * 16 < t0) || (st * 16 + 16 > t1);
    if (partial) {
      uint32_t vmask[VW];
#pragma unroll
      for (int w = 0; w < VW; ++w) vmask[w] = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = st * 16 + 4 * row + j;
        const bool ok = tok >= t0 && tok < t1;
        if (!ok) sc[j] = -INFINITY;
        if (ok) {
          if (KV == KV_BF16) vmask[j >> 1] |= 0xffffu << (16 * (j & 1));
          else vmask[0] |= 0xffu << (8 * j);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int w = 0; w < VW; ++w) b.v[nb][w] &= vmask[w];
    }

    // column max, lazy rescale, probabilities
    const float cmax = colmax4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const bool grow = cmax > m_ref + LAZY_RESCALE_LOG2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_ref, cmax);
      const float alpha = fast_exp2(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] *= alpha;
      m_ref = m_new;
    }
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(sc[j] - m_ref);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const uint32_t p01 = pack_bf16x2(pr[0], pr[1]), p23 = pack_bf16x2(pr[2], pr[3]);
    const s16x4_t pop = __builtin_bit_cast(s16x4_t, (u32x2_t){p01, p23});

    // O^T += V^T . P^T
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      u32x2_t vv;
      if (KV == KV_BF16) {
        vv = (u32x2_t){b.v[nb][0], b.v[nb][VW - 1]};
      } else {
        vv = (u32x2_t){fp8x2_to_bf16x2<false>(b.v[nb][0]), fp8x2_to_bf16x2<true>(b.v[nb][0])};
      }
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, vv), pop,
                                                         acc[nb], 0, 0, 0);
    }
  };

  for (int cb = b_lo; cb < b_hi; cb += MFMA_TBL_CAP) {
    const int ce = min(b_hi, cb + MFMA_TBL_CAP);
    __syncthreads();
    for (int i = threadIdx.x; i < ce - cb; i += blockDim.x) {
      const unsigned id = (unsigned)table_row[cb + i];
      sm.table[i] = (int)(id > nb_max ? nb_max : id);
    }
    __syncthreads();
    const int cs_lo = max(st_lo, cb * SPB), cs_hi = min(st_hi, ce * SPB);
    int st = cs_lo + ((wave - (cs_lo - st_lo) % nw) + nw) % nw;
    if (st < cs_hi) load_tile(buf0, st, cb);
    if (st + nw < cs_hi) load_tile(buf1, st + nw, cb);
    while (st < cs_hi) {
      if (st + 2 * nw < cs_hi) load_tile(buf2, st + 2 * nw, cb);
      compute_tile(buf0, st);
      st += nw;
      if (st >= cs_hi) break;
      if (st + 2 * nw < cs_hi) load_tile(buf0, st + 2 * nw, cb);
      compute_tile(buf1, st);
      st += nw;
      if (st >= cs_hi) break;
      if (st + 2 * nw < cs_hi) load_tile(buf1, st + 2 * nw, cb);
      compute_tile(buf2, st);
      st += nw;
    }
  }

  // ---- wave results -> LDS, merge, write ---------------------------------------
  const float l_col = colsum4(l_run);
  if (col < G) {
    if (row == 0) {
      sm.m[wave][col] = m_ref;
      sm.l[wave][col] = l_col;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.acc[wave][col][16 * nb + 4 * row + i] = acc[nb][i];
  }
  __syncthreads();

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
      ((uint16_t*)p.out)[((size_t)s * Hq + hq) * D + d] = to_bf16_bits(o);
    } else {
      const size_t pi = ((size_t)s * Hq + hq) * p.max_parts + part;
      p.part_out[pi * D + d] = o;
      if (d == 0) p.part_lse[pi] = (mx + __log2f(den)) * 0.69314718055994531f;
    }
  }
}

template <int KV, int D, int BS, int G>
hipError_t launch_decode_mfma(const DecodeParams& p, int parts, hipStream_t stream) {
  dim3 grid(p.num_kv_heads, parts, p.num_seqs);
  hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, G>), grid, dim3(64 * MFMA_WAVES), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace pa
