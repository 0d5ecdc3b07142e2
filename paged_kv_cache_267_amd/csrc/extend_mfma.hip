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
// block); each wave owns CW = 16 * NCB consecutive columns and walks the keys
// its columns need, 32 per step, loading K and V straight from the cache into
// registers (a double buffer: the next step's loads are in flight while this
// step computes).  The four waves read the same blocks, so the second and
// later reads hit L2; column blocks of one (sequence, KV head) are dealt to
// one XCD (workgroup j runs on XCD j % 8) so that they share its L2, and
// (sequence, KV head) pairs are dealt round robin over the 8 XCDs.  Within a
// pair the last column block (the most keys, causally) starts first.
//
// Per step and column block of 16 columns (v_mfma_f32_16x16x32_bf16 for both
// products, heads/tokens on N):
//   S^T = K . Q^T   A = K (16 keys x 32 dims per k-step, the cache's 16-byte
//                   groups as they lie), B = Q^T; two 16-key sub-tiles;
//   O^T += V^T P^T  A = V^T (16 dims x 32 keys), B = P^T: lane (row r, col c)
//                   holds keys 4r..4r+3 of both sub-tiles, which is exactly
//                   what the two S^T fragments leave in that lane, so P never
//                   moves between lanes.
// Softmax state (running max, sum) is per column and lane-local; the max over
// a fragment's 4 lane rows takes two lane swaps.  The running max is raised
// lazily (rescale only when a column's max grows by more than 2^8), and it
// starts at a large finite value so that a column whose keys are all masked
// in a step keeps p = 0 and no NaN.  E4M3 codes become bf16 in registers
// (exact); k_scale is folded into the score scale, v_scale applied at the end.
#include "dispatch.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int EX_WAVES = 4;
constexpr float EX_LAZY_LOG2 = 8.0f;
constexpr float EX_M_FLOOR = -1.0e30f;

__device__ __forceinline__ float ex_colmax4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float ex_colsum4(float x) {
  const float y = swap_add32(x, x);
  return swap_add16(y, y);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8_t, (u32x4_t){a, b, c, d});
}

template <int KV, int D, int BS, int NCB>
struct ExtendWave {
  static constexpr int E = KvTraits<KV>::E;
  static constexpr int KS = D / 32;       // QK k-steps of 32 dims
  static constexpr int NB = D / 16;       // output dim blocks of 16
  static constexpr int KL = D * E / 64;   // 16-byte K loads per lane per 16-key sub-tile
  static constexpr int VW = E;            // V dwords per lane per dim block per sub-tile
  static constexpr int CW = 16 * NCB;     // columns per wave

  struct Buf {
    uint4 k[2][KL];
    uint32_t v[2][NB][VW];
  };

  // Issue the loads of the 32 keys starting at key0 (a multiple of 32).
  __device__ __forceinline__ static void load(Buf& b, const ExtendParams& p, const int32_t* row_bt,
                                              int hk, int key0) {
    const int lane = threadIdx.x & 63, r = lane >> 4, c = lane & 15;
    const size_t tile = (size_t)D * BS * E;  // bytes of one (block, head) tile
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = key0 + 16 * h;
      int blk = row_bt[min(key / BS, p.max_blocks - 1)];
      blk = min(max(blk, 0), p.num_blocks - 1);
      const size_t base = ((size_t)blk * p.num_kv_heads + hk) * tile;
      const int sub = (key % BS) / 16;
      const char* kp = p.kc + base + sub * 256 + (r * BS + c) * 16;
      const char* vp = p.vc + base + (sub * 16 + c * BS + 4 * r) * E;
#pragma unroll
      for (int i = 0; i < KL; ++i) b.k[h][i] = load_nt16(kp + i * 4 * BS * 16);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const char* a = vp + (size_t)nb * 16 * BS * E;
        if (VW == 2) {
          const u32x2_t t = *(const u32x2_t*)a;
          b.v[h][nb][0] = t.x;
          b.v[h][nb][VW - 1] = t.y;
        } else {
          b.v[h][nb][0] = *(const uint32_t*)a;
        }
      }
    }
  }
};

template <int KV, int D, int BS, int NCB>
__global__ __launch_bounds__(EX_WAVES * 64) void extend_kernel(const ExtendParams p) {
  using W = ExtendWave<KV, D, BS, NCB>;
  constexpr int KS = W::KS, NB = W::NB, KL = W::KL, CW = W::CW;
  const int lane = threadIdx.x & 63, r = lane >> 4, c = lane & 15;
  const int wave = wave_id();

  // work item: XCD x takes pairs x, x + 8, ...; a pair's column blocks in a row
  const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int pair = x + 8 * (k / p.cblocks);
  if (pair >= p.pairs) return;
  const int cb = p.cblocks - 1 - k % p.cblocks;
  const int s = pair / p.num_kv_heads, hk = pair % p.num_kv_heads;
  const int G = 1 << p.log2g;

  const int L = min(max(p.seq_lens[s], 0), p.max_blocks * BS);
  const int q0 = min(max(p.qsl[s], 0), p.num_tokens);
  const int q1 = min(max(p.qsl[s + 1], q0), p.num_tokens);
  const int n = q1 - q0;
  const int col0 = (cb * EX_WAVES + wave) * CW;
  if (col0 >= (n << p.log2g)) return;  // no barriers below: a wave may leave alone
  const int t_first = col0 >> p.log2g;
  const int t_last = min(n - 1, (col0 + CW - 1) >> p.log2g);
  const int hi_min = L - n + t_first + 1;  // exclusive key end of the first token
  const int hi_max = L - n + t_last + 1;
  const int lo_max = p.window > 0 ? max(0, hi_max - p.window) : 0;
  const int klo = p.window > 0 ? max(0, max(hi_min, 0) - p.window) : 0;
  const int khi = max(hi_max, 0);
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
    lo_c[j] = valid && p.window > 0 ? max(0, hi_c[j] - p.window) : 0;
    const int tq = min(t, n - 1);
    const uint16_t* qrow =
        p.q + ((size_t)(q0 + tq) * p.num_q_heads + hk * G + g) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = (KV == KV_BF16) ? 32 * ks + 8 * r : 16 * (r + 4 * (ks >> 1)) + 8 * (ks & 1);
      uint4 v = *(const uint4*)(qrow + d0);
      if (t >= n) v = make_uint4(0, 0, 0, 0);
      qop[j][ks] = as_bf16x8(v.x, v.y, v.z, v.w);
    }
  }

  f32x4_t acc[NCB][NB];
  float m_ref[NCB], l_run[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    m_ref[j] = EX_M_FLOOR;
    l_run[j] = 0.f;
  }

  const int kq0 = klo >> 5;
  const int nsteps = khi > klo ? ((khi + 31) >> 5) - kq0 : 0;

  typename W::Buf buf[2];
  if (nsteps > 0) W::load(buf[0], p, row_bt, hk, kq0 * 32);

  for (int it = 0; it < nsteps; it += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int step = it + u;
      if (step >= nsteps) break;
      // next step's loads (the last step reloads itself: loads stay unconditional)
      W::load(buf[u ^ 1], p, row_bt, hk, (kq0 + min(step + 1, nsteps - 1)) * 32);
      typename W::Buf& b = buf[u];
      const int key0 = (kq0 + step) * 32;

      // K operands of both sub-tiles (E4M3 -> bf16 in registers)
      bf16x8_t kop[2][KS];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < KL; ++i) {
          const uint4 w = b.k[h][i];
          if (KV == KV_BF16) {
            kop[h][i] = as_bf16x8(w.x, w.y, w.z, w.w);
          } else {
            kop[h][2 * i] = as_bf16x8(fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x),
                                      fp8x2_to_bf16x2<false>(w.y), fp8x2_to_bf16x2<true>(w.y));
            kop[h][2 * i + 1] =
                as_bf16x8(fp8x2_to_bf16x2<false>(w.z), fp8x2_to_bf16x2<true>(w.z),
                          fp8x2_to_bf16x2<false>(w.w), fp8x2_to_bf16x2<true>(w.w));
          }
        }
      // V operands: k-slots 0..3 = keys 4r..4r+3 of sub-tile 0, 4..7 of sub-tile 1
      uint32_t vq[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (KV == KV_BF16) {
            vq[nb][2 * h] = b.v[h][nb][0];
            vq[nb][2 * h + 1] = b.v[h][nb][W::VW - 1];
          } else {
            vq[nb][2 * h] = fp8x2_to_bf16x2<false>(b.v[h][nb][0]);
            vq[nb][2 * h + 1] = fp8x2_to_bf16x2<true>(b.v[h][nb][0]);
          }
        }
      // keys outside [klo, khi) may be unwritten or outside the window's
      // blocks: zero their V so that p = 0 never meets a NaN
      if (key0 < klo || key0 + 32 > khi) {
        uint32_t vmask[4];
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const int kk = key0 + 16 * (w2 >> 1) + 4 * r + 2 * (w2 & 1);
          vmask[w2] = ((kk >= klo && kk < khi) ? 0xffffu : 0u) |
                      ((kk + 1 >= klo && kk + 1 < khi) ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) vq[nb][w2] &= vmask[w2];
      }
      const bool full = key0 >= lo_max && key0 + 32 <= hi_min && hi_min > 0;

#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][ks], qop[j][ks], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[1][ks], qop[j][ks], s1, 0, 0, 0);
        }
        float sc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[i] = s0[i] * p.qk_scale;
          sc[4 + i] = s1[i] * p.qk_scale;
        }
        if (!full) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int key = key0 + 16 * (i >> 2) + 4 * r + (i & 3);
            if (!(key >= lo_c[j] && key < hi_c[j])) sc[i] = -INFINITY;
          }
        }
        float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                         fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        mx = ex_colmax4(mx);
        if (__builtin_amdgcn_ballot_w64(mx > m_ref[j] + EX_LAZY_LOG2) != 0) {
          const float m_new = fmaxf(m_ref[j], mx);
          const float alpha = fast_exp2(m_ref[j] - m_new);
          l_run[j] *= alpha;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[j][nb] *= alpha;
          m_ref[j] = m_new;
        }
        float pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = fast_exp2(sc[i] - m_ref[j]);
        uint32_t pw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = pack_bf16x2(pr[2 * i], pr[2 * i + 1]);
        // the sum takes the same bf16 weights the P.V product multiplies: the
        // output stays a weighted mean of V rows, whatever the rounding of p
        l_run[j] += ((bf16_lo(pw[0]) + bf16_hi(pw[0])) + (bf16_lo(pw[1]) + bf16_hi(pw[1]))) +
                    ((bf16_lo(pw[2]) + bf16_hi(pw[2])) + (bf16_lo(pw[3]) + bf16_hi(pw[3])));
        const bf16x8_t pop = as_bf16x8(pw[0], pw[1], pw[2], pw[3]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[j][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(vq[nb][0], vq[nb][1], vq[nb][2], vq[nb][3]), pop, acc[j][nb], 0, 0, 0);
      }
    }
  }

  // normalise and store: lane (r, c) holds dims 16nb + 4r .. +3 of its column
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const float l = ex_colsum4(l_run[j]);
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

// Column blocks of 16 per wave: enough registers for the accumulators, the
// query operands and two steps of K/V in flight.
template <int D> constexpr int ex_ncb() { return D == 128 ? 2 : 4; }

template <int KV, int D, int BS>
hipError_t launch_ncb(const ExtendParams& p, hipStream_t stream) {
  constexpr int NCB = ex_ncb<D>();
  const long long grid = 8LL * ((p.pairs + 7) / 8) * p.cblocks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((extend_kernel<KV, D, BS, NCB>), dim3((unsigned)grid), dim3(EX_WAVES * 64),
                     0, stream, p);
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
