// cache_ops.hip -- reshape_and_cache, the partition LSE merge and the E4M3
// dequantise utility, for gfx950.
#include "common.h"

namespace pa {

// reshape_and_cache: token t's K/V for every KV head goes to block slot/bs,
// offset slot%bs ("vLLM 0.5 deep dive: PagedAttention architecture",
// chenxutan.com, s2.1: a request's tokens fill ceil(n/bs) fixed-size blocks;
// "vLLM deployment and PagedAttention", crazysre.cn, "Core concept": the block
// table maps them to physical blocks).  One thread per (token, head, 16-byte
// K group), the head on blockIdx.y: the K group is one 16-byte store (it is
// contiguous in the cache); the same X elements of V go to X rows of the V
// tile (stride bs elements).  Token fastest: neighbouring lanes take
// neighbouring tokens, whose slots are usually neighbours in one block (a
// chunk of new tokens), so their K groups and V elements land side by side.
// A launch covers tokens t_base .. t_base + nt - 1 (nt * groups <= 2^30) and
// heads h_base + blockIdx.y.  The source row does not depend on the slot, so
// its loads are issued together with the slot's: one memory round trip.
template <int E>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, const int32_t* __restrict__ slots,
    int nt, int t_base, int h_base, int Hkv, int D, int bs, long long num_slots) {
  constexpr int X = 16 / E;
  const int groups = D / X;
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= nt * groups) return;
  const int t = t_base + (int)((unsigned)i % (unsigned)nt);
  const int grp = (int)((unsigned)i / (unsigned)nt);
  const int h = h_base + (int)blockIdx.y;
  const size_t src = (((size_t)t * Hkv + h) * D + (size_t)grp * X) * E;
  const int slot = slots[t];
  const u32x4_t kk = *(const u32x4_t*)(key + src);
  const u32x4_t vv = *(const u32x4_t*)(value + src);
  // a use before the slot test keeps the source loads ahead of it: otherwise
  // the compiler moves them (or all but one dword of them) behind the test and
  // the thread waits twice
  asm volatile("" ::"v"(kk), "v"(vv));
  if (slot < 0 || (long long)slot >= num_slots) return;
  const int b = slot / bs, o = slot % bs;
  const size_t tile = ((size_t)b * Hkv + h) * (size_t)D * bs * E;
  // key: 16 contiguous bytes at group grp, token o
  *(u32x4_t*)(kc + tile + ((size_t)grp * bs + o) * 16) = kk;
  // value: element d goes to row d, column o
  const uint8_t* vb = (const uint8_t*)&vv;
#pragma unroll
  for (int x = 0; x < X; ++x) {
    uint8_t* dst = vc + tile + (((size_t)grp * X + x) * bs + o) * E;
    if (E == 4) *(uint32_t*)dst = *(const uint32_t*)(vb + 4 * x);
    else if (E == 2) *(uint16_t*)dst = *(const uint16_t*)(vb + 2 * x);
    else *dst = vb[x];
  }
}

// The same write for appends of few tokens (decode: one token per sequence,
// each in a block of its own), one thread per (token, head, element d) with
// d fastest: the 64 lanes of a V store write 64 rows of one token, which
// share D * E * bs / 128 cache lines instead of touching 64 lines of 64
// blocks; threads d < D * E / 16 also write K group d.  A launch covers
// tokens t_base .. t_base + nt - 1 (nt * D <= 2^30) and heads h_base +
// blockIdx.y.
template <int E>
__global__ __launch_bounds__(256) void reshape_and_cache_rows_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, const int32_t* __restrict__ slots,
    int nt, int t_base, int h_base, int Hkv, int D, int bs, long long num_slots) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= nt * D) return;
  const int t = t_base + (int)((unsigned)i / (unsigned)D), d = (int)((unsigned)i % (unsigned)D);
  const int h = h_base + (int)blockIdx.y;
  const size_t row = ((size_t)t * Hkv + h) * D * E;
  const bool kgroup = d < D * E / 16;
  const int slot = slots[t];
  // the neighbours' slots in this launch (a chunk's tokens take consecutive
  // slots); clamped indices, so the loads need no branch
  const int tp = max(t - 1, t_base), tn = min(t + 1, t_base + nt - 1);
  const int prev = slots[tp], next = slots[tn];
  uint32_t v;
  if (E == 4) v = *(const uint32_t*)(value + row + 4 * d);
  else if (E == 2) v = *(const uint16_t*)(value + row + 2 * d);
  else v = value[row + d];
  u32x4_t kk = {0u, 0u, 0u, 0u};
  if (kgroup) kk = *(const u32x4_t*)(key + row + 16 * d);
  asm volatile("" ::"v"(kk), "v"(v));   // the source loads stay ahead of the slot test
  if (slot < 0 || (long long)slot >= num_slots) return;
  const int b = slot / bs, o = slot % bs;
  const size_t tile = ((size_t)b * Hkv + h) * (size_t)D * bs * E;
  uint8_t* dst = vc + tile + ((size_t)d * bs + o) * E;
  uint8_t* kdst = kc + tile + ((size_t)d * bs + o) * 16;
  // A token whose neighbours in the launch do not take the slots next to its
  // own in its block (a decode step's append: one token per sequence) leaves
  // partial lines that nothing in the launch completes.  Stored non-temporal,
  // they are not held dirty in L2 for the write-back at the kernel's end,
  // which the decode launched next waits for (a decode step over 256
  // sequences of an E4M3 cache -3 %, over 64 sequences of a bf16 cache
  // -1.6 %).  A chunk's tokens fill their lines together: those stores stay
  // in L2, which merges them (stored non-temporal, each would reach memory on
  // its own: a prefix-extend append took 71 us instead of 21).
  // (unsigned: slot + 1 may exceed INT_MAX in a pool of more than 2^31 slots)
  const bool chained = (tp != t && o > 0 && (unsigned)prev + 1u == (unsigned)slot) ||
                       (tn != t && o + 1 < bs && (unsigned)slot + 1u == (unsigned)next);
  if (!chained) {
    if (E == 4) __builtin_nontemporal_store(v, (uint32_t*)dst);
    else if (E == 2) __builtin_nontemporal_store((uint16_t)v, (uint16_t*)dst);
    else __builtin_nontemporal_store((uint8_t)v, dst);
    if (kgroup) __builtin_nontemporal_store(kk, (u32x4_t*)kdst);
    // keeps the compiler from merging these stores with the plain ones below
    // (a merged store loses the non-temporal hint)
    asm volatile("" ::: "memory");
  } else {
    if (E == 4) *(uint32_t*)dst = v;
    else if (E == 2) *(uint16_t*)dst = (uint16_t)v;
    else *dst = (uint8_t)v;
    if (kgroup) *(u32x4_t*)kdst = kk;
  }
}

// E4M3 code of a binary32 value: nearest code, ties to even, saturating at
// +-448 (infinities included), NaN -> 0x7F.  Codes are (1 + m/8) * 2^(e-7) for
// exponent field e >= 1 and m/8 * 2^-6 for e = 0.  Normal range: the fp32
// exponent and top 3 mantissa bits, rounded half to even on the 20 dropped
// bits (a carry moves into the exponent), rebiased from 127 to 7.
// Subnormal range (|q| < 2^-6): |q| * 2^9 rounded to an integer 0..8 (8 is
// the smallest normal, code 0x08).
__device__ __forceinline__ uint32_t e4m3_from_f32(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;            // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;    // |q| >= 448
  if (a < 0x3c800000u)                          // |q| < 2^-6
    return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  return sign | (r - ((127u - 7u) << 3));
}

// reshape_and_cache with quantisation ("vLLM 0.5 deep dive: PagedAttention
// architecture", chenxutan.com, s3.4: an FP8 cache with a scale factor and
// zero point 0): element x of a new token's K (V) is stored as the E4M3 code
// of the binary32 quotient x / k_scale (x / v_scale).  One thread per (token,
// head, 16-element group): 16 codes make one 16-byte K store; the same 16
// elements of V go to 16 rows of the V tile.
template <int SE>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, const int32_t* __restrict__ slots,
    int nt, int t_base, int h_base, int Hkv, int D, int bs, long long num_slots, float k_scale,
    float v_scale) {
  const int groups = D / 16;
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= nt * groups) return;
  // token fastest, the head on blockIdx.y, as in reshape_and_cache_kernel
  const int t = t_base + (int)((unsigned)i % (unsigned)nt);
  const int grp = (int)((unsigned)i / (unsigned)nt);
  const int h = h_base + (int)blockIdx.y;
  const size_t src = (((size_t)t * Hkv + h) * D + (size_t)grp * 16) * SE;
  u32x4_t kr[SE], vr[SE];   // the 16 source elements, 16 bytes at a time
  const int slot = slots[t];
#pragma unroll
  for (int c = 0; c < SE; ++c) {
    kr[c] = *(const u32x4_t*)(key + src + 16 * c);
    vr[c] = *(const u32x4_t*)(value + src + 16 * c);
  }
#pragma unroll
  for (int c = 0; c < SE; ++c) asm volatile("" ::"v"(kr[c]), "v"(vr[c]));  // as above
  if (slot < 0 || (long long)slot >= num_slots) return;
  const int b = slot / bs, o = slot % bs;
  const size_t tile = ((size_t)b * Hkv + h) * (size_t)D * bs;
  float xk[16], xv[16];
#pragma unroll
  for (int c = 0; c < SE; ++c) {
    const uint32_t kw[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
    const uint32_t vw[4] = {vr[c].x, vr[c].y, vr[c].z, vr[c].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (SE == 4) {
        xk[4 * c + w] = __uint_as_float(kw[w]);
        xv[4 * c + w] = __uint_as_float(vw[w]);
      } else {
        xk[8 * c + 2 * w] = bf16_lo(kw[w]);
        xk[8 * c + 2 * w + 1] = bf16_hi(kw[w]);
        xv[8 * c + 2 * w] = bf16_lo(vw[w]);
        xv[8 * c + 2 * w + 1] = bf16_hi(vw[w]);
      }
    }
  }
  uint32_t kq[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) kq[e >> 2] |= e4m3_from_f32(xk[e] / k_scale) << (8 * (e & 3));
  *(uint4*)(kc + tile + ((size_t)grp * bs + o) * 16) = make_uint4(kq[0], kq[1], kq[2], kq[3]);
#pragma unroll
  for (int e = 0; e < 16; ++e)
    vc[tile + ((size_t)grp * 16 + e) * bs + o] = (uint8_t)e4m3_from_f32(xv[e] / v_scale);
}

// The same quantise-on-write for small appends (a decode step: one token per
// sequence, each in a block of its own), one thread per (token, head,
// element d), d fastest, as reshape_and_cache_rows_kernel: the 64 lanes of a
// V store write 64 rows of one token; threads d < D / 16 also quantise and
// write K group d.  The codes are those of reshape_and_cache_fp8_kernel (the
// same quotient and rounding).  A token alone in its block of the launch is
// stored non-temporal, as in the bit copy.  A launch covers tokens t_base ..
// t_base + nt - 1 (nt * D <= 2^30) and heads h_base + blockIdx.y.
template <int SE>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_rows_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, const int32_t* __restrict__ slots,
    int nt, int t_base, int h_base, int Hkv, int D, int bs, long long num_slots, float k_scale,
    float v_scale) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= nt * D) return;
  const int t = t_base + (int)((unsigned)i / (unsigned)D), d = (int)((unsigned)i % (unsigned)D);
  const int h = h_base + (int)blockIdx.y;
  const size_t row = ((size_t)t * Hkv + h) * D * SE;
  const bool kgroup = d < D / 16;
  const int slot = slots[t];
  const int tp = max(t - 1, t_base), tn = min(t + 1, t_base + nt - 1);
  const int prev = slots[tp], next = slots[tn];
  const uint32_t vraw = SE == 4 ? *(const uint32_t*)(value + row + 4 * d)
                                : (uint32_t)*(const uint16_t*)(value + row + 2 * d);
  u32x4_t kr[SE];   // K group d: 16 source elements, 16 bytes at a time
#pragma unroll
  for (int c = 0; c < SE; ++c)
    kr[c] = kgroup ? *(const u32x4_t*)(key + row + (size_t)d * 16 * SE + 16 * c)
                   : (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < SE; ++c) asm volatile("" ::"v"(kr[c]), "v"(vraw));  // loads ahead of the test
  if (slot < 0 || (long long)slot >= num_slots) return;
  const int b = slot / bs, o = slot % bs;
  const size_t tile = ((size_t)b * Hkv + h) * (size_t)D * bs;
  const float xv = SE == 4 ? __uint_as_float(vraw) : __uint_as_float(vraw << 16);
  const uint8_t vq = (uint8_t)e4m3_from_f32(xv / v_scale);
  uint32_t kq[4] = {0u, 0u, 0u, 0u};
  if (kgroup) {
#pragma unroll
    for (int c = 0; c < SE; ++c) {
      const uint32_t kw[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (SE == 4) {
          const int e = 4 * c + w;
          kq[e >> 2] |= e4m3_from_f32(__uint_as_float(kw[w]) / k_scale) << (8 * (e & 3));
        } else {
          const int e = 8 * c + 2 * w;
          kq[e >> 2] |= e4m3_from_f32(bf16_lo(kw[w]) / k_scale) << (8 * (e & 3));
          kq[(e + 1) >> 2] |= e4m3_from_f32(bf16_hi(kw[w]) / k_scale) << (8 * ((e + 1) & 3));
        }
      }
    }
  }
  uint8_t* vdst = vc + tile + (size_t)d * bs + o;
  uint8_t* kdst = kc + tile + ((size_t)d * bs + o) * 16;
  const bool chained = (tp != t && o > 0 && (unsigned)prev + 1u == (unsigned)slot) ||
                       (tn != t && o + 1 < bs && (unsigned)slot + 1u == (unsigned)next);
  if (!chained) {
    __builtin_nontemporal_store(vq, vdst);
    if (kgroup) __builtin_nontemporal_store((u32x4_t){kq[0], kq[1], kq[2], kq[3]}, (u32x4_t*)kdst);
    asm volatile("" ::: "memory");   // not merged with the plain stores below
  } else {
    *vdst = vq;
    if (kgroup) *(u32x4_t*)kdst = (u32x4_t){kq[0], kq[1], kq[2], kq[3]};
  }
}

// Merge of per-partition results by their log-sum-exp: for each (sequence,
// query head) with keys [lo, L), the partitions p with [pP, (p+1)P) meeting that
// range are combined as sum_p e^(lse_p - M) o_p / sum_p e^(lse_p - M).
// WPR waves serve one row (1 for short rows: four rows per workgroup; 4 when a
// row can span more partitions than one wave takes in a round).  Lane l of the
// row's lanes owns float4 column l % (D/4) of the partitions l / (D/4) +
// k * SLOTS: per round it issues all RED_LOADS of its partial-output loads and
// their LSE loads at once and keeps a running max of its own; the lane groups
// are folded with cross-lane swaps, then (WPR = 4) across waves through LDS.
constexpr int RED_THREADS = 256;
constexpr int RED_LOADS = 16;                // loads per lane per round

template <bool OUT_BF16, int D, int WPR>
__global__ __launch_bounds__(RED_THREADS) void reduce_lse_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, void* __restrict__ out, int rows, int Hq,
    int partition_size, int max_parts, int window) {
  constexpr int COLS = D / 4;                 // float4 columns per partition
  constexpr int SLOTS = 64 * WPR / COLS;      // partitions read in parallel by a row
  constexpr int ROWS = RED_THREADS / 64 / WPR;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int r = blockIdx.x * ROWS + wave / WPR;
  if (r >= rows) return;                      // whole row groups leave together
  const int s = r / Hq;
  const int rl = (wave % WPR) * 64 + lane;    // lane index within the row
  const int col = rl % COLS, slot = rl / COLS;
  int L = seq_lens[s];
  L = L < 0 ? 0 : L;
  const int lo = (window > 0 && L > window) ? L - window : 0;
  const int p_lo = lo / partition_size;
  const int p_hi = L > 0 ? min(max_parts, (L + partition_size - 1) / partition_size) : p_lo;
  const size_t row = (size_t)r;
  const float* lse = part_lse + row * max_parts;
  const float* po = part_out + row * max_parts * D + 4 * col;

  float m = -INFINITY, den = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q0 = p_lo + slot; q0 < p_hi; q0 += RED_LOADS * SLOTS) {
    float l[RED_LOADS];
    float4 o[RED_LOADS];
#pragma unroll
    for (int k = 0; k < RED_LOADS; ++k) {   // all loads of the round issue before any use
      const int q = q0 + k * SLOTS;
      l[k] = -INFINITY;
      o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (q < p_hi) {
        l[k] = lse[q];
        o[k] = *(const float4*)(po + (size_t)q * D);
      }
    }
    float cm = m;
#pragma unroll
    for (int k = 0; k < RED_LOADS; ++k) cm = fmaxf(cm, l[k]);
    if (cm == -INFINITY) continue;
    const float f = __expf(m - cm);   // m = -inf: f = 0 and a, den are still 0
    den *= f;
    a.x *= f; a.y *= f; a.z *= f; a.w *= f;
#pragma unroll
    for (int k = 0; k < RED_LOADS; ++k) {
      const float w = __expf(l[k] - cm);   // -inf: 0
      den += w;
      a.x += w * o[k].x; a.y += w * o[k].y; a.z += w * o[k].z; a.w += w * o[k].w;
    }
    m = cm;
  }
  // (m1, d1, a1) <- combination of (m1, d1, a1) and (m2, d2, a2)
  auto combine = [](float& m1, float& d1, float4& a1, float m2, float d2, float4 a2) {
    const float M = fmaxf(m1, m2);
    const float f1 = m1 == -INFINITY ? 0.f : __expf(m1 - M);
    const float f2 = m2 == -INFINITY ? 0.f : __expf(m2 - M);
    d1 = f1 * d1 + f2 * d2;
    a1.x = f1 * a1.x + f2 * a2.x; a1.y = f1 * a1.y + f2 * a2.y;
    a1.z = f1 * a1.z + f2 * a2.z; a1.w = f1 * a1.w + f2 * a2.w;
    m1 = M;
  };
  // fold the lane groups of a wave: lanes l and l + off hold the same column
#pragma unroll
  for (int off = 32; off >= COLS; off >>= 1) {
    const float4 a2 = make_float4(__shfl_xor(a.x, off, 64), __shfl_xor(a.y, off, 64),
                                  __shfl_xor(a.z, off, 64), __shfl_xor(a.w, off, 64));
    combine(m, den, a, __shfl_xor(m, off, 64), __shfl_xor(den, off, 64), a2);
  }
  if (WPR > 1) {   // fold the row's waves through LDS (one row per workgroup)
    __shared__ float m_s[WPR][COLS], d_s[WPR][COLS];
    __shared__ float4 a_s[WPR][COLS];
    if (lane < COLS) { m_s[wave][lane] = m; d_s[wave][lane] = den; a_s[wave][lane] = a; }
    __syncthreads();
    if (wave != 0) return;
    if (lane < COLS)
      for (int w = 1; w < WPR; ++w) combine(m, den, a, m_s[w][lane], d_s[w][lane], a_s[w][lane]);
  }
  if (lane < COLS) {
    if (den > 0.f) {
      const float inv = 1.f / den;
      a.x *= inv; a.y *= inv; a.z *= inv; a.w *= inv;
    } else {
      a = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (OUT_BF16) {
      uint2 b;
      b.x = pack_bf16x2(a.x, a.y);
      b.y = pack_bf16x2(a.z, a.w);
      *(uint2*)((uint16_t*)out + row * D + 4 * lane) = b;
    } else {
      *(float4*)((float*)out + row * D + 4 * lane) = a;
    }
  }
}

// E4M3 codes -> fp32 values times scale, with the same hardware conversion the
// decode kernels use (code pair -> bf16 pair, exact, then widened).
__global__ __launch_bounds__(256) void fp8_dequant_kernel(const uint8_t* __restrict__ codes,
                                                          float scale, float* __restrict__ out,
                                                          long long n) {
  const long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  uint32_t w = 0;
  for (int k = 0; k < 4 && i + k < n; ++k) w |= (uint32_t)codes[i + k] << (8 * k);
  const uint32_t lo = fp8x2_to_bf16x2<false>(w), hi = fp8x2_to_bf16x2<true>(w);
  const float v[4] = {bf16_lo(lo), bf16_hi(lo), bf16_lo(hi), bf16_hi(hi)};
  for (int k = 0; k < 4 && i + k < n; ++k) out[i + k] = v[k] * scale;
}

// Launches of an append, in chunks that keep the kernels' 32-bit indices in
// range: at most RC_TOKENS tokens (times at most 32 groups <= 2^30 threads;
// the element-per-thread mapping only runs appends of a few thousand tokens)
// and RC_HEADS heads (grid y) per launch.  One launch for any realistic call.
constexpr int RC_TOKENS = 1 << 25;
constexpr int RC_HEADS = 32768;

template <class F>
static hipError_t for_each_chunk(int T, int Hkv, int groups, F launch) {
  for (long long t0 = 0; t0 < T; t0 += RC_TOKENS) {
    const int nt = (int)min((long long)RC_TOKENS, T - t0);
    const unsigned bx = (unsigned)(((long long)nt * groups + 255) / 256);
    for (long long h0 = 0; h0 < Hkv; h0 += RC_HEADS) {
      launch(dim3(bx, (unsigned)min((long long)RC_HEADS, Hkv - h0)), nt, (int)t0, (int)h0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Appends that write at most this many V bytes (tokens x heads x head_dim x
// element size) take the element-per-thread mapping: a decode step's tokens
// sit in blocks of their own, where it writes fewer, fuller lines.  Larger
// appends take the token-per-lane mapping, whichever their pattern: chunks,
// whose neighbouring tokens share V rows, are written side by side, and even
// scattered tokens are written faster beyond this size (the element-per-
// thread stores of lone tokens bypass L2, at a cost that grows per token).
// Measured with 8 KV heads, head_dim 128, bs 16, one token per block: equal
// at 256 bf16 tokens (512 KiB), 384 bf16 tokens 8.4 us against 7.1; 768 E4M3
// tokens 8.8 against 9.6, 1024 E4M3 tokens 11.3 against 10.5.
constexpr long long RC_ROWS_MAX_BYTES = 640 << 10;

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kc, void* vc,
                                    const int32_t* slots, int T, int Hkv, int D, int bs,
                                    int num_blocks, int elem_bytes, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int groups = D * elem_bytes / 16;
  const long long nslots = (long long)num_blocks * bs;
  const uint8_t *k8 = (const uint8_t*)key, *v8 = (const uint8_t*)value;
  uint8_t *kc8 = (uint8_t*)kc, *vc8 = (uint8_t*)vc;
  if ((long long)T * Hkv * D * elem_bytes <= RC_ROWS_MAX_BYTES)
    return for_each_chunk(T, Hkv, D, [&](dim3 grid, int nt, int t0, int h0) {
      if (elem_bytes == 4)
        hipLaunchKernelGGL(reshape_and_cache_rows_kernel<4>, grid, dim3(256), 0, stream, k8, v8,
                           kc8, vc8, slots, nt, t0, h0, Hkv, D, bs, nslots);
      else if (elem_bytes == 2)
        hipLaunchKernelGGL(reshape_and_cache_rows_kernel<2>, grid, dim3(256), 0, stream, k8, v8,
                           kc8, vc8, slots, nt, t0, h0, Hkv, D, bs, nslots);
      else
        hipLaunchKernelGGL(reshape_and_cache_rows_kernel<1>, grid, dim3(256), 0, stream, k8, v8,
                           kc8, vc8, slots, nt, t0, h0, Hkv, D, bs, nslots);
    });
  return for_each_chunk(T, Hkv, groups, [&](dim3 grid, int nt, int t0, int h0) {
    if (elem_bytes == 4)
      hipLaunchKernelGGL(reshape_and_cache_kernel<4>, grid, dim3(256), 0, stream, k8, v8, kc8,
                         vc8, slots, nt, t0, h0, Hkv, D, bs, nslots);
    else if (elem_bytes == 2)
      hipLaunchKernelGGL(reshape_and_cache_kernel<2>, grid, dim3(256), 0, stream, k8, v8, kc8,
                         vc8, slots, nt, t0, h0, Hkv, D, bs, nslots);
    else
      hipLaunchKernelGGL(reshape_and_cache_kernel<1>, grid, dim3(256), 0, stream, k8, v8, kc8,
                         vc8, slots, nt, t0, h0, Hkv, D, bs, nslots);
  });
}

template <bool OUT_BF16, int D, int WPR>
static void launch_reduce_rows(const float* part_out, const float* part_lse,
                               const int32_t* seq_lens, int rows, int Hq, int P, int max_parts,
                               int window, void* out, hipStream_t stream) {
  constexpr int ROWS = RED_THREADS / 64 / WPR;
  hipLaunchKernelGGL((reduce_lse_kernel<OUT_BF16, D, WPR>), dim3((rows + ROWS - 1) / ROWS),
                     dim3(RED_THREADS), 0, stream, part_out, part_lse, seq_lens, out, rows, Hq, P,
                     max_parts, window);
}

template <bool OUT_BF16, int D>
static void launch_reduce_d(const float* part_out, const float* part_lse,
                            const int32_t* seq_lens, int rows, int Hq, int P, int max_parts,
                            int window, void* out, hipStream_t stream) {
  // partitions a row can meet: all of them, or those a window can touch
  int span = max_parts;
  if (window > 0) span = min(span, (window + P - 1) / P + 1);
  // one wave takes 16 * (64 / (D / 4)) partitions per round
  if (span > RED_LOADS * (256 / D))
    launch_reduce_rows<OUT_BF16, D, 4>(part_out, part_lse, seq_lens, rows, Hq, P, max_parts,
                                       window, out, stream);
  else
    launch_reduce_rows<OUT_BF16, D, 1>(part_out, part_lse, seq_lens, rows, Hq, P, max_parts,
                                       window, out, stream);
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* kc, void* vc,
                                        const int32_t* slots, int T, int Hkv, int D, int bs,
                                        int num_blocks, int src_bytes, float k_scale,
                                        float v_scale, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const long long nslots = (long long)num_blocks * bs;
  const uint8_t *k8 = (const uint8_t*)key, *v8 = (const uint8_t*)value;
  uint8_t *kc8 = (uint8_t*)kc, *vc8 = (uint8_t*)vc;
  // the bit copy's rule: appends of at most RC_ROWS_MAX_BYTES of V take the
  // element-per-thread mapping
  if ((long long)T * Hkv * D <= RC_ROWS_MAX_BYTES)
    return for_each_chunk(T, Hkv, D, [&](dim3 grid, int nt, int t0, int h0) {
      if (src_bytes == 4)
        hipLaunchKernelGGL(reshape_and_cache_fp8_rows_kernel<4>, grid, dim3(256), 0, stream, k8,
                           v8, kc8, vc8, slots, nt, t0, h0, Hkv, D, bs, nslots, k_scale, v_scale);
      else
        hipLaunchKernelGGL(reshape_and_cache_fp8_rows_kernel<2>, grid, dim3(256), 0, stream, k8,
                           v8, kc8, vc8, slots, nt, t0, h0, Hkv, D, bs, nslots, k_scale, v_scale);
    });
  return for_each_chunk(T, Hkv, D / 16, [&](dim3 grid, int nt, int t0, int h0) {
    if (src_bytes == 4)
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<4>, grid, dim3(256), 0, stream, k8, v8,
                         kc8, vc8, slots, nt, t0, h0, Hkv, D, bs, nslots, k_scale, v_scale);
    else
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<2>, grid, dim3(256), 0, stream, k8, v8,
                         kc8, vc8, slots, nt, t0, h0, Hkv, D, bs, nslots, k_scale, v_scale);
  });
}

hipError_t launch_reduce_lse(const float* part_out, const float* part_lse,
                             const int32_t* seq_lens, int S, int Hq, int D, int P, int max_parts,
                             int window, void* out, bool out_bf16, hipStream_t stream) {
  const int rows = S * Hq;
  if (D == 128) {
    if (out_bf16)
      launch_reduce_d<true, 128>(part_out, part_lse, seq_lens, rows, Hq, P, max_parts, window,
                                 out, stream);
    else
      launch_reduce_d<false, 128>(part_out, part_lse, seq_lens, rows, Hq, P, max_parts, window,
                                  out, stream);
  } else {
    if (out_bf16)
      launch_reduce_d<true, 64>(part_out, part_lse, seq_lens, rows, Hq, P, max_parts, window,
                                out, stream);
    else
      launch_reduce_d<false, 64>(part_out, part_lse, seq_lens, rows, Hq, P, max_parts, window,
                                 out, stream);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_dequant(const uint8_t* codes, float scale, float* out, long long n,
                              hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const long long threads = (n + 3) / 4;
  hipLaunchKernelGGL(fp8_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, codes, scale, out, n);
  return hipGetLastError();
}

}  // namespace pa
