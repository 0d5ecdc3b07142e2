// cache_ops.hip -- reshape_and_cache, the partition LSE merge and the E4M3
// dequantise utility, for gfx950.
#include "common.h"

namespace pa {

// reshape_and_cache: token t's K/V for every KV head goes to block slot/bs,
// offset slot%bs ("vLLM 0.5 deep dive: PagedAttention architecture",
// chenxutan.com, s2.1: a request's tokens fill ceil(n/bs) fixed-size blocks;
// "vLLM deployment and PagedAttention", crazysre.cn, "Core concept": the block
// table maps them to physical blocks).  One thread per (token, head, 16-byte
// K group): the K group is one 16-byte store (it is contiguous in the cache);
// the same X elements of V go to X rows of the V tile (stride bs elements).
template <int E>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, const int32_t* __restrict__ slots,
    int num_tokens, int Hkv, int D, int bs, long long num_slots) {
  constexpr int X = 16 / E;
  const int groups = D / X;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)num_tokens * Hkv * groups;
  if (gid >= total) return;
  const int grp = (int)(gid % groups);
  const int h = (int)((gid / groups) % Hkv);
  const int t = (int)(gid / ((long long)groups * Hkv));
  const int slot = slots[t];
  if (slot < 0 || (long long)slot >= num_slots) return;
  const int b = slot / bs, o = slot % bs;
  const size_t src = (((size_t)t * Hkv + h) * D + (size_t)grp * X) * E;
  const size_t tile = ((size_t)b * Hkv + h) * (size_t)D * bs * E;
  // key: 16 contiguous bytes at group grp, token o
  *(uint4*)(kc + tile + ((size_t)grp * bs + o) * 16) = *(const uint4*)(key + src);
  // value: element d goes to row d, column o
  const uint4 vv = *(const uint4*)(value + src);
  const uint8_t* vb = (const uint8_t*)&vv;
#pragma unroll
  for (int x = 0; x < X; ++x) {
    uint8_t* dst = vc + tile + (((size_t)grp * X + x) * bs + o) * E;
    if (E == 4) *(uint32_t*)dst = *(const uint32_t*)(vb + 4 * x);
    else if (E == 2) *(uint16_t*)dst = *(const uint16_t*)(vb + 2 * x);
    else *dst = vb[x];
  }
}

// Merge of per-partition results by their log-sum-exp: for each (sequence,
// query head) with keys [lo, L), the partitions p with [pP, (p+1)P) meeting that
// range are combined as sum_p e^(lse_p - M) o_p / sum_p e^(lse_p - M).
// One 256-thread workgroup per row.  Thread t owns float4 column t % (D/4) of
// the partitions t / (D/4) + k * SLOTS: per round it issues all RED_LOADS of
// its partial-output loads and their LSE loads at once (RED_LOADS * SLOTS = 128
// partitions per round, so a 64K-token sequence split at 512 is one round),
// keeps a running max of its own, and the slots are folded through LDS at the
// end with their maxima.
constexpr int RED_THREADS = 256;

template <bool OUT_BF16, int D>
__global__ __launch_bounds__(RED_THREADS) void reduce_lse_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, void* __restrict__ out, int Hq, int partition_size,
    int max_parts, int window) {
  constexpr int COLS = D / 4;                 // float4 columns per partition
  constexpr int SLOTS = RED_THREADS / COLS;   // partitions read in parallel
  constexpr int RED_LOADS = 128 / SLOTS;      // loads per thread per round
  __shared__ float m_s[SLOTS], den_s[SLOTS];
  __shared__ float4 acc_s[SLOTS][COLS];
  const int hq = blockIdx.x, s = blockIdx.y, t = threadIdx.x;
  const int col = t % COLS, slot = t / COLS;
  int L = seq_lens[s];
  L = L < 0 ? 0 : L;
  const int lo = (window > 0 && L > window) ? L - window : 0;
  const int p_lo = lo / partition_size;
  const int p_hi = L > 0 ? min(max_parts, (L + partition_size - 1) / partition_size) : p_lo;
  const size_t row = (size_t)s * Hq + hq;
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
    const float r = __expf(m - cm);   // m = -inf: r = 0 and a, den are still 0
    den *= r;
    a.x *= r; a.y *= r; a.z *= r; a.w *= r;
#pragma unroll
    for (int k = 0; k < RED_LOADS; ++k) {
      const float w = __expf(l[k] - cm);   // -inf: 0
      den += w;
      a.x += w * o[k].x; a.y += w * o[k].y; a.z += w * o[k].z; a.w += w * o[k].w;
    }
    m = cm;
  }
  if (col == 0) { m_s[slot] = m; den_s[slot] = den; }
  acc_s[slot][col] = a;
  __syncthreads();
  if (t < COLS) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) M = fmaxf(M, m_s[k]);
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    float dsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const float f = m_s[k] == -INFINITY ? 0.f : __expf(m_s[k] - M);
        const float4 v = acc_s[k][t];
        dsum += f * den_s[k];
        r.x += f * v.x; r.y += f * v.y; r.z += f * v.z; r.w += f * v.w;
      }
    }
    if (dsum > 0.f) {
      const float inv = 1.f / dsum;
      r.x *= inv; r.y *= inv; r.z *= inv; r.w *= inv;
    }
    if (OUT_BF16) {
      uint2 b;
      b.x = pack_bf16x2(r.x, r.y);
      b.y = pack_bf16x2(r.z, r.w);
      *(uint2*)((uint16_t*)out + row * D + 4 * t) = b;
    } else {
      *(float4*)((float*)out + row * D + 4 * t) = r;
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

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kc, void* vc,
                                    const int32_t* slots, int T, int Hkv, int D, int bs,
                                    int num_blocks, int elem_bytes, hipStream_t stream) {
  const int groups = D * elem_bytes / 16;
  const long long total = (long long)T * Hkv * groups;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  const long long nslots = (long long)num_blocks * bs;
  const uint8_t *k8 = (const uint8_t*)key, *v8 = (const uint8_t*)value;
  uint8_t *kc8 = (uint8_t*)kc, *vc8 = (uint8_t*)vc;
  if (elem_bytes == 4)
    hipLaunchKernelGGL(reshape_and_cache_kernel<4>, dim3(blocks), dim3(256), 0, stream, k8, v8,
                       kc8, vc8, slots, T, Hkv, D, bs, nslots);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(reshape_and_cache_kernel<2>, dim3(blocks), dim3(256), 0, stream, k8, v8,
                       kc8, vc8, slots, T, Hkv, D, bs, nslots);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<1>, dim3(blocks), dim3(256), 0, stream, k8, v8,
                       kc8, vc8, slots, T, Hkv, D, bs, nslots);
  return hipGetLastError();
}

hipError_t launch_reduce_lse(const float* part_out, const float* part_lse,
                             const int32_t* seq_lens, int S, int Hq, int D, int P, int max_parts,
                             int window, void* out, bool out_bf16, hipStream_t stream) {
  dim3 grid(Hq, S), block(RED_THREADS);
  if (D == 128) {
    if (out_bf16)
      hipLaunchKernelGGL((reduce_lse_kernel<true, 128>), grid, block, 0, stream, part_out,
                         part_lse, seq_lens, out, Hq, P, max_parts, window);
    else
      hipLaunchKernelGGL((reduce_lse_kernel<false, 128>), grid, block, 0, stream, part_out,
                         part_lse, seq_lens, out, Hq, P, max_parts, window);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((reduce_lse_kernel<true, 64>), grid, block, 0, stream, part_out,
                         part_lse, seq_lens, out, Hq, P, max_parts, window);
    else
      hipLaunchKernelGGL((reduce_lse_kernel<false, 64>), grid, block, 0, stream, part_out,
                         part_lse, seq_lens, out, Hq, P, max_parts, window);
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
