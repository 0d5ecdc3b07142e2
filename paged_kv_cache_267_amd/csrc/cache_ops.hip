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
// query head) with keys [lo, L), partitions p with [pP, (p+1)P) meeting that
// range are combined as sum_p e^(lse_p - M) o_p / sum_p e^(lse_p - M).
// One wave per row; lane l owns head_dim entries l, l+64.
template <bool OUT_BF16>
__global__ __launch_bounds__(64) void reduce_lse_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, void* __restrict__ out, int Hq, int D,
    int partition_size, int max_parts, int window) {
  const int hq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  int L = seq_lens[s];
  L = L < 0 ? 0 : L;
  const int lo = (window > 0 && L > window) ? L - window : 0;
  int p_lo = lo / partition_size;
  int p_hi = (L + partition_size - 1) / partition_size;
  if (p_hi > max_parts) p_hi = max_parts;
  const size_t row = (size_t)s * Hq + hq;
  float mx = -INFINITY;
  for (int q = p_lo + lane; q < p_hi; q += 64) mx = fmaxf(mx, part_lse[row * max_parts + q]);
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  float num0 = 0.f, num1 = 0.f, den = 0.f;
  if (L > 0 && mx != -INFINITY) {
    for (int q = p_lo; q < p_hi; ++q) {
      const float lse = part_lse[row * max_parts + q];
      const float w = lse == -INFINITY ? 0.f : __expf(lse - mx);
      const float* o = part_out + (row * max_parts + q) * D;
      den += w;
      if (w != 0.f) {
        num0 += w * o[lane];
        if (D > 64) num1 += w * o[lane + 64];
      }
    }
    num0 /= den;
    num1 /= den;
  }
  if (OUT_BF16) {
    uint16_t* ob = (uint16_t*)out + row * D;
    ob[lane] = to_bf16_bits(num0);
    if (D > 64) ob[lane + 64] = to_bf16_bits(num1);
  } else {
    float* of = (float*)out + row * D;
    of[lane] = num0;
    if (D > 64) of[lane + 64] = num1;
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
  dim3 grid(Hq, S);
  if (out_bf16)
    hipLaunchKernelGGL(reduce_lse_kernel<true>, grid, dim3(64), 0, stream, part_out, part_lse,
                       seq_lens, out, Hq, D, P, max_parts, window);
  else
    hipLaunchKernelGGL(reduce_lse_kernel<false>, grid, dim3(64), 0, stream, part_out, part_lse,
                       seq_lens, out, Hq, D, P, max_parts, window);
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
