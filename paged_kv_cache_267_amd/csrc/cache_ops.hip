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
// One 256-thread workgroup per row: the weights go to LDS, then thread t sums
// float4 column t % (D/4) over partitions t / (D/4), t / (D/4) + SLOTS, ...
// so 8 (D = 128) or 16 (D = 64) partitions are read at once, and the slots
// are folded through LDS at the end.
constexpr int RED_THREADS = 256;
constexpr int RED_CHUNK = 1024;  // partitions whose weights are staged at a time

template <bool OUT_BF16, int D>
__global__ __launch_bounds__(RED_THREADS) void reduce_lse_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, void* __restrict__ out, int Hq, int partition_size,
    int max_parts, int window) {
  constexpr int COLS = D / 4;                 // float4 columns per partition
  constexpr int SLOTS = RED_THREADS / COLS;   // partitions read in parallel
  __shared__ float w_s[RED_CHUNK];
  __shared__ float red[RED_THREADS / 64];
  __shared__ float4 acc_s[SLOTS][COLS];
  const int hq = blockIdx.x, s = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  int L = seq_lens[s];
  L = L < 0 ? 0 : L;
  const int lo = (window > 0 && L > window) ? L - window : 0;
  const int p_lo = lo / partition_size;
  const int p_hi = min(max_parts, (L + partition_size - 1) / partition_size);
  const size_t row = (size_t)s * Hq + hq;
  const float* lse = part_lse + row * max_parts;

  // M = max over the row's partitions
  float mx = -INFINITY;
  for (int q = p_lo + t; q < p_hi; q += RED_THREADS) mx = fmaxf(mx, lse[q]);
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const int col = t % COLS, slot = t / COLS;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  if (L > 0 && mx != -INFINITY) {
    for (int c0 = p_lo; c0 < p_hi; c0 += RED_CHUNK) {
      const int c1 = min(p_hi, c0 + RED_CHUNK);
      __syncthreads();
      for (int q = c0 + t; q < c1; q += RED_THREADS) {
        const float l = lse[q];
        w_s[q - c0] = l == -INFINITY ? 0.f : __expf(l - mx);
      }
      __syncthreads();
      if (t < COLS)
        for (int q = c0; q < c1; ++q) den += w_s[q - c0];
#pragma unroll 4
      for (int q = c0 + slot; q < c1; q += SLOTS) {
        const float w = w_s[q - c0];
        if (w != 0.f) {  // skipped partitions may hold anything
          const float4 o = *(const float4*)(part_out + (row * max_parts + q) * D + 4 * col);
          a.x += w * o.x; a.y += w * o.y; a.z += w * o.z; a.w += w * o.w;
        }
      }
    }
  }
  acc_s[slot][col] = a;
  __syncthreads();
  if (t < COLS) {
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < SLOTS; ++k) {
      const float4 v = acc_s[k][t];
      r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
    }
    if (den > 0.f) {
      const float inv = 1.f / den;
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
