// probe.hip -- a bandwidth probe with the decode kernels' access pattern:
// whole chunks (the size of one (block, head) K or V tile) read with 16-byte
// non-temporal loads, in the order of a chunk-id list.  With a random
// permutation it measures what HBM delivers to a paged gather; with ids in
// order, a plain streaming read.  Nothing is computed but an XOR of the data,
// which goes to one word so the loads cannot be dropped.
#include "common.h"

namespace pa {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_DEPTH = 8;   // 16-byte loads per thread in flight

// A wave reads one 1 KiB row per load (64 lanes x 16 bytes); chunk k holds
// rows [k << rpc_log2, (k + 1) << rpc_log2).  Row indices are wave-uniform,
// so the chunk lookup is scalar work.
__global__ __launch_bounds__(PROBE_THREADS) void gather_read_probe_kernel(
    const uint8_t* __restrict__ base, const int32_t* __restrict__ ids, long long rows,
    int rpc_log2, unsigned* __restrict__ sink) {
  constexpr int WAVES = PROBE_THREADS / 64;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const long long round = (long long)WAVES * PROBE_DEPTH;   // rows per workgroup round
  unsigned x = 0;
  for (long long r0 = (long long)blockIdx.x * round; r0 < rows; r0 += (long long)gridDim.x * round) {
    uint4 v[PROBE_DEPTH];
#pragma unroll
    for (int i = 0; i < PROBE_DEPTH; ++i) {
      long long w = r0 + (long long)i * WAVES + wave;
      if (w >= rows) w = rows - 1;
      const long long k = w >> rpc_log2, o = w & ((1ll << rpc_log2) - 1);
      const size_t off = (((size_t)ids[k] << rpc_log2) + (size_t)o) * 1024 + (size_t)lane * 16;
      v[i] = load_nt16(base + off);
    }
#pragma unroll
    for (int i = 0; i < PROBE_DEPTH; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if (lane == 0) atomicXor(sink, x);
}

hipError_t launch_gather_read_probe(const void* base, const int32_t* ids, long long num_chunks,
                                    int chunk_bytes, unsigned* sink, int grid,
                                    hipStream_t stream) {
  if (num_chunks == 0) return hipSuccess;
  int rpc_log2 = 0;
  while ((1024 << rpc_log2) < chunk_bytes) ++rpc_log2;
  hipLaunchKernelGGL(gather_read_probe_kernel, dim3(grid), dim3(PROBE_THREADS), 0, stream,
                     (const uint8_t*)base, ids, num_chunks << rpc_log2, rpc_log2, sink);
  return hipGetLastError();
}

}  // namespace pa
