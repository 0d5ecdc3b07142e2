// probe.hip -- a bandwidth probe with the decode kernels' access pattern:
// whole chunks (the size of one (block, head) K or V tile) read by one wave
// each with 16-byte non-temporal loads, in the order of a chunk-id list.  With a random
// permutation it measures what HBM delivers to a paged gather; with ids in
// order, a plain streaming read.  Nothing is computed but an XOR of the data.
#include "common.h"

namespace pa {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_DEPTH = 4;   // 1 KiB loads per wave in flight
constexpr unsigned PROBE_MAGIC = 0x9e3779b9u;

// Each wave reads whole chunks, one 1 KiB row per load (64 lanes x 16 bytes),
// as a decode wave reads a K or V tile: wave w of the grid takes list entries
// w, w + W, w + 2W, ... (W waves in the grid), and its rows run through them
// in order, PROBE_DEPTH rows per round.  Row indices are wave-uniform, so the
// chunk lookup is scalar work.
__global__ __launch_bounds__(PROBE_THREADS) void gather_read_probe_kernel(
    const uint8_t* __restrict__ base, const int32_t* __restrict__ ids, long long num_chunks,
    int rpc_log2, unsigned* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const long long nw = (long long)gridDim.x * (PROBE_THREADS / 64);
  const long long w = (long long)blockIdx.x * (PROBE_THREADS / 64) + wave_id();
  const long long mine = w < num_chunks ? (num_chunks - 1 - w) / nw + 1 : 0;  // chunks of this wave
  const long long rows = mine << rpc_log2;
  const long long rmask = (1ll << rpc_log2) - 1;
  unsigned x = 0;
  for (long long r0 = 0; r0 < rows; r0 += PROBE_DEPTH) {
    uint4 v[PROBE_DEPTH];
#pragma unroll
    for (int i = 0; i < PROBE_DEPTH; ++i) {
      long long n = r0 + i;
      if (n >= rows) n = rows - 1;
      const long long k = w + (n >> rpc_log2) * nw;
      const size_t off = (((size_t)ids[k] << rpc_log2) + (size_t)(n & rmask)) * 1024 +
                         (size_t)lane * 16;
      v[i] = load_nt16(base + off);
    }
#pragma unroll
    for (int i = 0; i < PROBE_DEPTH; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  // a store that depends on every loaded word keeps the loads; it happens only
  // for one value of the wave's XOR, so the waves do not contend for the word
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if (lane == 0 && x == PROBE_MAGIC) *sink = x;
}

hipError_t launch_gather_read_probe(const void* base, const int32_t* ids, long long num_chunks,
                                    int chunk_bytes, unsigned* sink, int grid,
                                    hipStream_t stream) {
  if (num_chunks == 0) return hipSuccess;
  int rpc_log2 = 0;
  while ((1024 << rpc_log2) < chunk_bytes) ++rpc_log2;
  hipLaunchKernelGGL(gather_read_probe_kernel, dim3(grid), dim3(PROBE_THREADS), 0, stream,
                     (const uint8_t*)base, ids, num_chunks, rpc_log2, sink);
  return hipGetLastError();
}

}  // namespace pa
