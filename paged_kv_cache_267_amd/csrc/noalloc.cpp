// noalloc.cpp -- pa_decode_split_noalloc: split decode + LSE merge with the
// partition workspace in a library-held device array, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array `scratch` is a file-scope device variable: every GPU the library
// runs on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in for the symbol; the device address is
// taken once per device with hipGetSymbolAddress (on the first call made on
// that device, with it current) and only that address reaches the kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/pa.h"
#include "common.h"
#include "dispatch.h"

namespace {

static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

std::atomic<uint8_t*> g_scratch_of[pa::PA_MAX_DEVICES];   // nullptr: not yet taken
std::mutex g_scratch_mu;

// Device address of device dev's copy of `scratch`; dev is the current device.
hipError_t scratch_address(int dev, uint8_t** out) {
  *out = g_scratch_of[dev].load(std::memory_order_acquire);
  if (*out) return hipSuccess;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  *out = g_scratch_of[dev].load(std::memory_order_relaxed);
  if (*out) return hipSuccess;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (addr == nullptr) return hipErrorInvalidSymbol;
  *out = static_cast<uint8_t*>(addr);
  g_scratch_of[dev].store(*out, std::memory_order_release);
  return hipSuccess;
}

}  // namespace

extern "C" int pa_decode_split_noalloc(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* seq_lens, int block_size, float scale, void* out,
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_blocks_per_seq,
    int num_blocks, int sliding_window, int q_dtype, int kv_dtype, float k_scale, float v_scale,
    int partition_size, void* stream) {
  // every check happens before the first HIP call
  int st = pa::check_decode(query, key_cache, value_cache, block_tables, seq_lens, block_size,
                            scale, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            max_blocks_per_seq, num_blocks, sliding_window, q_dtype, kv_dtype,
                            k_scale, v_scale);
  if (st != PA_OK) return st;
  if (!out) return PA_ERR_NULL;
  if (!pa::aligned16(out)) return PA_ERR_ALIGN;
  if (partition_size <= 0) return PA_ERR_PARTITION;
  const long long span = (long long)max_blocks_per_seq * block_size;
  const long long parts = (span + partition_size - 1) / partition_size;
  if (parts > 65535) return PA_ERR_PARTITION;
  st = pa::check_partition(block_size, max_blocks_per_seq, partition_size, (int)parts);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  // workspace: part_out [S][Hq][parts][D] fp32, then part_lse [S][Hq][parts]
  const unsigned long long rows = (unsigned long long)num_seqs * num_q_heads * parts;
  const unsigned long long out_bytes = rows * (unsigned long long)head_dim * 4;
  if (out_bytes + rows * 4 > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pa::hip_status(e);
  if (dev < 0 || dev >= pa::PA_MAX_DEVICES) return pa::hip_status(hipErrorInvalidDevice);
  uint8_t* ws = nullptr;
  e = scratch_address(dev, &ws);
  if (e != hipSuccess) return pa::hip_status(e);

  pa::DecodeParams p = pa::make_params(query, key_cache, value_cache, block_tables, seq_lens,
                                       scale, num_seqs, num_q_heads, num_kv_heads,
                                       max_blocks_per_seq, num_blocks, sliding_window, k_scale,
                                       v_scale);
  p.part_out = reinterpret_cast<float*>(ws);
  p.part_lse = reinterpret_cast<float*>(ws + out_bytes);   // out_bytes is a multiple of 256
  p.partition_size = partition_size;
  p.max_parts = (int)parts;
  e = pa::dispatch_decode(p, kv_dtype, head_dim, block_size, num_q_heads / num_kv_heads,
                          (hipStream_t)stream);
  if (e != hipSuccess) return pa::hip_status(e);
  // the merge reads only the partitions the split wrote in this call, so no
  // part of the workspace has to start at zero
  return pa::hip_status(pa::launch_reduce_lse(p.part_out, p.part_lse, seq_lens, num_seqs,
                                              num_q_heads, head_dim, partition_size, (int)parts,
                                              sliding_window, out, q_dtype == PA_BF16,
                                              (hipStream_t)stream));
}
