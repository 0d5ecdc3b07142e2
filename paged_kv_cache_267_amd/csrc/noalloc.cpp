// noalloc.cpp -- the partition workspace of pa_decode_split_noalloc in a
// library-held device array, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The entry point and its checks are in api.cpp.
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
#include "dispatch.h"
#include "params.h"

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

namespace pa {

hipError_t decode_split_noalloc(DecodeParams p, int kv_dtype, int D, int BS, int G, bool out_bf16,
                                hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= PA_MAX_DEVICES) return hipErrorInvalidDevice;
  uint8_t* ws = nullptr;
  e = scratch_address(dev, &ws);
  if (e != hipSuccess) return e;
  // part_out [S][Hq][parts][D] fp32, then part_lse [S][Hq][parts]; the caller
  // has checked that both fit in the array
  const size_t rows = (size_t)p.num_seqs * p.num_q_heads * p.max_parts;
  void* out = p.out;
  p.out = nullptr;
  p.part_out = reinterpret_cast<float*>(ws);
  p.part_lse = reinterpret_cast<float*>(ws + rows * (size_t)D * 4);   // a multiple of 256 bytes
  e = dispatch_decode(p, kv_dtype, D, BS, G, stream);
  if (e != hipSuccess) return e;
  // the merge reads only the partitions the split wrote in this call, so no
  // part of the workspace has to start at zero
  return launch_reduce_lse(p.part_out, p.part_lse, p.seq_lens, p.num_seqs, p.num_q_heads, D,
                           p.partition_size, p.max_parts, p.window, out, out_bf16, stream);
}

}  // namespace pa
