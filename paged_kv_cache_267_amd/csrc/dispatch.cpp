// dispatch.cpp -- picks the decode kernel family and launch shape.
#include "dispatch.h"

#include "../../include/pa.h"

#include <atomic>

namespace pa {

// The kernel-family choice belongs to the calling host thread: a call reads
// the setting of the thread that makes it, so threads never race on it.
static thread_local int g_choice = PA_KERNEL_AUTO;

int device_cu_count(int dev) {
  static std::atomic<int> cached[PA_MAX_DEVICES];   // 0: not yet known
  if (dev >= 0 && dev < PA_MAX_DEVICES) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return 256;
  if (dev < PA_MAX_DEVICES) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int set_decode_kernel(int choice) {
  if (choice != PA_KERNEL_AUTO && choice != PA_KERNEL_VALU && choice != PA_KERNEL_MFMA) return -1;
  g_choice = choice;
  return 0;
}
int get_decode_kernel() { return g_choice; }

// Automatic choice: the matrix cores take groups of 8 or more query heads per
// KV head; smaller groups use the VALU bandwidth path (f32 caches always do).
// Groups of 16 exist only on the matrix cores.
bool decode_uses_mfma(int kv_dtype, int G) {
  if (kv_dtype == PA_F32) return false;
  if (G > 8) return true;
  switch (get_decode_kernel()) {
    case PA_KERNEL_VALU: return false;
    case PA_KERNEL_MFMA: return true;
    default: return G >= 8;
  }
}

hipError_t dispatch_decode(const DecodeParams& p, int kv_dtype, int D, int BS, int G,
                           hipStream_t stream) {
  if (decode_uses_mfma(kv_dtype, G)) {
    if (kv_dtype == PA_BF16) return decode_mfma_bf16(p, D, BS, G, stream);
    return decode_mfma_fp8(p, D, BS, G, stream);
  }
  switch (kv_dtype) {
    case PA_F32: return decode_valu_f32(p, D, BS, G, stream);
    case PA_BF16: return decode_valu_bf16(p, D, BS, G, stream);
    case PA_FP8_E4M3: return decode_valu_fp8(p, D, BS, G, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
