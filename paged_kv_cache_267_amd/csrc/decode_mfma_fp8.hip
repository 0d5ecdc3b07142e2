// decode_mfma_fp8.hip -- instances of the matrix-core decode kernel for fp8 KV caches.
#include "decode_mfma.h"
#include "dispatch.h"

namespace pa {

template <int D, int BS>
static hipError_t by_group(const DecodeParams& p, int G, int parts, hipStream_t s) {
  switch (G) {
    case 1: return launch_decode_mfma<KV_FP8, D, BS, 1>(p, parts, s);
    case 2: return launch_decode_mfma<KV_FP8, D, BS, 2>(p, parts, s);
    case 4: return launch_decode_mfma<KV_FP8, D, BS, 4>(p, parts, s);
    case 8: return launch_decode_mfma<KV_FP8, D, BS, 8>(p, parts, s);
    case 16: return launch_decode_mfma<KV_FP8, D, BS, 16>(p, parts, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t decode_mfma_fp8(const DecodeParams& p, int D, int BS, int G, int parts,
                           hipStream_t s) {
  if (D == 64 && BS == 16) return by_group<64, 16>(p, G, parts, s);
  if (D == 64 && BS == 32) return by_group<64, 32>(p, G, parts, s);
  if (D == 128 && BS == 16) return by_group<128, 16>(p, G, parts, s);
  if (D == 128 && BS == 32) return by_group<128, 32>(p, G, parts, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
