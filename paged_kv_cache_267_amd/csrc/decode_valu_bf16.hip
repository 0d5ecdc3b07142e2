// decode_valu_bf16.hip -- vector-ALU decode instances for bf16 KV caches.
#include "decode_persistent.h"
#include "dispatch.h"
#include "tile_valu.h"

namespace pa {

template <int D, int BS>
static hipError_t by_group(const DecodeParams& p, int G, hipStream_t s) {
  switch (G) {
    case 1: return launch_decode_persistent<ValuTile<KV_BF16, D, BS, 1>>(p, s);
    case 2: return launch_decode_persistent<ValuTile<KV_BF16, D, BS, 2>>(p, s);
    case 4: return launch_decode_persistent<ValuTile<KV_BF16, D, BS, 4>>(p, s);
    case 8: return launch_decode_persistent<ValuTile<KV_BF16, D, BS, 8>>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t decode_valu_bf16(const DecodeParams& p, int D, int BS, int G, hipStream_t s) {
  if (D == 64 && BS == 16) return by_group<64, 16>(p, G, s);
  if (D == 64 && BS == 32) return by_group<64, 32>(p, G, s);
  if (D == 64 && BS == 64) return by_group<64, 64>(p, G, s);
  if (D == 128 && BS == 16) return by_group<128, 16>(p, G, s);
  if (D == 128 && BS == 32) return by_group<128, 32>(p, G, s);
  if (D == 128 && BS == 64) return by_group<128, 64>(p, G, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
