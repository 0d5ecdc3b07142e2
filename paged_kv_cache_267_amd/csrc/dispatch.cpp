// dispatch.cpp -- picks the decode kernel family and launch shape.
#include "dispatch.h"

#include "../../include/pa.h"

namespace pa {

hipError_t dispatch_decode(const DecodeParams& p, int kv_dtype, int D, int BS, int G, int parts,
                           hipStream_t stream) {
  const int waves = VALU_WAVES;
  switch (kv_dtype) {
    case PA_F32: return decode_valu_f32(p, D, BS, G, parts, waves, stream);
    case PA_BF16: return decode_valu_bf16(p, D, BS, G, parts, waves, stream);
    case PA_FP8_E4M3: return decode_valu_fp8(p, D, BS, G, parts, waves, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
