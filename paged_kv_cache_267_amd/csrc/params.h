// params.h -- parameter blocks of the decode and extend kernels and the launch
// facts the host side keeps; host-only code (no device builtins), shared by
// the kernels and the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pa {

enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

// Element bytes of a cache entry; a 16-byte group holds 16 / bytes elements.
template <int KV> struct KvTraits;
template <> struct KvTraits<KV_F32> { static constexpr int E = 4; };
template <> struct KvTraits<KV_BF16> { static constexpr int E = 2; };
template <> struct KvTraits<KV_FP8> { static constexpr int E = 1; };

// Devices whose launch facts (compute units, occupancy) are cached; a device
// index beyond this is queried on every launch.
constexpr int PA_MAX_DEVICES = 64;

// Compute units of device dev (host side; 256 if dev < 0 or the query fails),
// queried once per device and kept.
int device_cu_count(int dev);

// Parameters of one decode launch (unsplit when part_out == nullptr).
struct DecodeParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;            // unsplit output [S][Hq][D], query dtype
  float* part_out;      // split: [S][Hq][max_parts][D]
  float* part_lse;      // split: [S][Hq][max_parts]
  float qk_scale;       // scale * k_scale * log2(e): scores in base-2 units
  float v_scale;
  int num_seqs, num_q_heads, num_kv_heads;
  int max_blocks, num_blocks, window;
  int partition_size;   // tokens per partition (split); 0 = whole sequence
  int max_parts;
  int seq_begin, seq_count;  // sequences of this launch (persistent schedule)
};

// Parameters of one multi-token (extend) launch.  Sequence s owns query rows
// qsl[s] .. qsl[s+1]-1, the last of its seq_lens[s] keys.
struct ExtendParams {
  const uint16_t* q;    // [num_tokens][Hq][D] bf16
  const char* kc;
  const char* vc;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qsl;   // [num_seqs + 1]
  uint16_t* out;        // [num_tokens][Hq][D] bf16
  float qk_scale;       // scale * k_scale * log2(e)
  float v_scale;
  int num_seqs, num_tokens, num_q_heads, num_kv_heads, log2g;
  int max_blocks, num_blocks, window;
  int cblocks;          // column blocks per (sequence, KV head)
  int pairs;            // num_seqs * num_kv_heads
};

}  // namespace pa
