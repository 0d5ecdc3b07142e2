// api.cpp -- the C ABI of libpa.so (include/pa.h): host-side validation and
// dispatch to the gfx950 kernel instances.  Validation finishes before the
// first HIP call, so invalid calls never touch the device.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "../../include/pa.h"
#include "dispatch.h"
#include "params.h"

namespace {
thread_local std::string g_hip_error;
}  // namespace

namespace pa {

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  g_hip_error = hipGetErrorString(e);
  return PA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dt) { return dt == PA_F32 ? 4 : dt == PA_BF16 ? 2 : dt == PA_FP8_E4M3 ? 1 : 0; }

bool valid_pair(int q_dtype, int kv_dtype) {
  return (q_dtype == PA_F32 && kv_dtype == PA_F32) || (q_dtype == PA_BF16 && kv_dtype == PA_BF16) ||
         (q_dtype == PA_BF16 && kv_dtype == PA_FP8_E4M3);
}

bool group_supported(int kv_dtype, int G) {
  if (G == 1 || G == 2 || G == 4 || G == 8) return true;
  return G == 16 && kv_dtype != PA_F32;
}

int check_decode(const void* query, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, const int32_t* seq_lens, int block_size,
                 float scale, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                 int max_blocks_per_seq, int num_blocks, int sliding_window, int q_dtype,
                 int kv_dtype, float k_scale, float v_scale) {
  if (!query || !key_cache || !value_cache || !block_tables || !seq_lens) return PA_ERR_NULL;
  if (!valid_pair(q_dtype, kv_dtype)) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || sliding_window < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return PA_ERR_SHAPE;
  if ((long long)max_blocks_per_seq * block_size > (1ll << 30)) return PA_ERR_SHAPE;
  // block-table entries are indexed with 32-bit integers on the device
  if ((long long)num_seqs * max_blocks_per_seq >= (1ll << 31)) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 16 && block_size != 32 && block_size != 64) return PA_ERR_UNSUPPORTED;
  if (!group_supported(kv_dtype, num_q_heads / num_kv_heads)) return PA_ERR_UNSUPPORTED;
  if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache)) return PA_ERR_ALIGN;
  return PA_OK;
}

DecodeParams make_params(const void* query, const void* key_cache, const void* value_cache,
                             const int32_t* block_tables, const int32_t* seq_lens, float scale,
                             int num_seqs, int num_q_heads, int num_kv_heads,
                             int max_blocks_per_seq, int num_blocks, int sliding_window,
                             float k_scale, float v_scale) {
  DecodeParams p{};
  p.q = query;
  p.kc = key_cache;
  p.vc = value_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.qk_scale = (float)((double)scale * (double)k_scale * 1.4426950408889634);
  p.v_scale = v_scale;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.window = sliding_window;
  return p;
}

int check_partition(int block_size, int max_blocks_per_seq, int partition_size,
                    int max_num_partitions) {
  if (partition_size <= 0 || partition_size % block_size != 0 || max_num_partitions <= 0 ||
      max_num_partitions > 65535)
    return PA_ERR_PARTITION;
  if ((long long)max_num_partitions * partition_size < (long long)max_blocks_per_seq * block_size)
    return PA_ERR_PARTITION;
  return PA_OK;
}

}  // namespace pa

using pa::aligned16;
using pa::check_decode;
using pa::check_partition;
using pa::elem_bytes;
using pa::group_supported;
using pa::hip_status;
using pa::make_params;

extern "C" {

int pa_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                         const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int kv_dtype,
                         void* stream) {
  if (!key_cache || !value_cache) return PA_ERR_NULL;
  if (elem_bytes(kv_dtype) == 0) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 16 && block_size != 32 && block_size != 64) return PA_ERR_UNSUPPORTED;
  if (!aligned16(key_cache) || !aligned16(value_cache)) return PA_ERR_ALIGN;
  if (num_tokens == 0) return PA_OK;  // key / value / slot_mapping may be NULL then
  if (!key || !value || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value)) return PA_ERR_ALIGN;
  return hip_status(pa::launch_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping,
                                                 num_tokens, num_kv_heads, head_dim, block_size,
                                                 num_blocks, elem_bytes(kv_dtype),
                                                 (hipStream_t)stream));
}

int pa_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                             void* value_cache, const int32_t* slot_mapping, int num_tokens,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             int src_dtype, float k_scale, float v_scale, void* stream) {
  if (!key_cache || !value_cache) return PA_ERR_NULL;
  if (src_dtype != PA_F32 && src_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 16 && block_size != 32 && block_size != 64) return PA_ERR_UNSUPPORTED;
  if (!aligned16(key_cache) || !aligned16(value_cache)) return PA_ERR_ALIGN;
  if (num_tokens == 0) return PA_OK;  // key / value / slot_mapping may be NULL then
  if (!key || !value || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value)) return PA_ERR_ALIGN;
  return hip_status(pa::launch_reshape_and_cache_fp8(
      key, value, key_cache, value_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
      block_size, num_blocks, elem_bytes(src_dtype), k_scale, v_scale, (hipStream_t)stream));
}

int pa_decode(const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* seq_lens, int block_size, float scale,
              void* out, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
              int max_blocks_per_seq, int num_blocks, int sliding_window, int q_dtype,
              int kv_dtype, float k_scale, float v_scale, void* stream) {
  int st = check_decode(query, key_cache, value_cache, block_tables, seq_lens, block_size, scale,
                        num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                        num_blocks, sliding_window, q_dtype, kv_dtype, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (!out) return PA_ERR_NULL;
  if (!aligned16(out)) return PA_ERR_ALIGN;
  if (num_seqs == 0) return PA_OK;
  pa::DecodeParams p = make_params(query, key_cache, value_cache, block_tables, seq_lens, scale,
                                   num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq,
                                   num_blocks, sliding_window, k_scale, v_scale);
  p.out = out;
  p.partition_size = 0;
  p.max_parts = 1;
  return hip_status(pa::dispatch_decode(p, kv_dtype, head_dim, block_size,
                                        num_q_heads / num_kv_heads, (hipStream_t)stream));
}

int pa_decode_split(const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int block_size,
                    float scale, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                    int max_blocks_per_seq, int num_blocks, int sliding_window, int q_dtype,
                    int kv_dtype, float k_scale, float v_scale, int partition_size,
                    int max_num_partitions, float* part_out, float* part_lse, void* stream) {
  int st = check_decode(query, key_cache, value_cache, block_tables, seq_lens, block_size, scale,
                        num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                        num_blocks, sliding_window, q_dtype, kv_dtype, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (!part_out || !part_lse) return PA_ERR_NULL;
  st = check_partition(block_size, max_blocks_per_seq, partition_size, max_num_partitions);
  if (st != PA_OK) return st;
  if (!aligned16(part_out)) return PA_ERR_ALIGN;
  if (num_seqs == 0) return PA_OK;
  pa::DecodeParams p = make_params(query, key_cache, value_cache, block_tables, seq_lens, scale,
                                   num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq,
                                   num_blocks, sliding_window, k_scale, v_scale);
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.partition_size = partition_size;
  p.max_parts = max_num_partitions;
  return hip_status(pa::dispatch_decode(p, kv_dtype, head_dim, block_size,
                                        num_q_heads / num_kv_heads, (hipStream_t)stream));
}

int pa_decode_split_noalloc(const void* query, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, int block_size,
                            float scale, void* out, int num_seqs, int num_q_heads,
                            int num_kv_heads, int head_dim, int max_blocks_per_seq,
                            int num_blocks, int sliding_window, int q_dtype, int kv_dtype,
                            float k_scale, float v_scale, int partition_size, void* stream) {
  // every check, the workspace size included, happens before any HIP call
  int st = check_decode(query, key_cache, value_cache, block_tables, seq_lens, block_size, scale,
                        num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                        num_blocks, sliding_window, q_dtype, kv_dtype, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (!out) return PA_ERR_NULL;
  if (!aligned16(out)) return PA_ERR_ALIGN;
  if (partition_size <= 0) return PA_ERR_PARTITION;
  const long long span = (long long)max_blocks_per_seq * block_size;
  const long long parts = (span + partition_size - 1) / partition_size;
  if (parts > 65535) return PA_ERR_PARTITION;
  st = check_partition(block_size, max_blocks_per_seq, partition_size, (int)parts);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  if (pa_decode_split_workspace_bytes(num_seqs, num_q_heads, head_dim, (int)parts) >
      PA_NOALLOC_SCRATCH_BYTES)
    return PA_ERR_SCRATCH;
  pa::DecodeParams p = make_params(query, key_cache, value_cache, block_tables, seq_lens, scale,
                                   num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq,
                                   num_blocks, sliding_window, k_scale, v_scale);
  p.out = out;
  p.partition_size = partition_size;
  p.max_parts = (int)parts;
  return hip_status(pa::decode_split_noalloc(p, kv_dtype, head_dim, block_size,
                                             num_q_heads / num_kv_heads, q_dtype == PA_BF16,
                                             (hipStream_t)stream));
}

int pa_extend(const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* seq_lens,
              const int32_t* query_start_loc, int block_size, float scale, void* out,
              int num_seqs, int num_tokens, int max_query_len, int num_q_heads, int num_kv_heads,
              int head_dim, int max_blocks_per_seq, int num_blocks, int sliding_window,
              int q_dtype, int kv_dtype, float k_scale, float v_scale, void* stream) {
  if (q_dtype != PA_BF16 || (kv_dtype != PA_BF16 && kv_dtype != PA_FP8_E4M3))
    return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_tokens < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;  // nothing to read or write
  int st = check_decode(query, key_cache, value_cache, block_tables, seq_lens, block_size, scale,
                        num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                        num_blocks, sliding_window, q_dtype, kv_dtype, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (!query_start_loc || !out) return PA_ERR_NULL;
  if (!(scale > 0.f) || !(k_scale > 0.f)) return PA_ERR_SHAPE;  // the max is taken on raw scores
  if (num_tokens < 0 || max_query_len < 0 || max_query_len > (1 << 20)) return PA_ERR_SHAPE;
  if (num_tokens > (1 << 26)) return PA_ERR_SHAPE;  // column indices (token x head) stay in int
  if (num_tokens > 0 && max_query_len == 0) return PA_ERR_SHAPE;
  if ((long long)num_tokens * num_q_heads * head_dim >= (1ll << 40)) return PA_ERR_SHAPE;
  // one physical block of the cache (every KV head) is addressed with 32 bits
  if ((long long)num_kv_heads * head_dim * block_size * elem_bytes(kv_dtype) >= (1ll << 32))
    return PA_ERR_SHAPE;
  if (!aligned16(out)) return PA_ERR_ALIGN;
  const int G = num_q_heads / num_kv_heads;
  const long long pairs = (long long)num_seqs * num_kv_heads;
  const long long cblocks = (((long long)max_query_len * G) + 127) / 128;  // >= the launch's
  if (8 * ((pairs + 7) / 8) * cblocks >= (1ll << 31)) return PA_ERR_SHAPE;
  pa::ExtendParams p{};
  p.q = (const uint16_t*)query;
  p.kc = (const char*)key_cache;
  p.vc = (const char*)value_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.qsl = query_start_loc;
  p.out = (uint16_t*)out;
  p.qk_scale = (float)((double)scale * (double)k_scale * 1.4426950408889634);
  p.v_scale = v_scale;
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  int lg = 0;
  while ((1 << lg) < G) ++lg;
  p.log2g = lg;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.window = sliding_window;
  return hip_status(pa::launch_extend(p, kv_dtype == PA_BF16 ? pa::KV_BF16 : pa::KV_FP8, head_dim,
                                      block_size, max_query_len, (hipStream_t)stream));
}

int pa_reduce_lse(const float* part_out, const float* part_lse, const int32_t* seq_lens,
                  int num_seqs, int num_q_heads, int head_dim, int partition_size,
                  int max_num_partitions, int sliding_window, void* out, int out_dtype,
                  void* stream) {
  if (!part_out || !part_lse || !seq_lens || !out) return PA_ERR_NULL;
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || sliding_window < 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (partition_size <= 0 || max_num_partitions <= 0) return PA_ERR_PARTITION;
  if (!aligned16(part_out) || !aligned16(out)) return PA_ERR_ALIGN;
  if (num_seqs == 0) return PA_OK;
  if ((long long)num_seqs * num_q_heads >= (1ll << 31)) return PA_ERR_SHAPE;  // rows in int
  return hip_status(pa::launch_reduce_lse(part_out, part_lse, seq_lens, num_seqs, num_q_heads,
                                          head_dim, partition_size, max_num_partitions,
                                          sliding_window, out, out_dtype == PA_BF16,
                                          (hipStream_t)stream));
}

int pa_choose_block_size(const int32_t* seq_lens, int n, double max_waste_frac) {
  if (n < 0 || !(max_waste_frac > 0.0 && max_waste_frac <= 1.0)) return -PA_ERR_SHAPE;
  if (n > 0 && !seq_lens) return -PA_ERR_NULL;
  long long tokens = 0, waste[3] = {0, 0, 0};
  static const int sizes[3] = {64, 32, 16};
  for (int i = 0; i < n; ++i) {
    const long long L = seq_lens[i] > 0 ? seq_lens[i] : 0;
    tokens += L;
    for (int k = 0; k < 3; ++k) waste[k] += (L + sizes[k] - 1) / sizes[k] * sizes[k] - L;
  }
  if (tokens == 0) return 16;
  for (int k = 0; k < 3; ++k)
    if ((double)waste[k] <= max_waste_frac * (double)tokens) return sizes[k];
  return 16;
}

size_t pa_decode_split_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                       int max_num_partitions) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_num_partitions <= 0) return 0;
  const size_t rows = (size_t)num_seqs * num_q_heads * max_num_partitions;
  return rows * (size_t)head_dim * 4 + rows * 4;
}

int pa_fp8_e4m3_dequantize(const uint8_t* codes, float scale, float* out, long long n,
                           void* stream) {
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!codes || !out) return PA_ERR_NULL;
  if (!aligned16(out)) return PA_ERR_ALIGN;
  return hip_status(pa::launch_fp8_dequant(codes, scale, out, n, (hipStream_t)stream));
}

int pa_probe_gather_read(const void* base, const int32_t* ids, long long num_chunks,
                         int chunk_bytes, unsigned* sink, int grid, void* stream) {
  if (num_chunks < 0 || grid < 0) return PA_ERR_SHAPE;
  if (chunk_bytes < 1024 || chunk_bytes > (1 << 20) || (chunk_bytes & (chunk_bytes - 1)))
    return PA_ERR_SHAPE;
  if (num_chunks == 0) return PA_OK;
  if (!base || !ids || !sink) return PA_ERR_NULL;
  if (!aligned16(base)) return PA_ERR_ALIGN;
  if (grid == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    grid = 8 * pa::device_cu_count(dev);
  }
  return hip_status(pa::launch_gather_read_probe(base, ids, num_chunks, chunk_bytes, sink, grid,
                                                 (hipStream_t)stream));
}

int pa_set_decode_kernel(int choice) {
  return pa::set_decode_kernel(choice) == 0 ? PA_OK : PA_ERR_UNSUPPORTED;
}

int pa_get_decode_kernel(void) { return pa::get_decode_kernel(); }

const char* pa_decode_kernel_name(int kv_dtype, int num_q_heads, int num_kv_heads) {
  if (kv_dtype != PA_F32 && kv_dtype != PA_BF16 && kv_dtype != PA_FP8_E4M3) return "";
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return "";
  const int G = num_q_heads / num_kv_heads;
  if (!group_supported(kv_dtype, G)) return "";
  return pa::decode_uses_mfma(kv_dtype, G) ? "mfma" : "valu";
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_DTYPE: return "unsupported dtype or (query, KV) dtype pair";
    case PA_ERR_SHAPE: return "invalid size or head counts";
    case PA_ERR_UNSUPPORTED: return "head_dim, block_size, GQA group size or kernel choice not supported";
    case PA_ERR_PARTITION: return "invalid partition_size or max_num_partitions";
    case PA_ERR_HIP: return "HIP kernel launch failed";
    case PA_ERR_ALIGN: return "a buffer is not 16-byte aligned";
    case PA_ERR_EXHAUSTED: return "the block pool has too few free blocks";
    case PA_ERR_SCRATCH: return "the partition workspace exceeds the library's fixed scratch array";
    default: return "unknown status";
  }
}

const char* pa_last_hip_error(void) { return g_hip_error.c_str(); }

}  // extern "C"
