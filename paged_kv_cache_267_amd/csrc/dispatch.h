// dispatch.h -- host-side entry points of the kernel instances.
#pragma once

#include <hip/hip_runtime_api.h>

#include "params.h"

namespace pa {

// Decode instances on the persistent driver (decode_persistent.h), one function
// per (tile computation, KV element type); they switch over (head_dim,
// block_size, group) and return hipErrorInvalidValue for a combination that is
// not instantiated.  Vector-ALU tiles: G in {1, 2, 4, 8}; matrix-core tiles
// (bf16 / E4M3 caches): G in {1, 2, 4, 8, 16}.
hipError_t decode_valu_f32(const DecodeParams& p, int D, int BS, int G, hipStream_t stream);
hipError_t decode_valu_bf16(const DecodeParams& p, int D, int BS, int G, hipStream_t stream);
hipError_t decode_valu_fp8(const DecodeParams& p, int D, int BS, int G, hipStream_t stream);
hipError_t decode_mfma_bf16(const DecodeParams& p, int D, int BS, int G, hipStream_t stream);
hipError_t decode_mfma_fp8(const DecodeParams& p, int D, int BS, int G, hipStream_t stream);

// Kernel-family choice (pa_kernel_choice) of the calling host thread; set
// returns -1 for an unknown value.
int set_decode_kernel(int choice);
int get_decode_kernel();

// True when the matrix-core kernel serves (KV dtype, group size) under the
// current choice.
bool decode_uses_mfma(int kv_dtype, int G);

// Host-side argument handling shared by the entry points of api.cpp and
// noalloc.cpp: checks return a pa_status (PA_OK when the call may proceed).
int hip_status(hipError_t e);   // PA_OK, or PA_ERR_HIP with the text kept per thread
bool aligned16(const void* p);
int check_decode(const void* query, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, const int32_t* seq_lens, int block_size,
                 float scale, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                 int max_blocks_per_seq, int num_blocks, int sliding_window, int q_dtype,
                 int kv_dtype, float k_scale, float v_scale);
int check_partition(int block_size, int max_blocks_per_seq, int partition_size,
                    int max_num_partitions);
DecodeParams make_params(const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, float scale,
                         int num_seqs, int num_q_heads, int num_kv_heads, int max_blocks_per_seq,
                         int num_blocks, int sliding_window, float k_scale, float v_scale);

// Split decode + LSE merge with the partition workspace (part_out, then
// part_lse, for p.max_parts partitions) in the library's own device array
// (noalloc.cpp); p is a split launch whose arguments have been checked.
hipError_t decode_split_noalloc(DecodeParams p, int kv_dtype, int D, int BS, int G, bool out_bf16,
                                hipStream_t stream);

// Chooses the tile computation for (KV dtype, group size) and launches it.
hipError_t dispatch_decode(const DecodeParams& p, int kv_dtype, int D, int BS, int G,
                           hipStream_t stream);

// Multi-token attention (extend_mfma.hip): bf16 queries, bf16 or E4M3 caches,
// head_dim {64, 128}, block_size {16, 32, 64}, any power-of-two group.
// max_query_len bounds the chunk lengths; cblocks and pairs are filled in.
hipError_t launch_extend(ExtendParams p, int kv_dtype, int D, int BS, int max_query_len,
                         hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kc, void* vc,
                                    const int32_t* slots, int T, int Hkv, int D, int bs,
                                    int num_blocks, int elem_bytes, hipStream_t stream);
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* kc, void* vc,
                                        const int32_t* slots, int T, int Hkv, int D, int bs,
                                        int num_blocks, int src_bytes, float k_scale,
                                        float v_scale, hipStream_t stream);
hipError_t launch_reduce_lse(const float* part_out, const float* part_lse,
                             const int32_t* seq_lens, int S, int Hq, int D, int P, int max_parts,
                             int window, void* out, bool out_bf16, hipStream_t stream);
hipError_t launch_gather_read_probe(const void* base, const int32_t* ids, long long num_chunks,
                                    int chunk_bytes, unsigned* sink, int grid,
                                    hipStream_t stream);
hipError_t launch_fp8_dequant(const uint8_t* codes, float scale, float* out, long long n,
                              hipStream_t stream);

}  // namespace pa
