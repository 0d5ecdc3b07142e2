/*
 * pa.h -- C ABI of the MI355X (gfx950) paged decode-attention library, libpa.so.
 *
 * The operation is PagedAttention decode: one query token per sequence attends
 * to that sequence's keys and values, which live in fixed-size physical blocks
 * of a shared pool and are found through the sequence's block table.
 *
 * Sources (page title, section):
 *   [P2] "vLLM deployment and PagedAttention" (crazysre.cn), "Core concept":
 *        KV cache cut into blocks of block_size tokens; a per-request block
 *        table maps logical blocks to non-contiguous physical blocks, and
 *        requests with a common prefix may share physical blocks.
 *   [P3] "vLLM 0.5 deep dive: PagedAttention architecture" (chenxutan.com):
 *        s2.1 block pool and allocation, s2.2 the attention interface
 *        forward(query, key_cache, value_cache, block_table, seq_lens) with
 *        scale = head_dim^-0.5, s2.3 the kernel's argument list (query,
 *        key_cache, value_cache, int block_tables, output, scale, ...) and its
 *        max/sum softmax state, s3.4 FP8 KV cache with a scale and zero point 0.
 *   [P1] "vLLM 0.7.2 deep dive: PagedAttention v2 with FlashAttention-3"
 *        (jsqmd.com): s2.1 physical blocks shared by several sequences,
 *        s2.2 grouped-query heads and the fp8_e4m3 KV cache, s2.3 the 4K
 *        sliding window (mask keys outside it; never load blocks wholly
 *        outside it).
 *
 * Conventions shared by every entry point
 *   - All buffer pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing.  Its state: the decode kernel-family choice
 *     of each host thread (pa_set_decode_kernel), and per-device launch facts
 *     (compute units, kernel occupancy) found at a device's first launch and
 *     kept.  Calls from several host threads may overlap.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call validates its arguments on the host, enqueues its kernels on
 *     `stream` and returns without synchronising.  Validation happens before
 *     any HIP call, so an invalid call never touches the device.
 *   - query, out, both caches, key/value and part_out must be 16-byte aligned
 *     (PA_ERR_ALIGN otherwise); int32 arrays need only their natural alignment.
 *   - Return value: a pa_status.  PA_ERR_HIP reports a failed launch
 *     (hipGetLastError); pa_last_hip_error() gives its text.
 *   - dtype arguments take a pa_dtype.  Supported (query, KV) pairs:
 *     (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).  bf16 and f32 outputs are
 *     rounded to nearest even from fp32.
 *   - GQA: G = num_q_heads / num_kv_heads; query head h reads KV head h / G.
 *     Supported: head_dim in {64, 128}, block_size in {16, 32, 64} (the
 *     sizes [P3 s3.1] offers),
 *     G in {1, 2, 4, 8} for every KV dtype and G = 16 for bf16 / FP8 KV.
 *
 * Layouts (element = one cache entry; X = 16 / element bytes, so one X-group
 * is 16 bytes: X = 4 for f32, 8 for bf16, 16 for FP8):
 *   query, out      [num_seqs][num_q_heads][head_dim]
 *   value_cache     [num_blocks][num_kv_heads][head_dim][block_size]
 *                   -- the order of [P3 s2.2]; element (b,h,d,o) at
 *                   ((b*Hkv + h)*D + d)*bs + o.
 *   key_cache       [num_blocks][num_kv_heads][head_dim/X][block_size][X]
 *                   -- [P3 s2.2]'s order with head_dim cut into 16-byte
 *                   groups stored innermost; element (b,h,d,o) at
 *                   (((b*Hkv + h)*(D/X) + d/X)*bs + o)*X + d%X.
 *                   Each (block, head) tile of either cache is D*bs
 *                   contiguous elements.
 *   block_tables    int32 [num_seqs][max_blocks_per_seq]; logical block i of
 *                   sequence s lives in physical block block_tables[s][i].
 *   seq_lens        int32 [num_seqs]; keys of sequence s are positions
 *                   0..seq_lens[s]-1 and its query is position seq_lens[s]-1.
 *
 * Device-data preconditions (not checked on the host: the data lives on the
 * device):
 *   0 <= seq_lens[s] <= max_blocks_per_seq * block_size; table entries the
 *   call reads (logical blocks holding in-window keys) lie in [0, num_blocks).
 *   Entries past the last block or wholly before the window may hold
 *   anything (e.g. -1) and are never read.  Out-of-range lengths are clamped
 *   and out-of-range block ids are clamped into the pool, so a violating call
 *   gives unspecified values but never reads outside the caches.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  PA_ERR_DTYPE = 2,       /* unknown dtype or unsupported (query, KV) pair     */
  PA_ERR_SHAPE = 3,       /* non-positive size, or num_q_heads % num_kv_heads  */
  PA_ERR_UNSUPPORTED = 4, /* head_dim / block_size / group size not built      */
  PA_ERR_PARTITION = 5,   /* bad partition_size / max_num_partitions           */
  PA_ERR_HIP = 6,         /* a kernel launch failed                            */
  PA_ERR_ALIGN = 7,       /* a buffer is not 16-byte aligned                   */
  PA_ERR_EXHAUSTED = 8,   /* the block pool has too few free blocks            */
  PA_ERR_SCRATCH = 9      /* workspace beyond PA_NOALLOC_SCRATCH_BYTES         */
} pa_status;

/*
 * pa_reshape_and_cache -- append new tokens' K/V into their cache slots.
 *   [P3 s2.1] places a request's tokens in ceil(n/block_size) blocks; [P2]
 *   maps them through the block table.  slot_mapping[t] = physical_block *
 *   block_size + offset, computed by the caller from the table.
 * key, value     [num_tokens][num_kv_heads][head_dim] elements of kv_dtype
 *                (for FP8_E4M3 these are already E4M3 codes).
 * slot_mapping   int32 [num_tokens]; a negative slot skips the token; a slot
 *                >= num_blocks*block_size is also skipped.
 * The copy is bit-exact and touches only the named slots.  Non-negative slots
 * must be distinct (two tokens to one slot leave either one's bytes).
 * num_tokens = 0 is a valid no-op (key, value and slot_mapping may be NULL).
 */
int pa_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                         const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int kv_dtype,
                         void* stream);

/*
 * pa_reshape_and_cache_fp8 -- the same write into E4M3 caches, quantising on
 * the way ([P3 s3.4]: an FP8 KV cache with a per-tensor scale and zero point
 * 0; [P1 s2.2]: fp8_e4m3).  key / value are [num_tokens][num_kv_heads]
 * [head_dim] in src_dtype (PA_F32 or PA_BF16); element x of K is stored as the
 * E4M3 code nearest to the binary32 quotient x / k_scale (ties to even,
 * saturating at +-448 including infinities, NaN -> 0x7F), V likewise with
 * v_scale.  Caches, slots, alignment and errors as pa_reshape_and_cache;
 * k_scale and v_scale must be finite and > 0 (PA_ERR_SHAPE otherwise).  The
 * decode entry points then read the cache with kv_dtype = PA_FP8_E4M3 and the
 * same scales.
 */
int pa_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                             void* value_cache, const int32_t* slot_mapping, int num_tokens,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             int src_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_decode -- one query per sequence against its paged K/V, in one pass per
 * (sequence, KV head) ([P3 s2.2/s2.3], [P1 s2.2/s2.3]).
 *   For query head h of sequence s, with L = seq_lens[s], G = Hq/Hkv,
 *   lo = sliding_window > 0 ? max(0, L - sliding_window) : 0:
 *     s_j = scale * k_scale * sum_d q[d] k_j[d]          for j in [lo, L)
 *     out = v_scale * sum_j softmax(s)_j v_j             (fp32 accumulation)
 *   where k_j, v_j are the stored elements of key/value head h/G (E4M3 codes
 *   decoded to their value).  L = 0 gives a zero row.
 * query   [num_seqs][num_q_heads][head_dim] of q_dtype; out: same shape and dtype.
 * scale   the softmax scale as fp32 (normally head_dim^-0.5, [P3 s2.2]).
 * k_scale, v_scale  per-tensor FP8 dequantisation scales ([P3 s3.4], zero
 *         point 0); pass 1.0f for f32 / bf16 caches.
 * sliding_window  0 = off.
 * out must not alias any input.
 */
int pa_decode(const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* seq_lens, int block_size, float scale,
              void* out, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
              int max_blocks_per_seq, int num_blocks, int sliding_window, int q_dtype,
              int kv_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_decode_split -- the same attention cut into partitions of partition_size
 * logical tokens (partition p covers [p*P, (p+1)*P) intersected with
 * [lo, L)); each partition is normalised on its own and reports its
 * log-sum-exp, so that pa_reduce_lse can merge them.
 * partition_size      a multiple of block_size (and of 16), > 0.
 * max_num_partitions  >= ceil(max_blocks_per_seq * block_size / partition_size),
 *                     and at most 65535 (else PA_ERR_PARTITION).
 * part_out  fp32 [num_seqs][num_q_heads][max_num_partitions][head_dim]:
 *           softmax-weighted V of the partition (already divided by its sum).
 * part_lse  fp32 [num_seqs][num_q_heads][max_num_partitions]: natural-log
 *           log-sum-exp of the partition's scaled scores s_j.
 * Only partitions that meet [lo, L) are written; the entries of the others
 * are left as they are (pa_reduce_lse never reads them).
 * Both buffers together are pa_decode_split_workspace_bytes(...) bytes.
 */
int pa_decode_split(const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int block_size,
                    float scale, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                    int max_blocks_per_seq, int num_blocks, int sliding_window, int q_dtype,
                    int kv_dtype, float k_scale, float v_scale, int partition_size,
                    int max_num_partitions, float* part_out, float* part_lse, void* stream);

/*
 * pa_extend -- multi-token paged attention: each sequence appends a chunk of
 * new query tokens after its cached ones and attends causally over the paged
 * cache.  This is the attention step of prefix caching ([P3 s4.4]: requests
 * that share a cached system prompt compute only the tokens after it) and of
 * chunked prefill ([P3 s5.2]: a prompt enters in chunks).
 *   Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1]-1
 *   (n_s tokens); they are the last n_s of its L = seq_lens[s] keys, whose
 *   K/V must already be in the cache (pa_reshape_and_cache).  Token i sits at
 *   position p = L - n_s + i and, for query head h (KV head h / G):
 *     lo = sliding_window > 0 ? max(0, p + 1 - sliding_window) : 0
 *     s_j = scale * k_scale * sum_d q[d] k_j[d]            for j in [lo, p]
 *     out = v_scale * sum_j softmax(s)_j v_j               (fp32 accumulation)
 *   i.e. pa_decode's rule for the sequence cut after p.  A token at a
 *   negative position (n_s > L) gets a zero row.  n_s = 1 for every sequence
 *   is decode.
 * query, out        [num_tokens][num_q_heads][head_dim] bf16 (q_dtype must be
 *                   PA_BF16, out is bf16); kv_dtype PA_BF16 or PA_FP8_E4M3
 *                   (PA_ERR_DTYPE otherwise).
 * query_start_loc   int32 DEVICE array [num_seqs + 1], non-decreasing, from 0
 *                   to num_tokens.
 * max_query_len     >= every n_s (the launch is sized by it); 1 .. 2^20 when
 *                   num_tokens > 0.
 * num_tokens        <= 2^26.
 * scale, k_scale    finite and > 0 (PA_ERR_SHAPE otherwise).
 * Caches, block tables, seq_lens, head_dim, block_size, group sizes, scales,
 * alignment and the clamping of out-of-range device data are as for
 * pa_decode; rows of a sequence whose n_s exceeds max_query_len, or beyond
 * num_tokens, are left unspecified.  num_seqs = 0 or num_tokens = 0 is a
 * no-op once the dtypes pass (every pointer may then be NULL).  out must not
 * alias any input.
 */
int pa_extend(const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* seq_lens,
              const int32_t* query_start_loc, int block_size, float scale, void* out,
              int num_seqs, int num_tokens, int max_query_len, int num_q_heads, int num_kv_heads,
              int head_dim, int max_blocks_per_seq, int num_blocks, int sliding_window,
              int q_dtype, int kv_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_reduce_lse -- merge the partitions written by pa_decode_split:
 *   M = max_p lse_p;  out = sum_p e^(lse_p - M) o_p / sum_p e^(lse_p - M)
 * over the non-empty partitions of each row (found from seq_lens,
 * partition_size and sliding_window; the others are not read).  A row with
 * L = 0 gets zeros.  out: [num_seqs][num_q_heads][head_dim] of out_dtype
 * (F32 or BF16).  seq_lens must be the lengths pa_decode_split was given and
 * meet its precondition (L <= max_blocks_per_seq * block_size): the split
 * kernel clamps a longer length to the table's capacity, this merge does not
 * know that capacity, so for such a row it would merge partitions the split
 * never wrote and the row is unspecified (reads stay inside the workspace).
 */
int pa_reduce_lse(const float* part_out, const float* part_lse, const int32_t* seq_lens,
                  int num_seqs, int num_q_heads, int head_dim, int partition_size,
                  int max_num_partitions, int sliding_window, void* out, int out_dtype,
                  void* stream);

/*
 * pa_choose_block_size -- the automatic block size of [P3 s3.1] (16, 32 or 64
 * tokens; short requests want small pages, long ones large pages) and of the
 * tuning notes at the end of [P3] (small blocks: flexible, more to manage;
 * large blocks: simple, may waste).  Reading: the largest of 64, 32 and 16
 * whose tail waste over the given lengths, sum(ceil(L / bs) * bs - L), is at
 * most max_waste_frac * sum(L); 16 if none is.  seq_lens is a HOST array of n
 * expected lengths (negative values count as 0); an all-zero set gives 16.
 * Returns the block size, or -PA_ERR_NULL (seq_lens NULL with n > 0),
 * -PA_ERR_SHAPE (n < 0, or max_waste_frac not in (0, 1]).
 */
int pa_choose_block_size(const int32_t* seq_lens, int n, double max_waste_frac);

/*
 * pa_decode_split_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): pa_decode_split followed by pa_reduce_lse in one call, with
 * the partition workspace in a device array the library holds, so the call
 * allocates nothing.  Arguments are pa_decode's, then partition_size;
 * out [num_seqs][num_q_heads][head_dim] is of q_dtype.  The number of
 * partitions is ceil(max_blocks_per_seq * block_size / partition_size), and
 * the workspace, pa_decode_split_workspace_bytes(num_seqs, num_q_heads,
 * head_dim, that number), must fit in PA_NOALLOC_SCRATCH_BYTES
 * (PA_ERR_SCRATCH otherwise, before any HIP call).  Every GPU the library
 * runs on holds one such array from its first use until the process ends.
 * Calls that overlap on one GPU (other streams or host threads) share it and
 * race: order them.  Results equal pa_decode_split + pa_reduce_lse on the
 * same arguments.  Other errors as pa_decode_split.
 */
#define PA_NOALLOC_SCRATCH_BYTES (128u << 20)
int pa_decode_split_noalloc(const void* query, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, int block_size,
                            float scale, void* out, int num_seqs, int num_q_heads,
                            int num_kv_heads, int head_dim, int max_blocks_per_seq,
                            int num_blocks, int sliding_window, int q_dtype, int kv_dtype,
                            float k_scale, float v_scale, int partition_size, void* stream);

/* Bytes of part_out + part_lse for pa_decode_split (part_lse starts at
   offset num_seqs*num_q_heads*max_num_partitions*head_dim*4). */
size_t pa_decode_split_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                       int max_num_partitions);

/*
 * pa_fp8_e4m3_dequantize -- out[i] = value(codes[i]) * scale for i < n, with
 * the same device conversion of OCP E4M3 codes that the decode kernels use
 * ([P1 s2.2] fp8_e4m3 cache, [P3 s3.4] scale with zero point 0).  codes need
 * no alignment; out must be 16-byte aligned.  n = 0 is a no-op.
 */
int pa_fp8_e4m3_dequantize(const uint8_t* codes, float scale, float* out, long long n,
                           void* stream);

/*
 * Decode kernel family.  Both families run the same persistent, balanced
 * schedule over (sequence, KV head, partition) segments and differ in the
 * per-tile arithmetic: a vector-ALU tile (dot products on the VALU) and a
 * matrix-core tile (both contractions on MFMA; bf16 and E4M3 caches only).
 * PA_KERNEL_AUTO picks per call from the KV dtype and the group size
 * G = num_q_heads / num_kv_heads; the other values force a family wherever it
 * applies (f32 caches always run the vector-ALU tile, groups of 16 always the
 * matrix-core tile).  The choice is per host thread (a call uses the setting
 * of the thread that makes it) and exists for tests and tuning.
 */
typedef enum { PA_KERNEL_AUTO = 0, PA_KERNEL_VALU = 1, PA_KERNEL_MFMA = 2 } pa_kernel_choice;

/* Sets the calling thread's choice; PA_ERR_UNSUPPORTED for a value outside the enum. */
int pa_set_decode_kernel(int choice);

/* The calling thread's current choice. */
int pa_get_decode_kernel(void);

/* Name of the kernel family ("valu" or "mfma") that pa_decode / pa_decode_split
   run for these arguments under the current choice; "" if the combination is
   not supported. */
const char* pa_decode_kernel_name(int kv_dtype, int num_q_heads, int num_kv_heads);

/*
 * pa_probe_gather_read -- a measurement aid, not part of the attention path:
 * reads num_chunks chunks of chunk_bytes bytes, chunk k at
 * base + ids[k] * chunk_bytes, with the 16-byte non-temporal loads the decode
 * kernels use for K/V tiles (each chunk by one wave).  *sink (one device word)
 * is written only when the XOR of a wave's data equals 0x9e3779b9, a store
 * that keeps the loads from being dropped; callers need not read it.  With ids a random permutation it measures how fast HBM
 * serves a paged gather of tiles of that size; with ids in order, a streaming
 * read.  chunk_bytes: a power of two in [1024, 1 << 20]; base 16-byte aligned;
 * every ids[k] must address a chunk inside the caller's buffer (not checked).
 * grid = 0 picks 8 workgroups per compute unit.  num_chunks = 0 is a no-op.
 */
int pa_probe_gather_read(const void* base, const int32_t* ids, long long num_chunks,
                         int chunk_bytes, unsigned* sink, int grid, void* stream);

/*
 * Host block manager (no device memory, no GPU calls): the pool of physical
 * blocks behind the block tables.  [P3 s2.1]: a request holds ceil(n /
 * block_size) blocks of a fixed pool, allocated as its tokens arrive; [P2
 * "Core concept"] and [P1 s2.1]: block tables over non-contiguous blocks,
 * requests with a common prefix share its blocks; [P1 s2.3]: blocks wholly
 * before a sliding window are no longer needed.
 *   - Blocks carry reference counts; the free list is FIFO.
 *   - pa_bm_new_sequence(m, parent): parent < 0 starts an empty sequence;
 *     otherwise the new sequence shares every block of parent (a fork).
 *   - pa_bm_append(m, seq, n, slot_mapping, cow): appends n tokens, writing
 *     the slot (block * block_size + offset) of each to slot_mapping[n], the
 *     array pa_reshape_and_cache takes.  If the sequence's last block is
 *     partly filled and shared, it is first replaced by a fresh block
 *     (copy-on-write): cow[0] = old block, cow[1] = new block, and the caller
 *     must copy block cow[0] to cow[1] in both caches before writing the new
 *     tokens; else cow = {-1, -1}.  PA_ERR_EXHAUSTED (nothing changed) if the
 *     pool lacks blocks.
 *   - A block whose count drops to zero (pa_bm_free_sequence, or
 *     pa_bm_release_before for blocks wholly before token first_token) is
 *     parked with the caller's epoch (e.g. the step that last read it) and
 *     returns to the free list only at pa_bm_reclaim(m, completed) with
 *     epoch <= completed: a step still in flight never sees it reused.
 *   - pa_bm_block_table writes a sequence's row (released blocks and padding
 *     as -1) and returns its block count.
 * Functions returning int give a count / id >= 0 or -pa_status, except
 * pa_bm_append and pa_bm_free_sequence, which return a pa_status.  One host
 * thread per manager.
 */
typedef struct pa_block_manager pa_block_manager;
pa_block_manager* pa_bm_create(int num_blocks, int block_size);  /* NULL on bad sizes */
void pa_bm_destroy(pa_block_manager* m);
int pa_bm_num_free(const pa_block_manager* m);
int pa_bm_new_sequence(pa_block_manager* m, int parent);
int pa_bm_append(pa_block_manager* m, int seq, int num_tokens, int32_t* slot_mapping,
                 int32_t* cow);
int pa_bm_release_before(pa_block_manager* m, int seq, int first_token, uint64_t epoch);
int pa_bm_free_sequence(pa_block_manager* m, int seq, uint64_t epoch);
int pa_bm_reclaim(pa_block_manager* m, uint64_t completed_epoch);
int pa_bm_block_table(const pa_block_manager* m, int seq, int32_t* row, int max_blocks);
int pa_bm_seq_len(const pa_block_manager* m, int seq);
int pa_bm_refcount(const pa_block_manager* m, int block);

/* Human-readable name of a pa_status. */
const char* pa_status_string(int status);

/* Text of the last HIP error seen by this thread (empty if none). */
const char* pa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
