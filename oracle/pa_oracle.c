/*
 * pa_oracle.c -- plain fp64 CPU oracle for paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant with the HIP library in paged_kv_cache_267_amd/.
 *
 * What it computes is taken from these pages:
 *   [P2]  "vLLM deployment and PagedAttention" (crazysre.cn), section
 *         "Core concept: what PagedAttention solves": the KV cache is cut into
 *         fixed-size blocks; each request has a block table mapping its
 *         logical blocks to physical blocks, which need not be contiguous.
 *   [P3]  "vLLM 0.5 deep dive: PagedAttention architecture" (chenxutan.com),
 *         section 2.1 (block pool: ceil(num_tokens / block_size) blocks per
 *         request, a physical block is head_dim x block_size per layer),
 *         section 2.2 (PagedAttention.forward(query, key_cache, value_cache,
 *         block_table, seq_lens) with scale = head_dim ** -0.5), and
 *         section 2.3 (kernel sketch: per query, walk the sequence's blocks
 *         through the block table, scaled dot products, softmax with a running
 *         max and sum for stability, then the softmax-weighted sum of V).
 *   [P1]  "vLLM 0.7.2 deep dive: PagedAttention v2 with FlashAttention-3"
 *         (jsqmd.com), section 2.2 (FP8 e4m3 KV cache, grouped-query heads)
 *         and section 2.3 (a 4K sliding window: K/V outside the window are
 *         masked, and blocks wholly outside it are not loaded).
 *   [P3 s3.4] FP8 KV cache with a scale factor and zero point 0.
 *   [P3 s4.4, s5.2] prefix caching (requests reuse the cached KV of a shared
 *         prompt and compute only what follows it) and chunked prefill (a
 *         prompt enters in chunks): both attend a chunk of new query tokens
 *         to the cached keys -- ora_extend.
 *
 * Every function below is the plain definition: each output row is computed
 * on its own, in fp64, with the full (not online) softmax and sums taken in
 * ascending token / dimension order.  OpenMP only distributes independent
 * output rows over threads; it does not change any row's arithmetic.
 *
 * Readings taken where the pages are silent:
 *   - decode has one query per sequence, at position L-1; it attends to keys
 *     0..L-1 (its own K/V is already in the cache);
 *   - query head h uses KV head h / G with G = num_q_heads / num_kv_heads;
 *   - a window W > 0 keeps keys j with L-W <= j <= L-1; W = 0 means no window;
 *   - FP8 is the OCP E4M3FN format (bias 7, no infinities, S.1111.111 = NaN),
 *     dequantised as code value x per-tensor scale, zero point 0;
 *   - split partitions are aligned to logical token 0, the partition LSE is the
 *     natural-log log-sum-exp of the scaled scores, and an empty partition has
 *     LSE = -inf;
 *   - seq_len = 0 gives an all-zero output row;
 *   - extend: a sequence's n new tokens are the last n of its L keys (their
 *     K/V cached before the call), token i is at position L - n + i, and
 *     attends causally: keys 0..p, and only the last W of them when W > 0
 *     (the decode rule for the sequence cut after p); a token at a negative
 *     position (n > L) gets a zero row.
 *
 * Cache layouts (the library boundary fixes them; see include/pa.h):
 *   value_cache [num_blocks][H_kv][D][bs]           (the order printed in [P3 s2.2])
 *   key_cache   [num_blocks][H_kv][D/X][bs][X],  X = 16 / element size
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes of this oracle (the Python shim maps names to them) */
enum { ORA_F32 = 0, ORA_BF16 = 1, ORA_FP8 = 2 };

static size_t ora_elem_size(int dt) { return dt == ORA_F32 ? 4 : dt == ORA_BF16 ? 2 : 1; }

int ora_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- element decoding ---------------------------------------------------- */

/* OCP 8-bit floating point, E4M3 variant: sign, 4 exponent bits (bias 7),
   3 mantissa bits.  Exponent field 0 is subnormal (2^-6 * m/8); S.1111.111 is
   NaN; there are no infinities.  [P1 s2.2] names the format as fp8_e4m3. */
double ora_fp8_e4m3_value(uint8_t code) {
  int s = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Nearest E4M3 code to x, ties to the even mantissa code; |x| beyond the
   largest finite value (448) saturates; NaN maps to 0x7F.  Not used by the
   decode definition (inputs already hold codes); kept for the encoder pins and
   the quantising cache write. */
uint8_t ora_fp8_e4m3_encode(double x) {
  uint8_t sign;
  double a, n;
  int ex, e;
  if (isnan(x)) return 0x7F;
  sign = signbit(x) ? 0x80 : 0x00;
  a = fabs(x);
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  frexp(a, &ex);            /* a = f * 2^ex, f in [0.5, 1): a lies in binade 2^(ex-1) */
  e = ex - 1;
  if (e < -6) e = -6;       /* the subnormal range shares the quantum of binade -6 */
  n = rint(ldexp(a, 3 - e)); /* a / 2^(e-3), rounded half to even (default mode) */
  if (n >= 16.0) {          /* rounded up into the next binade */
    n = 8.0;
    e += 1;
  }
  if (n < 8.0) return sign | (uint8_t)n;            /* exponent field 0: subnormal */
  return sign | (uint8_t)(((e + 7) << 3) | ((int)n - 8));
}

/* bfloat16: the upper 16 bits of an IEEE binary32; widening is exact. */
double ora_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double ora_widen(const void* base, size_t idx, int dt) {
  if (dt == ORA_F32) {
    float f;
    memcpy(&f, (const char*)base + 4 * idx, 4);
    return (double)f;
  }
  if (dt == ORA_BF16) {
    uint16_t b;
    memcpy(&b, (const char*)base + 2 * idx, 2);
    return ora_bf16_value(b);
  }
  return ora_fp8_e4m3_value(((const uint8_t*)base)[idx]);
}

/* ---- cache addressing (element index, not bytes) ------------------------ */

static size_t ora_k_index(int dt, int Hkv, int D, int bs, int b, int h, int d, int o) {
  size_t X = 16 / ora_elem_size(dt);
  return ((((size_t)b * Hkv + h) * (D / X) + d / X) * bs + o) * X + d % X;
}

static size_t ora_v_index(int Hkv, int D, int bs, int b, int h, int d, int o) {
  return (((size_t)b * Hkv + h) * D + d) * bs + o;
}

/* ---- reshape_and_cache --------------------------------------------------- */

/* For each new token t with slot_mapping[t] >= 0, copy key[t][h][:] and
   value[t][h][:] bit for bit into block slot/bs, offset slot%bs.  Every other
   byte of both caches is left as it was.  Returns 0, or -1 if a slot lies
   outside the pool.  [P3 s2.1]: tokens live in ceil(n/bs) fixed-size blocks;
   [P2 core concept]: the block table maps logical blocks to physical ones. */
int ora_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int32_t* slot_mapping, int num_tokens, int Hkv, int D, int bs,
                          int num_blocks, int kv_dtype) {
  size_t es = ora_elem_size(kv_dtype);
  int t, h, d;
  for (t = 0; t < num_tokens; ++t) {
    int slot = slot_mapping[t];
    int b, o;
    if (slot < 0) continue;
    if ((int64_t)slot >= (int64_t)num_blocks * bs) return -1;
    b = slot / bs;
    o = slot % bs;
    for (h = 0; h < Hkv; ++h)
      for (d = 0; d < D; ++d) {
        size_t src = ((size_t)t * Hkv + h) * D + d;
        memcpy((char*)key_cache + es * ora_k_index(kv_dtype, Hkv, D, bs, b, h, d, o),
               (const char*)key + es * src, es);
        memcpy((char*)value_cache + es * ora_v_index(Hkv, D, bs, b, h, d, o),
               (const char*)value + es * src, es);
      }
  }
  return 0;
}

/*
 * Quantise-on-write: each element of the new tokens' K (V) is divided by
 * k_scale (v_scale) and stored as the nearest E4M3 code ([P3 s3.4]: a scale
 * factor and zero point 0; [P1 s2.2]: an fp8_e4m3 cache).  Reading: the
 * quotient is formed as one IEEE binary32 division of the binary32 source
 * value (the precision the code is decided in), then encoded by
 * ora_fp8_e4m3_encode (ties to even, saturating at 448, NaN -> 0x7F).
 * Returns -1 if a non-negative slot lies outside the pool.
 */
int ora_reshape_and_cache_fp8(const void* key, const void* value, int src_dtype,
                              uint8_t* key_cache, uint8_t* value_cache,
                              const int32_t* slot_mapping, int num_tokens, int Hkv, int D, int bs,
                              int num_blocks, float k_scale, float v_scale) {
  int t, h, d;
  for (t = 0; t < num_tokens; ++t) {
    int slot = slot_mapping[t];
    int b, o;
    if (slot < 0) continue;
    if ((int64_t)slot >= (int64_t)num_blocks * bs) return -1;
    b = slot / bs;
    o = slot % bs;
    for (h = 0; h < Hkv; ++h)
      for (d = 0; d < D; ++d) {
        size_t src = ((size_t)t * Hkv + h) * D + d;
        volatile float xk = (float)ora_widen(key, src, src_dtype);
        volatile float xv = (float)ora_widen(value, src, src_dtype);
        volatile float qk = xk / k_scale;   /* binary32 division */
        volatile float qv = xv / v_scale;
        key_cache[ora_k_index(ORA_FP8, Hkv, D, bs, b, h, d, o)] = ora_fp8_e4m3_encode((double)qk);
        value_cache[ora_v_index(Hkv, D, bs, b, h, d, o)] = ora_fp8_e4m3_encode((double)qv);
      }
  }
  return 0;
}

/* ---- decode -------------------------------------------------------------- */

typedef struct {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* seq_lens;
  int bs, S, Hq, Hkv, D, max_blocks, window, q_dtype, kv_dtype;
  double scale, k_scale, v_scale;
} ora_problem;

/* Softmax attention of query head h of query token row qrow (a row of the
   query array; sequence s supplies the block table) over logical keys
   [j0, j1):
   scores s_j = scale * sum_d q[d] * k_j[d]; m = max s_j; w_j = exp(s_j - m);
   Z = sum w_j; out[d] = sum_j w_j v_j[d] / Z.  Writes out[D] and returns
   m + ln Z (the natural-log LSE), or -inf for an empty range. */
static double ora_attend(const ora_problem* P, int s, int qrow, int h, int j0, int j1,
                         double* out, double* scratch /* >= j1-j0 */) {
  int G = P->Hq / P->Hkv;
  int hk = h / G;
  int n = j1 - j0, j, d;
  double m = -INFINITY, Z = 0.0;
  const int32_t* table = P->bt + (size_t)s * P->max_blocks;
  for (d = 0; d < P->D; ++d) out[d] = 0.0;
  if (n <= 0) return -INFINITY;
  for (j = j0; j < j1; ++j) {
    int b = table[j / P->bs], o = j % P->bs;
    double dot = 0.0;
    for (d = 0; d < P->D; ++d) {
      double qd = ora_widen(P->q, ((size_t)qrow * P->Hq + h) * P->D + d, P->q_dtype);
      double kd = ora_widen(P->kc, ora_k_index(P->kv_dtype, P->Hkv, P->D, P->bs, b, hk, d, o),
                            P->kv_dtype) * P->k_scale;
      dot += qd * kd;
    }
    scratch[j - j0] = P->scale * dot;
    if (scratch[j - j0] > m) m = scratch[j - j0];
  }
  for (j = 0; j < n; ++j) {
    scratch[j] = exp(scratch[j] - m);
    Z += scratch[j];
  }
  for (j = j0; j < j1; ++j) {
    int b = table[j / P->bs], o = j % P->bs;
    double w = scratch[j - j0];
    for (d = 0; d < P->D; ++d)
      out[d] += w * ora_widen(P->vc, ora_v_index(P->Hkv, P->D, P->bs, b, hk, d, o), P->kv_dtype) *
                P->v_scale;
  }
  for (d = 0; d < P->D; ++d) out[d] /= Z;
  return m + log(Z);
}

static int ora_window_lo(int L, int window) {
  if (window > 0 && L - window > 0) return L - window;
  return 0;
}

/* Decode for the listed rows (row = s * num_q_heads + h); out is [nrows][D].
   Covers [P3 s2.2/s2.3] plus the window of [P1 s2.3] and FP8 of [P1 s2.2]. */
void ora_decode(const void* q, const void* key_cache, const void* value_cache,
                const int32_t* block_tables, const int32_t* seq_lens, int block_size, float scale,
                int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                int max_blocks_per_seq, int sliding_window, int q_dtype, int kv_dtype,
                float k_scale, float v_scale, const int32_t* rows, int nrows, double* out) {
  ora_problem P = {q, key_cache, value_cache, block_tables, seq_lens, block_size, num_seqs,
                   num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sliding_window,
                   q_dtype, kv_dtype, (double)scale, (double)k_scale, (double)v_scale};
  int r;
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < nrows; ++r) {
    int s = rows[r] / num_q_heads, h = rows[r] % num_q_heads;
    int L = seq_lens[s];
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    ora_attend(&P, s, s, h, ora_window_lo(L, sliding_window), L > 0 ? L : 0,
               out + (size_t)r * head_dim, scratch);
    free(scratch);
  }
}

/* Split decode: partition p covers [p*P, (p+1)*P) intersected with the keys of
   the row.  part_out is [nrows][max_parts][D] (each partition normalised on
   its own), part_lse is [nrows][max_parts]; an empty partition gives a zero
   vector and -inf. */
void ora_decode_split(const void* q, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, const int32_t* seq_lens, int block_size,
                      float scale, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int max_blocks_per_seq, int sliding_window, int q_dtype, int kv_dtype,
                      float k_scale, float v_scale, int partition_size, int max_parts,
                      const int32_t* rows, int nrows, double* part_out, double* part_lse) {
  ora_problem P = {q, key_cache, value_cache, block_tables, seq_lens, block_size, num_seqs,
                   num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sliding_window,
                   q_dtype, kv_dtype, (double)scale, (double)k_scale, (double)v_scale};
  int r;
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < nrows; ++r) {
    int s = rows[r] / num_q_heads, h = rows[r] % num_q_heads;
    int L = seq_lens[s] > 0 ? seq_lens[s] : 0;
    int lo = ora_window_lo(L, sliding_window);
    int p;
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(partition_size));
    for (p = 0; p < max_parts; ++p) {
      int a = p * partition_size, b = a + partition_size;
      if (a < lo) a = lo;
      if (b > L) b = L;
      part_lse[(size_t)r * max_parts + p] =
          ora_attend(&P, s, s, h, a, b, part_out + ((size_t)r * max_parts + p) * head_dim,
                     scratch);
    }
    free(scratch);
  }
}

/* Extend (multi-token) attention.  Sequence s brings n_s = qsl[s+1] - qsl[s]
   new query tokens (query rows qsl[s] .. qsl[s+1]-1), which are the last n_s
   of its L = seq_lens[s] keys (their K/V already cached).  Its token i sits at
   position p = L - n_s + i and attends causally to keys 0..p, within its own
   window (keys p-W+1..p) when W > 0: the decode rule applied to the sequence
   cut after position p.  query and out are [num_tokens][num_q_heads][D]; rows
   lists qrow * num_q_heads + h.  A token at a negative position (n_s > L)
   gets a zero row. */
void ora_extend(const void* q, const void* key_cache, const void* value_cache,
                const int32_t* block_tables, const int32_t* seq_lens,
                const int32_t* query_start_loc, int block_size, float scale, int num_seqs,
                int num_q_heads, int num_kv_heads, int head_dim, int max_blocks_per_seq,
                int sliding_window, int q_dtype, int kv_dtype, float k_scale, float v_scale,
                const int32_t* rows, int nrows, double* out) {
  ora_problem P = {q, key_cache, value_cache, block_tables, seq_lens, block_size, num_seqs,
                   num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sliding_window,
                   q_dtype, kv_dtype, (double)scale, (double)k_scale, (double)v_scale};
  int r;
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < nrows; ++r) {
    int h = rows[r] % num_q_heads;
    int qrow = rows[r] / num_q_heads;
    int s = 0, Lp;
    double* scratch;
    while (s + 1 < num_seqs && query_start_loc[s + 1] <= qrow) ++s;
    /* keys 0 .. position of this token */
    Lp = seq_lens[s] - (query_start_loc[s + 1] - query_start_loc[s]) + (qrow - query_start_loc[s]) + 1;
    scratch = (double*)malloc(sizeof(double) * (size_t)(Lp > 0 ? Lp : 1));
    ora_attend(&P, s, qrow, h, ora_window_lo(Lp, sliding_window), Lp > 0 ? Lp : 0,
               out + (size_t)r * head_dim, scratch);
    free(scratch);
  }
}

/* Merge partitions: M = max_p lse_p; out = sum_p e^(lse_p - M) o_p / sum_p e^(lse_p - M),
   over the partitions with lse_p > -inf.  No partition -> zero row. */
void ora_reduce_lse(const double* part_out, const double* part_lse, int nrows, int head_dim,
                    int max_parts, double* out) {
  int r;
  for (r = 0; r < nrows; ++r) {
    const double* lse = part_lse + (size_t)r * max_parts;
    double M = -INFINITY, W = 0.0;
    int p, d;
    double* o = out + (size_t)r * head_dim;
    for (d = 0; d < head_dim; ++d) o[d] = 0.0;
    for (p = 0; p < max_parts; ++p)
      if (lse[p] > M) M = lse[p];
    if (M == -INFINITY) continue;
    for (p = 0; p < max_parts; ++p) {
      double w;
      if (lse[p] == -INFINITY) continue;
      w = exp(lse[p] - M);
      W += w;
      for (d = 0; d < head_dim; ++d)
        o[d] += w * part_out[((size_t)r * max_parts + p) * head_dim + d];
    }
    for (d = 0; d < head_dim; ++d) o[d] /= W;
  }
}
