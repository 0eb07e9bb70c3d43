/*
 * paged_attn.h - C ABI of the MI355X (gfx950) attention-over-paged-KV library.
 *
 * Four calls make up the hot path of attention over a paged KV cache:
 *   paged_kv_write          scatter new K/V rows into fixed-size physical blocks
 *   paged_attention_decode  one query token per sequence against its paged history
 *   paged_attention_reduce  log-sum-exp merge of split-KV partitions
 *   varlen_causal_prefill   causal attention of sequences packed by cu_seqlens
 * and a fifth extends prefill to a cached prefix:
 *   paged_prefill           a chunk of query rows against its sequence's paged cache
 * The four attention calls also come in *_window forms (sliding window), the cache
 * write and decode in *_fp8 forms over an FP8 (E4M3) cache, and the cache write in a
 * *_rope form that applies rotary position embedding to q and k in the same pass.
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *   library allocates and frees nothing, never synchronises, and never reads
 *   device memory from the host.  Every call is asynchronous on `stream` (a
 *   hipStream_t; NULL means the default stream) and returns as soon as its
 *   kernels are enqueued.
 * Layouts (all row-major, densely packed, no strides):
 *   KV pool           k_cache, v_cache : [num_blocks, num_kv_heads, block_size, head_dim]
 *                     one contiguous block_size x head_dim slab per (block, KV head)
 *   block_tables      int32 [num_seqs, max_blocks_per_seq]; entry j is the physical
 *                     block holding positions j*block_size .. (j+1)*block_size-1;
 *                     unused entries hold -1
 *   context_lens      int32 [num_seqs]; the number of cached positions a sequence's
 *                     query attends to, the position just written included
 *   slot_mapping      int32 [num_tokens]; slot = block * block_size + offset; < 0 skips
 *   cu_seqlens        int32 [num_seqs + 1]; cu_seqlens[0] = 0, non-decreasing
 * Element types.  PA_F32 = IEEE float32; PA_BF16 = bfloat16 (raw 16-bit patterns).
 *   q / k / v / out / caches use the call's dtype; lse and partial results are
 *   always float32.  Outputs in bf16 are rounded to nearest-even from float32.
 * GQA.  Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * Softmax statistics.  lse = natural log of the sum of exp(scale * q.k) over the
 *   keys a query sees; a query that sees no key gets out = 0 and lse = -inf.
 * Device-resident contents are preconditions the host cannot check without a
 *   sync: block ids in [0, num_blocks), unique slots below num_blocks*block_size,
 *   context_lens <= max_context_len, cu_seqlens within [0, total_tokens].  The
 *   kernels never access memory outside the buffers whatever these hold: a slot
 *   or block id out of range is skipped, a context length is clamped, and the
 *   result for such inputs is unspecified (but finite-time and fault-free).
 * Errors.  Each call returns PA_OK (0) or a PA_ERR_* code and then leaves a
 *   message for pa_last_error().  Host-side validation happens before any
 *   launch, so an error return means nothing was enqueued (PA_ERR_LAUNCH aside).
 *   Nothing throws or aborts across the ABI.
 *
 * Sources for the operations: the pages "Llama 4 inference doubling
 * (FlashAttention-3 + PagedAttention + vLLM)" (section 2.4: varlen call with
 * cu_seqlens, causal, returning out and lse; section 3.1: logical pages mapped
 * to physical blocks through an int32 table, -1 = unallocated; section 3.2:
 * 16-token blocks, power of two), "LLM inference optimisation: KV cache to
 * FlashAttention" (section 3.1: block table lookup then in-place update of
 * preallocated KV blocks), "PageAttention + FlashAttention golden combination"
 * (section 2.1: fixed-size blocks anywhere in memory, shared prompt blocks) and
 * "LLaMA inference performance: structure and source" (section 2.1: GQA groups;
 * section 3.1: scores, mask, softmax, weighted sum).
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent arguments */
  PA_ERR_UNSUPPORTED = 2, /* valid but no kernel for this dtype/head_dim/block_size */
  PA_ERR_LAUNCH = 3       /* the HIP runtime rejected a launch */
};

/* Version of this ABI (bumped on any signature or semantic change). */
int pa_abi_version(void);

/* Identity of the sources this library was built from: the first 16 hex digits
 * of a SHA-256 over the library's HIP sources and headers (file name, then
 * bytes, in name order), baked in at build time; "unknown" if the build did
 * not supply it.  The string is static; the caller must not free it. */
const char* pa_build_id(void);

/* Process-wide options.  PA_OPT_FORCE_VECTOR_PATH (value 0/1): run decode and
 * prefill on their vector-ALU kernels even where an MFMA kernel exists (both
 * compute the same result; used to cross-check one kernel against the other).
 * Returns PA_OK or PA_ERR_INVALID_ARG for an unknown option.  Not thread-safe
 * against concurrent calls. */
enum { PA_OPT_FORCE_VECTOR_PATH = 1 };
int pa_set_option(int option, int value);

/* Message describing the last error returned on the calling thread ("" if none).
 * The pointer stays valid until the next library call on that thread. */
const char* pa_last_error(void);

/*
 * paged_kv_write - write new tokens' K and V rows into the paged pools.
 *
 * For each t < num_tokens with s = slot_mapping[t] >= 0, and every KV head h:
 *   k_cache[s / block_size, h, s % block_size, :] = k[t, h, :]
 *   v_cache[s / block_size, h, s % block_size, :] = v[t, h, :]
 * A bit-exact copy; every other byte of the pools is left untouched.  This is
 * the in-place update through the block table that replaces re-allocating a
 * contiguous cache on every appended token.
 *   k, v          [num_tokens, num_kv_heads, head_dim], dtype
 *   k_cache, v_cache  pools as above, dtype; updated in place
 *   slot_mapping  int32 [num_tokens]; slots must be unique; s < 0 skips token t;
 *                 s >= num_blocks * block_size is skipped (precondition violation)
 * num_tokens = 0 is a no-op.  Supported: head_dim * sizeof(dtype) a multiple of 16.
 */
int paged_kv_write(const void* k, const void* v, void* k_cache, void* v_cache,
                   const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                   int head_dim, int block_size, int num_blocks, pa_dtype dtype,
                   void* stream);

/*
 * paged_attention_decode - attention of one query token per sequence over its
 * paged history (PagedAttention decode), with GQA and online softmax.
 *
 * For sequence b and query head h (KV head g = h / G), over positions
 * p < ctx = context_lens[b], each fetched from block block_tables[b][p / block_size]
 * at offset p % block_size:
 *   out[b, h, :] = sum_p softmax_p(scale * q[b,h,:] . K[p,g,:]) V[p,g,:]
 *   lse[b, h]    = log sum_p exp(scale * q[b,h,:] . K[p,g,:])
 * partition_size == 0: one pass per (sequence, KV head); writes out ([B, H_q, d],
 *   dtype) and lse ([B, H_q], float32).  part_out/part_lse are not touched.
 * partition_size > 0 (split-KV): positions are cut into partitions
 *   [i*partition_size, (i+1)*partition_size); for every partition i that holds at
 *   least one position (i*partition_size < ctx) the call writes the attention over
 *   that partition alone to part_out[b, h, i, :] (float32) and part_lse[b, h, i]
 *   (float32).  Partitions past the end are not written.  out/lse are not touched;
 *   paged_attention_reduce merges the partitions.  partition_size must be a
 *   multiple of block_size.  The partition dimension of part_out/part_lse is
 *   max_partitions = ceil(max_context_len / partition_size).
 *   Sequences whose block ids agree over a whole partition (blocks of a shared
 *   prompt) may be computed in one work unit; their results are the same up to
 *   rounding, and identical for any permutation of the pool's blocks.
 *   q             [B, H_q, head_dim], dtype
 *   block_tables  int32 [B, max_blocks_per_seq]
 *   context_lens  int32 [B]; each <= max_context_len
 *   max_context_len  host-side upper bound on context_lens (sizes the grid);
 *                 must be <= max_blocks_per_seq * block_size
 *   scale         multiplies q.k (typically 1/sqrt(head_dim))
 * Supported: dtype f32 or bf16; head_dim 64 or 128; block_size 8, 16, 32 or 64;
 *   H_q / H_kv in {1, 2, 4, 8}; num_seqs <= 65535.
 */
int paged_attention_decode(void* out, float* lse, float* part_out, float* part_lse,
                           const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int max_blocks_per_seq, int num_blocks,
                           int partition_size, int max_context_len, float scale,
                           pa_dtype dtype, void* stream);

/*
 * paged_attention_reduce - merge split-KV partitions by log-sum-exp.
 *
 * For sequence b, head h, the live partitions are i < n = ceil(ctx / partition_size)
 * (ctx = context_lens[b], n capped at max_partitions).  With M = max_i part_lse[b,h,i]
 * and w_i = exp(part_lse[b,h,i] - M):
 *   out[b, h, :] = sum_i w_i part_out[b,h,i,:] / sum_i w_i     (dtype)
 *   lse[b, h]    = M + log(sum_i w_i)                          (float32)
 * Partitions at or past n are never read; a sequence with ctx = 0 gets out = 0 and
 * lse = -inf.  part_out [B, H_q, max_partitions, head_dim] and
 * part_lse [B, H_q, max_partitions] are float32, as written by
 * paged_attention_decode with the same partition_size.
 */
int paged_attention_reduce(void* out, float* lse, const float* part_out,
                           const float* part_lse, const int32_t* context_lens,
                           int num_seqs, int num_q_heads, int head_dim,
                           int partition_size, int max_partitions, pa_dtype dtype,
                           void* stream);

/*
 * varlen_causal_prefill - causal self-attention of sequences packed back to back.
 *
 * Sequence s owns tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of q, k and v.  Row i
 * of sequence s (token t = cu_seqlens[s] + i) and query head h attend to the keys
 * of tokens cu_seqlens[s] .. t (same sequence, causal, the token itself included)
 * of KV head h / G:
 *   out[t, h, :] = sum_j softmax_j(scale * q[t,h,:] . k[j,g,:]) v[j,g,:]
 *   lse[t, h]    = log sum_j exp(scale * q[t,h,:] . k[j,g,:])
 *   q, out        [total_tokens, H_q, head_dim], dtype
 *   k, v          [total_tokens, H_kv, head_dim], dtype
 *   lse           float32 [total_tokens, H_q]
 *   cu_seqlens    int32 [num_seqs + 1]
 *   max_seqlen    host-side upper bound on any sequence length (sizes the grid);
 *                 rows of a longer sequence beyond max_seqlen are not computed
 * Tokens not covered by any sequence are not written.  The K/V are read from the
 * packed arrays, not from a paged pool; writing them into a pool is a separate
 * paged_kv_write call.
 * Supported: dtype bf16, head_dim 128 (MFMA path); dtype f32 or bf16 with
 *   head_dim 64 or 128 (vector path); H_q / H_kv in {1, 2, 4, 8}; num_seqs <= 65535.
 *   max_seqlen must not exceed total_tokens.
 */
int varlen_causal_prefill(void* out, float* lse, const void* q, const void* k,
                          const void* v, const int32_t* cu_seqlens, int num_seqs,
                          int total_tokens, int max_seqlen, int num_q_heads,
                          int num_kv_heads, int head_dim, float scale, pa_dtype dtype,
                          void* stream);

/*
 * paged_prefill - a chunk of new query rows per sequence against its paged cache.
 *
 * The varlen call of "Llama 4 inference doubling (FlashAttention-3 + PagedAttention +
 * vLLM)" takes separate cumulative lengths for queries and keys (section 2.4), and the
 * engine reuses cached KV of earlier requests (prefix caching, section 4.2).  Here the
 * keys of sequence s are its first ctx = context_lens[s] cached positions, read through
 * its block table as in paged_attention_decode, and its Lq = cu_seqlens_q[s+1] -
 * cu_seqlens_q[s] query rows are the LAST Lq of those positions (their own K/V already
 * written, e.g. by paged_kv_write): row i (token t = cu_seqlens_q[s] + i) sits at
 * position ctx - Lq + i and attends, for query head h, to positions 0 .. ctx - Lq + i
 * of KV head h / G (the causal mask aligned to the end of the cache).  With ctx = Lq
 * this is varlen_causal_prefill over the pool; with Lq = 1 it is a decode.
 *   out[t, h, :], lse[t, h] as in varlen_causal_prefill
 *   q, out        [total_q, H_q, head_dim], dtype; lse float32 [total_q, H_q]
 *   k_cache, v_cache, block_tables, block_size, max_blocks_per_seq, num_blocks,
 *                 max_context_len: as in paged_attention_decode
 *   cu_seqlens_q  int32 [num_seqs + 1], within [0, total_q]
 *   context_lens  int32 [num_seqs]; must be >= the sequence's query rows (a sequence
 *                 violating this has its rows left unwritten)
 *   max_seqlen_q  host-side upper bound on any sequence's query rows (sizes the grid)
 * Query rows not covered by any sequence are not written.
 * Supported: dtype bf16, head_dim 128 (MFMA path); dtype f32 or bf16 with head_dim 64
 *   or 128 (vector path); block_size 8, 16, 32 or 64; H_q / H_kv in {1, 2, 4, 8};
 *   num_seqs <= 65535; max_seqlen_q <= total_q.
 */
int paged_prefill(void* out, float* lse, const void* q, const void* k_cache,
                  const void* v_cache, const int32_t* block_tables,
                  const int32_t* cu_seqlens_q, const int32_t* context_lens, int num_seqs,
                  int total_q, int max_seqlen_q, int num_q_heads, int num_kv_heads,
                  int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                  int max_context_len, float scale, pa_dtype dtype, void* stream);

/*
 * Sliding-window variants.  Identical to paged_attention_decode, varlen_causal_prefill
 * and paged_prefill (which are these with window = 0), except that a query at position
 * p attends only to positions max(0, p - window + 1) .. p: the last `window` keys, the
 * mask that "PageAttention + FlashAttention golden combination" (section 4.1) builds.
 * window = 0 means no window; window < 0 is PA_ERR_INVALID_ARG.
 * Blocks wholly before the window are not read, nor are their block-table entries
 * used: for a sequence of ctx cached positions, entries of blocks that end at or before
 * position ctx - window (decode) or ctx - Lq - window + 1 (paged prefill, the first
 * row's window) may hold anything, so a caller may free those blocks.
 * Split decode (partition_size > 0) computes only the partitions that hold a visible
 * key, lo / P .. ceil(ctx / P) - 1 with lo = max(0, ctx - window); the partitions before
 * them are left unwritten.  Merge with paged_attention_reduce_window and the same
 * window, which starts at partition lo / P.
 */
int paged_attention_decode_window(void* out, float* lse, float* part_out, float* part_lse,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_blocks_per_seq, int num_blocks,
                                  int partition_size, int max_context_len, float scale,
                                  int window, pa_dtype dtype, void* stream);

int varlen_causal_prefill_window(void* out, float* lse, const void* q, const void* k,
                                 const void* v, const int32_t* cu_seqlens, int num_seqs,
                                 int total_tokens, int max_seqlen, int num_q_heads,
                                 int num_kv_heads, int head_dim, float scale, int window,
                                 pa_dtype dtype, void* stream);

int paged_attention_reduce_window(void* out, float* lse, const float* part_out,
                                  const float* part_lse, const int32_t* context_lens,
                                  int num_seqs, int num_q_heads, int head_dim,
                                  int partition_size, int max_partitions, int window,
                                  pa_dtype dtype, void* stream);

int paged_prefill_window(void* out, float* lse, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         const int32_t* cu_seqlens_q, const int32_t* context_lens, int num_seqs,
                         int total_q, int max_seqlen_q, int num_q_heads, int num_kv_heads,
                         int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                         int max_context_len, float scale, int window, pa_dtype dtype,
                         void* stream);

/*
 * FP8 KV cache.  "Llama 4 inference doubling (FlashAttention-3 + PagedAttention + vLLM)"
 * turns on KV-cache quantisation (section 3.2) and pairs GQA with FP8 under dynamic
 * scaling (chapter 1) without fixing the format; here the pools hold OCP FP8 E4M3
 * codes (uint8: sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals,
 * S.1111.111 = NaN, largest finite 448), one fp32 scale per pool, value = code * scale.
 * Pools are [num_blocks, num_kv_heads, block_size, head_dim] bytes.
 *
 * paged_kv_write_fp8 - paged_kv_write into E4M3 pools.  For each token with a slot,
 *   every element x of k (v) becomes the E4M3 code nearest to the IEEE fp32 quotient
 *   x / *k_scale (x / *v_scale), ties to the even code; quotients of magnitude 448 or
 *   more become +-448 (saturation); NaN becomes 0x7F.  bf16 inputs are widened
 *   exactly first.  k_scale and v_scale point to one float each in DEVICE memory
 *   (so a scale computed on the GPU needs no host round trip); a zero, negative or
 *   non-finite scale gives unspecified codes.  k, v: [num_tokens, H_kv, head_dim],
 *   dtype f32 or bf16.  Supported: head_dim a multiple of 16.  Other arguments and
 *   errors as paged_kv_write.
 *
 * paged_attention_decode_fp8 - paged_attention_decode_window over E4M3 pools: the
 *   attention of the dequantised K and V (code * scale), computed with bf16 matrix
 *   products on the exact bf16 image of each code (every E4M3 value is a bf16 value),
 *   the K scale folded into `scale` and the V scale into the output.  q, out, lse,
 *   part_out, part_lse, window and the split-KV contract as in
 *   paged_attention_decode_window; merge split results with
 *   paged_attention_reduce_window.  Supported: dtype bf16 (queries and output),
 *   head_dim 128, block_size 16, 32 or 64, H_q / H_kv in {1, 2, 4, 8}; anything else
 *   is PA_ERR_UNSUPPORTED.
 */
int paged_kv_write_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                       const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                       int head_dim, int block_size, int num_blocks, const float* k_scale,
                       const float* v_scale, pa_dtype dtype, void* stream);

int paged_attention_decode_fp8(void* out, float* lse, float* part_out, float* part_lse,
                               const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq, int num_blocks,
                               int partition_size, int max_context_len, float scale,
                               const float* k_scale, const float* v_scale, int window,
                               pa_dtype dtype, void* stream);

/*
 * Decode with the step's cache write folded in.  A decode step writes each sequence's
 * new token (paged_kv_write) and then attends over the cache including it; only the
 * work unit that reads position ctx - 1 needs that row, so it stores it itself and waits
 * for the stores before reading the block: one launch instead of two.
 *
 * paged_attention_decode_append - paged_attention_decode_window, except that k_new and
 *   v_new ([num_seqs, num_kv_heads, head_dim], dtype) hold the K and V of the token at
 *   position ctx - 1 of each sequence (ctx = context_lens[b]), which the call stores into
 *   the pools at block block_tables[b][(ctx-1) / block_size], offset (ctx-1) % block_size
 *   (exactly what paged_kv_write with that slot stores), before the attention reads it.
 *   A sequence with ctx = 0 stores nothing; an out-of-range block id stores nothing.
 *   The pools are written, so k_cache and v_cache are not const here.  Other arguments,
 *   supported shapes and errors as paged_attention_decode_window.
 *
 * paged_attention_decode_append_fp8 - the same over E4M3 pools: the new rows are
 *   quantised as paged_kv_write_fp8 quantises them (k_scale, v_scale), then the
 *   attention is paged_attention_decode_fp8's.
 */
int paged_attention_decode_append(void* out, float* lse, float* part_out, float* part_lse,
                                  const void* q, const void* k_new, const void* v_new, void* k_cache,
                                  void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int num_blocks, int partition_size,
                                  int max_context_len, float scale, int window, pa_dtype dtype,
                                  void* stream);

int paged_attention_decode_append_fp8(void* out, float* lse, float* part_out, float* part_lse,
                                      const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_dim, int block_size,
                                      int max_blocks_per_seq, int num_blocks, int partition_size,
                                      int max_context_len, float scale, const float* k_scale,
                                      const float* v_scale, int window, pa_dtype dtype,
                                      void* stream);

/*
 * Rotary position embedding fused into the cache write.  "LLaMA inference performance:
 * structure and source" (section 2.2, and step 1 of its attention listing) turns each
 * query and key vector by a position-dependent rotation computed from sin and cos, with
 * the table of those values worth precomputing; the pairing and frequencies are not
 * printed.  Here dims i and i + rot_dim/2 (i < rot_dim/2) of the first rot_dim dims of a
 * head form a pair, turned at position p by the angle p * base^(-2i/rot_dim):
 *   y_i = x_i cos - x_{i+rot_dim/2} sin,   y_{i+rot_dim/2} = x_{i+rot_dim/2} cos + x_i sin.
 *
 * rope_cos_sin_cache - fill the table cos_sin [max_positions, rot_dim] (float32, device):
 *   row p holds cos(p theta_i) for i < rot_dim/2, then sin(p theta_i); angles, cos and sin
 *   are evaluated in double precision and rounded once to float.  rot_dim even and
 *   positive; base finite and > 1 (10000 for LLaMA).
 *
 * paged_kv_write_rope - one pass over a step's rows: q [num_tokens, H_q, head_dim] and
 *   k [num_tokens, H_kv, head_dim] are rotated IN PLACE (token t at position positions[t],
 *   int32, read from cos_sin row positions[t]; arithmetic in float32, results rounded to
 *   dtype, nearest even), and the rotated k and the unrotated v are written into the
 *   pools exactly as paged_kv_write does (slot_mapping; s < 0 rotates q and k but writes
 *   nothing).  Dims past rot_dim pass through.  Positions outside [0, max_positions) give
 *   unspecified values (no access outside the table).  q, k, v must not overlap.
 *   Supported: dtype f32 or bf16 with head_dim * sizeof(dtype) and rot_dim/2 * sizeof(dtype)
 *   multiples of 16 bytes; rot_dim <= head_dim.
 */
int rope_cos_sin_cache(float* cos_sin, int max_positions, int rot_dim, double base, void* stream);

int paged_kv_write_rope(void* q, void* k, const void* v, void* k_cache, void* v_cache,
                        const int32_t* slot_mapping, const int32_t* positions, const float* cos_sin,
                        int num_tokens, int num_q_heads, int num_kv_heads, int head_dim, int rot_dim,
                        int block_size, int num_blocks, int max_positions, pa_dtype dtype, void* stream);

/*
 * paged_attention_decode_noalloc - split-KV decode and its merge in one call
 * that allocates nothing, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).
 *
 * Computes exactly what paged_attention_decode_window with this partition_size
 * followed by paged_attention_reduce_window computes (the same kernels), and
 * writes out [B, H_q, d] (dtype) and lse [B, H_q] (float32).  The split
 * partials do not come from the caller: they live in a scratch array inside
 * the library, one per GPU, allocated with the library's code on that GPU and
 * held until the process ends.  Limit: num_seqs * num_q_heads * P *
 * (head_dim + 1) * 4 bytes (P = ceil(max_context_len / partition_size), the
 * partials rounded up to 256 bytes) must fit in 32 MiB - e.g. 64 sequences x
 * 32 heads x 8 partitions (8.5 MB) or 4 x 32 x 256 (16.9 MB) at head_dim 128;
 * a larger call returns PA_ERR_INVALID_ARG and launches nothing.
 * partition_size must be > 0 (a multiple of block_size).
 * Every call on one GPU uses that GPU's one scratch array: calls that overlap
 * on one GPU (on different streams, or from several threads without ordering)
 * race and give undefined results.  The scratch needs no clearing: each call
 * writes every partition it later reads.  Nothing is allocated or freed by
 * the call itself; the first call on a device looks up that device's scratch
 * address (hipGetSymbolAddress) and keeps it.
 */
int paged_attention_decode_noalloc(void* out, float* lse, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                                   int num_blocks, int partition_size, int max_context_len, float scale,
                                   int window, pa_dtype dtype, void* stream);

/*
 * paged_kv_stream_read - a measurement call, not a step of the method: the
 * bandwidth ceiling of the split-KV decode's memory access pattern.
 *
 * It walks the work units paged_attention_decode walks with this
 * partition_size (KV head g, sequence b, partition i; the same balanced order)
 * and reads every K and V row of positions [i*partition_size,
 * min((i+1)*partition_size, ctx)) through the block table, in the same
 * 16-position tiles of one (block, KV head) slab, doing no attention.  So that
 * every fetched byte is used and the result can be checked, it writes
 *   checksums[b, g, i] = XOR of every 32-bit word of those K rows and V rows
 *                        of KV head g (uint32 [num_seqs, num_kv_heads, P],
 *                        P = ceil(max_context_len / partition_size));
 * partitions past the end of a sequence are not written.
 *   mode PA_STREAM_LDS_DMA:   tiles reach LDS by LDS-DMA (as in the decode
 *                             kernel) through a ring of `depth` slots (2, 3 or
 *                             4): depth - 1 tiles in flight per wave;
 *   mode PA_STREAM_REGISTERS: 16-byte loads into registers, `depth` tiles (1,
 *                             2 or 4) issued together.
 * Other arguments as for paged_attention_decode.  Supported: PA_BF16, head_dim
 * 128, block_size 16, 32 or 64.  Returns PA_ERR_UNSUPPORTED for an unsupported
 * depth.
 */
enum { PA_STREAM_LDS_DMA = 0, PA_STREAM_REGISTERS = 1 };
int paged_kv_stream_read(uint32_t* checksums, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                         int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                         int num_blocks, int partition_size, int max_context_len, int mode, int depth,
                         pa_dtype dtype, void* stream);

/*
 * pa_stream_read_contiguous - a measurement call, not a step of the method: the
 * plain read ceiling that paged_kv_stream_read's pattern is compared with.
 *
 * Reads bytes bytes of src front to back in 16-byte non-temporal loads, with no
 * table and no tiles.  With n = bytes / 16 and cpw = ceil(n / waves), wave w
 * (one per workgroup) reads the 16-byte chunks [w * cpw, min((w + 1) * cpw, n)),
 * `depth` loads in flight per lane (1, 2, 4 or 8; else PA_ERR_UNSUPPORTED), and
 * writes checksums[w] = XOR of every 32-bit word of its chunks (0 for a wave with
 * none), so every fetched byte is used and the result can be checked.
 *   src        device buffer, 16-byte aligned
 *   checksums  uint32 [waves], device
 * bytes must be a multiple of 16 and waves > 0 (else PA_ERR_INVALID_ARG);
 * bytes = 0 launches nothing and leaves checksums untouched.
 */
int pa_stream_read_contiguous(uint32_t* checksums, const void* src, uint64_t bytes, int waves,
                              int depth, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
