/*
 * kvq.h -- C ABI of libkvq.so: quantizing KV-cache writes and paged decode
 * attention over INT8 / FP8 / FP16 block pools, for AMD MI355X (gfx950).
 *
 * What the calls compute (web pages, cited by title and section):
 *   "KV Cache优化实战：大模型推理显存占用与加速方案详解" (0539edu.com)
 *     s1.1  each decode step computes only the new token's K/V, appends it to
 *           the end of the cache, and attends with the current query over all
 *           cached K/V.
 *     s2.1  GQA: the query heads are split into groups; each group shares one
 *           KV head (query head g reads KV head g / (Hq / Hkv)).
 *     s2.2  paged cache: fixed-size physical blocks, a per-sequence block table
 *           mapping logical blocks to physical ones anywhere in the pool.
 *     s2.3  INT8 absmax symmetric quantization storing a scale, dequantized at
 *           run time; per-channel scales; per-group scales (e.g. 128
 *           elements per group); FP8.
 *     s3.3  per_channel / per_group / per_token granularity, group size 128
 *           or 64.
 *     s4.3  dequantization fused into the attention kernel instead of separate
 *           small kernels.
 *   xpshop.cn article 312, s3: 16- or 32-token blocks; FP8 KV cache
 *     (kv_cache_dtype "fp8_e5m2").
 *
 * Conventions shared by every call
 *  - All buffers are device memory owned by the caller; the library never
 *    allocates, frees or keeps pointers.  Calls are asynchronous on `stream`
 *    (a hipStream_t; NULL = the legacy default stream) and never synchronize.
 *  - The library never prints, aborts or falls back to another format or a
 *    slower path: unsupported combinations return KVQ_ERR_UNSUPPORTED.
 *  - The synchronous return value covers host-side argument checks and launch
 *    errors.  Device contents (block ids, slots, lengths) are trusted, except
 *    that cache writes skip slots outside the pool.
 *  - Supported: head_dim 64 or 128; block_size 16 or 32; Hq / Hkv between 1
 *    and 16; gfx950 only.  Scale granularity by dtype and group_size:
 *      KVQ_INT8      group_size 64 / 128 (<= head_dim): per-group scales
 *                    computed by the cache write (per token when group_size
 *                    = head_dim); group_size 0: static per-channel scales.
 *      KVQ_FP8_E4M3  group_size 0: static per-KV-head scales; 64 / 128:
 *                    per-group scales computed by the cache write.
 *      KVQ_FP8_E5M2  group_size 0 only: static per-KV-head scales.
 *      KVQ_INT4      head_dim 128 only; group_size 64 / 128: per-group
 *                    scales computed by the cache write (s = absmax / 7).
 *      KVQ_FP16      group_size ignored, no scales.
 *  - Pointers to q, out, pools, scales and workspace must be 16-byte aligned.
 *
 * Pool layout (one layer; the caller keeps one set of pools per layer):
 *   k_pool, v_pool  [num_blocks][Hkv][tile], one tile of block_size * head_dim
 *   elements (EB bytes each: INT8 = codes in excess-128 form, byte = code +
 *   128, and FP8 = E4M3 / E5M2 bytes, EB = 1; FP16 = IEEE half, EB = 2) per
 *   (block, KV head).  Inside a tile, element
 *   (token t, dim d) sits at byte
 *     K:  ((d*EB/64) * block_size + t) * 64 + (d*EB) % 64
 *         (rows of 64 bytes: 64 one-byte dims or 32 fp16 dims of one token)
 *     V:  ((((t/16) * EB + e) * (head_dim/4) + d/4) * 4 + (t%16)/4) * 16
 *           + ((d%4) % (4/EB)) * 4 * EB + (t%4) * EB,   e = (d%4) / (4/EB)
 *         (16-byte micro-tiles of 4 tokens x 4/EB dims, grouped per 16-token
 *         half of a block).
 *   These orders let every 16-byte load of the decode kernel cover, across a
 *   wavefront, one contiguous KiB of whole cache lines.
 *   INT4 (head_dim 128): codes in excess-8 form (nibble = code + 8), tiles of
 *   block_size * 64 bytes.  Element (t, d) sits in the byte
 *     K:  t * 64 + 16 * ((d%64)/16) + 4 * (2*(d/64) + (d%16)/8) + d%4,
 *         high nibble if d%8 >= 4 (a dword holds 8 dims of one token),
 *     V:  (t/16) * 1024 + ((((d%64)/4) * 4 + (t%16)/4) * 4 + 2*(d/64)
 *           + (d%4)/2) * 4 + t%4,  high nibble if d is odd (a byte holds
 *         two dims of one token, so writes of different tokens never share
 *         a byte).
 *   Per-group scales (INT8, INT4 or E4M3, group_size G > 0): k_scale, v_scale
 *   [num_blocks][Hkv][block_size][head_dim/G] fp32, one per (token slot,
 *   group of G consecutive head_dim elements), written by the cache write.
 *   Static per-channel scales (INT8, group_size 0): k_scale, v_scale
 *   [Hkv][head_dim] fp32, read only.
 *   Static per-head scales (FP8, group_size 0): k_scale, v_scale [Hkv] fp32,
 *   read only.
 *   FP16: no scales (pass NULL).
 *   A slot is block * block_size + offset.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_API __attribute__((visibility("default")))

/* KV element formats (per layer). */
enum {
    KVQ_FP16 = 0,
    KVQ_INT8 = 1,      /* symmetric, |code| <= 127, per-group or per-channel */
    KVQ_FP8_E4M3 = 2,  /* OCP E4M3FN (max 448), per-head or per-group       */
    KVQ_FP8_E5M2 = 3,  /* OCP E5M2 (max 57344), per-head                    */
    KVQ_INT4 = 4       /* symmetric, |code| <= 7, two per byte, per-group   */
};

/* How kvq_paged_prefill cuts the work (its split_mode argument). */
enum {
    KVQ_PREFILL_AUTO = 0,
    KVQ_PREFILL_WALK = 1,   /* a wavefront per (sequence, KV head, token groups) */
    KVQ_PREFILL_SPLIT = 2   /* the decode partition over every wavefront         */
};

typedef int32_t kvq_status;
enum {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = -1,
    KVQ_ERR_UNSUPPORTED = -2,
    KVQ_ERR_WORKSPACE = -3,
    KVQ_ERR_HIP = -4
};

/* Human-readable name of a status code (static string, never NULL). */
KVQ_API const char *kvq_status_string(kvq_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
KVQ_API int32_t kvq_version(void);

/*
 * kvq_cache_write -- quantize the K/V of new tokens and store them in their
 * slots ("KV Cache优化实战" s1.1 append, s2.2 block placement, s2.3 / s3.3
 * per-group absmax quantization; xpshop.cn article 312 s3 FP8).
 *
 *   k, v          fp16 [num_tokens][num_kv_heads][head_dim], contiguous.
 *   slot_mapping  int64 [num_tokens]: slot of each token; a negative slot, or
 *                 one >= num_blocks * block_size, skips the token.
 *   dtype, group_size (see "Scale granularity" above):
 *                 KVQ_INT8, group_size G > 0: for each (token, head, group of
 *                   G elements): a = max |x|; s = fl32(a / 127);
 *                   code = clamp(round_half_even(fl32(x / s)), -127, 127);
 *                   a == 0 stores s = 0 and zero codes.  Codes go to the
 *                   pools as bytes code + 128, s to k_scale / v_scale
 *                   (written).
 *                 KVQ_INT8, group_size 0: code = clamp(round_half_even(
 *                   fl32(x / S[h][d])), -127, 127) with the static channel
 *                   scales S = k_scale / v_scale [num_kv_heads][head_dim]
 *                   (read only); S == 0 gives code 0.
 *                 KVQ_FP8_E4M3 / KVQ_FP8_E5M2, group_size 0: code =
 *                   FP8(fl32(x / S[h])) rounding to nearest-even and
 *                   saturating to the largest finite value (448 / 57344);
 *                   S = k_scale / v_scale [num_kv_heads] (read only);
 *                   S == 0 gives code 0.
 *                 KVQ_FP8_E4M3, group_size G > 0: per group, s = fl32(a /
 *                   448), code = E4M3(fl32(x / s)) (a == 0: s = 0, codes 0);
 *                   s written to k_scale / v_scale like INT8.
 *                 KVQ_INT4: the INT8 rule with 7 in place of 127; codes go
 *                   to the pools as nibbles code + 8.
 *                 KVQ_FP16: the values are copied.
 * Tokens are independent; two tokens mapped to the same slot race.
 */
KVQ_API kvq_status kvq_cache_write(const void *k, const void *v,
                           const int64_t *slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks,
                           int32_t dtype, int32_t group_size,
                           void *k_pool, void *v_pool,
                           float *k_scale, float *v_scale, void *stream);

/*
 * kvq_paged_decode -- one decode step of attention for a batch of sequences
 * over the paged pool ("KV Cache优化实战" s1.1, s2.1, s2.2, s4.3).
 *
 * For sequence b with ctx = context_lens[b] and query head g (KV head
 * h = g / (Hq / Hkv)):
 *   z_t = softmax_scale * q[b][g] . Khat[b][t][h]          for t < ctx
 *   out[b][g] = sum_t softmax(z)_t * Vhat[b][t][h]
 * where logical token t lives in slot block_tables[b][t / block_size] *
 * block_size + t % block_size and Khat / Vhat are the dequantized values
 * (code * scale; dequantization is fused into the kernel).
 *
 *   q             fp16 [num_seqs][num_q_heads][head_dim].
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entries past
 *                 ceil(ctx / block_size) are never read.  Bits 0..29 of an
 *                 entry are the physical block id; bit 30 may be set on
 *                 blocks that several sequences share (a prefix): it only
 *                 changes the cache policy of their loads, never the result.
 *                 Bit 31 must be 0.
 *   context_lens  int32 [num_seqs] on the device, each in
 *                 [1, max_context_len]; max_context_len is the host-side bound
 *                 (used to plan the split) and must not exceed
 *                 max_blocks_per_seq * block_size.
 *   softmax_scale 0 selects 1 / sqrt(head_dim).
 *   split_tokens  how the work is cut (the cut depends only on the lengths,
 *                 never on which physical blocks hold the data):
 *                 0 = balanced: the batch's 16-token tiles, taken unit by
 *                 unit ((sequence, KV head) units, sequence-major), are dealt
 *                 in equal contiguous runs to as many wavefronts as the GPU
 *                 holds at once; a unit cut by run boundaries is finished by
 *                 an exact log-sum-exp merge of its pieces.
 *                 > 0 (a multiple of 16): every unit is cut into spans of
 *                 split_tokens logical tokens, merged the same way.
 *   out           fp16 [num_seqs][num_q_heads][head_dim] (written).
 *   workspace     device scratch of at least kvq_decode_workspace_size(...)
 *                 bytes (required); its contents on entry do not matter.  It
 *                 holds the run plan and the partial results of cut units
 *                 between the launches of one call, so calls sharing a
 *                 workspace must be ordered (same stream).
 */
KVQ_API kvq_status kvq_paged_decode(const void *q, const void *k_pool,
                            const void *v_pool, const float *k_scale,
                            const float *v_scale, const int32_t *block_tables,
                            int32_t max_blocks_per_seq,
                            const int32_t *context_lens,
                            int32_t max_context_len, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t dtype,
                            int32_t group_size, float softmax_scale,
                            int32_t split_tokens, void *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * kvq_paged_prefill -- attention of a chunk of new tokens per sequence over
 * the paged pool: prefill, or chunked prefill of a long prompt ("KV Cache优化
 * 实战" s1.1: prefill computes the K/V of every prompt token, each token
 * attending to the tokens before it; xpshop.cn article 312 s6: long prompts
 * are processed in chunks).
 *
 * Sequence b's chunk is the last n_b = query_start[b+1] - query_start[b] of
 * its ctx = context_lens[b] tokens; their K/V must already be in the pool
 * (kvq_cache_write).  Chunk token i sits at position ctx - n_b + i and, for
 * query head g (KV head h = g / (Hq / Hkv)):
 *   out[query_start[b] + i][g] = sum_{t <= ctx - n_b + i} softmax_t(
 *       softmax_scale * q[query_start[b] + i][g] . Khat[b][t][h]) Vhat[b][t][h]
 *
 *   q, out        fp16 [total chunk tokens][num_q_heads][head_dim].
 *   query_start   int32 [num_seqs + 1] on the device, non-decreasing, with
 *                 n_b <= context_lens[b]; max_query_len >= every n_b is the
 *                 host-side bound that sizes the launch.
 *   split_mode    how the work is cut (KVQ_PREFILL_*):
 *     WALK: one workgroup per (sequence, KV head, block of
 *       128 / (Hq / Hkv) chunk tokens) walks the tokens it needs, each
 *       32-token step of K/V converted once into LDS for its 128
 *       (token, query head) rows;
 *     SPLIT: the decode partition -- the batch's 16-token tiles dealt in
 *       equal runs over every wavefront the GPU holds, an MFMA column per
 *       (chunk token, query head) of a KV head with its own causal bound
 *       (one or two groups of 16 columns per wavefront), cut units merged
 *       by log-sum-exp.  Chunks of more than 32 / (Hq / Hkv) tokens are
 *       first cut into virtual sequences of that many tokens (a small
 *       launch writes their lengths into the workspace);
 *     AUTO: SPLIT for chunks of at most 32 / (Hq / Hkv) tokens and
 *       whenever WALK would launch fewer wavefronts than the GPU holds (a
 *       few sequences with short chunks over long contexts), else WALK.
 *   workspace     device scratch of kvq_prefill_workspace_size(...) bytes
 *                 for these arguments (its contents on entry do not matter;
 *                 calls sharing it must be ordered).  That size is 0, and
 *                 workspace may be NULL, when the cut is WALK.
 *   The other arguments are those of kvq_paged_decode.
 */
KVQ_API kvq_status kvq_paged_prefill(const void *q, const int32_t *query_start,
                             int32_t max_query_len, const void *k_pool,
                             const void *v_pool, const float *k_scale,
                             const float *v_scale, const int32_t *block_tables,
                             int32_t max_blocks_per_seq,
                             const int32_t *context_lens,
                             int32_t max_context_len, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t dtype,
                             int32_t group_size, float softmax_scale,
                             int32_t split_mode, void *out, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Workspace bytes kvq_paged_prefill needs for these arguments and split_mode
 * on the current device (0 when the cut is WALK).  Returns SIZE_MAX for
 * invalid arguments. */
KVQ_API size_t kvq_prefill_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_context_len,
                                  int32_t max_query_len, int32_t split_mode);

/*
 * Per-head mixed precision (xpshop.cn article 312, s6: the attention heads
 * that are sensitive to quantization keep fp16, the others are quantized).
 * A layer then keeps one set of pools per format, each holding a subset of
 * the model's KV heads: pool head i is model KV head kv_head_ids[i]
 * (int32 [pool heads] on the device, distinct, each < the model's KV heads).
 *
 * kvq_cache_write_heads -- kvq_cache_write into such a pool: k, v are
 *   [num_tokens][num_kv_heads_src][head_dim] with all the model's KV heads;
 *   the pool (and its scales) have num_kv_heads heads.
 * kvq_paged_decode_heads -- kvq_paged_decode over such a pool: q and out
 *   are [num_seqs][num_q_heads][head_dim] with all the model's query heads
 *   (num_q_heads / num_kv_heads per KV head); only the rows of the query heads
 *   of the pool's KV heads are read and written, so one call per pool fills
 *   out.  The workspace is sized with kvq_decode_workspace_size(num_seqs,
 *   pool_heads * num_q_heads / num_kv_heads, pool_heads, ...); calls that
 *   share a workspace must be ordered.
 */
KVQ_API kvq_status kvq_cache_write_heads(const void *k, const void *v,
                                 const int64_t *slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads_src,
                                 const int32_t *kv_head_ids, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t dtype,
                                 int32_t group_size, void *k_pool, void *v_pool,
                                 float *k_scale, float *v_scale, void *stream);

KVQ_API kvq_status kvq_paged_decode_heads(const void *q, const void *k_pool,
                                  const void *v_pool, const float *k_scale,
                                  const float *v_scale,
                                  const int32_t *block_tables,
                                  int32_t max_blocks_per_seq,
                                  const int32_t *context_lens,
                                  int32_t max_context_len, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  const int32_t *kv_head_ids, int32_t pool_heads,
                                  int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, int32_t dtype,
                                  int32_t group_size, float softmax_scale,
                                  int32_t split_tokens, void *out,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Workspace bytes kvq_paged_decode needs for these arguments on the
 * current device (an upper bound over formats and kernel occupancy).
 * Returns SIZE_MAX for invalid arguments. */
KVQ_API size_t kvq_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_context_len,
                                 int32_t split_tokens);

/*
 * kvq_copy_blocks -- copy whole blocks (codes of every slot, and INT8 scales)
 * of one layer's pools: block pairs[2i] -> pairs[2i+1].  Used for
 * copy-on-write of a shared, partially filled block before a sequence writes
 * into it ("KV Cache优化实战" s4.4).  block_pairs: int32 [num_pairs][2] on the
 * device; destinations must be distinct and not be sources.  FP8 / FP16 pools
 * pass NULL scales.
 */
KVQ_API kvq_status kvq_copy_blocks(const int32_t *block_pairs, int32_t num_pairs,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks,
                           int32_t dtype, int32_t group_size, void *k_pool,
                           void *v_pool, float *k_scale, float *v_scale,
                           void *stream);

/*
 * Swap of whole blocks between one layer's pools and a staging buffer, for
 * preemption: under memory pressure a low-priority request's KV is swapped
 * out and brought back later (xpshop.cn article 312, s3 and s6), possibly
 * into other physical blocks (the caller rewrites the block table).
 *
 * A swap slot holds one block: [K codes][V codes][K scales][V scales] (the
 * scales only for per-group formats; static scales belong to the layer, not
 * to blocks), padded to 256 bytes; kvq_swap_block_bytes returns its size
 * (SIZE_MAX for unsupported arguments).  The buffer holds num_slots slots,
 * is owned by the caller and may be device memory or pinned host memory
 * (hipHostMalloc), which the kernel reads and writes across the bus.
 *
 *   block_slot_pairs  int32 [num_pairs][2] = (pool block, swap slot),
 *                     device-accessible; pairs with a block outside the pool
 *                     or a slot outside [0, num_slots) are skipped.  The
 *                     slots (swap out) or blocks (swap in) written must be
 *                     distinct.
 *   kvq_swap_out      copies each pool block into its slot of dst.
 *   kvq_swap_in       copies each slot of src into its pool block.
 * Asynchronous on stream; the caller synchronizes before it reads a host
 * buffer or reuses the swapped-out blocks.
 */
KVQ_API size_t kvq_swap_block_bytes(int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t dtype,
                                    int32_t group_size);

KVQ_API kvq_status kvq_swap_out(const int32_t *block_slot_pairs, int32_t num_pairs,
                        int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks,
                        int32_t dtype, int32_t group_size,
                        const void *k_pool, const void *v_pool,
                        const float *k_scale, const float *v_scale,
                        void *dst, int64_t num_slots, void *stream);

KVQ_API kvq_status kvq_swap_in(const int32_t *block_slot_pairs, int32_t num_pairs,
                       int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks,
                       int32_t dtype, int32_t group_size,
                       const void *src, int64_t num_slots,
                       void *k_pool, void *v_pool,
                       float *k_scale, float *v_scale, void *stream);

/*
 * kvq_paged_decode_noalloc -- kvq_paged_decode for callers that cannot
 * allocate device memory: code recorded into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments and result as
 * kvq_paged_decode, without the workspace: the run plan and the partial
 * results live in a static device array of KVQ_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on every GPU it runs on until the process ends.
 * The call allocates nothing (no hipMalloc, no hipFree).
 *
 * A call whose plan would need more scratch than that returns
 * KVQ_ERR_WORKSPACE (kvq_paged_decode with a caller workspace has no such
 * limit).  At split_tokens = 0 on a 256-CU GPU that holds any batch of up
 * to a million sequences whose (query heads / KV heads) x head_dim is at
 * most 512 (e.g. GQA 4:1 at head_dim 128); short fixed spans over large
 * batches can exceed it.  Every call on one GPU
 * shares that GPU's array: calls that may overlap on one GPU (different
 * streams, or threads) race and give wrong results; order them.  The
 * array's contents on entry never matter.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

KVQ_API kvq_status kvq_paged_decode_noalloc(const void *q, const void *k_pool,
                                    const void *v_pool, const float *k_scale,
                                    const float *v_scale, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq,
                                    const int32_t *context_lens,
                                    int32_t max_context_len, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t dtype,
                                    int32_t group_size, float softmax_scale,
                                    int32_t split_tokens, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
