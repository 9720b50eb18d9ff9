/*
 * pagedkv.h - C ABI of libpagedkv.so: paged grouped-query decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * One decode step of an LLM serving engine, per attention layer: every
 * running sequence contributes one query token; its new K/V is first written
 * into its slot of a pool of fixed-size KV blocks, then its query heads
 * attend, with grouped-query heads, over the K/V reached through the
 * sequence's block table, using online softmax.  Sources (by title and
 * section):
 *   - "rvLLM: High-performance LLM inference in Rust", section "CUDA
 *     Kernels": PagedAttention V2 (block-table indirection, online softmax),
 *     Reshape and Cache (write the new K/V into the paged cache), FP8 KV Cache
 *     (E4M3 quantisation/dequantisation with per-head scaling).
 *   - "rvllm - A Small LLM Inference Engine in Rust", section "How it's put
 *     together": the KV cache is a pool of fixed-size blocks, each step takes
 *     explicit write positions and read blocks; each KV head is shared by a
 *     group of query heads.
 *   - "LLM Serving Kernels", section "Projects": project 04 (page tables,
 *     GQA/MQA, online softmax), project 05 (E4M3 storage, page scales, fused
 *     dequantisation).
 *
 * Conventions for every entry point
 * ---------------------------------
 *   - All tensor pointers are device pointers owned by the caller, contiguous
 *     row-major.  The library never allocates, frees or synchronises, keeps no
 *     pointer after it returns, and enqueues all work on `stream` (a
 *     hipStream_t; NULL is the default stream).
 *   - Return value: PKV_OK (0) on success, else an error code; the message of
 *     the last error on the calling thread is returned by pkv_last_error().
 *     Arguments are checked on the host before anything is enqueued; on an
 *     error nothing is enqueued.  PKV_ERR_HIP reports a failed launch.
 *   - Values that live in device memory (block ids, context lengths, slots)
 *     are not read by the host.  Their ranges are preconditions:
 *     0 <= block id < num_blocks, 0 <= context_lens[b] <= max_blocks_per_seq*16,
 *     slots unique and < num_blocks*16.  The kernels clamp a context length
 *     to max_blocks_per_seq*16 and skip out-of-range slots; a block id out
 *     of range is undefined behaviour.
 *
 * Shapes and names
 * ----------------
 *   B = num_seqs, Hq = num_q_heads, Hkv = num_kv_heads, G = Hq / Hkv (query
 *   head i reads KV head i / G: contiguous groups), D = head_dim,
 *   NB = num_blocks, MBPS = max_blocks_per_seq, block_size = 16 tokens.
 *
 * KV cache byte layout (k_cache and v_cache are [NB][Hkv][tile])
 * ---------------------------------------------------------------
 *   One tile holds the 16 token slots x D elements of one (block, kv head),
 *   16*D*e bytes with e = element size (4 f32, 2 f16/bf16, 1 e4m3).  Slot s
 *   is token offset s % 16 of block s / 16.  Inside a tile:
 *     K: element (t, d) at ((d / x) * 16 + t) * x + d % x,   x = 16 / e
 *        (16-byte chunks of one token's dims; the 16 tokens of one chunk
 *        index are adjacent);
 *     V: element (t, d) at ((((d / (16n)) * 4 + t / 4) * 16 + d % 16) * n
 *                             + (d / 16) % n) * 4 + t % 4,   n = 4 / e
 *        (groups of 4 consecutive tokens of one dim are adjacent).
 *   Both place each 64-lane wave's 16-byte loads on one contiguous 1 KiB and
 *   hand the matrix cores their operands without a transpose.
 *   This byte layout is the library's own, not a [NB][Hkv][16][D] array:
 *   callers fill a pool only through the library's writers (kv_cache_write,
 *   paged_decode_step, kv_cache_quantize_e4m3, kv_cache_append_e4m3,
 *   kv_cache_copy_blocks) and treat the tiles as opaque.  Only the sizes
 *   above are part of the contract: NB * Hkv * 16 * D elements per cache.
 *
 * Supported combinations (q / KV / out): f32/f32/f32; f16/f16/{f32,f16};
 * bf16/bf16/{f32,bf16}; f16/e4m3/{f32,f16}.  D in {64, 128}, G in 1..16,
 * block_size 16.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad partition size, non-finite scale */
  PKV_ERR_UNSUPPORTED = 2, /* dtype combination, head_dim or group size not built */
  PKV_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
};

enum pkv_dtype { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_E4M3 = 3 };

/*
 * Sliding window.  With desc->sliding_window = W > 0 every attention entry
 * point attends, for sequence b, only to positions [lo, L) with L =
 * context_lens[b] and lo = max(0, L - W) (the pages list sliding-window
 * attention: "rvLLM: High-performance LLM inference in Rust", sections
 * "Project Status" and "Changelog"; Gemma 4 runs 50 of its 60 layers with it,
 * "rvLLM: The Inference Engine That Lets TPUs Compete by Writing Less Kernel
 * Code", section "The flat-scan trick that makes TPU inference work").  Table
 * entries before block lo / 16 are never read, so a cache may have released
 * them.  Partitions then start at a = 16 * floor(lo / 16): partition p covers
 * positions [max(lo, a + p P), min(a + (p+1) P, L)), and there are
 * ceil((L - a) / P) of them.
 */

/* Sizes and element types of one decode-attention problem.  */
typedef struct pkv_desc {
  int32_t num_seqs;           /* B >= 0 (0: nothing to do)                    */
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads               */
  int32_t num_kv_heads;       /* Hkv >= 1                                     */
  int32_t head_dim;           /* D: 64 or 128                                 */
  int32_t block_size;         /* tokens per block: must be 16                 */
  int32_t num_blocks;         /* NB: blocks in the pool                       */
  int32_t max_blocks_per_seq; /* MBPS: row length of block_tables (>= 1)      */
  int32_t q_dtype;            /* pkv_dtype of q (and of k/v for the write)    */
  int32_t kv_dtype;           /* pkv_dtype of the caches                      */
  int32_t out_dtype;          /* pkv_dtype of out                             */
  int32_t sliding_window;     /* W >= 0; 0: attend to the whole context; W > 0:
                                 each query attends only to positions
                                 [max(0, L - W), L) of its context (see
                                 "Sliding window" above)                      */
} pkv_desc;

/*
 * kv_cache_write - write each new token's K and V into its cache slot
 * ("rvLLM: High-performance LLM inference in Rust", section "CUDA Kernels",
 * row "Reshape and Cache"; "rvllm - A Small LLM Inference Engine in Rust",
 * section "How it's put together", write_positions).
 *
 *   k, v          [num_tokens][Hkv][D] in kv_dtype (f32, f16 or bf16)
 *   slot_mapping  int64 [num_tokens]; token t goes to slot slot_mapping[t];
 *                 a negative slot skips the token
 *   k_cache, v_cache  the pool, layout above; only the named slots change
 * Bitwise copy.  Two tokens naming the same slot: which one lands is
 * unspecified.  An e4m3 cache returns PKV_ERR_UNSUPPORTED (use
 * kv_cache_append_e4m3 for new tokens, kv_cache_quantize_e4m3 for whole
 * blocks).
 */
int kv_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                   int64_t num_tokens, void* k_cache, void* v_cache,
                   const pkv_desc* desc, void* stream);

/*
 * kv_cache_quantize_e4m3 - quantise whole blocks of fp32 K and V into an
 * e4m3 pool, one fp32 scale per (block, kv head) for K and one for V ("LLM
 * Serving Kernels", section "Projects", row 05: E4M3 storage, page scales;
 * "rvLLM: High-performance LLM inference in Rust", section "CUDA Kernels",
 * row "FP8 KV Cache": per-head scaling).
 *
 *   k_src, v_src    fp32 [num_src_blocks][16][Hkv][D]: the 16 token slots of
 *                   each source block in slot order
 *   block_ids       int32 [num_src_blocks]: destination block of each
 *   valid_tokens    int32 [num_src_blocks]: leading slots holding data; the
 *                   rest are ignored for the scale and receive code 0
 *   k_cache, v_cache  e4m3 pool (desc->kv_dtype must be PKV_E4M3)
 *   kv_scales       fp32 [2][NB][Hkv]; entry (0|1, block, head) is written
 * scale = fp32(amax / 448) over the valid slots of (block, kv head), 1 when
 * amax is 0; code = nearest-even OCP E4M3 (max 448) of clamp(fp32(x /
 * scale), -448, 448).  Distinct block_ids are required.
 */
int kv_cache_quantize_e4m3(const float* k_src, const float* v_src, const int32_t* block_ids,
                           const int32_t* valid_tokens, int32_t num_src_blocks, void* k_cache,
                           void* v_cache, float* kv_scales, const pkv_desc* desc, void* stream);

/*
 * kv_cache_append_e4m3 - write each new token's K and V into an e4m3 pool,
 * quantising on append with one fp32 scale per (block, kv head) for K and
 * one for V (the per-page, per-head scaling of "LLM Serving Kernels",
 * section "Projects", row 05, and "rvLLM: High-performance LLM inference in
 * Rust", section "CUDA Kernels", row "FP8 KV Cache", applied to the decode
 * step's new token).
 *
 *   k, v          fp32 [num_tokens][Hkv][D]
 *   slot_mapping  int64 [num_tokens]; negative skips the token
 *   k_cache, v_cache  e4m3 pool (desc->kv_dtype must be PKV_E4M3)
 *   kv_scales     fp32 [2][NB][Hkv], read and updated
 * Per (token, kv head), for K and for V, every step in fp32: s =
 * amax(|x|) / 448.  In slot 0 of a block the token sets the block's scale to
 * s (1 if s is 0).  In a later slot, if s exceeds the stored scale, the
 * block's earlier slots are re-encoded as code(clamp(decode(c) * old / s))
 * and the scale becomes s; so the scale is always fp32(amax / 448) over the
 * block's tokens, as kv_cache_quantize_e4m3 makes it.  The token's code is
 * code(clamp(x / scale)), nearest-even OCP E4M3.  At most one token per
 * block per call.  Slots past the token in its block are left as they are.
 */
int kv_cache_append_e4m3(const float* k, const float* v, const int64_t* slot_mapping,
                         int64_t num_tokens, void* k_cache, void* v_cache, float* kv_scales,
                         const pkv_desc* desc, void* stream);

/*
 * kv_cache_copy_blocks - copy whole blocks inside the pool, for
 * copy-on-write forks such as beam search ("rvLLM: High-performance LLM
 * inference in Rust", section "CUDA Kernels", row "Block Copy"; section
 * "Architecture": the block manager's copy-on-write and prefix sharing).
 *
 *   block_mapping  int32 [num_pairs][2]: (src, dst) block ids
 *   num_pairs      0 .. 65535
 *   k_cache, v_cache  the pool in desc->kv_dtype (any of the four)
 *   kv_scales      fp32 [2][NB][Hkv] for an e4m3 pool (its K and V scales
 *                  are copied too), else NULL
 * Block dst's K and V tiles of every kv head become bit copies of block
 * src's.  Reads desc->num_kv_heads, head_dim, num_blocks and kv_dtype only.
 * A pair naming a block outside [0, num_blocks) is skipped.  No block may
 * be a destination twice, or both a source and a destination, in one call
 * (the copies run in parallel).
 */
int kv_cache_copy_blocks(const int32_t* block_mapping, int32_t num_pairs, void* k_cache,
                         void* v_cache, float* kv_scales, const pkv_desc* desc, void* stream);

/*
 * paged_decode_attention - one decode step of attention for every sequence
 * in one pass: out[b][i] = softmax(q[b][i] . K_b^T * scale) V_b, where K_b,
 * V_b are the first context_lens[b] tokens of sequence b gathered through
 * block_tables[b] for KV head i / G ("rvLLM: High-performance LLM inference
 * in Rust", section "CUDA Kernels", row "PagedAttention V2"; "LLM Serving
 * Kernels", section "Projects", row 04).
 *
 *   q             [B][Hq][D] in q_dtype
 *   k_cache, v_cache  [NB][Hkv][tile] in kv_dtype
 *   block_tables  int32 [B][MBPS]; entries past ceil(context_lens[b]/16)
 *                 (and, with a sliding window, before the window's first
 *                 block) are never read
 *   context_lens  int32 [B]; includes the token written this step; a
 *                 sequence with 0 gets a zero output
 *   scale         softmax scale (finite), usually 1/sqrt(D)
 *   kv_scales     e4m3 caches only, else NULL: fp32 [2][NB][Hkv], the K (0)
 *                 and V (1) scale of each (block, kv head); the value of a
 *                 code c is decode(c) * scale ("LLM Serving Kernels",
 *                 "Projects", row 05: page scales, fused dequantisation)
 *   out           [B][Hq][D] in out_dtype
 * One workgroup per (sequence, kv head): suited to short contexts or many
 * sequences of similar length.  The longest sequence's item bounds the
 * step, so for a ragged batch (lengths spread over decades) or long
 * contexts use paged_decode_attention_balanced (or its _static form, which
 * needs no workspace argument): on a 128-sequence layer with lognormal
 * lengths it runs twice as fast as this one pass.
 */
int paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           float scale, const float* kv_scales, void* out,
                           const pkv_desc* desc, void* stream);

/*
 * paged_decode_attention_partial - split-context ("flash-decoding") first
 * half: the context of each sequence is cut into partitions of
 * partition_size tokens, and each (sequence, query head, partition) yields
 * the softmax-normalised output over its tokens and the log-sum-exp of its
 * scaled logits.  Arguments as paged_decode_attention, plus:
 *
 *   partition_size  tokens per partition: a positive multiple of 16
 *   tmp_out       fp32 [B][Hq][S][D], S = paged_decode_num_partitions()
 *   tmp_lse       fp32 [B][Hq][S], natural-log LSE of the scaled logits
 * Only partitions p < ceil(context_lens[b] / partition_size) are written;
 * the others are left untouched.
 */
int paged_decode_attention_partial(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   float scale, const float* kv_scales, int32_t partition_size,
                                   float* tmp_out, float* tmp_lse,
                                   const pkv_desc* desc, void* stream);

/*
 * paged_decode_attention_reduce - split-context second half: merges each
 * (sequence, query head)'s partitions p < ceil(context_lens[b] /
 * partition_size) by out = sum_p w_p o_p / sum_p w_p, w_p = exp(lse_p -
 * max lse).  tmp_out, tmp_lse, context_lens, partition_size and desc as
 * given to the partial call; out [B][Hq][D] in out_dtype.
 */
int paged_decode_attention_reduce(const float* tmp_out, const float* tmp_lse,
                                  const int32_t* context_lens, int32_t partition_size,
                                  void* out, const pkv_desc* desc, void* stream);

/*
 * paged_decode_attention_split - the partial and reduce halves in one
 * launch: same result as paged_decode_attention_partial followed by
 * paged_decode_attention_reduce.  A sequence whose context fits one
 * partition writes out directly; for the others, the last partition of each
 * (sequence, kv head) to finish merges all of them (flash-decoding with the
 * log-sum-exp merge done in-kernel).  Arguments as the partial call, plus:
 *
 *   workspace        device memory of workspace_bytes >=
 *                    paged_decode_split_workspace_bytes(desc, partition_size)
 *                    bytes, 256-byte aligned.  It holds per-(sequence, kv
 *                    head) int32 counters followed by the partials.  It must
 *                    be zero-filled before its first use; every call leaves
 *                    the counters zero again, so later calls may reuse it
 *                    without clearing.  Calls that run at the same time must
 *                    not share a workspace.
 *   out              [B][Hq][D] in out_dtype
 */
int paged_decode_attention_split(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 float scale, const float* kv_scales, int32_t partition_size,
                                 void* workspace, int64_t workspace_bytes, void* out,
                                 const pkv_desc* desc, void* stream);

/* Workspace bytes paged_decode_attention_split needs, or -1.  */
int64_t paged_decode_split_workspace_bytes(const pkv_desc* desc, int32_t partition_size);

/*
 * paged_decode_step - one decode step in one launch: each sequence's new
 * token is written into the cache at its position context_lens[b] - 1 (the
 * new token counts in the context, and is written before attention reads
 * it), then the attention of paged_decode_attention_split is computed
 * ("rvllm - A Small LLM Inference Engine in Rust", section "How it's put
 * together": explicit write positions, then the blocks to read).  The
 * result equals kv_cache_write of the same rows at those slots followed by
 * paged_decode_attention_split, bit for bit, in the cache and in out.
 *
 *   k_new, v_new     [B][Hkv][D] in the cache dtype (f32, f16 or bf16; an
 *                    E4M3 cache is rejected, its tokens go through
 *                    kv_cache_append_e4m3); row b is sequence b's token
 *   k_cache, v_cache written at slot block_tables[b][(L_b-1)/16]*16 +
 *                    (L_b-1)%16 for every b with L_b >= 1 (the block the
 *                    work item holding that position reads; it must not be
 *                    shared with another sequence)
 *   other arguments  as paged_decode_attention_split (no kv_scales); the
 *                    workspace is the split workspace
 *
 * The write is done inside the attention kernel by the work item that
 * reads the block, ahead of its loads, so the step costs one launch
 * instead of two.
 */
int paged_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t partition_size, void* workspace, int64_t workspace_bytes, void* out,
                      const pkv_desc* desc, void* stream);

/*
 * paged_decode_attention_balanced - the same attention output, with the
 * split-context work cut by load instead of at fixed partition_size
 * boundaries (flash-decoding's split and log-sum-exp merge as above, split
 * points chosen so that the work is even whatever the mix of context
 * lengths).  The tiles of all (sequence, kv head) pairs form one stream,
 * sequence-major.  For f32 / f16 / bf16 caches every compute unit takes an
 * equal contiguous stretch of it, and the unit's waves share their stretch
 * at run time; for E4M3 caches every wave of the resident grid takes an
 * equal stretch.  A (sequence, kv head) cut by a stretch's ends (or, in the
 * first form, longer than 48 tiles) is finished as partials merged by
 * log-sum-exp in a second kernel on the same stream.  Arguments as
 * paged_decode_attention, plus:
 *
 *   workspace        device memory of workspace_bytes >=
 *                    paged_decode_balanced_workspace_bytes(desc) bytes,
 *                    256-byte aligned, holding per-sequence tile offsets and
 *                    the partials.  No clearing is needed; calls that run at
 *                    the same time must not share a workspace.
 * Requires num_seqs <= 2048 (else PKV_ERR_UNSUPPORTED) and
 * num_seqs * num_kv_heads * max_blocks_per_seq < 2^31.  The summation order
 * depends on the batch, the GPU's compute-unit count and (for f32 / f16 /
 * bf16 caches) on which wave takes which tiles at run time, so results agree
 * with the other entry points, and two calls of this one with each other,
 * to fp32 rounding, not bitwise.
 */
int paged_decode_attention_balanced(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    float scale, const float* kv_scales, void* workspace,
                                    int64_t workspace_bytes, void* out, const pkv_desc* desc,
                                    void* stream);

/*
 * paged_decode_attention_balanced_partial / _reduce - the two launches of
 * paged_decode_attention_balanced, for callers that time or schedule them
 * apart ("LLM Serving Kernels", section "Evidence standard": the dominant
 * kernel is measured on its own).  _partial takes the same arguments and
 * streams the tiles: it writes the out rows of the (sequence, kv head) pairs
 * finished whole and leaves the partials and per-sequence tile offsets in the
 * workspace.  _reduce, enqueued after it on the same stream with the same
 * desc and workspace, merges the partials into the remaining out rows (and
 * writes zeros for empty contexts).  Together they equal
 * paged_decode_attention_balanced; the workspace must not be reused in
 * between.  Errors as paged_decode_attention_balanced.
 */
int paged_decode_attention_balanced_partial(const void* q, const void* k_cache, const void* v_cache,
                                            const int32_t* block_tables, const int32_t* context_lens,
                                            float scale, const float* kv_scales, void* workspace,
                                            int64_t workspace_bytes, void* out, const pkv_desc* desc,
                                            void* stream);
int paged_decode_attention_balanced_reduce(void* workspace, int64_t workspace_bytes, void* out,
                                           const pkv_desc* desc, void* stream);

/* Workspace bytes paged_decode_attention_balanced needs on the current
 * device (it grows with the device's compute units, or for E4M3 caches with
 * the number of waves it holds), or -1.  */
int64_t paged_decode_balanced_workspace_bytes(const pkv_desc* desc);

/*
 * paged_decode_attention_balanced_static - paged_decode_attention_balanced
 * without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It allocates nothing and calls no allocating routine;
 * its partials live in a 32 MiB device array inside the library, one copy
 * per GPU, held until the process ends (looked up on the first call on each
 * device, which must be the current device).  Same arguments and kernels
 * as paged_decode_attention_balanced, and its result to fp32 rounding (the
 * summation order is settled at run time).  Problems needing more than
 * 32 MiB of workspace (paged_decode_balanced_workspace_bytes) return
 * PKV_ERR_INVALID_ARG.  The array keeps the last call's contents and needs no
 * clearing (every byte is written before it is read within a call); calls
 * that overlap in time on one GPU (different streams, or different threads)
 * share it and race: serialise them.
 */
int paged_decode_attention_balanced_static(const void* q, const void* k_cache, const void* v_cache,
                                           const int32_t* block_tables, const int32_t* context_lens,
                                           float scale, const float* kv_scales, void* out,
                                           const pkv_desc* desc, void* stream);

/*
 * paged_prefill_attention - attention for several new tokens per sequence
 * (chunked prefill, speculative verification), causal inside the new
 * tokens ("rvLLM: High-performance LLM inference in Rust", section "CUDA
 * Kernels", row "FlashAttention-2": prefill and decode with causal
 * masking; row "PagedAttention V2": the block-table gather).
 *
 *   q             [num_query_tokens][Hq][D] in q_dtype: the query rows of all
 *                 sequences, sequence-major
 *   query_start   int32 [B + 1]: sequence b owns rows query_start[b] ..
 *                 query_start[b+1] - 1 (0 = query_start[0] <= ... <=
 *                 query_start[B] = num_query_tokens), its n_b newest tokens,
 *                 at positions L_b - n_b .. L_b - 1 of its context (n_b <=
 *                 L_b; their K/V are already in the cache)
 *   context_lens  int32 [B]: L_b, including the new tokens
 *   partition_size  0: one pass per (sequence, kv head, pack of tokens);
 *                 else a positive multiple of 16: split the keys into
 *                 partitions of that many positions and merge their
 *                 log-sum-exp partials (needs the workspace)
 *   workspace     device memory of workspace_bytes >=
 *                 paged_prefill_workspace_bytes(desc, num_query_tokens,
 *                 partition_size) bytes, 256-byte aligned (NULL when
 *                 partition_size is 0)
 *   out           [num_query_tokens][Hq][D] in out_dtype
 * The row of token j of sequence b (position p = L_b - n_b + j) attends to
 * positions 0 .. p.  Other arguments as paged_decode_attention.  Requires
 * num_seqs <= 2048 and sliding_window = 0 (else PKV_ERR_UNSUPPORTED).
 */
int paged_prefill_attention(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* query_start, int32_t num_query_tokens, float scale,
                            const float* kv_scales, int32_t partition_size, void* workspace,
                            int64_t workspace_bytes, void* out, const pkv_desc* desc, void* stream);

/* Workspace bytes paged_prefill_attention needs (0 for partition_size 0), or -1.  */
int64_t paged_prefill_workspace_bytes(const pkv_desc* desc, int32_t num_query_tokens,
                                      int32_t partition_size);

/* S = ceil(MBPS * 16 / partition_size), or -1 on invalid arguments.  */
int64_t paged_decode_num_partitions(const pkv_desc* desc, int32_t partition_size);

/* Bytes of tmp_out plus tmp_lse for the partial/reduce pair, or -1.  */
int64_t paged_decode_workspace_bytes(const pkv_desc* desc, int32_t partition_size);

/* Message of the last error on the calling thread ("" if none).  */
const char* pkv_last_error(void);

/* Library version string.  */
const char* pkv_version(void);

/* The same two helpers under the library's own prefix: pagedkv_last_error
 * returns exactly what pkv_last_error returns, pagedkv_version what
 * pkv_version returns.  */
const char* pagedkv_last_error(void);
const char* pagedkv_version(void);

/*
 * pkv_read_bandwidth_probe - a measurement aid, not part of the attention
 * path: reads `bytes` of device memory at src once with 16-byte
 * non-temporal loads (four in flight per thread, two 256-thread workgroups
 * per compute unit) and writes one XOR-folded word per workgroup to out.
 * Timing it (events on `stream`) gives the read bandwidth this GPU
 * sustains: a practical ceiling, beside the published HBM peak, for the
 * decode kernels' byte rates.  The pages define no such operation; it
 * belongs to the measurement, not to the method.
 *   src        device, 16-byte aligned, bytes > 0 and a multiple of 16
 *   out        device, out_words words (caller-owned); the grid is
 *              min(out_words, 2 x CUs) workgroups
 * Errors: PKV_ERR_INVALID_ARG on a null pointer, misalignment or a bad size.
 */
int pkv_read_bandwidth_probe(const void* src, int64_t bytes, uint32_t* out, int32_t out_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
