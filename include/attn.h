/*
 * attn.h — C ABI of the MI355X (gfx950) KV-cache attention library.
 *
 * Three operations (plus decode with a fused cache append, with or without
 * the rotary embedding, decode and prefill over a paged cache and the decoder
 * form of top-k), each one asynchronous launch sequence on the caller's HIP
 * stream:
 *
 *   attn_decode   single-token decode over a statically preallocated cache,
 *                 attending to rows [0, position_id] (or [0, seq_lens[b]) for
 *                 a ragged batch) with no materialised mask.
 *                 Source: "MiniCPM4 forward_step Attention Performance Fix",
 *                 §3 (pass only the valid cache rows; the slice bound is the
 *                 causal mask) and §4.1 (patched forward_step: SDPA with
 *                 enable_gqa over the sliced cache, default scale).
 *   attn_prefill  causal prefill of Lq new tokens against a cached prefix,
 *                 every head in one launch.
 *                 Source: "step14_3 — batched attention: removing the per-head
 *                 Python loop", solution section (all heads at once: Q·Kᵀ
 *                 scaled by 1/sqrt(d_head), causal -inf mask, softmax, ·V) and
 *                 the going-further section (one fused kernel).
 *   attn_topk     top-k sparsified scores: q·kᵀ with no scale, keep the
 *                 topk largest per row, zero the rest, multiply by v; no
 *                 softmax.
 *                 Source: "c2psa multi-head self-attention high-concurrency
 *                 inference", core implementation §2 (dynamic top-k
 *                 sparsification) and the full C2PSA class (topk=64).
 *   attn_topk_causal  the same scores in the decoder form: a query chooses
 *                 only among keys on its left and always keeps its most
 *                 recent topk/2.
 *                 Source: the same page, further thoughts.
 *
 * attn_read_probe is a measurement aid beside them: a streaming read that
 * gives the bandwidth the memory system attains.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers (memory the caller allocated with hipMalloc
 *   or through a framework) unless stated otherwise. The caller owns every
 *   buffer. The library allocates nothing, keeps no pointer after the call
 *   returns and never synchronises; results are valid once the caller has
 *   synchronised `stream`.
 * - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 * - Layouts are dense, row-major, innermost dimension contiguous. Data
 *   pointers must be 16-byte aligned. `out` must not alias an input.
 * - Every argument check is done on host scalars before any launch; a failed
 *   check launches nothing and returns a nonzero status. `attn_last_error()`
 *   then describes the failing argument (per thread).
 * - Device faults are sticky HIP errors: they surface as ATTN_E_HIP on this
 *   or a later call and the process must restart.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below are int-sized. In C++ their underlying type is fixed to
 * int, so that any int a caller passes (an unknown dtype, for instance, which
 * the library rejects with ATTN_E_ARG) is a valid value of the parameter. */
#ifdef __cplusplus
#define ATTN_ENUM_BASE : int
#else
#define ATTN_ENUM_BASE
#endif

typedef enum attn_status ATTN_ENUM_BASE {
  ATTN_OK = 0,
  ATTN_E_ARG = 1,         /* invalid argument (null pointer, bad size, ...) */
  ATTN_E_UNSUPPORTED = 2, /* valid, but outside the supported set          */
  ATTN_E_WORKSPACE = 3,   /* workspace missing or too small                */
  ATTN_E_HIP = 4          /* a HIP launch or runtime call failed           */
} attn_status;

typedef enum attn_dtype ATTN_ENUM_BASE {
  ATTN_F32 = 0,  /* IEEE binary32                                          */
  ATTN_BF16 = 1  /* bfloat16 (upper 16 bits of binary32)                    */
} attn_dtype;

/* Static description of a status code. Never NULL. */
const char *attn_status_str(attn_status status);

/* Human-readable reason for the last nonzero status returned on the calling
 * thread ("" if none). Valid until the next call on the same thread. */
const char *attn_last_error(void);

/* ABI version, bumped on any signature or semantic change. */
int attn_abi_version(void);

/* --------------------------------------------------------------------------
 * Decode
 * --------------------------------------------------------------------------
 * Workspace bytes attn_decode needs for these sizes. `split_rows` is the same
 * value later passed to attn_decode (0 = automatic choice). The result is an
 * upper bound valid for every position_id / seq_lens. Returns 0 for invalid
 * sizes. */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int D,
                                   int max_length, int split_rows);

/* out[b,h,:] = softmax_j(scale * q[b,h,:]·K[b,g,j,:]) · V[b,g,j,:] over the
 * valid rows j of sequence b, where g = h / (Hq/Hkv) (consecutive query heads
 * share one kv head, as enable_gqa does).
 *
 *   dtype      ATTN_F32 or ATTN_BF16; q, caches and out all use it. Scores,
 *              softmax and accumulation are fp32; bf16 output is rounded to
 *              nearest even.
 *   q          [B][Hq][D]
 *   k_cache,
 *   v_cache    [B][Hkv][max_length][D]; max_length is the token stride, so
 *              passing the whole cache plus position_id is the zero-copy form
 *              of slicing it to rows [0, position_id]. Rows past the valid
 *              length are never read (they may hold anything, NaN included).
 *              The current token's K/V must already be stored at its row.
 *   out        [B][Hq][D] (the same memory as [B][Hq*D]).
 *   position_id  used when seq_lens == NULL: every sequence attends to rows
 *              [0, position_id]; requires 0 <= position_id < max_length.
 *   seq_lens   optional DEVICE array int32[B]: sequence b attends to rows
 *              [0, seq_lens[b]). Values are clamped to [0, max_length] on the
 *              device; length 0 yields a zero output row.
 *   scale      multiplier of q·k, finite and > 0 (the Python binding passes
 *              1/sqrt(D) when the caller gives none).
 *   split_rows cache rows per split-KV work item (0 = automatic). Forcing it
 *              changes only the reduction order, never the math. At most
 *              1024 splits per sequence: a smaller value is raised to
 *              ceil(max_length / 1024). For bf16 with seq_lens and
 *              2 <= B <= 256 the work is balanced over the launch instead:
 *              every wave (with Hkv a multiple of 4, every workgroup, over
 *              four neighbouring kv heads) takes an equal run of the batch's
 *              rows, across sequence ends, and split_rows is the least run
 *              (rounded up to whole wave tiles of 4096 / D rows).
 *   workspace  device scratch of at least
 *              attn_decode_workspace_bytes(B,Hq,Hkv,D,max_length,split_rows)
 *              bytes, 256-byte aligned, for the per-split partial results; no
 *              initial contents required, contents undefined after the call.
 *              Calls that may overlap need distinct workspaces.
 * Supported: D in {64, 128}; Hq % Hkv == 0 with Hq/Hkv in {1, 2, 4, 8};
 * B, Hkv <= 65535. B == 0 is a no-op. */
attn_status attn_decode(attn_dtype dtype, const void *q, const void *k_cache,
                const void *v_cache, void *out, int B, int Hq, int Hkv, int D,
                int max_length, int position_id, const int32_t *seq_lens,
                float scale, int split_rows, void *workspace,
                size_t workspace_bytes, void *stream);

/* Fused append + decode: stores the current token's K/V into the caches and
 * attends to it in the same launch sequence (one split launch, plus the
 * combine launch when a sequence has several splits). The pages write k_new
 * and v_new into the static cache at position_id and then run the attention
 * over rows [0, position_id] ("MiniCPM4 forward_step Attention Performance
 * Fix", §4.1, the patched forward_step: cache update, then SDPA over the
 * slice); this call does both.
 *
 *   k_new,
 *   v_new      [B][Hkv][D], same dtype as q; not modified.
 *   k_cache,
 *   v_cache    as for attn_decode, but written: row r_b of sequence b, with
 *              r_b = position_id (seq_lens == NULL) or seq_lens[b] - 1 (after
 *              the clamp to [0, max_length]; a sequence of length 0 gets no
 *              append), receives k_new[b] / v_new[b] for every kv head.
 *              Other rows are not written.
 * Every other argument, the result and the supported set are those of
 * attn_decode: the output equals attn_decode on the caches after the append
 * (the appended row's values are read from k_new / v_new, so the cache write
 * and the reads of that row do not race). k_new / v_new must not alias the
 * caches or out. ATTN_E_ARG if B > 0 and k_new or v_new is NULL or not
 * 16-byte aligned. */
attn_status attn_decode_append(attn_dtype dtype, const void *q, const void *k_new,
                       const void *v_new, void *k_cache, void *v_cache,
                       void *out, int B, int Hq, int Hkv, int D, int max_length,
                       int position_id, const int32_t *seq_lens, float scale,
                       int split_rows, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Fused rotary embedding + append + decode. The patched forward_step of
 * "MiniCPM4 forward_step Attention Performance Fix" (§4.1) rotates the
 * current token's query and key with its position embedding (cos, sin) by
 * apply_rotary_pos_emb before the cache write and the attention; the page
 * does not spell that function out. This call uses the rotate-half
 * convention: for each head's row x of length D, element j is paired with
 * j + D/2 and
 *   x'_j = x_j·cos_j − x_{j+D/2}·sin_j        (j < D/2)
 *   x'_j = x_j·cos_j + x_{j−D/2}·sin_j        (j ≥ D/2),
 * computed in fp32 and rounded once to the storage type.
 *
 *   rope_cos,
 *   rope_sin   fp32 [B][D], 16-byte aligned: the cos / sin row of sequence
 *              b's current position (the same for every head); not modified.
 * q and k_new[b] are rotated with row b; k_cache row r_b receives the rotated
 * key and v_new unchanged, and the rotated query attends. Everything else is
 * attn_decode_append. ATTN_E_ARG if B > 0 and a table pointer is NULL or
 * misaligned. */
attn_status attn_decode_append_rope(attn_dtype dtype, const void *q, const void *k_new,
                            const void *v_new, const float *rope_cos,
                            const float *rope_sin, void *k_cache, void *v_cache,
                            void *out, int B, int Hq, int Hkv, int D,
                            int max_length, int position_id,
                            const int32_t *seq_lens, float scale, int split_rows,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

/* Page layouts of attn_decode_paged and attn_prefill_paged. */
typedef enum attn_page_layout ATTN_ENUM_BASE {
  ATTN_PAGES_TOKEN_MAJOR = 0, /* page [page_size][Hkv][D]                  */
  ATTN_PAGES_HEAD_MAJOR = 1   /* page [Hkv][page_size][D]                  */
} attn_page_layout;

/* Decode over a paged KV cache. The cache of a sequence is a list of pages
 * (the block-table indirection of paged serving caches). Within a page the
 * rows are token-major, as the prefix cache of "step14_3 — batched attention:
 * removing the per-head Python loop" (problem section) stores K and V with
 * the head after the token, or head-major (each head's rows contiguous, which
 * streams like the static cache). The result equals attn_decode on the
 * contiguous cache gathered from the pages.
 *
 *   dtype        ATTN_BF16 only.
 *   k_pages,
 *   v_pages      ATTN_PAGES_TOKEN_MAJOR: [num_pages][page_size][Hkv][D], row r
 *                of kv head g of sequence b is k_pages[block_table[b][r /
 *                page_size]][r % page_size][g][:]; ATTN_PAGES_HEAD_MAJOR:
 *                [num_pages][Hkv][page_size][D], the same row is
 *                k_pages[...][g][r % page_size][:]. Pages a sequence does not
 *                reach are never read; rows past its length in its last page
 *                may hold anything.
 *   page_layout  ATTN_PAGES_TOKEN_MAJOR or ATTN_PAGES_HEAD_MAJOR.
 *   block_table  DEVICE int32 [B][max_blocks]; entries are clamped to
 *                [0, num_pages) on the device (so a bad entry reads a wrong
 *                page, never outside the pages).
 *   position_id, seq_lens, scale, split_rows, workspace, q, out: as for
 *                attn_decode with max_length = max_blocks * page_size (the
 *                workspace size is attn_decode_workspace_bytes(B, Hq, Hkv, D,
 *                max_blocks * page_size, split_rows)). split_rows is rounded up
 *                to a multiple of the kernel's wave tile (4096 / D rows).
 * Supported: D in {64, 128}; page_size a multiple of 4096 / D (32 rows at
 * D = 128, 64 at D = 64) up to 65536; Hq/Hkv in {1, 2, 4, 8}; B, Hkv <=
 * 65535; max_blocks * page_size < 2^31. ATTN_E_ARG for page_size, max_blocks
 * or num_pages < 1, an unknown page_layout or a null block_table with B > 0. */
attn_status attn_decode_paged(attn_dtype dtype, const void *q, const void *k_pages,
                      const void *v_pages, const int32_t *block_table,
                      int max_blocks, int page_size, int num_pages,
                      attn_page_layout page_layout, void *out,
                      int B, int Hq, int Hkv, int D, int position_id,
                      const int32_t *seq_lens, float scale, int split_rows,
                      void *workspace, size_t workspace_bytes, void *stream);

/* --------------------------------------------------------------------------
 * Prefill
 * --------------------------------------------------------------------------
 * New token i (0 <= i < Lq) sits at cache row prefix_len + i and attends to
 * rows [0, prefix_len + i] (the causal mask aligned to the bottom-right; with
 * prefix_len == 0 it is the ordinary causal mask).
 *
 *   dtype      ATTN_BF16 (bf16 inputs, bf16 matrix cores, fp32 softmax and
 *              accumulation, probabilities rounded to bf16 before ·V, bf16
 *              output rounded to nearest even).
 *   q          [B][Hq][Lq][D]
 *   k_cache,
 *   v_cache    [B][Hkv][max_length][D]; rows [0, prefix_len + Lq) must hold
 *              the prefix and the new tokens' K/V; later rows are never read.
 *   out        [B][Hq][Lq][D]
 *   scale      finite and > 0 (binding default 1/sqrt(D)).
 * Requires 0 <= prefix_len, 0 <= Lq, prefix_len + Lq <= max_length.
 * Supported: D in {64, 128}; Hq % Hkv == 0; B, Hq <= 65535;
 * (prefix_len + Lq) * 2 * D < 2^31 (one kv head's rows are addressed with
 * 32-bit byte offsets; ATTN_E_UNSUPPORTED beyond). Lq == 0 or B == 0 is a
 * no-op. */
attn_status attn_prefill(attn_dtype dtype, const void *q, const void *k_cache,
                 const void *v_cache, void *out, int B, int Hq, int Hkv, int D,
                 int max_length, int Lq, int prefix_len, float scale,
                 void *stream);

/* Prefill against a paged prefix cache: the tutorial's prefix cache ("step14_3
 * — batched attention: removing the per-head Python loop", problem section)
 * keeps K and V token-major, [total_len, heads, d_head]; here the cache of
 * sequence b is the list of pages block_table[b][.], as for
 * attn_decode_paged. The result equals attn_prefill on the contiguous cache
 * gathered from the pages (rows [0, prefix_len + Lq) of each sequence, which
 * must already hold the new tokens' K and V).
 *
 *   k_pages, v_pages, block_table, page_layout, max_blocks, num_pages: as
 *                for attn_decode_paged; rows past prefix_len + Lq are never
 *                read (they may hold anything).
 *   q, out, B, Hq, Hkv, Lq, prefix_len, scale: as for attn_prefill, with
 *                max_length = max_blocks * page_size.
 * Supported: ATTN_BF16, D in {64, 128}; page_size a multiple of the kernel's
 * key tile, 4096 / D rows (64 at D = 64, 32 at D = 128), up to 65536;
 * max_blocks * page_size < 2^31. ATTN_E_UNSUPPORTED for another page_size;
 * ATTN_E_ARG as attn_decode_paged for the table arguments. */
attn_status attn_prefill_paged(attn_dtype dtype, const void *q, const void *k_pages,
                       const void *v_pages, const int32_t *block_table,
                       int max_blocks, int page_size, int num_pages,
                       attn_page_layout page_layout, void *out, int B, int Hq, int Hkv, int D,
                       int Lq, int prefix_len, float scale, void *stream);

/* --------------------------------------------------------------------------
 * Top-k sparse attention
 * --------------------------------------------------------------------------
 * For every row i of every (b, h): s_ij = Σ_d q[i,d]·k[j,d] (no scale), the
 * set S_i = the topk indices j with the largest s_ij (equal scores: the lower
 * index first), out[i,:] = Σ_{j∈S_i} s_ij · v[j,:]. Unselected j contribute
 * exactly zero; no softmax.
 *
 * Scores and the output sum are accumulated in fp64 (every fp32·fp32 product
 * is exact in fp64) and the selection is made on the fp64 scores; the output
 * is rounded once to fp32.
 *
 *   q, k, v, out  fp32 [b][h][n][d]
 *   idx_out       optional int32 [b][h][n][topk] (NULL to skip): the selected
 *                 indices of each row in ascending order.
 * Supported: d == 64; 1 <= n <= 1024; 1 <= topk <= n; b, h <= 65535 and
 * b·h·ceil(n/16) <= 2^23 (one workgroup per 16 rows). b == 0 or h == 0 is a
 * no-op. Inputs must be finite (a NaN or infinite input leaves the
 * selection unspecified). */
attn_status attn_topk(const float *q, const float *k, const float *v, float *out,
              int32_t *idx_out, int b, int h, int n, int d, int topk,
              void *stream);

/* Decoder-causal top-k sparsified scores.
 * Source: "c2psa multi-head self-attention high-concurrency inference",
 * further thoughts (in a decoder a query attends only to the tokens on its
 * left and keeps its most recent k/2 tokens), applied to the scores of core
 * implementation §2. The pages give no more of the rule; this library reads
 * it as: for every (b, h) and query row i, the candidates are the keys
 * j <= i (its own token included), s_ij = Σ_d q[i,d]·k[j,d] with no scale;
 *   - if i+1 <= topk, S_i = {0, ..., i} (every candidate);
 *   - else, with r = floor(topk/2), S_i = {i-r+1, ..., i} (kept whatever
 *     their scores) plus the topk-r keys j <= i-r with the largest s_ij
 *     (equal scores: the lower index first);
 * out[i,:] = Σ_{j∈S_i} s_ij · v[j,:]; no softmax.
 *
 * Arguments, layouts, precision, limits and errors are those of attn_topk.
 * idx_out (optional) [b][h][n][topk] receives S_i in ascending order,
 * followed by -1 in the topk - |S_i| slots of rows with i+1 < topk. */
attn_status attn_topk_causal(const float *q, const float *k, const float *v, float *out,
                     int32_t *idx_out, int b, int h, int n, int d, int topk,
                     void *stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): attn_decode with the split partials kept in a static scratch
 * array of the library instead of a caller workspace. Arguments, result and
 * supported set are attn_decode's, without workspace / workspace_bytes.
 *
 * - The library holds one scratch array of 64 MiB on every GPU it runs on,
 *   from the first call on that GPU until the process ends; this call itself
 *   allocates nothing.
 * - Sizes whose split partials need more than 64 MiB
 *   (attn_decode_workspace_bytes(B, Hq, Hkv, D, max_length, split_rows) >
 *   64 MiB) return ATTN_E_WORKSPACE before any launch.
 * - Every call on one GPU uses that GPU's same array: calls that may overlap
 *   on one GPU (different streams, or host threads racing on one stream)
 *   race on the partials and give wrong results. Serialise them. No initial
 *   contents are needed; the array keeps the last call's contents.
 * - The current device must be the stream's device (ATTN_E_ARG otherwise;
 *   NULL = the null stream of the current device). */
attn_status attn_decode_noalloc(attn_dtype dtype, const void *q,
                                const void *k_cache, const void *v_cache,
                                void *out, int B, int Hq, int Hkv, int D,
                                int max_length, int position_id,
                                const int32_t *seq_lens, float scale,
                                int split_rows, void *stream);

/* Streaming-read probe (a measurement aid, not part of the attention path):
 * reads `bytes` of device memory at src once, with 16-byte non-temporal
 * loads, to measure the read bandwidth the memory system actually delivers,
 * the context for the decode kernels' bandwidth.
 *
 *   src         device, 16-byte aligned, `bytes` readable (may be NULL when
 *               bytes = 0); bytes a multiple of 16.
 *   workgroups  in [1, 65536]; workgroup w reads the 16-byte words
 *               [w*per, min((w+1)*per, bytes/16)), per = ceil(bytes/16 /
 *               workgroups).
 *   sink        device, 16-byte aligned, sink_bytes >= 16 * workgroups;
 *               receives in sink[w] (four uint32) the XOR of the words
 *               workgroup w read (zero for an empty range), so that no load
 *               can be dropped and the coverage can be checked.
 * Errors: ATTN_E_ARG for a size, alignment or pointer outside the above. */
attn_status attn_read_probe(const void *src, size_t bytes, void *sink,
                    size_t sink_bytes, int workgroups, void *stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* ATTN_H */
