/*
 * attn_mi355x.h -- C ABI of a small attention library for AMD Instinct MI355X
 * (gfx950 / CDNA4): grouped-query attention over a KV cache (decode, also over
 * FP8 caches and fused with the new token's cache write; causal prefill, also
 * after a cached prefix), multi-head latent attention (MLA) decode and causal
 * prefill over a latent cache, and the cache write itself.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or synchronises: it validates its arguments, then
 *    enqueues kernels on `stream` (a hipStream_t passed as void*, NULL = the
 *    default stream) and returns.  Results are ready when the stream is.
 *  - All tensors are dense and row-major (C order) with the shapes given below.
 *  - Validation runs before any HIP call.  A call that returns an error status
 *    has enqueued nothing, and attn_last_error() (thread-local) describes why.
 *    ATTN_ERR_HIP is returned when the HIP runtime itself fails (no device,
 *    launch failure); no error is ever thrown across the ABI.
 *  - cache_lens[b] (int32, device memory) is the number of valid cached tokens
 *    of sequence b, INCLUDING the newest token: decode attends to positions
 *    t in [0, cache_lens[b]).  Values are clamped to [0, T_max] on the device
 *    (they are not checked on the host, which would need a synchronisation).
 *    A length of 0 yields an all-zero output row.  Cache slots at or beyond the
 *    length are never read, so they may hold anything (including NaN).
 *  - softmax_scale <= 0 selects the default: 1/sqrt(head_dim) for GQA and
 *    1/sqrt(nope_head_dim + rope_dim) for MLA.
 *  - Accumulation is fp32.  bf16 inputs are read as stored; softmax statistics,
 *    partial results and the merge are fp32.
 *  - Calls are reentrant; concurrent calls must not share a workspace.
 *
 * Head grouping (GQA-G): Hq query heads are split into Hkv = G contiguous
 * groups of n_rep = Hq/Hkv heads; query head h reads KV head floor(h/n_rep).
 * Hkv = Hq is MHA and Hkv = 1 is MQA.  Source: the "模型架构｜MQA & GQA 调研"
 * page (section Grouped-query attention, and the repeat_kv / Attention.forward
 * listing in its code section, whose expand-then-reshape gives the contiguous
 * grouping).  A group count that does not divide Hq is an error and is never
 * rounded ("MHA, MQA và GQA" e-book, third simulator step).
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 1

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL                        */
  ATTN_ERR_SHAPE = 2,       /* a size is <= 0, out of range, or inconsistent     */
  ATTN_ERR_GROUPS = 3,      /* Hkv does not divide Hq                            */
  ATTN_ERR_UNSUPPORTED = 4, /* head size / dtype combination not built           */
  ATTN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required           */
  ATTN_ERR_HIP = 6          /* the HIP runtime reported an error                 */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Version of this ABI (ATTN_ABI_VERSION of the built library). */
int attn_abi_version(void);

/* Short static description of a status code. */
const char* attn_status_string(attn_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* attn_last_error(void);

/* ------------------------------------------------------------------------ */
/* GQA / MQA / MHA decode: one new query token per sequence against its cache.
 *
 * Computes, for every sequence b and query head h (g = floor(h / (Hq/Hkv))):
 *   out[b,h,:] = sum_{t < L_b} softmax_t(scale * q[b,h,:] . k_cache[b,t,g,:]) v_cache[b,t,g,:]
 * i.e. the score / fp32-softmax / weighted-sum core of Attention.forward on the
 * "模型架构｜MQA & GQA 调研" page (code section) for one query position, after
 * the new token has been written to the cache.
 *
 *   q          [B, Hq, head_dim]          in_dtype
 *   k_cache    [B, T_max, Hkv, head_dim]  in_dtype   (the page's cache layout)
 *   v_cache    [B, T_max, Hkv, head_dim]  in_dtype
 *   cache_lens [B]                        int32
 *   out        [B, Hq, head_dim]          out_dtype
 *
 * Supported: in_dtype ATTN_BF16 with head_dim in {64, 96, 128} and
 * Hq/Hkv <= 64; in_dtype ATTN_F32 with head_dim in {64, 96, 128} and
 * Hq/Hkv <= 16.  out_dtype ATTN_F32 or ATTN_BF16.
 *
 * Work is cut into units: chunks of split_tokens cached positions of one
 * (sequence, KV head).  A workgroup reads a unit's K/V rows once for all Hq/Hkv
 * query heads of the group.  Sequences of one chunk are written directly; the
 * chunks of longer ones are combined by their log-sum-exp in a second, small
 * kernel on the same stream.  Batches of up to 1024 sequences whose
 * B * Hkv * ceil(T_max / chunk) blocks outnumber the 256 compute units run the
 * units through a device-wide queue taken by the resident workgroups (planned
 * on the device from cache_lens, so the host never reads the lengths); other
 * batches launch one workgroup per unit.  split_tokens = 0 lets the library choose the
 * chunk from the sizes; otherwise it is a multiple of 64 in [64, 65536].  The
 * result does not depend on the chunk beyond fp32 rounding.
 *
 * workspace: device memory of at least attn_decode_gqa_workspace_bytes(...)
 * bytes for the same arguments, 256-byte aligned.  Its first 4 bytes are the
 * work-queue counter: they must be zero before the first call that uses the
 * workspace (e.g. allocate it zero-filled), and every call leaves them zero, so
 * any later call whose size needs fit may reuse it as is.  The rest needs no
 * initialisation.  One workspace per concurrent call: calls that overlap in
 * time on one workspace race.
 */
size_t attn_decode_gqa_workspace_bytes(int B, int Hq, int Hkv, int head_dim, int T_max,
                                       int split_tokens);

attn_status attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* cache_lens, void* out, int B, int Hq, int Hkv,
                            int head_dim, int T_max, float softmax_scale, attn_dtype in_dtype,
                            attn_dtype out_dtype, int split_tokens, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* GQA decode that allocates nothing: attn_decode_gqa without a workspace.
 *
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The same computation,
 * kernels and arguments as attn_decode_gqa, minus workspace / workspace_bytes:
 * the partial results and the work-queue counter live in a scratch array of
 * ATTN_NOALLOC_SCRATCH_BYTES bytes that the library's code object holds in
 * device memory, one copy per device, kept until the process ends.  Its device
 * address is looked up on the first call on each device (a runtime query, no
 * allocation); each call first zeroes its queue counter with a one-thread
 * kernel on `stream`, then runs the decode.  The call allocates and frees
 * nothing.
 *
 * Sizes whose attn_decode_gqa_workspace_bytes(...) exceeds
 * ATTN_NOALLOC_SCRATCH_BYTES return ATTN_ERR_WORKSPACE and enqueue nothing
 * (the Llama-3-8B decode shape, B 32 x Hkv 8 x T_max 8192, needs about 8.5 MB).
 * Every call on one device shares that device's scratch and leaves the last
 * call's contents in it: calls that overlap in time on one device (different
 * streams, or threads) race and must be serialised by the caller.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

attn_status attn_decode_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* cache_lens, void* out, int B, int Hq, int Hkv, int head_dim,
                                    int T_max, float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype,
                                    int split_tokens, void* stream);

/* ------------------------------------------------------------------------ */
/* GQA decode over caches stored as 8-bit floats (OCP FP8 E4M3).
 *
 *   K[b,t,g,:] = k_scale * e4m3(k_cache[b,t,g,:]),  V likewise with v_scale,
 *   out[b,h,:] = sum_{t<L_b} softmax_t(scale * q[b,h,:] . K[b,t,g,:]) V[b,t,g,:]
 *
 * The same attention as attn_decode_gqa over caches of half the bytes: the fp8
 * number type of the "MHA, MQA và GQA" e-book's simulator configuration (8 bits
 * per cached number).  The pages give no quantisation scheme; the one taken here is one
 * byte per element in the OCP FP8 E4M3 format (sign, 4 exponent bits with bias
 * 7, 3 mantissa bits, largest finite 448; the byte 0x7F/0xFF is NaN) and one
 * fp32 scale per cache.  Encoding the cache is the caller's.  The codes are
 * widened to bf16 exactly; q is bf16; scores, softmax and accumulation are as
 * in attn_decode_gqa.
 *
 *   q [B, Hq, 128] bf16;  k_cache, v_cache [B, T_max, Hkv, 128] one byte each;
 *   k_scale, v_scale > 0 and finite (else ATTN_ERR_SHAPE);  cache_lens, out,
 *   split_tokens, workspace (attn_decode_gqa_workspace_bytes) as attn_decode_gqa
 *
 * split_tokens = 0 chooses a chunk a quarter longer than attn_decode_gqa's for
 * the same sizes (at least 64 positions longer, a multiple of 64, at most 1024;
 * 640 where attn_decode_gqa takes 512), so the workspace that
 * attn_decode_gqa_workspace_bytes gives for split_tokens = 0 always suffices.
 *
 * head_dim must be 128 (else ATTN_ERR_UNSUPPORTED); Hq/Hkv up to 64.
 */
attn_status attn_decode_gqa_fp8kv(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                                  float v_scale, const int32_t* cache_lens, void* out, int B, int Hq, int Hkv,
                                  int head_dim, int T_max, float softmax_scale, attn_dtype out_dtype, int split_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* GQA decode over caches stored as signed 4-bit integers with one scale per row.
 *
 *   K[b,t,g,2i]   = k_scales[b,g,t] * int4(low nibble of k_codes[b,g,t,i]),
 *   K[b,t,g,2i+1] = k_scales[b,g,t] * int4(high nibble of k_codes[b,g,t,i]),
 *   V likewise, and out is attn_decode_gqa over K and V.
 *
 * The int4 number type of the "MHA, MQA và GQA" e-book's simulator
 * configuration, where a number takes half a byte; the e-book gives no layout
 * or scale.  The reading taken: two's-complement codes in [-8, 7], two per
 * byte with the even element in the low nibble, and one fp32 scale per cached
 * row (one KV head of one position), so a row of 128 elements is 64 bytes of
 * codes plus 4 bytes of scale.  The codes and scales are stored head-major
 * (each KV head's positions contiguous), so a head's 64-byte rows fill whole
 * memory lines.  Encoding the cache is the caller's.  Each code
 * c enters the bf16 MFMA as the exact value 136 + c and the offset is removed
 * in fp32 after the products; q is bf16; scores, softmax and accumulation are
 * as in attn_decode_gqa.
 *
 *   q [B, Hq, 128] bf16;  k_codes, v_codes [B, Hkv, T_max, 64] bytes (16-byte
 *   aligned);  k_scales, v_scales [B, Hkv, T_max] fp32 (4-byte aligned; NULL
 *   is ATTN_ERR_NULL);  cache_lens, out, split_tokens, workspace
 *   (attn_decode_gqa_workspace_bytes) as attn_decode_gqa
 *
 * head_dim must be 128 (else ATTN_ERR_UNSUPPORTED); Hq/Hkv up to 64.  Rows at
 * or past cache_lens[b] are not read (codes or scales).
 */
attn_status attn_decode_gqa_int4kv(const void* q, const void* k_codes, const void* v_codes, const float* k_scales,
                                   const float* v_scales, const int32_t* cache_lens, void* out, int B, int Hq, int Hkv,
                                   int head_dim, int T_max, float softmax_scale, attn_dtype out_dtype,
                                   int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* GQA decode step with the new token's K/V: append and attend in one call.
 *
 *   L = cache_lens[b] (positions cached before this token, clamped to [0, T_max])
 *   out[b,h,:] = softmax over { k_cache[b,t,g] (t < L), k_new[b,g] } of
 *                scale * q[b,h,:] . key, applied to the matching V rows
 *   k_cache[b,L,g,:] = k_new[b,g,:], v_cache[b,L,g,:] = v_new[b,g,:]  when L < T_max
 *
 * This is one decode iteration of Attention.forward on the "模型架构｜MQA & GQA
 * 调研" page (code section) with start_pos = L: the new token's K/V rows are
 * written at start_pos and the query attends to the first start_pos + 1 rows.
 * The result equals attn_cache_append followed by attn_decode_gqa with
 * cache_lens + 1 (up to rounding: the new token's probability is not rounded
 * to bf16), without the separate launch.  The cache rows below L are read, row
 * L is written after they have been read; cache_lens itself is not changed (the
 * caller advances it).  When L = T_max the new token is attended to but not
 * stored.  Rotary embedding is the caller's (applied to q and k_new before).
 *
 *   q [B, Hq, head_dim], k_new, v_new [B, Hkv, head_dim] (in_dtype)
 *   k_cache, v_cache, cache_lens, out, T_max, split_tokens: as attn_decode_gqa
 *   workspace: at least attn_decode_gqa_append_workspace_bytes(...) bytes,
 *   256-byte aligned, the first 4 bytes zero before first use (as for
 *   attn_decode_gqa; every call leaves them zero)
 *
 * Supported shapes, errors and ownership as attn_decode_gqa, plus
 * ATTN_ERR_NULL for a NULL k_new or v_new.
 */
size_t attn_decode_gqa_append_workspace_bytes(int B, int Hq, int Hkv, int head_dim, int T_max,
                                              int split_tokens);

attn_status attn_decode_gqa_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                   void* v_cache, const int32_t* cache_lens, void* out, int B, int Hq, int Hkv,
                                   int head_dim, int T_max, float softmax_scale, attn_dtype in_dtype,
                                   attn_dtype out_dtype, int split_tokens, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ------------------------------------------------------------------------ */
/* GQA decode over paged K/V caches (a page pool and a block table).
 *
 *   T_max = page_size * max_pages_per_seq, L = cache_lens[b] clamped to [0, T_max];
 *   K[b,t,g,:] = k_pages[block_table[b * max_pages_per_seq + t / page_size], t % page_size, g, :]
 *   (V likewise from v_pages), and out is attn_decode_gqa over those rows.
 *
 * The pages mention paging only as the serving system's cost of handing out
 * cache memory to many requests (the "MHA, MQA và GQA" interactive e-book, whose
 * byte counts leave it out on purpose), and define no scheme.  Reading: the common
 * block-table layout -- fixed-size pages in one pool, per sequence a row of
 * page numbers in position order; a page holds page_size consecutive
 * positions, each row the same [Hkv, head_dim] layout as a contiguous cache.
 * Same arithmetic and results as attn_decode_gqa on the gathered caches.
 *
 *   q           [B, Hq, head_dim]                       bf16
 *   k_pages, v_pages [n_pages, page_size, Hkv, head_dim] bf16
 *   block_table [B, max_pages_per_seq] int32, device memory: entries for the
 *               pages below ceil(L / page_size) are read, each clamped to
 *               [0, n_pages); unused entries may hold anything
 *   cache_lens  [B] int32        out [B, Hq, head_dim] out_dtype
 *
 * Supported: in_dtype ATTN_BF16, head_dim 64/96/128, page_size a multiple of 32
 * (else ATTN_ERR_UNSUPPORTED), split_tokens 0 or a multiple of 64 up to 1024.
 * workspace: attn_decode_gqa_workspace_bytes(B, Hq, Hkv, head_dim,
 * page_size * max_pages_per_seq, split_tokens) bytes, 256-byte aligned; its
 * first 4 bytes zero before the first call (every call leaves them zero).
 * Errors as attn_decode_gqa, plus ATTN_ERR_NULL for a NULL block_table and
 * ATTN_ERR_SHAPE for non-positive page counts.
 */
attn_status attn_decode_gqa_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                                  const int32_t* cache_lens, void* out, int B, int Hq, int Hkv, int head_dim,
                                  int page_size, int n_pages, int max_pages_per_seq, float softmax_scale,
                                  attn_dtype in_dtype, attn_dtype out_dtype, int split_tokens, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* GQA decode step with the new token over paged K/V caches: attn_decode_gqa_append
 * with the caches as a page pool and a block table (attn_decode_gqa_paged).
 *
 *   T_max = page_size * max_pages_per_seq, L = cache_lens[b] clamped to [0, T_max];
 *   out[b,h,:] = softmax over { K[b,t,g] (t < L), k_new[b,g] } of
 *                scale * q[b,h,:] . key, applied to the matching V rows
 *   when L < T_max: row L % page_size of page P = block_table[b * max_pages_per_seq + L / page_size]
 *   (clamped to [0, n_pages)) gets k_new[b,g,:] in k_pages[P, L % page_size, g, :] and
 *   v_new[b,g,:] in v_pages likewise
 *
 * One decode iteration of Attention.forward on the "模型架构｜MQA & GQA 调研" page
 * (code section) with start_pos = L, over the block-table reading of a paged
 * cache that attn_decode_gqa_paged states.  The caller allocates the page that
 * holds position L (its block-table entry must name it before the call); rows
 * below L are read, the row of position L is written after they have been read,
 * and no other row of either pool is touched.  Bit for bit attn_decode_gqa_append
 * over the gathered caches, with the new row landing in its page.
 *
 *   q [B, Hq, head_dim], k_new, v_new [B, Hkv, head_dim]   bf16
 *   k_pages, v_pages, block_table, cache_lens, out, page sizes, split_tokens:
 *     as attn_decode_gqa_paged (the pools are written, so not const)
 *   workspace: attn_decode_gqa_append_workspace_bytes(B, Hq, Hkv, head_dim,
 *     page_size * max_pages_per_seq, split_tokens) bytes, 256-byte aligned,
 *     its first 4 bytes zero before the first call (every call leaves them zero)
 *
 * Supported shapes and errors as attn_decode_gqa_paged, plus ATTN_ERR_NULL for
 * a NULL k_new or v_new and ATTN_ERR_UNSUPPORTED for rows not 16-byte aligned.
 */
attn_status attn_decode_gqa_paged_append(const void* q, const void* k_new, const void* v_new, void* k_pages,
                                         void* v_pages, const int32_t* block_table, const int32_t* cache_lens,
                                         void* out, int B, int Hq, int Hkv, int head_dim, int page_size, int n_pages,
                                         int max_pages_per_seq, float softmax_scale, attn_dtype in_dtype,
                                         attn_dtype out_dtype, int split_tokens, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* GQA decode over paged FP8 caches.
 *
 * attn_decode_gqa_fp8kv over caches kept as page pools and a block table, as
 * attn_decode_gqa_paged keeps bf16 caches: the e-book "MHA, MQA và GQA" offers
 * the fp8 number type, and leaves out the paging cost of serving, whose layout
 * is the one read by attn_decode_gqa_paged (position t of sequence b is row
 * t mod page_size of page block_table[b][t / page_size]).
 *
 *   q [B, Hq, 128] bf16;  k_pages, v_pages [n_pages, page_size, Hkv, 128] one
 *   byte each (OCP FP8 E4M3 codes, K = k_scale * e4m3(code), V likewise);
 *   block_table [B, max_pages_per_seq] int32 (entries clamped to the pool);
 *   cache_lens [B] (clamped to page_size * max_pages_per_seq);  out [B, Hq, 128]
 *   of out_dtype;  workspace: attn_decode_gqa_workspace_bytes(B, Hq, Hkv, 128,
 *   page_size * max_pages_per_seq, split_tokens).
 *
 * The results are bit for bit those of attn_decode_gqa_fp8kv over the caches the
 * block table gathers (same chunk).  Errors: as attn_decode_gqa_fp8kv and
 * attn_decode_gqa_paged (NULL table ATTN_ERR_NULL, page_size not a multiple of
 * 32 or split_tokens above 1024 ATTN_ERR_UNSUPPORTED, scales not positive and
 * finite ATTN_ERR_SHAPE).
 */
attn_status attn_decode_gqa_paged_fp8kv(const void* q, const void* k_pages, const void* v_pages, float k_scale,
                                        float v_scale, const int32_t* block_table, const int32_t* cache_lens,
                                        void* out, int B, int Hq, int Hkv, int head_dim, int page_size, int n_pages,
                                        int max_pages_per_seq, float softmax_scale, attn_dtype out_dtype,
                                        int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Causal GQA prefill (no cached prefix): query i attends to keys j <= i.
 *
 *   out[b,i,h,:] = sum_{j <= i} softmax_j(scale * q[b,i,h,:] . k[b,j,g,:]) v[b,j,g,:]
 *
 * This is Attention.forward on the "模型架构｜MQA & GQA 调研" page with
 * start_pos = 0 and the additive causal mask, equivalently the
 * scaled_dot_product_attention(is_causal=True) call of the MultiHeadLatentAttention
 * listing on the qqstock DeepSeek MLA article.  QK^T and PV run on bf16 MFMA with
 * fp32 accumulation; the probabilities are rounded to bf16 before PV, as the
 * page's softmax(...).type_as(xq) does.
 *
 *   q   [B, S, Hq, head_dim]   bf16          k, v [B, S, Hkv, head_dim]   bf16
 *   out [B, S, Hq, head_dim]   out_dtype (ATTN_BF16 or ATTN_F32)
 *
 * Supported: in_dtype ATTN_BF16, head_dim 64, 96 or 128, any S >= 1,
 * Hq/Hkv any divisor split.  No workspace.
 */
attn_status attn_prefill_gqa_causal(const void* q, const void* k, const void* v, void* out, int B,
                                    int S, int Hq, int Hkv, int head_dim, float softmax_scale,
                                    attn_dtype in_dtype, attn_dtype out_dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Causal GQA prefill after a cached prefix (chunked prefill).
 *
 *   P = start_pos[b], n = q_lens[b] (q_lens NULL: n = S), for i < n:
 *   out[b,i,h,:] = sum_{j <= P+i} softmax_j(scale * q[b,i,h,:] . k[b,j,g,:]) v[b,j,g,:]
 *   out[b,i,h,:] = 0 for n <= i < S.
 *
 * This is Attention.forward on the "模型架构｜MQA & GQA 调研" page with
 * start_pos > 0: the new tokens' K/V rows have been written into the cache at
 * positions start_pos .. start_pos + seqlen - 1 before the call, the keys are
 * the first start_pos + seqlen cache rows, and the causal mask is aligned to
 * the bottom right, so new token i (at position P + i) sees every cached
 * position up to and including its own.  start_pos = 0 for every sequence is
 * attn_prefill_gqa_causal over the first S cache rows.  Same arithmetic as
 * attn_prefill_gqa_causal (bf16 MFMA, fp32 accumulation, probabilities rounded
 * to bf16 before PV).
 *
 *   q         [B, S, Hq, head_dim]      bf16 (the new tokens, padded to S)
 *   k_cache   [B, T_max, Hkv, head_dim] bf16, v_cache likewise; read only at
 *             rows 0 .. P + n - 1 of each sequence
 *   start_pos [B] int32, device memory, required; clamped to [0, T_max]
 *   q_lens    [B] int32, device memory, or NULL (all S); clamped to
 *             [0, min(S, T_max - P)]
 *   out       [B, S, Hq, head_dim]      out_dtype (ATTN_BF16 or ATTN_F32)
 *
 * All pointers are device memory owned by the caller.  Errors as for
 * attn_prefill_gqa_causal, plus ATTN_ERR_NULL for a NULL start_pos and
 * ATTN_ERR_SHAPE for T_max < 1.  The per-sequence values are not read on the
 * host (they are device memory); the kernel clamps them as stated.  No
 * workspace.
 */
attn_status attn_prefill_gqa_cached(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* start_pos, const int32_t* q_lens, void* out, int B, int S,
                                    int Hq, int Hkv, int head_dim, int T_max, float softmax_scale,
                                    attn_dtype in_dtype, attn_dtype out_dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Causal GQA prefill after a cached prefix, over a paged cache.
 *
 *   T_max = page_size * max_pages_per_seq;
 *   K[b,t,g,:] = k_pages[block_table[b * max_pages_per_seq + t / page_size], t % page_size, g, :]
 *   (V likewise from v_pages), and out is attn_prefill_gqa_cached over those rows.
 *
 * The chunked prefill of the "模型架构｜MQA & GQA 调研" page (Attention.forward
 * with start_pos > 0, the new rows already written into the cache) when the cache
 * is kept in the block-table layout that attn_decode_gqa_paged reads (the "MHA,
 * MQA và GQA" e-book names paging only as a serving cost, with no scheme).  Same
 * arithmetic and results as attn_prefill_gqa_cached on the gathered caches.
 *
 *   q            [B, S, Hq, head_dim]                     bf16 (the new tokens, padded to S)
 *   k_pages, v_pages [n_pages, page_size, Hkv, head_dim]   bf16 (16-byte aligned)
 *   block_table  [B, max_pages_per_seq] int32, device memory: entries for the
 *                pages below ceil((P + n) / page_size) are read, each clamped to
 *                [0, n_pages); unused entries may hold anything
 *   start_pos, q_lens, out: as attn_prefill_gqa_cached (clamped against T_max)
 *
 * Supported: as attn_prefill_gqa_cached, with page_size a multiple of 64 (one
 * 64-key tile per page; else ATTN_ERR_UNSUPPORTED).  Errors as
 * attn_prefill_gqa_cached, plus ATTN_ERR_NULL for a NULL block_table and
 * ATTN_ERR_SHAPE for non-positive page counts.  No workspace.
 */
attn_status attn_prefill_gqa_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                                   const int32_t* start_pos, const int32_t* q_lens, void* out, int B, int S, int Hq,
                                   int Hkv, int head_dim, int page_size, int n_pages, int max_pages_per_seq,
                                   float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Causal GQA prefill after a cached prefix that also appends the new rows.
 *
 *   P = start_pos[b], n = q_lens[b] (NULL: S), both clamped as for
 *   attn_prefill_gqa_cached; for i < n:
 *   out[b,i,h,:] = sum_{j <= P+i} softmax_j(scale * q[b,i,h,:] . key_j) val_j
 *     with key_j = k_cache[b,j,g,:] for j < P and k_new[b,j-P,g,:] for j >= P
 *     (val likewise from v_cache / v_new)
 *   k_cache[b,P+i,:,:] = k_new[b,i,:,:], v_cache[b,P+i,:,:] = v_new[b,i,:,:]
 *   out[b,i,h,:] = 0 for n <= i < S.
 *
 * The whole of Attention.forward with start_pos > 0 on the "模型架构｜MQA & GQA
 * 调研" page in one launch: the new tokens' K/V rows are written into the cache
 * at start_pos .. and the new tokens attend to the cached prefix and, causally,
 * to each other.  The kernel reads the new keys and values from k_new / v_new
 * and only rows below P from the caches, so the writes (made by the workgroups
 * of the first query head of each KV group) race with no read.  The result
 * equals attn_cache_append of (k_new, v_new) followed by
 * attn_prefill_gqa_cached (up to fp32 rounding: the first 64-key tile of the
 * new rows starts at P rather than at a multiple of 64).  Rows outside
 * [P, P + n) of the caches are untouched; start_pos and q_lens are not changed
 * (the caller advances them).
 *
 *   q             [B, S, Hq, head_dim]      bf16 (the new tokens, padded to S)
 *   k_new, v_new  [B, S, Hkv, head_dim]     bf16 (their keys and values)
 *   k_cache, v_cache [B, T_max, Hkv, head_dim] bf16, read at rows < P,
 *                 written at rows P .. P + n - 1
 *   start_pos     [B] int32, required; q_lens [B] int32 or NULL
 *   out           [B, S, Hq, head_dim]      out_dtype
 *
 * All pointers are device memory owned by the caller, 16-byte aligned; the new
 * rows must not overlap the caches.  Supported shapes and errors as for
 * attn_prefill_gqa_cached, plus ATTN_ERR_NULL for a NULL k_new or v_new.  No
 * workspace.
 */
attn_status attn_prefill_gqa_cached_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                           void* v_cache, const int32_t* start_pos, const int32_t* q_lens, void* out,
                                           int B, int S, int Hq, int Hkv, int head_dim, int T_max,
                                           float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype,
                                           void* stream);

/* ------------------------------------------------------------------------ */
/* MLA decode, absorbed form, over a latent cache plus one shared RoPE key.
 *
 * Source: qqstock DeepSeek MLA article -- sections 1 (only the low-rank latent
 * c is cached), 2 and 4 (the key up-projection W_UK is folded into the query,
 * the value up-projection W_UV is applied after attention), 3 (a separate
 * rotated key part shared by all heads), 6 (values share the latent with the
 * un-rotated key) -- and its MultiHeadLatentAttention listing, whose
 * decompress_k_nope / decompress_v_linear weights are w_uk / w_uv here and whose
 * score width nope+rope sets the default scale.  Per sequence b and head h:
 *
 *   q_lat  = [ w_uk[h]^T q_nope[b,h] ,  q_rope[b,h] ]              (r + dR wide)
 *   s_t    = scale * q_lat . [ c_kv[b,t] , k_rope[b,t] ]            t < L_b
 *   o_lat  = sum_t softmax(s)_t c_kv[b,t]                           (r wide)
 *   out[b,h] = w_uv[h] o_lat                                        (dv wide)
 *
 * which equals attention with decompressed keys [w_uk[h] c , k_rope] and values
 * w_uv[h] c.  The cache rows (c_kv, k_rope) are read once per sequence for all H
 * heads.
 *
 *   q_nope [B, H, nope_head_dim]      q_rope [B, H, rope_dim] (already rotated)
 *   w_uk   [H, nope_head_dim, kv_lora_rank]   (= decompress_k_nope.weight viewed per head)
 *   w_uv   [H, v_head_dim, kv_lora_rank]      (= decompress_v_linear.weight viewed per head)
 *   c_kv   [B, T_max, kv_lora_rank]   k_rope [B, T_max, rope_dim] (already rotated)
 *   cache_lens [B] int32              out [B, H, v_head_dim] out_dtype
 *   all of q_nope, q_rope, w_uk, w_uv, c_kv, k_rope in in_dtype (ATTN_BF16).
 *
 * Supported (attn_decode_mla_supported): in_dtype ATTN_BF16, kv_lora_rank in
 * {64, 128, 256}, rope_dim in {16, 32, 48, 64}, H <= 16; nope_head_dim a
 * multiple of 8 in [8, 256]; v_head_dim a multiple of 16 in [16, 256].  c_kv,
 * k_rope, w_uk, w_uv and out must be 16-byte aligned (else
 * ATTN_ERR_UNSUPPORTED).  One kernel
 * launch: the absorbed query, the cache pass, the merge of a sequence's chunks
 * and the W_UV product all run in it.
 * split_tokens: 0 lets the library choose the chunk length (a power of two of at
 * least 256 positions, about one chunk per compute unit of a 256-unit MI355X
 * over B * T_max; the choice, and so the workspace size, does not depend on the
 * current device); otherwise a multiple of 64 in [64, 65536].  Each (chunk,
 * sequence) is one workgroup serving all H heads; a sequence of length L uses
 * ceil(L / chunk) chunks, merged inside the same launch by the chunk that
 * finishes last.
 * workspace: at least attn_decode_mla_workspace_bytes(...) bytes, 256-byte
 * aligned: per-sequence counters of finished chunks (the first 4 * B bytes),
 * then the per-chunk partial results.  The counters must be zero before the
 * first call that uses the workspace (e.g. allocate it zero-filled) and every
 * call leaves them zero; the rest needs no initialisation.  One workspace per
 * concurrent call: calls that overlap in time on one workspace race.
 */
size_t attn_decode_mla_workspace_bytes(int B, int H, int kv_lora_rank, int rope_dim, int T_max,
                                       int split_tokens);

/* 1 if this (H, kv_lora_rank, rope_dim, in_dtype) combination is built, else 0. */
int attn_decode_mla_supported(int H, int kv_lora_rank, int rope_dim, attn_dtype in_dtype);

attn_status attn_decode_mla_absorbed(const void* q_nope, const void* q_rope, const void* w_uk,
                                     const void* w_uv, const void* c_kv, const void* k_rope,
                                     const int32_t* cache_lens, void* out, int B, int H,
                                     int nope_head_dim, int rope_dim, int v_head_dim,
                                     int kv_lora_rank, int T_max, float softmax_scale,
                                     attn_dtype in_dtype, attn_dtype out_dtype, int split_tokens,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* MLA decode over an FP8 latent cache.
 *
 *   c_kv_value[b,t,:] = c_scale * e4m3(c_kv[b,t,:]),
 *   out is attn_decode_mla_absorbed over (c_kv_value, k_rope).
 *
 * The MLA decode of the qqstock DeepSeek MLA article (sections 1 and 3: only
 * the latent c_kv and the shared rotated key part are cached) with the latent,
 * 128 of the 176 cached numbers per token at MiniMind-768's widths, stored as
 * OCP FP8 E4M3 codes with one fp32 scale per cache -- the fp8 number type of the
 * "MHA, MQA và GQA" e-book's simulator, read as in attn_decode_gqa_fp8kv.
 * k_rope stays bf16.  Encoding the cache is the caller's.  The codes are widened
 * to bf16 exactly; c_scale multiplies the latent part of the absorbed query and
 * the output, so the scores and the weighted sum see c_scale * code.
 *
 *   c_kv [B, T_max, kv_lora_rank] one byte each (16-byte aligned);
 *   c_scale > 0 and finite (else ATTN_ERR_SHAPE);  k_rope [B, T_max, rope_dim]
 *   bf16;  q_nope, q_rope, w_uk, w_uv bf16;  cache_lens, out, split_tokens,
 *   workspace (attn_decode_mla_workspace_bytes): as attn_decode_mla_absorbed
 *
 * Supported shapes and errors as attn_decode_mla_absorbed with in_dtype
 * ATTN_BF16.  Rows at or past cache_lens[b] are not read.
 */
attn_status attn_decode_mla_fp8kv(const void* q_nope, const void* q_rope, const void* w_uk, const void* w_uv,
                                  const void* c_kv, float c_scale, const void* k_rope, const int32_t* cache_lens,
                                  void* out, int B, int H, int nope_head_dim, int rope_dim, int v_head_dim,
                                  int kv_lora_rank, int T_max, float softmax_scale, attn_dtype out_dtype,
                                  int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* MLA decode over a paged FP8 latent cache.
 *
 * attn_decode_mla_fp8kv with c_kv and k_rope kept as page pools read through
 * one block table, as attn_decode_mla_paged keeps bf16 latents: the latent
 * cache of the qqstock DeepSeek MLA article (sections 1 and 3) in the fp8
 * number type of the "MHA, MQA và GQA" e-book, in the paging layout that
 * e-book leaves out of its byte counts (position t of sequence b is row
 * t mod page_size of page block_table[b][t / page_size]).
 *
 *   q_nope, q_rope, w_uk, w_uv, out, cache_lens: as attn_decode_mla_fp8kv;
 *   c_pages [n_pages, page_size, kv_lora_rank] one byte each (OCP FP8 E4M3
 *   codes, latent = c_scale * e4m3(code)), k_rope_pages [n_pages, page_size,
 *   rope_dim] bf16, block_table [B, max_pages_per_seq] int32 (entries clamped to
 *   the pool); workspace: attn_decode_mla_workspace_bytes(B, H, kv_lora_rank,
 *   rope_dim, page_size * max_pages_per_seq, split_tokens).
 *
 * The results are bit for bit those of attn_decode_mla_fp8kv over the caches the
 * block table gathers (same chunk).  Errors: as attn_decode_mla_fp8kv and
 * attn_decode_mla_paged (NULL table ATTN_ERR_NULL; page_size not a multiple of
 * 16, or a chunk spanning more than 128 pages, ATTN_ERR_UNSUPPORTED; c_scale not
 * positive and finite ATTN_ERR_SHAPE).
 */
attn_status attn_decode_mla_paged_fp8kv(const void* q_nope, const void* q_rope, const void* w_uk, const void* w_uv,
                                        const void* c_pages, float c_scale, const void* k_rope_pages,
                                        const int32_t* block_table, const int32_t* cache_lens, void* out, int B, int H,
                                        int nope_head_dim, int rope_dim, int v_head_dim, int kv_lora_rank,
                                        int page_size, int n_pages, int max_pages_per_seq, float softmax_scale,
                                        attn_dtype out_dtype, int split_tokens, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* MLA decode over paged latent caches.
 *
 *   T_max = page_size * max_pages_per_seq, L = cache_lens[b] clamped to [0, T_max];
 *   c_kv[b,t,:]   = c_pages[block_table[b * max_pages_per_seq + t / page_size], t % page_size, :]
 *   k_rope[b,t,:] = k_rope_pages[(the same page)], t % page_size, :]
 *   and out is attn_decode_mla_absorbed over those rows.
 *
 * The latent cache of the qqstock DeepSeek MLA article (sections 1 and 3: only
 * c_kv and the shared rotated key part are cached) held in the block-table
 * layout that attn_decode_gqa_paged reads (the "MHA, MQA và GQA" e-book names
 * paging only as a serving cost, with no scheme): fixed-size pages in one pool
 * per cache, per sequence a row of page numbers in position order.  Same
 * arithmetic and results as attn_decode_mla_absorbed on the gathered caches.
 *
 *   c_pages      [n_pages, page_size, kv_lora_rank]   in_dtype (16-byte aligned)
 *   k_rope_pages [n_pages, page_size, rope_dim]       in_dtype (16-byte aligned)
 *   block_table  [B, max_pages_per_seq] int32, device memory: entries for the
 *                pages below ceil(L / page_size) are read, each clamped to
 *                [0, n_pages); unused entries may hold anything
 *   q_nope, q_rope, w_uk, w_uv, cache_lens, out: as attn_decode_mla_absorbed
 *
 * Supported: the shapes of attn_decode_mla_absorbed, page_size a multiple of 16
 * (else ATTN_ERR_UNSUPPORTED); a chunk of split_tokens positions (the library's
 * choice when 0) may span at most 128 pages (else ATTN_ERR_UNSUPPORTED, with the
 * largest split_tokens that fits in the message).  workspace:
 * attn_decode_mla_workspace_bytes(B, H, kv_lora_rank, rope_dim,
 * page_size * max_pages_per_seq, split_tokens) bytes.  Errors as
 * attn_decode_mla_absorbed, plus ATTN_ERR_NULL for a NULL block_table and
 * ATTN_ERR_SHAPE for non-positive page counts.
 */
attn_status attn_decode_mla_paged(const void* q_nope, const void* q_rope, const void* w_uk, const void* w_uv,
                                  const void* c_pages, const void* k_rope_pages, const int32_t* block_table,
                                  const int32_t* cache_lens, void* out, int B, int H, int nope_head_dim, int rope_dim,
                                  int v_head_dim, int kv_lora_rank, int page_size, int n_pages, int max_pages_per_seq,
                                  float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype, int split_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* MLA decode step with the new token's latent row: append and attend in one call.
 *
 *   L = cache_lens[b] (positions cached before this token, clamped to [0, T_max])
 *   out[b,h,:] = attn_decode_mla_absorbed over { rows t < L of (c_kv, k_rope),
 *                and the new row (c_new[b], k_rope_new[b]) }
 *   c_kv[b,L,:] = c_new[b,:], k_rope[b,L,:] = k_rope_new[b,:]  when L < T_max
 *
 * One decode iteration of MLA with only the compressed latent and the rotated
 * shared key part cached (qqstock DeepSeek MLA article, sections 1 and 3): the
 * new token's rows are appended at position L and the query attends to the L + 1
 * rows.  The result equals attn_cache_append of the two rows followed by
 * attn_decode_mla_absorbed with cache_lens + 1 (up to rounding: the new token
 * is merged as one more partial), in one launch.  Rows below L are read, row L
 * is written by the workgroup that finishes the sequence after every chunk has
 * been read; cache_lens itself is not changed (the caller advances it).  When
 * L = T_max the new token is attended to but not stored.  Rotary embedding is
 * the caller's (q_rope and k_rope_new already rotated).
 *
 *   c_new [B, kv_lora_rank], k_rope_new [B, rope_dim]   in_dtype (16-byte aligned)
 *   everything else, supported shapes, errors and the workspace
 *   (attn_decode_mla_workspace_bytes): as attn_decode_mla_absorbed, plus
 *   ATTN_ERR_NULL for a NULL c_new or k_rope_new
 */
attn_status attn_decode_mla_append(const void* q_nope, const void* q_rope, const void* c_new, const void* k_rope_new,
                                   const void* w_uk, const void* w_uv, void* c_kv, void* k_rope,
                                   const int32_t* cache_lens, void* out, int B, int H, int nope_head_dim,
                                   int rope_dim, int v_head_dim, int kv_lora_rank, int T_max, float softmax_scale,
                                   attn_dtype in_dtype, attn_dtype out_dtype, int split_tokens, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* MLA causal prefill over the latent cache (absorbed form).
 *
 *   P = start_pos[b] (NULL: 0), n = q_lens[b] (NULL: S), for i < n:
 *   s_j = scale * (q_nope[b,i,h] . W_UK[h] c_kv[b,j] + q_rope[b,i,h] . k_rope[b,j])
 *   out[b,i,h,:] = W_UV[h] sum_{j <= P+i} softmax_j(s) c_kv[b,j]
 *   out[b,i,h,:] = 0 for n <= i < S.
 *
 * This is the scaled_dot_product_attention(is_causal=True) call of the
 * MultiHeadLatentAttention listing on the qqstock DeepSeek MLA article: keys
 * [W_UK c, k_rope] (k_rope shared by every head, section 3) and values W_UV c
 * rebuilt from the latent; folding W_UK into the query and applying W_UV after
 * the weighted sum (sections 2 and 4) gives the same result.  With a cached
 * prefix the causal cut is aligned to the bottom right, as for
 * attn_prefill_gqa_cached.  The default scale is 1/sqrt(nope_head_dim +
 * rope_dim), scaled_dot_product_attention's default over the listing's
 * recombined query.  Scores, softmax and accumulation in fp32 on bf16 MFMA; the
 * absorbed query, the probabilities and the latent output are rounded to bf16
 * before their MFMA products.
 *
 *   q_nope  [B, S, H, nope_head_dim]   q_rope [B, S, H, rope_dim]   bf16 (the
 *           new tokens, padded to S; q_rope already rotated)
 *   w_uk    [H, nope_head_dim, kv_lora_rank]   w_uv [H, v_head_dim, kv_lora_rank]
 *           bf16: the per-head rows of the key-nope and value up-projection
 *           weights
 *   c_kv    [B, T_max, kv_lora_rank]   k_rope [B, T_max, rope_dim]   bf16, the
 *           new tokens' rows already written at start_pos[b] ..; read only at
 *           rows 0 .. P + n - 1
 *   start_pos, q_lens  [B] int32 device memory, or NULL; clamped as for
 *           attn_prefill_gqa_cached
 *   out     [B, S, H, v_head_dim]   out_dtype (ATTN_BF16 or ATTN_F32)
 *
 * Built widths: nope 96, rope 48, v 96, kv_lora_rank 128 (MiniMind-768's MLA);
 * others return ATTN_ERR_UNSUPPORTED.  in_dtype must be ATTN_BF16.  All
 * pointers are device memory owned by the caller, 16-byte aligned.  No
 * workspace.
 */
attn_status attn_prefill_mla_causal(const void* q_nope, const void* q_rope, const void* w_uk, const void* w_uv,
                                    const void* c_kv, const void* k_rope, const int32_t* start_pos,
                                    const int32_t* q_lens, void* out, int B, int S, int H, int nope_head_dim,
                                    int rope_dim, int v_head_dim, int kv_lora_rank, int T_max, float softmax_scale,
                                    attn_dtype in_dtype, attn_dtype out_dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Cache append: write the new tokens' rows into one or two caches.
 *
 *   P = start_pos[b] (NULL: 0), n = n_new[b] (NULL: S), for i < n:
 *   cache_a[b, P + i, :] = new_a[b, i, :]   and, when row_bytes_b > 0,
 *   cache_b[b, P + i, :] = new_b[b, i, :]
 *
 * These are the cache_k / cache_v writes at start_pos .. start_pos + seqlen of
 * Attention.forward on the "模型架构｜MQA & GQA 调研" page (code section), which
 * come before the cache is read: (a, b) = (K cache, V cache) with rows of
 * Hkv * head_dim elements, or, for MLA, (c_kv, k_rope), the latent and the
 * shared rotated key that the qqstock DeepSeek MLA article caches (sections 1
 * and 3).  Rotary embedding is not applied: rows are copied as given.  After
 * the call, attn_decode_gqa with cache_lens = P + n, attn_prefill_gqa_cached,
 * attn_decode_mla_absorbed and attn_prefill_mla_causal read the new rows.
 *
 *   new_a   [B, S, row_bytes_a bytes]       cache_a [B, T_max, row_bytes_a bytes]
 *   new_b   [B, S, row_bytes_b bytes]       cache_b [B, T_max, row_bytes_b bytes]
 *           (row_bytes_b = 0: no second pair; new_b, cache_b may be NULL)
 *   start_pos, n_new  [B] int32 device memory or NULL; P clamped to [0, T_max],
 *           n to [0, min(S, T_max - P)]; rows outside [P, P + n) are untouched
 *
 * Bytes are moved as they are (any element type).  Row sizes must be
 * multiples of 16 bytes and every buffer 16-byte aligned (else
 * ATTN_ERR_UNSUPPORTED).  All pointers are device memory owned by the caller;
 * new and cache rows must not overlap.  No workspace.
 */
attn_status attn_cache_append(const void* new_a, void* cache_a, int row_bytes_a, const void* new_b, void* cache_b,
                              int row_bytes_b, const int32_t* start_pos, const int32_t* n_new, int B, int S,
                              int T_max, void* stream);

/* ------------------------------------------------------------------------ */
/* Rotary position embedding of the new tokens, fused with the cache write.
 *
 *   P = max(start_pos[b], 0) (NULL: 0), n = n_new[b] clamped to [0, S] (NULL: S);
 *   token i < n of sequence b sits at position m = P + i, and every head vector
 *   x (width d = rope_dim) of its query and key rows is rotated pair by pair:
 *     x'[2j]   = x[2j] cos(m t_j) - x[2j+1] sin(m t_j)
 *     x'[2j+1] = x[2j] sin(m t_j) + x[2j+1] cos(m t_j),   t_j = rope_base^(-2j/d)
 *   q[b,i]           <- rotated q[b,i]                (in place; q may be NULL)
 *   k_cache[b,m]     <- rotated k_new[b,i]            when m < T_max
 *                       (k_cache NULL: k_new[b,i] is rotated in place instead)
 *   x_cache[b,m]     <- x_new[b,i], bytes as given    when m < T_max and x_row_bytes > 0
 *   rows i >= n are not touched.
 *
 * The step of Attention.forward on the "模型架构｜MQA & GQA 调研" page (code
 * section) before the cache is read: apply_rotary_emb(xq, xk, freqs_cis), then
 * the cache_k / cache_v writes at start_pos.  The pages call the rotation but do
 * not print it; this is LLaMA-2's rotation (consecutive pairs as complex
 * numbers times exp(i m t_j)), whose Attention class that page prints, with
 * LLaMA's rope_base 10000 as the usual choice.  For MLA (qqstock DeepSeek MLA
 * article, sections 1 and 3, and the apply_rope call of its listing) q is
 * q_rope with Hq = H, k is the shared k_rope with Hk = 1, and x is the latent
 * c_kv row.  For GQA q is [.., Hq, head_dim], k the new K rows with Hk = Hkv and
 * x the new V rows.  Follow with attn_decode_gqa / attn_prefill_gqa_cached /
 * attn_decode_mla_absorbed / attn_prefill_mla_causal over the extended cache,
 * or rotate in place (k_cache NULL) and pass the rows to attn_decode_gqa_append,
 * attn_prefill_gqa_cached_append or attn_decode_mla_append.
 *
 * The angle m t_j and its reduction modulo 2 pi are computed in fp64, the sine
 * and cosine of the reduced angle and the rotation in fp32, and the result is
 * rounded once to dtype.
 *
 *   q       [B, S, Hq, rope_dim]  dtype, or NULL
 *   k_new   [B, S, Hk, rope_dim]  dtype, required
 *   k_cache [B, T_max, Hk, rope_dim] dtype, or NULL
 *   x_new   [B, S, x_row_bytes bytes], x_cache [B, T_max, x_row_bytes bytes]
 *           (x_row_bytes = 0: none; x needs k_cache)
 *   start_pos, n_new [B] int32 device memory, or NULL
 *   dtype   ATTN_BF16 or ATTN_F32 (of q, k_new and k_cache)
 *
 * rope_dim must be a multiple of 8 in [8, 1024] and x_row_bytes a multiple of
 * 16 (else ATTN_ERR_UNSUPPORTED); every buffer 16-byte aligned (else
 * ATTN_ERR_UNSUPPORTED); rope_base positive and finite (else ATTN_ERR_SHAPE);
 * T_max >= 1 when a cache is written.  All pointers are device memory owned by
 * the caller; new rows and caches must not overlap.  One launch, no workspace.
 */
attn_status attn_rope_append(void* q, void* k_new, void* k_cache, const void* x_new, void* x_cache,
                             const int32_t* start_pos, const int32_t* n_new, int B, int S, int Hq, int Hk,
                             int rope_dim, int x_row_bytes, int T_max, float rope_base, attn_dtype dtype,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
