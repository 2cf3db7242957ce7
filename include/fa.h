/*
 * fa.h -- C ABI of the fused exact-attention library for MI355X (gfx950):
 * forward, KV-cache decode (contiguous or paged, with append) and the
 * training backward.  Link against
 * libfa355.so.
 *
 * What is computed (all entry points): exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T + mask) V,   LSE = log of the softmax normaliser,
 * in one fused, tiled pass with an online (running max / running sum)
 * softmax, so the score matrix never reaches device memory.
 *   - "FlashAttention" explainer page, sections "What it is" and "How it
 *     works", steps 1-5 (tiling, on-chip scores, online softmax, one final
 *     normalisation, the saved per-row log-normaliser);
 *   - same page, step 6 (causal masking with whole-tile skipping), step 7
 *     (work spread over query blocks, heads and batch), step 8 (16-bit
 *     operands, fp32 accumulation and fp32 softmax statistics), step 9
 *     (decoding against a cache, split along the sequence and combined);
 *   - "Flash Attention" skill page, "Workflow 2": the flash_attn_func
 *     arguments (causal, window_size=(left, right), softmax_scale) and the
 *     [batch, seq_len, num_heads, head_dim] layout;
 *   - "The One-Line Change ... Flash Attention 2 in HuggingFace": packed
 *     sequences described by cumulative lengths, never attending across
 *     sequence borders.
 *
 * Mask semantics shared by every entry point.  For a sequence with sq query
 * rows and sk keys, query row i sits at key position pos = i + (sk - sq)
 * (bottom-right alignment; identical to top-left when sq == sk).  Key j is
 * visible from row i iff 0 <= j < sk and
 *     (!causal || j <= pos) && (window_left < 0 || j >= pos - window_left)
 *                           && (window_right < 0 || j <= pos + window_right).
 * Window bounds are inclusive; -1 means unbounded on that side.  Query head
 * h reads K/V head h / (Hq / Hkv) (grouped-query attention by consecutive
 * groups).  LSE is the natural log of sum_j exp(scale * q_i . k_j) over
 * visible keys; a row with no visible key gets O = 0 and LSE = -inf.
 *
 * Conventions for every entry point.
 *   - Pointers are DEVICE pointers, owned by the caller, 16-byte aligned,
 *     dense (no strides beyond the layouts stated).  k and v may be NULL
 *     only when there are no keys (Sk == 0, or max_seqlen_k == 0 packed).  The library never
 *     allocates or frees device memory, never keeps a pointer after it
 *     returns and never synchronises: all work is enqueued on `stream`
 *     (NULL = the null stream) and the call returns before it runs.
 *   - q/k/v/out are bf16 or fp16 (dtype); lse and workspaces are fp32;
 *     cumulative lengths and cache lengths are int32.
 *   - softmax_scale: any finite value (the Python layer maps "None" to
 *     1/sqrt(d)); it is applied in fp32 to the fp32 score accumulator.
 *   - Errors: argument problems are detected on the host before anything is
 *     enqueued and nothing is written (FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED,
 *     FA_ERR_WORKSPACE); a failed launch returns FA_ERR_HIP.  The detail of
 *     the last non-OK return of the calling thread is in fa_last_error().
 *     There is no fallback path.
 *   - Not checked (that would need a device-to-host copy): monotone
 *     cumulative lengths starting at 0, cache lengths within [0, max_seqlen_k].
 *     The decode kernels clamp cache lengths to [0, max_seqlen_k].
 *   - Determinism: the same call on the same inputs gives bitwise identical
 *     results (fixed reduction order, no floating-point atomics).
 */
#ifndef FA355_FA_H
#define FA355_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum { FA_BF16 = 0, FA_FP16 = 1 } fa_dtype_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, bad window, non-finite scale, misaligned */
    FA_ERR_UNSUPPORTED = 2,  /* head_dim not in {64, 128}, dtype not bf16/fp16 */
    FA_ERR_WORKSPACE = 3,    /* decode workspace missing or too small */
    FA_ERR_HIP = 4           /* the HIP runtime reported an error at launch */
} fa_status_t;

/* Padded batch (flash_attn_func on the skill page, "Workflow 2").
 *   q, out : [B, Sq, Hq, d]      k, v : [B, Sk, Hkv, d]
 *   lse    : [B, Hq, Sq] fp32, may be NULL (not written then)
 *   B, Hq, Hkv >= 1, Hq % Hkv == 0; Sq, Sk >= 0 (Sq == 0 enqueues nothing;
 *   Sk == 0 gives O = 0 and LSE = -inf); d in {64, 128};
 *   window_left, window_right >= -1. */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                   int B, int Hq, int Hkv, int Sq, int Sk, int d,
                   int causal, int window_left, int window_right, float softmax_scale,
                   fa_dtype_t dtype, hipStream_t stream);

/* Padded batch with score modifiers (the "FlashAttention" explainer page,
 * "Variants you may meet": bias terms such as ALiBi added to the scores, and
 * soft-capping of the scores, which needs kernel support; the project
 * summary lists ALiBi).  The pages give no formulas; the scores are those of
 * the fast library's alibi_slopes and softcap arguments:
 *     s_ij = scale * q_i . k_j
 *     s_ij = softcap * tanh(s_ij / softcap)        when softcap > 0
 *     s_ij = s_ij - alibi_slopes[h] * |pos_i - j|   when alibi_slopes != NULL
 * (pos_i as in the mask rule; h the query head), then softmax, O and LSE as
 * above over the modified scores.
 *   alibi_slopes : fp32 [Hq] DEVICE array, or NULL (no bias)
 *   softcap      : finite, >= 0; 0 = off
 * Other arguments, layouts and errors as fa_fwd; with no bias and no cap
 * the call is fa_fwd. */
fa_status_t fa_fwd_mod(const void* q, const void* k, const void* v, void* out, float* lse,
                       int B, int Hq, int Hkv, int Sq, int Sk, int d,
                       int causal, int window_left, int window_right, float softmax_scale,
                       const float* alibi_slopes, float softcap,
                       fa_dtype_t dtype, hipStream_t stream);

/* Bytes of workspace fa_fwd_fp8 needs: V transposed per K/V head,
 * B * Hkv * d * (Sk rounded up to 64) bytes. */
size_t fa_fwd_fp8_workspace_bytes(int B, int Hkv, int Sk, int d);

/* Padded batch on 8-bit inputs (the "FlashAttention" explainer page: the
 * later versions use lower-precision number formats, "What it is"; the
 * project summary lists FP8; no recipe is given).  q, k, v hold e4m3 codes
 * (the OCP 8-bit float: 1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; 448 the largest value) whose real values are descale_{q,k,v} times
 * the code values (one fp32 factor per tensor, > 0).  Both products run on
 * 8-bit matrix instructions with fp32 accumulation; the softmax weights are
 * rounded to e4m3 for P.V; statistics are fp32.  out is bf16.
 *   q : [B, Sq, Hq, d] e4m3    k, v : [B, Sk, Hkv, d] e4m3
 *   out : [B, Sq, Hq, d] bf16  lse : [B, Hq, Sq] fp32 (may be NULL)
 *   workspace : DEVICE scratch of at least fa_fwd_fp8_workspace_bytes(B,
 *               Hkv, Sk, d) bytes (V transposed by a first kernel), owned
 *               by the caller, contents ignored; may be NULL when Sk == 0
 * Other arguments, masks, LSE and errors as fa_fwd.  Two kernels are
 * enqueued (V transpose, attention). */
fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
                       int B, int Hq, int Hkv, int Sq, int Sk, int d,
                       int causal, int window_left, int window_right, float softmax_scale,
                       float descale_q, float descale_k, float descale_v,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Packed sequences (flash_attn_varlen_func; "The One-Line Change ..." page,
 * sequence packing).  B sequences; sequence z owns query rows
 * [cu_seqlens_q[z], cu_seqlens_q[z+1]) and key rows
 * [cu_seqlens_k[z], cu_seqlens_k[z+1]).
 *   q, out : [total_q, Hq, d]    k, v : [total_k, Hkv, d]
 *   lse    : [Hq, total_q] fp32, may be NULL
 *   cu_seqlens_q, cu_seqlens_k : int32 [B+1] DEVICE arrays (may alias)
 *   max_seqlen_q, max_seqlen_k : host upper bounds of the per-sequence
 *   lengths, used only to size the launch grid (rows past a bound are not
 *   computed, so they must be true bounds).
 *   total_q = cu_seqlens_q[B] is read by the kernels, never by the host. */
fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int B, int Hq, int Hkv, int max_seqlen_q, int max_seqlen_k,
                          int total_q, int d,
                          int causal, int window_left, int window_right, float softmax_scale,
                          fa_dtype_t dtype, hipStream_t stream);

/* Bytes of fp32 workspace fa_decode_kvcache needs for these sizes
 * (partial outputs and partial LSEs of every split). */
size_t fa_decode_workspace_bytes(int B, int Hq, int max_seqlen_k, int d, int split_size);

/* One-token decode against a contiguous KV cache, split along the cache and
 * merged by the LSE rule (explainer page, step 9 "decoding with a cache" and
 * "Long context beyond a single GPU": partial results combined with the same
 * online softmax rule).
 *   q, out           : [B, 1, Hq, d]
 *   k_cache, v_cache : [B, Sk_cap, Hkv, d]; the first cache_seqlens[b] rows
 *                      of sequence b are its keys (they include the token
 *                      being decoded)
 *   cache_seqlens    : int32 [B] DEVICE array
 *   lse              : [B, Hq] fp32, may be NULL
 *   max_seqlen_k     : host upper bound of cache_seqlens (grid and workspace
 *                      sizing), 1 <= max_seqlen_k <= Sk_cap; longer lengths
 *                      are clamped to it
 *   split_size       : keys per split, a positive multiple of 64
 *   workspace        : DEVICE scratch of at least
 *                      fa_decode_workspace_bytes(B, Hq, max_seqlen_k, d,
 *                      split_size) bytes, owned by the caller; contents on
 *                      entry are ignored.
 * Two kernels are enqueued on `stream` (split, then combine). */
fa_status_t fa_decode_kvcache(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* cache_seqlens, void* out, float* lse,
                              int B, int Hq, int Hkv, int Sk_cap, int max_seqlen_k, int d,
                              int causal, int window_left, int window_right,
                              float softmax_scale, int split_size,
                              void* workspace, size_t workspace_bytes,
                              fa_dtype_t dtype, hipStream_t stream);

/* Largest partial-result size, in bytes, of fa_decode_kvcache_noalloc:
 * fa_decode_workspace_bytes(B, Hq, max_seqlen_k, d, split_size) must not
 * exceed it (64 MiB: e.g. 64 sequences x 32 query heads x 31 splits at
 * d = 128). */
#define FA_DECODE_NOALLOC_MAX_BYTES ((size_t)64 << 20)

/* fa_decode_kvcache for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, layouts, results and errors as
 * fa_decode_kvcache, without the workspace: the split partials go to a
 * scratch array inside the library, FA_DECODE_NOALLOC_MAX_BYTES per GPU,
 * which every GPU the library runs on holds until the process ends.  The
 * call itself allocates nothing (its first call on a device looks up that
 * device's array address once).
 *   - Sizes whose partials exceed FA_DECODE_NOALLOC_MAX_BYTES are rejected
 *     with FA_ERR_WORKSPACE before anything is enqueued.
 *   - `stream` must belong to the current device (else FA_ERR_INVALID_ARG).
 *   - All such calls on one GPU share its array: calls that overlap in time
 *     on one GPU (on different streams, or from different threads without
 *     ordering) race and may return wrong results.  Calls ordered on one
 *     stream are safe; nothing in the array has to start at zero. */
fa_status_t fa_decode_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* cache_seqlens, void* out, float* lse,
                                      int B, int Hq, int Hkv, int Sk_cap, int max_seqlen_k, int d,
                                      int causal, int window_left, int window_right,
                                      float softmax_scale, int split_size,
                                      fa_dtype_t dtype, hipStream_t stream);

/* One-token decode against a PAGED KV cache, optionally appending the new
 * token's key and value first ("FlashAttention" project summary, feature
 * list: the cached-decode call with paged KV cache support; explainer page,
 * advice on generation with a cache: paged cache layouts cut waste; step 9
 * for the split and combine).  The pages fix no layout; this one is:
 *   k_pages, v_pages : [num_pages, page_size, Hkv, d], a pool of pages shared
 *                      by all sequences; token t of sequence b is row
 *                      t % page_size of page block_table[b][t / page_size]
 *   block_table      : int32 [B, max_pages_per_seq] DEVICE array of page
 *                      indices in [0, num_pages); entries past a sequence's
 *                      last page are never read
 *   cache_seqlens    : int32 [B] DEVICE array, tokens already in the cache
 *   k_new, v_new     : [B, 1, Hkv, d] or both NULL.  When given, row b is
 *                      written into the cache at position cache_seqlens[b]
 *                      (k_pages, v_pages are modified), then the query
 *                      attends over cache_seqlens[b] + 1 keys; when NULL it
 *                      attends over cache_seqlens[b] keys (as
 *                      fa_decode_kvcache, which includes the current token)
 *   q, out, lse      : as for fa_decode_kvcache
 *   page_size        : a positive multiple of 32
 *   max_seqlen_k     : host upper bound of the keys attended (including an
 *                      appended one), 1 <= max_seqlen_k <= max_pages_per_seq
 *                      * page_size; the device clamps cache_seqlens to
 *                      [0, max_seqlen_k] (with an append: to
 *                      [0, max_seqlen_k - 1], the new row going there)
 *   workspace        : at least fa_decode_workspace_bytes(B, Hq, max_seqlen_k,
 *                      d, split_size) bytes, as for fa_decode_kvcache.
 * Not checked (device data): table entries; an entry outside [0, num_pages)
 * reads as zero keys and receives no appended row.  Three kernels are
 * enqueued with an append (append, split, combine), two without.  Two calls
 * that append into the same page rows race unless ordered by the caller. */
fa_status_t fa_decode_paged(const void* q, void* k_pages, void* v_pages,
                            const int32_t* block_table, const int32_t* cache_seqlens,
                            const void* k_new, const void* v_new, void* out, float* lse,
                            int B, int Hq, int Hkv, int num_pages, int page_size,
                            int max_pages_per_seq, int max_seqlen_k, int d,
                            int causal, int window_left, int window_right,
                            float softmax_scale, int split_size,
                            void* workspace, size_t workspace_bytes,
                            fa_dtype_t dtype, hipStream_t stream);

/* Bytes of fp32 workspace fa_bwd needs: two values per query row and head
 * (D_i = dO_i . O_i, and LSE_i in log2 units), written by the first kernel
 * for the second. */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Sq);

/* Gradients of the padded-batch attention (the training backward): given
 * the forward's inputs, its output `out` and LSE, and the gradient `dout` of
 * a loss with respect to `out`, writes dq, dk, dv.  The score tiles are
 * recomputed from q and k and the weights rebuilt from the saved LSE; no
 * score matrix reaches memory ("FlashAttention" explainer page, "Step 5"
 * and "Backward pass in a bit more detail").  dK and dV of a K/V head
 * collect every query head of its group.
 *   q, out, dout, dq : [B, Sq, Hq, d]      k, v, dk, dv : [B, Sk, Hkv, d]
 *   lse              : [B, Hq, Sq] fp32, as written by fa_fwd for the same
 *                      arguments (rows with no visible key: -inf)
 *   workspace        : DEVICE scratch of at least fa_bwd_workspace_bytes(B,
 *                      Hq, Sq) bytes, owned by the caller, contents ignored
 *   other arguments as for fa_fwd.  Sq == 0 sets dk and dv to zero; Sk == 0
 *   sets dq to zero (k, v, dk, dv may then be NULL).  Keys no row sees get
 *   dk = dv = 0; rows with no visible key get dq = 0.
 * Two kernels are enqueued on `stream` (dQ with the row terms D, then dK
 * and dV); none accumulates with atomics, so repeated calls give bitwise
 * identical results. */
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* out,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int Sq, int Sk, int d,
                   int causal, int window_left, int window_right, float softmax_scale,
                   void* workspace, size_t workspace_bytes,
                   fa_dtype_t dtype, hipStream_t stream);

/* Static text of a status code. */
const char* fa_status_str(fa_status_t s);

/* Detail of the calling thread's last non-OK return ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_FA_H */
