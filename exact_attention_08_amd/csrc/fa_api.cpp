// fa_api.cpp -- the C ABI declared in include/fa.h: host-side argument
// validation, kernel-parameter setup and launch on the caller's stream.
// Every argument check runs before any HIP call, so an invalid call touches
// neither the device nor the runtime.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "fa_internal.hpp"

static_assert(FA_DECODE_NOALLOC_MAX_BYTES == fa::kDecodeScratchBytes,
              "the header states the scratch size of the allocation-free decode");

namespace {

thread_local char g_err[512] = "";

fa_status_t fail(fa_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

fa_status_t ok() {
    g_err[0] = '\0';
    return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Checks shared by all entry points.
// k and v may be null only when there are no keys at all (no_keys).
fa_status_t check_common(const void* q, const void* k, const void* v, const void* out,
                         const float* lse, int B, int Hq, int Hkv, int d, int wl, int wr,
                         float scale, fa_dtype_t dtype, bool no_keys = false) {
    if (!q || !out) return fail(FA_ERR_INVALID_ARG, "q and out must be non-null");
    if ((!k || !v) && !no_keys)
        return fail(FA_ERR_INVALID_ARG, "k and v must be non-null when there are keys");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(FA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if (lse && !aligned4(lse)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (B < 1 || Hq < 1 || Hkv < 1)
        return fail(FA_ERR_INVALID_ARG, "B, Hq, Hkv must be >= 1 (got %d, %d, %d)", B, Hq, Hkv);
    if (Hq % Hkv != 0)
        return fail(FA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", d);
    if (dtype != FA_BF16 && dtype != FA_FP16)
        return fail(FA_ERR_UNSUPPORTED, "dtype %d unsupported (bf16 or fp16)", (int)dtype);
    if (wl < -1 || wr < -1)
        return fail(FA_ERR_INVALID_ARG, "window bounds must be >= -1 (got %d, %d)", wl, wr);
    if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "softmax_scale must be finite");
    return FA_OK;
}

void set_scale(float scale, float* c, uint32_t* qsign) {
    // scores are scaled in fp32 inside the exponent; a negative scale is
    // folded into an exact sign flip of q so that c >= 0.
    // c is kept >= FLT_MIN: masked scores are -inf and -inf * c must stay
    // -inf; at scale 0 every exp2 argument is then |s|*FLT_MIN ~ 0, so the
    // weights are exactly uniform in fp32, as scale 0 requires.
    *c = std::fmax(std::fabs(scale) * fa::kLog2e_host, 1.17549435e-38f);
    *qsign = scale < 0.f ? 0x80008000u : 0u;
}

fa_status_t launch_status(hipError_t e) {
    if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

constexpr long long kMaxGridThreads = (1ll << 32) - 1;

// Buffer loads address one sequence of one tensor with 32-bit byte offsets.
constexpr long long kMaxSeqBytes = (1ll << 31) - 1;

fa_status_t check_seq_bytes(long long rows, int heads, int d, const char* what) {
    if (rows * heads * d * 2 > kMaxSeqBytes)
        return fail(FA_ERR_UNSUPPORTED, "%s: %lld rows x %d heads x %d exceeds 2 GiB per sequence",
                    what, rows, heads, d);
    return FA_OK;
}

// Contiguous-cache decode.  With use_scratch the split partials go to the
// library's per-GPU scratch array (fa_decode_kvcache_noalloc) instead of the
// caller's workspace; every check still runs before any HIP call.
fa_status_t decode_kvcache_impl(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* cache_seqlens, void* out, float* lse, int B,
                                int Hq, int Hkv, int Sk_cap, int max_seqlen_k, int d, int causal,
                                int window_left, int window_right, float softmax_scale,
                                int split_size, void* workspace, size_t workspace_bytes,
                                bool use_scratch, fa_dtype_t dtype, hipStream_t stream) {
    fa_status_t st = check_common(q, k_cache, v_cache, out, lse, B, Hq, Hkv, d, window_left,
                                  window_right, softmax_scale, dtype);
    if (st != FA_OK) return st;
    if (!cache_seqlens || !aligned4(cache_seqlens))
        return fail(FA_ERR_INVALID_ARG, "cache_seqlens must be non-null and 4-byte aligned");
    if (Sk_cap < 1) return fail(FA_ERR_INVALID_ARG, "Sk_cap must be >= 1 (got %d)", Sk_cap);
    if (max_seqlen_k < 1 || max_seqlen_k > Sk_cap)
        return fail(FA_ERR_INVALID_ARG, "max_seqlen_k must be in [1, Sk_cap] (got %d)", max_seqlen_k);
    if (split_size < 64 || split_size % 64 != 0)
        return fail(FA_ERR_INVALID_ARG, "split_size must be a positive multiple of 64 (got %d)",
                    split_size);
    if ((st = check_seq_bytes(Sk_cap, Hkv, d, "k/v cache")) != FA_OK) return st;
    const size_t need = fa_decode_workspace_bytes(B, Hq, max_seqlen_k, d, split_size);
    const int nsplit = (max_seqlen_k + split_size - 1) / split_size;
    const int qblocks = (Hq / Hkv + 15) / 16;
    if ((long long)nsplit * qblocks * Hkv * B * fa::kDecodeThreads > kMaxGridThreads)
        return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
    if (use_scratch) {
        if (need > fa::kDecodeScratchBytes)
            return fail(FA_ERR_WORKSPACE,
                        "partial results need %zu bytes, more than the %zu-byte scratch array of "
                        "the allocation-free decode (use a larger split_size, fewer sequences, "
                        "or fa_decode_kvcache with a workspace)",
                        need, fa::kDecodeScratchBytes);
        // the scratch address is per device: the stream must run on the
        // current device, whose copy decode_scratch() returns
        int cur = 0, sdev = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && stream != nullptr) e = hipStreamGetDevice(stream, &sdev);
        else sdev = cur;
        if (e != hipSuccess) return fail(FA_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
        if (sdev != cur)
            return fail(FA_ERR_INVALID_ARG, "the stream belongs to device %d, not the current "
                        "device %d", sdev, cur);
        e = fa::decode_scratch(&workspace);
        if (e != hipSuccess)
            return fail(FA_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(e));
        workspace_bytes = fa::kDecodeScratchBytes;
    }
    if (!workspace || !aligned16(workspace))
        return fail(FA_ERR_WORKSPACE, "workspace must be non-null and 16-byte aligned");
    if (workspace_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    fa::DecodeParams p{};
    p.q = q; p.k = k_cache; p.v = v_cache; p.o = out; p.lse = lse;
    p.seqlens = cache_seqlens;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.Sk_cap = Sk_cap;
    p.max_len = max_seqlen_k;
    p.split = split_size;
    p.nsplit = nsplit;
    p.qblocks = qblocks;
    p.ws_o = static_cast<float*>(workspace);
    p.ws_lse = p.ws_o + (size_t)B * Hq * p.nsplit * d;
    p.causal = causal ? 1 : 0; p.wl = window_left; p.wr = window_right;
    set_scale(softmax_scale, &p.c, &p.qsign);
    return launch_status(fa::launch_decode(p, d, dtype == FA_BF16, stream));
}

}  // namespace

extern "C" {

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                   int window_right, float softmax_scale, fa_dtype_t dtype, hipStream_t stream) {
    fa_status_t st = check_common(q, k, v, out, lse, B, Hq, Hkv, d, window_left, window_right,
                                  softmax_scale, dtype, Sk == 0);
    if (st != FA_OK) return st;
    if (Sq < 0 || Sk < 0) return fail(FA_ERR_INVALID_ARG, "Sq, Sk must be >= 0 (got %d, %d)", Sq, Sk);
    if (Sq == 0) return ok();
    if ((st = check_seq_bytes(Sq, Hq, d, "q")) != FA_OK) return st;
    if ((st = check_seq_bytes(Sk, Hkv, d, "k/v")) != FA_OK) return st;
    // A window bound that cuts no row is no bound (row positions run from
    // Sk - Sq to Sk - 1): dropping it keeps the plain kernel form, which is
    // faster where few steps cross a band edge.
    if (window_left >= Sk - 1) window_left = -1;
    if (window_right >= Sq - 1) window_right = -1;
    fa::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse;
    p.cu_q = nullptr; p.cu_k = nullptr;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.Sq = Sq; p.Sk = Sk;
    const bool wide = fa::fwd_use_wide(Sq, Sk, causal, window_left, window_right);
    p.gw = fa::fwd_heads_per_wg(p.G);
    p.bm = fa::fwd_rows_per_wg(p.G, wide ? fa::kFwdWideWaveRows : fa::kFwdWaveRows);
    p.nqt = (Sq + p.bm - 1) / p.bm;
    p.q_tok_stride = (long long)Hq * d;
    p.kv_tok_stride = (long long)Hkv * d;
    p.lse_b_stride = (long long)Hq * Sq;
    p.lse_h_stride = Sq;
    p.causal = causal ? 1 : 0; p.wl = window_left; p.wr = window_right;
    set_scale(softmax_scale, &p.c, &p.qsign);
    p.xcd_groups = ((long long)B * Hkv) % 8 == 0 ? (B * Hkv) / 8 : 0;
    if ((long long)p.nqt * (Hq / p.gw) * B * fa::kFwdThreads > kMaxGridThreads)
        return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
    return launch_status(wide ? fa::launch_fwd_wide(p, d, dtype == FA_BF16, false, stream)
                              : fa::launch_fwd(p, d, dtype == FA_BF16, false, stream));
}

fa_status_t fa_fwd_mod(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                       int window_right, float softmax_scale, const float* alibi_slopes,
                       float softcap, fa_dtype_t dtype, hipStream_t stream) {
    if (alibi_slopes && !aligned4(alibi_slopes))
        return fail(FA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    if (!std::isfinite(softcap) || softcap < 0.f)
        return fail(FA_ERR_INVALID_ARG, "softcap must be finite and >= 0 (0 = off)");
    if (!alibi_slopes && softcap == 0.f)
        return fa_fwd(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, d, causal, window_left, window_right,
                      softmax_scale, dtype, stream);
    fa_status_t st = check_common(q, k, v, out, lse, B, Hq, Hkv, d, window_left, window_right,
                                  softmax_scale, dtype, Sk == 0);
    if (st != FA_OK) return st;
    if (Sq < 0 || Sk < 0) return fail(FA_ERR_INVALID_ARG, "Sq, Sk must be >= 0 (got %d, %d)", Sq, Sk);
    if (Sq == 0) return ok();
    if ((st = check_seq_bytes(Sq, Hq, d, "q")) != FA_OK) return st;
    if ((st = check_seq_bytes(Sk, Hkv, d, "k/v")) != FA_OK) return st;
    fa::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse;
    p.cu_q = nullptr; p.cu_k = nullptr;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.Sq = Sq; p.Sk = Sk;
    const bool wide = fa::fwd_use_wide(Sq, Sk, causal, window_left, window_right);
    p.gw = fa::fwd_heads_per_wg(p.G);
    p.bm = fa::fwd_rows_per_wg(p.G, wide ? fa::kFwdWideWaveRows : fa::kFwdWaveRows);
    p.nqt = (Sq + p.bm - 1) / p.bm;
    p.q_tok_stride = (long long)Hq * d;
    p.kv_tok_stride = (long long)Hkv * d;
    p.lse_b_stride = (long long)Hq * Sq;
    p.lse_h_stride = Sq;
    p.causal = causal ? 1 : 0; p.wl = window_left; p.wr = window_right;
    set_scale(softmax_scale, &p.c, &p.qsign);
    p.xcd_groups = ((long long)B * Hkv) % 8 == 0 ? (B * Hkv) / 8 : 0;
    p.mod = (alibi_slopes ? 1 : 0) | (softcap > 0.f ? 2 : 0);
    p.alibi = alibi_slopes;
    if (softcap > 0.f) {
        p.sc_k = 2.f * std::fabs(softmax_scale) * fa::kLog2e_host / softcap;
        p.sc_c = softcap * fa::kLog2e_host;
    }
    if ((long long)p.nqt * (Hq / p.gw) * B * fa::kFwdThreads > kMaxGridThreads)
        return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
    return launch_status(wide ? fa::launch_fwd_wide(p, d, dtype == FA_BF16, false, stream)
                              : fa::launch_fwd(p, d, dtype == FA_BF16, false, stream));
}

fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int Hq,
                          int Hkv, int max_seqlen_q, int max_seqlen_k, int total_q, int d,
                          int causal, int window_left, int window_right, float softmax_scale,
                          fa_dtype_t dtype, hipStream_t stream) {
    fa_status_t st = check_common(q, k, v, out, lse, B, Hq, Hkv, d, window_left, window_right,
                                  softmax_scale, dtype, max_seqlen_k == 0);
    if (st != FA_OK) return st;
    if (!cu_seqlens_q || !cu_seqlens_k)
        return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be non-null");
    if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k))
        return fail(FA_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
    if (max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0)
        return fail(FA_ERR_INVALID_ARG, "max_seqlen_q, max_seqlen_k, total_q must be >= 0");
    if (max_seqlen_q == 0 || total_q == 0) return ok();
    if ((st = check_seq_bytes(max_seqlen_q, Hq, d, "q")) != FA_OK) return st;
    if ((st = check_seq_bytes(max_seqlen_k, Hkv, d, "k/v")) != FA_OK) return st;
    fa::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse;
    p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.Sq = max_seqlen_q; p.Sk = max_seqlen_k;
    const bool wide = fa::fwd_use_wide(max_seqlen_q, max_seqlen_k, causal, window_left,
                                        window_right);
    p.gw = fa::fwd_heads_per_wg(p.G);
    p.bm = fa::fwd_rows_per_wg(p.G, wide ? fa::kFwdWideWaveRows : fa::kFwdWaveRows);
    p.nqt = (max_seqlen_q + p.bm - 1) / p.bm;
    p.q_tok_stride = (long long)Hq * d;
    p.kv_tok_stride = (long long)Hkv * d;
    p.lse_b_stride = 0;
    p.lse_h_stride = total_q;
    p.causal = causal ? 1 : 0; p.wl = window_left; p.wr = window_right;
    set_scale(softmax_scale, &p.c, &p.qsign);
    p.xcd_groups = ((long long)B * Hkv) % 8 == 0 ? (B * Hkv) / 8 : 0;
    if ((long long)p.nqt * (Hq / p.gw) * B * fa::kFwdThreads > kMaxGridThreads)
        return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
    return launch_status(wide ? fa::launch_fwd_wide(p, d, dtype == FA_BF16, true, stream)
                              : fa::launch_fwd(p, d, dtype == FA_BF16, true, stream));
}

size_t fa_decode_workspace_bytes(int B, int Hq, int max_seqlen_k, int d, int split_size) {
    if (B < 1 || Hq < 1 || max_seqlen_k < 1 || d < 1 || split_size < 1) return 0;
    const size_t nsplit = ((size_t)max_seqlen_k + split_size - 1) / split_size;
    return (size_t)B * Hq * nsplit * ((size_t)d + 1) * sizeof(float);
}

fa_status_t fa_decode_kvcache(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* cache_seqlens, void* out, float* lse, int B, int Hq,
                              int Hkv, int Sk_cap, int max_seqlen_k, int d, int causal,
                              int window_left, int window_right, float softmax_scale,
                              int split_size, void* workspace, size_t workspace_bytes,
                              fa_dtype_t dtype, hipStream_t stream) {
    return decode_kvcache_impl(q, k_cache, v_cache, cache_seqlens, out, lse, B, Hq, Hkv, Sk_cap,
                               max_seqlen_k, d, causal, window_left, window_right, softmax_scale,
                               split_size, workspace, workspace_bytes, false, dtype, stream);
}

fa_status_t fa_decode_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* cache_seqlens, void* out, float* lse, int B,
                                      int Hq, int Hkv, int Sk_cap, int max_seqlen_k, int d,
                                      int causal, int window_left, int window_right,
                                      float softmax_scale, int split_size, fa_dtype_t dtype,
                                      hipStream_t stream) {
    return decode_kvcache_impl(q, k_cache, v_cache, cache_seqlens, out, lse, B, Hq, Hkv, Sk_cap,
                               max_seqlen_k, d, causal, window_left, window_right, softmax_scale,
                               split_size, nullptr, 0, true, dtype, stream);
}

fa_status_t fa_decode_paged(const void* q, void* k_pages, void* v_pages,
                            const int32_t* block_table, const int32_t* cache_seqlens,
                            const void* k_new, const void* v_new, void* out, float* lse,
                            int B, int Hq, int Hkv, int num_pages, int page_size,
                            int max_pages_per_seq, int max_seqlen_k, int d, int causal,
                            int window_left, int window_right, float softmax_scale,
                            int split_size, void* workspace, size_t workspace_bytes,
                            fa_dtype_t dtype, hipStream_t stream) {
    fa_status_t st = check_common(q, k_pages, v_pages, out, lse, B, Hq, Hkv, d, window_left,
                                  window_right, softmax_scale, dtype);
    if (st != FA_OK) return st;
    if (!block_table || !aligned4(block_table))
        return fail(FA_ERR_INVALID_ARG, "block_table must be non-null and 4-byte aligned");
    if (!cache_seqlens || !aligned4(cache_seqlens))
        return fail(FA_ERR_INVALID_ARG, "cache_seqlens must be non-null and 4-byte aligned");
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(FA_ERR_INVALID_ARG, "k_new and v_new must both be given or both be NULL");
    if (k_new && (!aligned16(k_new) || !aligned16(v_new)))
        return fail(FA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
    if (page_size < 32 || page_size % 32 != 0)
        return fail(FA_ERR_INVALID_ARG, "page_size must be a positive multiple of 32 (got %d)",
                    page_size);
    if (num_pages < 1 || max_pages_per_seq < 1)
        return fail(FA_ERR_INVALID_ARG, "num_pages and max_pages_per_seq must be >= 1 (got %d, %d)",
                    num_pages, max_pages_per_seq);
    const long long cap = (long long)max_pages_per_seq * page_size;
    if (max_seqlen_k < 1 || max_seqlen_k > cap)
        return fail(FA_ERR_INVALID_ARG,
                    "max_seqlen_k must be in [1, max_pages_per_seq * page_size] (got %d)",
                    max_seqlen_k);
    if (split_size < 64 || split_size % 64 != 0)
        return fail(FA_ERR_INVALID_ARG, "split_size must be a positive multiple of 64 (got %d)",
                    split_size);
    const size_t need = fa_decode_workspace_bytes(B, Hq, max_seqlen_k, d, split_size);
    if (!workspace || !aligned16(workspace))
        return fail(FA_ERR_WORKSPACE, "workspace must be non-null and 16-byte aligned");
    if (workspace_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    fa::DecodeParams p{};
    p.q = q; p.k = k_pages; p.v = v_pages; p.o = out; p.lse = lse;
    p.seqlens = cache_seqlens;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.Sk_cap = 0;                               // unused with a block table
    p.max_len = max_seqlen_k;
    p.split = split_size;
    p.nsplit = (max_seqlen_k + split_size - 1) / split_size;
    p.qblocks = (p.G + 15) / 16;
    p.ws_o = static_cast<float*>(workspace);
    p.ws_lse = p.ws_o + (size_t)B * Hq * p.nsplit * d;
    p.causal = causal ? 1 : 0; p.wl = window_left; p.wr = window_right;
    set_scale(softmax_scale, &p.c, &p.qsign);
    p.block_table = block_table;
    p.page_size = page_size; p.max_pages = max_pages_per_seq; p.num_pages = num_pages;
    p.append = k_new != nullptr;
    p.k_new = k_new; p.v_new = v_new;
    if ((long long)p.nsplit * p.qblocks * Hkv * B * fa::kDecodeThreads > kMaxGridThreads)
        return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
    return launch_status(fa::launch_decode(p, d, dtype == FA_BF16, stream));
}

size_t fa_fwd_fp8_workspace_bytes(int B, int Hkv, int Sk, int d) {
    if (B < 1 || Hkv < 1 || Sk < 1 || d < 1) return 0;
    return (size_t)B * Hkv * d * (((size_t)Sk + 63) / 64 * 64);
}

fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                       int window_right, float softmax_scale, float descale_q, float descale_k,
                       float descale_v, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    // dtype BF16 here only selects the checks; q/k/v are 8-bit, out is bf16
    fa_status_t st = check_common(q, k, v, out, lse, B, Hq, Hkv, d, window_left, window_right,
                                  softmax_scale, FA_BF16, Sk == 0);
    if (st != FA_OK) return st;
    if (!std::isfinite(descale_q) || !std::isfinite(descale_k) || !std::isfinite(descale_v) ||
        descale_q <= 0.f || descale_k <= 0.f || descale_v <= 0.f)
        return fail(FA_ERR_INVALID_ARG, "descale factors must be finite and > 0");
    if (Sq < 0 || Sk < 0) return fail(FA_ERR_INVALID_ARG, "Sq, Sk must be >= 0 (got %d, %d)", Sq, Sk);
    if (Sq == 0) return ok();
    if ((st = check_seq_bytes(Sq, Hq, d, "q/out")) != FA_OK) return st;
    if ((st = check_seq_bytes(Sk, Hkv, d, "k/v")) != FA_OK) return st;
    const size_t need = fa_fwd_fp8_workspace_bytes(B, Hkv, Sk, d);
    if (need > 0 && (!workspace || !aligned16(workspace)))
        return fail(FA_ERR_WORKSPACE, "workspace must be non-null and 16-byte aligned");
    if (workspace_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    fa::Fp8Params p{};
    p.q = q; p.k = k; p.v = v; p.vt = workspace; p.o = out; p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.Sq = Sq; p.Sk = Sk; p.sk_pad = (Sk + 63) / 64 * 64;
    // the 16-bit forward's rule picks the paired (32-row waves) or the wide
    // (64-row waves) form
    const bool wide = fa::fwd_use_wide(Sq, Sk, causal, window_left, window_right);
    p.gw = fa::fwd_heads_per_wg(p.G);
    p.bm = fa::fwd_rows_per_wg(p.G, wide ? fa::kFwdWideWaveRows : fa::kFwdWaveRows);
    p.nqt = (Sq + p.bm - 1) / p.bm;
    p.q_tok_stride = (long long)Hq * d;
    p.kv_tok_stride = (long long)Hkv * d;
    p.causal = causal ? 1 : 0; p.wl = window_left; p.wr = window_right;
    // scores are scaled in fp32: c = |scale| dq dk log2(e), kept >= FLT_MIN
    // (masked scores are -inf); a negative scale flips the sign bit of q
    p.c = std::fmax(std::fabs(softmax_scale) * descale_q * descale_k * fa::kLog2e_host,
                    1.17549435e-38f);
    p.qsign = softmax_scale < 0.f ? 0x80808080u : 0u;
    p.descale_v = descale_v;
    p.xcd_groups = ((long long)B * Hkv) % 8 == 0 ? (B * Hkv) / 8 : 0;
    if ((long long)p.nqt * (Hq / p.gw) * B * fa::kFwdThreads > kMaxGridThreads)
        return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
    return launch_status(fa::launch_fwd_fp8(p, d, wide, stream));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Sq) {
    if (B < 1 || Hq < 1 || Sq < 1) return 0;
    return 2 * (size_t)B * Hq * Sq * sizeof(float);
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
                   int Sk, int d, int causal, int window_left, int window_right,
                   float softmax_scale, void* workspace, size_t workspace_bytes, fa_dtype_t dtype,
                   hipStream_t stream) {
    if (Sq < 0 || Sk < 0) return fail(FA_ERR_INVALID_ARG, "Sq, Sk must be >= 0 (got %d, %d)", Sq, Sk);
    // tensors of a side with no rows may be NULL (an empty torch tensor has
    // no storage); the shared checks then see stand-ins that pass them
    alignas(16) static const uint64_t kNone[2] = {0, 0};
    const void* const none = kNone;
    fa_status_t st = check_common(Sq > 0 ? q : none, Sk > 0 ? k : none, Sk > 0 ? v : none,
                                  Sq > 0 ? out : none, Sq > 0 ? lse : nullptr, B, Hq, Hkv, d,
                                  window_left, window_right, softmax_scale, dtype);
    if (st != FA_OK) return st;
    if (Sq > 0 && (!dout || !aligned16(dout)))
        return fail(FA_ERR_INVALID_ARG, "dout must be non-null and 16-byte aligned");
    if (Sq > 0 && (!dq || !aligned16(dq)))
        return fail(FA_ERR_INVALID_ARG, "dq must be non-null and 16-byte aligned");
    if (Sk > 0 && (!dk || !dv || !aligned16(dk) || !aligned16(dv)))
        return fail(FA_ERR_INVALID_ARG, "dk and dv must be non-null and 16-byte aligned");
    if (Sq > 0 && !lse) return fail(FA_ERR_INVALID_ARG, "lse (the forward's) must be non-null");
    if (Sq == 0 && Sk == 0) return ok();
    if ((st = check_seq_bytes(Sq, Hq, d, "q")) != FA_OK) return st;
    if ((st = check_seq_bytes(Sk, Hkv, d, "k/v")) != FA_OK) return st;
    const size_t need = fa_bwd_workspace_bytes(B, Hq, Sq);
    if (need > 0 && (!workspace || !aligned16(workspace)))
        return fail(FA_ERR_WORKSPACE, "workspace must be non-null and 16-byte aligned");
    if (workspace_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    fa::BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.o = out; p.dout = dout; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv;
    p.dsum = static_cast<float*>(workspace);
    p.lse2 = p.dsum + (size_t)B * Hq * Sq;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.Sq = Sq; p.Sk = Sk;
    p.q_tok_stride = (long long)Hq * d;
    p.kv_tok_stride = (long long)Hkv * d;
    p.causal = causal ? 1 : 0; p.wl = window_left; p.wr = window_right;
    p.scale = softmax_scale;
    p.c2 = softmax_scale * fa::kLog2e_host;
    p.nkb = (Sk + fa::kBwdKeysPerWg - 1) / fa::kBwdKeysPerWg;
    p.gw = fa::fwd_heads_per_wg(p.G);
    const int bmq = 32 * fa::bwd_dq_waves(d) / p.gw;
    p.nqb = (Sq + bmq - 1) / bmq;
    if ((long long)p.nkb * Hkv * B * 64 * fa::kBwdDkdvWaves > kMaxGridThreads ||
        (long long)p.nqb * (Hq / p.gw) * B * 64 * fa::bwd_dq_waves(d) > kMaxGridThreads)
        return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
    return launch_status(fa::launch_bwd(p, d, dtype == FA_BF16, stream));
}

const char* fa_status_str(fa_status_t s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
        case FA_ERR_HIP: return "FA_ERR_HIP";
    }
    return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_err; }

}  // extern "C"
