// fa_internal.hpp -- parameter blocks shared by the host launcher (fa_api.cpp)
// and the kernels (fa_fwd.hip, fa_fwd_wide.hip, fa_fwd_fp8.hip, fa_decode.hip,
// fa_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Forward (padded or packed).  Element strides are in 16-bit elements.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;                 // may be null
    const int32_t* cu_q;        // packed only
    const int32_t* cu_k;        // packed only
    int B, Hq, Hkv, G;          // G = Hq / Hkv
    int Sq, Sk;                 // padded: lengths; packed: host upper bounds
    int nqt;                    // query tiles per (sequence, head)
    long long q_tok_stride;     // elements between consecutive tokens of q/o (Hq*d)
    long long kv_tok_stride;    // elements between consecutive tokens of k/v (Hkv*d)
    long long lse_b_stride;     // padded: Hq*Sq; packed: 0
    long long lse_h_stride;     // padded: Sq; packed: total_q
    int causal, wl, wr;
    float c;                    // |scale| * log2(e)
    uint32_t qsign;             // 0x80008000 when scale < 0 (q negated exactly), else 0
    int xcd_groups;             // (B*Hkv)/8 when B*Hkv % 8 == 0, else 0 (no remap)
    int gw;                     // query heads per work-group (fwd_heads_per_wg(G))
    int bm;                     // query rows per work-group (fwd_rows_per_wg)
    // score modifiers (padded forward only)
    int mod;                    // bit 0: ALiBi bias, bit 1: soft-capping
    const float* alibi;         // [Hq] slopes (bias -slope * |pos - j|, natural-log units)
    float sc_k;                 // soft-capping: 2 |scale| log2(e) / cap
    float sc_c;                 // soft-capping: cap * log2(e)
};

// Forward on 8-bit (e4m3) Q, K, V (padded batch).  Strides in bytes.
struct Fp8Params {
    const void* q;              // [B, Sq, Hq, d] e4m3
    const void* k;              // [B, Sk, Hkv, d] e4m3
    const void* v;              // [B, Sk, Hkv, d] e4m3
    void* vt;                   // workspace: V^T [B, Hkv, d, sk_pad], 64-key blocks permuted
    void* o;                    // [B, Sq, Hq, d] bf16
    float* lse;                 // [B, Hq, Sq] or null
    int B, Hq, Hkv, G;
    int Sq, Sk, sk_pad;         // sk_pad = Sk rounded up to 64
    int nqt;
    long long q_tok_stride;     // Hq * d
    long long kv_tok_stride;    // Hkv * d
    int causal, wl, wr;
    float c;                    // |scale| * descale_q * descale_k * log2(e)
    uint32_t qsign;             // 0x80808080 when scale < 0 (q negated exactly), else 0
    float descale_v;
    int xcd_groups, gw, bm;
};
// wide: the one-wave-per-SIMD kernel (64-row waves), else the paired one
hipError_t launch_fwd_fp8(const Fp8Params& p, int d, bool wide, hipStream_t s);

// Decode split kernel + combine kernel.
struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;                 // may be null
    const int32_t* seqlens;
    float* ws_o;                // [B, Hq, nsplit, d] fp32 partial outputs
    float* ws_lse;              // [B, Hq, nsplit] fp32 partial LSEs
    int B, Hq, Hkv, G;
    int Sk_cap;
    int max_len;                // host bound on cache lengths (lengths are clamped to it)
    int nsplit, split;
    int qblocks;                // ceil(G / 16)
    int causal, wl, wr;
    float c;                    // |scale| * log2(e)
    uint32_t qsign;
    // paged cache (k, v point at the page pools [num_pages, page_size, Hkv, d])
    const int32_t* block_table; // [B, max_pages]; null for a contiguous cache
    int page_size, max_pages, num_pages;
    // append: k_new, v_new [B, Hkv, d] are written at position seqlens[b]
    // (clamped to max_len - 1) and seen as one more key
    int append;
    const void* k_new;
    const void* v_new;
};

// Backward (gradients): the dQ kernel (which also forms the row terms D and
// the LSE in log2 units), then the dK/dV kernel.
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;           // [B, Hq, Sq], natural log
    void* dq;
    void* dk;
    void* dv;
    float* dsum;                // workspace [B, Hq, Sq]: -D_i = -(dO_i . O_i)
    float* lse2;                // workspace [B, Hq, Sq]: LSE_i log2(e), +inf for empty rows
    int B, Hq, Hkv, G;
    int Sq, Sk;
    long long q_tok_stride;     // Hq * d
    long long kv_tok_stride;    // Hkv * d
    int causal, wl, wr;
    float scale;                // softmax scale (any sign)
    float c2;                   // scale * log2(e)
    int nkb;                    // kBwdKeysPerWg-key blocks per (sequence, K/V head)
    int gw;                     // query heads per dQ work-group
    int nqb;                    // query blocks of 32*bwd_dq_waves(d)/gw rows per (sequence, head group)
};

// Host launchers (defined next to their kernels).
hipError_t launch_fwd(const FwdParams& p, int d, bool bf16, bool varlen, hipStream_t s);
hipError_t launch_fwd_wide(const FwdParams& p, int d, bool bf16, bool varlen, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, int d, bool bf16, hipStream_t s);

// Allocation-free decode: the split partials go to a fixed device array of
// this many bytes (one per GPU, alive until the process ends) instead of a
// caller workspace.  decode_scratch() returns that array's device address on
// the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t decode_scratch(void** ptr);

// Kernel tile geometry, shared with the host for grid sizing.
constexpr int kFwdWaveRows = 32;      // query rows per wave of the 16-bit forward kernel
constexpr int kFwdWideWaveRows = 64;  // rows per wave (two 32-row halves) of the wide 16-bit
                                      // and 8-bit kernels
constexpr int kFwdWaves = 4;          // waves per forward work-group (one per SIMD)
constexpr int kFwdThreads = 64 * kFwdWaves;
// A forward work-group covers gw query heads that share one K/V head (the
// largest of 4, 2, 1 dividing G) and wave_rows * 4 / gw query rows, so its
// waves need the same K/V tiles at the same steps.
inline int fwd_heads_per_wg(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }
inline int fwd_rows_per_wg(int G, int wave_rows) { return wave_rows * kFwdWaves / fwd_heads_per_wg(G); }
// Each forward (16-bit with or without score modifiers, 8-bit) runs on one
// of two kernels, chosen by how many keys a query row sees on average: the
// paired kernel (32-row waves, three work-groups per CU) up to
// kFwdWideMinKeys, the wide kernel (64-row waves) beyond.  sq, sk are the row and
// key counts (packed: their host bounds).  Under a causal mask the rows of
// the last min(sq, sk) positions see a prefix growing to sk keys, on
// average sk - min(sq, sk)/2; a left window bounds a row's keys by
// window_left + 1 (+ window_right without causal).  Measured crossover
// (bf16, d = 128): causal rows of 4096 keys (average 2048) run 2-3 %
// faster on the paired kernel and of 6144 keys (3072) 2 % slower;
// non-causal rows of 3072 keys tie, of 4096 keys the wide kernel is 5 %
// faster.
constexpr int kFwdWideMinKeys = 2560;
inline bool fwd_use_wide(int sq, int sk, int causal, int wl, int wr) {
    long long kpr = sk;
    if (causal) kpr -= (long long)(sq < sk ? sq : sk) / 2;
    if (wl >= 0 && (causal || wr >= 0)) {
        const long long band = (long long)wl + 1 + (causal ? 0 : wr);
        kpr = kpr < band ? kpr : band;
    }
    return kpr > kFwdWideMinKeys;
}
constexpr int kDecodeWaves = 4;    // waves per decode split work-group
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr float kLog2e_host = 1.4426950408889634f;
// dQ work-group: 32 rows per wave, two waves per SIMD; 8 waves split the
// three 8 KB tiles of a d = 128 stage evenly, 4 those of d = 64
constexpr int bwd_dq_waves(int d) { return d == 128 ? 8 : 4; }
constexpr int kBwdDkdvWaves = 8;   // dK/dV work-group: 32 keys per wave, two waves per SIMD
constexpr int kBwdKeysPerWg = 32 * kBwdDkdvWaves;

}  // namespace fa
