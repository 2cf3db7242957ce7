// fa_decode.hip -- one-token decode against a KV cache for gfx950, split
// along the cache and merged by the LSE rule: the "FlashAttention" explainer
// page, step 9 (a single query offers little parallelism, so the cache is
// split along the sequence, partial results are computed and combined) and
// "Long context beyond a single GPU" (partials merged with the same online
// softmax rule).
//
// Split kernel: one work-group of four waves per (split, query block of up
// to 16 query heads, K/V head, sequence).  The work-group owns all query
// heads that read its K/V head (G = Hq/Hkv, up to 16 per query block), so
// every cache byte is read exactly once; its waves take interleaved 32-key
// blocks of the split and merge their (m, l, O) partials through LDS at the
// end.  The Hkv heads of one split are adjacent in launch order, so the
// 2 KiB token rows they share stream from HBM at about the same time.  The
// path is HBM-bound (4 FLOP per cache byte at G=4): the MFMA tile is mostly
// padding and that is fine.  S^T = K Q^T and O^T = V^T P^T run on
// v_mfma_f32_16x16x32 (16 query columns):
//   * K: copied HBM -> LDS by buffer_load ... lds, each 1 KiB instruction
//     moving whole rows (whole 128-byte lines; an operand-order register
//     load would touch only 64 bytes per row per instruction, measurably
//     slower).  Rows are XOR-swizzled in 16-byte chunks so the operand
//     reads (lane = key l%16, quarter l/16 = d-chunk 4*ks + l/16) hit all
//     banks once.  Two slots per wave; block t+2 is copied while t+1 is in
//     flight.
//   * V: straight into operand registers: accumulator db row m is column
//     m*(d/16) + db, so a lane needs d/16 adjacent columns of each of its 8
//     keys, one 16-byte (d=128) load per key and 16 lanes covering a whole
//     row; 16-bit halves are regrouped in registers.
// Each split writes a normalised fp32 partial O_c and its LSE_c.
//
// Combine kernel: D/64 waves per (sequence, query head), 64 columns each;
// with M = max_c LSE_c, w_c = exp(LSE_c - M): LSE = M + ln(sum w_c),
// O = sum w_c O_c / sum w_c, summed in split order (deterministic), several
// partial rows in flight.
//
// Paged cache (the project summary lists paged KV cache support for the
// cached-decode call; the explainer advises paged cache layouts): the keys
// of sequence b live in pages of page_size token rows, token t at row
// t % page_size of page block_table[b][t / page_size].  page_size is a multiple of 32, so
// each 32-key block of the split kernel lies in one page and costs one
// table read; the buffer resource of a block then starts at that page row.
// With an append, a small kernel first writes the new token's key and value
// row at position cache_seqlens[b], and the split and combine kernels see
// one more key.
#include <mutex>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

constexpr float kDecodeRescaleThreshold = 8.0f;   // log2 units, as in the forward kernel

// Keys sequence b attends over: its cache length clamped to [0, max_len], or
// with an append the clamped position of the new token plus one.
__device__ __forceinline__ int decode_len(const DecodeParams& p, int b) {
    const int s = p.seqlens[b];
    return p.append ? min(max(s, 0), p.max_len - 1) + 1 : min(max(s, 0), p.max_len);
}

// The new token's key and value rows into their page (one thread per
// 16-byte chunk of a (sequence, K/V head) row).  A table entry outside the
// pool writes nothing.
template <int D>
__global__ __launch_bounds__(256) void fa_decode_append_kernel(DecodeParams p) {
    constexpr int CH = D / 8;
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= (long long)p.B * p.Hkv * CH) return;
    const int c = (int)(t % CH);
    const long long bh = t / CH;
    const int hkv = (int)(bh % p.Hkv), b = (int)(bh / p.Hkv);
    const int pos = decode_len(p, b) - 1;
    const int pg = pos / p.page_size;
    const int phys = p.block_table[(long long)b * p.max_pages + pg];
    if (phys < 0 || phys >= p.num_pages) return;
    const long long row = (long long)phys * p.page_size + (pos - pg * p.page_size);
    const long long dst = (row * p.Hkv + hkv) * D + c * 8;
    const long long src = ((long long)b * p.Hkv + hkv) * D + c * 8;
    *reinterpret_cast<u32x4*>((uint16_t*)const_cast<void*>(p.k) + dst) =
        *reinterpret_cast<const u32x4*>((const uint16_t*)p.k_new + src);
    *reinterpret_cast<u32x4*>((uint16_t*)const_cast<void*>(p.v) + dst) =
        *reinterpret_cast<const u32x4*>((const uint16_t*)p.v_new + src);
}

template <int D, bool BF16, bool PAGED>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(2)))
void fa_decode_split_kernel(DecodeParams p) {
    constexpr int KS = D / 32;            // reduction steps over d (16x16x32)
    constexpr int DB = D / 16;            // O^T accumulators (16 columns each)
    constexpr int NW = kDecodeWaves;
    constexpr int ROWB = 2 * D;           // bytes of one head's key row
    constexpr int CH = D / 8;             // 16-byte chunks per row
    constexpr int RPI = 1024 / ROWB;      // rows per 1 KiB DMA instruction
    constexpr int SLOT = 32 * ROWB;       // one 32-key K block in LDS
    constexpr int NKI = SLOT / 1024;      // DMA instructions per K block
    constexpr int NVI = 8;                // V loads per block (one per key slot)
    constexpr int RING = NW * 2 * SLOT;   // two K slots per wave
    constexpr int RED = NW * 16 * (D + 4) * 4;
    __shared__ __attribute__((aligned(16))) unsigned char lds[RING > RED ? RING : RED];
    __shared__ float red_s[NW][3][16];    // per-wave m, l (fp32), l (16-bit weights)

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int lq = lane & 15, q4 = lane >> 4;

    // the Hkv heads of one chunk are adjacent in launch order, so the whole
    // token rows they share are streamed at about the same time
    int i = blockIdx.x;
    const int hkv = i % p.Hkv; i /= p.Hkv;
    const int qb = i % p.qblocks; i /= p.qblocks;
    const int split_idx = i % p.nsplit;
    const int b = i / p.nsplit;
    const int L = decode_len(p, b);
    if (split_idx >= (L + p.split - 1) / p.split) return;   // uniform over the work-group

    // The query sits at key position L-1: causal and the right window never
    // hide a cached key; the left window hides keys before L-1-wl.
    const int lo = p.wl >= 0 ? max(0, L - 1 - p.wl) : 0;
    const int ka = max(split_idx * p.split, lo);
    const int kb = min((split_idx + 1) * p.split, L);

    const int qh_local = 16 * qb + lq;          // query head within the group
    const bool q_valid = qh_local < p.G;
    const int hq = hkv * p.G + qh_local;

    const int tok_bytes = p.Hkv * ROWB;
    const long long seq_bytes = (long long)b * p.Sk_cap * tok_bytes;

    // d order of the Q.K reduction: step ks, quarter q4 covers d-chunk
    // 4*ks + q4 (8 values); Q and K use the same order.
    u32x4 qreg[KS];
    {
        // rows of padding heads read as zeros
        const auto qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const uint16_t*)p.q + ((long long)b * p.Hq + hkv * p.G + 16 * qb) * D),
            (short)0, min(16, p.G - 16 * qb) * ROWB, 0x00020000);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qrs, lq * ROWB + (4 * ks + q4) * 16, 0, 0);
            qreg[ks] = x ^ p.qsign;
        }
    }

    // Buffer resource over keys [jb, kb) of this sequence (all heads); rows
    // at or past kb read as zeros, so no load leaves the cache (a block past
    // kb reads nothing at all).  Paged: the 32 keys of block jb lie in one
    // page; the resource starts at the block's row of that page and covers
    // at most 32 rows; a block past kb reads no table entry, and a table
    // entry outside the pool reads zeros.
    struct Span { const char* ptr; int bytes; };
    auto block_span = [&](const void* base, int jb) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            int rows = min(kb - jb, 32);
            long long off = 0;
            if (rows > 0) {
                const int pg = jb / p.page_size;
                const int phys = p.block_table[(long long)b * p.max_pages + pg];
                if (phys >= 0 && phys < p.num_pages)
                    off = ((long long)phys * p.page_size + (jb - pg * p.page_size)) * tok_bytes;
                else
                    rows = 0;
            } else {
                rows = 0;
            }
            return Span{(const char*)base + off, rows * tok_bytes};
        } else {
            return Span{(const char*)base + seq_bytes + (long long)jb * tok_bytes,
                        max(kb - jb, 0) * tok_bytes};
        }
    };
    auto block_rsrc = [&](const void* base, int jb) __attribute__((always_inline)) {
        const Span sp = block_span(base, jb);
        return make_rsrc(sp.ptr, sp.bytes);
    };
    // K rows in LDS: 16-byte chunk c of row r sits at chunk slot c ^ swz(r),
    // so the 16 rows one MFMA operand read touches hit 16 distinct bank
    // groups.
    auto swz = [](int r) __attribute__((always_inline)) {
        return (r / (256 / ROWB)) & (CH - 1);
    };
    const uint32_t ring = lds_addr(lds) + wave * 2 * SLOT;
    // K block at key jb into this wave's slot s: each 1 KiB instruction
    // copies RPI whole rows (whole 128-byte lines from HBM).
    auto dma_k = [&](int jb, int s) __attribute__((always_inline)) {
        const i32x4 rs = block_rsrc(p.k, jb);
#pragma unroll
        for (int t = 0; t < NKI; ++t) {
            const int r = t * RPI + lane / CH;
            const int c = (lane % CH) ^ swz(r);
            dma16_to_lds(rs, ring + s * SLOT + t * 1024, r * tok_bytes + hkv * ROWB + c * 16, 0);
        }
    };

    // key (within a 32-key block) of P.V reduction slot sl for this quarter
    auto slot_key = [&](int sl) __attribute__((always_inline)) {
        return sl < 4 ? 4 * q4 + sl : 16 + 4 * q4 + (sl - 4);
    };
    typedef uint32_t vec_t __attribute__((ext_vector_type(DB / 2)));
    struct VBlock { vec_t v[8]; };      // this lane's 8 keys x DB columns
    // V straight into operand registers: lane lq reads DB adjacent columns,
    // 16 lanes a whole row.  Keys before ka read as zeros (offset past the
    // resource), keys at or past kb through the resource bound.
    auto load_v = [&](VBlock& blk, int jb) __attribute__((always_inline)) {
        const Span sp = block_span(p.v, jb);
        const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)sp.ptr, (short)0, sp.bytes, 0x00020000);
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            const int r = slot_key(sl);
            const int off = jb + r < ka ? 0x7ffffff0 : r * tok_bytes + hkv * ROWB + lq * DB * 2;
            if constexpr (DB == 8)
                blk.v[sl] = __builtin_bit_cast(vec_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
            else
                blk.v[sl] = __builtin_bit_cast(vec_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
        }
    };

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f, lr_run = 0.f;
    const float c = p.c;

    auto process = [&](int s, const VBlock& vb, int jb) __attribute__((always_inline)) {
        const unsigned char* kbase = lds + (wave * 2 + s) * SLOT;
        f32x4 sc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 16 * h + lq;
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[h][e] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 kr = *reinterpret_cast<const u32x4*>(
                    kbase + r * ROWB + (((4 * ks + q4) ^ swz(r)) * 16));
                sc[h] = mfma16x16x32<BF16>(kr, qreg[ks], sc[h]);
            }
        }
        // element e of half h: key jb + 16*h + 4*q4 + e; visible iff ka <= key < kb
        const int rlo = ka - jb - 4 * q4, rhi = kb - 1 - jb - 4 * q4;
        const bool edge = jb < ka || jb + 31 >= kb;
        if (edge) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int off = 16 * h + e;
                    sc[h][e] = (off >= rlo && off <= rhi) ? sc[h][e] : -INFINITY;
                }
        }
        float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                         fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run, mx * c);
        // Per-row decision (rows are independent); rows keeping their max are
        // multiplied by exactly 1.
        const bool raise = m_new > m_run + kDecodeRescaleThreshold;
        if (wave_any(raise)) {
            asm volatile("");   // keep this rare block a real branch (not speculated)
            const float alpha = raise ? exp2_fast(m_run - m_new) : 1.f;
            l_run *= alpha;
            lr_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e) oacc[db][e] *= alpha;
            m_run = raise ? m_new : m_run;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;

        // P^T as the B operand: slots 0-3 are half 0, slots 4-7 half 1
        u32x4 pb;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                const float x0 = exp2_fast(fmaf(sc[h][e], c, -m_use));
                const float x1 = exp2_fast(fmaf(sc[h][e + 1], c, -m_use));
                const uint32_t pk = pack2<BF16>(x0, x1);
                pb[2 * h + (e >> 1)] = pk;
                l_run += x0 + x1;
                lr_run = sum2_16<BF16>(pk, lr_run);
            }

        // O^T += V^T P^T ; accumulator db row m is column m*DB + db
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u32x4 a;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t x0 = vb.v[2 * w][db >> 1];
                const uint32_t x1 = vb.v[2 * w + 1][db >> 1];
                a[w] = (db & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
            }
            oacc[db] = mfma16x16x32<BF16>(a, pb, oacc[db]);
        }
    };

    // This wave's blocks are jfirst + STEP*t, t < nb.  K of block t goes to
    // slot t%2 two blocks ahead; V of block t+1 is loaded while block t is
    // computed.  Issue order: K0 K1 V0 | V1 K2 | V2 K3 | ...  Every
    // iteration issues its V loads (past the last block they read nothing),
    // so the count of loads issued after block t's K is known: V(t), V(t+1)
    // and, while t+1 < nb, K(t+1).  The explicit vmcnt waits count them; the
    // compiler tracks the V loads but not the K copies, so its own waits for
    // V only ever wait for more.
    const int jfirst = (ka / 32) * 32 + 32 * wave;
    constexpr int STEP = 32 * NW;
    const int nb = jfirst < kb ? (kb - 1 - jfirst) / STEP + 1 : 0;
    VBlock va, vb;
    if (nb > 0) dma_k(jfirst, 0);
    if (nb > 1) dma_k(jfirst + STEP, 1);
    load_v(va, jfirst);
    auto iter = [&](int t, VBlock& cur, VBlock& next) __attribute__((always_inline)) {
        const int jb = jfirst + t * STEP;
        const int s = t & 1;
        load_v(next, jb + STEP);
        if (t + 1 < nb)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(FA_VMCNT(2 * NVI + NKI)) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(FA_VMCNT(2 * NVI)) : "memory");
        process(s, cur, jb);
        if (t + 2 < nb) {
            // the slot's K reads were consumed by the MFMAs above
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            dma_k(jb + 2 * STEP, s);
        }
    };
    // (no exit in the middle of the unrolled pair: the compiler's view of
    // which V loads are pending stays exact at the loop head)
    for (int t = 0; t + 1 < nb; t += 2) {
        iter(t, va, vb);
        iter(t + 1, vb, va);
    }
    if (nb & 1) iter(nb - 1, va, vb);

    // ---- merge the waves' partials (same rule as the combine kernel) ------
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += xor32(l_tot);
    float lr_tot = lr_run + __shfl_xor(lr_run, 16, 64);
    lr_tot += xor32(lr_tot);
    // the partials reuse the K ring: every wave must be done with it
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    float* red_o = reinterpret_cast<float*>(lds);     // [NW][16][D + 4]
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int m = 4 * q4 + k;
#pragma unroll
        for (int db = 0; db < DB; ++db) red_o[(wave * 16 + lq) * (D + 4) + m * DB + db] = oacc[db][k];
    }
    if (q4 == 0) {
        red_s[wave][0][lq] = m_run;
        red_s[wave][1][lq] = l_tot;
        red_s[wave][2][lq] = lr_tot;
    }
    __syncthreads();
    // thread t: query t / 16, columns t % 16 + 16*u (16 lanes store 64
    // contiguous bytes of one partial row)
    static_assert(NW * 64 == 16 * 16, "the merge maps the work-group's threads to 16 queries x 16 columns");
    const int tq = threadIdx.x >> 4, tc = threadIdx.x & 15;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_s[w][0][tq]);
    float wgt[NW], Lf = 0.f, Lr = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float mw = red_s[w][0][tq];
        wgt[w] = mw == -INFINITY ? 0.f : exp2_fast(mw - M);
        Lf = fmaf(wgt[w], red_s[w][1][tq], Lf);
        Lr = fmaf(wgt[w], red_s[w][2][tq], Lr);
    }
    const int tqh = 16 * qb + tq;
    if (tqh < p.G) {
        const int thq = hkv * p.G + tqh;
        const long long row = ((long long)b * p.Hq + thq) * p.nsplit + split_idx;
        const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
        float* orow = p.ws_o + row * D;
        for (int col = tc; col < D; col += 64 * NW / 16) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) acc = fmaf(wgt[w], red_o[(w * 16 + tq) * (D + 4) + col], acc);
            orow[col] = acc * inv;
        }
        if (tc == 0)
            p.ws_lse[row] = Lf > 0.f ? (M + log2_fast(Lf)) * kLn2 : -INFINITY;
    }
}

// Lane l of wave part owns column 64 part + l.  (Two waves per 128-column
// row rather than one: the kernel is latency bound, and twice the waves in
// flight take ~2 us off its ~9 us.)
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_decode_combine_kernel(DecodeParams p) {
    constexpr int CW = D / 64;         // waves per row
    constexpr int UNROLL = 32;         // partial rows in flight per lane
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int w = wv / CW, part = wv % CW;
    const int lane = threadIdx.x & 63;
    if (w >= p.B * p.Hq) return;
    const int b = w / p.Hq, hq = w - b * p.Hq;
    const int L = decode_len(p, b);
    const int n = (L + p.split - 1) / p.split;
    const long long row0 = ((long long)b * p.Hq + hq) * p.nsplit;
    const float* src = p.ws_o + row0 * D + part * 64 + lane;

    // The first 64 LSEs (lane s: split s) and the first UNROLL partial rows
    // are requested together: the rows do not depend on the weights.
    float lse0 = lane < n ? p.ws_lse[row0 + lane] : -INFINITY;
    float x0[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) x0[k] = k < n ? src[(long long)k * D] : 0.f;

    // M = max_c LSE_c, lanes over splits
    float M = lse0;
    for (int s0 = 64; s0 < n; s0 += 64)
        if (s0 + lane < n) M = fmaxf(M, p.ws_lse[row0 + s0 + lane]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));

    float acc = 0.f, sum = 0.f;
    if (M != -INFINITY) {
        // lane s holds the weight of split s0 + s; the sums below run in
        // split order (deterministic)
        auto weight = [&](float ls) { return ls == -INFINITY ? 0.f : exp2_fast((ls - M) * kLog2e); };
        auto add_row = [&](float wl, int k, float x) __attribute__((always_inline)) {
            const float wk = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), k));
            sum += wk;
            acc = fmaf(wk, x, acc);
        };
        float wl = weight(lse0);
#pragma unroll
        for (int k = 0; k < UNROLL; ++k)
            if (k < n) add_row(wl, k, x0[k]);
        for (int s0 = 0; s0 < n; s0 += 64) {
            if (s0 > 0) wl = s0 + lane < n ? weight(p.ws_lse[row0 + s0 + lane]) : 0.f;
            const int m = min(64, n - s0);
            for (int c0 = s0 == 0 ? UNROLL : 0; c0 < m; c0 += UNROLL) {
                float x[UNROLL];
#pragma unroll
                for (int k = 0; k < UNROLL; ++k)
                    x[k] = c0 + k < m ? src[(long long)(s0 + c0 + k) * D] : 0.f;
#pragma unroll
                for (int k = 0; k < UNROLL; ++k)
                    if (c0 + k < m) add_row(wl, c0 + k, x[k]);
            }
        }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    uint16_t* orow = (uint16_t*)p.o + ((long long)b * p.Hq + hq) * D + part * 64 + lane;
    *orow = (uint16_t)(pack2<BF16>(acc * inv, 0.f) & 0xffffu);
    if (p.lse != nullptr && lane == 0 && part == 0)
        p.lse[(long long)b * p.Hq + hq] = sum > 0.f ? M + log2_fast(sum) * kLn2 : -INFINITY;
}

template <int D, bool BF16>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
    if (p.append) {
        const long long n = (long long)p.B * p.Hkv * (D / 8);
        hipLaunchKernelGGL((fa_decode_append_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                           0, s, p);
    }
    const long long nsplit_blocks = (long long)p.nsplit * p.qblocks * p.Hkv * p.B;
    if (p.block_table != nullptr)
        hipLaunchKernelGGL((fa_decode_split_kernel<D, BF16, true>), dim3((unsigned)nsplit_blocks),
                           dim3(kDecodeThreads), 0, s, p);
    else
        hipLaunchKernelGGL((fa_decode_split_kernel<D, BF16, false>), dim3((unsigned)nsplit_blocks),
                           dim3(kDecodeThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long ncomb = ((long long)p.B * p.Hq * (D / 64) + 3) / 4;
    hipLaunchKernelGGL((fa_decode_combine_kernel<D, BF16>), dim3((unsigned)ncomb), dim3(256), 0, s,
                       p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t s) {
    if (d == 128) return bf16 ? launch_decode_t<128, true>(p, s) : launch_decode_t<128, false>(p, s);
    return bf16 ? launch_decode_t<64, true>(p, s) : launch_decode_t<64, false>(p, s);
}

// Split partials of the allocation-free decode entry point.  Every GPU the
// library runs on holds its own copy until the process ends, and every such
// call on that GPU shares it, so calls that overlap on one GPU race.
// Nothing in it needs to start at zero: the split kernel writes every
// partial row and LSE that the combine kernel then reads.  Host code must
// not pass this name to a kernel (on the host it is only a stand-in): the
// device address comes from decode_scratch().
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // with this device current: its own copy of the array
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace fa
