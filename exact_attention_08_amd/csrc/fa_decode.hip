// fa_decode.hip -- one-token decode against a KV cache for gfx950, split
// along the cache and merged by the LSE rule: the "FlashAttention" explainer
// page, step 9 (a single query offers little parallelism, so the cache is
// split along the sequence, partial results are computed and combined) and
// "Long context beyond a single GPU" (partials merged with the same online
// softmax rule).
//
// Split kernel: one wave per (split, query block, K/V head, sequence).  The
// wave owns all G = Hq/Hkv query heads that read its K/V head (up to 32 per
// query block), so every cache byte is read exactly once.  Keys are walked
// in blocks of 32; the next block's loads are issued before the current
// block is computed.  The path is HBM-bound (4 FLOP per cache byte at G=4),
// so the MFMA tile is mostly padding and that is fine: S^T = K Q^T and
// O^T = V^T P^T run on v_mfma_f32_32x32x16 with K and V loaded straight from
// HBM into operand registers (no LDS):
//   * K operand: lane (key l%32, half g) reads d-range [g*d/2, (g+1)*d/2)
//     of its key row, one contiguous d-byte run; Q uses the same d order.
//   * V operand: output row m of accumulator db is column m*DB + db, so a
//     lane needs DB adjacent columns of each of its 16 keys: one 2*DB-byte
//     load per key, then 16-bit halves are regrouped in registers.
// Each split writes a normalised fp32 partial O_c and its LSE_c.
//
// Combine kernel: one wave per (sequence, query head); with M = max_c LSE_c,
// w_c = exp(LSE_c - M): LSE = M + ln(sum w_c), O = sum w_c O_c / sum w_c,
// summed in split order (deterministic).
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

constexpr float kDecodeRescaleThreshold = 8.0f;   // log2 units, as in the forward kernel

template <int D, bool BF16>
__global__ __launch_bounds__(64) void fa_decode_split_kernel(DecodeParams p) {
    constexpr int KS = D / 16;          // reduction steps over d
    constexpr int DB = D / 32;          // O^T accumulators
    const int lane = threadIdx.x;
    const int lq = lane & 31, g = lane >> 5;

    int i = blockIdx.x;
    const int split_idx = i % p.nsplit; i /= p.nsplit;
    const int qb = i % p.qblocks; i /= p.qblocks;
    const int hkv = i % p.Hkv;
    const int b = i / p.Hkv;

    const int L = min(max(p.seqlens[b], 0), p.max_len);
    const int nsplit_b = (L + p.split - 1) / p.split;
    if (split_idx >= nsplit_b) return;

    // The query sits at key position L-1: causal and the right window never
    // hide a cached key; the left window hides keys before L-1-wl.
    const int lo = p.wl >= 0 ? max(0, L - 1 - p.wl) : 0;
    const int ka = max(split_idx * p.split, lo);
    const int kb = min((split_idx + 1) * p.split, L);

    const int qh_local = 32 * qb + lq;          // query head within the group
    const bool q_valid = qh_local < p.G;
    const int hq = hkv * p.G + qh_local;

    const long long tok_stride = (long long)p.Hkv * D;
    const uint16_t* kseq = (const uint16_t*)p.k + (long long)b * p.Sk_cap * tok_stride +
                           (long long)hkv * D;
    const uint16_t* vseq = (const uint16_t*)p.v + (long long)b * p.Sk_cap * tok_stride +
                           (long long)hkv * D;

    u32x4 qreg[KS];
    {
        const uint16_t* qrow = (const uint16_t*)p.q + ((long long)b * p.Hq + hq) * D + g * (D / 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = q_valid ? ld_global16(qrow + ks * 8) : (u32x4){0u, 0u, 0u, 0u};
            qreg[ks] = x ^ p.qsign;
        }
    }

    // key (within a 32-key block) of reduction slot sl of step kk for half g
    auto slot_key = [&](int kk, int sl) __attribute__((always_inline)) {
        return 16 * kk + (sl < 4 ? 4 * g + sl : 8 + 4 * g + (sl - 4));
    };

    typedef uint32_t vec_t __attribute__((ext_vector_type(DB / 2)));
    struct Block {
        u32x4 k[KS];
        vec_t v[16];
    };
    auto load_block = [&](Block& blk, int jb) __attribute__((always_inline)) {
        const int jk = jb + lq;
        const bool kin = jk >= ka && jk < kb;
        const uint16_t* krow = kseq + (long long)jk * tok_stride + g * (D / 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            blk.k[ks] = kin ? ld_global16(krow + ks * 8) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                const int j = jb + slot_key(kk, sl);
                const bool vin = j >= ka && j < kb;
                vec_t x;
                for (int w = 0; w < DB / 2; ++w) x[w] = 0u;
                if (vin) x = *reinterpret_cast<const vec_t*>(vseq + (long long)j * tok_stride + lq * DB);
                blk.v[8 * kk + sl] = x;
            }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c = p.c;

    auto process = [&](const Block& cur, int jb) __attribute__((always_inline)) {
        f32x16 s;
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma32x32x16<BF16>(cur.k[ks], qreg[ks], s);

        // element e: key jb + 8*(e>>2) + 4*g + (e&3); visible iff ka <= key < kb
        const int rlo = ka - jb - 4 * g, rhi = kb - 1 - jb - 4 * g;
        const bool edge = jb < ka || jb + 31 >= kb;
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int off = 8 * (e >> 2) + (e & 3);
            const bool vis = !edge || (off >= rlo && off <= rhi);
            mx = fmaxf(mx, vis ? s[e] : -INFINITY);
        }
        mx = fmaxf(mx, xor32(mx));
        const float m_tile = mx == -INFINITY ? -INFINITY : mx * c;
        const float m_new = fmaxf(m_run, m_tile);
        // Per-row decision (rows are independent); the branch only skips
        // the work when no row of the wave needs it.  Rows that keep their
        // max are multiplied by exactly 1.
        const bool raise = m_new > m_run + kDecodeRescaleThreshold;
        if (wave_any(raise)) {
            asm volatile("");   // keep this rare block a real branch (not speculated)
            const float alpha = raise ? exp2_fast(m_run - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            m_run = raise ? m_new : m_run;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;

        u32x4 pb[2];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            float pv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ee = e + u;
                const int off = 8 * (ee >> 2) + (ee & 3);
                const bool vis = !edge || (off >= rlo && off <= rhi);
                const float x = exp2_fast(fmaf(s[ee], c, -m_use));
                pv[u] = vis ? x : 0.f;
                l_run += pv[u];
            }
            pb[e >> 3][(e & 7) >> 1] = pack2<BF16>(pv[0], pv[1]);
        }

        // O^T += V^T P^T ; accumulator db row m is column m*DB + db
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                u32x4 a;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t x0 = cur.v[8 * kk + 2 * w][db >> 1];
                    const uint32_t x1 = cur.v[8 * kk + 2 * w + 1][db >> 1];
                    a[w] = (db & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u))
                                    : ((x0 & 0xffffu) | (x1 << 16));
                }
                oacc[db] = mfma32x32x16<BF16>(a, pb[kk], oacc[db]);
            }
    };

    // two register sets: the next block's loads are in flight while the
    // current block is computed
    const int jfirst = (ka / 32) * 32;
    Block b0, b1;
    if (jfirst < kb) load_block(b0, jfirst);
    for (int jb = jfirst; jb < kb; jb += 64) {
        if (jb + 32 < kb) load_block(b1, jb + 32);
        process(b0, jb);
        if (jb + 32 >= kb) break;
        if (jb + 64 < kb) load_block(b0, jb + 64);
        process(b1, jb + 32);
    }

    // normalised partial of this split
    const float l_tot = l_run + xor32(l_run);
    if (q_valid) {
        const long long row = ((long long)b * p.Hq + hq) * p.nsplit + split_idx;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* orow = p.ws_o + row * D;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int m = 8 * jj + 4 * g + k;
                float vals[DB];
#pragma unroll
                for (int db = 0; db < DB; ++db) vals[db] = oacc[db][4 * jj + k] * inv;
                if constexpr (DB == 4) {
                    *reinterpret_cast<f32x4*>(orow + m * DB) = (f32x4){vals[0], vals[1], vals[2], vals[3]};
                } else {
                    *reinterpret_cast<f32x2*>(orow + m * DB) = (f32x2){vals[0], vals[1]};
                }
            }
        if (g == 0)
            p.ws_lse[row] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
    }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_decode_combine_kernel(DecodeParams p) {
    constexpr int PER = D / 64;        // columns per lane
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w >= p.B * p.Hq) return;
    const int b = w / p.Hq, hq = w - b * p.Hq;
    const int L = min(max(p.seqlens[b], 0), p.max_len);
    const int n = (L + p.split - 1) / p.split;
    const long long row0 = ((long long)b * p.Hq + hq) * p.nsplit;

    float M = -INFINITY;
    for (int s = 0; s < n; ++s) M = fmaxf(M, p.ws_lse[row0 + s]);
    float acc[PER];
    for (int u = 0; u < PER; ++u) acc[u] = 0.f;
    float sum = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < n; ++s) {
            const float ls = p.ws_lse[row0 + s];
            const float wgt = ls == -INFINITY ? 0.f : exp2_fast((ls - M) * kLog2e);
            sum += wgt;
            const float* src = p.ws_o + (row0 + s) * D + lane * PER;
            for (int u = 0; u < PER; ++u) acc[u] = fmaf(wgt, src[u], acc[u]);
        }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    uint16_t* orow = (uint16_t*)p.o + ((long long)b * p.Hq + hq) * D + lane * PER;
    if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t*>(orow) = pack2<BF16>(acc[0] * inv, acc[1] * inv);
    } else {
        const uint32_t pk = pack2<BF16>(acc[0] * inv, 0.f);
        orow[0] = (uint16_t)(pk & 0xffffu);
    }
    if (p.lse != nullptr && lane == 0)
        p.lse[(long long)b * p.Hq + hq] = sum > 0.f ? M + log2_fast(sum) * kLn2 : -INFINITY;
}

template <int D, bool BF16>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
    const long long nsplit_blocks = (long long)p.nsplit * p.qblocks * p.Hkv * p.B;
    hipLaunchKernelGGL((fa_decode_split_kernel<D, BF16>), dim3((unsigned)nsplit_blocks), dim3(64),
                       0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long ncomb = ((long long)p.B * p.Hq + 3) / 4;
    hipLaunchKernelGGL((fa_decode_combine_kernel<D, BF16>), dim3((unsigned)ncomb), dim3(256), 0, s,
                       p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t s) {
    if (d == 128) return bf16 ? launch_decode_t<128, true>(p, s) : launch_decode_t<128, false>(p, s);
    return bf16 ? launch_decode_t<64, true>(p, s) : launch_decode_t<64, false>(p, s);
}

}  // namespace fa
