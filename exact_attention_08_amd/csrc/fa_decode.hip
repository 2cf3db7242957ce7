// fa_decode.hip -- one-token decode against a KV cache for gfx950, split
// along the cache and merged by the LSE rule: the "FlashAttention" explainer
// page, step 9 (a single query offers little parallelism, so the cache is
// split along the sequence, partial results are computed and combined) and
// "Long context beyond a single GPU" (partials merged with the same online
// softmax rule).
//
// Split kernel: one wave per (split, query block of up to 16 query heads,
// K/V head, sequence).  The wave owns all query heads that read its K/V head
// (G = Hq/Hkv, up to 16 per query block), so every cache byte is read exactly
// once.  Keys are walked in blocks of 32; the next block's loads are issued
// before the current block is computed.  The path is HBM-bound (4 FLOP per
// cache byte at G=4), so the MFMA tile is mostly padding and that is fine:
// S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_16x16x32 (16 query
// columns: little register space is spent on padding) with K and V loaded
// straight from HBM into operand registers (no LDS):
//   * K operand: lane (key l%16, quarter q = l/16) reads d-range
//     [q*d/4, (q+1)*d/4) of its key row, one contiguous run; Q uses the same
//     d order.
//   * V operand: accumulator db row m is column m*(d/16) + db, so a lane
//     needs d/16 adjacent columns of each of its 8 keys: one 16-byte (d=128)
//     load per key, 16 lanes covering a whole 256-byte row; 16-bit halves are
//     regrouped in registers.
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
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void fa_decode_split_kernel(DecodeParams p) {
    constexpr int KS = D / 32;          // reduction steps over d (16x16x32)
    constexpr int DQ = D / 4;           // d-range per lane quarter
    constexpr int DB = D / 16;          // O^T accumulators (16 columns each)
    const int lane = threadIdx.x;
    const int lq = lane & 15, q4 = lane >> 4;

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

    const int qh_local = 16 * qb + lq;          // query head within the group
    const bool q_valid = qh_local < p.G;
    const int hq = hkv * p.G + qh_local;

    const long long tok_stride = (long long)p.Hkv * D;
    const uint16_t* kseq = (const uint16_t*)p.k + (long long)b * p.Sk_cap * tok_stride +
                           (long long)hkv * D;
    const uint16_t* vseq = (const uint16_t*)p.v + (long long)b * p.Sk_cap * tok_stride +
                           (long long)hkv * D;

    u32x4 qreg[KS];
    {
        const uint16_t* qrow = (const uint16_t*)p.q + ((long long)b * p.Hq + hq) * D + q4 * DQ;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = q_valid ? ld_global16(qrow + ks * 8) : (u32x4){0u, 0u, 0u, 0u};
            qreg[ks] = x ^ p.qsign;
        }
    }

    // key (within a 32-key block) of P.V reduction slot sl for this quarter
    auto slot_key = [&](int sl) __attribute__((always_inline)) {
        return sl < 4 ? 4 * q4 + sl : 16 + 4 * q4 + (sl - 4);
    };

    typedef uint32_t vec_t __attribute__((ext_vector_type(DB / 2)));
    struct Block {
        u32x4 k[2][KS];                 // two 16-key halves
        vec_t v[8];                     // this lane's 8 keys x DB columns
    };
    auto load_block = [&](Block& blk, int jb) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int jk = jb + 16 * h + lq;
            const bool kin = jk >= ka && jk < kb;
            const uint16_t* krow = kseq + (long long)jk * tok_stride + q4 * DQ;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                blk.k[h][ks] = kin ? ld_global16(krow + ks * 8) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            const int j = jb + slot_key(sl);
            const bool vin = j >= ka && j < kb;
            vec_t x;
#pragma unroll
            for (int w = 0; w < DB / 2; ++w) x[w] = 0u;
            if (vin) x = *reinterpret_cast<const vec_t*>(vseq + (long long)j * tok_stride + lq * DB);
            blk.v[sl] = x;
        }
    };

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f, lr_run = 0.f;
    const float c = p.c;

    auto process = [&](const Block& cur, int jb) __attribute__((always_inline)) {
        f32x4 s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s[h][e] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) s[h] = mfma16x16x32<BF16>(cur.k[h][ks], qreg[ks], s[h]);
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
                    s[h][e] = (off >= rlo && off <= rhi) ? s[h][e] : -INFINITY;
                }
        }
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
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
                const float x0 = exp2_fast(fmaf(s[h][e], c, -m_use));
                const float x1 = exp2_fast(fmaf(s[h][e + 1], c, -m_use));
                const uint32_t pk = pack2<BF16>(x0, x1);
                pb[2 * h + (e >> 1)] = pk;
                l_run += x0 + x1;
                lr_run = dot2_ones<BF16>(pk, lr_run);
            }

        // O^T += V^T P^T ; accumulator db row m is column m*DB + db
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u32x4 a;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t x0 = cur.v[2 * w][db >> 1];
                const uint32_t x1 = cur.v[2 * w + 1][db >> 1];
                a[w] = (db & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
            }
            oacc[db] = mfma16x16x32<BF16>(a, pb, oacc[db]);
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

    // normalised partial of this split (O by the sum of the 16-bit weights,
    // LSE by the fp32 sum, as in the forward kernel)
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += xor32(l_tot);
    float lr_tot = lr_run + __shfl_xor(lr_run, 16, 64);
    lr_tot += xor32(lr_tot);
    if (q_valid) {
        const long long row = ((long long)b * p.Hq + hq) * p.nsplit + split_idx;
        const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
        float* orow = p.ws_o + row * D;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int m = 4 * q4 + k;
#pragma unroll
            for (int d4 = 0; d4 < DB; d4 += 4)
                *reinterpret_cast<f32x4*>(orow + m * DB + d4) =
                    (f32x4){oacc[d4][k] * inv, oacc[d4 + 1][k] * inv, oacc[d4 + 2][k] * inv,
                            oacc[d4 + 3][k] * inv};
        }
        if (q4 == 0)
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
