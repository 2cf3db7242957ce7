// fa_fwd.hip -- fused exact-attention forward for gfx950 (padded and packed).
//
// One work-group = 4 waves = 128 query rows of one (sequence, query head);
// each wave owns 32 rows.  The key axis is walked in tiles of BN keys
// (64 for d=128, 128 for d=64): the "FlashAttention" explainer page, steps 1-4
// (tile, score the tile on chip, online softmax, accumulate and normalise
// once), step 5 (the per-row LSE), step 6 (whole tiles outside the causal /
// window band are skipped, only boundary tiles are masked element-wise),
// step 7 (work-groups over query tiles x heads x batch) and step 8 (16-bit
// MFMA operands, fp32 accumulators and fp32 softmax statistics).
//
// Orientation.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16: the A operand is a 32-key slice of K read from LDS,
// the B operand is the wave's 32 query rows (kept in registers for the whole
// kernel).  In the accumulator each lane then holds ONE query row and 16 keys
// of it, so the row max and row sum are in-lane reductions plus a single
// exchange with lane l^32.  The probabilities are already in the B-operand
// layout of the second product O^T = V^T P^T, so P never leaves registers.
// V is stored transposed in LDS (V^T, written once per tile by the staging
// threads), so the A operand of the second product is one 16-byte LDS read.
//
// Online softmax in base 2: scores are scaled by c = |scale|*log2(e) inside
// one FMA feeding v_exp_f32.  The running max is only raised when a row's
// tile max exceeds it by more than 2^8 (exp2 argument 8); until then the
// stale max is kept, which is exact because the same max is used for the
// numerator, the sum and the final LSE.  This skips most O rescales.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <int D>
struct FwdTile {
    static constexpr int BM = kFwdBM;           // rows per work-group
    static constexpr int BN = 8192 / D;         // keys per tile
    static constexpr int NB = BN / 32;          // S^T accumulators (32 keys each)
    static constexpr int KS = D / 16;           // reduction steps over d
    static constexpr int DB = D / 32;           // O^T accumulators (32 columns each)
    static constexpr int KK = BN / 16;          // reduction steps over keys
    static constexpr int K_STRIDE = D + 8;      // LDS row stride of K (16-bit elements)
    static constexpr int VT_STRIDE = BN + 8;    // LDS row stride of V^T
    static constexpr int K_LDS = BN * K_STRIDE;
    static constexpr int VT_LDS = D * VT_STRIDE;
    static constexpr int K_CHUNKS = BN * D / 8 / 256;   // 16-byte K chunks per thread
    static constexpr int DG = D / 4;            // V staging: groups of 4 columns
    static_assert(K_CHUNKS == 4, "staging assumes 4 K chunks per thread");
    static_assert((256 / DG) * 8 == BN, "staging assumes 8 keys per thread");
};

constexpr float kRescaleThreshold = 8.0f;       // log2 units

template <int D, bool BF16, bool VARLEN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_kernel(FwdParams p) {
    using T = FwdTile<D>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[T::K_LDS];
    __shared__ __attribute__((aligned(16))) uint16_t lds_vt[T::VT_LDS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lq = lane & 31;          // query column of this lane
    const int g = lane >> 5;           // half of the wave

    // ---- work-group -> (query tile, head, sequence) ----------------------
    int t, hq, b;
    {
        const int i = blockIdx.x;
        if (p.xcd_groups > 0) {
            // Keep the G query heads of one K/V head (and its neighbouring
            // query tiles) on one XCD: work-group i runs on XCD i % 8.
            const int xcd = i & 7, r = i >> 3;
            const int per_row = p.xcd_groups * p.G;
            const int trev = r / per_row, rem = r - trev * per_row;
            const int jgrp = rem / p.G, gq = rem - jgrp * p.G;
            const int grp = xcd + 8 * jgrp;
            b = grp / p.Hkv;
            hq = (grp - b * p.Hkv) * p.G + gq;
            t = p.nqt - 1 - trev;
        } else {
            const int per_row = p.B * p.Hq;
            const int trev = i / per_row, rem = i - trev * per_row;
            b = rem / p.Hq;
            hq = rem - b * p.Hq;
            t = p.nqt - 1 - trev;
        }
    }
    const int hkv = hq / p.G;

    long long q_tok0, k_tok0;
    int sq, sk;
    if constexpr (VARLEN) {
        const int qa = p.cu_q[b], qb = p.cu_q[b + 1];
        const int ka = p.cu_k[b], kb = p.cu_k[b + 1];
        q_tok0 = qa; sq = qb - qa;
        k_tok0 = ka; sk = kb - ka;
    } else {
        q_tok0 = (long long)b * p.Sq; sq = p.Sq;
        k_tok0 = (long long)b * p.Sk; sk = p.Sk;
    }
    const int q0 = t * T::BM;
    if (q0 >= sq) return;                      // uniform over the work-group
    const int delta = sk - sq;
    const int causal = p.causal, wl = p.wl, wr = p.wr;

    // visible key interval [lo(i), hi(i)] of query row i (both nondecreasing in i)
    auto lo_of = [&](int i) { return wl >= 0 ? max(0, i + delta - wl) : 0; };
    auto hi_of = [&](int i) {
        int h = sk - 1;
        if (causal) h = min(h, i + delta);
        if (wr >= 0) h = min(h, i + delta + wr);
        return h;
    };

    const int wg_last = min(q0 + T::BM, sq) - 1;
    const int kv_lo = lo_of(q0), kv_hi = hi_of(wg_last);
    const int tile_lo = kv_lo / T::BN;
    const int tile_hi = kv_hi >= kv_lo ? kv_hi / T::BN : tile_lo - 1;

    // this wave's rows and key bounds
    const int r0 = q0 + 32 * wave;
    const bool wave_active = r0 < sq;
    const int r1 = min(r0 + 31, sq - 1);
    const int w_lo = lo_of(r0), w_hi = wave_active ? hi_of(r1) : -1;
    const int int_lo = lo_of(r1), int_hi = hi_of(r0);   // keys every row of the wave sees

    const uint16_t* kbase = (const uint16_t*)p.k + k_tok0 * p.kv_tok_stride + (long long)hkv * D;
    const uint16_t* vbase = (const uint16_t*)p.v + k_tok0 * p.kv_tok_stride + (long long)hkv * D;

    // ---- staging registers: one K/V tile in flight -----------------------
    u32x4 kreg[T::K_CHUNKS];
    u32x2 vreg[8];
    const int v_dg = tid % T::DG;              // columns 4*v_dg .. +3
    const int v_kg = tid / T::DG;              // LDS key positions 8*v_kg .. +7
    auto vkey = [&](int pidx) {                // key (within the tile) at LDS position
        const int grp16 = v_kg >> 1, gg = v_kg & 1;
        return 16 * grp16 + (pidx < 4 ? 4 * gg + pidx : 8 + 4 * gg + (pidx - 4));
    };

    auto load_tile = [&](int jt) {
        const int j0 = jt * T::BN;
#pragma unroll
        for (int c = 0; c < T::K_CHUNKS; ++c) {
            const int chunk = tid + 256 * c;
            const int row = chunk / (D / 8), col = chunk % (D / 8);
            const int j = j0 + row;
            kreg[c] = j < sk ? ld_global16(kbase + (long long)j * p.kv_tok_stride + col * 8)
                             : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            const int j = j0 + vkey(pi);
            vreg[pi] = j < sk ? ld_global8(vbase + (long long)j * p.kv_tok_stride + v_dg * 4)
                              : (u32x2){0u, 0u};
        }
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int c = 0; c < T::K_CHUNKS; ++c) {
            const int chunk = tid + 256 * c;
            const int row = chunk / (D / 8), col = chunk % (D / 8);
            *reinterpret_cast<u32x4*>(&lds_k[row * T::K_STRIDE + col * 8]) = kreg[c];
        }
        // transpose 8 keys x 4 columns into 4 rows of V^T (8 keys each)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            u32x4 w;
#pragma unroll
            for (int p2 = 0; p2 < 4; ++p2) {
                const uint32_t a = (cc >> 1) ? vreg[2 * p2].y : vreg[2 * p2].x;
                const uint32_t bb = (cc >> 1) ? vreg[2 * p2 + 1].y : vreg[2 * p2 + 1].x;
                w[p2] = (cc & 1) ? ((a >> 16) | (bb & 0xffff0000u))
                                 : ((a & 0xffffu) | (bb << 16));
            }
            *reinterpret_cast<u32x4*>(&lds_vt[(4 * v_dg + cc) * T::VT_STRIDE + v_kg * 8]) = w;
        }
    };

    if (tile_lo <= tile_hi) {
        load_tile(tile_lo);
        store_tile();
    }

    // ---- the wave's 32 query rows as MFMA B operands ---------------------
    const int my_row = r0 + lq;
    const uint16_t* qrow = (const uint16_t*)p.q + (q_tok0 + my_row) * p.q_tok_stride +
                           (long long)hq * D;
    u32x4 qreg[T::KS];
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
        u32x4 x = my_row < sq ? ld_global16(qrow + ks * 16 + g * 8) : (u32x4){0u, 0u, 0u, 0u};
        qreg[ks] = x ^ p.qsign;                // exact negation when scale < 0
    }

    f32x16 oacc[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY;                   // running max of scaled scores (log2 units)
    float l_run = 0.f;                         // this lane's share of the running sum
    const float c = p.c;

    // per-lane visible interval, relative to the lane's first key offset 4*g
    const int my_pos = my_row + delta;
    int my_lo = wl >= 0 ? my_pos - wl : -0x40000000;
    int my_hi = sk - 1;
    if (causal) my_hi = min(my_hi, my_pos);
    if (wr >= 0) my_hi = min(my_hi, my_pos + wr);

    for (int jt = tile_lo; jt <= tile_hi; ++jt) {
        __syncthreads();                       // tile jt is in LDS
        if (jt < tile_hi) load_tile(jt + 1);   // next tile in flight during compute

        const int j0 = jt * T::BN;
        const int j1 = j0 + T::BN - 1;
        if (wave_active && j0 <= w_hi && j1 >= w_lo) {
            // S^T = K Q^T
            f32x16 s[T::NB];
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb) {
                for (int e = 0; e < 16; ++e) s[nb][e] = 0.f;
#pragma unroll
                for (int ks = 0; ks < T::KS; ++ks) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(
                        &lds_k[(32 * nb + lq) * T::K_STRIDE + ks * 16 + g * 8]);
                    s[nb] = mfma32x32x16<BF16>(a, qreg[ks], s[nb]);
                }
            }

            const bool masked = !(j0 >= int_lo && j1 <= int_hi);
            // key of element e in block nb: j0 + 32*nb + 8*(e>>2) + 4*g + (e&3)
            const int rel_lo = my_lo - j0 - 4 * g;
            const int rel_hi = my_hi - j0 - 4 * g;

            float mx = -INFINITY;
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int off = 32 * nb + 8 * (e >> 2) + (e & 3);
                    const bool vis = !masked || (off >= rel_lo && off <= rel_hi);
                    mx = fmaxf(mx, vis ? s[nb][e] : -INFINITY);
                }
            mx = fmaxf(mx, xor32(mx));
            const float m_tile = mx == -INFINITY ? -INFINITY : mx * c;
            const float m_new = fmaxf(m_run, m_tile);
            // Per-row decision (rows are independent); the branch only skips
            // the work when no row of the wave needs it.  Rows that keep their
            // max are multiplied by exactly 1.
            const bool raise = m_new > m_run + kRescaleThreshold;
            if (wave_any(raise)) {
                const float alpha = raise ? exp2_fast(m_run - m_new) : 1.f;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < T::DB; ++db)
                    for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
                m_run = raise ? m_new : m_run;
            }
            const float m_use = m_run == -INFINITY ? 0.f : m_run;

            // P = exp2(S*c - m), packed to 16-bit B operands of O^T = V^T P^T
            u32x4 pb[T::KK];
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    float pv[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int ee = e + u;
                        const int off = 32 * nb + 8 * (ee >> 2) + (ee & 3);
                        const bool vis = !masked || (off >= rel_lo && off <= rel_hi);
                        const float x = exp2_fast(fmaf(s[nb][ee], c, -m_use));
                        pv[u] = vis ? x : 0.f;
                        l_run += pv[u];
                    }
                    // element e of block nb is slot (e & 7) of reduction step 2*nb + (e >> 3)
                    pb[2 * nb + (e >> 3)][(e & 7) >> 1] = pack2<BF16>(pv[0], pv[1]);
                }

            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int kk = 0; kk < T::KK; ++kk) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(
                        &lds_vt[(32 * db + lq) * T::VT_STRIDE + kk * 16 + g * 8]);
                    oacc[db] = mfma32x32x16<BF16>(a, pb[kk], oacc[db]);
                }
        }
        __syncthreads();                       // every wave is done with tile jt
        if (jt < tile_hi) store_tile();
    }

    // ---- epilogue: normalise once, write O and LSE -----------------------
    const float l_tot = l_run + xor32(l_run);
    if (my_row < sq) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* orow = (uint16_t*)p.o + (q_tok0 + my_row) * p.q_tok_stride + (long long)hq * D;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                u32x2 w;
                w.x = pack2<BF16>(oacc[db][4 * jj + 0] * inv, oacc[db][4 * jj + 1] * inv);
                w.y = pack2<BF16>(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
                st_global8(orow + 32 * db + 8 * jj + 4 * g, w);
            }
        if (p.lse != nullptr && g == 0) {
            const long long row_base = VARLEN ? q_tok0 : 0;
            const float lse = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
            p.lse[(long long)b * p.lse_b_stride + (long long)hq * p.lse_h_stride + row_base +
                  my_row] = lse;
        }
    }
}

template <int D, bool BF16, bool VARLEN>
static hipError_t launch_one(const FwdParams& p, hipStream_t s) {
    const long long nblocks = (long long)p.nqt * p.Hq * p.B;
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, VARLEN>), dim3((unsigned)nblocks), dim3(256), 0, s,
                       p);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int d, bool bf16, bool varlen, hipStream_t s) {
    if (d == 128) {
        if (bf16) return varlen ? launch_one<128, true, true>(p, s) : launch_one<128, true, false>(p, s);
        return varlen ? launch_one<128, false, true>(p, s) : launch_one<128, false, false>(p, s);
    }
    if (bf16) return varlen ? launch_one<64, true, true>(p, s) : launch_one<64, true, false>(p, s);
    return varlen ? launch_one<64, false, true>(p, s) : launch_one<64, false, false>(p, s);
}

}  // namespace fa
