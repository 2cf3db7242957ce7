// fa_fwd.hip -- fused exact-attention forward for gfx950 (padded and packed).
//
// The method: the "FlashAttention" explainer page, steps 1-4 (tile the
// sequence axis, score a tile on chip, online softmax with running max and
// running sum, accumulate P.V and normalise once), step 5 (the per-row LSE),
// step 6 (tiles outside the causal / window band are skipped; only boundary
// tiles are masked element by element), step 7 (work-groups over query tiles
// x heads x batch) and step 8 (16-bit MFMA operands, fp32 accumulators and
// fp32 softmax statistics).
//
// Work decomposition.  One work-group = 256 query rows of one (sequence,
// query head), 8 waves of 32 rows (two waves per SIMD, so one wave's MFMAs
// overlap the other's softmax).  The key axis is walked in tiles of 32 keys.
//
// Orientation.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16: the A operand is a 32-key slice of K read from LDS,
// the B operand is a 32-row query block held in registers for the whole
// kernel.  In the accumulator each lane holds ONE query row and 16 keys of
// it, so the row max and row sum are in-lane reductions plus one exchange
// with lane l^32, and the probabilities are already in the B-operand layout
// of the second product O^T = V^T P^T: P never leaves registers.
//
// Data movement.  K and V tiles go from HBM/L2 straight into LDS with
// bounds-checked buffer loads (buffer_load_dwordx4 ... lds): rows past the
// end of a sequence read as zeros, no staging registers, no branches.  Each
// lane of such a load picks its own 16-byte source chunk, so the tiles are
// laid out in LDS in MFMA-operand order rather than row-major:
//   * K: unit (ks, half, key) holds d-chunk 2*ks+half of that key, so the
//     A operand of reduction step ks is one contiguous 1 KB wave read
//     (ds_read_b128 at lane*16);
//   * V: 8-byte slot (kk, h, db, lane) holds the four columns that lane
//     contributes to the gfx950 transpose read ds_read_b64_tr_b16 (16 lanes
//     read a 4-key x 16-column block and each lane receives one column), so
//     each V^T operand half is one contiguous 512-byte wave read.
// Contiguous wave reads are bank-conflict free.  K and V are buffered in LDS
// in a ring of STAGES tiles each, so loads are issued STAGES-1 tiles ahead of
// use; one barrier per tile.
//
// Pipelining.  While the softmax of tile j runs on the VALU, the MFMAs of
// S(j+1) = K_{j+1} Q^T are already issued; the row max of tile j+1 is taken
// while the P.V MFMAs of tile j run.
//
// Online softmax in base 2: scores are scaled by c = |scale|*log2(e) inside
// one FMA feeding v_exp_f32.  A row's running max is raised only when its
// tile max exceeds it by more than 8 (log2 units); until then the stale max
// is kept, which is exact because the same max is used for the numerator,
// the sum and the final LSE, and it skips most rescales of O.  O is normalised
// by the sum of the 16-bit probabilities fed to P.V (v_dot2 against (1, 1)),
// LSE by the fp32 sum.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <int D>
struct FwdGeo {
    static constexpr int QB = 1;                // 32-row query blocks per wave
    static constexpr int WR = 32 * QB;          // rows per wave
    static constexpr int BM = kFwdBM;           // rows per work-group
    static constexpr int NW = BM / WR;          // waves per work-group
    static constexpr int BN = 32;               // keys per tile
    static constexpr int KS = D / 16;           // reduction steps over d (= 1 KB K blocks per tile)
    static constexpr int DB = D / 32;           // O^T accumulators per query block
    static constexpr int NB = BN / 32;          // S^T accumulators per query block
    static constexpr int KK = BN / 16;          // reduction steps over keys
    static constexpr int VBLK = BN * D * 2 / 1024;   // 1 KB V blocks per tile (= KS)
    static constexpr int STAGES = 6;            // LDS ring depth (tiles of K and of V)
    static constexpr int LPS = 2 * KS / NW;     // DMA loads per wave per tile step
    static_assert(BN == 32, "LDS operand layouts assume 32-key tiles");
    static_assert(VBLK == KS, "K and V tiles have the same number of 1 KB blocks");
    static_assert(NW * 64 <= 1024, "work-group size");
    static_assert(LPS * NW == 2 * KS, "every wave issues the same number of loads per step");
};

constexpr float kRescaleThreshold = 8.0f;       // log2 units
constexpr int kFwdThreads = 512;                // 8 waves
static_assert(FwdGeo<128>::NW * 64 == kFwdThreads && FwdGeo<64>::NW * 64 == kFwdThreads, "block size");

typedef __attribute__((address_space(3))) short lds_short;
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds_short*)(p));
    return __builtin_bit_cast(u32x2, r);
}

template <bool BF16>
__device__ __forceinline__ float dot2_ones(uint32_t packed, float acc) {
    if constexpr (BF16) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                               __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed),
                                      __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
    }
}

template <int D, bool BF16, bool VARLEN>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(FwdParams p) {
    using T = FwdGeo<D>;
    constexpr int TILE_ELEMS = T::BN * D;
    __shared__ __attribute__((aligned(1024))) uint16_t k_ring[T::STAGES * TILE_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t v_ring[T::STAGES * TILE_ELEMS];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 31;          // query row (within a 32-row block) of this lane
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
    auto lo_of = [&](int i) __attribute__((always_inline)) { return wl >= 0 ? max(0, i + delta - wl) : 0; };
    auto hi_of = [&](int i) __attribute__((always_inline)) {
        int h = sk - 1;
        if (causal) h = min(h, i + delta);
        if (wr >= 0) h = min(h, i + delta + wr);
        return h;
    };

    const int wg_last = min(q0 + T::BM, sq) - 1;
    const int kv_lo = lo_of(q0), kv_hi = hi_of(wg_last);
    const int tile_lo = kv_lo / T::BN;
    const int ntiles = kv_hi >= kv_lo ? kv_hi / T::BN - tile_lo + 1 : 0;
    const int tile_last = tile_lo + ntiles - 1;

    // this wave's rows and key bounds
    const int r0 = q0 + T::WR * wave;
    const bool wave_active = r0 < sq;
    const int r1 = min(r0 + T::WR - 1, sq - 1);
    const int w_lo = lo_of(r0), w_hi = wave_active ? hi_of(r1) : -1;
    const int int_lo = lo_of(r1), int_hi = hi_of(r0);   // keys every row of the wave sees
    auto part = [&](int jt) __attribute__((always_inline)) {                  // wave has a visible key in tile jt
        return wave_active && jt * T::BN <= w_hi && jt * T::BN + T::BN - 1 >= w_lo;
    };
    auto interior = [&](int jt) __attribute__((always_inline)) {              // every row of the wave sees every key of jt
        return jt * T::BN >= int_lo && jt * T::BN + T::BN - 1 <= int_hi;
    };

    // ---- buffer resources ------------------------------------------------
    const long long tok_bytes_kv = p.kv_tok_stride * 2;
    const long long tok_bytes_q = p.q_tok_stride * 2;
    const char* kseq = (const char*)p.k + (k_tok0 * p.kv_tok_stride + (long long)hkv * D) * 2;
    const char* vseq = (const char*)p.v + (k_tok0 * p.kv_tok_stride + (long long)hkv * D) * 2;
    // tiles outside [tile_lo, tile_last] get zero records: their loads write
    // zeros to LDS without touching memory (keeps per-step load counts fixed)
    auto tile_rsrc = [&](const char* base, int jt) __attribute__((always_inline)) {
        const bool valid = jt >= tile_lo && jt <= tile_last;
        const int rows_left = valid ? max(sk - jt * T::BN, 0) : 0;
        return make_rsrc(base + (long long)jt * T::BN * tok_bytes_kv,
                         (int)(rows_left * tok_bytes_kv));
    };
    // 1 KB LDS blocks of a tile and their per-lane sources.  K block ks, lane
    // L: key L%32, d-chunk 2*ks + L/32.  V block b, 16-byte unit u = 64*b + L:
    // blk = u/32 = (2*kk + h)*DB + db, r = u%32 -> key 16*kk + 8*h + 4*(r/16)
    // + (r/2)%4, d-chunk 4*db + 2*((r/8)%2) + r%2.  The 2*KS blocks of a step
    // (K blocks, then V blocks) are spread over the waves: wave w issues
    // blocks w, w + NW, ...
    int dma_src[T::LPS], dma_soff[T::LPS], dma_dst[T::LPS];
    bool dma_is_k[T::LPS];
#pragma unroll
    for (int i = 0; i < T::LPS; ++i) {
        const int gb = wave + i * T::NW;
        dma_is_k[i] = gb < T::KS;
        if (dma_is_k[i]) {
            dma_src[i] = (lane & 31) * (int)tok_bytes_kv + (lane >> 5) * 16;
            dma_soff[i] = gb * 32;
            dma_dst[i] = gb * 1024;
        } else {
            const int vb = gb - T::KS;
            const int u = vb * 64 + lane;
            const int blk = u >> 5, r = u & 31;
            const int db = blk % T::DB, kh = blk / T::DB;
            const int row = 8 * kh + 4 * (r >> 4) + ((r >> 1) & 3);
            const int chunk = 4 * db + 2 * ((r >> 3) & 1) + (r & 1);
            dma_src[i] = row * (int)tok_bytes_kv + chunk * 16;
            dma_soff[i] = 0;
            dma_dst[i] = vb * 1024;
        }
    }

    // ---- query blocks as MFMA B operands ---------------------------------
    u32x4 qreg[T::QB][T::KS];
    {
        const auto qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const char*)p.q + (q_tok0 * p.q_tok_stride + (long long)hq * D) * 2),
            (short)0, (int)(sq * tok_bytes_q), 0x00020000);   // zero rows past the sequence
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks) {
                const int row = r0 + 32 * qb + lq;
                u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
                    qrs, (int)(row * tok_bytes_q) + (16 * ks + 8 * g) * 2, 0, 0);
                qreg[qb][ks] = x ^ p.qsign;    // exact negation when scale < 0
            }
    }

    f32x16 oacc[T::QB][T::DB];
#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[qb][db][e] = 0.f;
    // running max (log2 units) and this lane's share of the fp32 / 16-bit-rounded sums
    float m_run[T::QB], l_run[T::QB], lr_run[T::QB];
#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.f; lr_run[qb] = 0.f; }
    const float c = p.c;

    // per-lane visible interval of each query block, relative to its first key 4*g
    int rel_lo[T::QB], rel_hi[T::QB];
#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb) {
        const int pos = r0 + 32 * qb + lq + delta;
        rel_lo[qb] = (wl >= 0 ? pos - wl : -0x40000000) - 4 * g;
        int h = sk - 1;
        if (causal) h = min(h, pos);
        if (wr >= 0) h = min(h, pos + wr);
        rel_hi[qb] = h - 4 * g;
    }

    f32x16 sacc[2][T::QB][T::NB];              // [parity][query block][key block]
    u32x4 pb[T::QB][T::KK];                    // P as 16-bit B operands

    // ---- phases ----------------------------------------------------------
    auto qk = [&](f32x16 (&s)[T::QB][T::NB], const uint16_t* kt) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) s[qb][nb][e] = 0.f;
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(kt + ks * 512 + lane * 8);
#pragma unroll
                for (int qb = 0; qb < T::QB; ++qb)
                    s[qb][nb] = mfma32x32x16<BF16>(a, qreg[qb][ks], s[qb][nb]);
            }
    };
    // row max of a tile (masking it first when needed) and the lazy rescale
    auto rowmax = [&](f32x16 (&s)[T::QB][T::NB], int jt, bool masked) __attribute__((always_inline)) {
        float mnew[T::QB];
        bool raise[T::QB];
        bool any_raise = false;
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb) {
            if (masked) {
                const int lo = rel_lo[qb] - jt * T::BN, hi = rel_hi[qb] - jt * T::BN;
#pragma unroll
                for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int off = 32 * nb + 8 * (e >> 2) + (e & 3);
                        s[qb][nb][e] = (off >= lo && off <= hi) ? s[qb][nb][e] : -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[qb][nb][e]);
            mx = fmaxf(mx, xor32(mx));
            mnew[qb] = fmaxf(m_run[qb], mx * c);      // -inf stays -inf (c > 0)
            raise[qb] = mnew[qb] > m_run[qb] + kRescaleThreshold;
            any_raise = any_raise || raise[qb];
        }
        // Per-row decision (rows are independent); the branch only skips the
        // work when no row of the wave needs it.  Rows keeping their max are
        // multiplied by exactly 1.
        if (wave_any(any_raise)) {
            asm volatile("");   // keep this rare block a real branch (not speculated)
#pragma unroll
            for (int qb = 0; qb < T::QB; ++qb) {
                const float alpha = raise[qb] ? exp2_fast(m_run[qb] - mnew[qb]) : 1.f;
                l_run[qb] *= alpha;
                lr_run[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < T::DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[qb][db][e] *= alpha;
                m_run[qb] = raise[qb] ? mnew[qb] : m_run[qb];
            }
        }
    };
    // P = exp2(S*c - m) as 16-bit B operands; masked scores are -inf -> 0
    auto softmax_exp = [&](f32x16 (&s)[T::QB][T::NB]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb) {
            const float m_use = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const float x0 = exp2_fast(fmaf(s[qb][nb][e], c, -m_use));
                    const float x1 = exp2_fast(fmaf(s[qb][nb][e + 1], c, -m_use));
                    const uint32_t pk = pack2<BF16>(x0, x1);
                    // element e of key block nb is slot (e & 7) of reduction step 2*nb + (e >> 3)
                    pb[qb][2 * nb + (e >> 3)][(e & 7) >> 1] = pk;
                    // two normalisers: O is divided by the sum of the 16-bit weights
                    // actually fed to P.V (so its weights sum to one); LSE uses the sum
                    // of the fp32 values (16-bit rounding would bias it by up to 2^-9)
                    l_run[qb] += x0 + x1;
                    lr_run[qb] = dot2_ones<BF16>(pk, lr_run[qb]);
                }
        }
    };
    auto pv = [&](const uint16_t* vt) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int kk = 0; kk < T::KK; ++kk) {
                const uint16_t* base = vt + ((2 * kk) * T::DB + db) * 256 + lane * 4;
                const u32x2 lo = ds_read_tr16(base);                    // keys 16kk + 4g + 0..3
                const u32x2 hi = ds_read_tr16(base + T::DB * 256);      // keys 16kk + 8 + 4g + 0..3
                const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
                for (int qb = 0; qb < T::QB; ++qb)
                    oacc[qb][db] = mfma32x32x16<BF16>(a, pb[qb][kk], oacc[qb][db]);
            }
    };

    // Ring slot of tile t (t >= tile_lo - 1).
    auto kslot = [&](int t) __attribute__((always_inline)) {
        return k_ring + ((t - tile_lo + T::STAGES) % T::STAGES) * TILE_ELEMS;
    };
    auto vslot = [&](int t) __attribute__((always_inline)) {
        return v_ring + ((t - tile_lo + T::STAGES) % T::STAGES) * TILE_ELEMS;
    };
    // Load set of step t: K_t and V_{t-1}.  Step j issues set j + STAGES,
    // which refills the slots of K_j and V_{j-1} (both consumed by step j-1).
    auto issue = [&](int t) __attribute__((always_inline)) {
        const i32x4 krs = tile_rsrc(kseq, t), vrs = tile_rsrc(vseq, t - 1);
        const uint32_t kdst = lds_addr(kslot(t)), vdst = lds_addr(vslot(t - 1));
#pragma unroll
        for (int i = 0; i < T::LPS; ++i) {
            if (dma_is_k[i])
                dma16_to_lds(krs, kdst + dma_dst[i], dma_src[i], dma_soff[i]);
            else
                dma16_to_lds(vrs, vdst + dma_dst[i], dma_src[i], dma_soff[i]);
        }
    };
    // Before step j the sets up to j+1 (K_{j+1}, V_j) must have landed in
    // every wave; the STAGES-2 sets issued after it may still be in flight.
    // The wait and the barrier form one asm statement so that no LDS access
    // is moved across them.
    auto sync_tile = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier"
                     ::"n"(T::LPS * (T::STAGES - 2)) : "memory");
    };

    // One tile step.  On entry tile j's scores (scur) carry their final row
    // max; K_{j+1} and V_j are in the ring.
    auto step = [&](f32x16 (&scur)[T::QB][T::NB], f32x16 (&snext)[T::QB][T::NB], int j)
        __attribute__((always_inline)) {
        issue(j + T::STAGES);
        const bool has_next = j + 1 <= tile_last;
        const bool pj = part(j), pn = has_next && part(j + 1);
        if (pj && pn && interior(j + 1)) {
            // steady state: one straight-line block
            qk(snext, kslot(j + 1));
            softmax_exp(scur);
            pv(vslot(j));
            rowmax(snext, j + 1, false);
        } else {
            if (pn) qk(snext, kslot(j + 1));
            if (pj) {
                softmax_exp(scur);
                pv(vslot(j));
            }
            if (pn) rowmax(snext, j + 1, !interior(j + 1));
        }
        sync_tile();
    };

    if (ntiles > 0) {
        for (int t = tile_lo; t < tile_lo + T::STAGES; ++t) issue(t);
        sync_tile();
        if (part(tile_lo)) {
            qk(sacc[0], kslot(tile_lo));
            rowmax(sacc[0], tile_lo, !interior(tile_lo));
        }
        // unrolled by two so that the score buffers swap roles statically
        for (int r = 0; r < ntiles; r += 2) {
            step(sacc[0], sacc[1], tile_lo + r);
            if (r + 1 >= ntiles) break;
            step(sacc[1], sacc[0], tile_lo + r + 1);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // DMA loads of unused sets still in flight

    // ---- epilogue: normalise once, write O and LSE -----------------------
    const auto ors = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((char*)p.o + (q_tok0 * p.q_tok_stride + (long long)hq * D) * 2), (short)0,
        (int)(sq * tok_bytes_q), 0x00020000);
#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb) {
        const float l_tot = l_run[qb] + xor32(l_run[qb]);
        const float lr_tot = lr_run[qb] + xor32(lr_run[qb]);
        const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
        const int row = r0 + 32 * qb + lq;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                u32x2 w;
                w.x = pack2<BF16>(oacc[qb][db][4 * jj + 0] * inv, oacc[qb][db][4 * jj + 1] * inv);
                w.y = pack2<BF16>(oacc[qb][db][4 * jj + 2] * inv, oacc[qb][db][4 * jj + 3] * inv);
                __builtin_amdgcn_raw_buffer_store_b64(
                    w, ors, (int)(row * tok_bytes_q) + (32 * db + 8 * jj + 4 * g) * 2, 0, 0);
            }
        if (p.lse != nullptr && g == 0 && row < sq) {
            const long long row_base = VARLEN ? q_tok0 : 0;
            const float lse = l_tot > 0.f ? (m_run[qb] + log2_fast(l_tot)) * kLn2 : -INFINITY;
            p.lse[(long long)b * p.lse_b_stride + (long long)hq * p.lse_h_stride + row_base + row] =
                lse;
        }
    }
}

template <int D, bool BF16, bool VARLEN>
static hipError_t launch_one(const FwdParams& p, hipStream_t s) {
    const long long nblocks = (long long)p.nqt * p.Hq * p.B;
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, VARLEN>), dim3((unsigned)nblocks),
                       dim3(kFwdThreads), 0, s, p);
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
