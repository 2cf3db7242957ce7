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
// in a ring of STAGES tiles each; loads are issued in pairs of tiles, 5 to 6
// tiles ahead of use, and one barrier per pair of tiles both publishes the
// next pair's data and frees the ring slots for the next copies.
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
    static constexpr int WR = 32;               // rows per wave (one 32-row query block)
    static constexpr int BM = kFwdBM;           // rows per work-group
    static constexpr int NW = BM / WR;          // waves per work-group
    static constexpr int BN = 32;               // keys per tile
    static constexpr int NB = BN / 32;          // S^T accumulators (32 keys each)
    static constexpr int KS = D / 16;           // reduction steps over d
    static constexpr int DB = D / 32;           // O^T accumulators (32 columns each)
    static constexpr int KK = BN / 16;          // reduction steps over keys
    static constexpr int TILE_ELEMS = BN * D;
    static constexpr int TILE_BLOCKS = TILE_ELEMS * 2 / 1024;   // 1 KB blocks per K (or V) tile
    static constexpr int STAGES = 8;            // LDS ring depth (power of two)
    static constexpr int LPS = 2 * TILE_BLOCKS / NW;            // DMA loads per wave per step
    static_assert((2 * TILE_BLOCKS) % NW == 0, "the blocks of a step split evenly over the waves");
    static_assert((STAGES & (STAGES - 1)) == 0, "ring depth must be a power of two");
    static_assert(STAGES >= 6, "pairs of tiles need two sets in flight");
};

constexpr float kRescaleThreshold = 8.0f;       // log2 units
static_assert(FwdGeo<128>::NW * 64 == kFwdThreads && FwdGeo<64>::NW * 64 == kFwdThreads, "block size");

typedef __attribute__((address_space(3))) short lds_short;
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds_short*)(p));
    return __builtin_bit_cast(u32x2, r);
}

template <int D, bool BF16, bool VARLEN>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(FwdParams p) {
    using T = FwdGeo<D>;
    constexpr int TE = T::TILE_ELEMS;
    __shared__ __attribute__((aligned(1024))) uint16_t k_ring[T::STAGES * TE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_ring[T::STAGES * TE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 31;          // query row (within the wave's 32 rows) of this lane
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
    auto lo_of = [&](int i) __attribute__((always_inline)) {
        return wl >= 0 ? max(0, i + delta - wl) : 0;
    };
    auto hi_of = [&](int i) __attribute__((always_inline)) {
        int h = sk - 1;
        if (causal) h = min(h, i + delta);
        if (wr >= 0) h = min(h, i + delta + wr);
        return h;
    };

    // ---- tile ranges -------------------------------------------------------
    const int wg_last = min(q0 + T::BM, sq) - 1;
    const int kv_lo = lo_of(q0), kv_hi = hi_of(wg_last);
    const int tile_lo = kv_lo / T::BN;
    const int ntiles = kv_hi >= kv_lo ? kv_hi / T::BN - tile_lo + 1 : 0;
    const int tile_last = tile_lo + ntiles - 1;

    // This wave's rows r0..r1; it computes tiles [pw_lo, pw_hi] and needs no
    // mask on tiles [in_lo, in_hi] (every row of the wave sees every key).
    const int r0 = q0 + T::WR * wave;
    const int r1 = min(r0 + T::WR - 1, sq - 1);
    int pw_lo = 1, pw_hi = 0;
    if (r0 < sq) {
        const int wlo = lo_of(r0), whi = hi_of(r1);
        if (whi >= wlo) { pw_lo = wlo / T::BN; pw_hi = whi / T::BN; }
    }
    const int int_lo = lo_of(r1), int_hi = hi_of(r0);
    const int in_lo = (int_lo + T::BN - 1) / T::BN;
    const int in_hi = int_hi + 1 >= T::BN ? (int_hi + 1) / T::BN - 1 : -1;
    auto part = [&](int jt) __attribute__((always_inline)) { return jt >= pw_lo && jt <= pw_hi; };
    auto interior = [&](int jt) __attribute__((always_inline)) {
        return jt >= in_lo && jt <= in_hi;
    };
    // steps j whose next tile is computed unmasked by this wave: the
    // straight-line fast path
    const int fast_lo = max(pw_lo, in_lo - 1);
    const int fast_hi = min(min(pw_hi - 1, in_hi - 1), tile_last - 1);

    // ---- DMA sources -------------------------------------------------------
    // A step loads TILE_BLOCKS 1 KB blocks of K, then as many of V; wave w
    // issues blocks w, w + NW, ... of that list.
    //   K block kb = nb*KS + ks, lane L: key 32*nb + L%32, d-chunk 2*ks + L/32.
    //   V block vb, 16-byte unit u = 64*vb + L: half-block hb = u/32 =
    //   kh*DB + db, r = u%32 -> key 8*kh + 4*(r/16) + (r/2)%4, d-chunk
    //   4*db + 2*((r/8)%2) + r%2.
    const int tok_bytes_kv = (int)(p.kv_tok_stride * 2);
    const int tok_bytes_q = (int)(p.q_tok_stride * 2);
    __builtin_assume(wave >= 0 && wave < T::NW);
    int dma_voff[T::LPS];
    uint32_t dma_loff[T::LPS];
    bool dma_k[T::LPS];
#pragma unroll
    for (int i = 0; i < T::LPS; ++i) {
        const int gb = wave + i * T::NW;
        dma_k[i] = gb < T::TILE_BLOCKS;
        const int blk = dma_k[i] ? gb : gb - T::TILE_BLOCKS;
        dma_loff[i] = blk * 1024;
        if (dma_k[i]) {
            dma_voff[i] = (32 * (blk / T::KS) + (lane & 31)) * tok_bytes_kv +
                          (2 * (blk % T::KS) + (lane >> 5)) * 16;
        } else {
            const int hb = 2 * blk + (lane >> 5), r = lane & 31;
            const int kh = hb / T::DB, db = hb % T::DB;
            const int row = 8 * kh + 4 * (r >> 4) + ((r >> 1) & 3);
            const int chunk = 4 * db + 2 * ((r >> 3) & 1) + (r & 1);
            dma_voff[i] = row * tok_bytes_kv + chunk * 16;
        }
    }
    const char* kseq = (const char*)p.k + (k_tok0 * p.kv_tok_stride + (long long)hkv * D) * 2;
    const char* vseq = (const char*)p.v + (k_tok0 * p.kv_tok_stride + (long long)hkv * D) * 2;
    // Tiles outside [tile_lo, tile_last] get zero records: their loads write
    // zeros to LDS without touching memory (keeps per-step load counts fixed).
    auto tile_rsrc = [&](const char* base, int jt) __attribute__((always_inline)) {
        const bool valid = jt >= tile_lo && jt <= tile_last;
        const int rows = valid ? min(sk - jt * T::BN, T::BN) : 0;
        return make_rsrc(base + (long long)jt * (T::BN * tok_bytes_kv), rows * tok_bytes_kv);
    };
    auto kslot = [&](int jt) __attribute__((always_inline)) {
        return k_ring + ((jt - tile_lo) & (T::STAGES - 1)) * TE;
    };
    auto vslot = [&](int jt) __attribute__((always_inline)) {
        return v_ring + ((jt - tile_lo) & (T::STAGES - 1)) * TE;
    };
    // Load set of step s: K_s and V_{s-1}.  Set s refills the slots of
    // K_{s-STAGES} and V_{s-1-STAGES}, both last read in step s-STAGES-1
    // (step -1 being the first tile's Q.K product before the loop).
    auto issue = [&](int s) __attribute__((always_inline)) {
        const i32x4 krs = tile_rsrc(kseq, s), vrs = tile_rsrc(vseq, s - 1);
        const uint32_t kdst = lds_addr(kslot(s)), vdst = lds_addr(vslot(s - 1));
#pragma unroll
        for (int i = 0; i < T::LPS; ++i) {
            if (dma_k[i])
                dma16_to_lds(krs, kdst + dma_loff[i], dma_voff[i], 0);
            else
                dma16_to_lds(vrs, vdst + dma_loff[i], dma_voff[i], 0);
        }
    };
    // Steps run in pairs (relative steps 2k, 2k+1).  The even step issues
    // sets 2k+STAGES-2 and 2k+STAGES-1; the odd step ends with a barrier
    // after which every wave has finished step 2k+1, so the next pair's
    // copies only refill slots last read at step 2k or earlier.  Steps
    // 2k+2, 2k+3 read sets 2k+3, 2k+4 (K_{j+1}, V_j), so before that
    // barrier each wave waits until its copies up to set 2k+4 have landed:
    // the STAGES-5 sets issued after it may still be in flight.  The wait and
    // the barrier form one asm statement so that no LDS access is moved
    // across them.
    auto sync_pair = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier"
                     ::"n"(T::LPS * (T::STAGES - 5)) : "memory");
    };

    // ---- the wave's 32 query rows as MFMA B operands ---------------------
    u32x4 qreg[T::KS];
    {
        const auto qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const char*)p.q + (q_tok0 * p.q_tok_stride + (long long)hq * D) * 2),
            (short)0, sq * tok_bytes_q, 0x00020000);   // rows past the sequence read as zeros
        const int row = r0 + lq;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
                qrs, row * tok_bytes_q + (16 * ks + 8 * g) * 2, 0, 0);
            qreg[ks] = x ^ p.qsign;            // exact negation when scale < 0
        }
    }

    f32x16 oacc[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    // running max (log2 units) and this lane's share of the fp32 / 16-bit sums
    float m_run = -INFINITY, l_run = 0.f, lr_run = 0.f;
    const float c = p.c;

    // this lane's visible key interval, relative to its first key offset 4*g
    int rel_lo, rel_hi;
    {
        const int pos = r0 + lq + delta;
        rel_lo = (wl >= 0 ? pos - wl : -0x40000000) - 4 * g;
        int h = sk - 1;
        if (causal) h = min(h, pos);
        if (wr >= 0) h = min(h, pos + wr);
        rel_hi = h - 4 * g;
    }

    f32x16 sacc[2][T::NB];                     // [parity][key block]
    u32x4 pb[T::KK];                           // P as 16-bit B operands

    // ---- phases ----------------------------------------------------------
    auto qk = [&](f32x16 (&s)[T::NB], const uint16_t* kt) __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s[nb][e] = 0.f;
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(
                    kt + (nb * T::KS + ks) * 512 + lane * 8);
                s[nb] = mfma32x32x16<BF16>(a, qreg[ks], s[nb]);
            }
        }
    };
    // row max of a tile (masking it first when needed) and the lazy rescale
    auto rowmax = [&](f32x16 (&s)[T::NB], int jt, bool masked) __attribute__((always_inline)) {
        if (masked) {
            const int lo = rel_lo - jt * T::BN, hi = rel_hi - jt * T::BN;
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int off = 32 * nb + 8 * (e >> 2) + (e & 3);
                    s[nb][e] = (off >= lo && off <= hi) ? s[nb][e] : -INFINITY;
                }
        }
        // tree reduction (short dependency chain)
        float m4[4 * T::NB];
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                m4[4 * nb + q4] = fmaxf(fmaxf(s[nb][4 * q4], s[nb][4 * q4 + 1]),
                                        fmaxf(s[nb][4 * q4 + 2], s[nb][4 * q4 + 3]));
#pragma unroll
        for (int w = 4 * T::NB; w > 1; w >>= 1)
#pragma unroll
            for (int i = 0; i < w / 2; ++i) m4[i] = fmaxf(m4[i], m4[i + w / 2]);
        float mx = m4[0];
        mx = fmaxf(mx, xor32(mx));
        const float mnew = fmaxf(m_run, mx * c);       // -inf stays -inf (c > 0)
        // Per-row decision (rows are independent); the branch only skips the
        // work when no row of the wave needs it.  Rows keeping their max are
        // multiplied by exactly 1.
        const bool raise = mnew > m_run + kRescaleThreshold;
        if (wave_any(raise)) {
            asm volatile("");   // keep this rare block a real branch (not speculated)
            const float alpha = raise ? exp2_fast(m_run - mnew) : 1.f;
            l_run *= alpha;
            lr_run *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            m_run = raise ? mnew : m_run;
        }
    };
    // P = exp2(S*c - m) as 16-bit B operands; masked scores are -inf -> 0
    auto softmax_exp = [&](f32x16 (&s)[T::NB]) __attribute__((always_inline)) {
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float x0 = exp2_fast(fmaf(s[nb][e], c, -m_use));
                const float x1 = exp2_fast(fmaf(s[nb][e + 1], c, -m_use));
                const uint32_t pk = pack2<BF16>(x0, x1);
                // element e of key block nb is slot (e & 7) of reduction step 2*nb + (e >> 3)
                pb[2 * nb + (e >> 3)][(e & 7) >> 1] = pk;
                // two normalisers: O is divided by the sum of the 16-bit weights
                // actually fed to P.V (so its weights sum to one); LSE uses the sum
                // of the fp32 values (16-bit rounding would bias it by up to 2^-9)
                l_run += x0 + x1;
                lr_run = dot2_ones<BF16>(pk, lr_run);
            }
    };
    auto pv = [&](const uint16_t* vt) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
                const uint16_t* base = vt + ((2 * kk) * T::DB + db) * 256 + lane * 4;
                const u32x2 lo = ds_read_tr16(base);                    // keys 16kk + 4g + 0..3
                const u32x2 hi = ds_read_tr16(base + T::DB * 256);      // keys 16kk + 8 + 4g + 0..3
                const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
                oacc[db] = mfma32x32x16<BF16>(a, pb[kk], oacc[db]);
            }
    };

    // One tile step.  On entry tile j's scores (scur) carry their final row
    // max; K_{j+1} and V_j are in the ring.
    auto step = [&](f32x16 (&scur)[T::NB], f32x16 (&snext)[T::NB], int j, bool even)
        __attribute__((always_inline)) {
        if (even) {
            issue(j + T::STAGES - 2);
            issue(j + T::STAGES - 1);
        }
        if (j >= fast_lo && j <= fast_hi) {
            // steady state: one straight-line block
            qk(snext, kslot(j + 1));
            softmax_exp(scur);
            pv(vslot(j));
            rowmax(snext, j + 1, false);
        } else {
            const bool pn = j + 1 <= tile_last && part(j + 1);
            if (pn) qk(snext, kslot(j + 1));
            if (part(j)) {
                softmax_exp(scur);
                pv(vslot(j));
            }
            if (pn) rowmax(snext, j + 1, !interior(j + 1));
        }
        if (!even) sync_pair();
    };

    if (ntiles > 0) {
        // sets 0 .. STAGES-3; the first pair of steps reads sets 0 .. 2
        for (int s = tile_lo; s < tile_lo + T::STAGES - 2; ++s) issue(s);
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier"
                     ::"n"(T::LPS * (T::STAGES - 5)) : "memory");
        if (part(tile_lo)) {
            qk(sacc[0], kslot(tile_lo));
            rowmax(sacc[0], tile_lo, !interior(tile_lo));
        }
        // unrolled by two so that the score buffers swap roles statically
        for (int r = 0; r < ntiles; r += 2) {
            step(sacc[0], sacc[1], tile_lo + r, true);
            if (r + 1 >= ntiles) break;
            step(sacc[1], sacc[0], tile_lo + r + 1, false);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // DMA loads of unused sets still in flight

    // ---- epilogue: normalise once, write O and LSE -----------------------
    const auto ors = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((char*)p.o + (q_tok0 * p.q_tok_stride + (long long)hq * D) * 2), (short)0,
        sq * tok_bytes_q, 0x00020000);          // rows past the sequence are dropped
    const float l_tot = l_run + xor32(l_run);
    const float lr_tot = lr_run + xor32(lr_run);
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    const int row = r0 + lq;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            u32x2 w;
            w.x = pack2<BF16>(oacc[db][4 * jj + 0] * inv, oacc[db][4 * jj + 1] * inv);
            w.y = pack2<BF16>(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
            __builtin_amdgcn_raw_buffer_store_b64(
                w, ors, row * tok_bytes_q + (32 * db + 8 * jj + 4 * g) * 2, 0, 0);
        }
    if (p.lse != nullptr && g == 0 && row < sq) {
        const long long row_base = VARLEN ? q_tok0 : 0;
        const float lse = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
        p.lse[(long long)b * p.lse_b_stride + (long long)hq * p.lse_h_stride + row_base + row] = lse;
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
