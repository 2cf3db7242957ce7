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
// Work decomposition.  One work-group = 4 waves, one per SIMD, each owning
// 64 query rows of one query head as two 32-row halves A and B.  The waves
// of a work-group cover gw query heads that read the same K/V head (gw = 4,
// 2 or 1, the largest dividing G) and 256/gw rows, so they walk the same
// K/V tiles with the same masks in lockstep (little waiting at barriers).
// The key axis is walked in tiles of 32 keys.  Each K and V tile is read
// from LDS once per wave and feeds both halves, so LDS traffic per MFMA is
// half of what 32-row waves would need (with 32 rows per wave the LDS read
// rate equals the MFMA rate and both stall).
//
// Orientation.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16: the A operand is a 32-key slice of K, the B operand
// a 32-row query block held in registers for the whole kernel.  In the
// accumulator each lane holds ONE query row and 16 keys of it, so the row
// max and row sum are in-lane reductions plus one exchange with lane l^32,
// and the probabilities are already in the B-operand layout of the second
// product O^T = V^T P^T: P never leaves registers.
//
// Software pipeline.  With one wave per SIMD the overlap of matrix and
// vector work has to come from one instruction stream, so the two halves
// run half a tile apart.  The step with new tile t is four phases, each
// pairing the MFMAs of one half with the vector work of the other:
//     P1: S_A(t)   = K_t Q_A^T        ||  P_B(t-1) = exp2(S_B(t-1) c - m_B)
//     P2: O_B     += V_{t-1}^T P_B^T  ||  row max of S_A(t)
//     P3: S_B(t)   = K_t Q_B^T        ||  P_A(t)   = exp2(S_A(t) c - m_A)
//     P4: O_A     += V_t^T P_A^T      ||  row max of S_B(t)
// K_t is read from LDS once (P1) and kept in registers for P3; V_t is read
// once (P4) and kept for P2 of the next step.
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
// in a ring of STAGES tiles; copies are issued in pairs of tiles, 6 tiles
// ahead, and one barrier per pair of steps both publishes the next tiles
// and frees ring slots for the next copies.
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
    static constexpr int HR = 32;               // rows per half (one 32-row query block)
    static constexpr int WR = 2 * HR;           // rows per wave
    static constexpr int NW = kFwdWaves;        // waves per work-group
    static constexpr int BN = 32;               // keys per tile
    static constexpr int KS = D / 16;           // reduction steps over d
    static constexpr int DB = D / 32;           // O^T accumulators per half (32 columns each)
    static constexpr int KK = BN / 16;          // reduction steps over keys
    static constexpr int TILE_ELEMS = BN * D;
    static constexpr int TILE_BLOCKS = TILE_ELEMS * 2 / 1024;   // 1 KB blocks per K (or V) tile
    static constexpr int STAGES = 8;            // LDS ring depth (power of two)
    static constexpr int LPS = 2 * TILE_BLOCKS / NW;            // DMA loads per wave per set
    static_assert((2 * TILE_BLOCKS) % NW == 0, "the blocks of a set split evenly over the waves");
    static_assert((STAGES & (STAGES - 1)) == 0, "ring depth must be a power of two");
    static_assert(STAGES >= 6, "pairs of steps need two sets in flight");
};

constexpr float kRescaleThreshold = 8.0f;       // log2 units
static_assert(FwdGeo<128>::WR == kFwdWaveRows && FwdGeo<128>::NW * 64 == kFwdThreads, "block size");

typedef __attribute__((address_space(3))) short lds_short;
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds_short*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Make v count as used here, so that its computation stays before this
// point (an empty asm statement the scheduler keeps in order).
__device__ __forceinline__ void pin(float v) { asm volatile("" ::"v"(v)); }

// Keep an MFMA operand in the accumulation registers: MFMAs read A and B
// operands from there directly (and LDS / buffer loads write there
// directly, so this folds into the load).  The 256 architectural VGPRs then
// hold the fp32 accumulators (O of both halves and S) and the softmax.
__device__ __forceinline__ u32x4 in_acc_regs(u32x4 v) {
    u32x4 r;
    asm("" : "=a"(r) : "0"(v));
    return r;
}

template <int D, bool BF16, bool VARLEN>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_fwd_kernel(FwdParams p) {
    using T = FwdGeo<D>;
    constexpr int TE = T::TILE_ELEMS;
    __shared__ __attribute__((aligned(1024))) uint16_t k_ring[T::STAGES * TE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_ring[T::STAGES * TE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 31;          // query row (within a 32-row half) of this lane
    const int g = lane >> 5;           // half of the wave's lanes

    // ---- work-group -> (query tile, head group, sequence) ----------------
    // The work-group's waves cover gw query heads of one K/V head (wave w:
    // head hg*gw + w%gw) and bm = 64*4/gw rows (wave w: row block w/gw), so
    // they all need the same K/V tiles at the same steps.
    const int gw = p.gw, gpk = p.G / gw;       // head groups per K/V head
    int t, hg, b;
    {
        const int i = blockIdx.x;
        if (p.xcd_groups > 0) {
            // Keep the head groups of one K/V head (and its neighbouring
            // query tiles) on one XCD: work-group i runs on XCD i % 8.
            const int xcd = i & 7, r = i >> 3;
            const int per_row = p.xcd_groups * gpk;
            const int trev = r / per_row, rem = r - trev * per_row;
            const int jgrp = rem / gpk, gq = rem - jgrp * gpk;
            const int grp = xcd + 8 * jgrp;
            b = grp / p.Hkv;
            hg = (grp - b * p.Hkv) * gpk + gq;
            t = p.nqt - 1 - trev;
        } else {
            const int ngrp = p.Hq / gw;
            const int per_row = p.B * ngrp;
            const int trev = i / per_row, rem = i - trev * per_row;
            b = rem / ngrp;
            hg = rem - b * ngrp;
            t = p.nqt - 1 - trev;
        }
    }
    const int hq = hg * gw + wave % gw;
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
    const int q0 = t * p.bm;
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
    const int wg_last = min(q0 + p.bm, sq) - 1;
    const int kv_lo = lo_of(q0), kv_hi = hi_of(wg_last);
    const int tile_lo = kv_lo / T::BN;
    const int ntiles = kv_hi >= kv_lo ? kv_hi / T::BN - tile_lo + 1 : 0;
    const int tile_last = tile_lo + ntiles - 1;

    // Half h of this wave has rows r0[h]..; it computes tiles [pw_lo, pw_hi]
    // and needs no mask on tiles [in_lo, in_hi] (each of its rows sees every
    // key of the tile).
    int r0[2], pw_lo[2], pw_hi[2], in_lo[2], in_hi[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        r0[h] = q0 + T::WR * (wave / gw) + T::HR * h;
        const int r1 = min(r0[h] + T::HR - 1, sq - 1);
        pw_lo[h] = 1; pw_hi[h] = 0;
        if (r0[h] < sq) {
            const int wlo = lo_of(r0[h]), whi = hi_of(r1);
            if (whi >= wlo) { pw_lo[h] = wlo / T::BN; pw_hi[h] = whi / T::BN; }
        }
        const int int_lo = lo_of(r1), int_hi = hi_of(r0[h]);
        in_lo[h] = (int_lo + T::BN - 1) / T::BN;
        in_hi[h] = int_hi + 1 >= T::BN ? (int_hi + 1) / T::BN - 1 : -1;
    }
    auto interior = [&](int h, int jt) __attribute__((always_inline)) {
        return jt >= in_lo[h] && jt <= in_hi[h];
    };
    // Steps with new tile jt in [act_lo, act_hi] compute (the last one
    // finishes half B); outside it this wave only copies and synchronises.
    // Inside it a tile outside a half's range is computed fully masked
    // (P = 0), which keeps one straight-line body per step.  Steps in
    // [fast_lo, fast_hi] need no mask at all.
    const int act_lo = min(pw_lo[0], pw_lo[1]);
    const int act_hi = max(pw_hi[0], pw_hi[1]) + 1;
    const int fast_lo = max(in_lo[0], in_lo[1]);
    const int fast_hi = min(in_hi[0], in_hi[1]);

    // ---- K/V ring in LDS, filled by DMA -----------------------------------
    // Set s = (K_s, V_s); 2*TILE_BLOCKS 1 KB blocks, wave w issues blocks w,
    // w + NW, ...
    //   K block kb = ks, lane L: key L%32, d-chunk 2*ks + L/32.
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
            dma_voff[i] = (lane & 31) * tok_bytes_kv + (2 * blk + (lane >> 5)) * 16;
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
    // zeros to LDS without touching memory (keeps per-set load counts fixed).
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
    auto issue = [&](int s) __attribute__((always_inline)) {
        const i32x4 krs = tile_rsrc(kseq, s), vrs = tile_rsrc(vseq, s);
        const uint32_t kdst = lds_addr(kslot(s)), vdst = lds_addr(vslot(s));
#pragma unroll
        for (int i = 0; i < T::LPS; ++i) {
            if (dma_k[i])
                dma16_to_lds(krs, kdst + dma_loff[i], dma_voff[i], 0);
            else
                dma16_to_lds(vrs, vdst + dma_loff[i], dma_voff[i], 0);
        }
    };
    // Step w (relative to tile_lo) reads set w only, and set s + STAGES
    // refills the slots of set s, so it may be issued once every wave has
    // finished step s.  Steps run in pairs (2k, 2k+1): the even step issues
    // sets 2k+STAGES-2 and 2k+STAGES-1; the odd step ends with a barrier.
    // Before that barrier each wave waits until its copies of the sets read
    // by the next pair (2k+2, 2k+3) have landed; the STAGES-4 sets issued
    // after them may still be in flight.  The wait and the barrier form one
    // asm statement so that no LDS access is moved across them.
    auto sync_pair = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier"
                     ::"n"(T::LPS * (T::STAGES - 4)) : "memory");
    };

    // ---- the wave's 2 x 32 query rows as MFMA B operands ------------------
    u32x4 qreg[2][T::KS];
    {
        const auto qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const char*)p.q + (q_tok0 * p.q_tok_stride + (long long)hq * D) * 2),
            (short)0, sq * tok_bytes_q, 0x00020000);   // rows past the sequence read as zeros
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = r0[h] + lq;
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks) {
                u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
                    qrs, row * tok_bytes_q + (16 * ks + 8 * g) * 2, 0, 0);
                qreg[h][ks] = in_acc_regs(x ^ p.qsign);   // exact negation when scale < 0
            }
        }
    }

    f32x16 oacc[2][T::DB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[h][db][e] = 0.f;
    // running max (log2 units) and this lane's share of the fp32 / 16-bit sums
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f}, lr_run[2] = {0.f, 0.f};
    const float c = p.c;

    // this lane's visible key interval, relative to its first key offset 4*g
    int rel_lo[2], rel_hi[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int pos = r0[h] + lq + delta;
        rel_lo[h] = (wl >= 0 ? pos - wl : -0x40000000) - 4 * g;
        int hh = sk - 1;
        if (causal) hh = min(hh, pos);
        if (wr >= 0) hh = min(hh, pos + wr);
        rel_hi[h] = hh - 4 * g;
    }

    f32x16 sacc[2];                            // S^T of each half
    u32x4 pb[2][T::KK];                        // P of each half as 16-bit B operands
    u32x4 kreg[T::KS];                         // K_t operands (P1 and P3)
    u32x4 vreg[T::KK][T::DB];                  // V_t operands (P4, then P2 of the next step)

    // ---- phases ----------------------------------------------------------
    auto load_k = [&](const uint16_t* kt) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks)
            kreg[ks] = in_acc_regs(*reinterpret_cast<const u32x4*>(kt + ks * 512 + lane * 8));
    };
    auto load_v = [&](const uint16_t* vt) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
                const uint16_t* base = vt + ((2 * kk) * T::DB + db) * 256 + lane * 4;
                const u32x2 lo = ds_read_tr16(base);                    // keys 16kk + 4g + 0..3
                const u32x2 hi = ds_read_tr16(base + T::DB * 256);      // keys 16kk + 8 + 4g + 0..3
                vreg[kk][db] = in_acc_regs((u32x4){lo.x, lo.y, hi.x, hi.y});
            }
    };
    auto qk = [&](int h) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[h][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) sacc[h] = mfma32x32x16<BF16>(kreg[ks], qreg[h][ks], sacc[h]);
    };
    // lazy rescale of half h after its tile max mnew (log2 units).
    // Per-row decision (rows are independent); the branch only skips the
    // work when no row of the wave needs it.  Rows keeping their max are
    // multiplied by exactly 1.
    auto rescale = [&](int h, float mnew) __attribute__((always_inline)) {
        const bool raise = mnew > m_run[h] + kRescaleThreshold;
        if (wave_any(raise)) {
            asm volatile("");   // keep this rare block a real branch (not speculated)
            const float alpha = raise ? exp2_fast(m_run[h] - mnew) : 1.f;
            l_run[h] *= alpha;
            lr_run[h] *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[h][db][e] *= alpha;
            m_run[h] = raise ? mnew : m_run[h];
        }
    };
    // row max of half h's tile jt (masking it first when needed), then the
    // lazy rescale
    auto rowmax = [&](int h, int jt, bool masked) __attribute__((always_inline)) {
        f32x16& s = sacc[h];
        if (masked) {
            const int lo = rel_lo[h] - jt * T::BN, hi = rel_hi[h] - jt * T::BN;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int off = 8 * (e >> 2) + (e & 3);
                s[e] = (off >= lo && off <= hi) ? s[e] : -INFINITY;
            }
        }
        // tree reduction (short dependency chain)
        float m4[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            m4[q4] = fmaxf(fmaxf(s[4 * q4], s[4 * q4 + 1]), fmaxf(s[4 * q4 + 2], s[4 * q4 + 3]));
        float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        mx = max_halves(mx);
        rescale(h, fmaxf(m_run[h], mx * c));           // -inf stays -inf (c > 0)
    };
    // P = exp2(S*c - m) as 16-bit B operands; masked scores are -inf -> 0
    auto softmax_exp = [&](int h) __attribute__((always_inline)) {
        const float m_use = m_run[h] == -INFINITY ? 0.f : m_run[h];
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = exp2_fast(fmaf(sacc[h][e], c, -m_use));
        // two normalisers: O is divided by the sum of the 16-bit weights
        // actually fed to P.V (so its weights sum to one); LSE uses the sum
        // of the fp32 values (16-bit rounding would bias it by up to 2^-9).
        // Both are summed as trees: with one wave per SIMD a serial chain of
        // dependent adds would stall the wave.
        float lr2[2] = {0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t pk = pack2<BF16>(x[e], x[e + 1]);
            // element e is slot (e & 7) of reduction step e >> 3
            pb[h][e >> 3][(e & 7) >> 1] = pk;
            lr2[(e >> 1) & 1] = dot2_ones<BF16>(pk, lr2[(e >> 1) & 1]);
        }
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
            for (int e = 0; e < w; ++e) x[e] += x[e + w];
        l_run[h] += x[0];
        lr_run[h] += lr2[0] + lr2[1];
    };
    auto pv = [&](int h) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
                oacc[h][db] = mfma32x32x16<BF16>(vreg[kk][db], pb[h][kk], oacc[h][db]);
    };

    // One half-step of the unmasked body in a fixed instruction order: the
    // S MFMAs of half hs interleaved with the exponentials of half hp, then
    // half hp's P.V MFMAs interleaved with its sums and half hs's row max.
    // With one wave per SIMD the matrix and vector pipes only overlap as far
    // as the instruction stream alternates them, so sched_barrier(0) fences
    // keep this order.
    auto region = [&](int hs, int hp) __attribute__((always_inline)) {
        constexpr int EPK = 16 / T::KS;                 // exponentials per S MFMA
        const float m_use = m_run[hp] == -INFINITY ? 0.f : m_run[hp];
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[hs][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            sacc[hs] = mfma32x32x16<BF16>(kreg[ks], qreg[hs][ks], sacc[hs]);
#pragma unroll
            for (int j = 0; j < EPK; ++j) {
                const int e = ks * EPK + j;
                x[e] = exp2_fast(fmaf(sacc[hp][e], c, -m_use));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int e = 0; e < 16; e += 2) pb[hp][e >> 3][(e & 7) >> 1] = pack2<BF16>(x[e], x[e + 1]);
        __builtin_amdgcn_sched_barrier(0);
        // P.V of half hp; beside it: 8 v_dot2 (16-bit sum), 15 adds (fp32
        // sum tree), then half hs's row max once its S MFMAs have drained
        float lr2[2] = {0.f, 0.f};
        float m4[4];
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < T::KK * T::DB; ++i) {
            const int kk = i / T::DB, db = i % T::DB;
            oacc[hp][db] = mfma32x32x16<BF16>(vreg[kk][db], pb[hp][kk], oacc[hp][db]);
            // (the sums are pinned to their slot: left alone the compiler
            // sinks them to their next use, outside this interleave)
            if (i == 0) {
#pragma unroll
                for (int u = 0; u < 4; ++u) lr2[u & 1] = dot2_ones<BF16>(pb[hp][u >> 2][u & 3], lr2[u & 1]);
                pin(lr2[0]); pin(lr2[1]);
            } else if (i == 1) {
#pragma unroll
                for (int u = 4; u < 8; ++u) lr2[u & 1] = dot2_ones<BF16>(pb[hp][u >> 2][u & 3], lr2[u & 1]);
                lr_run[hp] += lr2[0] + lr2[1];
                pin(lr_run[hp]);
            } else if (i == 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] += x[e + 8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pin(x[e]);
            } else if (i == 3) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] += x[e + 4];
                x[0] += x[2]; x[1] += x[3];
                l_run[hp] += x[0] + x[1];
                pin(l_run[hp]);
            } else if (i == T::KK * T::DB - 3) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    m4[q4] = fmaxf(fmaxf(sacc[hs][4 * q4], sacc[hs][4 * q4 + 1]),
                                   fmaxf(sacc[hs][4 * q4 + 2], sacc[hs][4 * q4 + 3]));
            } else if (i == T::KK * T::DB - 2) {
                mx = max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        rescale(hs, fmaxf(m_run[hs], mx * c));
    };
    auto body_fast = [&](int jt) __attribute__((always_inline)) {
        load_k(kslot(jt));
        region(0, 1);
        load_v(vslot(jt));
        region(1, 0);
    };

    // Step with new tile jt (see the pipeline above).  On entry half B's
    // scores of tile jt-1 carry their final row max and V_{jt-1} is in vreg.
    auto body = [&](int jt, bool masked) __attribute__((always_inline)) {
        load_k(kslot(jt));
        qk(0);
        softmax_exp(1);
        pv(1);
        rowmax(0, jt, masked);
        qk(1);
        softmax_exp(0);
        load_v(vslot(jt));
        pv(0);
        rowmax(1, jt, masked);
    };
    // A step with new tile jt: copies (even steps), the body, the barrier
    // (odd steps).  Steps that need a mask (or compute nothing) run in the
    // loops before and after the unmasked run, so the unmasked loop body is
    // straight-line code.
    auto step = [&](int jt, bool even, bool fast) __attribute__((always_inline)) {
        if (even) {
            issue(jt + T::STAGES - 2);
            issue(jt + T::STAGES - 1);
        }
        if (fast)
            body_fast(jt);
        else if (jt >= act_lo && jt <= act_hi)
            body(jt, true);
        if (!even) sync_pair();
    };

    // before the first computed step half B has no previous tile: scores
    // -inf give P = 0, and zero V keeps 0 * V exact
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[1][e] = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
        for (int db = 0; db < T::DB; ++db) vreg[kk][db] = (u32x4){0u, 0u, 0u, 0u};

    if (ntiles > 0) {
        // sets 0 .. STAGES-3; the first pair of steps reads sets 0 and 1
        for (int s = tile_lo; s < tile_lo + T::STAGES - 2; ++s) issue(s);
        sync_pair();
        // steps r = 0 .. ntiles (new tile tile_lo + r; the last one only
        // finishes half B); the unmasked ones [rf_lo, rf_hi] run two per
        // iteration (static parity), starting at an even step
        const int rf_lo = max(fast_lo - tile_lo, 0), rf_hi = fast_hi - tile_lo;
        int r = 0;
        for (; r < rf_lo || (r <= rf_hi && (r & 1)); ++r) step(tile_lo + r, (r & 1) == 0, false);
        for (; r + 1 <= rf_hi; r += 2) {
            step(tile_lo + r, true, true);
            step(tile_lo + r + 1, false, true);
        }
        for (; r <= ntiles; ++r) step(tile_lo + r, (r & 1) == 0, false);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // DMA loads of unused sets still in flight

    // ---- epilogue: normalise once, write O and LSE -----------------------
    // O goes through LDS so that every store writes whole rows: in the
    // accumulator layout a store instruction would cover 16 bytes of each of
    // 32 rows.  Each wave stages its 64 x D tile in its own part of the
    // (now idle) K ring, rows of D/8 16-byte chunks with chunk c of row r at
    // c ^ (r % (D/8)) (conflict-free reads), then stores D/8 lanes per row.
    constexpr int CH = D / 8;                  // 16-byte chunks per row
    asm volatile("s_barrier" ::: "memory");    // every wave is done with the ring
    char* stage = reinterpret_cast<char*>(k_ring) + wave * (T::WR * D * 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float l_tot = sum_halves(l_run[h]);
        const float lr_tot = sum_halves(lr_run[h]);
        const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
        const int r = T::HR * h + lq;          // row within the wave's tile
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                u32x2 w;
                w.x = pack2<BF16>(oacc[h][db][4 * jj + 0] * inv, oacc[h][db][4 * jj + 1] * inv);
                w.y = pack2<BF16>(oacc[h][db][4 * jj + 2] * inv, oacc[h][db][4 * jj + 3] * inv);
                const int chunk = (4 * db + jj) ^ (r % CH);   // columns 32db + 8jj .. +7
                *reinterpret_cast<u32x2*>(stage + r * (2 * D) + chunk * 16 + 8 * g) = w;
            }
        const int row = r0[h] + lq;
        if (p.lse != nullptr && g == 0 && row < sq) {
            const long long row_base = VARLEN ? q_tok0 : 0;
            const float lse = l_tot > 0.f ? (m_run[h] + log2_fast(l_tot)) * kLn2 : -INFINITY;
            p.lse[(long long)b * p.lse_b_stride + (long long)hq * p.lse_h_stride + row_base + row] =
                lse;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's own staging writes
    const auto ors = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((char*)p.o + (q_tok0 * p.q_tok_stride + (long long)hq * D) * 2), (short)0,
        sq * tok_bytes_q, 0x00020000);          // rows past the sequence are dropped
    constexpr int RPI = 64 / CH;               // rows per store instruction
#pragma unroll
    for (int i = 0; i < T::WR / RPI; ++i) {
        const int r = RPI * i + lane / CH, c = lane % CH;
        const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * (2 * D) + ((c ^ (r % CH)) * 16));
        __builtin_amdgcn_raw_buffer_store_b128(x, ors, (r0[0] + r) * tok_bytes_q + c * 16, 0, 0);
    }
}

template <int D, bool BF16, bool VARLEN>
static hipError_t launch_one(const FwdParams& p, hipStream_t s) {
    const long long nblocks = (long long)p.nqt * (p.Hq / p.gw) * p.B;
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
