// fa_fwd_wide.hip -- the wide fused exact-attention forward for gfx950:
// 64 query rows per wave, one wave per SIMD.  Used where query rows see
// many keys (more than kFwdWideMinKeys on average), where reading each K/V
// operand once for 64 rows (half the LDS bytes per MFMA of 32-row waves)
// pays for having one instruction stream per SIMD, with or without score
// modifiers (fa_fwd_mod).  Rows that see fewer keys go to fa_fwd.hip's
// paired kernel.
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
// vector work has to come from one instruction stream.  The step with new
// tile t is two regions, one per half h (A, then B), each with 16 MFMA
// slots: the 8 MFMAs of S_h(t) = K_t Q_h^T, then the 8 of O_h += V_{t-1}
// P_h(t-1) (P from the region before); beside them, one exponential per
// slot, the weights P of the other half's newest tile (S from the region
// before) are computed, packed and summed.  No slot waits for a result of
// its own region.  K_t and V_{t-1} serve both regions; K_{t+1} and V_t are
// read from LDS during step t (one read per slot) into the other half of
// double-buffered operand registers.
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
// in a ring of STAGES tiles; each step copies one tile 6 tiles ahead (its
// copies spread over the MFMA slots), and one barrier per pair of steps
// both publishes the next tiles and frees ring slots for the next copies.
//
// Online softmax in base 2: scores are scaled by c = |scale|*log2(e) inside
// one FMA feeding v_exp_f32.  A row's running max is raised only when its
// tile max exceeds it by more than 8 (log2 units); until then the stale max
// is kept, which is exact because the same max is used for the numerator,
// the sum and the final LSE, and it skips most rescales of O.  A tile is
// exponentiated with the stale max first; only when a lane's sum of weights
// exceeds 2^8 (or a row has no max yet) is the true tile max taken and the
// tile redone, so unmasked steps compute no row max at all.  O is normalised
// by the sum of the 16-bit probabilities fed to P.V, LSE by the fp32 sum.
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
    static_assert(STAGES >= 7, "pairs of steps need two sets in flight");
};

constexpr float kRescaleThreshold = 8.0f;       // log2 units
static_assert(FwdGeo<128>::WR == kFwdWideWaveRows && FwdGeo<128>::NW * 64 == kFwdThreads, "block size");

template <int V>
struct int_c {
    static constexpr int value = V;
};

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
__device__ __forceinline__ void pin_u(uint32_t v) { asm volatile("" ::"v"(v)); }

// Keep an MFMA operand in the accumulation registers: MFMAs read A and B
// operands from there directly (and LDS / buffer loads write there
// directly, so this folds into the load).  The 256 architectural VGPRs then
// hold the fp32 accumulators (O of both halves and S) and the softmax.
__device__ __forceinline__ u32x4 in_acc_regs(u32x4 v) {
    u32x4 r;
    asm("" : "=a"(r) : "0"(v));
    return r;
}

// MOD selects the score modifiers (bit 0: ALiBi, bit 1: soft-capping): the
// explainer page's "Variants you may meet" (a bias term added to the scores;
// capped scores need explicit kernel support).  With them the exponent of
// score s of key j in row i (log2 units, before the running max) is
//     u = cap log2(e) tanh(scale s / cap) - slope log2(e) |pos_i - j|
// (each part only when enabled); tanh(y) = 1 - 2 / (exp2(2 y log2 e) + 1).
// MOD = 0 compiles to the unmodified kernel.  Masked steps take a generic
// order and only unmasked ones the interleaved pipeline.
template <int D, bool BF16, bool VARLEN, int MOD>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_fwd_wide_kernel(FwdParams p) {
    using T = FwdGeo<D>;
    constexpr int TE = T::TILE_ELEMS;
    __shared__ __attribute__((aligned(1024))) uint16_t k_ring[T::STAGES * TE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_ring[T::STAGES * TE];
    debug_poison_lds(k_ring, (int)sizeof(k_ring));
    debug_poison_lds(v_ring, (int)sizeof(v_ring));

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
            // query tiles) on one XCD: work-group i runs on XCD i % 8.  A
            // padded batch interleaves the XCD's (sequence, K/V head) groups
            // tile by tile; packed sequences take one group after another,
            // so the work-groups in flight on an XCD share one group's K/V
            // in its L2 (16 packed sequences of 2 K-8 K tokens: 4.1 ms
            // interleaved, 3.3 ms group after group).
            const int xcd = i & 7, r = i >> 3;
            int trev, jgrp, gq;
            if constexpr (VARLEN) {
                const int per_grp = p.nqt * gpk;
                jgrp = r / per_grp;
                const int rem = r - jgrp * per_grp;
                trev = rem / gpk;
                gq = rem - trev * gpk;
            } else {
                const int per_row = p.xcd_groups * gpk;
                trev = r / per_row;
                const int rem = r - trev * per_row;
                jgrp = rem / gpk;
                gq = rem - jgrp * gpk;
            }
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
    constexpr bool ALIBI = (MOD & 1) != 0, SOFTCAP = (MOD & 2) != 0;

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
    // copy i (of LPS) of this wave for set s
    struct SetCopy {
        i32x4 krs, vrs;
        uint32_t kdst, vdst;
    };
    auto set_copy = [&](int s) __attribute__((always_inline)) {
        return SetCopy{tile_rsrc(kseq, s), tile_rsrc(vseq, s), lds_addr(kslot(s)), lds_addr(vslot(s))};
    };
    auto copy_one = [&](const SetCopy& sc, int i) __attribute__((always_inline)) {
        if (dma_k[i])
            dma16_to_lds(sc.krs, sc.kdst + dma_loff[i], dma_voff[i], 0);
        else
            dma16_to_lds(sc.vrs, sc.vdst + dma_loff[i], dma_voff[i], 0);
    };
    auto issue = [&](int s) __attribute__((always_inline)) {
        const SetCopy sc = set_copy(s);
#pragma unroll
        for (int i = 0; i < T::LPS; ++i) copy_one(sc, i);
    };
    // Step w (relative to tile_lo) reads K of set w+1 and V of set w (and
    // K of set w itself when it needs masks), and set s + STAGES refills the
    // slots of set s, so it may be issued once every wave has finished step
    // s.  Step w issues set w+STAGES-2; steps run in pairs (2k, 2k+1) and the
    // odd step ends with a barrier.  Before that barrier each wave waits
    // until its copies of the sets read by the next pair (2k+2 .. 2k+4) have
    // landed; the STAGES-5 sets issued after them may still be in flight.  The wait and the barrier form one asm
    // statement so that no LDS access is moved across them.
    auto sync_pair = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier"
                     ::"n"(FA_VMCNT(T::LPS * (T::STAGES - 5))) : "memory");
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
    // ALiBi: slope in log2 units; element e of tile jt of half h lies at
    // signed distance 4g - lq - (r0[h] + delta) + 32 jt + 8 (e / 4) + e % 4
    // from its row
    const float slope2 = ALIBI ? p.alibi[hq] * kLog2e : 0.f;
    const float sc_k = p.sc_k, sc_c = p.sc_c;

    f32x16 sacc[2];                            // S^T of each half
    int js[2] = {0, 0};                        // key tile of each half's S (for ALiBi)
    u32x4 pb[2][T::KK];                        // P of each half as 16-bit B operands
    u32x4 kbuf[2][T::KS];                      // K operands, by step parity
    u32x4 vbuf[2][T::KK][T::DB];               // V operands, by step parity

    // ---- operand loads from the LDS ring ----------------------------------
    auto k_load = [&](const uint16_t* kt, int ks) __attribute__((always_inline)) {
        return *reinterpret_cast<const u32x4*>(kt + ks * 512 + lane * 8);
    };
    // half hh (keys 16kk + 8hh + 4g + 0..3) of V^T operand (kk, db)
    auto v_half = [&](const uint16_t* vt, int q, int hh) __attribute__((always_inline)) {
        const int kk = q / T::DB, db = q % T::DB;
        return ds_read_tr16(vt + ((2 * kk + hh) * T::DB + db) * 256 + lane * 4);
    };
    auto load_k_now = [&](auto pc, const uint16_t* kt) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) kbuf[decltype(pc)::value][ks] = in_acc_regs(k_load(kt, ks));
    };
    auto load_v_now = [&](const uint16_t* vt) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < T::KK * T::DB; ++q) {
            const u32x2 lo = v_half(vt, q, 0), hi = v_half(vt, q, 1);
            vbuf[1][q / T::DB][q % T::DB] = in_acc_regs((u32x4){lo.x, lo.y, hi.x, hi.y});
        }
    };

    // ---- softmax of one tile ------------------------------------------------
    // The running max m is lazy: a row's weights are exp2(S c - m) with the
    // stale m as long as none exceeds 2^8 (threshold 8 in log2 units).  A
    // tile is first exponentiated with the stale max; when some lane's sum of
    // weights exceeds 2^8 (only then can one weight exceed 2^8) or a row has
    // no max yet, the rare path takes the true row max, raises m (rescaling
    // O and l) where it exceeds m by more than the threshold, and
    // exponentiates the tile again.  The result equals raising m whenever a
    // tile max exceeds it by more than the threshold.
    // Two normalisers: O is divided by the sum of the 16-bit weights
    // actually fed to P.V (so its weights sum to one: a row dominated by one
    // key reproduces that key's V row), LSE by the sum of the fp32 values
    // (16-bit rounding would bias it by up to 2^-9).  Both are summed as
    // trees: with one wave per SIMD a chain of dependent adds stalls.
    // exp2 argument of element e of half h with running max m; tb is the
    // distance of the half's tile's element 0 (ALiBi only)
    auto earg = [&](int h, int e, float tb, float m) __attribute__((always_inline)) {
        const float s = sacc[h][e];
        if constexpr (MOD == 0) {
            return fmaf(s, c, -m);
        } else {
            float v;
            if constexpr (SOFTCAP) {
                const float ex = exp2_fast(s * sc_k);
                const float th = fmaf(-2.f, __builtin_amdgcn_rcpf(ex + 1.f), 1.f);
                v = s == -INFINITY ? -INFINITY : fmaf(th, sc_c, -m);   // masked stays masked
            } else {
                v = fmaf(s, c, -m);
            }
            if constexpr (ALIBI)
                v = fmaf(-slope2, fabsf(tb + (float)(8 * (e >> 2) + (e & 3))), v);
            return v;
        }
    };
    auto tile_base = [&](int h) __attribute__((always_inline)) {
        return ALIBI ? (float)(4 * g - lq + (js[h] * T::BN - r0[h] - delta)) : 0.f;
    };
    auto exps_plain = [&](int h) __attribute__((always_inline)) {
        const float m_use = m_run[h] == -INFINITY ? 0.f : m_run[h];
        const float tb = tile_base(h);
        float x[16], r2[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = exp2_fast(earg(h, e, tb, m_use));
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t pk = pack2<BF16>(x[e], x[e + 1]);
            pb[h][e >> 3][(e & 7) >> 1] = pk;
            r2[(e >> 1) & 1] = e < 4 ? sum2_16_first<BF16>(pk) : sum2_16<BF16>(pk, r2[(e >> 1) & 1]);
        }
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
            for (int e = 0; e < w; ++e) x[e] += x[e + w];
        return f32x2{x[0], r2[0] + r2[1]};
    };
    auto refresh = [&](int h) __attribute__((always_inline)) {
        asm volatile("");   // keep this rare block a real branch (not speculated)
        f32x16 s;
        if constexpr (MOD == 0) {
            s = sacc[h];
        } else {
            const float tb = tile_base(h);
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = earg(h, e, tb, 0.f);   // u, log2 units
        }
        float m4[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            m4[q4] = fmaxf(fmaxf(s[4 * q4], s[4 * q4 + 1]), fmaxf(s[4 * q4 + 2], s[4 * q4 + 3]));
        const float mx = max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
        const float mnew = fmaxf(m_run[h], MOD == 0 ? mx * c : mx);   // -inf stays -inf (c > 0)
        const bool raise = mnew > m_run[h] + kRescaleThreshold;
        const float alpha = raise ? exp2_fast(m_run[h] - mnew) : 1.f;
        l_run[h] *= alpha;
        lr_run[h] *= alpha;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[h][db][e] *= alpha;
        m_run[h] = raise ? mnew : m_run[h];
        return exps_plain(h);
    };
    // sums: (fp32, 16-bit) of this lane's weights of the tile
    auto settle = [&](int h, f32x2 sums, bool first) __attribute__((always_inline)) {
        if ((__builtin_amdgcn_ballot_w64(first) | __builtin_amdgcn_ballot_w64(sums.x > 256.f)) != 0ull)
            sums = refresh(h);
        l_run[h] += sums.x;
        lr_run[h] += sums.y;
    };
    auto softmax_tile = [&](int h) __attribute__((always_inline)) {
        const bool first = m_run[h] == -INFINITY;
        settle(h, exps_plain(h), first);
    };
    // invisible scores of half h's tile jt -> -inf
    auto apply_mask = [&](int h, int jt) __attribute__((always_inline)) {
        mask_acc32(sacc[h], rel_lo[h] - jt * T::BN, rel_hi[h] - jt * T::BN);
    };
    auto qk = [&](int h, const u32x4 (&kq)[T::KS]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[h][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) sacc[h] = mfma32x32x16<BF16>(kq[ks], qreg[h][ks], sacc[h]);
    };
    auto pv = [&](int h, const u32x4 (&vq)[T::KK][T::DB]) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
                oacc[h][db] = mfma32x32x16<BF16>(vq[kk][db], pb[h][kk], oacc[h][db]);
    };

    // One region of an unmasked step in a fixed instruction order.  Its
    // slots are the S MFMAs of half hs (new tile), then the P.V MFMAs of
    // half hs (previous tile, P from the region before); beside them the
    // exponentials of the other half hp (its S from the region before) are
    // spread evenly, with their packing and sums, and load(i) issues the
    // operand loads of slot i.  Nothing in a region waits for a result of
    // the same region.  sched_barrier(0) fences keep the order: with one
    // wave per SIMD the matrix and vector pipes only overlap as far as the
    // instruction stream alternates them.
    auto fast_region = [&](auto hsc, int jt, const u32x4 (&kq)[T::KS],
                           const u32x4 (&vq)[T::KK][T::DB], auto&& load) __attribute__((always_inline)) {
        constexpr int hs = decltype(hsc)::value, hp = 1 - hs;
        constexpr int NS = T::KS + T::KK * T::DB;       // MFMA slots
        constexpr int EPS = 16 / NS;                    // exponentials per slot
        static_assert(EPS * NS == 16, "whole exponentials per slot");
        const bool first = m_run[hp] == -INFINITY;
        const float m_use = first ? 0.f : m_run[hp];
        const float tb = tile_base(hp);
        js[hs] = jt;
        float x[16], a[8], bsum[4], r2[2];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i < T::KS) {
                sacc[hs] = mfma32x32x16<BF16>(kq[i], qreg[hs][i], i == 0 ? f32x16{} : sacc[hs]);
            } else {
                const int kk = (i - T::KS) / T::DB, db = (i - T::KS) % T::DB;
                oacc[hs][db] = mfma32x32x16<BF16>(vq[kk][db], pb[hs][kk], oacc[hs][db]);
            }
            load(i);
#pragma unroll
            for (int j = 0; j < EPS; ++j) {
                const int e = i * EPS + j;
                x[e] = exp2_fast(earg(hp, e, tb, m_use));
            }
            // pair j (elements 2j, 2j+1) is packed and summed in the slot
            // after its second exponential; pairs of sums one slot later
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if ((2 * j + 1) / EPS + 1 == i) {
                    pb[hp][j >> 2][j & 3] = pack2<BF16>(x[2 * j], x[2 * j + 1]);
                    pin_u(pb[hp][j >> 2][j & 3]);   // (else sunk past the rare-path branch)
                    a[j] = x[2 * j] + x[2 * j + 1];
                }
                if ((2 * j + 1) / EPS + 2 == i) {
                    r2[j & 1] = j < 2 ? sum2_16_first<BF16>(pb[hp][j >> 2][j & 3])
                                      : sum2_16<BF16>(pb[hp][j >> 2][j & 3], r2[j & 1]);
                    pin(r2[j & 1]);
                    if (j & 1) bsum[j >> 1] = a[j - 1] + a[j];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // pairs not yet done
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if ((2 * j + 1) / EPS + 1 >= NS) {
                pb[hp][j >> 2][j & 3] = pack2<BF16>(x[2 * j], x[2 * j + 1]);
                pin_u(pb[hp][j >> 2][j & 3]);
                a[j] = x[2 * j] + x[2 * j + 1];
            }
            if ((2 * j + 1) / EPS + 2 >= NS) {
                r2[j & 1] = j < 2 ? sum2_16_first<BF16>(pb[hp][j >> 2][j & 3])
                                  : sum2_16<BF16>(pb[hp][j >> 2][j & 3], r2[j & 1]);
                if (j & 1) bsum[j >> 1] = a[j - 1] + a[j];
            }
        }
        settle(hp, f32x2{(bsum[0] + bsum[1]) + (bsum[2] + bsum[3]), r2[0] + r2[1]}, first);
    };

    // An unmasked step with new tile jt and static parity P.  On entry K_jt
    // is in kbuf[P] and V_{jt-1} in vbuf[1-P]; the step loads K_{jt+1} and
    // V_jt into the other two buffers (the loads are issued one per slot and
    // claimed at the end of the step, so no slot waits for LDS).
    auto fast_step = [&](auto pc, int jt, bool even) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value;
        // this step's set copies go out one every few slots: issued all at
        // once by the four waves of a CU they queue at its address unit
        const SetCopy sc = set_copy(jt + T::STAGES - 2);
        constexpr int CSTEP = (T::KS + T::KK * T::DB) / T::LPS;
        const uint16_t* kt = kslot(jt + 1);
        const uint16_t* vt = vslot(jt);
        constexpr int NQ = T::KK * T::DB;
        u32x4 kn[T::KS];
        u32x2 vlo[NQ], vhi[NQ];
        fast_region(int_c<0>{}, jt, kbuf[P], vbuf[1 - P], [&](int i) __attribute__((always_inline)) {
            if (i < T::KS) kn[i] = k_load(kt, i);
            else vlo[i - T::KS] = v_half(vt, i - T::KS, 0);
            if (i % CSTEP == CSTEP / 2) copy_one(sc, i / CSTEP);
        });
        fast_region(int_c<1>{}, jt, kbuf[P], vbuf[1 - P], [&](int i) __attribute__((always_inline)) {
            if (i < NQ) vhi[i] = v_half(vt, i, 1);
        });
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) kbuf[1 - P][ks] = in_acc_regs(kn[ks]);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            vbuf[P][q / T::DB][q % T::DB] =
                in_acc_regs((u32x4){vlo[q].x, vlo[q].y, vhi[q].x, vhi[q].y});
        if (!even) sync_pair();
    };

    // A step with new tile jt that needs masks (or computes nothing): same
    // pipeline, generic instruction order, operands loaded when needed (K_jt
    // into kbuf[0] first, V_jt into vbuf[1] once V_{jt-1} is done).
    auto step_masked = [&](int jt, bool even) __attribute__((always_inline)) {
        issue(jt + T::STAGES - 2);
        if (jt >= act_lo && jt <= act_hi) {
            load_k_now(int_c<0>{}, kslot(jt));
            qk(0, kbuf[0]);
            softmax_tile(1);
            js[0] = jt;
            pv(0, vbuf[1]);
            apply_mask(0, jt);
            qk(1, kbuf[0]);
            softmax_tile(0);
            js[1] = jt;
            pv(1, vbuf[1]);
            apply_mask(1, jt);
            load_v_now(vslot(jt));
        }
        if (!even) sync_pair();
    };

    // ALiBi: the bias grows toward each row's own position, so in key order
    // a row's running max would climb tile after tile (and take the rare
    // path on most steps).  Instead the max starts at the row's largest
    // modified score in the tile holding the half's last diagonal key,
    // loaded straight from memory here: a value the row attains, so the
    // running max never exceeds the true one and later tiles are scaled
    // against it from the start.  (A zero slope keeps the plain order of
    // maxima, hence the plain result bit for bit.)
    if constexpr (ALIBI) {
        if (ntiles > 0 && slope2 != 0.f) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (pw_lo[h] > pw_hi[h]) continue;              // uniform per wave
                const int dt = min(max((r0[h] + T::HR - 1 + delta) / T::BN, pw_lo[h]), pw_hi[h]);
                const auto krs = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(kseq + (long long)dt * (T::BN * tok_bytes_kv)), (short)0,
                    min(sk - dt * T::BN, T::BN) * tok_bytes_kv, 0x00020000);
                u32x4 kq[T::KS];
#pragma unroll
                for (int ks = 0; ks < T::KS; ++ks)
                    kq[ks] = __builtin_amdgcn_raw_buffer_load_b128(
                        krs, (lane & 31) * tok_bytes_kv + (2 * ks + g) * 16, 0, 0);
                qk(h, kq);
                apply_mask(h, dt);
                js[h] = dt;
                const float tb = tile_base(h);
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, earg(h, e, tb, 0.f));
                m_run[h] = max_halves(mx);
            }
        }
    }

    // Pipeline: step jt computes S_A(jt), S_B(jt) = K_jt Q^T; P_B(jt-1) and
    // P_A(jt); O_A and O_B += V_{jt-1} P(jt-1).  Before the first computed
    // step there is no previous tile: S_B = -inf gives P_B = 0, and P_A = 0
    // with V = 0 keeps 0 * V exact.  The step after the last tile only
    // finishes the previous one.
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[1][e] = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) pb[h][kk] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
        for (int db = 0; db < T::DB; ++db) vbuf[1][kk][db] = (u32x4){0u, 0u, 0u, 0u};

    if (ntiles > 0) {
        // sets 0 .. STAGES-3; the first pair of steps reads sets 0 .. 2
        for (int s = tile_lo; s < tile_lo + T::STAGES - 2; ++s) issue(s);
        sync_pair();
        // steps r = 0 .. ntiles (new tile tile_lo + r); the unmasked ones
        // [rf_lo, rf_hi] run two per iteration (static parity), starting at
        // an even step
        const int rf_lo = max(fast_lo - tile_lo, 0), rf_hi = fast_hi - tile_lo;
        int r = 0;
        for (; r < rf_lo || (r <= rf_hi && (r & 1)); ++r) step_masked(tile_lo + r, (r & 1) == 0);
        if (r + 1 <= rf_hi) {
            load_k_now(int_c<0>{}, kslot(tile_lo + r));
            for (; r + 1 <= rf_hi; r += 2) {
                fast_step(int_c<0>{}, tile_lo + r, true);
                fast_step(int_c<1>{}, tile_lo + r + 1, false);
            }
        }
        for (; r <= ntiles; ++r) step_masked(tile_lo + r, (r & 1) == 0);
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

template <int D, bool BF16, bool VARLEN, int MOD>
static hipError_t launch_one(const FwdParams& p, hipStream_t s) {
    const long long nblocks = (long long)p.nqt * (p.Hq / p.gw) * p.B;
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((fa_fwd_wide_kernel<D, BF16, VARLEN, MOD>), dim3((unsigned)nblocks),
                       dim3(kFwdThreads), 0, s, p);
    return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_wide_t(const FwdParams& p, bool varlen, hipStream_t s) {
    if (varlen) return launch_one<D, BF16, true, 0>(p, s);
    switch (p.mod) {
        case 0: return launch_one<D, BF16, false, 0>(p, s);
        case 1: return launch_one<D, BF16, false, 1>(p, s);
        case 2: return launch_one<D, BF16, false, 2>(p, s);
        default: return launch_one<D, BF16, false, 3>(p, s);
    }
}

hipError_t launch_fwd_wide(const FwdParams& p, int d, bool bf16, bool varlen, hipStream_t s) {
    if (d == 128) return bf16 ? launch_wide_t<128, true>(p, varlen, s) : launch_wide_t<128, false>(p, varlen, s);
    return bf16 ? launch_wide_t<64, true>(p, varlen, s) : launch_wide_t<64, false>(p, varlen, s);
}

}  // namespace fa
