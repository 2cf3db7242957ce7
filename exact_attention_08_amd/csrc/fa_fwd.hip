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
// 32 query rows of one query head.  The waves of a work-group cover gw query
// heads that read the same K/V head (gw = 4, 2 or 1, the largest dividing
// G) and 128/gw rows, so they walk the same K/V tiles with the same masks in
// lockstep.  Three work-groups share a CU (at most 168 registers per wave,
// 48 KB of LDS each at d = 128): the waves on each SIMD belong to different
// work-groups and never synchronise with each other, so while one is in its
// softmax the others' matrix instructions keep the MFMA pipe busy, and one
// work-group's prologue and epilogue overlap the others' key loops.  (One
// wave per SIMD has to interleave matrix and vector work within a single
// instruction stream and stalls wherever that stream waits; waves of one
// work-group fall into lockstep at every barrier.)
//
// Orientation.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16: the A operand is a 32-key slice of K, the B operand
// the wave's 32 query rows held in registers for the whole kernel.  In the
// accumulator each lane holds ONE query row and 16 keys of it, so the row
// max and row sum are in-lane reductions plus one exchange with lane l^32,
// and the probabilities are already in the B-operand layout of the second
// product O^T = V^T P^T: P never leaves registers.
//
// Data movement.  K and V tiles of 32 keys go from HBM/L2 straight into LDS
// with bounds-checked buffer loads (buffer_load_dwordx4 ... lds): rows past
// the end of a sequence read as zeros, no staging registers, no branches.
// Each lane of such a load picks its own 16-byte source chunk, so a tile's
// layout in LDS is free:
//   * K at d = 128: row-major with the 16-byte chunks of key r XOR-swizzled
//     by r % 16, so that each copy reads 4 whole rows and each A-operand read
//     (lane = key, one chunk) touches every bank once; with ALiBi and at
//     d = 64, operand order: unit (ks, half, key) holds d-chunk 2*ks+half of
//     that key, so the A operand of reduction step ks is one contiguous 1 KB
//     wave read (ds_read_b128 at lane*16);
//   * V: 8-byte slot (kk, h, db, lane) holds the four columns that lane
//     contributes to the gfx950 transpose read ds_read_b64_tr_b16 (16 lanes
//     read a 4-key x 16-column block and each lane receives one column), so
//     each V^T operand half is one contiguous 512-byte wave read.
// Contiguous wave reads are bank-conflict free.  K and V are buffered in a
// ring of 3 tiles; step r copies tile r+2 (its copies shared by the four
// waves) and ends with one barrier that both publishes tile r+1 and frees
// the slot tile r+3 will use.
//
// Online softmax in base 2: scores are scaled by c = |scale|*log2(e) inside
// one FMA feeding v_exp_f32.  A row's running max is raised only when its
// tile max exceeds it by more than 8 (log2 units); until then the stale max
// is kept, which is exact because the same max is used for the numerator,
// the sum and the final LSE, and it skips most rescales of O.  A tile is
// exponentiated with the stale max first; only when a lane's sum of weights
// exceeds 2^8 (or a row has no max yet) is the true tile max taken and the
// tile redone, so most steps compute no row max at all.  O is normalised by
// the sum of the 16-bit probabilities fed to P.V, LSE by the fp32 sum.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <int D>
struct FwdGeo {
    static constexpr int R = 32;                // query rows per wave
    static constexpr int NW = kFwdWaves;        // waves per work-group
    static constexpr int BN = 32;               // keys per tile
    static constexpr int KS = D / 16;           // reduction steps over d
    static constexpr int DB = D / 32;           // O^T accumulators (32 columns each)
    static constexpr int KK = BN / 16;          // reduction steps over keys
    static constexpr int TE = BN * D;           // elements of one K (or V) tile
    static constexpr int TB = TE * 2 / 1024;    // 1 KB blocks per K (or V) tile
    static constexpr int STAGES = 3;            // LDS ring depth
    static constexpr int AHEAD = 2;             // step r copies tile r + AHEAD (into the
                                                // slot that tile r - 1 used)
    static constexpr int LPS = 2 * TB / NW;     // DMA loads per wave per step
    static_assert((2 * TB) % NW == 0, "the blocks of a tile pair split evenly over the waves");
    static_assert(AHEAD + 1 == STAGES, "a slot is refilled right after the barrier that retires it");
};
static_assert(FwdGeo<128>::R == kFwdWaveRows && FwdGeo<128>::NW * 64 == kFwdThreads, "block size");

constexpr float kRescaleThreshold = 8.0f;       // log2 units

typedef __attribute__((address_space(3))) short lds_short;
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds_short*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// MOD selects the score modifiers (padded forward only; bit 0: ALiBi, bit
// 1: soft-capping), as in the wide kernel (fa_fwd_wide.hip): the explainer
// page's "Variants you may meet" (a bias term added to the scores; capped
// scores need explicit kernel support).  The exponent of score s of key j in
// row i (log2 units, before the running max) becomes
//     u = cap log2(e) tanh(scale s / cap) - slope log2(e) |pos_i - j|
// (each part only when enabled); tanh(y) = 1 - 2 / (exp2(2 y log2 e) + 1).
// MOD = 0 compiles to the plain kernel.
template <int D, bool BF16, bool VARLEN, int MOD>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void fa_fwd_kernel(FwdParams p) {
    using T = FwdGeo<D>;
    constexpr bool ALIBI = (MOD & 1) != 0, SOFTCAP = (MOD & 2) != 0;
    static_assert(!(VARLEN && MOD != 0), "score modifiers are padded-only");
    // K tiles as whole rows (XOR-swizzled) rather than in operand order; not
    // with ALiBi, whose extra registers would then spill
    constexpr bool KROW = D == 128 && !ALIBI;
    constexpr int TE = T::TE;
    // K slots 0 .. STAGES-1, then V slots; after the key loop the first
    // 32 x D rows per wave stage the output
    __shared__ __attribute__((aligned(1024))) uint16_t ring[2 * T::STAGES * TE];
    static_assert(T::NW * T::R * D <= 2 * T::STAGES * TE, "output staging fits in the ring");
    debug_poison_lds(ring, (int)sizeof(ring));

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 31;          // query row of this lane (within the wave's 32)
    const int g = lane >> 5;           // half of the wave's lanes

    // ---- work-group -> (query tile, head group, sequence) ----------------
    // The work-group's waves cover gw query heads of one K/V head (wave w:
    // head hg*gw + w%gw) and bm = 32*4/gw rows (wave w: row block w/gw), so
    // they all need the same K/V tiles at the same steps.  Launch order is
    // heaviest (latest) query tiles first.
    const int gw = p.gw, gpk = p.G / gw;       // head groups per K/V head
    int t, hg, b;
    {
        const int i = blockIdx.x;
        if (p.xcd_groups > 0) {
            // Keep the head groups of one K/V head (and its neighbouring
            // query tiles) on one XCD: work-group i runs on XCD i % 8.  A
            // padded batch interleaves the XCD's (sequence, K/V head) groups
            // tile by tile (measured best for few groups per XCD); packed
            // sequences (many short groups) take one group after another,
            // so the work-groups in flight on an XCD share one group's K/V
            // in its L2 (the packed workload fetched 7.3 GB per call
            // interleaved, 0.9 GB group after group, and ran 15 % faster).
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
    // The work-group walks tiles [tile_lo, tile_last]; this wave computes
    // [w_lo, w_hi] of them and needs no mask on [in_lo, in_hi] (each of its
    // rows sees every key of such a tile).
    const int wg_last = min(q0 + p.bm, sq) - 1;
    const int kv_lo = lo_of(q0), kv_hi = hi_of(wg_last);
    const int tile_lo = kv_lo / T::BN;
    const int ntiles = kv_hi >= kv_lo ? kv_hi / T::BN - tile_lo + 1 : 0;
    const int tile_last = tile_lo + ntiles - 1;
    const int r0 = q0 + T::R * (wave / gw);
    int w_lo = 1, w_hi = 0;
    if (r0 < sq) {
        const int wlo = lo_of(r0), whi = hi_of(min(r0 + T::R - 1, sq - 1));
        if (whi >= wlo) { w_lo = wlo / T::BN; w_hi = whi / T::BN; }
    }
    const int in_lo = (lo_of(min(r0 + T::R - 1, sq - 1)) + T::BN - 1) / T::BN;
    const int int_hi = hi_of(r0);
    const int in_hi = int_hi + 1 >= T::BN ? (int_hi + 1) / T::BN - 1 : -1;

    // ---- K/V ring in LDS, filled by DMA -----------------------------------
    // Tile pair s = (K_s, V_s): 2*TB 1 KB blocks; wave w issues blocks w,
    // w + NW, ...
    //   K block kb = ks, lane L: key L%32, d-chunk 2*ks + L/32 (operand
    //   order), except with KROW (d = 128, no ALiBi): key 4*kb + L/16, the
    //   key's 16-byte chunk (L%16) ^ (key%16), so that each copy reads 4
    //   whole rows (32 bytes of 32 rows per copy measured 6 % slower on the
    //   sliding window, 1-2 % on the causal and packed workloads) and chunk c
    //   of key r sits at r*256 + 16*(c ^ (r%16)); the A-operand reads stay
    //   conflict free (16 lanes = 16 keys, one chunk each, 16 distinct slots).
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
        dma_k[i] = gb < T::TB;
        const int blk = dma_k[i] ? gb : gb - T::TB;
        dma_loff[i] = blk * 1024;
        if (dma_k[i]) {
            if constexpr (KROW) {
                const int row = 4 * blk + (lane >> 4);
                dma_voff[i] = row * tok_bytes_kv + (((lane & 15) ^ (row & 15)) * 16);
            } else {
                dma_voff[i] = (lane & 31) * tok_bytes_kv + (2 * blk + (lane >> 5)) * 16;
            }
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
    // Bytes of tile jt's rows; callers pass a tile of [tile_lo, tile_last]
    // or -1, which gets a zero record: its loads write zeros to LDS without
    // touching memory (keeps per-step load counts fixed).
    auto tile_bytes = [&](int jt) __attribute__((always_inline)) {
        return jt >= 0 ? min(sk - jt * T::BN, T::BN) * tok_bytes_kv : 0;
    };
    auto tile_rsrc = [&](const char* base, int jt, int bytes) __attribute__((always_inline)) {
        return make_rsrc(base + (long long)jt * (T::BN * tok_bytes_kv), bytes);
    };
    // ring slot i of K and of V (tile jt sits in slot (jt - tile_lo) % STAGES;
    // the steps carry that slot number instead of dividing)
    auto kslot = [&](int i) __attribute__((always_inline)) { return ring + i * TE; };
    auto vslot = [&](int i) __attribute__((always_inline)) { return ring + (T::STAGES + i) * TE; };
    auto next_slot = [&](int i) __attribute__((always_inline)) {
        return i == T::STAGES - 1 ? 0 : i + 1;
    };
    // this wave's LPS copies of tile pair jt into ring slot i
    auto issue = [&](int jt, int i) __attribute__((always_inline)) {
        const int bytes = tile_bytes(jt);
        const i32x4 krs = tile_rsrc(kseq, jt, bytes), vrs = tile_rsrc(vseq, jt, bytes);
        const uint32_t kdst = lds_addr(kslot(i)), vdst = lds_addr(vslot(i));
#pragma unroll
        for (int l = 0; l < T::LPS; ++l) {
            if (dma_k[l]) dma16_to_lds(krs, kdst + dma_loff[l], dma_voff[l], 0);
            else dma16_to_lds(vrs, vdst + dma_loff[l], dma_voff[l], 0);
        }
    };
    // End of step s: this wave's copies of the tiles of every step up to
    // s + 1 have landed (step s + 2's may still be in flight), its LDS reads
    // have returned, then the barrier makes both true for all waves: step
    // s + 1's tile is published and the slot of step s, which step s + 1
    // refills with step s + 3's tile, is free.  The wait and the barrier
    // form one asm statement so that no LDS access is moved across them.
    auto sync_step = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier"
                     ::"n"(FA_VMCNT(T::LPS * (T::AHEAD - 1))) : "memory");
    };

    // ---- the wave's 32 query rows as MFMA B operands ----------------------
    u32x4 qreg[T::KS];
    {
        const auto qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const char*)p.q + (q_tok0 * p.q_tok_stride + (long long)hq * D) * 2),
            (short)0, sq * tok_bytes_q, 0x00020000);   // rows past the sequence read as zeros
        const int row = r0 + lq;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
                qrs, row * tok_bytes_q + (16 * ks + 8 * g) * 2, 0, 0);
            qreg[ks] = x;
        }
        if (p.qsign) {                             // exact negation when scale < 0 (uniform)
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks) qreg[ks] ^= p.qsign;
        }
        // wait for the Q loads here, before any tile copy is issued (a wait
        // the compiler placed at their first use, inside the loop, would
        // drain the copies on every step)
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) asm volatile("" ::"v"(qreg[ks]));
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
        int hh = sk - 1;
        if (causal) hh = min(hh, pos);
        if (wr >= 0) hh = min(hh, pos + wr);
        rel_hi = hh - 4 * g;
    }

    u32x4 pb[T::KK];                           // the weights of a tile as 16-bit B operands
    const float slope2 = ALIBI ? p.alibi[hq] * kLog2e : 0.f;
    const float sc_k = p.sc_k, sc_c = p.sc_c;
    // exp2 argument of element e of a tile with running max m; tb is the
    // distance (key - row position) of the lane's element 0 (ALiBi only)
    auto earg = [&](const f32x16& sacc, int e, float tb, float m) __attribute__((always_inline)) {
        const float sv = sacc[e];
        if constexpr (MOD == 0) {
            return fmaf(sv, c, -m);
        } else {
            float v;
            if constexpr (SOFTCAP) {
                const float ex = exp2_fast(sv * sc_k);
                const float th = fmaf(-2.f, __builtin_amdgcn_rcpf(ex + 1.f), 1.f);
                v = sv == -INFINITY ? -INFINITY : fmaf(th, sc_c, -m);   // masked stays masked
            } else {
                v = fmaf(sv, c, -m);
            }
            if constexpr (ALIBI)
                v = fmaf(-slope2, fabsf(tb + (float)(8 * (e >> 2) + (e & 3))), v);
            return v;
        }
    };
    auto tile_base = [&](int jt) __attribute__((always_inline)) {
        return ALIBI ? (float)(4 * g - lq + (jt * T::BN - r0 - delta)) : 0.f;
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
    // trees (no long chains of dependent adds).
    auto exps = [&](const f32x16& sacc, float tb) __attribute__((always_inline)) {
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float x[16], r2[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = exp2_fast(earg(sacc, e, tb, m_use));
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t pk = pack2<BF16>(x[e], x[e + 1]);
            pb[e >> 3][(e & 7) >> 1] = pk;
            r2[(e >> 1) & 1] = sum2_16_dot<BF16>(pk, e < 4 ? 0.f : r2[(e >> 1) & 1]);
        }
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
            for (int e = 0; e < w; ++e) x[e] += x[e + w];
        return f32x2{x[0], r2[0] + r2[1]};
    };
    auto refresh = [&](const f32x16& sacc, float tb) __attribute__((always_inline)) {
        asm volatile("");   // keep this rare block a real branch (not speculated)
        f32x16 u;                                  // scores (plain) or exponents u (modifiers)
        if constexpr (MOD == 0) {
            u = sacc;
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) u[e] = earg(sacc, e, tb, 0.f);
        }
        float m4[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            m4[q4] = fmaxf(fmaxf(u[4 * q4], u[4 * q4 + 1]), fmaxf(u[4 * q4 + 2], u[4 * q4 + 3]));
        const float mx = max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
        const float mnew = fmaxf(m_run, MOD == 0 ? mx * c : mx);   // -inf stays -inf (c > 0)
        const bool raise = mnew > m_run + kRescaleThreshold;
        const float alpha = raise ? exp2_fast(m_run - mnew) : 1.f;
        l_run *= alpha;
        lr_run *= alpha;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        m_run = raise ? mnew : m_run;
        return exps(sacc, tb);
    };
    auto softmax_tile = [&](const f32x16& sacc, int jt) __attribute__((always_inline)) {
        const bool first = m_run == -INFINITY;
        const float tb = tile_base(jt);
        f32x2 sums = exps(sacc, tb);
        if ((__builtin_amdgcn_ballot_w64(first) | __builtin_amdgcn_ballot_w64(sums.x > 256.f)) != 0ull)
            sums = refresh(sacc, tb);
        l_run += sums.x;
        lr_run += sums.y;
    };

    // operands of S^T = K Q^T from the K tile in slot i
    auto load_k = [&](u32x4 (&kq)[T::KS], int i) __attribute__((always_inline)) {
        const uint16_t* kt = kslot(i);
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks)
            kq[ks] = KROW
                ? *reinterpret_cast<const u32x4*>(kt + (lane & 31) * D + (((2 * ks + (lane >> 5)) ^ (lane & 15)) * 8))
                : *reinterpret_cast<const u32x4*>(kt + ks * 512 + lane * 8);
    };
    // operands of O^T += V^T P^T from the V tile in slot i; operand (kk, db)
    // holds keys 16kk + 8hh + 4g + 0..3 in half hh
    auto load_v = [&](u32x4 (&vq)[T::KK][T::DB], int i) __attribute__((always_inline)) {
        const uint16_t* vt = vslot(i);
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
                const u32x2 lo = ds_read_tr16(vt + ((2 * kk) * T::DB + db) * 256 + lane * 4);
                const u32x2 hi = ds_read_tr16(vt + ((2 * kk + 1) * T::DB + db) * 256 + lane * 4);
                vq[kk][db] = (u32x4){lo.x, lo.y, hi.x, hi.y};
            }
    };
    auto qk = [&](int i) __attribute__((always_inline)) {
        u32x4 kq[T::KS];
        load_k(kq, i);
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) acc = mfma32x32x16<BF16>(kq[ks], qreg[ks], acc);
        return acc;
    };

    // Step on tile jt (in ring slot i): this wave's copies of tile jt_ahead
    // (the tile two steps later, or none), then, for the tiles of this wave, S^T = K Q^T, the mask (boundary
    // tiles only), the softmax and O^T += V^T P^T; steps outside [w_lo,
    // w_hi] only copy and synchronise.
    auto step = [&](int jt, int jt_ahead, int i) __attribute__((always_inline)) {
        issue(jt_ahead, i == 0 ? T::STAGES - 1 : i - 1);
        if (jt >= w_lo && jt <= w_hi) {                // uniform per wave
            f32x16 cur = qk(i);
            if (jt < in_lo || jt > in_hi)
                mask_acc32(cur, rel_lo - jt * T::BN, rel_hi - jt * T::BN);
            softmax_tile(cur, jt);
            u32x4 vq[T::KK][T::DB];
            load_v(vq, i);
#pragma unroll
            for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
                for (int db = 0; db < T::DB; ++db)
                    oacc[db] = mfma32x32x16<BF16>(vq[kk][db], pb[kk], oacc[db]);
        }
        sync_step();
        return next_slot(i);
    };
    // ALiBi: the bias grows toward each row's own position, so in key order
    // a row's running max would climb tile after tile (and take the rare
    // path on most steps).  Instead the max starts at the row's largest
    // modified score in the tile holding the wave's last diagonal key,
    // loaded straight from memory here: a value the row attains, so the
    // running max never exceeds the true one.  (A zero slope keeps the plain
    // order of maxima, hence the plain result bit for bit.)
    if constexpr (ALIBI) {
        if (ntiles > 0 && slope2 != 0.f && w_lo <= w_hi) {          // uniform per wave
            const int dt = min(max((r0 + T::R - 1 + delta) / T::BN, w_lo), w_hi);
            const auto krs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(kseq + (long long)dt * (T::BN * tok_bytes_kv)), (short)0,
                min(sk - dt * T::BN, T::BN) * tok_bytes_kv, 0x00020000);
            f32x16 acc;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks) {
                const u32x4 kq = __builtin_amdgcn_raw_buffer_load_b128(
                    krs, (lane & 31) * tok_bytes_kv + (2 * ks + g) * 16, 0, 0);
                acc = mfma32x32x16<BF16>(kq, qreg[ks], acc);
            }
            mask_acc32(acc, rel_lo - dt * T::BN, rel_hi - dt * T::BN);
            const float tb = tile_base(dt);
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, earg(acc, e, tb, 0.f));
            m_run = max_halves(mx);
        }
    }

    if (ntiles > 0) {
        // Step s takes tile tile_lo + (s - tile_lo) mod ntiles, the tile
        // congruent to s modulo the range length.  With a causal mask
        // (tile_lo = 0) that is tile s; under a sliding window every work-
        // group's range has the same length, so neighbouring query tiles,
        // which run at about the same time on one XCD, read each K/V tile
        // they share at the same step and the second read hits L2 (window
        // workload: 1.77 -> 0.89 GB fetched, 7 % faster).  The online
        // softmax takes the keys in any order.
        auto tile_at = [&](int s) __attribute__((always_inline)) {
            if (s >= ntiles) return -1;                    // past the range: no copy
            int r = (s - tile_lo) % ntiles;
            r += r < 0 ? ntiles : 0;
            return tile_lo + r;
        };
        for (int s = 0; s < T::AHEAD; ++s) issue(tile_at(s), s);
        sync_step();
        // the tiles of steps s and s + AHEAD, advanced by one per step with
        // the wrap of the rotated order (no division in the loop)
        const int tile_end = tile_lo + ntiles;
        int jt = tile_at(0);
        int ja = T::AHEAD < ntiles ? tile_at(T::AHEAD) : tile_lo;
        int i = 0;
        for (int s = 0; s < ntiles; ++s) {
            i = step(jt, s + T::AHEAD < ntiles ? ja : -1, i);
            jt = jt + 1 == tile_end ? tile_lo : jt + 1;
            ja = ja + 1 == tile_end ? tile_lo : ja + 1;
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // DMA loads of unused tiles still in flight

    // ---- epilogue: normalise once, write O and LSE -----------------------
    // O goes through LDS so that every store writes whole rows: in the
    // accumulator layout a store instruction would cover 16 bytes of each of
    // 32 rows.  Each wave stages its 32 x D tile in its own part of the
    // (now idle) ring, rows of D/8 16-byte chunks with chunk c of row r at
    // c ^ (r % (D/8)) (conflict-free reads), then stores D/8 lanes per row.
    constexpr int CH = D / 8;                  // 16-byte chunks per row
    asm volatile("s_barrier" ::: "memory");    // every wave is done with the ring
    char* stage = reinterpret_cast<char*>(ring) + wave * (T::R * D * 2);
    const float l_tot = sum_halves(l_run);
    const float lr_tot = sum_halves(lr_run);
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            u32x2 w;
            w.x = pack2<BF16>(oacc[db][4 * jj + 0] * inv, oacc[db][4 * jj + 1] * inv);
            w.y = pack2<BF16>(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
            const int chunk = (4 * db + jj) ^ (lq % CH);   // columns 32db + 8jj .. +7
            *reinterpret_cast<u32x2*>(stage + lq * (2 * D) + chunk * 16 + 8 * g) = w;
        }
    const int row = r0 + lq;
    if (p.lse != nullptr && g == 0 && row < sq) {
        const long long row_base = VARLEN ? q_tok0 : 0;
        const float lse = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
        p.lse[(long long)b * p.lse_b_stride + (long long)hq * p.lse_h_stride + row_base + row] = lse;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's own staging writes
    const auto ors = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((char*)p.o + (q_tok0 * p.q_tok_stride + (long long)hq * D) * 2), (short)0,
        sq * tok_bytes_q, 0x00020000);          // rows past the sequence are dropped
    constexpr int RPI = 64 / CH;               // rows per store instruction
#pragma unroll
    for (int i = 0; i < T::R / RPI; ++i) {
        const int r = RPI * i + lane / CH, cc = lane % CH;
        const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * (2 * D) + ((cc ^ (r % CH)) * 16));
        __builtin_amdgcn_raw_buffer_store_b128(x, ors, (r0 + r) * tok_bytes_q + cc * 16, 0, 0);
    }
}

template <int D, bool BF16, bool VARLEN, int MOD>
static hipError_t launch_one(const FwdParams& p, hipStream_t s) {
    const long long nblocks = (long long)p.nqt * (p.Hq / p.gw) * p.B;
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, VARLEN, MOD>), dim3((unsigned)nblocks),
                       dim3(kFwdThreads), 0, s, p);
    return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_padded(const FwdParams& p, hipStream_t s) {
    switch (p.mod) {
        case 1: return launch_one<D, BF16, false, 1>(p, s);
        case 2: return launch_one<D, BF16, false, 2>(p, s);
        case 3: return launch_one<D, BF16, false, 3>(p, s);
        default: return launch_one<D, BF16, false, 0>(p, s);
    }
}

hipError_t launch_fwd(const FwdParams& p, int d, bool bf16, bool varlen, hipStream_t s) {
    if (varlen) {
        if (d == 128) return bf16 ? launch_one<128, true, true, 0>(p, s) : launch_one<128, false, true, 0>(p, s);
        return bf16 ? launch_one<64, true, true, 0>(p, s) : launch_one<64, false, true, 0>(p, s);
    }
    if (d == 128) return bf16 ? launch_padded<128, true>(p, s) : launch_padded<128, false>(p, s);
    return bf16 ? launch_padded<64, true>(p, s) : launch_padded<64, false>(p, s);
}

}  // namespace fa
