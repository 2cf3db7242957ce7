// fa_bwd.hip -- gradients of the fused attention (the training backward) for
// gfx950.
//
// The method: the "FlashAttention" explainer page, "Step 5" and "Backward
// pass in a bit more detail".  No score or weight matrix is stored by the
// forward; the backward recomputes the score tiles from Q and K and rebuilds
// the weights from the saved per-row log-normaliser (P = exp(S - LSE) is
// already normalised, so there is no running max here), then forms the local
// gradient pieces on chip.  Gradients of K and V accumulate across query
// blocks, the gradient of Q across key blocks.  Each of the two accumulations
// stays on chip in a kernel of its own, so no partial sums go to memory and
// no floating-point atomics are used (results are bitwise reproducible):
//
//   fa_bwd_dkdv_kernel  one work-group per 256 keys of one K/V head: for
//                       every query head of the group and every 32-row query
//                       block that sees those keys
//                           S = Q K^T,  P = exp2(S c2 - LSE_2),
//                           dP - D = dO V^T accumulated from -D,
//                           dS = P (dP - D),  dV^T += dO^T P,  dK^T += Q^T dS;
//   fa_bwd_dq_kernel    (enqueued first) one work-group per query block (the
//                       query heads of one K/V head); first the row term of dS,
//                       D_i = dO_i . O_i (O = the forward's output), which
//                       it also stores, negated, for the next kernel; then for every
//                       32-key tile it sees
//                           S^T = K Q^T,  dP^T = V dO^T,  the same P and dS,
//                           dQ^T += K^T dS^T;
// with c2 = scale * log2(e), LSE_2 = LSE * log2(e), and dK, dQ multiplied by
// the scale at the end (chain rule of S = scale * Q K^T).
//
// Data movement follows the forward kernel: 32-row tiles go from HBM/L2
// straight into LDS with bounds-checked buffer_load_dwordx4 ... lds (rows
// past the end read as zeros), in one of two operand orders:
//   * A order: block b holds d-chunk 2b + L/32 of row L%32 at lane L, so the
//     A operand of reduction step b is one contiguous 1 KB read;
//   * T order: the 8-byte slots ds_read_b64_tr_b16 reads, so the transposed
//     operand (d x 16 rows) of a 32x32x16 MFMA is two contiguous 512 B reads.
// A ring of stages holds the tiles (4 in the dK/dV kernel, whose stage also
// carries the rows' LSE and D, 5 in the dQ kernel); one barrier per step
// publishes a stage and frees the oldest one for the next copy.  The
// operands that stay fixed for a work-group (K and V of the wave's keys in
// the dK/dV kernel, Q and dO of the wave's rows in the dQ kernel) are loaded
// once into registers (in the dQ kernel the accumulation registers, which
// MFMAs read directly).  Both kernels run two waves per SIMD at d = 128.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <int D, int WAVES>
struct BwdGeo {
    static constexpr int R = 32;                 // rows (or keys) per tile and per wave
    static constexpr int NW = WAVES;             // waves per work-group
    static constexpr int KS = D / 16;            // reduction steps over d
    static constexpr int DB = D / 32;            // 32-column blocks of d
    static constexpr int TE = R * D;             // elements per tile
    static constexpr int TB = TE * 2 / 1024;     // 1 KB blocks per tile
};
constexpr int kDkdvStages = 4;   // ring depth of the dK/dV kernel (stage: 4 tiles + row terms)
constexpr int kDqStages = 5;     // ring depth of the dQ kernel (stage: 3 tiles)

// 4 bytes per lane from a buffer straight into LDS (buffer_load_dword ...
// lds): lane i writes lds_base + 4*i; out-of-range offsets write zeros.  Not
// tracked by the compiler (no destination registers): the caller waits
// with s_waitcnt vmcnt before reading the LDS it fills.
__device__ __forceinline__ void dma4_to_lds(i32x4 rsrc, uint32_t lds_base, int voffset) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %0, %1, 0 offen lds"
        :
        : "v"(voffset), "s"(rsrc), "s"(lds_base)
        : "memory", "m0");
}

typedef __attribute__((address_space(3))) short bwd_lds_short;
typedef short bwd_i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 tr16_read(const uint16_t* p) {
    bwd_i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) bwd_i16x4*)(bwd_lds_short*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// A buffer resource whose fields are wave-uniform values computed in vector
// registers (integer division has no scalar form): copy them to scalars.
__device__ __forceinline__ i32x4 uniform_rsrc(i32x4 r) {
    return (i32x4){__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                   __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w)};
}

__device__ __forceinline__ u32x4 to_acc_regs(u32x4 v) {
    u32x4 r;
    asm("" : "=a"(r) : "0"(v));
    return r;
}

// Source byte offset of lane L's 16-byte chunk for block b of a 32-row tile
// (rows tok_bytes apart) in A order.
__device__ __forceinline__ int a_order_off(int b, int lane, int tok_bytes) {
    return (lane & 31) * tok_bytes + (2 * b + (lane >> 5)) * 16;
}
// ... in T order: 16-byte unit u = 64 b + L, half-block hb = u / 32 =
// kh*DB + db, r = u % 32 -> row 8 kh + 4 (r/16) + (r/2) % 4, d-chunk
// 4 db + 2 ((r/8) % 2) + r % 2.
template <int DB>
__device__ __forceinline__ int t_order_off(int b, int lane, int tok_bytes) {
    const int hb = 2 * b + (lane >> 5), r = lane & 31;
    const int kh = hb / DB, db = hb % DB;
    const int row = 8 * kh + 4 * (r >> 4) + ((r >> 1) & 3);
    const int chunk = 4 * db + 2 * ((r >> 3) & 1) + (r & 1);
    return row * tok_bytes + chunk * 16;
}

// Operand reads from a tile in LDS.
template <int D>
__device__ __forceinline__ u32x4 a_operand(const uint16_t* tile, int ks, int lane) {
    return *reinterpret_cast<const u32x4*>(tile + ks * 512 + lane * 8);
}
// Transposed operand (kk, db): d columns 32 db .. +31 (lane l: column l%32)
// by rows 16 kk + 4 (l/32) + {0..3} and 16 kk + 8 + 4 (l/32) + {0..3}.
template <int D>
__device__ __forceinline__ u32x4 t_operand(const uint16_t* tile, int kk, int db, int lane) {
    constexpr int DB = D / 32;
    const u32x2 lo = tr16_read(tile + ((2 * kk) * DB + db) * 256 + lane * 4);
    const u32x2 hi = tr16_read(tile + ((2 * kk + 1) * DB + db) * 256 + lane * 4);
    return (u32x4){lo.x, lo.y, hi.x, hi.y};
}

// Accumulator element e of a 32x32 MFMA result sits at row 8*(e/4) +
// 4*(lane/32) + e%4 of the 32-row block: its offset without the lane term.
__device__ __forceinline__ constexpr int acc_row(int e) { return 8 * (e >> 2) + (e & 3); }
template <bool B>
struct mask_c {
    static constexpr bool value = B;
};

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// dK and dV of 32*NW keys of one K/V head.  Wave w owns keys k0 + 32w ..
// +31; the work-group walks (query head of the group) x (32-row query
// block).  NW = 8: two waves per SIMD (one's vector work runs beside the
// other's matrix instructions) and each Q/dO stage copied to LDS serves 256
// keys.  At two waves per SIMD a wave has 256 registers; using none of the
// accumulation registers keeps all 256 as ordinary ones (the compiler
// splits the budget in halves once any accumulation register is used), and
// the rows' LSE and D are read from the stage where they are used.
template <int D, bool BF16>
__global__ __launch_bounds__(64 * kBwdDkdvWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(BwdParams p) {
    using T = BwdGeo<D, kBwdDkdvWaves>;
    constexpr int TE = T::TE;
    // stage s: Q (A order), dO (A order), Q (T order), dO (T order), then
    // the LSE and D of the block's rows (256 bytes each, the first 128 used)
    constexpr int SE = 4 * TE + 256;             // stage size in 16-bit elements
    constexpr int NS = kDkdvStages;
    __shared__ __attribute__((aligned(1024))) uint16_t ring[NS * SE];
    debug_poison_lds(ring, (int)sizeof(ring));

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 5;
    __builtin_assume(wave >= 0 && wave < T::NW);

    // work-group -> (key block, K/V head, sequence); all first key blocks
    // (the most-seen ones under a causal mask) are launched first
    const int nbh = p.B * p.Hkv;
    const int kb = blockIdx.x / nbh;
    const int bh = blockIdx.x - kb * nbh;
    const int b = bh / p.Hkv, hkv = bh - b * p.Hkv;
    const int sq = p.Sq, sk = p.Sk, delta = sk - sq;
    const int k0 = kb * kBwdKeysPerWg;
    const int k1 = min(k0 + kBwdKeysPerWg, sk) - 1;
    static_assert(kBwdKeysPerWg == T::R * T::NW, "keys per work-group");
    const int kw0 = k0 + T::R * wave;           // this wave's first key
    const int j = kw0 + (lane & 31);            // this lane's key

    // rows that see any key of [k0, k1] form one interval [ia, ib]
    int ia = 0, ib = sq - 1;
    if (p.causal) ia = max(ia, k0 - delta);
    if (p.wr >= 0) ia = max(ia, k0 - delta - p.wr);
    if (p.wl >= 0) ib = min(ib, k1 - delta + p.wl);
    const int qb_a = ia <= ib ? ia / T::R : 0;
    const int nqb = ia <= ib ? ib / T::R - qb_a + 1 : 0;
    const int nsteps = nqb * p.G;

    // key j is visible from row i iff t = j - delta - i lies in [t_lo, t_hi]
    const int t_hi = p.causal ? (p.wr >= 0 ? min(0, p.wr) : 0) : (p.wr >= 0 ? p.wr : 0x3fffffff);
    const int t_lo = p.wl >= 0 ? -p.wl : -0x3fffffff;

    const int tok_q = (int)(p.q_tok_stride * 2), tok_kv = (int)(p.kv_tok_stride * 2);

    // ---- K and V of this wave's keys as B operands (lane: key l%32) ------
    u32x4 kop[T::KS], vop[T::KS];
    {
        const long long base = ((long long)b * sk * p.Hkv + hkv) * D * 2;
        const auto krs = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.k + base), (short)0,
                                                           sk * tok_kv, 0x00020000);
        const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.v + base), (short)0,
                                                           sk * tok_kv, 0x00020000);
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            const int off = j * tok_kv + (16 * ks + 8 * g) * 2;
            kop[ks] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
            vop[ks] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
        }
        // Wait for these loads here, before any tile copy is issued: the
        // compiler does not see the copies (they are written in asm), and a
        // wait it placed at the first use, inside the loop, would run on
        // every step and drain every copy in flight.
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) asm volatile("" ::"v"(kop[ks]), "v"(vop[ks]));
    }

    // ---- copies of step s: Q and dO rows of query block qb_a + s % nqb of
    // head hkv*G + s / nqb, in A and T order, and the LSE and D of those
    // rows (every wave copies those two 256-byte pieces to the same place,
    // so all waves issue the same number of loads); stages past the last
    // step read nothing (zero records) so every step issues the same number
    // of loads.  The row terms come through the copy path too: a plain
    // vector load would complete in order behind the copies, and waiting
    // for it would wait for every copy issued before it.
    constexpr int NB = 4 * T::TB;                // blocks per stage
    constexpr int LPS = NB / T::NW + 2;          // copies per wave per stage
    static_assert(NB % T::NW == 0, "blocks split evenly over the waves");
    // The copied step's first query row and head, the byte offset of its Q
    // and dO rows and the element offset of its row terms; stepped by
    // advance() (no multiplications in the loop but at a change of head).
    struct Cursor {
        int i0, h;
        long long qo, ro;
    };
    auto cursor_at = [&](int ih) __attribute__((always_inline)) {
        Cursor c;
        c.i0 = qb_a * T::R;
        c.h = hkv * p.G + ih;
        c.qo = (((long long)b * sq + c.i0) * p.Hq + c.h) * D * 2;
        c.ro = ((long long)b * p.Hq + c.h) * sq + c.i0;
        return c;
    };
    auto advance = [&](Cursor& c, int& iq, int& ih) __attribute__((always_inline)) {
        if (++iq == nqb) {
            iq = 0;
            c = cursor_at(++ih);
        } else {
            c.i0 += T::R;
            c.qo += (long long)T::R * p.Hq * D * 2;
            c.ro += T::R;
        }
    };
    auto issue = [&](int s, const Cursor& cu) __attribute__((always_inline)) {
        const int rows = s < nsteps ? max(min(sq - cu.i0, T::R), 0) : 0;
        const i32x4 qrs = uniform_rsrc(make_rsrc((const char*)p.q + cu.qo, rows * tok_q));
        const i32x4 ors = uniform_rsrc(make_rsrc((const char*)p.dout + cu.qo, rows * tok_q));
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(ring + (s % NS) * SE));
        dma4_to_lds(uniform_rsrc(make_rsrc(p.lse2 + cu.ro, rows * 4)), dst + 4 * TE * 2, lane * 4);
        dma4_to_lds(uniform_rsrc(make_rsrc(p.dsum + cu.ro, rows * 4)), dst + 4 * TE * 2 + 256, lane * 4);
#pragma unroll
        for (int c = 0; c < LPS - 2; ++c) {
            const int blk = wave + c * T::NW;    // 0 .. NB-1
            const int tile = blk / T::TB, bb = blk % T::TB;   // tile 0 Q_A, 1 dO_A, 2 Q_T, 3 dO_T
            const int voff = tile < 2 ? a_order_off(bb, lane, tok_q) : t_order_off<T::DB>(bb, lane, tok_q);
            dma16_to_lds((tile & 1) ? ors : qrs, dst + tile * TE * 2 + bb * 1024, voff, 0);
        }
    };
    // wait for this wave's copies of step s (those of steps s+1 .. s+NS-2
    // may still fly), then a barrier: every wave's copies of step s are
    // visible and every wave is done with step s-1, whose stage step s+NS-1
    // refills
    auto sync_step = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(FA_VMCNT(LPS * (NS - 2))) : "memory");
    };

    f32x16 dkt[T::DB], dvt[T::DB];               // dK^T, dV^T: lane = key, element = d
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) { dkt[db][e] = 0.f; dvt[db][e] = 0.f; }

    if (nsteps > 0) {
        // query block and head of the next step to copy, and the query
        // block of step s, advanced per step (no division in the loop)
        int iq = 0, ih = 0, cq = 0;
        Cursor cur = cursor_at(0);
        for (int s = 0; s < NS - 1; ++s) {
            issue(s, cur);
            advance(cur, iq, ih);
        }
        for (int s = 0; s < nsteps; ++s) {
            sync_step();
            issue(s + NS - 1, cur);
            advance(cur, iq, ih);
            const int i0 = (qb_a + cq) * T::R;
            if (++cq == nqb) cq = 0;
            // rows of this block that see a key of this wave: t = j - delta -
            // i spans [kw0 - delta - i0 - 31, kw0 + 31 - delta - i0]
            const int tmax = kw0 + T::R - 1 - delta - i0, tmin = kw0 - delta - i0 - (T::R - 1);
            if (tmax < t_lo || tmin > t_hi || kw0 >= sk) continue;   // uniform per wave
            const uint16_t* st = ring + (s % NS) * SE;
            const uint16_t* qa = st;
            const uint16_t* oa = st + TE;
            const uint16_t* qt = st + 2 * TE;
            const uint16_t* ot = st + 3 * TE;
            const float* lse_s = reinterpret_cast<const float*>(st + 4 * TE);
            const float* d_s = lse_s + 64;

            // dP starts from -D of its rows (element e: row i0 + acc_row(e) +
            // 4g; the dQ kernel stores the row terms negated), so the
            // accumulator ends as dP - D, the factor of dS
            f32x16 sacc = {}, dpacc;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(d_s + 8 * q4 + 4 * g);
#pragma unroll
                for (int k = 0; k < 4; ++k) dpacc[4 * q4 + k] = d4[k];
            }
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks) {
                sacc = mfma32x32x16<BF16>(a_operand<D>(qa, ks, lane), kop[ks], sacc);
                dpacc = mfma32x32x16<BF16>(a_operand<D>(oa, ks, lane), vop[ks], dpacc);
            }
            // P and dS; element e is row i0 + acc_row(e) + 4g of key j.  The
            // rows' LSE (log2 units) are read from the stage four at a time,
            // where they are used.
            u32x4 pp[2], pds[2];
            auto weights = [&](auto maskc) __attribute__((always_inline)) {
                // (distinct markers keep the compiler from hoisting the two
                // versions' common arithmetic above the branch, which would
                // hold all 32 intermediate values at once)
                uint32_t vis = 0u;
                if constexpr (decltype(maskc)::value) {
                    asm volatile("; masked block");
                    const int tb = j - delta - i0 - 4 * g;
                    // visible iff tb - t_hi <= acc_row(e) <= tb - t_lo
                    vis = j < sk ? vis_bits(tb - t_hi, tb - t_lo) : 0u;
                } else {
                    asm volatile("; unmasked block");
                }
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + 8 * q4 + 4 * g);
#pragma unroll
                    for (int e2 = 0; e2 < 4; e2 += 2) {
                        const int e = 4 * q4 + e2;
                        float pv[2], dv2[2];
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            // LSE in log2 units, +inf for a row with no
                            // visible key (weights exp2(x - inf) = 0, never inf)
                            pv[u] = exp2_fast(fmaf(sacc[e + u], p.c2, -l4[e2 + u]));
                            if constexpr (decltype(maskc)::value)
                                pv[u] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, pv[u]) &
                                                                      bit_mask(vis, acc_row(e + u)));
                            dv2[u] = pv[u] * dpacc[e + u];
                        }
                        pp[e >> 3][(e & 7) >> 1] = pack2<BF16>(pv[0], pv[1]);
                        pds[e >> 3][(e & 7) >> 1] = pack2<BF16>(dv2[0], dv2[1]);
                    }
                }
            };
            // every (row, key) pair of the block visible (under a causal mask:
            // all blocks off the diagonal): no mask
            if (kw0 + T::R <= sk && tmin >= t_lo && tmax <= t_hi) weights(mask_c<false>{});
            else weights(mask_c<true>{});
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int db = 0; db < T::DB; ++db) {
                    dvt[db] = mfma32x32x16<BF16>(t_operand<D>(ot, kk, db, lane), pp[kk], dvt[db]);
                    dkt[db] = mfma32x32x16<BF16>(t_operand<D>(qt, kk, db, lane), pds[kk], dkt[db]);
                }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // copies of unused stages

    // ---- store dK = scale * dK^T and dV (lane: key j, element e: d index
    // 32 db + acc_row(e) + 4g), 8 bytes per (db, e/4)
    const long long kbase = ((long long)b * sk * p.Hkv + hkv) * D * 2;
    const auto dkrs = __builtin_amdgcn_make_buffer_rsrc((void*)((char*)p.dk + kbase), (short)0,
                                                        sk * tok_kv, 0x00020000);
    const auto dvrs = __builtin_amdgcn_make_buffer_rsrc((void*)((char*)p.dv + kbase), (short)0,
                                                        sk * tok_kv, 0x00020000);
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int off = j * tok_kv + (32 * db + 8 * q4 + 4 * g) * 2;
            u32x2 wk, wv;
            wk.x = pack2<BF16>(dkt[db][4 * q4] * p.scale, dkt[db][4 * q4 + 1] * p.scale);
            wk.y = pack2<BF16>(dkt[db][4 * q4 + 2] * p.scale, dkt[db][4 * q4 + 3] * p.scale);
            wv.x = pack2<BF16>(dvt[db][4 * q4], dvt[db][4 * q4 + 1]);
            wv.y = pack2<BF16>(dvt[db][4 * q4 + 2], dvt[db][4 * q4 + 3]);
            if (j < sk) {
                __builtin_amdgcn_raw_buffer_store_b64(wk, dkrs, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(wv, dvrs, off, 0, 0);
            }
        }
}

// ---------------------------------------------------------------------------
// dQ of one query block: gw query heads of one K/V head (wave w: head
// hg*gw + w%gw) and 32*NW/gw rows (wave w: rows q0 + 32*(w/gw) .. +31).
// NW = 8 at d = 128: two waves per SIMD, so one wave's vector work (the
// weights, dS) runs beside the other's matrix instructions, and each K/V
// stage copied to LDS serves twice the rows.
template <int D, bool BF16>
__global__ __launch_bounds__(64 * bwd_dq_waves(D)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(BwdParams p) {
    using T = BwdGeo<D, bwd_dq_waves(D)>;
    constexpr int TE = T::TE;
    // stage s: K (A order), V (A order), K (T order)
    constexpr int NS = kDqStages;
    __shared__ __attribute__((aligned(1024))) uint16_t ring[NS * 3 * TE];
    debug_poison_lds(ring, (int)sizeof(ring));

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 31;
    const int g = lane >> 5;
    __builtin_assume(wave >= 0 && wave < T::NW);

    const int gw = p.gw, bm = T::R * T::NW / gw;
    const int ngrp = p.Hq / gw;
    const int per_t = p.B * ngrp;
    const int trev = blockIdx.x / per_t, rem = blockIdx.x - trev * per_t;
    const int b = rem / ngrp, hg = rem - b * ngrp;
    const int qt_idx = p.nqb - 1 - trev;                 // latest (most-seeing) blocks first
    const int hq = hg * gw + wave % gw;
    const int hkv = hq / p.G;
    const int sq = p.Sq, sk = p.Sk, delta = sk - sq;
    const int q0 = qt_idx * bm;                          // first row of the work-group
    const int r0 = q0 + T::R * (wave / gw);              // first row of this wave
    const int row = r0 + lq;
    const int tok_q = (int)(p.q_tok_stride * 2), tok_kv = (int)(p.kv_tok_stride * 2);

    auto lo_of = [&](int i) __attribute__((always_inline)) {
        return p.wl >= 0 ? max(0, i + delta - p.wl) : 0;
    };
    auto hi_of = [&](int i) __attribute__((always_inline)) {
        int hh = sk - 1;
        if (p.causal) hh = min(hh, i + delta);
        if (p.wr >= 0) hh = min(hh, i + delta + p.wr);
        return hh;
    };
    const int wg_last = min(q0 + bm, sq) - 1;
    const int kv_lo = lo_of(q0), kv_hi = wg_last >= q0 ? hi_of(wg_last) : -1;
    const int tile_lo = kv_lo / T::R;
    const int ntiles = kv_hi >= kv_lo ? kv_hi / T::R - tile_lo + 1 : 0;

    // ---- Q and dO of this wave's rows as B operands (lane: row l%32) ------
    u32x4 qop[T::KS], oop[T::KS];
    float dd_row;
    {
        const long long base = ((long long)b * sq * p.Hq + hq) * D * 2;
        const auto qrs = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.q + base), (short)0,
                                                           sq * tok_q, 0x00020000);
        const auto ors = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.dout + base), (short)0,
                                                           sq * tok_q, 0x00020000);
        const auto outrs = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.o + base), (short)0,
                                                             sq * tok_q, 0x00020000);
        // the row term D = dO . O of this lane's row: each lane holds half of
        // the row's d values (fp32 products and sums of exactly widened
        // 16-bit values), the lane l ^ 32 the other half
        float dpart = 0.f;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            const int off = row * tok_q + (16 * ks + 8 * g) * 2;
            const u32x4 go = __builtin_amdgcn_raw_buffer_load_b128(ors, off, 0, 0);
            const u32x4 oo = __builtin_amdgcn_raw_buffer_load_b128(outrs, off, 0, 0);
            qop[ks] = to_acc_regs(__builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t x = go[w], y = oo[w];
                float xl, xh, yl, yh;
                if constexpr (BF16) {
                    xl = __builtin_bit_cast(float, x << 16); xh = __builtin_bit_cast(float, x & 0xffff0000u);
                    yl = __builtin_bit_cast(float, y << 16); yh = __builtin_bit_cast(float, y & 0xffff0000u);
                } else {
                    const f16x2 xv = __builtin_bit_cast(f16x2, x), yv = __builtin_bit_cast(f16x2, y);
                    xl = (float)xv[0]; xh = (float)xv[1]; yl = (float)yv[0]; yh = (float)yv[1];
                }
                dpart = fmaf(xl, yl, dpart);
                dpart = fmaf(xh, yh, dpart);
            }
            oop[ks] = to_acc_regs(go);
        }
        dd_row = sum_halves(dpart);
    }
    float lse2 = INFINITY, dd = 0.f;                      // rows past the end: no weight
    if (row < sq) {
        const long long ri = ((long long)b * p.Hq + hq) * sq + row;
        const float l = p.lse[ri];
        lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
        dd = dd_row;
        if (g == 0) {                                     // for the dK/dV kernel, which runs next
            p.dsum[ri] = -dd;
            p.lse2[ri] = lse2;
        }
    }
    // this lane's visible key interval, relative to its first key offset 4g
    int rel_lo, rel_hi;
    {
        const int pos = row + delta;
        rel_lo = (p.wl >= 0 ? pos - p.wl : -0x40000000) - 4 * g;
        int hh = sk - 1;
        if (p.causal) hh = min(hh, pos);
        if (p.wr >= 0) hh = min(hh, pos + p.wr);
        rel_hi = (row < sq ? hh : -0x40000000) - 4 * g;
    }

    constexpr int NB = 3 * T::TB;
    static_assert(NB % T::NW == 0, "blocks split evenly over the waves");
    constexpr int LPS = NB / T::NW;
    const long long kvbase = ((long long)b * sk * p.Hkv + hkv) * D * 2;
    // copies of step s (tile tile_lo + s, K/V byte offset off) into ring
    // slot si; past the last tile they read nothing (zero records)
    auto issue = [&](int s, int si, long long off) __attribute__((always_inline)) {
        const int jt = tile_lo + s;
        const int rows = s < ntiles ? max(min(sk - jt * T::R, T::R), 0) : 0;
        const i32x4 krs = uniform_rsrc(make_rsrc((const char*)p.k + off, rows * tok_kv));
        const i32x4 vrs = uniform_rsrc(make_rsrc((const char*)p.v + off, rows * tok_kv));
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(ring + si * 3 * TE));
#pragma unroll
        for (int c = 0; c < LPS; ++c) {
            const int blk = wave + c * T::NW;
            const int tile = blk / T::TB, bb = blk % T::TB;   // tile 0 K_A, 1 V_A, 2 K_T
            const int voff = tile < 2 ? a_order_off(bb, lane, tok_kv) : t_order_off<T::DB>(bb, lane, tok_kv);
            dma16_to_lds(tile == 1 ? vrs : krs, dst + tile * TE * 2 + bb * 1024, voff, 0);
        }
    };
    auto sync_step = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(FA_VMCNT(LPS * (NS - 2))) : "memory");
    };

    f32x16 dqt[T::DB];                                    // dQ^T: lane = row, element = d
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dqt[db][e] = 0.f;

    if (ntiles > 0) {
        // the copied step's K/V offset and the ring slots of the copied and
        // the current step, advanced per step (no multiply or division)
        const long long tile_step = (long long)T::R * tok_kv;
        long long coff = kvbase + tile_lo * tile_step;
        for (int s = 0; s < NS - 1; ++s, coff += tile_step) issue(s, s, coff);
        int ci = NS - 1, si = 0;
        for (int s = 0; s < ntiles; ++s) {
            sync_step();
            issue(s + NS - 1, ci, coff);
            coff += tile_step;
            ci = ci == NS - 1 ? 0 : ci + 1;
            const int jt = tile_lo + s;
            const uint16_t* st = ring + si * 3 * TE;
            si = si == NS - 1 ? 0 : si + 1;
            const uint16_t* ka = st;
            const uint16_t* va = st + TE;
            const uint16_t* kt = st + 2 * TE;
            // does any row of this wave see a key of tile jt?
            const int wlast = min(r0 + T::R, sq) - 1;
            if (wlast < r0 || hi_of(wlast) < jt * T::R || lo_of(r0) > jt * T::R + T::R - 1) continue;
            f32x16 sacc = {}, dpacc = {};
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks) {
                sacc = mfma32x32x16<BF16>(a_operand<D>(ka, ks, lane), qop[ks], sacc);
                dpacc = mfma32x32x16<BF16>(a_operand<D>(va, ks, lane), oop[ks], dpacc);
            }
            u32x4 pds[2];
            auto weights = [&](auto maskc) __attribute__((always_inline)) {
                uint32_t vis = 0u;
                if constexpr (decltype(maskc)::value) vis = vis_bits(rel_lo - jt * T::R, rel_hi - jt * T::R);
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    float dv2[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        float pv = exp2_fast(fmaf(sacc[e + u], p.c2, -lse2));
                        if constexpr (decltype(maskc)::value)
                            pv = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, pv) &
                                                               bit_mask(vis, acc_row(e + u)));
                        dv2[u] = pv * (dpacc[e + u] - dd);
                    }
                    pds[e >> 3][(e & 7) >> 1] = pack2<BF16>(dv2[0], dv2[1]);
                }
            };
            // every valid row of the wave sees every key of the tile (rows
            // past the end have no weight anyway): no mask
            if (lo_of(wlast) <= jt * T::R && hi_of(r0) >= jt * T::R + T::R - 1) weights(mask_c<false>{});
            else weights(mask_c<true>{});
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int db = 0; db < T::DB; ++db)
                    dqt[db] = mfma32x32x16<BF16>(t_operand<D>(kt, kk, db, lane), pds[kk], dqt[db]);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const long long qbase = ((long long)b * sq * p.Hq + hq) * D * 2;
    const auto dqrs = __builtin_amdgcn_make_buffer_rsrc((void*)((char*)p.dq + qbase), (short)0,
                                                        sq * tok_q, 0x00020000);
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            u32x2 w;
            w.x = pack2<BF16>(dqt[db][4 * q4] * p.scale, dqt[db][4 * q4 + 1] * p.scale);
            w.y = pack2<BF16>(dqt[db][4 * q4 + 2] * p.scale, dqt[db][4 * q4 + 3] * p.scale);
            if (row < sq)
                __builtin_amdgcn_raw_buffer_store_b64(w, dqrs, row * tok_q + (32 * db + 8 * q4 + 4 * g) * 2, 0, 0);
        }
}

template <int D, bool BF16>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
    // dQ first: it also writes the row terms -D the dK/dV kernel reads
    if (p.Sq > 0) {
        const long long n = (long long)p.nqb * (p.Hq / p.gw) * p.B;
        hipLaunchKernelGGL((fa_bwd_dq_kernel<D, BF16>), dim3((unsigned)n), dim3(64 * bwd_dq_waves(D)), 0, s, p);
    }
    if (p.Sk > 0) {
        const long long n = (long long)p.nkb * p.Hkv * p.B;
        hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, BF16>), dim3((unsigned)n), dim3(64 * kBwdDkdvWaves), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int d, bool bf16, hipStream_t s) {
    if (d == 128) return bf16 ? launch_bwd_t<128, true>(p, s) : launch_bwd_t<128, false>(p, s);
    return bf16 ? launch_bwd_t<64, true>(p, s) : launch_bwd_t<64, false>(p, s);
}

}  // namespace fa
