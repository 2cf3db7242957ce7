// fa_fwd_fp8.hip -- forward attention on 8-bit (e4m3) Q, K, V for gfx950.
//
// The "FlashAttention" explainer page names lower-precision number formats
// among the later versions' means to higher utilisation ("What it is", the
// third version) and the project summary lists FP8; neither fixes a recipe.
// This path takes Q, K, V as e4m3 codes (the OCP 8-bit format) with one fp32
// descale per tensor (real value = descale * code value), runs both products
// on v_mfma_f32_32x32x64_f8f6f4 (four times the work of the bf16 32x32x16
// instruction in twice its time), and otherwise computes what the 16-bit
// forward computes: the same tiles, masks, online softmax (lazy max in base
// 2, fp32 statistics) and LSE.  The weights P enter P.V as e4m3 values too
// (RNE; they lie in [0, 2^8] under the lazy max, inside the format's range);
// O is normalised by the fp32 sum and written as bf16.
//
// Work decomposition, rows per wave and the XCD-aware work-group order are
// those of the 16-bit kernel (one wave per SIMD, 64 query rows per wave in two
// 32-row halves, gw query heads of one K/V head per work-group).  A step
// covers 64 keys (the P.V reduction length of the instruction) as two
// 32-key sub-tiles.
//
// Operand layouts.  An f8f6f4 32x32x64 operand is 32 bytes per lane: lane l
// holds row (or column) l % 32 and 32 of the 64 reduction values, the two
// lane halves g = l / 32 the two halves.  Which byte of a lane stands for
// which reduction index is the same for A and B, so a product is correct
// whenever both operands put the same index at the same byte:
//   * S^T = K Q^T over d: lane (key or row r, g) holds d bytes
//     [64 kc + 32 g, +32) of its row, for K and Q alike;
//   * O^T += V^T P^T over keys: the accumulator of S^T gives lane (row j, g)
//     element e of sub-tile t = key 32 t + 8 (e / 4) + e % 4 + 4 g, and P is
//     packed in that order (byte 16 t + e); V^T must hold at byte p of lane
//     (column c, g) the value of that same key, so a pre-pass writes V^T
//     row-major per head with each 64-key block permuted accordingly
//     (fa_fp8_vt_kernel, into the caller's workspace).
// In LDS every operand is two contiguous 1 KB halves (bytes 0-15 of every
// lane, then bytes 16-31), filled by buffer_load_dwordx4 ... lds copies.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int V>
struct fp8_int_c {
    static constexpr int value = V;
};

template <int D>
struct Fp8Geo {
    static constexpr int HR = 32;                 // rows per half
    static constexpr int WR = 64;                 // rows per wave
    static constexpr int NW = kFwdWaves;          // waves per work-group
    static constexpr int BN = 64;                 // keys per step
    static constexpr int KC = D / 64;             // reduction chunks of S over d
    static constexpr int DB = D / 32;             // O^T accumulators per half
    static constexpr int KBLK = 2 * KC * 2;       // 1 KB blocks of a K tile (sub-tile, kc, half)
    static constexpr int VBLK = DB * 2;           // 1 KB blocks of a V^T tile (db, half)
    static constexpr int TILE = (KBLK + VBLK) * 1024;   // bytes per stage (K then V^T)
    static constexpr int STAGES = 6;
    static constexpr int LPS = (KBLK + VBLK) / NW;      // copies per wave per stage
    static_assert((KBLK + VBLK) % NW == 0, "blocks split evenly over the waves");
};

constexpr float kFp8RescaleThreshold = 8.0f;   // log2 units

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
    // format 0 = e4m3 for both operands, no block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ i32x8 acc_regs8(i32x8 v) {
    i32x8 r;
    asm("" : "=a"(r) : "0"(v));
    return r;
}

// a buffer resource built from wave-uniform values, placed in scalar
// registers (the copy instruction takes it from there)
__device__ __forceinline__ i32x4 scalar_rsrc(i32x4 r) {
    return (i32x4){__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                   __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w)};
}

// ---------------------------------------------------------------------------
// V^T pre-pass: one work-group per (64-key block, K/V head, sequence).
// vt[((b * Hkv + h) * D + c) * sk_pad + 64 blk + 32 g + 16 t + e] =
//     v[b][64 blk + 32 t + 8 (e / 4) + e % 4 + 4 g][h][c]   (0 past Sk).
template <int D>
__global__ __launch_bounds__(256) void fa_fp8_vt_kernel(Fp8Params p) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[64 * D];
    const int nblk = p.sk_pad / 64;
    int i = blockIdx.x;
    const int blk = i % nblk; i /= nblk;
    const int h = i % p.Hkv;
    const int b = i / p.Hkv;
    const int k0 = blk * 64;
    // load 64 key rows of this head (16 bytes per thread per round)
    const uint8_t* vbase = (const uint8_t*)p.v + ((long long)b * p.Sk * p.Hkv + h) * D;
    for (int u = threadIdx.x; u < 64 * D / 16; u += 256) {
        const int key = u / (D / 16), ch = u % (D / 16);
        u32x4 x = {0u, 0u, 0u, 0u};
        if (k0 + key < p.Sk)
            x = *reinterpret_cast<const u32x4*>(vbase + (long long)(k0 + key) * p.Hkv * D + ch * 16);
        *reinterpret_cast<u32x4*>(tile + key * D + ch * 16) = x;
    }
    __syncthreads();
    // write D rows x 64 permuted bytes (16 bytes per thread per round)
    uint8_t* vt = (uint8_t*)p.vt + ((long long)b * p.Hkv + h) * D * p.sk_pad + k0;
    for (int u = threadIdx.x; u < D * 4; u += 256) {
        const int c = u / 4, q = u % 4;            // bytes 16q .. 16q+15 of row c
        const int g = q / 2, t = q % 2;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t x = 0;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int e = 4 * j + bb;
                const int key = 32 * t + 8 * (e >> 2) + (e & 3) + 4 * g;
                x |= (uint32_t)tile[key * D + c] << (8 * bb);
            }
            w[j] = x;
        }
        *reinterpret_cast<u32x4*>(vt + (long long)c * p.sk_pad + 16 * q) = (u32x4){w[0], w[1], w[2], w[3]};
    }
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_fwd_fp8_kernel(Fp8Params p) {
    using T = Fp8Geo<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[T::STAGES * T::TILE];
    debug_poison_lds(ring, (int)sizeof(ring));

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 31;
    const int g = lane >> 5;
    __builtin_assume(wave >= 0 && wave < T::NW);

    // ---- work-group -> (query tile, head group, sequence), as the 16-bit kernel
    const int gw = p.gw, gpk = p.G / gw;
    int t, hg, b;
    {
        const int i = blockIdx.x;
        if (p.xcd_groups > 0) {
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
    const int sq = p.Sq, sk = p.Sk, delta = sk - sq;
    const int q0 = t * p.bm;
    if (q0 >= sq) return;
    const int causal = p.causal, wl = p.wl, wr = p.wr;
    auto lo_of = [&](int i) __attribute__((always_inline)) { return wl >= 0 ? max(0, i + delta - wl) : 0; };
    auto hi_of = [&](int i) __attribute__((always_inline)) {
        int h = sk - 1;
        if (causal) h = min(h, i + delta);
        if (wr >= 0) h = min(h, i + delta + wr);
        return h;
    };

    // ---- tile ranges (64-key tiles) ---------------------------------------
    const int wg_last = min(q0 + p.bm, sq) - 1;
    const int kv_lo = lo_of(q0), kv_hi = hi_of(wg_last);
    const int tile_lo = kv_lo / T::BN;
    const int ntiles = kv_hi >= kv_lo ? kv_hi / T::BN - tile_lo + 1 : 0;
    const int tile_last = tile_lo + ntiles - 1;
    int r0[2], in_lo[2], in_hi[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        r0[h] = q0 + T::WR * (wave / gw) + T::HR * h;
        const int r1 = min(r0[h] + T::HR - 1, sq - 1);
        const int int_lo = lo_of(r1), int_hi = hi_of(r0[h]);
        in_lo[h] = (int_lo + T::BN - 1) / T::BN;
        in_hi[h] = int_hi + 1 >= T::BN ? (int_hi + 1) / T::BN - 1 : -1;
        if (r0[h] >= sq) { in_lo[h] = 1; in_hi[h] = 0; }   // no rows: every tile masked
    }
    // this lane's visible key interval, relative to its key offset 4g
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

    // ---- copies HBM/L2 -> LDS ring ----------------------------------------
    // K block kb = (st * KC + kc) * 2 + hh: lane L: key 32 st + L % 32, d
    // bytes 64 kc + 32 (L / 32) + 16 hh.  V^T block vb = db * 2 + hh: lane L:
    // row c = 32 db + L % 32, bytes 32 (L / 32) + 16 hh of the tile's 64.
    const int tok_q = (int)p.q_tok_stride, tok_kv = (int)p.kv_tok_stride;
    const uint8_t* kseq = (const uint8_t*)p.k + ((long long)b * sk * p.Hkv + hkv) * D;
    const uint8_t* vtrow = (const uint8_t*)p.vt + ((long long)b * p.Hkv + hkv) * D * p.sk_pad;
    int dma_voff[T::LPS];
    uint32_t dma_loff[T::LPS];
    bool dma_isk[T::LPS];
#pragma unroll
    for (int i = 0; i < T::LPS; ++i) {
        const int blk = wave + i * T::NW;
        dma_isk[i] = blk < T::KBLK;
        dma_loff[i] = blk * 1024;
        if (dma_isk[i]) {
            const int hh = blk & 1, kc = (blk >> 1) % T::KC, st = (blk >> 1) / T::KC;
            dma_voff[i] = (32 * st + (lane & 31)) * tok_kv + 64 * kc + 32 * (lane >> 5) + 16 * hh;
        } else {
            const int vb = blk - T::KBLK, hh = vb & 1, db = vb >> 1;
            dma_voff[i] = (32 * db + (lane & 31)) * p.sk_pad + 32 * (lane >> 5) + 16 * hh;
        }
    }
    auto slot = [&](int jt) __attribute__((always_inline)) {
        return ring + ((jt - tile_lo) % T::STAGES) * T::TILE;
    };
    // tiles outside [tile_lo, tile_last] get zero records (zeros, no memory access)
    struct SetCopy {
        i32x4 krs, vrs;
        uint32_t dst;
    };
    auto set_copy = [&](int jt) __attribute__((always_inline)) {
        const bool valid = jt >= tile_lo && jt <= tile_last;
        const int rows = valid ? min(sk - jt * T::BN, T::BN) : 0;
        const i32x4 krs = make_rsrc(kseq + (long long)jt * T::BN * tok_kv, rows * tok_kv);
        // V^T rows are sk_pad long; a tile is 64 bytes of each of D rows
        const i32x4 vrs = make_rsrc(vtrow + (long long)jt * T::BN,
                                    valid ? (D - 1) * p.sk_pad + T::BN : 0);
        return SetCopy{krs, vrs, (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(slot(jt)))};
    };
    auto copy_one = [&](const SetCopy& sc, int i) __attribute__((always_inline)) {
        dma16_to_lds(scalar_rsrc(dma_isk[i] ? sc.krs : sc.vrs), sc.dst + dma_loff[i], dma_voff[i], 0);
    };
    auto issue = [&](int jt) __attribute__((always_inline)) {
        const SetCopy sc = set_copy(jt);
#pragma unroll
        for (int i = 0; i < T::LPS; ++i) copy_one(sc, i);
    };
    // At the top of step jt this wave's copies of tiles jt and jt + 1 have
    // landed (those of jt + 2 .. jt + STAGES - 3 may fly); the barrier then
    // makes every wave's copies visible and frees the slot of jt - 2.
    auto sync_step = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(FA_VMCNT(T::LPS * (T::STAGES - 4))) : "memory");
    };

    auto ld_op = [&](const uint8_t* base) __attribute__((always_inline)) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + lane * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + 1024 + lane * 16);
        return (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    // K operand (sub-tile st, chunk kc) and V^T operand (d block db) of a tile
    auto k_op = [&](const uint8_t* tl, int st, int kc) __attribute__((always_inline)) {
        return ld_op(tl + ((st * T::KC + kc) * 2) * 1024);
    };
    auto v_op = [&](const uint8_t* tl, int db) __attribute__((always_inline)) {
        return ld_op(tl + (T::KBLK + 2 * db) * 1024);
    };

    f32x16 oacc[2][T::DB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[h][db][e] = 0.f;
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    const float c = p.c;

    i32x8 qop[2][T::KC];               // Q of each half as B operands
    f32x16 sacc[2][2];                 // [half][sub-tile] S^T
    int stile[2] = {0, 0};             // tile of each half's S
    i32x8 pb[2];                       // P of each half (e4m3)
    i32x8 kbuf[2][T::KC], vbuf[T::DB]; // K operands of the next S, V^T of the previous tile

    auto interior = [&](int h, int jt) __attribute__((always_inline)) {
        return jt >= in_lo[h] && jt <= in_hi[h];
    };
    auto apply_mask = [&](int h) __attribute__((always_inline)) {
        const int base = stile[h] * T::BN;
#pragma unroll
        for (int st = 0; st < 2; ++st)
            mask_acc32(sacc[h][st], rel_lo[h] - base - 32 * st, rel_hi[h] - base - 32 * st);
    };
    // exps of half h with max m: packs P and returns this lane's fp32 sum
    auto exps = [&](int h, float m_use) __attribute__((always_inline)) {
        float x[2][16];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 16; ++e) x[st][e] = exp2_fast(fmaf(sacc[h][st][e], c, -m_use));
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int st = w >> 2, e = 4 * (w & 3);
            pb[h][w] = (int)pack4_fp8(x[st][e], x[st][e + 1], x[st][e + 2], x[st][e + 3]);
        }
        float s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s4[j] = (x[0][4 * j] + x[0][4 * j + 1]) + (x[0][4 * j + 2] + x[0][4 * j + 3]) +
                    ((x[1][4 * j] + x[1][4 * j + 1]) + (x[1][4 * j + 2] + x[1][4 * j + 3]));
        return (s4[0] + s4[1]) + (s4[2] + s4[3]);
    };
    // weights of half h's newest S: lazy max as in the 16-bit kernel (redo
    // with the true max when some lane's sum exceeds 2^8 or a row has no max)
    auto softmax_half = [&](int h) __attribute__((always_inline)) {
        const bool first = m_run[h] == -INFINITY;
        float sum = exps(h, first ? 0.f : m_run[h]);
        if ((__builtin_amdgcn_ballot_w64(first) | __builtin_amdgcn_ballot_w64(sum > 256.f)) != 0ull) {
            asm volatile("");
            float mx = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[h][st][e]);
            mx = max_halves(mx);
            const float mnew = fmaxf(m_run[h], mx * c);
            const bool raise = mnew > m_run[h] + kFp8RescaleThreshold;
            const float alpha = raise ? exp2_fast(m_run[h] - mnew) : 1.f;
            l_run[h] *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[h][db][e] *= alpha;
            m_run[h] = raise ? mnew : m_run[h];
            sum = exps(h, m_run[h] == -INFINITY ? 0.f : m_run[h]);
        }
        l_run[h] += sum;
    };

    // One region of a step: the S MFMAs of half hs on the new tile, the P.V
    // MFMAs of half hs on the previous tile, and the weights of the other
    // half's newest S (masked first when its tile needs masks).
    // (The step after the last tile computes no S and, in its second
    // region, no weights.)
    auto region = [&](int hs, int jt, bool masked_other, bool with_s, bool with_p)
        __attribute__((always_inline)) {
        const int hp = 1 - hs;
        if (with_s) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[hs][st][e] = 0.f;
#pragma unroll
                for (int kc = 0; kc < T::KC; ++kc)
                    sacc[hs][st] = mfma_f8(kbuf[st][kc], qop[hs][kc], sacc[hs][st]);
            }
        }
#pragma unroll
        for (int db = 0; db < T::DB; ++db) oacc[hs][db] = mfma_f8(vbuf[db], pb[hs], oacc[hs][db]);
        if (with_p) {
            if (masked_other) apply_mask(hp);
            softmax_half(hp);
        }
        stile[hs] = jt;
    };

    // The same region with one matrix instruction per slot and, beside each,
    // an equal share of the other half's exponentials with their packing
    // and sums (a slot never waits for its own results); hook(i) adds the
    // slot's operand loads or copies.  sched_barrier(0) keeps the order:
    // with one wave per SIMD the matrix and vector pipes only overlap as
    // far as the instruction stream alternates them.
    auto fast_region = [&](auto hsc, int jt, bool masked_other, auto&& hook)
        __attribute__((always_inline)) {
        constexpr int hs = decltype(hsc)::value, hp = 1 - hs;
        constexpr int NS = 2 * T::KC + T::DB;         // matrix slots
        constexpr int EPS = 32 / NS;                  // weights per slot
        static_assert(EPS * NS == 32 && EPS % 4 == 0, "whole packed words per slot");
        if (masked_other) apply_mask(hp);
        const bool first = m_run[hp] == -INFINITY;
        const float m_use = first ? 0.f : m_run[hp];
        float part[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i < 2 * T::KC) {
                const int st = i / T::KC, kc = i % T::KC;
                sacc[hs][st] = mfma_f8(kbuf[st][kc], qop[hs][kc], kc == 0 ? f32x16{} : sacc[hs][st]);
            } else {
                const int db = i - 2 * T::KC;
                oacc[hs][db] = mfma_f8(vbuf[db], pb[hs], oacc[hs][db]);
            }
            hook(i);
            float x[EPS];
#pragma unroll
            for (int j = 0; j < EPS; ++j) {
                const int el = i * EPS + j;
                x[j] = exp2_fast(fmaf(sacc[hp][el >> 4][el & 15], c, -m_use));
            }
#pragma unroll
            for (int w = 0; w < EPS / 4; ++w)
                pb[hp][i * (EPS / 4) + w] = (int)pack4_fp8(x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3]);
            float t2[EPS / 2];
#pragma unroll
            for (int j = 0; j < EPS / 2; ++j) t2[j] = x[2 * j] + x[2 * j + 1];
#pragma unroll
            for (int wdt = EPS / 4; wdt >= 1; wdt >>= 1)
#pragma unroll
                for (int j = 0; j < wdt; ++j) t2[j] += t2[j + wdt];
            part[i] = t2[0];
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int wdt = NS / 2; wdt >= 1; wdt >>= 1)
#pragma unroll
            for (int j = 0; j < wdt; ++j) part[j] += part[j + wdt];
        float sum = part[0];
        if ((__builtin_amdgcn_ballot_w64(first) | __builtin_amdgcn_ballot_w64(sum > 256.f)) != 0ull) {
            asm volatile("");
            float mx = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[hp][st][e]);
            mx = max_halves(mx);
            const float mnew = fmaxf(m_run[hp], mx * c);
            const bool raise = mnew > m_run[hp] + kFp8RescaleThreshold;
            const float alpha = raise ? exp2_fast(m_run[hp] - mnew) : 1.f;
            l_run[hp] *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[hp][db][e] *= alpha;
            m_run[hp] = raise ? mnew : m_run[hp];
            sum = exps(hp, m_run[hp] == -INFINITY ? 0.f : m_run[hp]);
        }
        l_run[hp] += sum;
        stile[hs] = jt;
    };

    // first step: no previous tile (P = 0, V = 0), no S of half B yet
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[1][st][e] = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 8; ++w) pb[h][w] = 0;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int w = 0; w < 8; ++w) vbuf[db][w] = 0;

    // The first copies go out before the Q loads so that the two latencies
    // overlap (the Q operands are waited for where they are placed).
    if (ntiles > 0)
        for (int s = tile_lo; s < tile_lo + T::STAGES - 2; ++s) issue(s);
    // ---- Q as B operands --------------------------------------------------
    {
        const auto qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const uint8_t*)p.q + ((long long)b * sq * p.Hq + hq) * D), (short)0, sq * tok_q,
            0x00020000);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kc = 0; kc < T::KC; ++kc) {
                const int off = (r0[h] + lq) * tok_q + 64 * kc + 32 * g;
                const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0) ^ p.qsign;
                const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 16, 0, 0) ^ p.qsign;
                qop[h][kc] = acc_regs8((i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w});
            }
    }

    if (ntiles > 0) {
        // tiles tile_lo .. +STAGES-3 in flight; the first step needs the
        // first two landed (K of the first now, K of the second at its end)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(FA_VMCNT(T::LPS * (T::STAGES - 4))) : "memory");
        {
            const uint8_t* tl = slot(tile_lo);
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int kc = 0; kc < T::KC; ++kc) kbuf[st][kc] = acc_regs8(k_op(tl, st, kc));
        }
        // step jt: S(jt) and P.V of jt - 1; the step after the last tile
        // only finishes the previous one
        for (int jt = tile_lo; jt <= tile_last; ++jt) {
            if (jt > tile_lo) sync_step();
            // the other half's newest S: half B of jt - 1 (region 0), half A
            // of jt (region 1)
            const bool mB = !interior(1, jt - 1), mA = !interior(0, jt);
            // region 0 spreads this step's copies over its slots; region 1
            // reloads each operand register right after its last use: K of
            // jt + 1 and V^T of jt for the next step
            const SetCopy sc = set_copy(jt + T::STAGES - 2);
            fast_region(fp8_int_c<0>{}, jt, mB, [&](int i) __attribute__((always_inline)) {
                if (i < T::LPS) copy_one(sc, i);
            });
            const uint8_t* tn = slot(jt + 1);
            const uint8_t* tc = slot(jt);
            fast_region(fp8_int_c<1>{}, jt, mA, [&](int i) __attribute__((always_inline)) {
                if (i < 2 * T::KC) kbuf[i / T::KC][i % T::KC] = acc_regs8(k_op(tn, i / T::KC, i % T::KC));
                else vbuf[i - 2 * T::KC] = acc_regs8(v_op(tc, i - 2 * T::KC));
            });
        }
        // the step after the last tile: P.V of the last tile only (its
        // operands are in registers; no LDS access, no copies)
        region(0, tile_last + 1, !interior(1, tile_last), false, true);
        region(1, tile_last + 1, false, false, false);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: O / l * descale_v -> bf16, LSE ------------------------
    const auto ors = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((char*)p.o + ((long long)b * sq * p.Hq + hq) * D * 2), (short)0, sq * p.Hq * D * 2,
        0x00020000);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float l_tot = sum_halves(l_run[h]);
        const float inv = l_tot > 0.f ? p.descale_v / l_tot : 0.f;
        const int row = r0[h] + lq;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                u32x2 w;
                w.x = pack2<true>(oacc[h][db][4 * jj] * inv, oacc[h][db][4 * jj + 1] * inv);
                w.y = pack2<true>(oacc[h][db][4 * jj + 2] * inv, oacc[h][db][4 * jj + 3] * inv);
                const int col = 32 * db + 8 * jj + 4 * g;
                __builtin_amdgcn_raw_buffer_store_b64(w, ors, (row * p.Hq * D + col) * 2, 0, 0);
            }
        if (p.lse != nullptr && g == 0 && row < sq)
            p.lse[((long long)b * p.Hq + hq) * sq + row] =
                l_tot > 0.f ? (m_run[h] + log2_fast(l_tot)) * kLn2 : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Paired form of the 8-bit forward, for rows that see up to kFwdWideMinKeys
// keys on average (the rule of the 16-bit forward): 32 query rows per wave
// and three work-groups per CU, whose waves share each SIMD, as in the
// 16-bit paired kernel.  One wave per SIMD (the kernel above) issues its
// vector work from one instruction stream, and the weights' vector work
// (scale, exponential, e4m3 packing, sum) outweighs the 8-bit MFMAs beside
// it; three independent waves per SIMD issue it side by side.  Operand
// layouts, copies, masks, lazy max and epilogue are those of the kernel
// above; the ring has three stages of one 64-key tile (K, then V^T), copies
// go out two tiles ahead, and a window's tiles are taken in the rotated
// order of the 16-bit paired kernel.
template <int D>
struct Fp8PairGeo {
    static constexpr int R = 32;                  // rows per wave
    static constexpr int NW = kFwdWaves;          // waves per work-group
    static constexpr int BN = 64;                 // keys per step (two 32-key sub-tiles)
    static constexpr int KC = D / 64;             // reduction chunks of S over d
    static constexpr int DB = D / 32;             // O^T accumulators
    static constexpr int KBLK = 2 * KC * 2;       // 1 KB blocks of a K tile (sub-tile, kc, half)
    static constexpr int VBLK = DB * 2;           // 1 KB blocks of a V^T tile (db, half)
    static constexpr int TILE = (KBLK + VBLK) * 1024;
    static constexpr int STAGES = 3;
    static constexpr int AHEAD = 2;
    static constexpr int LPS = (KBLK + VBLK) / NW;
    static_assert((KBLK + VBLK) % NW == 0, "blocks split evenly over the waves");
    static_assert(AHEAD == STAGES - 1, "a slot is refilled one step after its tile is used");
};

template <int D>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void fa_fwd_fp8_paired_kernel(Fp8Params p) {
    using T = Fp8PairGeo<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[T::STAGES * T::TILE];
    debug_poison_lds(ring, (int)sizeof(ring));

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 31;
    const int g = lane >> 5;
    __builtin_assume(wave >= 0 && wave < T::NW);

    // ---- work-group -> (query tile, head group, sequence), heaviest first
    const int gw = p.gw, gpk = p.G / gw;
    int t, hg, b;
    {
        const int i = blockIdx.x;
        if (p.xcd_groups > 0) {
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
    const int sq = p.Sq, sk = p.Sk, delta = sk - sq;
    const int q0 = t * p.bm;
    if (q0 >= sq) return;                      // uniform over the work-group
    const int causal = p.causal, wl = p.wl, wr = p.wr;
    auto lo_of = [&](int i) __attribute__((always_inline)) { return wl >= 0 ? max(0, i + delta - wl) : 0; };
    auto hi_of = [&](int i) __attribute__((always_inline)) {
        int h = sk - 1;
        if (causal) h = min(h, i + delta);
        if (wr >= 0) h = min(h, i + delta + wr);
        return h;
    };

    // ---- tile ranges (64-key tiles): the work-group walks [tile_lo,
    // tile_last], this wave computes [w_lo, w_hi] and needs no mask on
    // [in_lo, in_hi]
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
    // this lane's visible key interval, relative to its key offset 4g
    int rel_lo, rel_hi;
    {
        const int pos = r0 + lq + delta;
        rel_lo = (wl >= 0 ? pos - wl : -0x40000000) - 4 * g;
        int hh = sk - 1;
        if (causal) hh = min(hh, pos);
        if (wr >= 0) hh = min(hh, pos + wr);
        rel_hi = hh - 4 * g;
    }

    // ---- copies HBM/L2 -> LDS ring (block layout of the kernel above) -----
    // except K at d = 128 (KROW): row-major, each copy 8 whole 128-byte rows
    // (lane L: key 8*blk + L/8, its 16-byte chunk (L%8) ^ ((key/2)%8)), so
    // chunk c of key r sits at r*128 + 16*(c ^ ((r/2)%8)); the operand reads
    // below (16 lanes = 16 keys, one chunk) then cover 16 distinct bank
    // groups.  The operand-order copy read 32 bytes from each of 32 rows.
    constexpr bool KROW = D == 128;
    const int tok_q = (int)p.q_tok_stride, tok_kv = (int)p.kv_tok_stride;
    const uint8_t* kseq = (const uint8_t*)p.k + ((long long)b * sk * p.Hkv + hkv) * D;
    const uint8_t* vtrow = (const uint8_t*)p.vt + ((long long)b * p.Hkv + hkv) * D * p.sk_pad;
    int dma_voff[T::LPS];
    uint32_t dma_loff[T::LPS];
    bool dma_isk[T::LPS];
#pragma unroll
    for (int i = 0; i < T::LPS; ++i) {
        const int blk = wave + i * T::NW;
        dma_isk[i] = blk < T::KBLK;
        dma_loff[i] = blk * 1024;
        if (dma_isk[i] && KROW) {
            const int row = 8 * blk + (lane >> 3);
            dma_voff[i] = row * tok_kv + (((lane & 7) ^ ((row >> 1) & 7)) * 16);
        } else if (dma_isk[i]) {
            const int hh = blk & 1, kc = (blk >> 1) % T::KC, st = (blk >> 1) / T::KC;
            dma_voff[i] = (32 * st + (lane & 31)) * tok_kv + 64 * kc + 32 * (lane >> 5) + 16 * hh;
        } else {
            const int vb = blk - T::KBLK, hh = vb & 1, db = vb >> 1;
            dma_voff[i] = (32 * db + (lane & 31)) * p.sk_pad + 32 * (lane >> 5) + 16 * hh;
        }
    }
    auto slot = [&](int i) __attribute__((always_inline)) { return ring + i * T::TILE; };
    auto next_slot = [&](int i) __attribute__((always_inline)) {
        return i == T::STAGES - 1 ? 0 : i + 1;
    };
    // this wave's copies of tile jt into ring slot i; tiles outside
    // [tile_lo, tile_last] get zero records (zeros, no memory access)
    auto issue = [&](int jt, int i) __attribute__((always_inline)) {
        const bool valid = jt >= tile_lo && jt <= tile_last;
        const int rows = valid ? min(sk - jt * T::BN, T::BN) : 0;
        const i32x4 krs = scalar_rsrc(make_rsrc(kseq + (long long)(valid ? jt : 0) * T::BN * tok_kv,
                                                rows * tok_kv));
        const i32x4 vrs = scalar_rsrc(make_rsrc(vtrow + (long long)(valid ? jt : 0) * T::BN,
                                                valid ? (D - 1) * p.sk_pad + T::BN : 0));
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(slot(i)));
#pragma unroll
        for (int l = 0; l < T::LPS; ++l)
            dma16_to_lds(dma_isk[l] ? krs : vrs, dst + dma_loff[l], dma_voff[l], 0);
    };
    // End of step s: this wave's copies of the tiles of every step up to
    // s + 1 have landed (step s + 2's may still be in flight), its LDS reads
    // have returned; the barrier makes both true for all waves.
    auto sync_step = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier"
                     ::"n"(FA_VMCNT(T::LPS * (T::AHEAD - 1))) : "memory");
    };
    auto ld_op = [&](const uint8_t* base) __attribute__((always_inline)) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + lane * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + 1024 + lane * 16);
        return (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    // ---- the wave's 32 query rows as B operands ---------------------------
    i32x8 qop[T::KC];
    {
        const auto qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const uint8_t*)p.q + ((long long)b * sq * p.Hq + hq) * D), (short)0, sq * tok_q,
            0x00020000);
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc) {
            const int off = (r0 + lq) * tok_q + 64 * kc + 32 * g;
            const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0) ^ p.qsign;
            const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 16, 0, 0) ^ p.qsign;
            qop[kc] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                              (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    }

    f32x16 oacc[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c = p.c;
    i32x8 pb;

    // weights of a tile (lazy max as in the kernel above): packs P, returns
    // this lane's fp32 sum
    auto exps = [&](const f32x16 (&sacc)[2], float m_use) __attribute__((always_inline)) {
        float x[2][16];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 16; ++e) x[st][e] = exp2_fast(fmaf(sacc[st][e], c, -m_use));
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int st = w >> 2, e = 4 * (w & 3);
            pb[w] = (int)pack4_fp8(x[st][e], x[st][e + 1], x[st][e + 2], x[st][e + 3]);
        }
        float s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s4[j] = (x[0][4 * j] + x[0][4 * j + 1]) + (x[0][4 * j + 2] + x[0][4 * j + 3]) +
                    ((x[1][4 * j] + x[1][4 * j + 1]) + (x[1][4 * j + 2] + x[1][4 * j + 3]));
        return (s4[0] + s4[1]) + (s4[2] + s4[3]);
    };
    auto softmax_tile = [&](const f32x16 (&sacc)[2]) __attribute__((always_inline)) {
        const bool first = m_run == -INFINITY;
        float sum = exps(sacc, first ? 0.f : m_run);
        if ((__builtin_amdgcn_ballot_w64(first) | __builtin_amdgcn_ballot_w64(sum > 256.f)) != 0ull) {
            asm volatile("");   // keep this rare block a real branch (not speculated)
            float mx = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[st][e]);
            mx = max_halves(mx);
            const float mnew = fmaxf(m_run, mx * c);
            const bool raise = mnew > m_run + kFp8RescaleThreshold;
            const float alpha = raise ? exp2_fast(m_run - mnew) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            m_run = raise ? mnew : m_run;
            sum = exps(sacc, m_run == -INFINITY ? 0.f : m_run);
        }
        l_run += sum;
    };

    // Step on tile jt (in ring slot i): this wave's copies of tile jt_ahead,
    // then, for the tiles of this wave, S^T of both sub-tiles, the mask
    // (boundary tiles only), the weights and O^T += V^T P^T.
    auto step = [&](int jt, int jt_ahead, int i) __attribute__((always_inline)) {
        issue(jt_ahead, i == 0 ? T::STAGES - 1 : i - 1);
        if (jt >= w_lo && jt <= w_hi) {                // uniform per wave
            const uint8_t* tl = slot(i);
            f32x16 sacc[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[st][e] = 0.f;
#pragma unroll
                for (int kc = 0; kc < T::KC; ++kc) {
                    i32x8 a;
                    if constexpr (KROW) {
                        // key 32st + l%32, bytes 64kc + 32(l/32) .. +31 of it
                        const uint8_t* kr = tl + (32 * st + (lane & 31)) * D;
                        const int c = 4 * kc + 2 * (lane >> 5), sw = (lane >> 1) & 7;
                        const u32x4 lo = *reinterpret_cast<const u32x4*>(kr + (c ^ sw) * 16);
                        const u32x4 hi = *reinterpret_cast<const u32x4*>(kr + ((c + 1) ^ sw) * 16);
                        a = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    } else {
                        a = ld_op(tl + ((st * T::KC + kc) * 2) * 1024);
                    }
                    sacc[st] = mfma_f8(a, qop[kc], sacc[st]);
                }
            }
            if (jt < in_lo || jt > in_hi) {
#pragma unroll
                for (int st = 0; st < 2; ++st)
                    mask_acc32(sacc[st], rel_lo - jt * T::BN - 32 * st, rel_hi - jt * T::BN - 32 * st);
            }
            softmax_tile(sacc);
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
                oacc[db] = mfma_f8(ld_op(tl + (T::KBLK + 2 * db) * 1024), pb, oacc[db]);
        }
        sync_step();
        return next_slot(i);
    };
    if (ntiles > 0) {
        // step s takes the tile congruent to s modulo the range length, as
        // the 16-bit paired kernel (causal: tile s; a window: rotated)
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
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // copies of unused tiles still in flight

    // ---- epilogue: O / l * descale_v -> bf16, LSE ------------------------
    const auto ors = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((char*)p.o + ((long long)b * sq * p.Hq + hq) * D * 2), (short)0, sq * p.Hq * D * 2,
        0x00020000);
    const float l_tot = sum_halves(l_run);
    const float inv = l_tot > 0.f ? p.descale_v / l_tot : 0.f;
    const int row = r0 + lq;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            u32x2 w;
            w.x = pack2<true>(oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv);
            w.y = pack2<true>(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
            const int col = 32 * db + 8 * jj + 4 * g;
            __builtin_amdgcn_raw_buffer_store_b64(w, ors, (row * p.Hq * D + col) * 2, 0, 0);
        }
    if (p.lse != nullptr && g == 0 && row < sq)
        p.lse[((long long)b * p.Hq + hq) * sq + row] =
            l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
}

template <int D>
static hipError_t launch_fp8_t(const Fp8Params& p, bool wide, hipStream_t s) {
    const long long nvt = (long long)(p.sk_pad / 64) * p.Hkv * p.B;
    if (nvt > 0) hipLaunchKernelGGL((fa_fp8_vt_kernel<D>), dim3((unsigned)nvt), dim3(256), 0, s, p);
    const long long nblocks = (long long)p.nqt * (p.Hq / p.gw) * p.B;
    if (nblocks > 0) {
        if (wide)
            hipLaunchKernelGGL((fa_fwd_fp8_kernel<D>), dim3((unsigned)nblocks), dim3(kFwdThreads), 0, s, p);
        else
            hipLaunchKernelGGL((fa_fwd_fp8_paired_kernel<D>), dim3((unsigned)nblocks), dim3(kFwdThreads),
                               0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8Params& p, int d, bool wide, hipStream_t s) {
    return d == 128 ? launch_fp8_t<128>(p, wide, s) : launch_fp8_t<64>(p, wide, s);
}

}  // namespace fa
