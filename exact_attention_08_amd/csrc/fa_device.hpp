// fa_device.hpp -- gfx950 device helpers shared by the attention kernels:
// vector types, the 32x32x16 MFMA wrappers, 16-bit packing and wave-level
// exchanges.  Everything here is CDNA4-only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Checking build (FA_DEBUG_SYNC, the library libfa355_debug.so): every wait
// of a copy pipeline drains all outstanding copies (FA_VMCNT(n) is 0), and
// the forward and backward kernels fill their LDS rings with NaN before the
// first copy, so that a tile read before its copy has landed, or a read of
// bytes no copy writes, shows up as NaN in the results.  (The decode split
// kernel, whose K slots are private to each wave, only drains.)  Its results
// must equal the pipelined build's bit for bit.
#ifdef FA_DEBUG_SYNC
#define FA_VMCNT(n) 0
constexpr bool kDebugSync = true;
#else
#define FA_VMCNT(n) (n)
constexpr bool kDebugSync = false;
#endif

// (checking build only) all-ones words over [p, p + bytes): NaN as bf16,
// fp16, e4m3 and fp32; then a barrier
__device__ __forceinline__ void debug_poison_lds(void* p, int bytes) {
    if constexpr (kDebugSync) {
        // (an LDS pointer: stores through a generic one could alias the
        // kernel arguments, which would then no longer be known uniform)
        __attribute__((address_space(3))) uint32_t* w =
            (__attribute__((address_space(3))) uint32_t*)(p);
        const int n = bytes / 4;
        for (int i = 0; i < n; i += blockDim.x)   // (a uniform trip count)
            if (i + (int)threadIdx.x < n) w[i + threadIdx.x] = 0xffffffffu;
        __syncthreads();
    }
}

// One v_mfma_f32_32x32x16_{bf16,f16}: C[32x32] += A[32x16] * B[16x32].
// Operand registers: lane l holds row (A) / column (B) l%32 and the 8
// reduction slots of half l/32.  Result: lane l holds column l%32, element
// 4*jj+k of the accumulator is row 8*jj + 4*(l/32) + k.
// One v_mfma_f32_16x16x32_{bf16,f16}: C[16x16] += A[16x32] * B[32x16].
// Lane l holds row (A) / column (B) l%16 and the 8 reduction slots of
// quarter l/16; result lane l holds column l%16, rows 4*(l/16) + 0..3.
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// Two fp32 -> one dword of two 16-bit values, round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950 for bf16).
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if constexpr (BF16) {
        bf16x2 r = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
        return __builtin_bit_cast(uint32_t, r);
    } else {
        f16x2 r = __builtin_convertvector((f32x2){lo, hi}, f16x2);
        return __builtin_bit_cast(uint32_t, r);
    }
}

// Build one dword from the low (SEL_HI=false) or high 16-bit halves of two
// dwords: result = {half(lo_src), half(hi_src)}.
template <bool SEL_HI>
__device__ __forceinline__ uint32_t pick_halves(uint32_t lo_src, uint32_t hi_src) {
    // v_perm_b32: byte selector over {hi_src (bytes 4-7), lo_src (bytes 0-3)}
    return __builtin_amdgcn_perm(hi_src, lo_src, SEL_HI ? 0x07060302u : 0x05040100u);
}

// The two 16-bit values of a dword as fp32 (lo, hi), on the plain VALU: a
// bf16 value is the high half of its fp32 value, so a mask and a shift give
// both exactly; fp16 values are converted.
template <bool BF16>
__device__ __forceinline__ f32x2 halves16(uint32_t packed) {
    if constexpr (BF16)
        return f32x2{__builtin_bit_cast(float, packed << 16), __builtin_bit_cast(float, packed & 0xffff0000u)};
    else
        return f32x2{(float)__builtin_bit_cast(_Float16, (uint16_t)(packed & 0xffffu)),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)(packed >> 16))};
}
// (acc + lo) + hi
template <bool BF16>
__device__ __forceinline__ float sum2_16(uint32_t packed, float acc) {
    const f32x2 h = halves16<BF16>(packed);
    return (acc + h.x) + h.y;
}
// the first pair of such a sum (weights are >= +0, so starting from a zero
// would add nothing: the same bits, one instruction less)
template <bool BF16>
__device__ __forceinline__ float sum2_16_first(uint32_t packed) {
    const f32x2 h = halves16<BF16>(packed);
    return h.x + h.y;
}

// acc + lo + hi by one v_dot2c_f32 against (1, 1).  It issues through the
// matrix pipe: where one wave per SIMD interleaves it with its own MFMAs it
// waits behind them, where several independent waves share the SIMD it is
// the cheaper form (one instruction per pair instead of four).
template <bool BF16>
__device__ __forceinline__ float sum2_16_dot(uint32_t packed, float acc) {
    if constexpr (BF16) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed),
                                               __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
    } else {
        typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, packed), __builtin_bit_cast(f16x2_t, 0x3c003c00u),
                                      acc, false);
    }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Value held by lane l ^ 32 (the other half of a 64-wide wave), via the
// gfx950 v_permlane32_swap (a VALU lane swap, no LDS round trip).  Swapping
// x with itself leaves lanes 0-31 of the first result and lanes 32-63 of the
// second result unchanged; the other halves receive the partner's value.
__device__ __forceinline__ float xor32(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const bool lower = (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & 32) == 0;
    return __builtin_bit_cast(float, lower ? r[1] : r[0]);
}

// max / sum of x over lanes l and l^32, the same value in both lanes.
// Swapping x with itself leaves one register holding the lower half's
// values in every lane and the other the upper half's (one v_permlane32_swap,
// no lane select); the operands are in the same order in every lane.  (The
// two results are copied out as scalars first: a bit_cast applied directly
// to an element of the returned pair read the wrong element.)
__device__ __forceinline__ float max_halves(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t lo = r[0], hi = r[1];
    return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}
__device__ __forceinline__ float sum_halves(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t lo = r[0], hi = r[1];
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// Mask of one 32 x 32 score accumulator as a lane holds it: element e lies
// at key offset 8 (e / 4) + e % 4 (0 .. 27) from the lane's first key, and
// offsets outside [lo, hi] become -inf.  Bit k of vis marks offset k
// visible; each element takes its bit, sign-extended to a whole-word mask
// (one bit-field extract and one bitwise select, no compares).
__device__ __forceinline__ uint32_t vis_bits(int lo, int hi) {
    lo = min(max(lo, 0), 31);
    hi = min(max(hi, -1), 30);
    return __builtin_amdgcn_ubfe(0xffffffffu, 0, max(hi + 1 - lo, 0)) << lo;
}
// all ones when bit off of vis is set, else zero
__device__ __forceinline__ uint32_t bit_mask(uint32_t vis, int off) {
    return (uint32_t)((int)(vis << (31 - off)) >> 31);
}
__device__ __forceinline__ void mask_acc32(f32x16& s, int lo, int hi) {
    const uint32_t vis = vis_bits(lo, hi);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int off = 8 * (e >> 2) + (e & 3);
        const uint32_t m = bit_mask(vis, off);
        const float x = s[e];   // (a bit_cast of the vector element itself reads element 0)
        s[e] = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & m) | (0xff800000u & ~m));
    }
}

__device__ __forceinline__ bool wave_any(bool p) {
    return __builtin_amdgcn_ballot_w64(p) != 0ull;
}

// 16-byte / 8-byte global and LDS accesses.
__device__ __forceinline__ u32x4 ld_global16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld_global8(const void* p) {
    return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ void st_global8(void* p, u32x2 v) {
    *reinterpret_cast<u32x2*>(p) = v;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for raw (stride 0) 32-bit-offset loads/stores of [base,
// base + num_bytes); out-of-range loads return zeros, stores are dropped.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int num_bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return (i32x4){(int)(uint32_t)a, (int)(uint32_t)(a >> 32), num_bytes, 0x00020000};
}

// LDS byte address of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(p);
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ...
// lds): lane i writes lds_base + 16*i, lds_base wave-uniform; out-of-range
// offsets write zeros.  Written as inline asm so that the compiler does not
// track it: the instruction has no destination registers, and the caller
// waits for it explicitly (s_waitcnt vmcnt) before reading the LDS it fills.
__device__ __forceinline__ void dma16_to_lds(i32x4 rsrc, uint32_t lds_base, int voffset,
                                             int soffset) {
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds"
        :
        : "v"(voffset), "s"(rsrc), "s"(soffset), "s"(lds_base)
        : "memory", "m0");
}

}  // namespace fa
