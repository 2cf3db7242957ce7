// Host stand-ins for the kernel launchers and for the three HIP runtime calls
// the C ABI makes (hipGetDevice, hipStreamGetDevice, hipGetErrorString), so
// that the C-ABI source builds with g++ -- with or without AddressSanitizer
// and UBSan -- and runs on a machine without a GPU.  Each launcher records
// which kernel the call chose and the parameter block it was given, then
// returns the HIP status the test asked for; nothing is ever dereferenced.
// Test infrastructure: built only by the tests, never part of the library.
#include <cstdio>
#include <cstring>

#include "fa_internal.hpp"

namespace {

int g_launch_error = 0;     // status every launcher returns
int g_device_error = 0;     // status of hipGetDevice
int g_stream_device = 0;    // device hipStreamGetDevice reports
int g_scratch_error = 0;    // status of the scratch-address lookup
int g_calls = 0;
char g_kernel[16] = "";
int g_d = 0, g_bf16 = 0, g_varlen = 0;
fa::FwdParams g_fwd;
fa::Fp8Params g_fp8;
fa::DecodeParams g_dec;
fa::BwdParams g_bwd;
alignas(256) unsigned char g_scratch_stand_in[256];   // its address only is used

void record(const char* name, int d, bool bf16, bool varlen) {
    ++g_calls;
    std::snprintf(g_kernel, sizeof(g_kernel), "%s", name);
    g_d = d;
    g_bf16 = bf16 ? 1 : 0;
    g_varlen = varlen ? 1 : 0;
}

long long addr(const void* p) { return (long long)(uintptr_t)p; }

}  // namespace

namespace fa {

hipError_t launch_fwd(const FwdParams& p, int d, bool bf16, bool varlen, hipStream_t) {
    record("paired", d, bf16, varlen);
    g_fwd = p;
    return (hipError_t)g_launch_error;
}

hipError_t launch_fwd_wide(const FwdParams& p, int d, bool bf16, bool varlen, hipStream_t) {
    record("wide", d, bf16, varlen);
    g_fwd = p;
    return (hipError_t)g_launch_error;
}

hipError_t launch_fwd_fp8(const Fp8Params& p, int d, bool wide, hipStream_t) {
    record(wide ? "fp8_wide" : "fp8_paired", d, true, false);
    g_fp8 = p;
    return (hipError_t)g_launch_error;
}

hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t) {
    record(p.block_table ? "paged" : "decode", d, bf16, false);
    g_dec = p;
    return (hipError_t)g_launch_error;
}

hipError_t launch_bwd(const BwdParams& p, int d, bool bf16, hipStream_t) {
    record("bwd", d, bf16, false);
    g_bwd = p;
    return (hipError_t)g_launch_error;
}

hipError_t decode_scratch(void** ptr) {
    if (g_scratch_error) return (hipError_t)g_scratch_error;
    *ptr = g_scratch_stand_in;
    return hipSuccess;
}

}  // namespace fa

hipError_t hipGetDevice(int* device) {
    if (g_device_error) return (hipError_t)g_device_error;
    *device = 0;
    return hipSuccess;
}

hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
    *device = g_stream_device;
    return hipSuccess;
}

const char* hipGetErrorString(hipError_t e) {
    static thread_local char text[48];
    std::snprintf(text, sizeof(text), "stub HIP error %d", (int)e);
    return text;
}

extern "C" {

void fa_stub_set(int launch_error, int device_error, int stream_device, int scratch_error) {
    g_launch_error = launch_error;
    g_device_error = device_error;
    g_stream_device = stream_device;
    g_scratch_error = scratch_error;
}

void fa_stub_reset() {
    g_calls = 0;
    g_kernel[0] = '\0';
}

int fa_stub_calls() { return g_calls; }
const char* fa_stub_kernel() { return g_kernel; }
long long fa_stub_scratch_address() { return addr(g_scratch_stand_in); }

// The last forward parameter block as integers (order fixed by the tests).
void fa_stub_fwd(long long* o) {
    const fa::FwdParams& p = g_fwd;
    const long long v[] = {g_d, g_bf16, g_varlen, p.B, p.Hq, p.Hkv, p.G, p.Sq, p.Sk, p.nqt,
                           p.q_tok_stride, p.kv_tok_stride, p.lse_b_stride, p.lse_h_stride,
                           p.causal, p.wl, p.wr, (long long)p.qsign, p.xcd_groups, p.gw, p.bm,
                           p.mod, addr(p.alibi), addr(p.cu_q), addr(p.cu_k), addr(p.lse)};
    std::memcpy(o, v, sizeof(v));
}
float fa_stub_fwd_c() { return g_fwd.c; }
float fa_stub_fwd_sc_k() { return g_fwd.sc_k; }
float fa_stub_fwd_sc_c() { return g_fwd.sc_c; }

void fa_stub_fp8(long long* o) {
    const fa::Fp8Params& p = g_fp8;
    const long long v[] = {p.B, p.Hq, p.Hkv, p.G, p.Sq, p.Sk, p.sk_pad, p.nqt, p.causal, p.wl,
                           p.wr, (long long)p.qsign, p.xcd_groups, p.gw, p.bm, addr(p.vt)};
    std::memcpy(o, v, sizeof(v));
}
float fa_stub_fp8_c() { return g_fp8.c; }
float fa_stub_fp8_descale_v() { return g_fp8.descale_v; }

void fa_stub_decode(long long* o) {
    const fa::DecodeParams& p = g_dec;
    const long long v[] = {g_d, g_bf16, p.B, p.Hq, p.Hkv, p.G, p.Sk_cap, p.max_len, p.nsplit,
                           p.split, p.qblocks, p.causal, p.wl, p.wr, (long long)p.qsign,
                           p.page_size, p.max_pages, p.num_pages, p.append, addr(p.ws_o),
                           addr(p.ws_lse), addr(p.block_table), addr(p.k_new), addr(p.v_new)};
    std::memcpy(o, v, sizeof(v));
}
float fa_stub_decode_c() { return g_dec.c; }

void fa_stub_bwd(long long* o) {
    const fa::BwdParams& p = g_bwd;
    const long long v[] = {g_d, g_bf16, p.B, p.Hq, p.Hkv, p.G, p.Sq, p.Sk, p.q_tok_stride,
                           p.kv_tok_stride, p.causal, p.wl, p.wr, p.nkb, p.gw, p.nqb,
                           addr(p.dsum), addr(p.lse2)};
    std::memcpy(o, v, sizeof(v));
}
float fa_stub_bwd_scale() { return g_bwd.scale; }
float fa_stub_bwd_c2() { return g_bwd.c2; }

}  // extern "C"
