// mx4_device.h -- device-side building blocks shared by the MXFP4 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx4_layout.h"

namespace mx4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// MXFP4 group scale (rule of the kernelindex.com amd-mxfp4-mm pages,
// submission 755056, section "Software MXFP4 quant"): the group amax is
// rounded to a power of two R by adding 0x00200000 to its fp32 bits and
// clearing the significand; s = clamp(E(R) - 129, -127, 127), byte = s + 127.
// `amax_bits16` is the largest |x| of the group as a bf16 bit pattern (an
// integer max of the sign-cleared patterns is the float max for finite x).
__device__ __forceinline__ uint32_t scale_byte_from_amax16(uint32_t amax_bits16) {
    uint32_t r = ((amax_bits16 << 16) + 0x00200000u) & 0xFF800000u;
    int e = (int)(r >> 23);
    int byte = e - 2;                 // (e - 129) + 127
    byte = byte < 0 ? 0 : byte;       // s clamped at -127
    byte = byte > 254 ? 254 : byte;   // s clamped at +127
    return (uint32_t)byte;
}

// 2^s as the fp32 scale operand of the gfx950 fp4 convert, which computes
// e2m1(x / scale) with round-to-nearest-even and saturation at 6; byte 0
// (s = -127) is the denormal 2^-127.
__device__ __forceinline__ float scale_operand(uint32_t byte) {
    uint32_t bits = byte ? (byte << 23) : 0x00400000u;
    return __uint_as_float(bits);
}

// Largest sign-cleared bf16 pattern among 32 bf16 held in 16 dwords.
__device__ __forceinline__ uint32_t amax16_of_32(const uint32_t (&w)[16]) {
    u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 16; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    return m.x > m.y ? m.x : m.y;
}

// Convert 8 bf16 (4 dwords) to 8 e2m1 codes (one dword, element 0 in the low
// nibble) under scale operand `sc`.
__device__ __forceinline__ uint32_t cvt8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, float sc) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w0), sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w1), sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w2), sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w3), sc, 3);
    return r;
}

// Quantise one whole 32-element group held by one lane (64 bytes of bf16 as
// four 16-byte vectors) into 16 bytes of codes; returns the scale byte.
__device__ __forceinline__ uint32_t quant_group32(const u32x4 (&x)[4], u32x4& codes) {
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[4 * i + 0] = x[i].x;
        w[4 * i + 1] = x[i].y;
        w[4 * i + 2] = x[i].z;
        w[4 * i + 3] = x[i].w;
    }
    uint32_t byte = scale_byte_from_amax16(amax16_of_32(w));
    float sc = scale_operand(byte);
    codes.x = cvt8(w[0], w[1], w[2], w[3], sc);
    codes.y = cvt8(w[4], w[5], w[6], w[7], sc);
    codes.z = cvt8(w[8], w[9], w[10], w[11], sc);
    codes.w = cvt8(w[12], w[13], w[14], w[15], sc);
    return byte;
}

// One lane per 8 consecutive bf16 (one 16-byte vector); the four lanes of a
// DPP quad hold one 32-element group and reduce its amax across the quad with
// two lane swaps.  Returns the lane's 8 codes as one dword and the group's
// scale byte.  Every lane of the quad must be active.
__device__ __forceinline__ uint32_t quad_quant8(const u32x4& v, uint32_t& byte) {
    u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
    a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu));
    a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu));
    a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu));
    uint32_t m = a.x > a.y ? a.x : a.y;
    // quad_perm [1,0,3,2] then [2,3,0,1]: max over the four lanes of the quad
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);
    m = m > o ? m : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false);
    m = m > o ? m : o;
    byte = scale_byte_from_amax16(m);
    return cvt8(v.x, v.y, v.z, v.w, scale_operand(byte));
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> two bf16 (lo in the low half), round to nearest even: the
// gfx950 v_cvt_pk_bf16_f32, which rounds by the kernel's fp32 round mode
// (nearest even) and keeps fp32 denormals (the kernels' denormal mode), so
// it equals bf16_rne on every finite input.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// One block-scaled fp4 x fp4 MFMA step: acc += (A_tile * 2^sa) x (B_tile * 2^sb)^T
// where each operand is one lane's 16-byte fragment and its scale byte sits
// in the low byte of the scale register.
__device__ __forceinline__ f32x16 mfma_fp4_32x32x64(const u32x4& a, const u32x4& b, f32x16 acc,
                                                   uint32_t scale_a, uint32_t scale_b) {
    i32x8 va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    i32x8 vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 4, 4, 0, (int)scale_a, 0,
                                                           (int)scale_b);
}

// Eight e2m1 codes (one dword, element 0 in the low nibble) widened to bf16
// times the scale operand 2^s by the gfx950 fp4 convert.  The product is
// exact in bf16 (a subnormal below 2^-126) for every scale byte the rule
// makes (s <= 126), except 4 * 2^126 and 6 * 2^126, past bf16's range.
__device__ __forceinline__ bf16x8 widen8_fp4(uint32_t codes, float sc) {
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// One bf16 MFMA over 16 K: acc += a x b^T, each operand one lane's 8 bf16.
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(const bf16x8& a, const bf16x8& b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// 32 wait states after an MFMA whose result is read next: more than the
// longest MFMA-result-to-VALU distance of the 32x32x64 scaled MFMA.
__device__ __forceinline__ void mfma_result_fence(f32x16& acc) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

__device__ __forceinline__ u32x4 load16_nt(const void* p) {
    return __builtin_nontemporal_load((const u32x4*)p);
}

// Buffer resources (gfx9 descriptor, raw 32-bit data format): the base and
// size live in SGPRs, each load adds a 32-bit lane offset and a wave-uniform
// offset, and any byte past `bytes` reads as zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kBufferDword3 = 0x00020000;
constexpr int kNonTemporal = 2;   // cache-policy bit: streamed once, do not keep

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferDword3);
}

template <int AUX = 0>
__device__ __forceinline__ u32x4 bload16(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX);
}

// 16 bytes per lane straight into LDS (gfx950 buffer_load_dwordx4 ... lds):
// lane l's bytes land at lds_base + 16 l, whatever its global offset; a lane
// whose offset is past the buffer writes zeros.  lds_base is wave-uniform.
// Completion is counted by vmcnt, in order with the wave's other loads.
__device__ __forceinline__ void bload16_lds(Rsrc r, uint8_t* lds_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, (int)voff, 0, 0,
                                             0);
}

// s_waitcnt for at most n outstanding vector-memory operations (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their
// maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t bload4(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
    return *(const u32x4*)p;
}

}  // namespace mx4
