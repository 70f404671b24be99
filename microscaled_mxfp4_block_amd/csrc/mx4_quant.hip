// mx4_quant.hip -- MXFP4 quantisation kernels for gfx950.
//
//   quant_natural_kernel : bf16 [rows, K] -> codes [rows, K/2] + scales [rows, K/32]
//   pack_kernel          : bf16 [rows, K] -> packed operand layout (mx4_layout.h);
//                          used once for the weight B and per call for A
//   unpack_kernel        : packed operand layout -> natural codes + scales
//   import_kernel        : natural codes + scales (already quantised elsewhere)
//                          -> packed operand layout, bytes moved unchanged
//
// The rule is the MXFP4 quantisation of the kernelindex.com amd-mxfp4-mm pages
// (submission 755056, "Software MXFP4 quant"): per 32-element group, amax
// rounded to a power of two by (bits + 0x00200000) & 0xFF800000, scale byte
// clamp(E - 129, -127, 127) + 127, element codes e2m1(x * 2^-s) with round to
// nearest even and saturation at 6, sign kept.  The e2m1 conversion uses the
// gfx950 v_cvt_scalef32_pk_fp4_bf16 instruction, which divides by the scale
// operand 2^s and rounds that way.
#include "mx4_device.h"
#include "mx4_internal.h"

namespace mx4 {

// Natural-layout quantiser.  One lane per 8 consecutive bf16 (one 16-byte
// load); the four lanes of a DPP quad hold one 32-element group and reduce
// its amax across the quad with two lane swaps.  Each lane writes its 8 codes
// as one dword; the first lane of the quad writes the scale byte.
__global__ void __launch_bounds__(256) quant_natural_kernel(const uint16_t* __restrict__ x, int rows,
                                                            int K, int ld, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
    const int chunks_per_row = K / 8;
    const long long total = (long long)rows * chunks_per_row;
    const long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    // Every lane of a quad exists: total is a multiple of 4 (K % 32 == 0) and
    // the grid is rounded to whole blocks of 256, so quads never straddle the end.
    const bool live = c < total;
    const int r = live ? (int)(c / chunks_per_row) : 0;
    const int kc = live ? (int)(c % chunks_per_row) : 0;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (live) v = load16(x + (size_t)r * ld + (size_t)kc * 8);
    uint32_t m = 0;
    {
        u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
        a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu));
        a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu));
        a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu));
        m = a.x > a.y ? a.x : a.y;
    }
    // quad_perm [1,0,3,2] then [2,3,0,1]: max over the four lanes of the quad
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);
    m = m > o ? m : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false);
    m = m > o ? m : o;
    const uint32_t byte = scale_byte_from_amax16(m);
    if (!live) return;
    const float sc = scale_operand(byte);
    const uint32_t q = cvt8(v.x, v.y, v.z, v.w, sc);
    *(uint32_t*)(codes + (size_t)r * (K / 2) + (size_t)kc * 4) = q;
    if ((kc & 3) == 0) scales[(size_t)r * (K / 32) + kc / 4] = (uint8_t)byte;
}

// Packed-layout quantiser.  One lane per operand slot (rb, t, L): it loads
// the 64 bytes of row 32 rb + L % 32, group 2t + L / 32 with four 16-byte
// loads, quantises them, writes the 16-byte code fragment to its slot (the
// 64 lanes of a wave write one contiguous 1 KiB tile) and its scale byte into
// byte t % 4 of the lane's scale word.  Every lane does one load round trip.
__global__ void __launch_bounds__(256) pack_kernel(const uint16_t* __restrict__ x, int rows, int K, int ld,
                                                   uint8_t* __restrict__ packed, int RB, int KS, int KW,
                                                   size_t code_bytes) {
    // grid (ceil(KW * 4 * 64 / 256), min(RB, 65535)): slot (t, L) from x with
    // 32-bit math, row blocks rb from y (walked when there are more than 65535)
    const int slot = (int)(blockIdx.x * 256u + threadIdx.x);
    if (slot >= KW * kStepsPerWord * 64) return;
    const int L = slot & 63;
    const int t = slot >> 6;
    const int g = 2 * t + (L >> 5);
    for (int rb = (int)blockIdx.y; rb < RB; rb += (int)gridDim.y) {
        const int row = rb * kRowBlock + (L & 31);
        u32x4 codes = {0u, 0u, 0u, 0u};
        uint32_t byte = 0u;
        if (row < rows && g < K / kGroup) {
            const uint16_t* src = x + (size_t)row * ld + (size_t)g * kGroup;
            u32x4 v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = load16(src + 8 * i);
            byte = quant_group32(v, codes);
        }
        // steps past KS exist only as padding bytes of the last scale word
        if (t < KS) *(u32x4*)(packed + ((size_t)(rb * KS + t) * 64 + L) * 16) = codes;
        packed[code_bytes + ((size_t)(rb * KW + t / kStepsPerWord) * 64 + L) * 4 + t % kStepsPerWord] = (uint8_t)byte;
    }
}

// Packed layout -> natural layouts.  One lane per (rb, t, L) tile slot.
__global__ void __launch_bounds__(256) unpack_kernel(const uint8_t* __restrict__ packed, int rows, int K,
                                                     int RB, int KS, int KW, size_t code_bytes,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)RB * KS * 64;
    if (gid >= total) return;
    const int L = (int)(gid & 63);
    const long long rt = gid >> 6;
    const int t = (int)(rt % KS);
    const int rb = (int)(rt / KS);
    const int row = rb * kRowBlock + (L & 31);
    const int g = 2 * t + (L >> 5);
    if (row >= rows || g >= K / kGroup) return;
    const u32x4 c = load16(packed + ((size_t)(rb * KS + t) * 64 + L) * 16);
    *(u32x4*)(codes + (size_t)row * (K / 2) + (size_t)g * 16) = c;
    const uint32_t word = *(const uint32_t*)(packed + code_bytes +
                                             ((size_t)(rb * KW + t / kStepsPerWord) * 64 + L) * 4);
    scales[(size_t)row * (K / kGroup) + g] = (uint8_t)(word >> (8 * (t % kStepsPerWord)));
}

// Natural layouts -> packed layout, no re-quantisation.  One lane per
// (rb, t, L) slot as in pack_kernel; padding slots get zero codes, byte 0.
__global__ void __launch_bounds__(256) import_kernel(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int rows, int K,
                                                     uint8_t* __restrict__ packed, int RB, int KS, int KW,
                                                     size_t code_bytes) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)RB * KW * kStepsPerWord * 64;
    if (gid >= total) return;
    const int L = (int)(gid & 63);
    const long long rt = gid >> 6;
    const int t = (int)(rt % (KW * kStepsPerWord));
    const int rb = (int)(rt / (KW * kStepsPerWord));
    const int row = rb * kRowBlock + (L & 31);
    const int g = 2 * t + (L >> 5);
    u32x4 c = {0u, 0u, 0u, 0u};
    uint32_t byte = 0u;
    if (row < rows && g < K / kGroup) {
        c = load16(codes + (size_t)row * (K / 2) + (size_t)g * 16);
        byte = scales[(size_t)row * (K / kGroup) + g];
    }
    if (t < KS) *(u32x4*)(packed + ((size_t)(rb * KS + t) * 64 + L) * 16) = c;
    packed[code_bytes + ((size_t)(rb * KW + t / kStepsPerWord) * 64 + L) * 4 + t % kStepsPerWord] = (uint8_t)byte;
}

hipError_t launch_quant_natural(const uint16_t* x, int rows, int K, int ld, uint8_t* codes, uint8_t* scales,
                                hipStream_t s) {
    const long long total = (long long)rows * (K / 8);
    const long long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(quant_natural_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, K, ld, codes,
                       scales);
    return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* x, int rows, int K, int ld, uint8_t* packed, hipStream_t s) {
    const OperandGeom g = operand_geom(rows, K);
    const unsigned gx = (unsigned)((g.KW * kStepsPerWord * 64 + 255) / 256);
    const unsigned gy = (unsigned)(g.RB < 65535 ? g.RB : 65535);
    hipLaunchKernelGGL(pack_kernel, dim3(gx, gy), dim3(256), 0, s, x, rows, K, ld, packed, g.RB, g.KS, g.KW,
                       g.code_bytes);
    return hipGetLastError();
}

hipError_t launch_import(const uint8_t* codes, const uint8_t* scales, int rows, int K, uint8_t* packed,
                         hipStream_t s) {
    const OperandGeom g = operand_geom(rows, K);
    const long long total = (long long)g.RB * g.KW * kStepsPerWord * 64;
    const long long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(import_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scales, rows, K, packed, g.RB,
                       g.KS, g.KW, g.code_bytes);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
    const OperandGeom g = operand_geom(rows, K);
    const long long total = (long long)g.RB * g.KS * 64;
    const long long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, packed, rows, K, g.RB, g.KS, g.KW,
                       g.code_bytes, codes, scales);
    return hipGetLastError();
}

}  // namespace mx4
