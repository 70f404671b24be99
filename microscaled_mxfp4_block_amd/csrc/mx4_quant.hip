// mx4_quant.hip -- MXFP4 quantisation kernels for gfx950.
//
//   quant_natural_kernel : bf16 [rows, K] -> codes [rows, K/2] + scales [rows, K/32]
//   pack_kernel          : bf16 [rows, K] -> packed operand layout (mx4_layout.h),
//                          coalesced row loads, one DPP quad per group;
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

// No kernel here reads blockDim or gridDim (the two that walk rows take the
// grid's y extent as an argument), so each argument segment holds only the
// kernel's own scalars, no hidden arguments: the host writes that segment on
// every launch.

// Natural-layout quantiser.  Grid (ceil(K / 8 / 256), rstep = min(rows,
// 65535)): one lane per 16-byte column of a row (rows past 65535 walked by
// y); each lane writes its 8 codes as one dword, the first lane of a quad the
// scale byte.
__global__ void __launch_bounds__(256) quant_natural_kernel(const uint16_t* __restrict__ x, int rows,
                                                            int K, int ld, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int rstep) {
    const int c = (int)(blockIdx.x * 256u + threadIdx.x);
    // whole quads leave together: K / 8 is a multiple of 4 and blocks are 256 wide
    if (c >= K / 8) return;
    for (int r = (int)blockIdx.y; r < rows; r += rstep) {
        const u32x4 v = load16(x + (size_t)r * ld + (size_t)c * 8);
        uint32_t byte;
        const uint32_t q = quad_quant8(v, byte);
        *(uint32_t*)(codes + (size_t)r * (K / 2) + (size_t)c * 4) = q;
        if ((c & 3) == 0) scales[(size_t)r * (K / 32) + c / 4] = (uint8_t)byte;
    }
}

// Packed-layout quantiser, coalesced.  Grid (ceil(KW * 32 / 256),
// rstep = min(RB * 32, 65535)): one lane per 16-byte column c of row r of the operand
// padded to RB * 32 rows and KW * 4 K steps (rows past 65535 walked by y).
// The quad of group g = c / 4 quantises it; lane q of the quad writes dword q
// of the 16-byte code fragment of slot (rb, t, L) = (r / 32, g / 2,
// r % 32 + 32 (g % 2)) (mx4_layout.h), the quad's first lane the scale byte
// into byte t % 4 of that lane's scale word.  Padding rows and groups get
// zero codes and byte 0; steps past KS exist only as scale-word bytes.
__global__ void __launch_bounds__(256) pack_kernel(const uint16_t* __restrict__ x, int rows, int K, int ld,
                                                   uint8_t* __restrict__ packed, int RB, int KS, int KW,
                                                   size_t code_bytes, int rstep) {
    const int c = (int)(blockIdx.x * 256u + threadIdx.x);
    if (c >= KW * 32) return;   // whole quads leave together
    const int g = c >> 2, q = c & 3, t = g >> 1, h = g & 1;
    const bool group_live = g < K / kGroup;
    for (int r = (int)blockIdx.y; r < RB * kRowBlock; r += rstep) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < rows && group_live) v = load16(x + (size_t)r * ld + (size_t)c * 8);
        uint32_t byte;
        const uint32_t codes = quad_quant8(v, byte);
        const int rb = r >> 5, L = (r & 31) + 32 * h;
        if (t < KS) *(uint32_t*)(packed + ((size_t)(rb * KS + t) * 64 + L) * 16 + 4 * q) = codes;
        if (q == 0)
            packed[code_bytes + ((size_t)(rb * KW + t / kStepsPerWord) * 64 + L) * 4 + t % kStepsPerWord] =
                (uint8_t)byte;
    }
}

// Packed layout -> natural layouts.  One lane per (rb, t, L) tile slot.
__global__ void __launch_bounds__(256) unpack_kernel(const uint8_t* __restrict__ packed, int rows, int K,
                                                     int RB, int KS, int KW, size_t code_bytes,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
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
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
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
    const unsigned gx = (unsigned)((K / 8 + 255) / 256);
    const unsigned gy = (unsigned)(rows < 65535 ? rows : 65535);
    return launch_kernel(quant_natural_kernel, dim3(gx, gy), dim3(256), 0, s, x, rows, K, ld, codes, scales, (int)gy);
}

hipError_t launch_pack(const uint16_t* x, int rows, int K, int ld, uint8_t* packed, hipStream_t s) {
    const OperandGeom g = operand_geom(rows, K);
    const unsigned gx = (unsigned)((g.KW * 32 + 255) / 256);
    const unsigned gy = (unsigned)(g.RB * kRowBlock < 65535 ? g.RB * kRowBlock : 65535);
    return launch_kernel(pack_kernel, dim3(gx, gy), dim3(256), 0, s, x, rows, K, ld, packed, g.RB, g.KS, g.KW,
                         g.code_bytes, (int)gy);
}

hipError_t launch_import(const uint8_t* codes, const uint8_t* scales, int rows, int K, uint8_t* packed,
                         hipStream_t s) {
    const OperandGeom g = operand_geom(rows, K);
    const long long total = (long long)g.RB * g.KW * kStepsPerWord * 64;
    const long long blocks = (total + 255) / 256;
    return launch_kernel(import_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scales, rows, K, packed, g.RB,
                         g.KS, g.KW, g.code_bytes);
}

hipError_t launch_unpack(const uint8_t* packed, int rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
    const OperandGeom g = operand_geom(rows, K);
    const long long total = (long long)g.RB * g.KS * 64;
    const long long blocks = (total + 255) / 256;
    return launch_kernel(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, packed, rows, K, g.RB, g.KS, g.KW,
                         g.code_bytes, codes, scales);
}

}  // namespace mx4
