// mx4_quant.hip -- MXFP4 quantisation kernels for gfx950.
//
//   quant_natural_kernel : bf16 [rows, K] -> codes [rows, K/2] + scales [rows, K/32]
//   pack_kernel          : bf16 [rows, K] -> packed operand layout (mx4_layout.h),
//                          one wave per 32 x 64 operand tile, coalesced row
//                          loads and tile stores; used once for the weight B
//                          and per call for A
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

// Packed-layout quantiser: one wave per operand tile (32 rows x 64 K), four
// waves per workgroup on four consecutive K steps; grid (ceil(KS / 4),
// rbstep = min(RB, 65535)), row blocks past 65535 walked by y.  The wave
// loads its tile's rows whole (8 lanes per 128-byte row segment, four
// 1 KiB loads) into its own padded LDS slab, reads back the 64 bytes of the
// 32-element group its lane quantises in the MFMA lane order (row L % 32,
// group L / 32 of the step), quantises it in registers and stores the tile
// as the 1 KiB it occupies (16 bytes per lane, one coalesced store) and the
// scale byte into byte t % 4 of its lane's scale word.  Rows past the matrix
// and a group past K read zeros (zero codes, byte 0); the wave of the last
// step also zeroes the scale bytes of the steps past KS in its word.
constexpr int kPackSlabRow = 144;   // 128 bytes of a row plus 16 of padding
__global__ void __launch_bounds__(256) pack_kernel(const uint16_t* __restrict__ x, int rows, int K, int ld,
                                                   uint8_t* __restrict__ packed, int RB, int KS, int KW,
                                                   uint32_t code_bytes, int rbstep) {
    __shared__ __attribute__((aligned(16))) uint8_t slab[4][kRowBlock * kPackSlabRow];
    const int wave = threadIdx.x >> 6;
    const int L = threadIdx.x & 63;
    const int t = (int)blockIdx.x * 4 + wave;
    if (t >= KS) return;   // whole waves leave; no barrier below
    const int G = K / kGroup;
    const Rsrc rx = make_rsrc(x, (uint32_t)rows * (uint32_t)ld * 2u);
    uint8_t* my = slab[wave];
    for (int rb = (int)blockIdx.y; rb < RB; rb += rbstep) {
        u32x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = q * 64 + L;
            const int r = c >> 3, j = c & 7;
            const bool live = 2 * t + (j >> 2) < G;
            const uint32_t off = (uint32_t)(rb * kRowBlock + r) * (uint32_t)ld * 2u + (uint32_t)t * 128u + j * 16u;
            v[q] = bload16(rx, live ? off : 0x80000000u, 0u);   // rows past the matrix read zeros
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = q * 64 + L;
            *(u32x4*)(my + (c >> 3) * kPackSlabRow + (c & 7) * 16) = v[q];
        }
        u32x4 g[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) g[c] = *(const u32x4*)(my + (L & 31) * kPackSlabRow + (L >> 5) * 64 + c * 16);
        u32x4 codes;
        const uint32_t byte = quant_group32(g, codes);
        *(u32x4*)(packed + ((size_t)(rb * KS + t) * 64 + L) * 16) = codes;
        uint8_t* word = packed + code_bytes + ((size_t)(rb * KW + t / kStepsPerWord) * 64 + L) * 4;
        word[t % kStepsPerWord] = (uint8_t)byte;
        if (t == KS - 1)
            for (int t2 = KS; t2 < KW * kStepsPerWord; ++t2) word[t2 % kStepsPerWord] = 0;
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
    const unsigned gx = (unsigned)((g.KS + 3) / 4);
    const unsigned gy = (unsigned)(g.RB < 65535 ? g.RB : 65535);
    return launch_kernel(pack_kernel, dim3(gx, gy), dim3(256), 0, s, x, rows, K, ld, packed, g.RB, g.KS, g.KW,
                         (uint32_t)g.code_bytes, (int)gy);
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
