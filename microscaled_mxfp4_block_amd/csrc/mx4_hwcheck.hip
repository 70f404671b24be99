// mx4_hwcheck.hip -- one-wave checks of the two gfx950 instructions the MXFP4
// path rests on, through the same device wrappers the GEMM and quantisation
// kernels use (mx4_device.h).  Test infrastructure: built into its own
// library (libmx4hw.so, include/mx4_hwcheck.h), never linked into libmx4.so.
//
//   mxhw_cvt_fp4   every input bf16 converted to an e2m1 code under the scale
//                  operand of each scale byte (v_cvt_scalef32_pk_fp4_bf16 via
//                  cvt8 / scale_operand), as the quantisers convert;
//   mxhw_widen_fp4 every e2m1 code widened to bf16 under each scale byte
//                  (v_cvt_scalef32_pk_bf16_fp4 via widen8_fp4), as the
//                  a16wfp4 product does;
//   mxhw_mfma_fp4  one v_mfma_scale_f32_32x32x64_f8f6f4 on per-lane fragments
//                  and scale registers given by the caller (mfma_fp4_32x32x64),
//                  writing every lane's 16 accumulators.
//
// And one measurement reference, mxhw_stream_read: a kernel that only reads
// bytes with the GEMM's kind of loads (128-bit buffer loads, several in
// flight per lane, non-temporal) and stores one dword per wave, so that a
// GEMM's time can be set against what merely streaming its bytes costs with
// the same grid.
#include "mx4_device.h"
#include "mx4_internal.h"
#include "../../include/mx4_hwcheck.h"

namespace mx4 {

// Grid (ceil(n / 8 / 64), bytes): lane i of block x converts the 8 bf16
// x[8 i .. 8 i + 7] under scale byte blockIdx.y into one dword of codes.
__global__ void __launch_bounds__(64) hw_cvt_kernel(const uint16_t* __restrict__ x, int n8,
                                                    uint32_t* __restrict__ codes) {
    const int i = (int)(blockIdx.x * 64u + threadIdx.x);
    if (i >= n8) return;
    const u32x4 v = *(const u32x4*)(x + 8 * (size_t)i);
    const float sc = scale_operand(blockIdx.y);
    codes[(size_t)blockIdx.y * n8 + i] = cvt8(v.x, v.y, v.z, v.w, sc);
}

// Grid (bytes): lane L < 2 widens the codes 8 L .. 8 L + 7 (all 16 codes)
// under scale byte blockIdx.x into 8 bf16.
__global__ void __launch_bounds__(64) hw_widen_kernel(uint16_t* __restrict__ out) {
    const int L = threadIdx.x;
    if (L >= 2) return;
    // codes 8 L .. 8 L + 7, element e in nibble e
    const uint32_t codes = L == 0 ? 0x76543210u : 0xFEDCBA98u;
    const bf16x8 v = widen8_fp4(codes, scale_operand(blockIdx.x));
    *(bf16x8*)(out + (size_t)blockIdx.x * 16 + 8 * L) = v;
}

// One wave: lane L passes fragment bytes a[16 L .. 16 L + 15] and
// b[16 L .. 16 L + 15] and the scale registers sa[L], sb[L] to one scaled
// MFMA from a zero accumulator; out[16 L + e] is its element e.
__global__ void __launch_bounds__(64) hw_mfma_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                     const uint32_t* __restrict__ sa,
                                                     const uint32_t* __restrict__ sb, float* __restrict__ out) {
    const int L = threadIdx.x;
    const u32x4 fa = *(const u32x4*)(a + 16 * L);
    const u32x4 fb = *(const u32x4*)(b + 16 * L);
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    acc = mfma_fp4_32x32x64(fa, fb, acc, sa[L], sb[L]);
    mfma_result_fence(acc);
#pragma unroll
    for (int e = 0; e < 16; ++e) out[16 * L + e] = acc[e];
}

// Workgroup g reads bytes [g * stride, g * stride + chunk) of buf (clipped
// at `bytes`: past it the buffer bound reads zeros), LPL 16-byte loads per
// lane in flight per round, and xors them into one dword per wave.
// Workgroup g starts its walk through the piece at byte (g * rot) % chunk and
// wraps around, so that workgroups reading one piece need not all ask for
// the same lines at the same time.
template <int LPL>
__global__ void __launch_bounds__(1024) hw_stream_kernel(const uint8_t* buf, uint32_t bytes, uint32_t chunk,
                                                         uint32_t stride, uint32_t rot, uint32_t* out) {
    const Rsrc r = make_rsrc(buf, bytes);
    const uint32_t nt = blockDim.x;
    const uint32_t base = blockIdx.x * stride;
    const uint32_t start = (uint32_t)(((uint64_t)blockIdx.x * rot) % chunk);
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (uint32_t off = 0; off < chunk; off += nt * 16u * LPL) {
        u32x4 v[LPL];
#pragma unroll
        for (int i = 0; i < LPL; ++i) {
            uint32_t o = off + ((uint32_t)i * nt + threadIdx.x) * 16u;
            const bool in = o < chunk;
            o += start;
            o = o >= chunk ? o - chunk : o;
            v[i] = bload16<kNonTemporal>(r, in ? base + o : 0x80000000u, 0u);
        }
#pragma unroll
        for (int i = 0; i < LPL; ++i) acc ^= v[i];
    }
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * (nt / 64) + threadIdx.x / 64] = x;
}

}  // namespace mx4

extern "C" {

int mxhw_stream_read(const void* buf_dev, unsigned bytes, int wgs, int waves, int lpl, unsigned chunk,
                     unsigned stride, unsigned rot, void* out_dev, void* stream) {
    if (!buf_dev || !out_dev || wgs <= 0 || waves <= 0 || waves > 16 || bytes >= 0x80000000u || chunk == 0)
        return -1;
    if ((uintptr_t)buf_dev % 16 || (uintptr_t)out_dev % 4 || chunk % 16 || rot % 16) return -2;
    auto k = lpl == 1 ? mx4::hw_stream_kernel<1> : lpl == 2 ? mx4::hw_stream_kernel<2>
           : lpl == 4 ? mx4::hw_stream_kernel<4> : lpl == 8 ? mx4::hw_stream_kernel<8>
           : lpl == 16 ? mx4::hw_stream_kernel<16> : nullptr;
    if (!k) return -1;
    hipLaunchKernelGGL(k, dim3((unsigned)wgs), dim3((unsigned)(64 * waves)), 0, (hipStream_t)stream,
                       (const uint8_t*)buf_dev, (uint32_t)bytes, (uint32_t)chunk, (uint32_t)stride,
                       (uint32_t)rot, (uint32_t*)out_dev);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mxhw_cvt_fp4(const void* x_dev, int n, int bytes, void* codes_dev, void* stream) {
    if (n <= 0 || n % 8 != 0 || bytes <= 0 || bytes > 255 || !x_dev || !codes_dev) return -1;
    if ((uintptr_t)x_dev % 16 || (uintptr_t)codes_dev % 4) return -2;
    const int n8 = n / 8;
    hipLaunchKernelGGL(mx4::hw_cvt_kernel, dim3((unsigned)((n8 + 63) / 64), (unsigned)bytes), dim3(64), 0,
                       (hipStream_t)stream, (const uint16_t*)x_dev, n8, (uint32_t*)codes_dev);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mxhw_widen_fp4(int bytes, void* out_dev, void* stream) {
    if (bytes <= 0 || bytes > 255 || !out_dev) return -1;
    if ((uintptr_t)out_dev % 16) return -2;
    hipLaunchKernelGGL(mx4::hw_widen_kernel, dim3((unsigned)bytes), dim3(64), 0, (hipStream_t)stream,
                       (uint16_t*)out_dev);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mxhw_mfma_fp4(const void* a_dev, const void* b_dev, const void* sa_dev, const void* sb_dev, void* out_dev,
                  void* stream) {
    if (!a_dev || !b_dev || !sa_dev || !sb_dev || !out_dev) return -1;
    if ((uintptr_t)a_dev % 16 || (uintptr_t)b_dev % 16 || (uintptr_t)sa_dev % 4 || (uintptr_t)sb_dev % 4 ||
        (uintptr_t)out_dev % 4)
        return -2;
    hipLaunchKernelGGL(mx4::hw_mfma_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a_dev,
                       (const uint8_t*)b_dev, (const uint32_t*)sa_dev, (const uint32_t*)sb_dev, (float*)out_dev);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mxhw_xcd_map(int mtiles, int ntiles, int splits, double a_tile_bytes, double b_tile_bytes, int conc, int runs,
                 int* map_out, int* mt_out, int* nt_out) {
    if (mtiles < 1 || ntiles < 1 || (long long)mtiles * ntiles > (1 << 20) || splits < 1 || !(a_tile_bytes > 0.0) ||
        !(b_tile_bytes > 0.0) || conc < 0 || runs < 0 || runs > 2 || !map_out || !mt_out || !nt_out)
        return -1;
    const int map = runs ? (splits == 1 ? mx4::tile_xcd_map(mtiles, ntiles, a_tile_bytes, b_tile_bytes, conc, runs) : 0)
                         : mx4::shared_xcd_map(mtiles, ntiles, splits, a_tile_bytes, b_tile_bytes, conc);
    *map_out = map;
    for (int by = 0; by < mtiles; ++by)
        for (int bx = 0; bx < ntiles; ++bx) {
            const int lin = bx + ntiles * by;
            mx4::shared_tile_of(bx, by, ntiles, mtiles, map, mt_out[lin], nt_out[lin]);
        }
    return 0;
}

}  // extern "C"
