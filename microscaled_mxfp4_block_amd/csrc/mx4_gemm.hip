// mx4_gemm.hip -- block-scaled MXFP4 GEMM for gfx950 (MI355X).
//
//   C[M,N] = sum_k deq(A)[m,k] * deq(B)[n,k]   (fp32 accumulation, bf16 RNE out)
//
// The product is the block-scaled fp4 contraction the kernelindex.com
// amd-mxfp4-mm pages express as tl.dot_scaled(a, a_scale, "e2m1", b,
// b_scale, "e2m1") (e.g. submission 748756, kernel_fused_mxfp4_gemm); here it
// is written directly on v_mfma_scale_f32_32x32x64_f8f6f4, whose per-lane
// e8m0 scale applies 2^(byte-127) to that lane's 32-element group.
//
// Work decomposition (one workgroup = WK waves):
//   - a wave owns an output tile of (32 * MBLK) m x (32 * NBLK) n;
//   - the WK waves of a workgroup split the tile's K steps and add their
//     accumulators through LDS;
//   - `splits` workgroups split K further and write fp32 partials that a
//     second kernel sums in a fixed order (deterministic split-K).
// Each wave streams its weight tiles straight from HBM into VGPRs with one
// coalesced non-temporal 128-bit load per lane per 1 KiB tile (no LDS
// staging: every weight byte is used by exactly one wave of the tile's
// workgroup), prefetching PF K steps ahead.  With FUSEQ the wave also
// quantises its own activation groups (one lane = one 32-element group, so
// the group amax is a per-lane max) right before the MFMA; without it the
// activation operand comes pre-packed from the workspace.
#include "mx4_device.h"
#include "mx4_internal.h"

namespace mx4 {

// Workgroups are dispatched round-robin over the 8 XCDs (blockIdx i runs on
// XCD i % 8).  Remap so that consecutive logical tile indices share an XCD,
// which keeps the M tiles that read the same weight tiles on one L2.
__device__ __forceinline__ int xcd_linear(int i, int G) {
    const int q = G / 8, r = G % 8, x = i % 8;
    return x * q + (x < r ? x : r) + i / 8;
}

template <int MBLK, int NBLK, bool FUSEQ>
struct Slot {
    u32x4 b[NBLK];
    uint32_t bs[NBLK];
    u32x4 a[MBLK][FUSEQ ? 4 : 1];
    uint32_t as[MBLK];
};

template <int MBLK, int NBLK, bool FUSEQ>
__device__ __forceinline__ void load_step(Slot<MBLK, NBLK, FUSEQ>& sl, const GemmParams& p, int mb0, int nb0,
                                          int t, int L) {
    const int w = t >> 2;
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
        const int nb = nb0 + j;
        if (nb < p.RBn) {
            sl.b[j] = load16_nt(p.bp + ((size_t)(nb * p.KS + t) * 64 + L) * 16);
            sl.bs[j] = *(const uint32_t*)(p.bp + p.b_code_bytes + ((size_t)(nb * p.KW + w) * 64 + L) * 4);
        } else {
            sl.b[j] = u32x4{0u, 0u, 0u, 0u};
            sl.bs[j] = 0x7F7F7F7Fu;
        }
    }
#pragma unroll
    for (int i = 0; i < MBLK; ++i) {
        const int mb = mb0 + i;
        if constexpr (FUSEQ) {
            const int row = mb * kRowBlock + (L & 31);
            const int g = 2 * t + (L >> 5);
            if (row < p.M && g * kGroup < p.K) {
                const uint16_t* src = p.A + (size_t)row * p.lda + (size_t)g * kGroup;
#pragma unroll
                for (int q = 0; q < 4; ++q) sl.a[i][q] = load16(src + 8 * q);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) sl.a[i][q] = u32x4{0u, 0u, 0u, 0u};
            }
        } else {
            if (mb < p.RBm) {
                sl.a[i][0] = load16(p.aop + ((size_t)(mb * p.KS + t) * 64 + L) * 16);
                sl.as[i] = *(const uint32_t*)(p.aop + p.a_code_bytes + ((size_t)(mb * p.KW + w) * 64 + L) * 4);
            } else {
                sl.a[i][0] = u32x4{0u, 0u, 0u, 0u};
                sl.as[i] = 0x7F7F7F7Fu;
            }
        }
    }
}

template <int MBLK, int NBLK, bool FUSEQ>
__device__ __forceinline__ void compute_step(const Slot<MBLK, NBLK, FUSEQ>& sl, f32x16 (&acc)[MBLK][NBLK],
                                             int t) {
    const int sh = 8 * (t & 3);
    u32x4 af[MBLK];
    uint32_t as[MBLK];
#pragma unroll
    for (int i = 0; i < MBLK; ++i) {
        if constexpr (FUSEQ) {
            as[i] = quant_group32(sl.a[i], af[i]);
        } else {
            af[i] = sl.a[i][0];
            as[i] = sl.as[i] >> sh;
        }
    }
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
        const uint32_t bs = sl.bs[j] >> sh;
#pragma unroll
        for (int i = 0; i < MBLK; ++i) acc[i][j] = mfma_fp4_32x32x64(sl.b[j], af[i], acc[i][j], bs, as[i]);
    }
}

// Write 4 consecutive outputs (n0..n0+3) of row m: bf16 to C, or fp32 to the
// split-K partial buffer.
__device__ __forceinline__ void store4(const GemmParams& p, int split, int m, int n0, float v0, float v1, float v2,
                                       float v3) {
    if (m >= p.M) return;
    if (p.splits > 1) {
        f32x4 v = {v0, v1, v2, v3};
        *(f32x4*)(p.partial + ((size_t)split * p.M + m) * p.ldp + n0) = v;
        return;
    }
    uint16_t* dst = p.C + (size_t)m * p.ldc + n0;
    if (p.c_vec && n0 + 3 < p.N) {
        uint2 w;
        w.x = pack_bf16x2(v0, v1);
        w.y = pack_bf16x2(v2, v3);
        *(uint2*)dst = w;
    } else {
        const float v[4] = {v0, v1, v2, v3};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (n0 + q < p.N) dst[q] = (uint16_t)bf16_rne(v[q]);
    }
}

template <int MBLK, int NBLK, int WK, bool FUSEQ, int PF>
__global__ void __launch_bounds__(64 * WK) gemm_kernel(GemmParams p) {
    const int wave = threadIdx.x >> 6;
    const int L = threadIdx.x & 63;
    const int lin = xcd_linear(blockIdx.x, gridDim.x);
    const int mt = lin % p.mtiles;
    const int rest = lin / p.mtiles;
    const int split = rest % p.splits;
    const int nt = rest / p.splits;
    const int mb0 = mt * MBLK;
    const int nb0 = nt * NBLK;

    const int kb = split * p.steps_per_split;
    const int ke = min(kb + p.steps_per_split, p.KS);
    const int per_wave = (ke - kb + WK - 1) / WK;
    const int wb = kb + wave * per_wave;
    const int we = min(wb + per_wave, ke);

    f32x16 acc[MBLK][NBLK];
#pragma unroll
    for (int i = 0; i < MBLK; ++i)
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    Slot<MBLK, NBLK, FUSEQ> sl[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (wb + u < we) load_step(sl[u], p, mb0, nb0, wb + u, L);
    for (int t0 = wb; t0 < we; t0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int t = t0 + u;
            if (t < we) {
                compute_step(sl[u], acc, t);
                if (t + PF < we) load_step(sl[u], p, mb0, nb0, t + PF, L);
            }
        }
    }

    // lane L, accumulator element e of tile (i, j): m = 32 mb + L % 32,
    // n = 32 nb + 8 (e / 4) + 4 (L / 32) + e % 4.
    const int m_lane = L & 31;
    const int n_lane = 4 * (L >> 5);
    if constexpr (WK == 1) {
#pragma unroll
        for (int i = 0; i < MBLK; ++i)
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (nb0 + j >= p.RBn) continue;
                    store4(p, split, (mb0 + i) * kRowBlock + m_lane, (nb0 + j) * kRowBlock + 8 * r + n_lane,
                           acc[i][j][4 * r], acc[i][j][4 * r + 1], acc[i][j][4 * r + 2], acc[i][j][4 * r + 3]);
                }
    } else {
        constexpr int E = MBLK * NBLK * 16;
        __shared__ float red[WK][E][64];
#pragma unroll
        for (int i = 0; i < MBLK; ++i)
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) red[wave][(i * NBLK + j) * 16 + e][L] = acc[i][j][e];
        __syncthreads();
        constexpr int GE = E / 4;   // groups of 4 consecutive n
        for (int gi = wave; gi < GE; gi += WK) {
            const int ij = gi >> 2, r = gi & 3;
            const int i = ij / NBLK, j = ij % NBLK;
            if (nb0 + j >= p.RBn) continue;
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float s = 0.0f;
#pragma unroll
                for (int w2 = 0; w2 < WK; ++w2) s += red[w2][gi * 4 + q][L];
                v[q] = s;
            }
            store4(p, split, (mb0 + i) * kRowBlock + m_lane, (nb0 + j) * kRowBlock + 8 * r + n_lane, v[0], v[1],
                   v[2], v[3]);
        }
    }
}

// Sum the split-K partials in split order and round to bf16.  One lane per
// 4 consecutive outputs of a row.
__global__ void __launch_bounds__(256) reduce_kernel(const float* __restrict__ partial, int splits, int M, int N,
                                                     int ldp, uint16_t* __restrict__ C, int ldc, int c_vec) {
    const int n4 = (N + 3) / 4;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (long long)M * n4) return;
    const int m = (int)(gid / n4);
    const int n0 = (int)(gid % n4) * 4;
    f32x4 s = *(const f32x4*)(partial + (size_t)m * ldp + n0);
    for (int k = 1; k < splits; ++k) {
        const f32x4 v = *(const f32x4*)(partial + ((size_t)k * M + m) * ldp + n0);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    uint16_t* dst = C + (size_t)m * ldc + n0;
    if (c_vec && n0 + 3 < N) {
        uint2 w;
        w.x = pack_bf16x2(s.x, s.y);
        w.y = pack_bf16x2(s.z, s.w);
        *(uint2*)dst = w;
    } else {
        const float v[4] = {s.x, s.y, s.z, s.w};
        for (int q = 0; q < 4; ++q)
            if (n0 + q < N) dst[q] = (uint16_t)bf16_rne(v[q]);
    }
}

// ---------------------------------------------------------------------------
// Instantiation table.

typedef void (*GemmFn)(GemmParams);

template <int MBLK, int NBLK, int WK, bool FUSEQ>
constexpr GemmFn pick() {
    return gemm_kernel<MBLK, NBLK, WK, FUSEQ, FUSEQ ? 2 : 4>;
}

template <int MBLK, int NBLK, bool FUSEQ>
GemmFn pick_wk(int wk) {
    // the LDS reduction buffer holds WK x (MBLK * NBLK * 16) x 64 floats
    constexpr bool big = MBLK * NBLK >= 4;
    switch (wk) {
        case 1: return pick<MBLK, NBLK, 1, FUSEQ>();
        case 2: return pick<MBLK, NBLK, 2, FUSEQ>();
        case 4: return pick<MBLK, NBLK, 4, FUSEQ>();
        case 8: return pick<MBLK, NBLK, 8, FUSEQ>();
        case 16: return big ? nullptr : pick<MBLK, NBLK, big ? 1 : 16, FUSEQ>();
        default: return nullptr;
    }
}

static GemmFn find_kernel(const Plan& plan) {
    if (plan.fuse) {
        // fused quantisation keeps four raw 16-byte vectors per activation
        // block and prefetch slot in VGPRs: one activation block per wave
        if (plan.mb == 1 && plan.nb == 1) return pick_wk<1, 1, true>(plan.wk);
        if (plan.mb == 1 && plan.nb == 2) return pick_wk<1, 2, true>(plan.wk);
        return nullptr;
    }
    if (plan.mb == 1 && plan.nb == 1) return pick_wk<1, 1, false>(plan.wk);
    if (plan.mb == 1 && plan.nb == 2) return pick_wk<1, 2, false>(plan.wk);
    if (plan.mb == 2 && plan.nb == 1) return pick_wk<2, 1, false>(plan.wk);
    if (plan.mb == 2 && plan.nb == 2) return pick_wk<2, 2, false>(plan.wk);
    return nullptr;
}

bool gemm_plan_supported(const Plan& plan) {
    return plan.splits >= 1 && find_kernel(plan) != nullptr;
}

hipError_t launch_gemm(const Plan& plan, const GemmParams& p, hipStream_t s) {
    GemmFn fn = find_kernel(plan);
    if (!fn) return hipErrorInvalidValue;
    const long long grid = (long long)p.mtiles * p.ntiles * p.splits;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64 * plan.wk), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_reduce(const float* partial, int splits, int M, int N, int ldp, uint16_t* C, int ldc,
                         int c_vec, hipStream_t s) {
    const long long total = (long long)M * ((N + 3) / 4);
    const long long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, partial, splits, M, N, ldp, C, ldc, c_vec);
    return hipGetLastError();
}

}  // namespace mx4
